// topk.hip -- a5: exact top-k selection over the indexer scores.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: each query keeps the
// top-k compressed entries chosen by the lightning indexer (k = 1024 for Pro);
// "DeepSeek V4 preview and technical report" (chooseai.net), section 1: k = 512 for Flash.
//
// Order: score descending, then index ascending (the lowest index wins ties); the selection
// is written in ascending index order, padded with -1.  Equivalently each key i carries the
// distinct 64-bit rank (orderable score key << 32) | ~i and the k largest ranks win.
//
// Radix select in two kernels (the kernel boundary orders the stages; no workgroup waits on
// another and no device-wide fence is needed):
//   scan:     the indexer counted the top 12 bits of every score key (in kHistCopies copies).
//             Each workgroup finds the threshold bin T (the bin holding the k-th best key)
//             from the top of that histogram, then lists, in index order, every key of its
//             slice whose bin is >= T, with its score key.
//   finalize: one workgroup per query reads the listed keys in global index order (slice by
//             slice), resolves the keys inside bin T exactly with LDS radix passes over the
//             remaining 20 score bits and the inverted index, and compacts the winners in
//             order, so the output is ascending without a sort.
#include "common.hpp"

namespace v4a {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kLdsList = 12288;   // listed keys the finalize kernel keeps in LDS
constexpr int kMaxSlices = 1024;  // n_max <= 8M keys

int select_slices(int64_t n_max) {
    int64_t s = (n_max + kSelSlice - 1) / kSelSlice;
    return (int)(s < 1 ? 1 : s);
}

struct SelParams {
    const uint32_t *keys;
    const uint32_t *hist;    // [BQ][copies][4096]
    int copies;
    int64_t n_max;
    int k, slices;
    uint32_t *list;
    uint32_t *counts;
    int32_t *meta;
    int32_t *out;
};

// Block-wide inclusive prefix sum of one value per thread (thread order); `total` gets the
// sum over the block.  Uses wavefront shuffles and one LDS exchange.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t *wsum, uint32_t *total) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(v, o);
        if (lane >= o) v += u;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    uint32_t base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < kSelWaves; i++) {
        const uint32_t x = wsum[i];
        base += i < w ? x : 0u;
        tot += x;
    }
    *total = tot;
    __syncthreads();
    return base + v;
}

// Walks a histogram from its top bin down, nb bins, in rounds of kSelThreads bins, and finds
// the bin T where the count from the top first reaches `need`; returns T (or -1) and the
// count strictly above T.  `bin_count(b)` gives the count of bin b.
template <class F>
__device__ __forceinline__ void top_down_threshold(int nb, uint32_t need, F bin_count, uint32_t *wsum,
                                                   int *sT, uint32_t *sAbove, int *T, uint32_t *above) {
    const int t = threadIdx.x;
    if (t == 0) { *sT = -1; *sAbove = 0; }
    uint32_t run = 0;
    for (int r0 = 0; r0 < nb; r0 += kSelThreads) {
        const int bin = nb - 1 - (r0 + t);
        const uint32_t c = bin >= 0 ? bin_count(bin) : 0u;
        uint32_t tot;
        const uint32_t incl = block_scan(c, wsum, &tot);
        if (run + incl >= need && run + incl - c < need) {
            *sT = bin;
            *sAbove = run + incl - c;
        }
        run += tot;
        __syncthreads();
        if (*sT >= 0 || run >= need) break;  // uniform: every thread reads the same LDS value
    }
    __syncthreads();
    *T = *sT;
    *above = *sAbove;
    __syncthreads();
}

__global__ void __launch_bounds__(kSelThreads) select_scan_kernel(SelParams P, QueryPos QP) {
    __shared__ uint32_t wsum[2 * kSelWaves];  // double-buffered so one barrier per round suffices
    __shared__ int sT;
    __shared__ uint32_t sAbove;
    const int qi = blockIdx.y, s = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int64_t n_vis = visible_keys(QP, qi);
    const uint32_t k_eff = (uint32_t)(n_vis < P.k ? n_vis : P.k);
    uint32_t *cnt = P.counts + (int64_t)qi * P.slices + s;
    if (k_eff == 0) {
        if (t == 0) {
            *cnt = 0;
            if (s == 0) { P.meta[2 * qi] = -1; P.meta[2 * qi + 1] = 0; }
        }
        return;
    }
    const uint32_t *h = P.hist + (int64_t)qi * P.copies * kHistBins;
    const bool one_copy = P.copies == 1;
    int T;
    uint32_t above;
    top_down_threshold(kHistBins, k_eff, [&](int bin) {
        if (one_copy) return h[bin];
        uint32_t c = 0;
#pragma unroll
        for (int cp = 0; cp < kHistCopies; cp++) c += h[cp * kHistBins + bin];
        return c;
    }, wsum, &sT, &sAbove, &T, &above);
    if (s == 0 && t == 0) {
        P.meta[2 * qi] = T;
        P.meta[2 * qi + 1] = (int32_t)above;
    }
    // list, in index order, the slice's keys whose bin is >= T
    const int64_t lo = (int64_t)s * kSelSlice;
    const int64_t hi = lo + kSelSlice < n_vis ? lo + kSelSlice : n_vis;
    const uint32_t *keys = P.keys + (int64_t)qi * P.n_max;
    uint32_t *lst = P.list + ((int64_t)qi * P.slices * kSelSlice + lo) * 2;
    // every key of the slice is loaded before the first is used (kSelSlice / kSelThreads each)
    constexpr int kPer = kSelSlice / kSelThreads;
    uint32_t kv[kPer];
#pragma unroll
    for (int r = 0; r < kPer; r++) {
        const int64_t i = lo + (int64_t)r * kSelThreads + t;
        kv[r] = i < hi ? keys[i] : 0u;
    }
    uint32_t off = 0;
#pragma unroll
    for (int r = 0; r < kPer; r++) {
        const int64_t i = lo + (int64_t)r * kSelThreads + t;
        const uint32_t key = kv[r];
        const bool take = i < hi && (int)(key >> 20) >= T;
        const uint64_t m = __ballot(take);
        if (lane == 0) wsum[(r & 1) * kSelWaves + w] = (uint32_t)__popcll(m);
        __syncthreads();
        uint32_t base = off, tot = 0;
#pragma unroll
        for (int j = 0; j < kSelWaves; j++) {
            const uint32_t x = wsum[(r & 1) * kSelWaves + j];
            base += j < w ? x : 0u;
            tot += x;
        }
        if (take) {
            const uint32_t pos = base + (uint32_t)__popcll(m & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
            lst[2 * pos] = (uint32_t)i;
            lst[2 * pos + 1] = key;
        }
        off += tot;
    }
    if (t == 0) *cnt = off;
}

__global__ void __launch_bounds__(kSelThreads) select_final_kernel(SelParams P, QueryPos QP) {
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ int sT;
    __shared__ uint32_t sAbove;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t lidx[kLdsList];
    __shared__ uint32_t lkey[kLdsList];
    __shared__ uint32_t soff[kMaxSlices + 1];
    const int qi = blockIdx.x, t = threadIdx.x;
    const int64_t n_vis = visible_keys(QP, qi);
    const uint32_t k_eff = (uint32_t)(n_vis < P.k ? n_vis : P.k);
    int32_t *out = P.out + (int64_t)qi * P.k;
    if (k_eff == 0) {
        for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
        return;
    }
    const int T = P.meta[2 * qi];
    const uint32_t above = (uint32_t)P.meta[2 * qi + 1];
    const uint32_t need = k_eff > above ? k_eff - above : 0u;  // keys still to take from bin T
    // global order of the listed keys: slice offsets
    const uint32_t *cnts = P.counts + (int64_t)qi * P.slices;
    const int S = P.slices;
    if (t == 0) soff[0] = 0;
    uint32_t run = 0;
    for (int r0 = 0; r0 < S; r0 += kSelThreads) {
        const int sidx = r0 + t;
        const uint32_t c = sidx < S ? cnts[sidx] : 0u;
        uint32_t tot;
        const uint32_t incl = block_scan(c, wsum, &tot);
        if (sidx < S) soff[sidx + 1] = run + incl;
        run += tot;
    }
    __syncthreads();
    const uint32_t L = soff[S];
    const bool in_lds = L <= (uint32_t)kLdsList;
    const uint32_t *lst = P.list + (int64_t)qi * S * kSelSlice * 2;
    // entry j of the global order lives in slice s at position j - soff[s]
    auto entry = [&](uint32_t j, uint32_t *idx, uint32_t *key) {
        if (in_lds) { *idx = lidx[j]; *key = lkey[j]; return; }
        int lo = 0, hi = S;  // find s with soff[s] <= j < soff[s+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (soff[mid] <= j) lo = mid; else hi = mid;
        }
        const uint32_t *e = lst + ((int64_t)lo * kSelSlice + (j - soff[lo])) * 2;
        *idx = e[0];
        *key = e[1];
    };
    if (in_lds) {
        // each thread loads entries j = t, t + kSelThreads, ... of the global order (its slice by
        // binary search over the offsets), all loads issued before any LDS store
        constexpr int kBatch = 8;
        for (uint32_t j0 = 0; j0 < L; j0 += kBatch * kSelThreads) {
            uint2 e[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const uint32_t j = j0 + (uint32_t)u * kSelThreads + t;
                e[u] = make_uint2(0, 0);
                if (j < L) {
                    int lo = 0, hi = S;
                    while (hi - lo > 1) {
                        const int mid = (lo + hi) >> 1;
                        if (soff[mid] <= j) lo = mid; else hi = mid;
                    }
                    e[u] = *(const uint2 *)(lst + ((int64_t)lo * kSelSlice + (j - soff[lo])) * 2);
                }
            }
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const uint32_t j = j0 + (uint32_t)u * kSelThreads + t;
                if (j < L) { lidx[j] = e[u].x; lkey[j] = e[u].y; }
            }
        }
    }
    __syncthreads();

    // radix select of the need-th largest sub-rank (low 20 score bits, inverted index) among
    // the keys of bin T; digits from the top: 10 + 10 score bits, then 11 + 11 + 10 index bits
    const int dig_lo[5] = {42, 32, 21, 10, 0};
    const int dig_w[5] = {10, 10, 11, 11, 10};
    uint64_t prefix = 0, pmask = 0;
    uint32_t rem = need;
    for (int p = 0; p < 5 && need > 0; p++) {
        const int w = dig_w[p], lo_bit = dig_lo[p];
        const int nb = 1 << w;
        for (int i = t; i < nb; i += kSelThreads) hist[i] = 0;
        __syncthreads();
        for (uint32_t j = t; j < L; j += kSelThreads) {
            uint32_t idx, key;
            entry(j, &idx, &key);
            if ((int)(key >> 20) != T) continue;
            const uint64_t v = ((uint64_t)(key & 0xFFFFFu) << 32) | (uint64_t)(~idx);
            if ((v & pmask) == prefix) atomicAdd(&hist[(v >> lo_bit) & (uint64_t)(nb - 1)], 1u);
        }
        __syncthreads();
        int d;
        uint32_t ab;
        top_down_threshold(nb, rem, [&](int bin) { return hist[bin]; }, wsum, &sT, &sAbove, &d, &ab);
        rem -= ab;
        prefix |= (uint64_t)(d < 0 ? 0 : d) << lo_bit;
        pmask |= (uint64_t)(nb - 1) << lo_bit;
    }
    // ordered compaction: keep keys above bin T and keys of bin T with sub-rank >= prefix
    uint32_t written = 0;
    for (uint32_t j0 = 0; j0 < L; j0 += kSelThreads) {
        const uint32_t j = j0 + t;
        bool keep = false;
        uint32_t idx = 0;
        if (j < L) {
            uint32_t key;
            entry(j, &idx, &key);
            const int bin = (int)(key >> 20);
            const uint64_t v = ((uint64_t)(key & 0xFFFFFu) << 32) | (uint64_t)(~idx);
            keep = bin > T || (bin == T && need > 0 && v >= prefix);
        }
        uint32_t tot;
        const uint32_t incl = block_scan(keep ? 1u : 0u, wsum, &tot);
        const uint32_t pos = written + incl - (keep ? 1u : 0u);
        if (keep && pos < k_eff) out[pos] = (int32_t)idx;
        written += tot;
    }
    for (int j = (int)k_eff + t; j < P.k; j += kSelThreads) out[j] = -1;
}

hipError_t launch_select(const SelectArgs &a, const QueryPos &qp, hipStream_t s) {
    if (a.BQ == 0) return hipSuccess;
    SelParams P{};
    P.keys = a.score_keys;
    P.hist = a.hist;
    P.copies = a.hist_copies > 0 ? a.hist_copies : 1;
    P.n_max = a.n_max;
    P.k = a.k;
    P.slices = select_slices(a.n_max);
    P.list = a.list;
    P.counts = a.counts;
    P.meta = a.meta;
    P.out = a.out;
    hipLaunchKernelGGL(select_scan_kernel, dim3((unsigned)P.slices, (unsigned)a.BQ), dim3(kSelThreads), 0, s, P, qp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(select_final_kernel, dim3((unsigned)a.BQ), dim3(kSelThreads), 0, s, P, qp);
    return hipGetLastError();
}

}  // namespace v4a
