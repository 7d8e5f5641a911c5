// topk.hip -- a5: exact top-k selection over the indexer scores.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: each query keeps the
// top-k compressed entries chosen by the lightning indexer (k = 1024 for Pro);
// "DeepSeek V4 preview and technical report" (chooseai.net), section 1: k = 512 for Flash.
//
// Order: score descending, then index ascending (the lowest index wins ties); the selection
// is written in ascending index order, padded with -1.  Equivalently, each key i has the
// distinct 64-bit rank key K = (orderable score key << 32) | ~i and the k largest K win.
//
// Radix select in two levels.  Level 1: the indexer already counted the top 12 bits of every
// score key, so every workgroup of this kernel finds the threshold bin T (the bin in which the
// k-th best key lies) from that histogram.  Each workgroup then scans a slice of the scores:
// keys above T are selected outright, keys in T become candidates.  Level 2: the last
// workgroup to finish (an atomic ticket; no workgroup ever waits for another) resolves the
// candidates exactly with LDS radix passes over the remaining 20 score bits and the 32 index
// bits, gathers the k selected indices and sorts them with an LDS bitonic sort.  Integer
// atomics only count and reserve slots, so the result is independent of scheduling.
#include "common.hpp"

namespace v4a {

constexpr int kSelThreads = 512;
constexpr int kSelSlice = 8192;     // keys scanned per workgroup
constexpr int kBins = 4096;
constexpr int kMaxK = 2048;
constexpr int kLdsCand = 6144;      // candidates cached in LDS for the refinement

struct SelParams {
    const uint32_t *keys;
    const uint32_t *hist;
    int64_t n_max;
    int k;
    uint32_t *cand;
    int64_t cand_cap;
    int32_t *sel;
    uint32_t *counters;
    int32_t *out;
    int slices;
};

// Block-wide: from a histogram (in LDS, nb bins), find the largest bin T with
// count(bins >= T) >= need; return T and count(bins > T) through LDS.
__device__ void find_threshold(const uint32_t *h, int nb, uint32_t need, uint32_t *scratch,
                               int *T_out, uint32_t *above_out) {
    // each thread sums a run of bins; runs are ordered from the top bin down
    const int per = (nb + kSelThreads - 1) / kSelThreads;
    const int t = threadIdx.x;
    const int hi = nb - 1 - t * per;  // this thread's bins: hi, hi-1, ..., hi-per+1
    uint32_t sum = 0;
    for (int j = 0; j < per; j++) {
        int bin = hi - j;
        if (bin >= 0) sum += h[bin];
    }
    scratch[t] = sum;
    __syncthreads();
    // inclusive prefix over threads (thread 0 holds the top run): Hillis-Steele in LDS
    for (int off = 1; off < kSelThreads; off <<= 1) {
        uint32_t v = t >= off ? scratch[t - off] : 0u;
        __syncthreads();
        scratch[t] += v;
        __syncthreads();
    }
    uint32_t before = t ? scratch[t - 1] : 0u;  // count in all higher runs
    if (before < need && scratch[t] >= need) {
        uint32_t c = before;
        for (int j = 0; j < per; j++) {
            int bin = hi - j;
            if (bin < 0) break;
            if (c + h[bin] >= need) {
                *T_out = bin;
                *above_out = c;
                break;
            }
            c += h[bin];
        }
    }
    __syncthreads();
}

__global__ void __launch_bounds__(kSelThreads) select_kernel(SelParams P, QueryPos QP) {
    __shared__ uint32_t sh[kBins];          // level-1 histogram, then radix histograms
    __shared__ uint32_t scan[kSelThreads];
    __shared__ uint32_t cand_k[kLdsCand];   // candidate score keys (low 20 bits)
    __shared__ uint32_t cand_i[kLdsCand];   // candidate indices
    __shared__ int32_t fin[kMaxK];
    __shared__ int s_T;
    __shared__ uint32_t s_above, s_last;

    const int qi = blockIdx.y;
    const int t = threadIdx.x;
    const int64_t n_vis = visible_keys(QP, qi);
    const uint32_t k_eff = (uint32_t)(n_vis < P.k ? n_vis : P.k);
    uint32_t *ctr = P.counters + (int64_t)qi * 4;  // [0] n_sel, [1] n_cand, [2] done
    int32_t *out = P.out + (int64_t)qi * P.k;

    int T = -1;
    uint32_t above = 0;
    if (k_eff > 0) {
        for (int i = t; i < kBins; i += kSelThreads) sh[i] = P.hist[(int64_t)qi * kBins + i];
        if (t == 0) { s_T = -1; s_above = 0; }
        __syncthreads();
        find_threshold(sh, kBins, k_eff, scan, &s_T, &s_above);
        T = s_T;
        above = s_above;

        // scan this workgroup's slice
        const int64_t lo = (int64_t)blockIdx.x * kSelSlice;
        const int64_t hi = lo + kSelSlice < n_vis ? lo + kSelSlice : n_vis;
        const uint32_t *keys = P.keys + (int64_t)qi * P.n_max;
        const int lane = t & 63;
        for (int64_t base = lo; base < hi; base += kSelThreads) {
            const int64_t i = base + t;
            uint32_t key = 0;
            int bin = -1;
            if (i < hi) {
                key = keys[i];
                bin = (int)(key >> 20);
            }
            const bool take = bin > T;
            const bool cnd = bin == T;
            // one atomic per wavefront and category
            const uint64_t mt = __ballot(take), mc = __ballot(cnd);
            const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            uint32_t bt = 0, bc = 0;
            if (lane == 0) {
                if (mt) bt = atomicAdd(&ctr[0], (uint32_t)__popcll(mt));
                if (mc) bc = atomicAdd(&ctr[1], (uint32_t)__popcll(mc));
            }
            bt = __shfl(bt, 0);
            bc = __shfl(bc, 0);
            if (take) {
                const uint32_t slot = bt + __popcll(mt & below);
                if (slot < (uint32_t)P.k) P.sel[(int64_t)qi * P.k + slot] = (int32_t)i;
            }
            if (cnd) {
                const uint64_t slot = bc + __popcll(mc & below);
                if ((int64_t)slot < P.cand_cap) {
                    uint32_t *c = P.cand + ((int64_t)qi * P.cand_cap + (int64_t)slot) * 2;
                    c[0] = key;
                    c[1] = (uint32_t)i;
                }
            }
        }
    }
    // ticket: the last workgroup of this query finishes the selection
    __threadfence();
    __syncthreads();
    if (t == 0) s_last = (atomicAdd(&ctr[2], 1u) == (uint32_t)(gridDim.x - 1)) ? 1u : 0u;
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    if (k_eff == 0) {
        for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
        return;
    }
    // the counts are exact by construction; the clamps only keep every access in bounds
    uint32_t n_sel = __atomic_load_n(&ctr[0], __ATOMIC_RELAXED);
    uint32_t n_cand = __atomic_load_n(&ctr[1], __ATOMIC_RELAXED);
    if (n_sel > k_eff) n_sel = k_eff;
    if ((int64_t)n_cand > P.cand_cap) n_cand = (uint32_t)P.cand_cap;
    const uint32_t need = k_eff - n_sel;  // >= 1 by the choice of T
    const uint32_t *cg = P.cand + (int64_t)qi * P.cand_cap * 2;
    const bool in_lds = n_cand <= (uint32_t)kLdsCand;
    if (in_lds) {
        for (uint32_t j = t; j < n_cand; j += kSelThreads) {
            cand_k[j] = cg[2 * j] & 0xFFFFFu;
            cand_i[j] = cg[2 * j + 1];
        }
    }
    __syncthreads();

    // Level 2: radix select of the need-th largest 52-bit sub-key (score low 20 bits, ~index)
    // among the candidates.  Digits from the top: 10 bits of score, 10 bits of score, then the
    // inverted index in 11, 11, 10 bits.
    const int dig_hi[5] = {51, 41, 31, 20, 9};
    const int dig_w[5] = {10, 10, 11, 11, 10};
    uint64_t prefix = 0, pmask = 0;
    uint32_t rem = need;
    for (int p = 0; p < 5; p++) {
        const int w = dig_w[p], lo_bit = dig_hi[p] - w + 1;
        const int nb = 1 << w;
        for (int i = t; i < nb; i += kSelThreads) sh[i] = 0;
        __syncthreads();
        for (uint32_t j = t; j < n_cand; j += kSelThreads) {
            uint32_t sk, idx;
            if (in_lds) { sk = cand_k[j]; idx = cand_i[j]; }
            else { sk = cg[2 * j] & 0xFFFFFu; idx = cg[2 * j + 1]; }
            const uint64_t v = ((uint64_t)sk << 32) | (uint64_t)(~idx);
            if ((v & pmask) == prefix) atomicAdd(&sh[(v >> lo_bit) & (uint64_t)(nb - 1)], 1u);
        }
        __syncthreads();
        if (t == 0) { s_T = -1; s_above = 0; }
        __syncthreads();
        find_threshold(sh, nb, rem, scan, &s_T, &s_above);
        const int dsel = s_T;
        rem -= s_above;
        prefix |= (uint64_t)dsel << lo_bit;
        pmask |= (uint64_t)(nb - 1) << lo_bit;
        __syncthreads();
    }
    // prefix is now the exact need-th largest sub-key: take candidates >= prefix
    if (t == 0) s_above = 0;
    __syncthreads();
    const int32_t *sel = P.sel + (int64_t)qi * P.k;
    for (uint32_t j = t; j < n_sel; j += kSelThreads) fin[j] = sel[j];
    for (uint32_t j = t; j < n_cand; j += kSelThreads) {
        uint32_t sk, idx;
        if (in_lds) { sk = cand_k[j]; idx = cand_i[j]; }
        else { sk = cg[2 * j] & 0xFFFFFu; idx = cg[2 * j + 1]; }
        const uint64_t v = ((uint64_t)sk << 32) | (uint64_t)(~idx);
        if (v >= prefix) {
            const uint32_t slot = atomicAdd(&s_above, 1u);
            if (n_sel + slot < k_eff) fin[n_sel + slot] = (int32_t)idx;
        }
    }
    __syncthreads();
    // bitonic sort of fin[0..n) ascending, padded to a power of two with INT_MAX
    int n2 = 1;
    while (n2 < (int)k_eff) n2 <<= 1;
    for (int j = (int)k_eff + t; j < n2; j += kSelThreads) fin[j] = 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= n2; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int j = t; j < n2 / 2; j += kSelThreads) {
                const int lo = 2 * j - (j & (stride - 1));
                const int hi = lo + stride;
                const bool up = (lo & size) == 0;
                const int32_t a = fin[lo], c = fin[hi];
                if ((a > c) == up) { fin[lo] = c; fin[hi] = a; }
            }
            __syncthreads();
        }
    }
    for (int j = t; j < P.k; j += kSelThreads) out[j] = j < (int)k_eff ? fin[j] : -1;
}

hipError_t launch_select(const SelectArgs &a, const QueryPos &qp, hipStream_t s) {
    if (a.BQ == 0) return hipSuccess;
    SelParams P{};
    P.keys = a.score_keys;
    P.hist = a.hist;
    P.n_max = a.n_max;
    P.k = a.k;
    P.cand = a.cand;
    P.cand_cap = a.cand_cap;
    P.sel = a.sel;
    P.counters = a.counters;
    P.out = a.out;
    int slices = (int)((a.n_max + kSelSlice - 1) / kSelSlice);
    if (slices < 1) slices = 1;
    P.slices = slices;
    hipLaunchKernelGGL(select_kernel, dim3((unsigned)slices, (unsigned)a.BQ), dim3(kSelThreads), 0, s, P, qp);
    return hipGetLastError();
}

}  // namespace v4a
