// topk.hip -- a5: exact top-k selection over the indexer scores.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: each query keeps the
// top-k compressed entries chosen by the lightning indexer (k = 1024 for Pro);
// "DeepSeek V4 preview and technical report" (chooseai.net), section 1: k = 512 for Flash.
//
// Order: score descending, then index ascending (the lowest index wins ties); the selection
// is written in ascending index order, padded with -1.  Equivalently each key i carries the
// distinct 64-bit rank (orderable score key << 32) | ~i and the k largest ranks win.
//
// The BF16 selector ("DeepSeek-V4 technical report walkthrough", section 3.4: the index score
// kept in BF16) reads 16-bit keys of the scores rounded to BF16; the scan widens each to 32
// bits (key << 16), which orders identically, so everything after the scan is shared.
//
// Radix select in two kernels (the kernel boundary orders the stages; no workgroup waits on
// another and no device-wide fence is needed):
//   scan:     the indexer counted the top 12 bits of every score key (in kHistCopies copies).
//             Each workgroup finds the threshold bin T (the bin holding the k-th best key)
//             from the top of that histogram, then lists, in index order, every key of its
//             slice whose bin is >= T, with its score key.
//   finalize: one workgroup per query reads the listed keys in global index order (slice by
//             slice), finds the exact k-th best score key inside bin T with LDS radix passes
//             over the remaining 20 bits, and compacts the winners in index order (keys equal
//             to the threshold go lowest index first), so the output is ascending without a
//             sort.
#include "compress.hpp"
#include "select_logic.hpp"

namespace v4a {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kLdsList = 12288;   // listed keys the finalize kernel keeps in LDS
constexpr int kMaxSlices = 1024;  // n_max <= 8M keys
constexpr int kSubBins = 1024;    // 10-bit digits of the low 20 score-key bits
constexpr int kSelTPS = 16;       // finalize: fewest threads per slice placing its listed keys
constexpr int kSelSpec = 8;       // finalize: listed keys per thread requested with the counts
constexpr int kRankMax = 64;      // finalize: keys left in the first digit's bin ranked by one wavefront

int select_slices(int64_t n_max) {
    int64_t s = (n_max + kSelSlice - 1) / kSelSlice;
    return (int)(s < 1 ? 1 : s);
}

struct SelParams {
    const void *keys;        // [BQ][key_stride] uint32, or uint16 (BF16 scores)
    int64_t key_stride;
    const uint32_t *hist;    // [BQ][copies][4096]
    int copies;
    int64_t n_max;
    int k, slices;
    bool key16;              // 16-bit keys (listed as key << 16): one 4-bit digit pass
    uint32_t *list;
    uint32_t *counts;
    int32_t *meta;
    int32_t *out;
    CompressParams rec;      // entry records of the decode step (n_rec > 0)
    int n_rec;               // extra workgroups of the final launch: one per sequence
    uint4 *hist_clear;       // with n_rec: the histograms, cleared by those workgroups
    int hist_n16;            // 16-byte words of one query's histograms
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

// Threshold search over a histogram whose bins are held BPT per thread, thread t owning bins
// BPT*t .. BPT*t+BPT-1 (counts c[]): finds the bin T where the count walking down from the top
// bin first reaches `need`, and the count strictly above T.  One block scan: thread t's bins
// sit below everything owned by threads > t.  T = -1 if the histogram holds fewer than need.
template <int BPT>
__device__ __forceinline__ void find_threshold(const uint32_t (&c)[BPT], uint32_t need, uint32_t *wsum, int *sT,
                                               uint32_t *sAbove, int *T, uint32_t *above) {
    const int t = threadIdx.x;
    uint32_t mine = 0;
#pragma unroll
    for (int b = 0; b < BPT; b++) mine += c[b];
    if (t == 0) { *sT = -1; *sAbove = 0; }
    uint32_t tot;
    const uint32_t incl = block_scan(mine, wsum, &tot);
    const uint32_t over = tot - incl;  // held by threads above this one
    int b;
    uint32_t ab;
    if (sel_threshold_in_run<BPT>(c, over, need, &b, &ab)) {
        *sT = BPT * t + b;
        *sAbove = ab;
    }
    __syncthreads();
    *T = *sT;
    *above = *sAbove;
    __syncthreads();
}

// Scan: one workgroup per (slice of kSelSlice keys, query).  The histogram (all copies) is
// read with 16-byte loads in one round, the threshold bin T found with one block scan, and the
// slice's keys whose bin is >= T listed in index order (each thread owns a contiguous run of
// keys; one block scan places the runs).  K16: the keys are 16 bits wide and listed as
// key << 16.
template <bool K16>
__global__ void __launch_bounds__(kSelThreads) select_scan_kernel(SelParams P, QueryPos QP) {
    constexpr int kBPT = kHistBins / kSelThreads;       // 8 bins per thread
    constexpr int kPer = kSelSlice / kSelThreads;       // 16 keys per thread
    static_assert(kBPT == 8, "each thread reads its histogram bins as two 16-byte loads per copy");
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ int sT;
    __shared__ uint32_t sAbove;
    const int qi = blockIdx.y, s = blockIdx.x, t = threadIdx.x;
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
    // this slice's keys are requested first, so their latency overlaps the histogram's
    const int64_t lo = (int64_t)s * kSelSlice;
    const int64_t hi = lo + kSelSlice < n_vis ? lo + kSelSlice : n_vis;
    const int64_t my0 = lo + (int64_t)t * kPer;
    constexpr int kPerLoad = K16 ? 8 : 4;  // keys per 16-byte load
    uint4 kq[kPer / kPerLoad];
#pragma unroll
    for (int r = 0; r < kPer / kPerLoad; r++) {  // rows are padded to a multiple of 64 keys
        const int64_t i = my0 + kPerLoad * r;
        const void *src = K16 ? (const void *)((const uint16_t *)P.keys + (int64_t)qi * P.key_stride + i)
                              : (const void *)((const uint32_t *)P.keys + (int64_t)qi * P.key_stride + i);
        kq[r] = i < hi ? *(const uint4 *)src : make_uint4(0, 0, 0, 0);
    }
    uint32_t c[kBPT];
    {
        const uint32_t *h = P.hist + (int64_t)qi * P.copies * kHistBins + kBPT * t;
        uint4 a = *(const uint4 *)h, b = *(const uint4 *)(h + 4);
        if (kHistCopies > 1 && P.copies > 1) {
            uint4 ha[kHistCopies > 1 ? kHistCopies - 1 : 1], hb[kHistCopies > 1 ? kHistCopies - 1 : 1];
#pragma unroll
            for (int cp = 1; cp < kHistCopies; cp++) {
                ha[cp - 1] = *(const uint4 *)(h + cp * kHistBins);
                hb[cp - 1] = *(const uint4 *)(h + cp * kHistBins + 4);
            }
#pragma unroll
            for (int cp = 0; cp < kHistCopies - 1; cp++) {
                a.x += ha[cp].x; a.y += ha[cp].y; a.z += ha[cp].z; a.w += ha[cp].w;
                b.x += hb[cp].x; b.y += hb[cp].y; b.z += hb[cp].z; b.w += hb[cp].w;
            }
        }
        c[0] = a.x; c[1] = a.y; c[2] = a.z; c[3] = a.w;
        c[4] = b.x; c[5] = b.y; c[6] = b.z; c[7] = b.w;
    }
    int T;
    uint32_t above;
    find_threshold<kBPT>(c, k_eff, wsum, &sT, &sAbove, &T, &above);
    if (s == 0 && t == 0) {
        P.meta[2 * qi] = T;
        P.meta[2 * qi + 1] = (int32_t)above;
    }
    uint32_t kv[kPer];
#pragma unroll
    for (int r = 0; r < kPer / kPerLoad; r++) {
        const uint32_t w4[4] = {kq[r].x, kq[r].y, kq[r].z, kq[r].w};
#pragma unroll
        for (int c = 0; c < 4; c++) {
            if (K16) {
                kv[8 * r + 2 * c] = w4[c] << 16;
                kv[8 * r + 2 * c + 1] = w4[c] & 0xFFFF0000u;
            } else {
                kv[4 * r + c] = w4[c];
            }
        }
    }
    uint32_t mine = 0;
#pragma unroll
    for (int r = 0; r < kPer; r++) mine += (my0 + r < hi && (int)(kv[r] >> 20) >= T) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = block_scan(mine, wsum, &tot) - mine;
    uint32_t *lst = P.list + ((int64_t)qi * P.slices * kSelSlice + lo) * 2;
#pragma unroll
    for (int r = 0; r < kPer; r++) {
        if (my0 + r < hi && (int)(kv[r] >> 20) >= T) {
            *(uint2 *)(lst + 2 * pos) = make_uint2((uint32_t)(my0 + r), kv[r]);
            pos++;
        }
    }
    if (t == 0) *cnt = tot;
}

// Finalize: one workgroup per query.  The listed keys are read in global index order (slice
// by slice) into LDS.  Inside bin T two 10-bit digit passes find the exact threshold score
// key S* and how many keys equal to it are still needed (rem); the ordered compaction then
// keeps every key above S* and the first rem keys equal to S* in index order (the lowest
// indices win the tie).  One block scan places every kept key.
//
// With n_rec > 0 the launch also carries the decode step's record compression: workgroup
// BQ + b compresses, with its first wavefront, the entry record that sequence b's newest token
// completes (one query per sequence), overlapping the selection; attention reads the records
// after this launch.  Its other wavefronts clear query b's histograms (hist_clear): the scan
// kernel, their only reader, has finished, and the next call finds them clear.
__global__ void __launch_bounds__(kSelThreads) select_final_kernel(SelParams P, QueryPos QP) {
    __shared__ uint32_t wsum[kSelWaves];
    __shared__ int sT;
    __shared__ uint32_t sAbove;
    __shared__ uint32_t hist[kSubBins];
    __shared__ uint32_t lidx[kLdsList];
    __shared__ uint32_t lkey[kLdsList];
    __shared__ uint32_t soff[kMaxSlices + 1];
    __shared__ uint32_t cand[kRankMax];
    __shared__ uint32_t n_cand, r_sub, r_rem;
    const int BQ = (int)gridDim.x - P.n_rec;
    if ((int)blockIdx.x >= BQ) {
        // sequence b, whose QP.Q queries (its new tokens) are queries b*Q .. b*Q+Q-1
        const int b = (int)blockIdx.x - BQ, Q = QP.Q;
        if (threadIdx.x >= 64) {  // one wavefront per record; the others clear the histograms
            if (P.hist_clear) {
                uint4 *h = P.hist_clear + (int64_t)b * Q * P.hist_n16;
                for (int j = (int)threadIdx.x - 64; j < Q * P.hist_n16; j += kSelThreads - 64) h[j] = make_uint4(0, 0, 0, 0);
            }
            return;
        }
        const int m = P.rec.m;
        float *scratch = (float *)hist;  // kMaxCand floats; this workgroup does no selection
        for (int j = 0; j < Q; j++) {  // Q <= m: at most one of the tokens completes a block
            const int64_t pos = query_pos(QP, b * Q + j);
            if ((pos + 1) % m != 0) continue;  // no block completed by this token
            const int64_t i = (pos + 1) / m - 1;
            if (P.rec.D == 512 && entry_two_phase(P.rec)) {
                // every candidate row requested at once, then merged and finished bitwise as
                // compress_entry would: a shorter serial chain for the one wavefront
                KeyPrefetch<8> kr;
                key_prefetch<8>(P.rec, b, i, (int64_t)m * (i - 1), kr);
                prefetched_entry_finish<8>(P.rec, kr, b, i, nullptr, 0);
            } else if (P.rec.D == 512) {
                compress_entry<8>(P.rec, scratch, b, i, (int64_t)m * (i - 1));
            } else {
                compress_entry<2>(P.rec, scratch, b, i, (int64_t)m * (i - 1));
            }
        }
        return;
    }
    const int qi = blockIdx.x, t = threadIdx.x;
    const int64_t n_vis = visible_keys(QP, qi);
    const uint32_t k_eff = (uint32_t)(n_vis < P.k ? n_vis : P.k);
    int32_t *out = P.out + (int64_t)qi * P.k;
    if (k_eff == 0) {
        for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
        return;
    }
    // global order of the listed keys: slice offsets, then the keys themselves into LDS
    const uint32_t *cnts = P.counts + (int64_t)qi * P.slices;
    const int S = P.slices;
    const uint32_t *lst = P.list + (int64_t)qi * S * kSelSlice * 2;
    // Up to 32 slices: tps threads per slice (512 over the slice count rounded up to a power of
    // two, at least kSelTPS) request its count and its first tps * kSelSpec listed keys at once
    // (slots past the count lie inside the slice's list region and are dropped), before the
    // scan's threshold is read, so counts, keys and threshold take one memory round trip
    const bool few_slices = S <= kSelThreads / kSelTPS;
    int tps = kSelThreads;
    while (tps > kSelTPS && tps * S > kSelThreads) tps >>= 1;
    const int sl = t / tps, p0 = t % tps;
    const bool live = few_slices && sl < S;
    const uint32_t c_raw = live ? cnts[sl] : 0u;
    const uint32_t *ls = lst + (int64_t)(live ? sl : 0) * kSelSlice * 2;
    uint2 e[kSelSpec];
#pragma unroll
    for (int u = 0; u < kSelSpec; u++) {
        const int pos = p0 + tps * u;  // < kSelSlice: inside the slice's list region
        e[u] = live ? *(const uint2 *)(ls + 2 * pos) : make_uint2(0, 0);
    }
    const int T = P.meta[2 * qi];
    const uint32_t above = (uint32_t)P.meta[2 * qi + 1];
    // the scan's result is trusted only if it is consistent (a threshold bin, fewer than k_eff
    // keys above it); otherwise nothing is selected rather than reading past a list
    if (!sel_meta_consistent(T, above, k_eff)) {  // uniform over the workgroup
        for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
        return;
    }
    const uint32_t need = k_eff - above;  // >= 1: keys still to take from bin T
    // the first digit pass: bits 10..19 of the keys in bin T (bits 16..19 of widened 16-bit keys)
    const int shift0 = P.key16 ? 16 : 10;
    const uint32_t dmask0 = P.key16 ? 15u : (uint32_t)(kSubBins - 1);
    bool hist0 = false;  // the first pass's histogram was counted while the keys were placed
    uint32_t L;
    if (few_slices) {
        // one block scan of the counts requested above places every key
        const uint32_t c = live ? sel_clamp_count(c_raw, (uint32_t)kSelSlice) : 0u;
        for (int i = t; i < kSubBins; i += kSelThreads) hist[i] = 0;
        uint32_t tot;
        const uint32_t mine = (live && p0 == 0) ? c : 0u;
        const uint32_t off = block_scan(mine, wsum, &tot) - c;  // the slice's first position (its barriers also order the clear)
        if (live && p0 == 0) soff[sl] = off;
        if (t == 0) soff[S] = tot;
        L = tot;
        if (L <= (uint32_t)kLdsList) {
            hist0 = true;
            auto put = [&](uint32_t pos, uint2 v) {
                lidx[off + pos] = v.x;
                lkey[off + pos] = v.y;
                if ((int)(v.y >> 20) == T) atomicAdd(&hist[(v.y >> shift0) & dmask0], 1u);
            };
#pragma unroll
            for (int u = 0; u < kSelSpec; u++) {
                const uint32_t pos = (uint32_t)(p0 + tps * u);
                if (live && pos < c) put(pos, e[u]);
            }
            // a slice that listed more keys than were requested: further rounds of kSelSpec
            // loads per thread, all issued before any is placed
            for (uint32_t pos0 = (uint32_t)(p0 + tps * kSelSpec); live && pos0 < c; pos0 += (uint32_t)(tps * kSelSpec)) {
                uint2 e2[kSelSpec];
#pragma unroll
                for (int u = 0; u < kSelSpec; u++) {
                    const uint32_t pos = pos0 + (uint32_t)(tps * u);
                    e2[u] = pos < c ? *(const uint2 *)(ls + 2 * pos) : make_uint2(0, 0);
                }
#pragma unroll
                for (int u = 0; u < kSelSpec; u++) {
                    const uint32_t pos = pos0 + (uint32_t)(tps * u);
                    if (pos < c) put(pos, e2[u]);
                }
            }
        }
        __syncthreads();
    } else {
        if (t == 0) soff[0] = 0;
        uint32_t run = 0;
        for (int r0 = 0; r0 < S; r0 += kSelThreads) {
            const int sidx = r0 + t;
            const uint32_t c = sidx < S ? sel_clamp_count(cnts[sidx], (uint32_t)kSelSlice) : 0u;
            uint32_t tot;
            const uint32_t incl = block_scan(c, wsum, &tot);
            if (sidx < S) soff[sidx + 1] = run + incl;
            run += tot;
        }
        __syncthreads();
        L = soff[S];
    }
    const bool in_lds = L <= (uint32_t)kLdsList;
    // entry j of the global order lives in slice s at position j - soff[s]
    auto fetch = [&](uint32_t j) -> uint2 {
        int lo = 0, hi = S;  // s with soff[s] <= j < soff[s+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (soff[mid] <= j) lo = mid; else hi = mid;
        }
        return *(const uint2 *)(lst + ((int64_t)lo * kSelSlice + (j - soff[lo])) * 2);
    };
    auto entry = [&](uint32_t j, uint32_t *idx, uint32_t *key) {
        if (in_lds) { *idx = lidx[j]; *key = lkey[j]; return; }
        const uint2 e = fetch(j);
        *idx = e.x;
        *key = e.y;
    };
    if (in_lds && !hist0) {
        // all loads of a batch are issued before any LDS store
        constexpr int kBatch = 8;
        for (uint32_t j0 = 0; j0 < L; j0 += kBatch * kSelThreads) {
            uint2 e[kBatch];
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const uint32_t j = j0 + (uint32_t)u * kSelThreads + t;
                e[u] = j < L ? fetch(j) : make_uint2(0, 0);
            }
#pragma unroll
            for (int u = 0; u < kBatch; u++) {
                const uint32_t j = j0 + (uint32_t)u * kSelThreads + t;
                if (j < L) { lidx[j] = e[u].x; lkey[j] = e[u].y; }
            }
        }
        __syncthreads();
    }

    // digit passes over the low 20 bits of the keys in bin T: bits 10..19, then 0..9; keys
    // widened from 16 bits hold only bits 16..19 below the bin, one pass
    uint32_t rem = need, sub = 0, sub_mask = 0;
    const int n_pass = P.key16 ? 1 : 2;
    for (int p = 0; p < n_pass; p++) {
        const int shift = P.key16 ? 16 : (p == 0 ? 10 : 0);
        const uint32_t dmask = P.key16 ? 15u : (uint32_t)(kSubBins - 1);
        if (p > 0 || !hist0) {
            for (int i = t; i < kSubBins; i += kSelThreads) hist[i] = 0;
            __syncthreads();
            for (uint32_t j = t; j < L; j += kSelThreads) {
                uint32_t idx, key;
                entry(j, &idx, &key);
                if ((int)(key >> 20) == T && (key & sub_mask) == sub) atomicAdd(&hist[(key >> shift) & dmask], 1u);
            }
            __syncthreads();
        }
        uint32_t c[kSubBins / kSelThreads];
#pragma unroll
        for (int b = 0; b < kSubBins / kSelThreads; b++) c[b] = hist[(kSubBins / kSelThreads) * t + b];
        int d;
        uint32_t ab;
        find_threshold<kSubBins / kSelThreads>(c, rem, wsum, &sT, &sAbove, &d, &ab);
        if (d < 0) {  // fewer listed keys in bin T than the scan promised: select nothing (uniform)
            for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
            return;
        }
        rem -= ab;
        sub |= (uint32_t)d << shift;
        sub_mask |= dmask << shift;
        if (p == 0 && n_pass == 2 && hist[d] <= (uint32_t)kRankMax) {
            // few keys share the first digit (bits 10..19): instead of a second histogram pass
            // they are gathered and one wavefront ranks them; the rem-th largest of them (with
            // repeats) is the threshold key, and rem becomes the count of its equals still
            // needed, as the second pass would leave them
            const uint32_t nd = hist[d];
            if (t == 0) {
                n_cand = 0;
                r_rem = 0;
            }
            __syncthreads();
            const uint32_t pre = (((uint32_t)T << 20) | sub) >> 10;
            for (uint32_t j = t; j < L; j += kSelThreads) {
                uint32_t idx, key;
                entry(j, &idx, &key);
                if ((key >> 10) == pre) {
                    const uint32_t slot = atomicAdd(&n_cand, 1u);
                    if (slot < (uint32_t)kRankMax) cand[slot] = key;
                }
            }
            __syncthreads();
            if (t < 64) {
                const uint32_t n = min(min(n_cand, nd), (uint32_t)kRankMax);
                const uint32_t x = (uint32_t)t < n ? cand[t] : 0u;
                uint32_t gt = 0, ge = 0;
                for (uint32_t q = 0; q < n; q++) {
                    const uint32_t y = cand[q];
                    gt += y > x ? 1u : 0u;
                    ge += y >= x ? 1u : 0u;
                }
                if ((uint32_t)t < n && gt < rem && rem <= ge) {  // every such lane holds the same key
                    r_sub = x & (uint32_t)(kSubBins - 1);
                    r_rem = rem - gt;
                }
            }
            __syncthreads();
            if (r_rem == 0) {  // the gathered keys do not hold the rem-th: select nothing (uniform)
                for (int j = t; j < P.k; j += kSelThreads) out[j] = -1;
                return;
            }
            sub |= r_sub;
            rem = r_rem;
            break;
        }
    }
    const uint32_t tkey = ((uint32_t)T << 20) | sub;  // the k_eff-th best score key
    // ordered compaction: thread t owns a contiguous run of the global order; keys > tkey are
    // kept, keys == tkey are kept while fewer than rem of them come earlier
    const uint32_t per = (L + kSelThreads - 1) / kSelThreads;
    const uint32_t j0 = per * (uint32_t)t, j1 = min(L, j0 + per);
    uint32_t n_gt = 0, n_eq = 0;
    for (uint32_t j = j0; j < j1; j++) {
        uint32_t idx, key;
        entry(j, &idx, &key);
        n_gt += key > tkey ? 1u : 0u;
        n_eq += key == tkey ? 1u : 0u;
    }
    uint32_t tot;
    const uint32_t incl = block_scan((n_eq << 16) | n_gt, wsum, &tot);  // both counts < 2^16 when in LDS
    uint32_t gt_before, eq_before;
    if (in_lds) {
        gt_before = (incl & 0xFFFFu) - n_gt;
        eq_before = (incl >> 16) - n_eq;
    } else {
        // long lists: two separate scans (counts may exceed 16 bits)
        uint32_t t1, t2;
        gt_before = block_scan(n_gt, wsum, &t1) - n_gt;
        eq_before = block_scan(n_eq, wsum, &t2) - n_eq;
    }
    // the LDS form has a loop of its own: a global read in the loop (the long-list form) would
    // make every iteration wait for the previous iteration's store as well
    if (in_lds) {
        for (uint32_t j = j0; j < j1; j++) {
            const uint32_t idx = lidx[j], key = lkey[j];
            const int p = sel_place(key, tkey, rem, k_eff, &gt_before, &eq_before);
            if (p >= 0) out[p] = (int32_t)idx;
        }
    } else {
        for (uint32_t j = j0; j < j1; j++) {
            const uint2 e = fetch(j);
            const int p = sel_place(e.y, tkey, rem, k_eff, &gt_before, &eq_before);
            if (p >= 0) out[p] = (int32_t)e.x;
        }
    }
    for (int j = (int)k_eff + t; j < P.k; j += kSelThreads) out[j] = -1;
}

hipError_t launch_select(const SelectArgs &a, const QueryPos &qp, hipStream_t s) {
    if (a.BQ == 0) return hipSuccess;
    SelParams P{};
    P.keys = a.score_keys;
    P.key_stride = a.key_stride;
    P.hist = a.hist;
    P.copies = a.hist_copies > 0 ? a.hist_copies : 1;
    P.n_max = a.n_max;
    P.k = a.k;
    P.key16 = a.key16;
    P.slices = select_slices(a.n_max);
    P.list = a.list;
    P.counts = a.counts;
    P.meta = a.meta;
    P.out = a.out;
    if (a.key16)
        V4A_LAUNCH("select_scan_kernel", select_scan_kernel<true>, dim3((unsigned)P.slices, (unsigned)a.BQ), dim3(kSelThreads), 0, s,
                           P, qp);
    else
        V4A_LAUNCH("select_scan_kernel", select_scan_kernel<false>, dim3((unsigned)P.slices, (unsigned)a.BQ), dim3(kSelThreads), 0, s,
                           P, qp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.rec) {  // one workgroup per sequence, whose Q queries are its new tokens
        if (qp.Q < 1 || a.BQ % qp.Q != 0 || qp.Q > a.rec->m) return hipErrorInvalidValue;
        P.rec = compress_params(*a.rec);
        P.n_rec = a.BQ / qp.Q;
        P.hist_clear = (uint4 *)a.hist_clear;
        P.hist_n16 = P.copies * kHistBins / 4;  // one query's histograms
    } else if (a.hist_clear) {
        return hipErrorInvalidValue;
    }
    V4A_LAUNCH("select_final_kernel", select_final_kernel, dim3((unsigned)(a.BQ + P.n_rec)), dim3(kSelThreads), 0, s, P, qp);
    return hipGetLastError();
}

}  // namespace v4a
