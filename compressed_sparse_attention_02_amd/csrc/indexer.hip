// indexer.hip -- a4: lightning-indexer scores.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: a low-rank,
// low-precision multi-head indexer scores the compressed entries so each query can keep its
// top-k; section 3.4: its QK path runs in FP4 (MXFP4).
//
// Score of key i for one query: s_h = q_h . key_i for each indexer head h, then
// score = sum_h w_h * ReLU(s_h) as four fp32 fma chains (chain (h>>2)&3 over ascending h)
// combined as ((c0+c1)+c2)+c3 with -0 made +0.
//
// MXFP4 kernel (the decode hot loop, HBM-bound at 68 bytes per key): one workgroup of four
// wavefronts scores a contiguous chunk of keys for one query.  Per group of 16 keys a
// wavefront issues one scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 per 16 heads: heads
// are the A rows, keys the B columns, and each lane holds exactly one 32-element MX block
// (16 bytes of E2M1 codes) with its own E8M0 scale, so a 64-lane load of 16 bytes per lane
// reads the group's 1 KB of codes contiguously.  The MFMA sums exact E2M1 products in fp32;
// on N(0,1)-like data every per-head dot is an fp32 number, so the result does not depend
// on the order of the hardware's accumulation.  The output layout puts heads 16g+4q+i
// (i = 0..3) of key l%16 in lane l with q = l/16: lane group q holds exactly fma chain q,
// so each lane runs its chain in registers (16 fmas) and three cross-lane reads finish
// the fixed-order sum.
//
// Each score is written as an orderable key (larger score -> larger key): 32 bits of the fp32
// score, or 16 bits of the score rounded to BF16 for the BF16 selector.  Its top 12 bits are
// counted in a 4096-bin histogram (LDS per workgroup, then one global atomic add per
// non-empty bin), which the top-k select uses to find the threshold bin.
#include "compress.hpp"

namespace v4a {

constexpr int kGroupsPerIter = 4;   // key groups of 16 per load batch (two batches in flight)
constexpr int kMaxKeysPerWG = 4 * 64 * 16;  // 4 wavefronts x at most 64 groups of 16 keys
struct IndexerParams {
    const uint8_t *kc;   // key codes [B][cap][d/2]
    const uint8_t *ks;   // key scales [B][cap][d/32]
    const float *kf;     // fp32 keys [B][cap][d]
    int64_t kcap;
    const uint8_t *qc;
    const uint8_t *qs;
    const float *qf;
    int64_t qcap;
    const float *w;      // [B*Q][H_I]
    int H, d;
    int64_t n_max;
    int64_t key_stride;
    void *score_keys;      // [BQ][key_stride] uint32, or uint16 when key16; or NULL
    bool key16;
    float *scores;         // [BQ][n_max] or NULL
    uint32_t *hist;        // [BQ][hist_copies][4096] or NULL
    int hist_copies;
    int groups_per_wave;   // key groups of 16 per wavefront (a multiple of kGroupsPerIter)
    bool key_rec;          // decode step (one query per sequence, d = 128): the key that the
    CompressParams key;    // query's newest token completes is compressed here (see below)
};
static_assert(sizeof(IndexerParams) + sizeof(QueryPos) <= 4096, "kernel arguments");

__device__ __forceinline__ void emit_score(const IndexerParams &P, int qi, int64_t i, float score,
                                           uint32_t *lhist) {
    if (score == 0.0f) score = 0.0f;  // -0 -> +0
    if (P.scores) P.scores[(int64_t)qi * P.n_max + i] = score;
    if (P.key16) {
        const uint32_t key = score_key16(score);
        if (P.score_keys) ((uint16_t *)P.score_keys)[(int64_t)qi * P.key_stride + i] = (uint16_t)key;
        if (lhist) atomicAdd(&lhist[key >> 4], 1u);
    } else {
        const uint32_t key = score_key(score);
        if (P.score_keys) ((uint32_t *)P.score_keys)[(int64_t)qi * P.key_stride + i] = key;
        if (lhist) atomicAdd(&lhist[key >> 20], 1u);
    }
}

// Workgroup barrier that orders LDS only: each wavefront waits for its own LDS operations, not
// for its global stores, whose latency then overlaps what follows.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Adds the workgroup's LDS histogram into copy (blockIdx.x % hist_copies) of the query's
// global histogram; spreading the copies keeps many workgroups off the same hot bins.  The
// score stores before it need not have completed.
__device__ __forceinline__ void flush_hist(const IndexerParams &P, int qi, uint32_t *lhist) {
    lds_barrier();
    if (!P.hist) return;
    uint32_t *gh = P.hist + ((int64_t)qi * P.hist_copies + (int)(blockIdx.x % (unsigned)P.hist_copies)) * kHistBins;
    // consecutive bins in consecutive lanes, so the few hot bins of a query leave in one wide
    // atomic instruction per cache line; all LDS reads are issued before the first atomic
    constexpr int kPer = 16;  // bins per thread with 256 threads
    if (blockDim.x * kPer == kHistBins) {
        uint32_t c[kPer];
#pragma unroll
        for (int i = 0; i < kPer; i++) c[i] = lhist[threadIdx.x + i * 256];
#pragma unroll
        for (int i = 0; i < kPer; i++)
            if (c[i]) atomicAdd(&gh[threadIdx.x + i * 256], c[i]);
        return;
    }
    for (int bin = threadIdx.x; bin < kHistBins; bin += blockDim.x) {
        uint32_t c = lhist[bin];
        if (c) atomicAdd(&gh[bin], c);
    }
}

// MXFP4, d = 128 (one 16x16x128 scaled MFMA per 16 heads and 16 keys), H <= 64.
// A workgroup scores 64 * groups_per_wave consecutive keys; wavefront wv owns groups_per_wave
// groups of 16 keys and processes them kGroupsPerIter at a time: every load of an iteration is issued
// before the first MFMA (out-of-range lanes read a clamped, valid key and are masked after),
// so kGroupsPerIter * 1 KB per wavefront is in flight.
//
// With key_rec (the decode step), the wavefront whose keys include the entry that the query's
// newest token completes also compresses that entry's indexer key: it requests the candidate
// rows before its first key batch, scores its range as usual (reading that entry's stale cache
// row), then merges and encodes the key, writes it to the cache and, through LDS, scores it
// with the same arithmetic, replacing the stale score before any score leaves the workgroup.
// The key is bitwise the one the compressor kernel would write, so is its score.
template <bool KEYREC>
__global__ void __launch_bounds__(256) indexer_mxfp4_kernel(IndexerParams P, QueryPos QP) {
    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(16))) float sbuf[kMaxKeysPerWG];  // this workgroup's scores
    __shared__ __attribute__((aligned(16))) uint8_t knew[80];           // the new key's codes + scales
    const int qi = blockIdx.y;
    const int b = qi / QP.Q;
    const int64_t n_vis = visible_keys(QP, qi);
    const int64_t keys_per_wg = (int64_t)4 * P.groups_per_wave * 16;
    const int64_t k0 = (int64_t)blockIdx.x * keys_per_wg;
    if (k0 >= n_vis) return;  // uniform over the workgroup

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;  // col: head/key within 16; grp: MX block / chain

    const uint8_t *kc = P.kc + (int64_t)b * P.kcap * 64;
    const uint8_t *ks = P.ks + (int64_t)b * P.kcap * 4;
    const int64_t kend = k0 + keys_per_wg < n_vis ? k0 + keys_per_wg : n_vis;
    uint32_t *hist = P.hist ? lhist : nullptr;
    const int64_t wbase = k0 + (int64_t)wv * P.groups_per_wave * 16;
    const int n_it = P.groups_per_wave / kGroupsPerIter;

    // the new key of this query (decode step), owned by the wavefront whose range holds it
    int64_t i_new = -1;
    if (KEYREC) {
        const int64_t pos = QP.pos[qi];
        if ((pos + 1) % P.key.m == 0) i_new = (pos + 1) / P.key.m - 1;
    }
    const int64_t wend = wbase + (int64_t)P.groups_per_wave * 16;
    const bool own = KEYREC && i_new >= wbase && i_new < (wend < kend ? wend : kend);  // uniform over the wavefront
    KeyPrefetch<2> kp;
    if (own) key_prefetch<2>(P.key, qi, i_new, (int64_t)P.key.m * (i_new - 1), kp);

    // Double-buffered: the loads of iteration it+1 are issued before iteration it is computed.
    // Lanes past the end read a clamped, valid key of this query and are masked afterwards.
    auto load_iter = [&](int it, uint4 (&kd)[kGroupsPerIter], uint32_t (&ksc)[kGroupsPerIter]) {
        const int64_t base = wbase + (int64_t)it * kGroupsPerIter * 16;
#pragma unroll
        for (int u = 0; u < kGroupsPerIter; u++) {
            int64_t key = base + 16 * u + col;
            key = key < kend ? key : kend - 1;
            const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(kc + key * 64 + grp * 16));
            kd[u] = make_uint4(v.x, v.y, v.z, v.w);
            ksc[u] = *(const uint32_t *)(ks + key * 4);
        }
    };
    // the first key batch is requested before the query, so the two latencies overlap
    uint4 kdA[kGroupsPerIter], kdB[kGroupsPerIter];
    uint32_t kscA[kGroupsPerIter], kscB[kGroupsPerIter];
    if (wbase < kend) load_iter(0, kdA, kscA);
    for (int bin = threadIdx.x; bin < kHistBins; bin += 256) lhist[bin] = 0;

    // query: 4 head groups of 16 heads; lane holds head 16g+col, MX block grp.  Heads past H
    // read head H-1 (all loads issued together) and are zeroed: code 0 and weight 0.
    v8i qa[4];
    int qscale[4];
    float wt[4][4];  // w of heads 16g + 4*grp + i
    {
        uint4 qc[4];
        uint32_t qsb[4];
        float wr[4][4];
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const int h = min(16 * g + col, P.H - 1);
            const int64_t row = (int64_t)b * P.qcap + (int64_t)(qi % QP.Q) * P.H + h;
            qc[g] = *(const uint4 *)(P.qc + row * 64 + grp * 16);
            qsb[g] = P.qs[row * 4 + grp];
#pragma unroll
            for (int i = 0; i < 4; i++) wr[g][i] = P.w[(int64_t)qi * P.H + min(16 * g + 4 * grp + i, P.H - 1)];
        }
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const bool on = 16 * g + col < P.H;
            qa[g] = v8i{on ? (int)qc[g].x : 0, on ? (int)qc[g].y : 0, on ? (int)qc[g].z : 0, on ? (int)qc[g].w : 0,
                        0, 0, 0, 0};
            qscale[g] = on ? (int)qsb[g] : 127;
#pragma unroll
            for (int i = 0; i < 4; i++) wt[g][i] = (16 * g + 4 * grp + i < P.H) ? wr[g][i] : 0.0f;
        }
    }
    __syncthreads();

    // fma chain grp of key col of a group (codes kdu, the key's four scale bytes kscu)
    auto key_chain = [&](const uint4 &kdu, uint32_t kscu) -> float {
        const v8i kb = v8i{(int)kdu.x, (int)kdu.y, (int)kdu.z, (int)kdu.w, 0, 0, 0, 0};
        const int sc = (int)((kscu >> (8 * grp)) & 0xFFu);
        v4f acc[4];
#pragma unroll
        for (int g = 0; g < 4; g++)
            acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[g], kb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0,
                                                                      qscale[g], 0, sc);
        // ReLU on the bit pattern: a finite float is negative (or -0) exactly when its bits
        // read as a negative int, so max(int bits, 0) gives s for s > 0 and +0 otherwise
        float cu = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; g++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float si = acc[g][i];  // a scalar copy: bit casts read whole objects
                const float r = __builtin_bit_cast(float, max(__builtin_bit_cast(int, si), 0));
                cu = fmaf(wt[g][i], r, cu);
            }
        }
        return cu;
    };
    auto compute_iter = [&](int it, const uint4 (&kd)[kGroupsPerIter], const uint32_t (&ksc)[kGroupsPerIter]) {
        const int64_t base = wbase + (int64_t)it * kGroupsPerIter * 16;
        float c[kGroupsPerIter];
#pragma unroll
        for (int u = 0; u < kGroupsPerIter; u++) c[u] = key_chain(kd[u], ksc[u]);
        // the four chains of each key sit in lanes col, col+16, col+32, col+48
        float c1[kGroupsPerIter], c2[kGroupsPerIter], c3[kGroupsPerIter];
#pragma unroll
        for (int u = 0; u < kGroupsPerIter; u++) {
            c1[u] = __shfl_down(c[u], 16);
            c2[u] = __shfl_down(c[u], 32);
            c3[u] = __shfl_down(c[u], 48);
        }
        if (grp == 0) {
#pragma unroll
            for (int u = 0; u < kGroupsPerIter; u++) {
                float sc = ((c[u] + c1[u]) + c2[u]) + c3[u];
                if (sc == 0.0f) sc = 0.0f;  // -0 -> +0
                sbuf[base - k0 + 16 * u + col] = sc;  // slots past kend are never read
            }
        }
    };
    // the new key: merged, encoded (into LDS) and scored right after the first iteration, while
    // the rest of the stream is in flight; its score replaces the stale one after the stream
    float sc_new = 0.0f;
    auto new_key = [&]() {
        key_finish<2>(P.key, kp, qi, i_new, knew, false);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // every key column of the group holds the new key; the chains meet as in compute_iter
        const float c = key_chain(*(const uint4 *)(knew + 16 * grp), *(const uint32_t *)(knew + 64));
        float sc = ((lane_value(c, 0) + lane_value(c, 16)) + lane_value(c, 32)) + lane_value(c, 48);
        if (sc == 0.0f) sc = 0.0f;  // -0 -> +0
        sc_new = sc;
    };
    for (int it = 0; it < n_it; it += 2) {
        if (wbase + (int64_t)it * kGroupsPerIter * 16 >= kend) break;  // uniform over the wavefront
        const bool more1 = it + 1 < n_it && wbase + (int64_t)(it + 1) * kGroupsPerIter * 16 < kend;
        if (more1) load_iter(it + 1, kdB, kscB);
        compute_iter(it, kdA, kscA);
        if (own && it == 0) new_key();
        if (!more1) break;
        const bool more2 = it + 2 < n_it && wbase + (int64_t)(it + 2) * kGroupsPerIter * 16 < kend;
        if (more2) load_iter(it + 2, kdA, kscA);
        compute_iter(it + 1, kdB, kscB);
    }
    if (own) {
        if (lane == 0) sbuf[i_new - k0] = sc_new;
        // the key's cache row (64 code bytes, 4 scale bytes) from its LDS copy; global stores
        // wait until here since they would hold up the stream's loads (one shared counter)
        const int64_t row = P.key.out_row0 + (int64_t)qi * P.key.cap + i_new;
        if (lane < 16) ((uint32_t *)((uint8_t *)P.key.idx.codes + row * 64))[lane] = ((const uint32_t *)knew)[lane];
        if (lane == 16) *(uint32_t *)(P.key.idx.scales + row * 4) = *(const uint32_t *)(knew + 64);
    }
    // the streaming loop touched only registers and LDS; now the scores leave in 16-byte stores
    // and the histogram is counted from LDS
    __syncthreads();
    const int n_here = (int)(kend - k0);
    float *g_sc = P.scores ? P.scores + (int64_t)qi * P.n_max + k0 : nullptr;
    uint32_t *g_key = P.score_keys && !P.key16 ? (uint32_t *)P.score_keys + (int64_t)qi * P.key_stride + k0 : nullptr;
    uint16_t *g_key16 = P.score_keys && P.key16 ? (uint16_t *)P.score_keys + (int64_t)qi * P.key_stride + k0 : nullptr;
    const int hshift = P.key16 ? 4 : 20;  // the top 12 bits of either key
    const bool sc_aligned = ((k0 + (int64_t)qi * P.n_max) & 3) == 0;
    for (int i0 = 4 * threadIdx.x; i0 < n_here; i0 += 4 * 256) {
        const float4 v = *(const float4 *)(sbuf + i0);
        const float vv[4] = {v.x, v.y, v.z, v.w};
        uint32_t kk[4];
#pragma unroll
        for (int j = 0; j < 4; j++) kk[j] = P.key16 ? score_key16(vv[j]) : score_key(vv[j]);
        const bool whole = i0 + 4 <= n_here;
        // rows are padded to a multiple of 64 keys and k0 is a multiple of 4
        if (g_key) {
            if (whole) {
                *(uint4 *)(g_key + i0) = make_uint4(kk[0], kk[1], kk[2], kk[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (i0 + j < n_here) g_key[i0 + j] = kk[j];
            }
        }
        if (g_key16) {
            if (whole) {
                *(uint2 *)(g_key16 + i0) = make_uint2(kk[0] | (kk[1] << 16), kk[2] | (kk[3] << 16));
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (i0 + j < n_here) g_key16[i0 + j] = (uint16_t)kk[j];
            }
        }
        if (g_sc) {
            if (whole && sc_aligned) {
                *(float4 *)(g_sc + i0) = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++)
                    if (i0 + j < n_here) g_sc[i0 + j] = vv[j];
            }
        }
        if (hist) {
#pragma unroll
            for (int j = 0; j < 4; j++)
                if (i0 + j < n_here) atomicAdd(&lhist[kk[j] >> hshift], 1u);
        }
    }
    flush_hist(P, qi, lhist);
}

// fp32 keys and queries: one thread per key; per head an fma chain over ascending dims.
__global__ void __launch_bounds__(256) indexer_f32_kernel(IndexerParams P, QueryPos QP) {
    __shared__ uint32_t lhist[kHistBins];
    const int qi = blockIdx.y;
    const int b = qi / QP.Q;
    const int64_t n_vis = visible_keys(QP, qi);
    const int64_t k0 = (int64_t)blockIdx.x * 256;
    if (k0 >= n_vis) return;
    for (int bin = threadIdx.x; bin < kHistBins; bin += 256) lhist[bin] = 0;
    __syncthreads();
    const int64_t i = k0 + threadIdx.x;
    if (i < n_vis) {
        const float *key = P.kf + ((int64_t)b * P.kcap + i) * P.d;
        const float *q = P.qf + ((int64_t)b * P.qcap + (int64_t)(qi % QP.Q) * P.H) * P.d;
        const float *w = P.w + (int64_t)qi * P.H;
        float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int h = 0; h < P.H; h++) {
            float acc = 0.0f;
            for (int e = 0; e < P.d; e++) acc = fmaf(q[h * P.d + e], key[e], acc);
            const float r = acc > 0.0f ? acc : 0.0f;
            c[(h >> 2) & 3] = fmaf(w[h], r, c[(h >> 2) & 3]);
        }
        emit_score(P, qi, i, ((c[0] + c[1]) + c[2]) + c[3], P.hist ? lhist : nullptr);
    }
    flush_hist(P, qi, lhist);
}

// Scores of invisible positions (for the scores-only entry point).
__global__ void fill_invisible_kernel(float *scores, int64_t n_max, QueryPos QP) {
    const int qi = blockIdx.y;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n_max && i >= visible_keys(QP, qi)) scores[(int64_t)qi * n_max + i] = -INFINITY;
}

// Clears a workspace region with vector stores (used instead of a runtime memset so the
// whole call can be captured into a graph).
__global__ void zero_kernel(uint4 *p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
    const size_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    V4A_LAUNCH("zero_kernel", zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)p, n16);
    return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs &a, const QueryPos &qp, hipStream_t s) {
    IndexerParams P{};
    const bool mx = a.keys->fmt == V4A_IDX_MXFP4;
    P.kcap = a.keys->cap;
    P.qcap = a.q->cap;
    if (mx) {
        P.kc = (const uint8_t *)a.keys->codes;
        P.ks = a.keys->scales;
        P.qc = (const uint8_t *)a.q->codes;
        P.qs = a.q->scales;
    } else {
        P.kf = (const float *)a.keys->codes;
        P.qf = (const float *)a.q->codes;
    }
    P.w = a.w;
    P.H = a.H_I;
    P.d = a.keys->d;
    P.n_max = a.n_max;
    P.key_stride = a.key_stride;
    P.score_keys = a.score_keys;
    P.key16 = a.key16;
    P.scores = a.scores;
    P.hist = a.hist;
    P.hist_copies = a.hist_copies > 0 ? a.hist_copies : 1;
    P.key_rec = a.key_rec != nullptr;
    if (a.key_rec) {
        P.key = compress_params(*a.key_rec);
        if (!mx || P.d != 128 || a.Q != 1 || !entry_two_phase(P.key)) return hipErrorInvalidValue;
    }
    const int BQ = a.B * a.Q;
    if (a.n_max == 0 || BQ == 0) return hipSuccess;
    if (mx) {
        // keys per workgroup: doubled from 512 while the grid keeps at least 1024 workgroups, so
        // a large scan runs as 512-1024 workgroups (two to four per CU) of up to 4096 keys; it
        // changes only the work split, never a result.  (At the 1M-context decode, 2048-key
        // workgroups, two per CU, measured 20-21 us on every device tried; 1024-key ones 19-24.)
        int gpw = 2 * kGroupsPerIter;  // keys per workgroup = 4 wavefronts * gpw groups * 16 keys
        while (gpw < 64 && (int64_t)BQ * ((a.n_max + 64 * gpw - 1) / (64 * gpw)) >= 1024) gpw *= 2;
        P.groups_per_wave = gpw;
        const int64_t kpw = (int64_t)64 * gpw;
        dim3 grid((unsigned)((a.n_max + kpw - 1) / kpw), (unsigned)BQ);
        if (P.key_rec)
            V4A_LAUNCH("indexer_mxfp4_kernel", indexer_mxfp4_kernel<true>, grid, dim3(256), 0, s, P, qp);
        else
            V4A_LAUNCH("indexer_mxfp4_kernel", indexer_mxfp4_kernel<false>, grid, dim3(256), 0, s, P, qp);
    } else {
        dim3 grid((unsigned)((a.n_max + 255) / 256), (unsigned)BQ);
        V4A_LAUNCH("indexer_f32_kernel", indexer_f32_kernel, grid, dim3(256), 0, s, P, qp);
    }
    if (a.scores) {
        dim3 grid((unsigned)((a.n_max + 255) / 256), (unsigned)BQ);
        V4A_LAUNCH("fill_invisible_kernel", fill_invisible_kernel, grid, dim3(256), 0, s, a.scores, a.n_max, qp);
    }
    return hipGetLastError();
}

}  // namespace v4a
