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

constexpr int kGroupsPerIter = 4;   // key groups of 16 per load batch
constexpr int kMaxGroupsPerWave = 64;
constexpr int kStreamMaxKeys = 4096;  // keys per workgroup of the streaming kernel
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
    int stream_kpw;        // streaming kernel: keys per workgroup (a multiple of 64, <= kStreamMaxKeys)
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
template <int NT>
__device__ __forceinline__ void flush_hist_nobarrier(const IndexerParams &P, int qi, const uint32_t *lhist) {
    if (!P.hist) return;
    uint32_t *gh = P.hist + ((int64_t)qi * P.hist_copies + (int)(blockIdx.x % (unsigned)P.hist_copies)) * kHistBins;
    // consecutive bins in consecutive lanes, so the few hot bins of a query leave in one wide
    // atomic instruction per cache line; all LDS reads are issued before the first atomic
    static_assert(kHistBins % NT == 0, "whole bins per thread");
    constexpr int kPer = kHistBins / NT;  // bins per thread
    uint32_t c[kPer];
#pragma unroll
    for (int i = 0; i < kPer; i++) c[i] = lhist[threadIdx.x + i * NT];
#pragma unroll
    for (int i = 0; i < kPer; i++)
        if (c[i]) atomicAdd(&gh[threadIdx.x + i * NT], c[i]);
}

template <int NT>
__device__ __forceinline__ void flush_hist(const IndexerParams &P, int qi, uint32_t *lhist) {
    lds_barrier();
    flush_hist_nobarrier<NT>(P, qi, lhist);
}

// A query's MFMA operands: 4 head groups of 16 heads; lane (col, grp) holds head 16g+col's
// MX block grp and the weights of heads 16g + 4 grp + i.  Heads past H read head H-1 (all loads
// issued together) and are zeroed: code 0 and weight 0.
struct QueryOperands {
    v8i qa[4];
    int qscale[4];
    float wt[4][4];
};

__device__ __forceinline__ QueryOperands load_query(const IndexerParams &P, const QueryPos &QP, int qi, int b, int col,
                                                    int grp) {
    QueryOperands o;
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
        o.qa[g] = v8i{on ? (int)qc[g].x : 0, on ? (int)qc[g].y : 0, on ? (int)qc[g].z : 0, on ? (int)qc[g].w : 0,
                      0, 0, 0, 0};
        o.qscale[g] = on ? (int)qsb[g] : 127;
#pragma unroll
        for (int i = 0; i < 4; i++) o.wt[g][i] = (16 * g + 4 * grp + i < P.H) ? wr[g][i] : 0.0f;
    }
    return o;
}

// fma chain grp of key col of a group (codes kdu, the key's four scale bytes kscu)
__device__ __forceinline__ float key_chain(const QueryOperands &qo, const uint4 &kdu, uint32_t kscu, int grp) {
    const v8i kb = v8i{(int)kdu.x, (int)kdu.y, (int)kdu.z, (int)kdu.w, 0, 0, 0, 0};
    const int sc = (int)((kscu >> (8 * grp)) & 0xFFu);
    v4f acc[4];
#pragma unroll
    for (int g = 0; g < 4; g++)
        acc[g] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qo.qa[g], kb, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 4, 4, 0,
                                                                  qo.qscale[g], 0, sc);
    // ReLU on the bit pattern: a finite float is negative (or -0) exactly when its bits read as
    // a negative int, so max(int bits, 0) gives s for s > 0 and +0 otherwise
    float cu = 0.0f;
#pragma unroll
    for (int g = 0; g < 4; g++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float si = acc[g][i];  // a scalar copy: bit casts read whole objects
            const float r = __builtin_bit_cast(float, max(__builtin_bit_cast(int, si), 0));
            cu = fmaf(qo.wt[g][i], r, cu);
        }
    }
    return cu;
}

// Scores of a batch of four key groups: lane 16 q + col returns the score of key col of group
// q.  Lane group q holds chain q of key col of every group u; a 4 x 4 transpose across the lane
// groups (swap the upper half of c0/c1 with the lower half of c2/c3, then the odd rows of those
// with the even rows) leaves lane group q holding chains 0..3 of key col of group q, so every
// lane finishes one key with the fixed-order sum.
static_assert(kGroupsPerIter == 4, "the chain transpose pairs four groups with four lane groups");
__device__ __forceinline__ float batch_scores(const QueryOperands &qo, const uint4 (&kd)[kGroupsPerIter],
                                              const uint32_t (&ksc)[kGroupsPerIter], int grp) {
    uint32_t c[kGroupsPerIter];
#pragma unroll
    for (int u = 0; u < kGroupsPerIter; u++) c[u] = fbits(key_chain(qo, kd[u], ksc[u], grp));
    const auto a02 = __builtin_amdgcn_permlane32_swap(c[0], c[2], false, false);
    const auto a13 = __builtin_amdgcn_permlane32_swap(c[1], c[3], false, false);
    const auto t01 = __builtin_amdgcn_permlane16_swap(a02[0], a13[0], false, false);
    const auto t23 = __builtin_amdgcn_permlane16_swap(a02[1], a13[1], false, false);
    float sc = ((bitsf(t01[0]) + bitsf(t01[1])) + bitsf(t23[0])) + bitsf(t23[1]);
    if (sc == 0.0f) sc = 0.0f;  // -0 -> +0
    return sc;
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
// STREAM: the keys are read once per launch (decode: one query per sequence), so they are
// loaded non-temporally; otherwise (a prefill chunk: every query of the chunk reads the same
// keys) they are loaded through the caches, which serve the other queries' re-reads.
template <int NW, int NB, bool KEYREC, bool STREAM>
__global__ void __launch_bounds__(64 * NW) indexer_mxfp4_kernel(IndexerParams P, QueryPos QP) {
    constexpr int NT = 64 * NW;
    static_assert(NB >= 2 && NB <= 4, "load batches in flight");
    __shared__ uint32_t lhist[kHistBins];
    __shared__ __attribute__((aligned(16))) float sbuf[NW * kMaxGroupsPerWave * 16];  // this workgroup's scores
    __shared__ __attribute__((aligned(16))) uint8_t knew[80];  // the new key's codes + scales
    const int qi = blockIdx.y;
    const int b = qi / QP.Q;
    const int64_t n_vis = visible_keys(QP, qi);
    const int64_t keys_per_wg = (int64_t)NW * P.groups_per_wave * 16;
    const int64_t k0 = (int64_t)blockIdx.x * keys_per_wg;
    if (k0 >= n_vis) return;  // uniform over the workgroup

    // the wavefront index read as a uniform value, so that everything derived from it (the
    // wavefront's key range, whole-iteration tests) stays in scalar registers and branches
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
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
    // Keys are addressed as the sequence's (uniform) base plus a 32-bit offset per lane (a
    // sequence's key rows span less than 4 GiB); lanes past the end read a clamped, valid key of
    // this query and are masked afterwards.
    const uint32_t lane_key0 = (uint32_t)(wbase + col);
    const uint32_t key_last = (uint32_t)(kend - 1);
    auto load_iter = [&](int it, uint4 (&kd)[kGroupsPerIter], uint32_t (&ksc)[kGroupsPerIter]) {
#pragma unroll
        for (int u = 0; u < kGroupsPerIter; u++) {
            const uint32_t key = min(lane_key0 + (uint32_t)(it * kGroupsPerIter * 16 + 16 * u), key_last);
            const u32x4 *pc = (const u32x4 *)(kc + (key * 64u + (uint32_t)grp * 16u));
            const u32x4 v = STREAM ? __builtin_nontemporal_load(pc) : *pc;
            kd[u] = make_uint4(v.x, v.y, v.z, v.w);
            ksc[u] = *(const uint32_t *)(ks + key * 4u);
        }
    };
    // iterations holding at least one visible key (uniform over the wavefront)
    const int n_live = wbase >= kend ? 0 : min(n_it, (int)((kend - wbase + kGroupsPerIter * 16 - 1) / (kGroupsPerIter * 16)));
    // the first NB-1 key batches are requested before the query, so their latencies overlap
    uint4 kd[NB][kGroupsPerIter];
    uint32_t ksc[NB][kGroupsPerIter];
    if (n_live > 0) {
#pragma unroll
        for (int j = 0; j < NB - 1; j++) load_iter(min(j, n_live - 1), kd[j], ksc[j]);
    }
    for (int bin = threadIdx.x; bin < kHistBins; bin += NT) lhist[bin] = 0;

    const QueryOperands qo = load_query(P, QP, qi, b, col, grp);
    __syncthreads();

    auto compute_iter = [&](int it, const uint4 (&kd)[kGroupsPerIter], const uint32_t (&ksc)[kGroupsPerIter]) {
        const int64_t base = wbase + (int64_t)it * kGroupsPerIter * 16;
        sbuf[base - k0 + 16 * grp + col] = batch_scores(qo, kd, ksc, grp);  // slots past kend are never read
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
        const float c = key_chain(qo, *(const uint4 *)(knew + 16 * grp), *(const uint32_t *)(knew + 64), grp);
        float sc = ((lane_value(c, 0) + lane_value(c, 16)) + lane_value(c, 32)) + lane_value(c, 48);
        if (sc == 0.0f) sc = 0.0f;  // -0 -> +0
        sc_new = sc;
    };
    // A ring of NB load batches: batch it + NB - 1 is requested before batch it is computed.
    // Past the wavefront's last iteration the request repeats that iteration (valid addresses,
    // never computed), so every iteration issues the same loads and each wait leaves the later
    // batches in flight.
    for (int it0 = 0; it0 < n_live; it0 += NB) {
#pragma unroll
        for (int j = 0; j < NB; j++) {
            const int it = it0 + j;
            if (it >= n_live) break;  // uniform over the wavefront
            load_iter(min(it + NB - 1, n_live - 1), kd[(j + NB - 1) % NB], ksc[(j + NB - 1) % NB]);
            compute_iter(it, kd[j], ksc[j]);
            if (own && it == 0) new_key();
        }
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
    for (int i0 = 4 * threadIdx.x; i0 < n_here; i0 += 4 * NT) {
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
    flush_hist<NT>(P, qi, lhist);
}

// Streaming form of the MXFP4 kernel for a long decode scan (one query per sequence, d = 128,
// H <= 64): one workgroup of kStreamWaves wavefronts per CU owns kpw consecutive keys of one
// query, cut into batches of 64 keys (four groups of 16).
//  - Wavefronts claim batches from an LDS counter (each claim is made one batch before its
//    loads, so its latency hides behind the arithmetic) and keep two batches in flight: a
//    batch's key codes and scales are copied straight into the wavefront's LDS stage by
//    direct-to-LDS loads, so no register waits on them and the only wait is for the older
//    stage.  A wavefront keeps claiming until the workgroup's keys run out, whichever
//    wavefronts the hardware favours.
//  - Each lane ends a batch holding one key's score: its orderable key leaves at once (one
//    256-byte store per batch) and is counted in the LDS histogram, so nothing remains to do
//    after the stream but the histogram flush.
//  - key_rec: wavefront 0 of the workgroup holding the query's new entry requests the entry's
//    candidate rows before the stream and, after its last batch, merges, encodes and scores
//    the new key with the same arithmetic; the batch holding that entry leaves its slot to it.
// Scores, keys and histogram are bitwise those of indexer_mxfp4_kernel.
constexpr int kStreamWaves = 8;   // wavefronts per workgroup
constexpr int kStreamStages = 3;  // key batches in flight per wavefront (LDS stages of 5 KB)

template <int QT, bool KEYREC>
__global__ void __launch_bounds__(64 * kStreamWaves) indexer_mxfp4_stream_kernel(IndexerParams P, QueryPos QP) {
    constexpr int NW = kStreamWaves;
    constexpr int NST = QT == 1 ? kStreamStages : 2;  // stages per wavefront (LDS holds QT histograms)
    constexpr int kBatch = kGroupsPerIter * 16;  // keys per batch
    static_assert(QT == 1 || !KEYREC, "the new key is compressed here for one query per sequence only");
    __shared__ uint32_t lhist[QT][kHistBins];
    __shared__ uint32_t next_batch;
    __shared__ __attribute__((aligned(16))) uint8_t knew[80];
    __shared__ __attribute__((aligned(16))) uint8_t qcodes[QT][4][1024];  // head group g: lane l's 16 code bytes
    __shared__ __attribute__((aligned(16))) uint32_t qscl[QT][4][64];      // head group g: lane l's head's scale word
    __shared__ __attribute__((aligned(16))) float qw[QT][64];              // w of head h (h < H; H - 1 past it)
    // load stages: NST per wavefront, used round robin
    __shared__ __attribute__((aligned(16))) uint8_t codes[NST][NW][kGroupsPerIter * 1024];
    __shared__ __attribute__((aligned(16))) uint32_t scl[NST][NW][kGroupsPerIter * 64];
    // queries qi0 .. qi0 + QT - 1: one query, or the QT queries (tokens) of one sequence
    const int qi0 = (int)blockIdx.y * QT;
    const int b = qi0 / QP.Q;
    int64_t nv[QT];
    int64_t n_vis = 0;  // keys this workgroup streams: the most any of its queries sees
#pragma unroll
    for (int j = 0; j < QT; j++) {
        nv[j] = visible_keys(QP, qi0 + j);
        n_vis = nv[j] > n_vis ? nv[j] : n_vis;
    }
    const int64_t k0 = (int64_t)blockIdx.x * P.stream_kpw;
    if (k0 >= n_vis) return;  // uniform over the workgroup
    const int64_t kend = k0 + P.stream_kpw < n_vis ? k0 + P.stream_kpw : n_vis;
    const int n_batches = (int)((kend - k0 + kBatch - 1) / kBatch);
    const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const uint8_t *kc = P.kc + (int64_t)b * P.kcap * 64;
    const uint8_t *ks = P.ks + (int64_t)b * P.kcap * 4;
    const uint32_t key_last = (uint32_t)(kend - 1);

    const int qi = qi0;  // (QT == 1)
    int64_t i_new = -1;
    if (KEYREC) {
        const int64_t pos = QP.pos[qi];
        if ((pos + 1) % P.key.m == 0) i_new = (pos + 1) / P.key.m - 1;
        if (i_new < k0 || i_new >= kend) i_new = -1;  // not this workgroup's
    }
    const bool own = KEYREC && wv == 0 && i_new >= 0;  // uniform over the wavefront
    KeyPrefetch<2> kp;
    if (own) key_prefetch<2>(P.key, qi, i_new, (int64_t)P.key.m * (i_new - 1), kp);

    // batch bt into a stage: group u is keys k0 + 64 bt + 16 u + (0..15); lane l copies its 16
    // code bytes (MX block grp of key col) to byte 1024 u + 16 l and its key's scale word to
    // word 64 u + l.  Lanes past the end read a clamped, valid key of this query, masked later.
    auto load_batch = [&](int bt, uint8_t *cst, uint32_t *sst) {
        const uint32_t kb0 = (uint32_t)k0 + (uint32_t)(bt * kBatch + col);
#pragma unroll
        for (int u = 0; u < kGroupsPerIter; u++) {
            const uint32_t key = min(kb0 + (uint32_t)(16 * u), key_last);
            lds_copy16_nt(kc + (key * 64u + (uint32_t)grp * 16u), lds_addr(cst + 1024 * u));
            lds_copy4(ks + key * 4u, lds_addr(sst + 64 * u));
        }
    };
    // The stream's LDS instructions are written out too (the compiler, which cannot tell the
    // stages' copies apart, would otherwise wait for every copy in flight before each LDS
    // access); the explicit vmcnt wait before a stage is read covers that stage's copies.
    auto stage_scores = [&](const uint8_t *cst, const uint32_t *sst, const QueryOperands (&qo)[QT], float (&sc)[QT]) {
        u32x4 c0, c1, c2, c3;
        uint32_t s0, s1, s2, s3;
        const uint32_t ca = lds_addr(cst) + 16u * (uint32_t)lane;
        const uint32_t sa = lds_addr(sst) + 4u * (uint32_t)lane;
        asm volatile(
            "ds_read_b128 %0, %8\n\t"
            "ds_read_b128 %1, %8 offset:1024\n\t"
            "ds_read_b128 %2, %8 offset:2048\n\t"
            "ds_read_b128 %3, %8 offset:3072\n\t"
            "ds_read_b32 %4, %9\n\t"
            "ds_read_b32 %5, %9 offset:256\n\t"
            "ds_read_b32 %6, %9 offset:512\n\t"
            "ds_read_b32 %7, %9 offset:768\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(c0), "=&v"(c1), "=&v"(c2), "=&v"(c3), "=&v"(s0), "=&v"(s1), "=&v"(s2), "=&v"(s3)
            : "v"(ca), "v"(sa)
            : "memory");
        const uint4 kd[kGroupsPerIter] = {make_uint4(c0.x, c0.y, c0.z, c0.w), make_uint4(c1.x, c1.y, c1.z, c1.w),
                                          make_uint4(c2.x, c2.y, c2.z, c2.w), make_uint4(c3.x, c3.y, c3.z, c3.w)};
        const uint32_t ksc[kGroupsPerIter] = {s0, s1, s2, s3};
#pragma unroll
        for (int j = 0; j < QT; j++) sc[j] = batch_scores(qo[j], kd, ksc, grp);
    };
    const int hshift = P.key16 ? 4 : 20;  // the top 12 bits of either key
    // batch bt's scores leave: one key per lane and query, for the keys that query sees (the new
    // entry's slot is left to its owner)
    auto emit = [&](int bt, const float (&sc)[QT]) {
        const int64_t i = k0 + (int64_t)bt * kBatch + lane;
#pragma unroll
        for (int j = 0; j < QT; j++) {
            if (i < kend && i < nv[j] && i != i_new) {
                const int64_t row = (int64_t)(qi0 + j);
                const uint32_t key = P.key16 ? score_key16(sc[j]) : score_key(sc[j]);
                if (P.score_keys && !P.key16) ((uint32_t *)P.score_keys)[row * P.key_stride + i] = key;
                if (P.score_keys && P.key16) ((uint16_t *)P.score_keys)[row * P.key_stride + i] = (uint16_t)key;
                if (P.scores) P.scores[row * P.n_max + i] = sc[j];
                if (P.hist)
                    asm volatile("ds_add_u32 %0, %1" ::"v"(lds_addr(lhist[j]) + 4u * (key >> hshift)), "v"(1u) : "memory");
            }
        }
    };

    // Wavefront 0 copies the query (codes, scales, weights) to LDS before its first batches and
    // waits only for those copies; every wavefront then reads its operands from LDS, so no
    // register of the stream waits on a global load the compiler would drain the copies for.
#pragma unroll
    for (int j = 0; j < QT; j++)
        for (int bin = threadIdx.x; bin < kHistBins; bin += 64 * NW) lhist[j][bin] = 0;
    if (threadIdx.x == 0) next_batch = NST * NW;
    if (wv == 0) {
#pragma unroll
        for (int j = 0; j < QT; j++) {
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int h = min(16 * g + col, P.H - 1);
                const int64_t row = (int64_t)b * P.qcap + (int64_t)((qi0 + j) % QP.Q) * P.H + h;
                lds_copy16(P.qc + row * 64 + grp * 16, lds_addr(qcodes[j][g]));
                lds_copy4(P.qs + row * 4, lds_addr(qscl[j][g]));
            }
            lds_copy4(P.w + (int64_t)(qi0 + j) * P.H + min(lane, P.H - 1), lds_addr(qw[j]));
        }
    }
    // the first NST batches of every wavefront are fixed (batch j NW + wv for stage j); the
    // rest are claimed
    int bq[NST];  // the batches in stages st, st + 1, ... (mod NST)
#pragma unroll
    for (int j = 0; j < NST; j++) {
        bq[j] = j * NW + wv;
        load_batch(min(bq[j], n_batches - 1), codes[j][wv], scl[j][wv]);
    }
    if (wv == 0) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kGroupsPerIter * NST) : "memory");
    lds_barrier();
    QueryOperands qo[QT];
#pragma unroll
    for (int jq = 0; jq < QT; jq++) {
        u32x4 c[4], w4[4];
        uint32_t sc[4];
        const uint32_t ca = lds_addr(qcodes[jq]) + 16u * (uint32_t)lane, sa = lds_addr(qscl[jq]) + 4u * (uint32_t)lane;
        const uint32_t wa = lds_addr(qw[jq]) + 16u * (uint32_t)grp;
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %12 offset:1024\n\t"
            "ds_read_b128 %2, %12 offset:2048\n\t"
            "ds_read_b128 %3, %12 offset:3072\n\t"
            "ds_read_b32 %4, %13\n\t"
            "ds_read_b32 %5, %13 offset:256\n\t"
            "ds_read_b32 %6, %13 offset:512\n\t"
            "ds_read_b32 %7, %13 offset:768\n\t"
            "ds_read_b128 %8, %14\n\t"
            "ds_read_b128 %9, %14 offset:64\n\t"
            "ds_read_b128 %10, %14 offset:128\n\t"
            "ds_read_b128 %11, %14 offset:192\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(c[0]), "=&v"(c[1]), "=&v"(c[2]), "=&v"(c[3]), "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]),
              "=&v"(sc[3]), "=&v"(w4[0]), "=&v"(w4[1]), "=&v"(w4[2]), "=&v"(w4[3])
            : "v"(ca), "v"(sa), "v"(wa)
            : "memory");
        // as load_query: heads past H get code 0, scale 127 and weight 0
#pragma unroll
        for (int g = 0; g < 4; g++) {
            const bool on = 16 * g + col < P.H;
            qo[jq].qa[g] = v8i{on ? (int)c[g].x : 0, on ? (int)c[g].y : 0, on ? (int)c[g].z : 0,
                               on ? (int)c[g].w : 0, 0, 0, 0, 0};
            qo[jq].qscale[g] = on ? (int)((sc[g] >> (8 * grp)) & 0xFFu) : 127;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const uint32_t wb = w4[g][i];  // a scalar copy: bit casts read whole objects
                qo[jq].wt[g][i] = (16 * g + 4 * grp + i < P.H) ? __builtin_bit_cast(float, wb) : 0.0f;
            }
        }
    }

    const uint32_t nb_addr = lds_addr(&next_batch);
    // a claim: lane 0 adds one to the batch counter; the old value, read later by the whole
    // wavefront, is the claimed batch
    auto claim_next = [&]() {
        uint32_t c = 0;
        if (lane == 0)
            asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=&v"(c) : "v"(nb_addr), "v"(1u)
                         : "memory");
        return c;
    };
    uint32_t claim = claim_next();
    // Every step refills the stage it has read (a finished wavefront repeats the last batch:
    // valid addresses, never computed), so each wait leaves exactly the other stages' copies in
    // flight: at most (NST - 1) x 8 newer loads (the key stores in between may still travel;
    // loads complete in order, so these counts leave the stage read complete).
    for (int st = 0;;) {
        if (bq[0] >= n_batches) break;  // uniform over the wavefront
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kGroupsPerIter * (NST - 1)) : "memory");
        float sc[QT];
        stage_scores(codes[st][wv], scl[st][wv], qo, sc);
        emit(bq[0], sc);
        const int nb = __builtin_amdgcn_readfirstlane(claim);
        load_batch(min(nb, n_batches - 1), codes[st][wv], scl[st][wv]);
        claim = claim_next();
#pragma unroll
        for (int j = 0; j + 1 < NST; j++) bq[j] = bq[j + 1];
        bq[NST - 1] = nb;
        st = st + 1 == NST ? 0 : st + 1;
    }
    if (own) {
        // the new key: merged, encoded (into LDS), scored as the stream's keys are, counted and
        // stored; then its cache row (64 code bytes, 4 scale bytes) from the LDS copy
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        key_finish<2>(P.key, kp, qi, i_new, knew, false);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const float c = key_chain(qo[0], *(const uint4 *)(knew + 16 * grp), *(const uint32_t *)(knew + 64), grp);
        float sn = ((lane_value(c, 0) + lane_value(c, 16)) + lane_value(c, 32)) + lane_value(c, 48);
        if (sn == 0.0f) sn = 0.0f;  // -0 -> +0
        if (lane == 0) {
            const uint32_t key = P.key16 ? score_key16(sn) : score_key(sn);
            if (P.score_keys && !P.key16) ((uint32_t *)P.score_keys)[(int64_t)qi * P.key_stride + i_new] = key;
            if (P.score_keys && P.key16) ((uint16_t *)P.score_keys)[(int64_t)qi * P.key_stride + i_new] = (uint16_t)key;
            if (P.scores) P.scores[(int64_t)qi * P.n_max + i_new] = sn;
            if (P.hist) atomicAdd(&lhist[0][key >> hshift], 1u);
        }
        const int64_t row = P.key.out_row0 + (int64_t)qi * P.key.cap + i_new;
        if (lane < 16) ((uint32_t *)((uint8_t *)P.key.idx.codes + row * 64))[lane] = ((const uint32_t *)knew)[lane];
        if (lane == 16) *(uint32_t *)(P.key.idx.scales + row * 4) = *(const uint32_t *)(knew + 64);
    }
    lds_barrier();
#pragma unroll
    for (int j = 0; j < QT; j++) flush_hist_nobarrier<64 * NW>(P, qi0 + j, lhist[j]);
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
    flush_hist<256>(P, qi, lhist);
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

// Launch shape of the MXFP4 scoring kernel.
constexpr int kScoreWaves = 4;      // wavefronts per workgroup
constexpr int kScoreBatches = 2;    // key load batches in flight per wavefront
constexpr int kScoreMinWGs = 1024;  // keys per workgroup grow while the grid keeps this many
// Launch shape of the streaming kernel (one query per sequence, at least kStreamMinKeys keys).
constexpr int kStreamWGs = 256;     // workgroups aimed at (one per CU)
constexpr int64_t kStreamMinKeys = (int64_t)kStreamWGs * 1024;

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
    if (mx && (a.Q == 1 || a.Q == 2) && (int64_t)BQ * a.n_max >= kStreamMinKeys && !(a.Q == 2 && P.key_rec)) {
        // a long decode scan: one streaming workgroup per CU; with two queries per sequence (a
        // two-token step) both are scored from each batch a workgroup loads.  Keys per workgroup
        // the largest of 1024, 2048, 4096 that still gives kStreamWGs workgroups.
        const int rows = a.B;  // workgroup rows: one per sequence (its Q queries)
        int kpw = kStreamMaxKeys;
        while (kpw > 1024 && (int64_t)rows * ((a.n_max + kpw - 1) / kpw) < kStreamWGs) kpw /= 2;
        P.stream_kpw = kpw;
        dim3 grid((unsigned)((a.n_max + kpw - 1) / kpw), (unsigned)rows);
        if (a.Q == 2)
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_stream_kernel<2, false>), grid, dim3(64 * kStreamWaves), 0,
                       s, P, qp);
        else if (P.key_rec)
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_stream_kernel<1, true>), grid, dim3(64 * kStreamWaves), 0,
                       s, P, qp);
        else
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_stream_kernel<1, false>), grid, dim3(64 * kStreamWaves), 0,
                       s, P, qp);
    } else if (mx) {
        // keys per wavefront: doubled from 128 while the grid keeps at least kScoreMinWGs
        // workgroups; it changes only the work split, never a result
        constexpr int NW = kScoreWaves;
        int gpw = 2 * kGroupsPerIter;
        while (gpw < kMaxGroupsPerWave && (int64_t)BQ * ((a.n_max + 16 * NW * gpw - 1) / (16 * NW * gpw)) >= kScoreMinWGs)
            gpw *= 2;
        P.groups_per_wave = gpw;
        const int64_t kpw = (int64_t)16 * NW * gpw;
        dim3 grid((unsigned)((a.n_max + kpw - 1) / kpw), (unsigned)BQ);
        if (P.key_rec)
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_kernel<NW, kScoreBatches, true, true>), grid, dim3(64 * NW), 0,
                       s, P, qp);
        else if (a.Q == 1)
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_kernel<NW, kScoreBatches, false, true>), grid, dim3(64 * NW),
                       0, s, P, qp);
        else
            V4A_LAUNCH("indexer_mxfp4_kernel", (indexer_mxfp4_kernel<NW, kScoreBatches, false, false>), grid,
                       dim3(64 * NW), 0, s, P, qp);
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
