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
// Each score is written as an orderable 32-bit key (larger score -> larger key) and counted
// in a 4096-bin histogram of its top 12 bits (LDS per workgroup, then one global atomic add
// per non-empty bin), which the top-k select uses to find the threshold bin.
#include "common.hpp"

namespace v4a {

constexpr int kKeysPerWG = 1024;
constexpr int kHistBins = 4096;
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
    uint32_t *score_keys;  // [BQ][n_max] or NULL
    float *scores;         // [BQ][n_max] or NULL
    uint32_t *hist;        // [BQ][4096] or NULL
};

__device__ __forceinline__ void emit_score(const IndexerParams &P, int qi, int64_t i, float score,
                                           uint32_t *lhist) {
    if (score == 0.0f) score = 0.0f;  // -0 -> +0
    if (P.scores) P.scores[(int64_t)qi * P.n_max + i] = score;
    uint32_t key = score_key(score);
    if (P.score_keys) P.score_keys[(int64_t)qi * P.n_max + i] = key;
    if (lhist) atomicAdd(&lhist[key >> 20], 1u);
}

__device__ __forceinline__ void flush_hist(const IndexerParams &P, int qi, uint32_t *lhist) {
    __syncthreads();
    if (!P.hist) return;
    for (int bin = threadIdx.x; bin < kHistBins; bin += blockDim.x) {
        uint32_t c = lhist[bin];
        if (c) atomicAdd(&P.hist[(int64_t)qi * kHistBins + bin], c);
    }
}

// MXFP4, d = 128 (one 16x16x128 scaled MFMA per 16 heads and 16 keys), H <= 64.
__global__ void __launch_bounds__(256) indexer_mxfp4_kernel(IndexerParams P, QueryPos QP) {
    __shared__ uint32_t lhist[kHistBins];
    const int qi = blockIdx.y;
    const int b = qi / QP.Q;
    const int64_t n_vis = visible_keys(QP, qi);
    const int64_t k0 = (int64_t)blockIdx.x * kKeysPerWG;
    if (k0 >= n_vis) return;  // uniform over the workgroup
    for (int bin = threadIdx.x; bin < kHistBins; bin += 256) lhist[bin] = 0;

    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;  // col: head/key within 16; grp: MX block / chain

    // query: 4 head groups of 16 heads; lane holds head 16g+col, MX block grp
    v8i qa[4];
    int qscale[4];
    float wt[4][4];  // w of heads 16g + 4*grp + i
#pragma unroll
    for (int g = 0; g < 4; g++) {
        const int h = 16 * g + col;
        const int64_t row = (int64_t)b * P.qcap + (int64_t)(qi % QP.Q) * P.H + h;
        qa[g] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        qscale[g] = 127;
        if (h < P.H) {
            const uint4 c = *(const uint4 *)(P.qc + row * 64 + grp * 16);
            qa[g][0] = (int)c.x; qa[g][1] = (int)c.y; qa[g][2] = (int)c.z; qa[g][3] = (int)c.w;
            qscale[g] = P.qs[row * 4 + grp];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int hh = 16 * g + 4 * grp + i;
            wt[g][i] = hh < P.H ? P.w[(int64_t)qi * P.H + hh] : 0.0f;
        }
    }
    __syncthreads();

    const uint8_t *kc = P.kc + (int64_t)b * P.kcap * 64;
    const uint8_t *ks = P.ks + (int64_t)b * P.kcap * 4;
    const int64_t kend = k0 + kKeysPerWG < n_vis ? k0 + kKeysPerWG : n_vis;
    constexpr int kUnroll = 4;
    // wavefront wv takes key groups wv, wv+4, ... of the chunk, kUnroll at a time
    for (int64_t g0 = k0 + 16 * wv; g0 < kend; g0 += 16 * 4 * kUnroll) {
        uint4 kd[kUnroll];
        uint32_t ksc[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t key = g0 + (int64_t)u * 64 + col;
            if (key < kend) {
                kd[u] = *(const uint4 *)(kc + key * 64 + grp * 16);
                ksc[u] = (*(const uint32_t *)(ks + key * 4) >> (8 * grp)) & 0xFFu;
            } else {
                kd[u] = make_uint4(0, 0, 0, 0);
                ksc[u] = 127;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int64_t gbase = g0 + (int64_t)u * 64;
            if (gbase >= kend) break;  // uniform
            const v8i kb = v8i{(int)kd[u].x, (int)kd[u].y, (int)kd[u].z, (int)kd[u].w, 0, 0, 0, 0};
            float c = 0.0f;
#pragma unroll
            for (int g = 0; g < 4; g++) {
                v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
                acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[g], kb, acc, 4, 4, 0, qscale[g], 0,
                                                                       (int)ksc[u]);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const float r = acc[i] > 0.0f ? acc[i] : 0.0f;
                    c = fmaf(wt[g][i], r, c);
                }
            }
            const float c1 = __shfl_down(c, 16), c2 = __shfl_down(c, 32), c3 = __shfl_down(c, 48);
            const int64_t key = gbase + col;
            if (grp == 0 && key < kend) emit_score(P, qi, key, ((c + c1) + c2) + c3, P.hist ? lhist : nullptr);
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
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4 *)p, n16);
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
    P.score_keys = a.score_keys;
    P.scores = a.scores;
    P.hist = a.hist;
    const int BQ = a.B * a.Q;
    if (a.n_max == 0 || BQ == 0) return hipSuccess;
    if (mx) {
        dim3 grid((unsigned)((a.n_max + kKeysPerWG - 1) / kKeysPerWG), (unsigned)BQ);
        hipLaunchKernelGGL(indexer_mxfp4_kernel, grid, dim3(256), 0, s, P, qp);
    } else {
        dim3 grid((unsigned)((a.n_max + 255) / 256), (unsigned)BQ);
        hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), 0, s, P, qp);
    }
    if (a.scores) {
        dim3 grid((unsigned)((a.n_max + 255) / 256), (unsigned)BQ);
        hipLaunchKernelGGL(fill_invisible_kernel, grid, dim3(256), 0, s, a.scores, a.n_max, qp);
    }
    return hipGetLastError();
}

}  // namespace v4a
