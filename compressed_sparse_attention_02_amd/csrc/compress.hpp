// compress.hpp -- one compressed entry computed by one wavefront (a1/a2), shared by the
// compressor kernels and by the decode step's launches that carry a compression alongside
// other work.  "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2; "DeepSeek V4
// preview and technical report" (chooseai.net), section 1.
#pragma once

#include "encoders.hpp"

namespace v4a {


constexpr int kMaxCand = 256;  // 2 * 128 candidates at most

struct CompressParams {
    const void *x0, *x1;
    const float *g0, *g1, *b0, *b1;
    int n_streams, D, G, m, R;
    bool bf16_in, rope;
    int64_t tok0, first_entry, n_entries;
    RopeTable rt;
    v4a_kv kv;
    v4a_idx idx;
    bool to_idx;
    int64_t out_row0;  // b0 * cap
    int64_t cap;
    int64_t n_tok;
    const float *norm_w;  // [D] or NULL
    bool ring;            // stream rows are a ring: position p at row p mod n_tok
    bool vec_in;          // the streams are aligned for one vector load per lane and row
};

template <int VPT>
__device__ __forceinline__ void load_row(const void *base, bool bf16, int64_t row, int D, int d0,
                                         bool active, float (&v)[VPT], int64_t off) {
    if (!active) {
#pragma unroll
        for (int i = 0; i < VPT; i++) v[i] = 0.0f;
        return;
    }
    if (bf16) {
        const uint16_t *p = (const uint16_t *)base + off + row * D + d0;
#pragma unroll
        for (int i = 0; i < VPT; i++) v[i] = bf16_to_f32(p[i]);
    } else {
        const float *p = (const float *)base + off + row * D + d0;
#pragma unroll
        for (int i = 0; i < VPT; i++) v[i] = p[i];
    }
}

// Candidates of entry i: stream s = c / m (0: own block i, 1: B-block i-1), position j = c % m;
// the stream row of token position p is p - tok0, or p mod n_tok for a ring.
__device__ __forceinline__ int entry_candidates(const CompressParams &P, int64_t i) {
    return (P.n_streams == 2 && i >= 1) ? 2 * P.m : P.m;
}
__device__ __forceinline__ int64_t candidate_row(const CompressParams &P, int64_t i, int c, int64_t tok0) {
    const int m = P.m, s = c / m, j = c % m;
    const int64_t pos = (s == 0 ? (int64_t)m * i : (int64_t)m * (i - 1)) + j;
    return P.ring ? pos % P.n_tok : pos - tok0;
}

// A uniform pointer held in scalar registers (read lane by lane), so that choosing between two
// kernel-argument pointers stays a choice of register values instead of becoming a load of
// the argument block at a computed address ahead of every row load.
template <typename T>
__device__ __forceinline__ const T *uniform_ptr(const T *p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return (const T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// The streams of one entry's candidates: per stream (0: block i, 1: B-block i-1) the first
// element of this sequence's rows, its gates and biases, and the stream row of the block's
// first token; candidate c = s*m + j sits at row base[s] + j (wrapped once in a ring, whose
// n_tok >= m rows hold a block).
struct EntryStreams {
    const char *x[2];
    const float *g[2], *b[2];
    int64_t base[2];
    int m;
    int64_t n_tok;
    bool ring;
    __device__ __forceinline__ EntryStreams(const CompressParams &P, int64_t seq, int64_t i, int64_t tok0) {
        const int esz = P.bf16_in ? 2 : 4;
        x[0] = uniform_ptr((const char *)P.x0) + seq * P.n_tok * P.D * esz;
        x[1] = P.n_streams == 2 ? uniform_ptr((const char *)P.x1) + seq * P.n_tok * P.D * esz : x[0];
        g[0] = uniform_ptr(P.g0) + seq * P.n_tok * P.G;
        g[1] = P.n_streams == 2 ? uniform_ptr(P.g1) + seq * P.n_tok * P.G : g[0];
        b[0] = uniform_ptr(P.b0);
        b[1] = P.n_streams == 2 ? uniform_ptr(P.b1) : b[0];
        m = P.m;
        n_tok = P.n_tok;
        ring = P.ring;
        for (int st = 0; st < 2; st++) {
            const int64_t pos = (int64_t)m * (st == 0 ? i : i - 1);
            base[st] = ring ? (pos >= 0 ? pos % n_tok : 0) : pos - tok0;
        }
    }
    __device__ __forceinline__ int64_t row(int c) const {
        const int s = c >= m ? 1 : 0, j = c - s * m;
        int64_t r = base[s] + j;
        if (ring && r >= n_tok) r -= n_tok;
        return r;
    }
};

// One candidate row's VPT values of this lane as raw words: BF16 pairs (VPT/2 words, or one
// zero-extended value for VPT = 1) or fp32 bits; converted at use, so the loads of a batch
// of rows are all in flight before the first value is needed.
template <int VPT>
__device__ __forceinline__ void load_raw(const char *p, bool bf16, bool vec, uint32_t (&w)[VPT]) {
    if (bf16) {
        if constexpr (VPT == 1) {
            w[0] = *(const uint16_t *)p;
        } else if (vec) {
            if constexpr (VPT == 8) {
                const uint4 q = *(const uint4 *)p;
                w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
            } else if constexpr (VPT == 4) {
                const uint2 q = *(const uint2 *)p;
                w[0] = q.x; w[1] = q.y;
            } else {
                w[0] = *(const uint32_t *)p;
            }
        } else {
#pragma unroll
            for (int v = 0; v < VPT; v += 2)
                w[v / 2] = (uint32_t)((const uint16_t *)p)[v] | ((uint32_t)((const uint16_t *)p)[v + 1] << 16);
        }
    } else {
        if (vec && VPT % 4 == 0) {
#pragma unroll
            for (int v = 0; v < VPT; v += 4) {
                const uint4 q = *(const uint4 *)(p + 4 * v);
                w[v] = q.x; w[v + 1] = q.y; w[v + 2] = q.z; w[v + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < VPT; v++) w[v] = ((const uint32_t *)p)[v];
        }
    }
}
template <int VPT>
__device__ __forceinline__ float raw_value(const uint32_t (&w)[VPT], bool bf16, int v) {
    if (!bf16) return bitsf(w[v]);
    if constexpr (VPT == 1) return bf16_to_f32((uint16_t)w[0]);
    return bf16_to_f32((uint16_t)((v & 1) ? (w[v / 2] >> 16) : (w[v / 2] & 0xFFFFu)));
}

// Gate-per-token merge (G = 1) by one wavefront: the softmax weights of all candidates of entry i
// go to wsh (exp(z - max), computed once per wavefront: lane c holds candidate c, c + 64, ...)
// and their sum is returned; candidates [c_begin, c_end) are accumulated into acc in order.
// Candidate rows are loaded in batches of kRowBatch as raw words, the first two batches issued
// before the gate logits and each batch refilled once it has been accumulated.
// PK: the streams are BF16 with one vector load per lane and row (bf16_in and vec_in), whose
// rows are kept as packed BF16 pairs (VPT / 2 words) instead of VPT words.
template <int VPT, bool PK>
__device__ __forceinline__ float merge_gate1(const CompressParams &P, float *wsh, int64_t seq, int64_t i,
                                             int64_t tok0, int c_begin, int c_end, float (&acc)[VPT]) {
    static_assert(!PK || VPT % 2 == 0, "packed rows hold BF16 pairs");
    constexpr int W = PK ? VPT / 2 : VPT;  // raw words per row
    const int lane = threadIdx.x & 63;
    const int D = P.D;
    const int d0 = lane * VPT;
    const bool active = d0 < D;
    const int esz = P.bf16_in ? 2 : 4;
    const int64_t lane_off = (int64_t)(active ? d0 : 0) * esz;  // inactive lanes read dim 0
    const int n_cand = entry_candidates(P, i);
    const EntryStreams es(P, seq, i, tok0);
    // two batches of rows in flight from the start (a wavefront's share of an HCA block is 16
    // candidates: all of its rows are requested before the gate logits are used)
    constexpr int kRowBatch = 8;
    uint32_t xa[kRowBatch][W], xb[kRowBatch][W];
    auto load_batch = [&](uint32_t (&dst)[kRowBatch][W], int c0) {
#pragma unroll
        for (int u = 0; u < kRowBatch; u++) {
            const int c = min(c0 + u, c_end - 1);
            const char *src = es.x[c >= es.m ? 1 : 0] + es.row(c) * D * esz + lane_off;
            if constexpr (PK) {
                if constexpr (VPT == 8) {
                    const uint4 q = *(const uint4 *)src;
                    dst[u][0] = q.x; dst[u][1] = q.y; dst[u][2] = q.z; dst[u][3] = q.w;
                } else if constexpr (VPT == 4) {
                    const uint2 q = *(const uint2 *)src;
                    dst[u][0] = q.x; dst[u][1] = q.y;
                } else {
                    dst[u][0] = *(const uint32_t *)src;
                }
            } else {
                load_raw<VPT>(src, P.bf16_in, P.vec_in, dst[u]);
            }
        }
    };
    auto value = [&](const uint32_t (&w)[W], int v) -> float {
        if constexpr (PK) return bf16_to_f32((uint16_t)((v & 1) ? (w[v / 2] >> 16) : (w[v / 2] & 0xFFFFu)));
        else return raw_value<VPT>(w, P.bf16_in, v);
    };
    if (c_begin < c_end) load_batch(xa, c_begin);
    if (c_begin + kRowBatch < c_end) load_batch(xb, c_begin + kRowBatch);
    // gate logits of this lane's candidates (up to kMaxCand / 64), all requested before use
    constexpr int kPerLane = kMaxCand / 64;
    float gl[kPerLane], bl[kPerLane];
#pragma unroll
    for (int r = 0; r < kPerLane; r++) {
        const int c = min(lane + 64 * r, n_cand - 1);
        const int s = c >= es.m ? 1 : 0;
        gl[r] = es.g[s][es.row(c)];
        bl[r] = es.b[s][c - s * es.m];
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < kPerLane; r++) {
        const int c = lane + 64 * r;
        if (c < n_cand) {
            const float z = gl[r] + bl[r];
            wsh[c] = z;
            zmax = fmaxf(zmax, z);
        }
    }
    zmax = wave_max(zmax);
    float den = 0.0f;
    for (int c = lane; c < n_cand; c += 64) {
        const float ex = expf(wsh[c] - zmax);
        wsh[c] = ex;
        den += ex;
    }
    den = wave_sum(den);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // candidates in ascending order: batch xa holds c0 .. c0+7, batch xb c0+8 .. c0+15; each is
    // refilled with the candidates 16 further once it has been added
    auto merge_batch = [&](const uint32_t (&x)[kRowBatch][W], int c0) {
#pragma unroll
        for (int u = 0; u < kRowBatch; u++) {
            if (c0 + u < c_end) {
                const float wgt = wsh[c0 + u];
#pragma unroll
                for (int v = 0; v < VPT; v++) acc[v] = fmaf(wgt, active ? value(x[u], v) : 0.0f, acc[v]);
            }
        }
    };
    for (int c0 = c_begin; c0 < c_end; c0 += 2 * kRowBatch) {
        merge_batch(xa, c0);
        if (c0 + 2 * kRowBatch < c_end) load_batch(xa, c0 + 2 * kRowBatch);
        if (c0 + kRowBatch < c_end) {
            merge_batch(xb, c0 + kRowBatch);
            if (c0 + 3 * kRowBatch < c_end) load_batch(xb, c0 + 3 * kRowBatch);
        }
    }
    return den;
}

// The merged entry acc (one wavefront) is normalised, rotated and written as entry i of sequence
// seq: RMSNorm with the lane's weights nw, RoPE at position m*i, the record or key encoder.
// rl_pre (uniform): the cos/sin of position m*i already evaluated, pair j in lane rl_lane0 + j.
template <int VPT>
__device__ __forceinline__ void finish_entry(const CompressParams &P, float (&acc)[VPT], const float (&nw)[VPT],
                                             int64_t seq, int64_t i, uint8_t *idx_mirror = nullptr,
                                             const RopeLanes *rl_pre = nullptr, int rl_lane0 = 0) {
    const int lane = threadIdx.x & 63;
    const int m = P.m, D = P.D;
    const int d0 = lane * VPT;
    const bool active = d0 < D;
    // RMSNorm of the merged entry ("DeepSeek-V4 technical report walkthrough", section 2.3:
    // RMSNorm acts directly on the KV entries): x * w / sqrt(mean(x^2) + eps), before RoPE
    if (P.norm_w) {
        float ss = 0.0f;
        if (active) {
#pragma unroll
            for (int v = 0; v < VPT; v++) ss = fmaf(acc[v], acc[v], ss);
        }
        ss = __shfl(wave_sum(ss), 0);  // one value for every lane
        const float r = 1.0f / sqrtf(ss / (float)D + kNormEps);
#pragma unroll
        for (int v = 0; v < VPT; v++) acc[v] = acc[v] * r * nw[v];
    }

    // partial RoPE on the last R dims at position m*i (interleaved pairs); lane j < R/2
    // evaluates pair j's cos/sin and the owning lanes read them across the wavefront
    if (P.rope) {
        const int rs = D - P.R, npairs = P.R / 2;
        RopeLanes rl_own;
        if (!rl_pre) rl_own.eval(P.rt, npairs, (double)(m * i));
        const RopeLanes &rl = rl_pre ? *rl_pre : rl_own;
        if constexpr (VPT >= 2) {
#pragma unroll
            for (int v = 0; v < VPT; v += 2) {
                const int j = min(max((d0 - rs + v) / 2, 0), npairs - 1);
                const float2 cs = rl.get(rl_lane0 + j);
                if (active && d0 >= rs) {
                    const float x = acc[v], y = acc[v + 1];
                    acc[v] = x * cs.x - y * cs.y;
                    acc[v + 1] = x * cs.y + y * cs.x;
                }
            }
        } else {
            const float partner = __shfl_xor(acc[0], 1);
            const int j = min(max((d0 - rs) / 2, 0), npairs - 1);
            const float2 cs = rl.get(rl_lane0 + j);
            if (active && d0 >= rs) {
                const bool even = ((d0 - rs) & 1) == 0;
                const float x = even ? acc[0] : partner, y = even ? partner : acc[0];
                acc[0] = even ? (x * cs.x - y * cs.y) : (x * cs.y + y * cs.x);
            }
        }
    }

    const int64_t orow = P.out_row0 + seq * P.cap + i;
    if (P.to_idx)
        store_mxfp4<VPT>(acc, lane, active, D, P.idx, orow, idx_mirror);
    else
        store_record<VPT>(acc, d0, active, D, P.R, P.kv, orow);
}

// RMSNorm weights of this lane's dims (requested early so their latency overlaps the rows').
template <int VPT>
__device__ __forceinline__ void load_norm_weights(const CompressParams &P, float (&nw)[VPT]) {
    const int d0 = (threadIdx.x & 63) * VPT;
#pragma unroll
    for (int v = 0; v < VPT; v++) nw[v] = (P.norm_w && d0 < P.D) ? P.norm_w[d0 + v] : 0.0f;
}

// Entries whose candidates a whole workgroup of kEntryWaves wavefronts shares (gate per token,
// blocks of at least 64 tokens: the HCA blocks); every caller decides with this one rule.
constexpr int kEntryWaves = 8;
__host__ __device__ __forceinline__ bool entry_uses_workgroup(const CompressParams &P) {
    return P.G == 1 && P.m >= 64;
}

// Entry i of sequence seq, computed by one whole wavefront; row 0 of the sequence's streams
// is position tok0 (its streams and gates start n_tok rows further per sequence); wsh is the
// wavefront's scratch for the candidate weights.
template <int VPT, bool PK = false>
__device__ __forceinline__ void compress_entry(const CompressParams &P, float *wsh, int64_t seq, int64_t i,
                                               int64_t tok0, const RopeLanes *rl_pre = nullptr, int rl_lane0 = 0) {
    const int lane = threadIdx.x & 63;
    const int64_t x_off = seq * P.n_tok * P.D, g_off = seq * P.n_tok * P.G;
    const int m = P.m, D = P.D;
    const int d0 = lane * VPT;
    const bool active = d0 < D;
    const int n_cand = entry_candidates(P, i);
    auto row_of = [&](int64_t pos) -> int64_t { return P.ring ? pos % P.n_tok : pos - tok0; };
    float acc[VPT];
#pragma unroll
    for (int v = 0; v < VPT; v++) acc[v] = 0.0f;
    float nw[VPT];
    load_norm_weights<VPT>(P, nw);
    if (P.G == 1) {
        const float den = merge_gate1<VPT, PK>(P, wsh, seq, i, tok0, 0, n_cand, acc);
#pragma unroll
        for (int v = 0; v < VPT; v++) acc[v] = acc[v] / den;
    } else {
        // per-channel gates: online softmax over the candidates for each of this lane's dims
        float mx[VPT], l[VPT];
#pragma unroll
        for (int v = 0; v < VPT; v++) { mx[v] = -INFINITY; l[v] = 0.0f; }
        for (int c = 0; c < n_cand; c++) {
            int s = c / m, j = c % m;
            int64_t r = row_of((s == 0 ? m * i : m * (i - 1)) + j);
            float x[VPT];
            load_row<VPT>(s == 0 ? P.x0 : P.x1, P.bf16_in, r, D, d0, active, x, x_off);
            const float *g = (s == 0 ? P.g0 : P.g1) + g_off + r * D + d0;
            const float *bb = (s == 0 ? P.b0 : P.b1) + (int64_t)j * D + d0;
#pragma unroll
            for (int v = 0; v < VPT; v++) {
                float z = active ? g[v] + bb[v] : 0.0f;
                float mn = fmaxf(mx[v], z);
                float corr = (mx[v] == -INFINITY) ? 0.0f : expf(mx[v] - mn);
                float ex = (z == -INFINITY) ? 0.0f : expf(z - mn);
                l[v] = l[v] * corr + ex;
                acc[v] = acc[v] * corr + ex * x[v];
                mx[v] = mn;
            }
        }
#pragma unroll
        for (int v = 0; v < VPT; v++) acc[v] = acc[v] / l[v];
    }
    finish_entry<VPT>(P, acc, nw, seq, i, nullptr, rl_pre, rl_lane0);
}

// Entry i of sequence seq computed by all kEntryWaves wavefronts of the workgroup (gate per
// token): wavefront w accumulates its contiguous share of the candidates, the partial sums meet
// in LDS (red: kEntryWaves x D floats) and wavefront 0 adds them in wavefront order, divides by
// the weight sum and finishes the entry.  wsh: kEntryWaves x kMaxCand floats.  Every thread of
// the workgroup must call it.
template <int VPT, bool PK = false>
__device__ __forceinline__ void compress_entry_wg(const CompressParams &P, float *wsh, float *red, int64_t seq,
                                                  int64_t i, int64_t tok0) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int d0 = lane * VPT;
    const bool active = d0 < P.D;
    const int n_cand = entry_candidates(P, i);
    const int per = (n_cand + kEntryWaves - 1) / kEntryWaves;
    const int c0 = min(n_cand, wv * per), c1 = min(n_cand, c0 + per);
    float acc[VPT];
#pragma unroll
    for (int v = 0; v < VPT; v++) acc[v] = 0.0f;
    float nw[VPT];
    if (wv == 0) load_norm_weights<VPT>(P, nw);
    const float den = merge_gate1<VPT, PK>(P, wsh + wv * kMaxCand, seq, i, tok0, c0, c1, acc);
    if (active) {
#pragma unroll
        for (int v = 0; v < VPT; v++) red[wv * P.D + d0 + v] = acc[v];
    }
    __syncthreads();
    if (wv != 0) return;
#pragma unroll
    for (int v = 0; v < VPT; v++) {
        float sum = 0.0f;
        if (active) {
            sum = red[d0 + v];
            for (int w = 1; w < kEntryWaves; w++) sum += red[w * P.D + d0 + v];
        }
        acc[v] = sum / den;
    }
    finish_entry<VPT>(P, acc, nw, seq, i);
}

// Two-phase form of compress_entry for short gate-per-token entries of BF16 streams (G = 1, at
// most kRowBatchMax candidates; a ring holds exactly 2m rows), for a wavefront that has other
// work between the two phases.  key_prefetch only issues loads (row words, gate logits, biases,
// norm weights; no branch on a loaded value, so nothing waits for them); key_finish (the same
// wavefront, later) merges and finishes the entry.  The arithmetic is that of compress_entry
// step for step (same maxima, exponentials, wavefront sums and fma order), so the entry is
// bitwise the same.
constexpr int kRowBatchMax = 8;
__host__ __device__ __forceinline__ bool entry_two_phase(const CompressParams &P) {
    return P.G == 1 && P.bf16_in && P.vec_in && (P.n_streams == 2 ? 2 * P.m : P.m) <= kRowBatchMax &&
           (!P.ring || P.n_tok == 2 * P.m);
}

template <int VPT>
struct KeyPrefetch {
    uint32_t raw[kRowBatchMax][(VPT + 1) / 2];  // BF16 pairs of this lane's dims, per candidate
    float gl, bl;                                 // gate logit and positional bias of candidate lane
    float nw[VPT];                                // RMSNorm weights of this lane's dims
};

// Stream row of candidate c of entry i (c / m: 0 own block, 1 the B-block i - 1); a ring of 2m
// rows holds position p at p mod 2m, which for these positions needs no division.
__device__ __forceinline__ int64_t candidate_row2(const CompressParams &P, int64_t i, int c, int64_t tok0) {
    const int m = P.m, s = c / m, j = c - s * m;
    const int64_t blk = s == 0 ? i : i - 1;
    return P.ring ? (int64_t)m * (blk & 1) + j : (int64_t)m * blk + j - tok0;
}

template <int VPT>
__device__ __forceinline__ void key_prefetch(const CompressParams &P, int64_t seq, int64_t i, int64_t tok0,
                                             KeyPrefetch<VPT> &kp) {
    static_assert(VPT % 2 == 0, "BF16 pairs");
    const int lane = threadIdx.x & 63;
    const int64_t x_off = seq * P.n_tok * P.D, g_off = seq * P.n_tok * P.G;
    const int d0 = lane * VPT;  // D = 64 * VPT: every lane is active
    const int n_cand = entry_candidates(P, i);
#pragma unroll
    for (int u = 0; u < kRowBatchMax; u++) {
        const int c = min(u, n_cand - 1);
        const uint16_t *x = (const uint16_t *)(c < P.m ? P.x0 : P.x1);
        const uint32_t *src = (const uint32_t *)(x + x_off + candidate_row2(P, i, c, tok0) * P.D + d0);
        if constexpr (VPT == 8) {  // vec_in: the lane's 16 bytes in one load
            const uint4 q = *(const uint4 *)src;
            kp.raw[u][0] = q.x; kp.raw[u][1] = q.y; kp.raw[u][2] = q.z; kp.raw[u][3] = q.w;
        } else {
#pragma unroll
            for (int w = 0; w < VPT / 2; w++) kp.raw[u][w] = src[w];
        }
    }
    const int c = min(lane, n_cand - 1);
    kp.gl = (c < P.m ? P.g0 : P.g1)[g_off + candidate_row2(P, i, c, tok0)];
    kp.bl = (c < P.m ? P.b0 : P.b1)[c % P.m];
#pragma unroll
    for (int v = 0; v < VPT; v++) kp.nw[v] = 0.0f;
    if (P.norm_w) {
#pragma unroll
        for (int v = 0; v < VPT; v++) kp.nw[v] = P.norm_w[d0 + v];
    }
}

// Lane l's float, read by the whole wavefront (l a constant).
__device__ __forceinline__ float lane_value(float v, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}

// The candidates' weights are read lane by lane instead of with wavefront reductions: lanes
// past the candidates hold -inf and 0, so the maximum is the candidates' maximum, and the
// butterfly sum over 64 lanes (xor 32, 16, 8 add zeros exactly) is ((e0 + e4) + (e2 + e6)) +
// ((e1 + e5) + (e3 + e7)), written here in that order.
// The merge of a prefetched entry into acc (divided by the weight sum): compress_entry's
// arithmetic step for step.
template <int VPT>
__device__ __forceinline__ void key_merge(const CompressParams &P, KeyPrefetch<VPT> &kp, int64_t i,
                                          float (&acc)[VPT]) {
    const int lane = threadIdx.x & 63;
    const int n_cand = entry_candidates(P, i);
    const float z = lane < n_cand ? kp.gl + kp.bl : -INFINITY;
    float zmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kRowBatchMax; u++) zmax = fmaxf(zmax, lane_value(z, u));
    const float ex = lane < n_cand ? expf(z - zmax) : 0.0f;
    float e[kRowBatchMax];
#pragma unroll
    for (int u = 0; u < kRowBatchMax; u++) e[u] = lane_value(ex, u);
    const float den = ((e[0] + e[4]) + (e[2] + e[6])) + ((e[1] + e[5]) + (e[3] + e[7]));
#pragma unroll
    for (int v = 0; v < VPT; v++) acc[v] = 0.0f;
#pragma unroll
    for (int u = 0; u < kRowBatchMax; u++) {
        if (u < n_cand) {
#pragma unroll
            for (int v = 0; v < VPT; v++) {
                const uint32_t w2 = kp.raw[u][v / 2];
                acc[v] = fmaf(e[u], bf16_to_f32((uint16_t)((v & 1) ? (w2 >> 16) : (w2 & 0xFFFFu))), acc[v]);
            }
        }
    }
#pragma unroll
    for (int v = 0; v < VPT; v++) acc[v] = acc[v] / den;
}

template <int VPT>
__device__ __forceinline__ void key_finish(const CompressParams &P, KeyPrefetch<VPT> &kp, int64_t seq, int64_t i,
                                           uint8_t *idx_mirror, bool to_global = true) {
    const int lane = threadIdx.x & 63;
    float acc[VPT];
    key_merge<VPT>(P, kp, i, acc);
    // finish_entry's steps for an indexer key (RMSNorm if any, no RoPE, MXFP4), without its
    // other branches: this runs once per query in a kernel whose other wavefronts never do
    if (P.norm_w) {
        float ss = 0.0f;
#pragma unroll
        for (int v = 0; v < VPT; v++) ss = fmaf(acc[v], acc[v], ss);
        ss = __shfl(wave_sum(ss), 0);
        const float r = 1.0f / sqrtf(ss / (float)P.D + kNormEps);
#pragma unroll
        for (int v = 0; v < VPT; v++) acc[v] = acc[v] * r * kp.nw[v];
    }
    store_mxfp4<VPT>(acc, lane, true, P.D, P.idx, P.out_row0 + seq * P.cap + i, idx_mirror, to_global);
}

// A prefetched entry merged and finished as compress_entry would (RoPE from rl_pre when given).
template <int VPT>
__device__ __forceinline__ void prefetched_entry_finish(const CompressParams &P, KeyPrefetch<VPT> &kp, int64_t seq,
                                                        int64_t i, const RopeLanes *rl_pre, int rl_lane0) {
    float acc[VPT];
    key_merge<VPT>(P, kp, i, acc);
    finish_entry<VPT>(P, acc, kp.nw, seq, i, nullptr, rl_pre, rl_lane0);
}

// Kernel parameters of a checked CompressArgs (host).
CompressParams compress_params(const CompressArgs &a);

}  // namespace v4a
