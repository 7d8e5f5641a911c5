// common.hpp -- device helpers shared by the gfx950 kernels of the CSA/HCA hot path:
// number-format encoders written from the OCP FP8/MX format definitions, bf16 packing,
// wavefront reductions, and the host-side launch interface of each kernel family.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>
#include <stdint.h>

#include "../../include/v4attn.h"

namespace v4a {

constexpr int kWave = 64;

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// Direct-to-LDS copies (global_load_lds), written out as instructions: lane l's 16 (or 4)
// bytes from gsrc land at LDS byte lds + 16 l (or 4 l); lds is uniform over the wavefront.
// The compiler does not see these as LDS writes, so its conservative rule (wait for every
// direct-to-LDS copy in flight before any LDS access) does not drain a prefetched buffer; the
// caller waits for the copies with an explicit s_waitcnt vmcnt before the buffer is read, and
// orders the copies after the reads of the buffer they overwrite (barrier or program order).
// No VGPR is written by these instructions.
__device__ __forceinline__ void lds_copy16(const void *gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gsrc) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy16_nt(const void *gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off nt" ::"s"(lds), "v"(gsrc) : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void *gsrc, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gsrc) : "memory", "m0");
}
// LDS byte address of a shared-memory object
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// bf16 <-> f32.  Encoding rounds to nearest even on bit 16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = fbits(x);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return bitsf((uint32_t)b << 16); }

// OCP FP8 E4M3FN codes (nearest, ties to even, the sign kept: a negative value rounding to zero
// gives 0x80) of two or four fp32 values, byte v holding the code of the v-th, from the hardware
// conversion v_cvt_pk_fp8_f32.  For every finite |x| <= 449 its code equals the plain nearest-
// even E4M3 encoding saturating at 448 (checked exhaustively, all 2.28e9 such fp32 values, on
// gfx950); callers pass values of magnitude at most 448 (1 + 2^-23).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// E2M1 (FP4) encoding of a value already divided by its block scale: nearest with ties
// to the even code, saturating at 6; bit 3 is the sign.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    uint32_t s = (fbits(v) >> 28) & 0x8u;
    float a = fabsf(v);
    uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
               : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
    return s | c;
}

// floor(log2(a)) - 2 for a > 0, clamped to [-127, 127]: the MXFP4 block exponent.
__device__ __forceinline__ int mx_block_exp(float amax) {
    if (!(amax > 0.0f)) return -127;
    uint32_t u = fbits(amax);
    int e = (int)(u >> 23);
    int fl = e ? e - 127 : -127 - (__builtin_clz(u & 0x7FFFFFu) - 9);  // subnormal: below 2^-126
    int X = fl - 2;
    return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Wavefront reductions over all 64 lanes (result in every lane).
__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Orderable key of an fp32 score: larger score -> larger unsigned key (-0 canonical +0).
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = fbits(s);
    if (u == 0x80000000u) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Orderable 16-bit key of an fp32 score held in BF16: the score is rounded to the nearest
// BF16 value with ties to the even one (integer rounding of the top 16 bits; scores are
// finite), a -0 result becomes +0, and the 16 bits are mapped as score_key maps 32.
// Shifted left by 16 it orders exactly as score_key of that BF16 value.
__device__ __forceinline__ uint32_t score_key16(float s) {
    uint32_t u = fbits(s);
    u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    if (u == 0x8000u) u = 0;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
}

// RoPE frequencies of the R/2 interleaved pairs: inv_freq_j = theta^(-2j/R), computed on the
// host in double (a kernel argument, so no kernel evaluates pow).
constexpr int kMaxRopePairs = 32;
struct RopeTable {
    double inv_freq[kMaxRopePairs];
};

// cos and sin of the angle pos * inv_freq (double), each rounded once to fp32.  The angle is
// first reduced by pi/2 with a two-term constant (Cody-Waite), which keeps the double sin/cos
// on |r| <= pi/4 for positions up to millions.
__device__ __forceinline__ void rope_cs_freq(double pos, double inv_freq, float *c, float *s) {
    const double kPio2Hi = 1.5707963267948966;       // pi/2 rounded to double
    const double kPio2Lo = 6.123233995736766e-17;    // pi/2 - kPio2Hi
    const double kTwoOverPi = 0.6366197723675814;
    const double ang = pos * inv_freq;
    const double k = rint(ang * kTwoOverPi);
    double r = fma(-k, kPio2Hi, ang);
    r = fma(-k, kPio2Lo, r);
    const double sr = sin(r), cr = cos(r);
    switch (((long long)k) & 3) {
        case 0: *c = (float)cr; *s = (float)sr; break;
        case 1: *c = (float)-sr; *s = (float)cr; break;
        case 2: *c = (float)-cr; *s = (float)-sr; break;
        default: *c = (float)sr; *s = (float)-cr; break;
    }
}

// Every lane of the wavefront gets (cos, sin) of pair `want` (< R/2) at position pos: lane j
// < R/2 evaluates pair j once and the values travel by cross-lane reads.  Must be reached by
// the whole wavefront.
struct RopeLanes {
    float c, s;
    __device__ __forceinline__ void eval(const RopeTable &T, int npairs, double pos) {
        const int lane = threadIdx.x & 63;
        c = 1.0f;
        s = 0.0f;
        if (lane < npairs) rope_cs_freq(pos, T.inv_freq[lane], &c, &s);
    }
    // Two positions in one pass (npairs <= 32): lane j < 32 evaluates pair j at pos0, lane
    // 32 + j pair j at pos1; get(j) and get(32 + j) then serve them.
    __device__ __forceinline__ void eval2(const RopeTable &T, int npairs, double pos0, double pos1) {
        const int lane = threadIdx.x & 63, j = lane & 31;
        c = 1.0f;
        s = 0.0f;
        if (j < npairs) rope_cs_freq(lane < 32 ? pos0 : pos1, T.inv_freq[j], &c, &s);
    }
    __device__ __forceinline__ float2 get(int want) const {
        return make_float2(__shfl(c, want), __shfl(s, want));
    }
};

}  // namespace v4a

// ---------------------------------------------------------------- host side ----------
namespace v4a {

// Kernel timing: while a trace is armed, claims the next pair of the library's timing events
// for `kernel` and returns true; false otherwise (api.hip).
bool trace_claim(const char *kernel, hipEvent_t *start, hipEvent_t *stop);

// Every kernel launch of the library: while a trace is armed the launch carries a start and a
// stop event that time the dispatch itself (hipExtLaunchKernelGGL); otherwise a plain launch.
#define V4A_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                                      \
    do {                                                                                               \
        hipEvent_t v4a_ev0_, v4a_ev1_;                                                                 \
        if (::v4a::trace_claim(name, &v4a_ev0_, &v4a_ev1_))                                            \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, v4a_ev0_, v4a_ev1_, 0, __VA_ARGS__); \
        else                                                                                           \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                       \
    } while (0)

// Per-sequence / per-query positions travel as kernel arguments (no host-to-device copy,
// so every call stays asynchronous and capturable).
constexpr int kMaxSeq = 128;
constexpr int kHistBins = 4096;   // top-12-bit histogram of the orderable score keys
constexpr int kHistCopies = 2;    // copies of each query's histogram (contention spreading)

// Histogram copies per query: many workgroups score one decode query and spread their adds
// over kHistCopies copies; a prefill chunk has few workgroups per query and keeps one copy.
inline int hist_copies(int64_t BQ) { return BQ <= 32 ? kHistCopies : 1; }

struct QueryPos {
    int mode;  // 0: pos[qi] per query (B*Q <= kMaxSeq); 1: pos[b] + j for query j of sequence b
    int Q, m;
    int64_t pos[kMaxSeq];
    int64_t n_ent[kMaxSeq];
};

__host__ __device__ __forceinline__ int64_t query_pos(const QueryPos &P, int qi) {
    const int b = qi / P.Q, j = qi % P.Q;
    return P.mode == 0 ? P.pos[qi] : P.pos[b] + j;
}

__host__ __device__ __forceinline__ int64_t visible_keys(const QueryPos &P, int qi) {
    int b = qi / P.Q;
    int64_t pos = query_pos(P, qi);
    int64_t v = (pos + 1) / P.m;
    int64_t n = P.n_ent[b];
    v = v < n ? v : n;
    return v < 0 ? 0 : v;
}

// The queries an attention launch serves.  Mode 0 (decode): query b is a new token of sequence
// b / qps (qps consecutive tokens per sequence, one unless a multi-token step), described by the
// arrays; the window buffer holds win_stride rows per sequence.  Mode 1 (prefill): query b is
// the token at tok0 + b of one sequence; its window is the W stream rows ending at itself, read
// from a buffer whose row 0 holds position tok0 - n_prev; it attends over fixed_ent top-k entries
// (CSA) or, when fixed_ent is 0, over its visible prefix of the n_total cached entries (ratio m).
struct SeqInfo {
    int mode;
    int ring;                  // mode 0: the window buffer is a ring (position p at row p mod win_stride)
    int64_t tok0;
    int n_prev, W, m, fixed_ent;
    int64_t n_total;
    int qps;                   // mode 0: queries per sequence (0 or 1: one)
    int win_stride;            // mode 0: window rows per sequence (0: W)
    int32_t n_ent[kMaxSeq];    // entry keys of query b (k for CSA, visible entries for HCA)
    int32_t win_len[kMaxSeq];
    int32_t win_off[kMaxSeq];  // mode 0, rows: query b's oldest window row within its sequence's rows
    int64_t q_pos[kMaxSeq];
};

// Cache slot (sequence) of query b.
__host__ __device__ __forceinline__ int sq_slot(const SeqInfo &S, int b) {
    return (!S.mode && S.qps > 1) ? b / S.qps : b;
}

__host__ __device__ __forceinline__ int64_t sq_pos(const SeqInfo &S, int b) {
    return S.mode ? S.tok0 + b : S.q_pos[b];
}
__host__ __device__ __forceinline__ int sq_win_len(const SeqInfo &S, int b) {
    if (!S.mode) return S.win_len[b];
    const int64_t t = S.tok0 + b;
    return (int)(t + 1 < (int64_t)S.W ? t + 1 : (int64_t)S.W);
}
__host__ __device__ __forceinline__ int sq_n_ent(const SeqInfo &S, int b) {
    if (!S.mode) return S.n_ent[b];
    if (S.fixed_ent) return S.fixed_ent;
    const int64_t v = (S.tok0 + b + 1) / S.m;
    return (int)(v < S.n_total ? v : S.n_total);
}
// Window rows per sequence in mode 0.
__host__ __device__ __forceinline__ int sq_win_stride(const SeqInfo &S, int W) {
    return S.win_stride > 0 ? S.win_stride : W;
}
// Row of the window buffer holding query b's oldest window token.
__host__ __device__ __forceinline__ int64_t sq_win_row0(const SeqInfo &S, int b, int W) {
    return S.mode ? (int64_t)b + S.n_prev - sq_win_len(S, b) + 1
                  : (int64_t)sq_slot(S, b) * sq_win_stride(S, W) + S.win_off[b];
}

// Rows of query b's window tokens, token j = 0 the oldest: consecutive rows from the oldest's,
// or, for a ring (mode 0), the sequence's win_stride rows with position p at row p mod win_stride.
struct WinRows {
    int64_t base;
    int start, W;
    bool ring;
    __host__ __device__ __forceinline__ int64_t row(int j) const {
        if (!ring) return base + j;
        const int r = start + j;
        return base + (r >= W ? r - W : r);
    }
};
__host__ __device__ __forceinline__ WinRows sq_win_rows(const SeqInfo &S, int b, int W) {
    WinRows w;
    w.W = W;
    w.ring = S.ring && !S.mode;
    w.start = 0;
    if (w.ring) {
        const int stride = sq_win_stride(S, W);
        w.W = stride;
        w.base = (int64_t)sq_slot(S, b) * stride;
        const int64_t p0 = S.q_pos[b] - S.win_len[b] + 1;  // the oldest window position, >= 0
        w.start = (int)(p0 % stride);
    } else {
        w.base = sq_win_row0(S, b, W);
    }
    return w;
}

void set_error(const char *fmt, ...);
void fill_rope_table(RopeTable &t, int R, double theta);

hipError_t launch_quantize_kv(const float *x, int64_t rows, const v4a_kv &out, int64_t row0,
                              hipStream_t s);
hipError_t launch_quantize_mxfp4(const float *x, int64_t rows, const v4a_idx &out, int64_t row0,
                                 hipStream_t s);

struct CompressArgs {
    const void *x[2];        // stream A (or the HCA stream) and stream B (CSA only)
    const float *gate[2];
    const float *bias[2];
    int n_streams;           // 2 for CSA (overlapped), 1 for HCA
    bool bf16_in;
    int D, G, m;
    int64_t tok0, n_tok, first_entry, n_entries;
    bool rope;
    int R;
    double theta;
    const v4a_kv *kv;        // exactly one of kv / idx
    const v4a_idx *idx;
    int b0, n_seq;           // output slots b0 .. b0+n_seq-1; stream s at x + s * n_tok * D
    const float *norm_w;     // [D] RMSNorm weights of the merged entry, or NULL
    bool ring;               // rows are a ring: position p at row p mod n_tok (else p - tok0)
};
constexpr float kNormEps = 1e-6f;  // RMSNorm epsilon of the compressed entries
hipError_t launch_compress(const CompressArgs &a, hipStream_t s);
// One launch: the entries (key: records or indexer keys) of entry[b] for every sequence b with
// entry[b] >= 0 (each sequence's streams hold rows from blocks_before blocks before the entry's
// own, or a ring), plus clearing zero_bytes at zero.
hipError_t launch_decode_prologue(const CompressArgs &key, int blocks_before, int B, const int64_t *entry,
                                  void *zero, size_t zero_bytes, hipStream_t s);

struct IndexerArgs {
    const v4a_idx *keys;
    const v4a_idx *q;
    const float *w;
    int B, Q, H_I;
    int64_t n_max;            // max visible keys over the queries (grid size)
    int64_t key_stride;       // score-key row stride (a multiple of 64 >= n_max)
    void *score_keys;         // [B*Q][key_stride] orderable keys (or NULL): uint32 of the fp32
                              // scores, or uint16 of the BF16 scores when key16
    bool key16;
    float *scores;            // [B*Q][n_max] raw scores (or NULL)
    uint32_t *hist;           // [B*Q][copies][4096] histogram of the top 12 key bits (or NULL)
    int hist_copies;
    const CompressArgs *key_rec;  // decode step: compress each query's new key (MXFP4,
                                  // d = 128, Q = 1, two-phase entries) in the scoring kernel
};
hipError_t launch_indexer(const IndexerArgs &a, const QueryPos &qp, hipStream_t s);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);

struct SelectArgs {
    const void *score_keys;       // [BQ][key_stride] uint32, or uint16 when key16
    int64_t key_stride;
    bool key16;
    const uint32_t *hist;         // [BQ][copies][4096]
    int hist_copies;
    int64_t n_max;
    int BQ, k;
    uint32_t *list;               // [BQ][slices * kSelSlice][2]: (index, score key) at or above the threshold bin
    uint32_t *counts;             // [BQ][slices] entries listed per slice
    int32_t *meta;                // [BQ][2]: threshold bin, count above it
    int32_t *out;                 // [BQ][k]
    // optional: the decode step's entry records, compressed by B extra workgroups of the final
    // selection's launch (query b = sequence b, one query each; the entry is the one its
    // position completes, if any)
    const CompressArgs *rec;
    // optional, with rec: the histograms (hist, writable), which the same extra workgroups
    // clear after the scan, their only reader, has finished (left clear for the next call)
    uint32_t *hist_clear;
};
int select_slices(int64_t n_max);
constexpr int kSelSlice = 8192;
inline int64_t score_key_stride(int64_t n_max) { return (n_max + 63) / 64 * 64; }
hipError_t launch_select(const SelectArgs &a, const QueryPos &qp, hipStream_t s);

struct AttnArgs {
    const void *q;
    bool q_bf16;
    int B, H, D, R;
    const v4a_kv *kv;
    int64_t kv_bstride;       // record rows between consecutive queries' caches (cap, or 0)
    const int32_t *topk;      // [B][k] or NULL (dense)
    int k;
    const void *win;
    bool win_bf16;
    int W;
    const float *sink;
    float scale;
    bool rope_inv;
    double theta;
    void *out;
    bool out_bf16;
    float *partial;           // workspace for split partials (or NULL when split_cap == 1)
    int target_splits;        // splits aimed at per sequence
    int split_cap;            // max splits of any sequence (partial stride)
    const float *q_norm_w;    // [D]: queries arrive projected only; RMSNorm + RoPE in the kernel
    bool no_split;            // every (query, head group) attends over all its keys in one
                              // workgroup: full waves of 64-head workgroups, then 16-head ones
};
bool attn_uses_mfma(const AttnArgs &a);

struct OutProjArgs {
    const void *o;            // [T][H*D] bf16: the attention output, heads in order
    int T, H, D, G, r, d;
    const void *wg;           // [G][r][H*D/G] bf16
    const void *wf;           // [d][G*r] bf16
    void *y;                  // [T][G*r] bf16 (workspace): the reduced groups, concatenated
    void *out;                // [T][d]
    bool out_bf16;
};
hipError_t launch_output_projection(const OutProjArgs &a, hipStream_t s);
hipError_t launch_attention(const AttnArgs &a, const SeqInfo &sq, hipStream_t s);
void split_plan_host(int n_keys, int target, int *tps, int *splits);
constexpr int kAttnTile = 32;

}  // namespace v4a
