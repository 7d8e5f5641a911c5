// attention.hip -- a6/a7: shared-KV multi-query attention over compressed entries plus the
// sliding window, with the attention sink, split over keys and combined in a fixed order.
// "DeepSeek V4 technical report explained" (firecat-web.com), item 2 "Hybrid attention":
// multi-query attention over the selected compressed entries, head dim 512, partial RoPE on
// the last 64 dims, a 128-token sliding window and a learnable sink logit.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: the window branch joins
// the core attention and the sink is a learnable extra term of the softmax denominator.
// "DeepSeek-V4: the engineering answer to million-token context" (mewclaw), "Partial RoPE":
// the attention output is treated so that values carry no absolute position (here: its RoPE
// slice is rotated back by the query position).
//
// Keys of sequence b, in order: its entries (the top-k indices for CSA, the visible prefix
// for HCA) then its window tokens; every key is also its own value over all D dims.
//
// MFMA kernel (FP8/BF16 records, BF16 queries and window).  A workgroup owns one sequence and
// one split of its keys, 16 heads per wavefront: either all heads (up to 8 wavefronts, for
// grids that fill the chip) or 64 of them (4 wavefronts); in the latter case with 128 heads
// the two head-group workgroups of a split get linear ids 8 apart, so they land on the same
// XCD and share its L2 for the key tiles.  Per tile of 32 keys:
//   staging: an entry tile is its 32 records copied byte for byte into LDS rows (FP8 codes,
//            then BF16 RoPE dims) by direct-to-LDS loads issued one tile ahead; a window tile
//            (BF16 window) is copied the same way as BF16 rows; a tile mixing entries and
//            window tokens, or an fp32 window, is written as BF16 rows by the wavefronts;
//   scores:  S^T = E Q^T with v_mfma_f32_16x16x32_bf16 (A = 16 keys x 32 dims read key-major,
//            FP8 codes converted exactly to BF16 in registers; B = the wavefront's 16 query
//            heads held in registers), accumulating the FP8 dims and the BF16 RoPE dims
//            separately so the per-entry scale folds in as s = scale_e * (q.codes) + q.rope;
//   softmax: online, in the exp2 domain, each lane owning one head and 8 keys;
//   values:  O^T += E^T P^T with A = 16 dims x 32 keys read transposed from the same rows
//            (gfx950 transpose LDS reads) and B = the lane's own probabilities (times scale_e
//            for the FP8 dims), whose key order the A reads follow, so P never leaves
//            registers.
// A split's (m, l, O) go to the workspace unless the sequence has a single split, in which
// case the workgroup finishes the output itself (sink, normalisation, inverse RoPE, cast).
// Split boundaries depend only on the sequence's own key count.
#include <type_traits>

#include "common.hpp"

namespace v4a {

constexpr int kTile = 32;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running maximum may lag the scores
constexpr int kMaxSelKeys = 2048;  // top-k entries per sequence (k <= 2048)
constexpr int kQkAhead = 1;        // score k-steps whose operands are requested ahead of use
constexpr int kPvAhead = 2;        // value dim tiles whose operands are requested ahead of use

struct AttnParams {
    const void *q;           // [B][H][D]
    bool q_bf16;
    int B, H, D, R;
    int fmt;                 // v4a_kv_fmt
    const uint8_t *nope;     // FP8: [B][cap][D-R]; F32: float [B][cap][D]
    const uint16_t *rope;    // [B][cap][R]
    const float *kscale;     // [B][cap]
    int64_t cap;
    int64_t kv_bstride;      // record rows between consecutive queries' caches (cap, or 0)
    const int32_t *topk;     // [B][k] or NULL
    int k;
    const void *win;         // [B][W][D] (decode) or the prefill stream [n_prev + C][D]
    bool win_bf16;
    int W;
    const float *sink;       // [H]
    float scale2;            // softmax scale * log2(e)
    bool rope_inv;
    const float *q_norm_w;   // [D] or NULL: queries arrive projected only (RMSNorm + RoPE here)
    RopeTable rt;
    void *out;
    bool out_bf16;
    uint16_t *part_o;        // BF16 [B][S][D/16][H][16]: per dim tile, the heads' 16 dims contiguous
    float *part_ml;          // [B][S][H][2]
    int S;                   // split capacity per sequence
    int target;              // splits aimed at per sequence
    int n_hg;                // head groups (workgroups) per split
    int hpw;                 // split-free launches: heads per workgroup (0: split layout)
    int item0;               // split-free launches: first (query, head group) item
};

static_assert(sizeof(AttnParams) + sizeof(SeqInfo) <= 4096, "kernel arguments");

constexpr int kShortTiles = 48;  // key lists of at most this many tiles take <= 2 tiles per split

__host__ __device__ __forceinline__ void split_plan(int n_keys, int target, int *tps, int *splits) {
    int tiles = (n_keys + kTile - 1) / kTile;
    int t = (tiles + target - 1) / target;
    if (t < 1) t = 1;
    // a short key list (a top-k selection and its window) is latency-bound: at most two tiles
    // per split, so each workgroup's serial chain is short (a function of the key count only)
    if (target > 1 && tiles <= kShortTiles && t > 2) t = 2;
    int s = (tiles + t - 1) / t;
    if (s < 1) s = 1;
    *tps = t;
    *splits = s;
}

// 2^x for a softmax weight or a rescale factor (x <= kRescaleSlack): the hardware v_exp_f32
// alone.  Results below 2^-126 come out as zero instead of subnormal; such a weight is below
// every rounding of the sums it enters (the running sum is at least 1).
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

// Element v (0..3) of four BF16 values packed in two words, as fp32.
__device__ __forceinline__ float bf16_half(const u32x2 &w, int v) {
    const uint32_t x = w[v >> 1];
    return bitsf((v & 1) ? (x & 0xFFFF0000u) : (x << 16));
}

// Factor turning one head's accumulated sum into the output: exp(m - M) / den with
// M = max(sink, m) and den = exp(sink - M) + l exp(m - M) (exp2 domain; 0 if nothing is left).
__device__ __forceinline__ float finish_factor(const AttnParams &P, int h, float m2, float l) {
    const float sink2 = P.sink[h] * kLog2e;
    const float M = fmaxf(sink2, m2);
    if (M == -INFINITY) return 0.0f;
    const float c = (m2 == -INFINITY) ? 0.0f : exp2f(m2 - M);
    const float den = exp2f(sink2 - M) + l * c;
    return den > 0.0f ? c / den : 0.0f;
}

// Inverse rotation (by -pos) of one RoPE pair (x, y) given its (cos, sin).
__device__ __forceinline__ float2 rope_unrotate(float2 cs, float x, float y) {
    return make_float2(x * cs.x + y * cs.y, -x * cs.y + y * cs.x);
}

// Output of head h of query b, dims d0 .. d0+3 (d0 a multiple of 4): one 8- or 16-byte store.
__device__ __forceinline__ void store_out4(const AttnParams &P, int b, int h, int d0, const float (&o)[4]) {
    const int64_t base = ((int64_t)b * P.H + h) * P.D + d0;
    if (P.out_bf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *(uint2 *)((uint16_t *)P.out + base) = make_uint2(lo, hi);
    } else {
        *(float4 *)((float *)P.out + base) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// Final output of head h, dims d0 .. d0+3: normalisation with the sink, inverse RoPE on the
// RoPE dims, cast.  Reached by the whole wavefront; rope_wave says whether any of its lanes
// holds RoPE dims (uniform), and only then is rl (the cos/sin of the query position, which the
// caller evaluates while its loads are in flight) read.
__device__ __forceinline__ void finish4(const AttnParams &P, int b, int h, int d0, bool rope_wave,
                                        const RopeLanes &rl, float m2, float l, float (&o)[4]) {
    const float f = finish_factor(P, h, m2, l);
#pragma unroll
    for (int v = 0; v < 4; v++) o[v] *= f;
    const int Dn = P.D - P.R;
    if (P.rope_inv && rope_wave) {
#pragma unroll
        for (int v = 0; v < 4; v += 2) {
            const float2 cs = rl.get(min(max((d0 + v - Dn) / 2, 0), P.R / 2 - 1));
            if (d0 >= Dn) {
                const float2 r = rope_unrotate(cs, o[v], o[v + 1]);
                o[v] = r.x;
                o[v + 1] = r.y;
            }
        }
    }
    store_out4(P, b, h, d0, o);
}

// ------------------------------------------------------------------ MFMA kernel -----
// Every head's arithmetic is the same whatever the workgroup shape, so results do not depend
// on it.  The key tile stays in LDS in its storage layout:
//   entry tiles: the 32 records' bytes (FP8 codes, then BF16 RoPE dims) are copied row by row
//     from the cache straight into LDS by direct-to-LDS loads, one tile ahead, without holding
//     registers (invalid keys copy a zero row);
//   window and mixed tiles: converted to BF16 rows by the wavefronts, as before;
//   scores:  the A operand (16 keys x 32 dims) is read key-major; FP8 codes are converted to
//            BF16 (exactly) in registers;
//   values:  the A operand (16 dims x 32 keys, the keys in the order of the lane's
//            probabilities) is read transposed with ds_read_b64_tr_b8 (FP8 codes) or two
//            ds_read_b64_tr_b16 (BF16 dims): within each group of 16 lanes, lane i receives
//            byte i%8 of the 8-byte chunks of lanes 2j + i/8 (tr_b8), or element i%4 of
//            the chunks of lanes 4j + i/4 (tr_b16), j = 0..7 (0..3); so source lane s of
//            group g addresses key k(g, s/2) at dims 16dt + 8(s%2) (FP8) or key k(g, s/4)
//            at dims 16dt + 4(s%4) (BF16), and lane i gets dim 16dt + i of those keys.
typedef __attribute__((address_space(3))) void *lds_ptr_t;
typedef __attribute__((address_space(1))) void *glb_ptr_t;
typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __align__(16) uint8_t g_zero_row[1024];  // source of the rows of invalid keys

// k(g, j): key j of the value operand's k-block g, in the order the lanes' probabilities
// follow (keys 4g..4g+3, then 16+4g..16+4g+3)
__device__ __forceinline__ int pv_key(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

__device__ __forceinline__ v8bf fp8x8_bf16(uint32_t lo, uint32_t hi) {
    uint4 v;
    v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return __builtin_bit_cast(v8bf, v);
}

template <int D, int R, int WAVES>
__global__ void __launch_bounds__(64 * WAVES, 8 / WAVES) attn_mfma_kernel(AttnParams P, SeqInfo Sq) {
    constexpr int NKS = D / 32;   // k-steps of the score MFMA
    constexpr int NDT = D / 16;   // dim tiles of the value MFMA
    constexpr int Dn = D - R;
    constexpr int RB8 = Dn + 2 * R;        // bytes of one record (FP8 codes, BF16 RoPE dims)
    constexpr int RC8 = RB8 / 16 + 1;      // 16-byte chunks per LDS row (one of padding)
    constexpr int RS8 = 16 * RC8;          // LDS row stride of an entry tile
    constexpr int RS16 = D + 8;            // LDS row stride of a BF16 tile (in BF16)
    static_assert(Dn % 32 == 0 && R % 32 == 0, "k-steps are all FP8 or all BF16 dims");
    static_assert(RB8 % 16 == 0 && RB8 / 16 <= 64 && 2 * D / 16 <= 64, "one direct-load instruction covers an LDS row");
    constexpr int TBYTES = kTile * RS8 > 2 * kTile * RS16 ? kTile * RS8 : 2 * kTile * RS16;
    // two tile buffers: an entry tile in its storage layout or a BF16 tile (window rows)
    __shared__ __attribute__((aligned(16))) uint8_t TB[2][TBYTES];
    __shared__ __attribute__((aligned(16))) float ksc[2][kTile];
    __shared__ int kval[2][kTile];
    __shared__ int32_t sidx[kMaxSelKeys];  // this split's top-k entry indices (CSA)

    // workgroup -> (sequence, split, head group); head groups of one split 8 ids apart.  A
    // split-free launch numbers (query, group of hpw heads) items from item0 instead.
    int L = blockIdx.x, hg = 0, p = L;
    const int hpg = P.hpw ? P.hpw : 16 * (int)(blockDim.x >> 6);  // heads per workgroup
    if (P.hpw) {
        const int item = P.item0 + L, groups = P.H / P.hpw;
        hg = item % groups;
        p = (item / groups) * P.S;  // split 0 of its query (S = 1)
    } else if (P.n_hg > 1) {  // n_hg a power of two
        hg = (L >> 3) & (P.n_hg - 1);
        p = (L >> (3 + __builtin_ctz((unsigned)P.n_hg))) * 8 + (L & 7);
    }
    const int b = p / P.S, split = p % P.S;
    if (b >= P.B) return;
    const int n_ent = sq_n_ent(Sq, b), n_keys = n_ent + sq_win_len(Sq, b);
    const WinRows wr = sq_win_rows(Sq, b, P.W);
    int tps, splits;
    split_plan(n_keys, P.target, &tps, &splits);
    if (split >= splits) return;
    const int kb0 = split * tps * kTile;
    const int kb1 = min(n_keys, kb0 + tps * kTile);

    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int h0 = hg * hpg + wv * 16;
    const bool wave_on = h0 < P.H;
    const int h = h0 + col;
    const int NT = blockDim.x;

    // query heads as the B operand of S^T: lane holds head h, dims 32*ks + 8*grp + j
    uint4 qu[NKS];  // the raw query rows: unconditional loads (a wavefront without heads reads head 0 and never uses it)
    {
        // the split's selected entry indices (read once for all its tiles) are requested before
        // the queries and stored to LDS as soon as they arrive, so the first tile's loads leave
        // while the queries are still in flight
        const int e1 = P.topk ? min(kb1, n_ent) : kb0;
        const bool has0 = kb0 + t < e1;
        const int sidx0 = has0 ? P.topk[(int64_t)b * P.k + kb0 + t] : 0;
        const uint16_t *qr = (const uint16_t *)P.q + ((int64_t)b * P.H + (wave_on ? h : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < NKS; ks++) qu[ks] = *(const uint4 *)(qr + 32 * ks + 8 * grp);
        if (has0) sidx[t] = sidx0;
        for (int j = kb0 + t + NT; j < e1; j += NT) sidx[j - kb0] = P.topk[(int64_t)b * P.k + j];
    }
    v4f O[NDT];
#pragma unroll
    for (int i = 0; i < NDT; i++) O[i] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;

    const int NW = NT >> 6;
    // ---- entry tile tb -> TB[q]: one direct-to-LDS load instruction per LDS row, wavefront w
    // taking rows w, w + NW, ...: M0 at the row's start, lane c copying 16-byte chunk c of the
    // key's record (FP8 codes, then BF16 RoPE dims).  The row's address arithmetic is scalar
    // except for the lane's choice of codes or RoPE dims; the row's entry index is uniform (the tile's position for a visible prefix; for a top-k
    // list lane r of every wavefront reads row r's index once per tile and readlane hands it over).
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int64_t krow0 = (int64_t)sq_slot(Sq, b) * P.kv_bstride;  // this sequence's first record row
    const uint8_t *const kbase_n = P.nope + krow0 * Dn;  // uniform
    const uint8_t *const kbase_r = (const uint8_t *)P.rope + krow0 * (2 * R);
    const int cap32 = (int)min(P.cap, (int64_t)INT32_MAX);
    auto issue_entries = [&](int tb, int q) {
        const int my_e = P.topk ? (lane < kTile ? sidx[tb + lane - kb0] : 0) : tb + lane;
        for (int r = wvu; r < kTile; r += NW) {
            const int e = P.topk ? __builtin_amdgcn_readlane(my_e, r) : tb + r;  // uniform
            const bool ok = e >= 0 && e < cap32;
            const bool lane_rope = 16 * lane >= Dn;
            const uint8_t *src = !ok ? g_zero_row
                                     : (lane_rope ? kbase_r + (uint64_t)(uint32_t)e * (2 * R) + (16 * lane - Dn)
                                                  : kbase_n + (uint64_t)(uint32_t)e * Dn + 16 * lane);
            if (lane < RB8 / 16) lds_copy16(src, lds_addr(&TB[q][r * RS8]));
        }
        if (wv == NW - 1 && lane < kTile) {
            const bool ok = my_e >= 0 && my_e < cap32;
            const float *src = ok ? P.kscale + krow0 + my_e : (const float *)g_zero_row;
            lds_copy4(src, lds_addr(&ksc[q][0]));
            kval[q][lane] = ok ? 1 : 0;
        }
    };
    // ---- window tile tb (BF16 rows, 16-byte aligned) -> TB[q] as BF16 LDS rows, one direct load
    // instruction per row as for the entry tiles; keys past the split read zeros and are masked
    const bool win_dma = P.win_bf16 && ((uintptr_t)P.win & 15) == 0;
    auto issue_window = [&](int tb, int q) {
        for (int r = wvu; r < kTile; r += NW) {
            const bool ok = tb + r < kb1;
            const uint8_t *src = ok ? (const uint8_t *)P.win + wr.row(tb + r - n_ent) * (2 * D) + 16 * lane : g_zero_row;
            if (lane < 2 * D / 16) lds_copy16(src, lds_addr(&TB[q][r * 2 * RS16]));
        }
        // a window tile's scales (1) and validity (key < kb1) are derived where they are used
    };
    // 0: entry tile (direct loads); 1: window tile (direct loads); 2: staged by the wavefronts
    // (entries and window rows mixed, or an fp32 window)
    auto tile_kind = [&](int tb) { return tb + kTile <= n_ent ? 0 : (tb >= n_ent && win_dma ? 1 : 2); };
    // ---- mixed tile (or fp32 window) -> TB[q] as BF16 rows, by the wavefronts: task (kg, seg) = keys
    // 4kg..4kg+3, dims 8seg..8seg+7; all loads of a task are issued before any is used
    constexpr int NSEG = D / 8;
    constexpr int NTASK = 8 * NSEG;
    auto stage_bf16 = [&](int tb, int q) {
        uint16_t *E16 = (uint16_t *)TB[q];
        const bool win_only = tb >= n_ent;
        for (int task = t; task < NTASK; task += NT) {
            const int kg = task & 7, seg = task >> 3, dim = 8 * seg;
            uint4 v[4];
            bool valid[4];
            float scl[4];
            if (win_only) {
                int64_t row[4];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    valid[j] = tb + 4 * kg + j < kb1;
                    row[j] = wr.row(valid[j] ? tb + 4 * kg + j - n_ent : 0);
                }
#pragma unroll
                for (int j = 0; j < 4; j++) v[j] = *(const uint4 *)((const uint16_t *)P.win + row[j] * D + dim);
#pragma unroll
                for (int j = 0; j < 4; j++) scl[j] = 1.0f;
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int kidx = tb + 4 * kg + j;
                    scl[j] = 0.0f;
                    v[j] = make_uint4(0, 0, 0, 0);
                    valid[j] = false;
                    if (kidx < n_ent) {
                        const int64_t e = P.topk ? (int64_t)sidx[kidx - kb0] : (int64_t)kidx;
                        if (e >= 0 && e < P.cap) {
                            const int64_t row = (int64_t)sq_slot(Sq, b) * P.kv_bstride + e;
                            valid[j] = true;
                            scl[j] = P.kscale[row];
                            if (dim < Dn) {
                                const uint2 c = *(const uint2 *)(P.nope + row * Dn + dim);
                                v[j] = __builtin_bit_cast(uint4, fp8x8_bf16(c.x, c.y));
                            } else {
                                v[j] = *(const uint4 *)(P.rope + row * R + (dim - Dn));
                            }
                        }
                    } else if (kidx < kb1) {
                        valid[j] = true;
                        scl[j] = 1.0f;
                        v[j] = *(const uint4 *)((const uint16_t *)P.win + wr.row(kidx - n_ent) * D + dim);
                    }
                }
            }
            if (seg == 0) {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    ksc[q][4 * kg + j] = scl[j];
                    kval[q][4 * kg + j] = valid[j] ? 1 : 0;
                }
            }
#pragma unroll
            for (int j = 0; j < 4; j++) *(uint4 *)(E16 + (4 * kg + j) * RS16 + dim) = valid[j] ? v[j] : make_uint4(0, 0, 0, 0);
        }
    };

    const float *tksc = ksc[0];
    const int *tkval = kval[0];
    const uint8_t *e8 = TB[0];
    const uint16_t *e16 = (const uint16_t *)TB[0];
    // A operand of the scores: key r, dims 32ks + 8grp .. +7
    auto qk_operand = [&](auto f8, int r, int ks) -> v8bf {
        if constexpr (decltype(f8)::value) {
            if (32 * ks < Dn) {
                const uint2 c = *(const uint2 *)(e8 + r * RS8 + 32 * ks + 8 * grp);
                return fp8x8_bf16(c.x, c.y);
            }
            return __builtin_bit_cast(v8bf, *(const uint4 *)(e8 + r * RS8 + Dn + 2 * (32 * ks - Dn + 8 * grp)));
        } else {
            return __builtin_bit_cast(v8bf, *(const uint4 *)(e16 + r * RS16 + 32 * ks + 8 * grp));
        }
    };
    // A operand of the values: dims 16dt + col, keys k(grp, 0..7)
    auto pv_operand = [&](auto f8, int dt) -> v8bf {
        if constexpr (decltype(f8)::value) {
            if (16 * dt < Dn) {
                const v2i_t c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) v2i_t *)(e8 + pv_key(grp, col >> 1) * RS8 + 16 * dt + 8 * (col & 1)));
                return fp8x8_bf16((uint32_t)c.x, (uint32_t)c.y);
            }
            const int off = Dn + 2 * (16 * dt - Dn + 4 * (col & 3));
            const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)(e8 + pv_key(grp, col >> 2) * RS8 + off));
            const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)(e8 + pv_key(grp, 4 + (col >> 2)) * RS8 + off));
            return __builtin_bit_cast(v8bf, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                                       __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
        } else {
            const int off = 16 * dt + 4 * (col & 3);
            const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)(e16 + pv_key(grp, col >> 2) * RS16 + off));
            const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) v4s_t *)(e16 + pv_key(grp, 4 + (col >> 2)) * RS16 + off));
            return __builtin_bit_cast(v8bf, make_uint4(__builtin_bit_cast(uint2, lo).x, __builtin_bit_cast(uint2, lo).y,
                                                       __builtin_bit_cast(uint2, hi).x, __builtin_bit_cast(uint2, hi).y));
        }
    };

    // the split's indices are in LDS before the first tile's loads (an LDS-only barrier: the
    // query loads may still be in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    int q = 0;
    auto issue = [&](int tb, int q) {
        const int kind = tile_kind(tb);
        if (kind == 0) issue_entries(tb, q);
        else if (kind == 1) issue_window(tb, q);
    };
    if (kb0 < kb1) issue(kb0, 0);
    // the queries as MFMA operands (after the first tile's loads left: the wait for the query
    // rows falls here)
    v8bf qT[NKS];
    {
        if (P.q_norm_w) {
            // Query prologue ("DeepSeek-V4 technical report walkthrough", section 2.3: RMSNorm acts
            // directly on the queries): RMSNorm of the head over its D dims (a head's dims sit in
            // lanes col, col+16, col+32, col+48), RoPE at the query position on the last R dims
            // (pairs inside a lane's 8 consecutive dims; Dn is a multiple of 32, so a k-step is
            // all RoPE dims or none), then BF16 (nearest even) as the MFMA operand.
            float ss = 0.0f;
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                const uint32_t w4[4] = {qu[ks].x, qu[ks].y, qu[ks].z, qu[ks].w};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float lo = __builtin_bit_cast(float, w4[j] << 16);
                    const float hi = __builtin_bit_cast(float, w4[j] & 0xFFFF0000u);
                    ss = fmaf(lo, lo, ss);
                    ss = fmaf(hi, hi, ss);
                }
            }
            ss += __shfl_xor(ss, 16);
            ss += __shfl_xor(ss, 32);
            const float rn = 1.0f / sqrtf(ss / (float)D + kNormEps);
            RopeLanes rl;
            rl.eval(P.rt, R / 2, (double)sq_pos(Sq, b));
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) {
                const uint32_t w4[4] = {qu[ks].x, qu[ks].y, qu[ks].z, qu[ks].w};
                const float4 wa = *(const float4 *)(P.q_norm_w + 32 * ks + 8 * grp);
                const float4 wb = *(const float4 *)(P.q_norm_w + 32 * ks + 8 * grp + 4);
                const float wv8[8] = {wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
                float y[8];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    y[2 * j] = __builtin_bit_cast(float, w4[j] << 16) * rn * wv8[2 * j];
                    y[2 * j + 1] = __builtin_bit_cast(float, w4[j] & 0xFFFF0000u) * rn * wv8[2 * j + 1];
                }
                if (32 * ks >= Dn) {
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const float2 cs = rl.get(16 * (ks - Dn / 32) + 4 * grp + i);
                        const float x0 = y[2 * i], x1 = y[2 * i + 1];
                        y[2 * i] = x0 * cs.x - x1 * cs.y;
                        y[2 * i + 1] = x0 * cs.y + x1 * cs.x;
                    }
                }
                v8bf qv;
#pragma unroll
                for (int j = 0; j < 8; j++) qv[j] = (__bf16)y[j];
                qT[ks] = qv;
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ks++) qT[ks] = __builtin_bit_cast(v8bf, qu[ks]);
        }
    }
    for (int tb = kb0; tb < kb1; tb += kTile) {
        const int kind = tile_kind(tb);  // uniform
        if (kind == 2) stage_bf16(tb, q);
        // this tile is in LDS: each wavefront waits for its own direct loads, then the barrier
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        // the next tile travels while this one is computed
        const int tn = tb + kTile;
        if (tn < kb1) issue(tn, q ^ 1);
        tksc = ksc[q];
        tkval = kval[q];
        if (wave_on && kind == 0) {
            e8 = TB[q];
                // ---- scores S^T for keys 0-15 (st = 0) and 16-31 (st = 1)
                float s2[8], ks8[8];
                // both halves' chains advance together, the raw operands of k-step ks + kQkAhead
                // requested before k-step ks is converted and multiplied
                v4f an2[2], ar2[2];
                {
                    uint2 raw8[NKS][2];
                    uint4 raw16[NKS][2];
                    auto request = [&](int ks) {
#pragma unroll
                        for (int st = 0; st < 2; st++) {
                            const uint8_t *row = e8 + (16 * st + col) * RS8;
                            if (32 * ks < Dn) raw8[ks][st] = *(const uint2 *)(row + 32 * ks + 8 * grp);
                            else raw16[ks][st] = *(const uint4 *)(row + Dn + 2 * (32 * ks - Dn + 8 * grp));
                        }
                    };
#pragma unroll
                    for (int st = 0; st < 2; st++) {
                        an2[st] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                        ar2[st] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
                    }
#pragma unroll
                    for (int ks = 0; ks < kQkAhead; ks++) request(ks);
#pragma unroll
                    for (int ks = 0; ks < NKS; ks++) {
                        if (ks + kQkAhead < NKS) request(ks + kQkAhead);
#pragma unroll
                        for (int st = 0; st < 2; st++) {
                            if (32 * ks < Dn)
                                an2[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_bf16(raw8[ks][st].x, raw8[ks][st].y),
                                                                                 qT[ks], an2[st], 0, 0, 0);
                            else
                                ar2[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, raw16[ks][st]),
                                                                                 qT[ks], ar2[st], 0, 0, 0);
                        }
                    }
                }
#pragma unroll
                for (int st = 0; st < 2; st++) {
                    const v4f an = an2[st], ar = ar2[st];
                    const float4 sc4 = *(const float4 *)(tksc + 16 * st + 4 * grp);
                    const int4 kv4 = *(const int4 *)(tkval + 16 * st + 4 * grp);
                    const float scv[4] = {sc4.x, sc4.y, sc4.z, sc4.w};
                    const int kvv[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        s2[4 * st + i] = kvv[i] ? P.scale2 * fmaf(scv[i], an[i], ar[i]) : -INFINITY;
                        ks8[4 * st + i] = scv[i];
                    }
                }
                // ---- online softmax (exp2 domain); lane: head h, keys {4grp+i, 16+4grp+i}
                float mt = s2[0];
#pragma unroll
                for (int i = 1; i < 8; i++) mt = fmaxf(mt, s2[i]);
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                // The running reference moves only when a score exceeds it by more than kRescaleSlack
                // (log2 units): until then the weights, at most 2^kRescaleSlack, stay exact in fp32 and
                // BF16 range, and O and l need no rescaling.  Same decision in all four lanes of a head.
                if (mt > m_run + kRescaleSlack) {
                    const float alpha = exp2_weight(m_run - mt);  // 0 when m_run = -inf
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < NDT; i++) O[i] *= alpha;
                    m_run = mt;
                }
                float pn[8], pr[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float pi = (s2[i] == -INFINITY) ? 0.0f : exp2_weight(s2[i] - m_run);
                    l_run += pi;
                    pr[i] = pi;
                    pn[i] = pi * ks8[i];
                }
                v8bf Pn, Pr;  // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    Pn[i] = (__bf16)pn[i];
                    Pr[i] = (__bf16)pr[i];
                }
                // ---- values O^T += E^T P^T; A row = dim 16*dt + col, keys {4grp..+3, 16+4grp..+3}
                {
                    // raw operands of dim tile dt + kPvAhead requested before tile dt is used
                    v2i_t rv8[NDT];
                    v4s_t rlo[NDT], rhi[NDT];
                    auto request = [&](int dt) {
                        if (16 * dt < Dn) {
                            rv8[dt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                                (__attribute__((address_space(3))) v2i_t *)(e8 + pv_key(grp, col >> 1) * RS8 + 16 * dt + 8 * (col & 1)));
                        } else {
                            const int off = Dn + 2 * (16 * dt - Dn + 4 * (col & 3));
                            rlo[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) v4s_t *)(e8 + pv_key(grp, col >> 2) * RS8 + off));
                            rhi[dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                (__attribute__((address_space(3))) v4s_t *)(e8 + pv_key(grp, 4 + (col >> 2)) * RS8 + off));
                        }
                    };
#pragma unroll
                    for (int dt = 0; dt < kPvAhead; dt++) request(dt);
#pragma unroll
                    for (int dt = 0; dt < NDT; dt++) {
                        if (dt + kPvAhead < NDT) request(dt + kPvAhead);
                        v8bf a;
                        if (16 * dt < Dn) {
                            a = fp8x8_bf16((uint32_t)rv8[dt].x, (uint32_t)rv8[dt].y);
                        } else {
                            const uint2 lo = __builtin_bit_cast(uint2, rlo[dt]), hi = __builtin_bit_cast(uint2, rhi[dt]);
                            a = __builtin_bit_cast(v8bf, make_uint4(lo.x, lo.y, hi.x, hi.y));
                        }
                        O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, (16 * dt < Dn) ? Pn : Pr, O[dt], 0, 0, 0);
                    }
                }
        } else if (wave_on) {
            e16 = (const uint16_t *)TB[q];
                // ---- scores S^T for keys 0-15 (st = 0) and 16-31 (st = 1)
                float s2[8], ks8[8];
#pragma unroll
                for (int st = 0; st < 2; st++) {
                    v4f an = {0.0f, 0.0f, 0.0f, 0.0f}, ar = {0.0f, 0.0f, 0.0f, 0.0f};
                    const int r = 16 * st + col;
#pragma unroll
                    for (int ks = 0; ks < NKS; ks++) {
                        const v8bf a = qk_operand(std::false_type{}, r, ks);
                        if (32 * ks < Dn) an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qT[ks], an, 0, 0, 0);
                        else ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qT[ks], ar, 0, 0, 0);
                    }
                    const float4 sc4 = *(const float4 *)(tksc + 16 * st + 4 * grp);
                    const int4 kv4 = *(const int4 *)(tkval + 16 * st + 4 * grp);
                    const bool wt = kind == 1;  // a window tile: scale 1, keys below kb1 valid
                    const int kr = tb + 16 * st + 4 * grp;
                    const float scv[4] = {wt ? 1.0f : sc4.x, wt ? 1.0f : sc4.y, wt ? 1.0f : sc4.z, wt ? 1.0f : sc4.w};
                    const int kvv[4] = {wt ? (int)(kr < kb1) : kv4.x, wt ? (int)(kr + 1 < kb1) : kv4.y,
                                        wt ? (int)(kr + 2 < kb1) : kv4.z, wt ? (int)(kr + 3 < kb1) : kv4.w};
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        s2[4 * st + i] = kvv[i] ? P.scale2 * fmaf(scv[i], an[i], ar[i]) : -INFINITY;
                        ks8[4 * st + i] = scv[i];
                    }
                }
                // ---- online softmax (exp2 domain); lane: head h, keys {4grp+i, 16+4grp+i}
                float mt = s2[0];
#pragma unroll
                for (int i = 1; i < 8; i++) mt = fmaxf(mt, s2[i]);
                mt = fmaxf(mt, __shfl_xor(mt, 16));
                mt = fmaxf(mt, __shfl_xor(mt, 32));
                // The running reference moves only when a score exceeds it by more than kRescaleSlack
                // (log2 units): until then the weights, at most 2^kRescaleSlack, stay exact in fp32 and
                // BF16 range, and O and l need no rescaling.  Same decision in all four lanes of a head.
                if (mt > m_run + kRescaleSlack) {
                    const float alpha = exp2_weight(m_run - mt);  // 0 when m_run = -inf
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < NDT; i++) O[i] *= alpha;
                    m_run = mt;
                }
                float pn[8], pr[8];
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    const float pi = (s2[i] == -INFINITY) ? 0.0f : exp2_weight(s2[i] - m_run);
                    l_run += pi;
                    pr[i] = pi;
                    pn[i] = pi * ks8[i];
                }
                v8bf Pn, Pr;  // round to nearest even (v_cvt_pk_bf16_f32)
#pragma unroll
                for (int i = 0; i < 8; i++) {
                    Pn[i] = (__bf16)pn[i];
                    Pr[i] = (__bf16)pr[i];
                }
                // ---- values O^T += E^T P^T; A row = dim 16*dt + col, keys {4grp..+3, 16+4grp..+3}
#pragma unroll
                for (int dt = 0; dt < NDT; dt++) {
                    const v8bf a = pv_operand(std::false_type{}, dt);
                    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, (16 * dt < Dn) ? Pn : Pr, O[dt], 0, 0, 0);
                }
        }
        q ^= 1;
        // No barrier here: the buffer this tile used is refilled (by direct loads, or by
        // stage_bf16) only after the next iteration's barrier, which every wavefront reaches
        // after its last read of it.
    }
    if (!wave_on) return;
    // l over the four lane groups of each head
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    if (h >= P.H) return;
    if (splits == 1) {
        const float f = finish_factor(P, h, m_run, l_run);
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) O[dt] *= f;
        if (P.rope_inv) {  // H is a multiple of 16: the whole wavefront is here
            RopeLanes rl;
            rl.eval(P.rt, R / 2, (double)sq_pos(Sq, b));
#pragma unroll
            for (int dt = Dn / 16; dt < NDT; dt++) {
                const int j = (16 * dt + 4 * grp - Dn) / 2;
                const float2 r0 = rope_unrotate(rl.get(j), O[dt][0], O[dt][1]);
                const float2 r1 = rope_unrotate(rl.get(j + 1), O[dt][2], O[dt][3]);
                O[dt] = v4f{r0.x, r0.y, r1.x, r1.y};
            }
        }
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
            const float o[4] = {O[dt][0], O[dt][1], O[dt][2], O[dt][3]};
            store_out4(P, b, h, 16 * dt + 4 * grp, o);
        }
    } else {
        // the unnormalised sums leave rounded to BF16 (fp32's exponent range, so no scaling;
        // relative error 2^-9 per element), halving the round trip through the combine; each
        // store writes 512 bytes contiguous: the wavefront's 16 heads x 16 dims of one tile
        // (streaming stores: the combine reads them once)
        uint16_t *po = P.part_o + ((int64_t)(b * P.S + split) * NDT * P.H + h) * 16 + 4 * grp;
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
            const v2bf lo = {(__bf16)O[dt][0], (__bf16)O[dt][1]}, hi = {(__bf16)O[dt][2], (__bf16)O[dt][3]};
            const u32x2 w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
            __builtin_nontemporal_store(w, (u32x2 *)(po + (int64_t)dt * P.H * 16));
        }
        if (grp == 0) {
            float *pm = P.part_ml + (((int64_t)b * P.S + split) * P.H + h) * 2;
            pm[0] = m_run;
            pm[1] = l_run;
        }
    }
}


// ---------------------------------------------------------------- combine kernel ----
// One wavefront per (16-dim tile, 16 heads, sequence), four wavefronts (four consecutive dim
// tiles) per workgroup: lane l holds head 16*hy + l/4 and dims 16*dt + 4*(l%4) .. +3.  The
// splits' (m, l) and partial tiles (each one contiguous 1 KB read per split) are requested
// together, only for the splits the sequence has; the tiles are then merged in split order
// and the sink is added once (splits <= kMaxSplits).
constexpr int kMaxSplits = 32;
constexpr int kCombineWaves = 4;

// NS: splits per sequence the launch provides for (16 or kMaxSplits), so launches with few splits
// keep the register count (and occupancy) of a 16-entry array.
template <int NS>
__global__ void __launch_bounds__(64 * kCombineWaves) attn_combine_kernel(AttnParams P, SeqInfo Sq) {
    const int dt = blockIdx.x * kCombineWaves + (threadIdx.x >> 6), b = blockIdx.z, lane = threadIdx.x & 63;
    const int h = 16 * blockIdx.y + (lane >> 2);
    const int d0 = 16 * dt + 4 * (lane & 3);
    const int ndt = P.D / 16;
    const int n_keys = sq_n_ent(Sq, b) + sq_win_len(Sq, b);
    int tps, splits;
    split_plan(n_keys, P.target, &tps, &splits);
    if (splits == 1) return;  // uniform over the workgroup
    // every split's (m, l) and partial tile are requested before any is used (one memory round trip)
    float m2s[NS], ls[NS];
    const uint16_t *pbase = P.part_o + ((int64_t)b * P.S * ndt + dt) * P.H * 16 + (int64_t)h * 16 + 4 * (lane & 3);
    const int64_t sstride = (int64_t)ndt * P.H * 16;
    u32x2 po[NS];  // four BF16 partial sums of split s
#pragma unroll
    for (int s = 0; s < NS; s++)
        po[s] = s < splits ? __builtin_nontemporal_load((const u32x2 *)(pbase + s * sstride)) : u32x2{0u, 0u};
#pragma unroll
    for (int s = 0; s < NS; s++) {
        float2 ml = make_float2(-INFINITY, 0.0f);
        if (s < splits) ml = *(const float2 *)(P.part_ml + ((int64_t)(b * P.S + s) * P.H + h) * 2);
        m2s[s] = ml.x;
        ls[s] = ml.y;
    }
    // the cos/sin of the inverse RoPE, while the partials are in flight
    const bool rope_wave = 16 * dt + 16 > P.D - P.R;
    RopeLanes rl;
    if (P.rope_inv && rope_wave) rl.eval(P.rt, P.R / 2, (double)sq_pos(Sq, b));
    float M = P.sink[h] * kLog2e;
#pragma unroll
    for (int s = 0; s < NS; s++)
        if (s < splits) M = fmaxf(M, m2s[s]);
    float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
#pragma unroll
    for (int s = 0; s < NS; s++) {
        const float c = (s >= splits || m2s[s] == -INFINITY) ? 0.0f : exp2f(m2s[s] - M);
        l = fmaf(ls[s], c, l);
#pragma unroll
        for (int v = 0; v < 4; v++) o[v] = fmaf(bf16_half(po[s], v), c, o[v]);
    }
    // finish with m2 = M and l as the merged sum (the factor exp2(M - M) is 1)
    finish4(P, b, h, d0, rope_wave, rl, M, l, o);
}

// ---------------------------------------------------------------- fp32 kernel -------
// Any record format, fp32 or BF16 queries/window: one workgroup per (head, sequence),
// scores in LDS, fp32 arithmetic throughout (no split).
constexpr int kF32MaxKeys = 8192 + 2048;

__device__ __forceinline__ float load_key_dim(const AttnParams &P, int64_t kvb, const WinRows &wr, int64_t e, int wtok,
                                              int d) {
    const int Dn = P.D - P.R;
    if (e >= 0) {
        const int64_t row = kvb + e;
        if (P.fmt == V4A_KV_F32) return ((const float *)P.nope)[row * P.D + d];
        if (d < Dn) {
            const uint8_t c = P.nope[row * Dn + d];
            const uint32_t c4 = c;
            const uint32_t pr = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c4, 1.0f, false));
            return bf16_to_f32((uint16_t)(pr & 0xFFFFu)) * P.kscale[row];
        }
        return bf16_to_f32(P.rope[row * P.R + (d - Dn)]);
    }
    const int64_t wi = wr.row(wtok) * P.D + d;
    return P.win_bf16 ? bf16_to_f32(((const uint16_t *)P.win)[wi]) : ((const float *)P.win)[wi];
}

__global__ void __launch_bounds__(256) attn_f32_kernel(AttnParams P, SeqInfo Sq) {
    __shared__ float sc[kF32MaxKeys];
    __shared__ float qs[512];
    __shared__ float red[256];
    __shared__ float osh[512];
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int n_ent = sq_n_ent(Sq, b), n_keys = n_ent + sq_win_len(Sq, b);
    const WinRows wr = sq_win_rows(Sq, b, P.W);
    const int D = P.D;
    for (int d = t; d < D; d += 256) {
        const int64_t qi = ((int64_t)b * P.H + h) * D + d;
        qs[d] = P.q_bf16 ? bf16_to_f32(((const uint16_t *)P.q)[qi]) : ((const float *)P.q)[qi];
    }
    __syncthreads();
    const float scale = P.scale2 / kLog2e;
    float mx = -INFINITY;
    for (int j = t; j < n_keys; j += 256) {
        int64_t e = -1;
        int wtok = -1;
        if (j < n_ent) {
            e = P.topk ? (int64_t)P.topk[(int64_t)b * P.k + j] : (int64_t)j;
            if (e >= P.cap) e = -1;
        } else {
            wtok = j - n_ent;
        }
        float s = -INFINITY;
        if (e >= 0 || wtok >= 0) {
            float acc = 0.0f;
            for (int d = 0; d < D; d++) acc = fmaf(qs[d], load_key_dim(P, (int64_t)sq_slot(Sq, b) * P.kv_bstride, wr, e, wtok, d), acc);
            s = scale * acc;
        }
        sc[j] = s;
        mx = fmaxf(mx, s);
    }
    red[t] = mx;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (t < o) red[t] = fmaxf(red[t], red[t + o]);
        __syncthreads();
    }
    const float sink = P.sink[h];
    const float M = fmaxf(red[0], sink);
    __syncthreads();
    float part = 0.0f;
    for (int j = t; j < n_keys; j += 256) {
        const float pj = sc[j] == -INFINITY ? 0.0f : expf(sc[j] - M);
        sc[j] = pj;
        part += pj;
    }
    red[t] = part;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (t < o) red[t] += red[t + o];
        __syncthreads();
    }
    const float den = (M == -INFINITY) ? 0.0f : red[0] + expf(sink - M);
    for (int d = t; d < D; d += 256) {
        float acc = 0.0f;
        for (int j = 0; j < n_keys; j++) {
            if (sc[j] == 0.0f) continue;
            int64_t e = -1;
            int wtok = -1;
            if (j < n_ent) {
                e = P.topk ? (int64_t)P.topk[(int64_t)b * P.k + j] : (int64_t)j;
                if (e >= P.cap) e = -1;
            } else {
                wtok = j - n_ent;
            }
            if (e < 0 && wtok < 0) continue;
            acc = fmaf(sc[j], load_key_dim(P, (int64_t)sq_slot(Sq, b) * P.kv_bstride, wr, e, wtok, d), acc);
        }
        osh[d] = den > 0.0f ? acc / den : 0.0f;
    }
    __syncthreads();
    const int Dn = D - P.R;
    for (int d = 2 * t; d < D; d += 512) {
        float o[2] = {osh[d], osh[d + 1]};
        if (P.rope_inv && d >= Dn) {
            float c, s;
            rope_cs_freq((double)sq_pos(Sq, b), P.rt.inv_freq[(d - Dn) / 2], &c, &s);
            const float x = o[0], y = o[1];
            o[0] = x * c + y * s;
            o[1] = -x * s + y * c;
        }
        const int64_t base = ((int64_t)b * P.H + h) * D + d;
        if (P.out_bf16) {
            ((uint16_t *)P.out)[base] = f32_to_bf16(o[0]);
            ((uint16_t *)P.out)[base + 1] = f32_to_bf16(o[1]);
        } else {
            ((float *)P.out)[base] = o[0];
            ((float *)P.out)[base + 1] = o[1];
        }
    }
}

bool attn_uses_mfma(const AttnArgs &a) {
    return a.kv->fmt == V4A_KV_FP8_BF16 && a.q_bf16 && a.win_bf16 && (a.H % 16) == 0 && a.H <= 128 &&
           ((a.D == 512 && a.R == 64) || (a.D == 128 && a.R == 32));
}

void split_plan_host(int n_keys, int target, int *tps, int *splits) {
    split_plan(n_keys, target, tps, splits);
}

// Compute units of the current device (cached per device).
static int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = n;
    }
    return cached[dev];
}

hipError_t launch_attention(const AttnArgs &a, const SeqInfo &sq, hipStream_t s) {
    AttnParams P{};
    P.q = a.q;
    P.q_bf16 = a.q_bf16;
    P.B = a.B;
    P.H = a.H;
    P.D = a.D;
    P.R = a.R;
    P.fmt = a.kv->fmt;
    P.nope = (const uint8_t *)a.kv->nope;
    P.rope = (const uint16_t *)a.kv->rope;
    P.kscale = a.kv->scale;
    P.cap = a.kv->cap;
    P.kv_bstride = a.kv_bstride;
    P.topk = a.topk;
    P.k = a.k;
    P.win = a.win;
    P.win_bf16 = a.win_bf16;
    P.W = a.W;
    P.sink = a.sink;
    P.scale2 = a.scale * kLog2e;
    P.rope_inv = a.rope_inv;
    P.q_norm_w = a.q_norm_w;
    if (a.rope_inv || a.q_norm_w) fill_rope_table(P.rt, a.R, a.theta);
    P.out = a.out;
    P.out_bf16 = a.out_bf16;
    P.part_o = (uint16_t *)a.partial;
    P.target = a.target_splits;
    P.S = a.split_cap;
    P.part_ml = a.partial ? (float *)((uint16_t *)a.partial + (size_t)a.B * P.S * a.H * a.D) : nullptr;
    if (a.B == 0) return hipSuccess;
    if (!attn_uses_mfma(a)) {
        V4A_LAUNCH("attn_f32_kernel", attn_f32_kernel, dim3(a.H, a.B), dim3(256), 0, s, P, sq);
        return hipGetLastError();
    }
    if (a.no_split) {
        // Split-free: each (query, head group) attends over all its keys in one workgroup, so a
        // head's result is the same whatever the batch and equals the prefill path's.  Full
        // waves of 64-head workgroups first; the last partial wave runs as 16-head workgroups,
        // which spread it over more CUs without changing any head's order of accumulation.
        if (P.S != 1) return hipErrorInvalidValue;
        const int cus = device_cu_count();
        int full = 0;  // 64-head items of the full waves
        if (a.H % 64 == 0 && cus > 0) full = (a.B * (a.H / 64) / cus) * cus;
        const int units = a.B * (a.H / 16) - 4 * full;  // remaining 16-head items
        if (full > 0) {
            P.hpw = 64;
            P.item0 = 0;
            if (a.D == 512)
                V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<512, 64, 4>), dim3(full), dim3(256), 0, s, P, sq);
            else
                V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<128, 32, 4>), dim3(full), dim3(256), 0, s, P, sq);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
        if (units > 0) {
            P.hpw = 16;
            P.item0 = 4 * full;
            if (a.D == 512)
                V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<512, 64, 4>), dim3(units), dim3(64), 0, s, P, sq);
            else
                V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<128, 32, 4>), dim3(units), dim3(64), 0, s, P, sq);
        }
        return hipGetLastError();
    }
    // Workgroup shape: with enough (query, split) pairs to fill the chip, one workgroup of up to
    // 8 wavefronts covers all heads, so each staged key tile serves every head (half the
    // staging per head); with few pairs (latency-bound decode) two 4-wavefront head groups per
    // split double the workgroups instead.  Every wavefront computes the same keys in the same
    // order for its 16 heads either way, so the choice never changes a result.
    const int pairs = a.B * P.S;
    const bool wide = a.H > 64 && pairs >= 256;
    const int hpg = wide ? a.H : (a.H >= 64 ? 64 : a.H);  // heads per workgroup
    P.n_hg = 1;  // head groups per split: a power of two (groups past H have no heads)
    while (P.n_hg * hpg < a.H) P.n_hg *= 2;
    const int waves = hpg / 16;
    int blocks = pairs;
    if (P.n_hg > 1) blocks = ((pairs + 7) / 8) * 8 * P.n_hg;
    if (a.D == 512) {
        if (wide)
            V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<512, 64, 8>), dim3(blocks), dim3(64 * waves), 0, s, P, sq);
        else
            V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<512, 64, 4>), dim3(blocks), dim3(64 * waves), 0, s, P, sq);
    } else {
        if (wide)
            V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<128, 32, 8>), dim3(blocks), dim3(64 * waves), 0, s, P, sq);
        else
            V4A_LAUNCH("attn_mfma_kernel", (attn_mfma_kernel<128, 32, 4>), dim3(blocks), dim3(64 * waves), 0, s, P, sq);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || P.S <= 1) return e;
    const dim3 cgrid(a.D / 16 / kCombineWaves, a.H / 16, a.B);
    if (P.S <= 16)
        V4A_LAUNCH("attn_combine_kernel", attn_combine_kernel<16>, cgrid, dim3(64 * kCombineWaves), 0, s, P, sq);
    else
        V4A_LAUNCH("attn_combine_kernel", attn_combine_kernel<kMaxSplits>, cgrid, dim3(64 * kCombineWaves), 0, s, P, sq);
    return hipGetLastError();
}

}  // namespace v4a
