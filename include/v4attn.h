/*
 * v4attn.h -- C ABI of the MI355X (gfx950) hot path of DeepSeek-V4 hybrid attention
 * (CSA + HCA) for one layer: KV compressors, lightning indexer with top-k, and
 * shared-KV multi-query attention with a sliding window and an attention sink.
 *
 * The operations follow these pages (cited by site, title and section):
 *   [cyqw]     "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2 "Hybrid
 *              attention CSA+HCA", section 3.4 "FP4 QAT", section 3.5 "KV cache layering".
 *   [firecat]  "DeepSeek V4 technical report explained" (firecat-web.com), "Core
 *              architecture upgrades", item 2 "Hybrid attention", and the model table.
 *   [chooseai] "DeepSeek V4 preview and technical report" (chooseai.net/news/3476),
 *              section 1 "CSA + HCA hybrid attention".
 *   [mewclaw]  "DeepSeek-V4: the engineering answer to million-token context"
 *              (tutorial.mewclaw.fun), "Hybrid Attention", "Partial RoPE", "Attention sink".
 *
 * Conventions shared by every call
 *   - Pointers marked (device) are device memory owned by the caller; pointers marked
 *     (host) are host memory read before the call returns.  The library allocates no
 *     device memory: scratch space is the caller's workspace `ws` of `ws_bytes` bytes,
 *     sized by the matching *_workspace() function, 256-byte aligned.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default stream).
 *     Buffers must stay alive until the stream has executed the call.
 *   - Every call validates its arguments on the host before launching anything.  On a
 *     status other than V4A_OK nothing was launched and no output was written;
 *     v4a_last_error() returns a message for the calling thread.  No C++ exception
 *     crosses this boundary.
 *   - State between calls: the library keeps none of its own except (a) the kernel-timing
 *     trace (v4a_trace_*: process-global events and records, off unless armed) and (b) the
 *     per-device scratch array of v4a_decode_step_csa_noalloc (see there).  A workspace's
 *     contents can carry over between calls where a call says so: v4a_decode_step_csa leaves
 *     its selection histograms clear and, with ws_clean, relies on that.  Calls may run from
 *     several threads and streams at once; calls sharing a workspace must not overlap.
 *   - Results are deterministic and batch invariant: the work split of a sequence depends
 *     only on its own lengths and the shape constants, never on the batch size or on
 *     device occupancy, and no floating-point reduction uses atomics.
 *
 * Positions: tokens of a sequence sit at positions 0..T-1.  A decode query is the token
 * at q_pos = T-1.  Compressed entry i of ratio m covers the block of tokens
 * [m*i, m*i + m - 1] and is visible to a query at position t iff m*(i+1) - 1 <= t.
 */
#ifndef V4ATTN_H
#define V4ATTN_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define V4A_API __attribute__((visibility("default")))
#else
#define V4A_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    V4A_OK = 0,
    V4A_EINVAL = 1,        /* a pointer, size or position is invalid */
    V4A_EUNSUPPORTED = 2,  /* a shape or format the library does not implement */
    V4A_EWORKSPACE = 3,    /* workspace missing, too small or misaligned */
    V4A_EHIP = 4           /* the HIP runtime reported an error at launch */
} v4a_status;

/* Element type of raw KV streams, queries, window tokens and outputs. */
typedef enum { V4A_F32 = 0, V4A_BF16 = 1 } v4a_float;

/* Compressed-entry record formats.
 * V4A_KV_FP8_BF16 ([chooseai] section 1, [mewclaw] "Low-precision path": RoPE dims in
 * BF16, the other dims in FP8): per entry, the first D-R dims as OCP FP8 E4M3FN codes
 * with one fp32 scale per entry (value = code * scale; scale = amax/448 over those dims,
 * 1 when they are all zero), the last R dims as BF16.
 * V4A_KV_F32: all D dims in fp32. */
typedef enum { V4A_KV_F32 = 0, V4A_KV_FP8_BF16 = 1 } v4a_kv_fmt;

/* Indexer key/query formats.  V4A_IDX_MXFP4 ([cyqw] section 3.4: the indexer QK path in
 * FP4): OCP MXFP4, blocks of 32 E2M1 elements sharing an E8M0 scale byte (2^(byte-127)),
 * element 2j in the low nibble of byte j.  V4A_IDX_F32: plain fp32 vectors. */
typedef enum { V4A_IDX_F32 = 0, V4A_IDX_MXFP4 = 1 } v4a_idx_fmt;

/* A batch of entry records: slot b holds entries [0, cap) of sequence b.
 *   FP8_BF16: nope  u8   [B][cap][D-R]  (device)
 *             rope  bf16 [B][cap][R]    (device, raw 16-bit words)
 *             scale f32  [B][cap]       (device)
 *   F32:      nope  f32  [B][cap][D]    (device); rope and scale unused (NULL). */
typedef struct {
    v4a_kv_fmt fmt;
    int32_t D, R;
    void *nope;
    void *rope;
    float *scale;
    int64_t cap;
} v4a_kv;

/* A batch of indexer vectors (keys, or query heads): slot b holds rows [0, cap).
 *   MXFP4: codes u8 [B][cap][d/2], scales u8 [B][cap][d/32]  (device; cap <= 2^26)
 *   F32:   codes f32 [B][cap][d] (device); scales unused (NULL). */
typedef struct {
    v4a_idx_fmt fmt;
    int32_t d;
    void *codes;
    uint8_t *scales;
    int64_t cap;
} v4a_idx;

/* ---------------------------------------------------------------- a3: quantisers ----
 * Quantise fp32 rows x [rows][D] (device) into records row0 .. row0+rows-1 of `out`,
 * counting rows across slots (row r lives in slot r / cap).  Encoding: round to nearest
 * even everywhere; FP8 codes are the E4M3 encoding (saturating at +-448) of the fp32
 * product x * (448/amax); BF16 is the nearest-even rounding of x.  Requires D-R a multiple
 * of 8, D <= 512, R even, rows >= 0.  [chooseai] section 1. */
V4A_API v4a_status v4a_quantize_kv(const float *x, int64_t rows, const v4a_kv *out, int64_t row0,
                           void *stream);

/* MXFP4 quantisation of fp32 rows x [rows][d] (device) into rows row0.. of `out`:
 * per 32-element block, X = floor(log2(amax)) - 2 clamped to [-127, 127] (amax = 0 gives
 * X = -127 and zero codes), codes = E2M1 nearest-even of x * 2^-X, saturating at 6.
 * Requires d a multiple of 32, d <= 512.  [cyqw] section 3.4. */
V4A_API v4a_status v4a_quantize_mxfp4(const float *x, int64_t rows, const v4a_idx *out, int64_t row0,
                              void *stream);

/* ------------------------------------------------------------ a1/a2: compressors ----
 * CSA compressor ([cyqw] section 2.2: every m tokens become one entry; two independent KV
 * sequences merged with softmax-normalised gate weights; adjacent compressed blocks share
 * indices. [chooseai] section 1: softmax with positional bias).
 * Entry i merges A-block i (tokens m*i .. m*i+m-1 of stream A, logits gate_a[t] +
 * bias_a[j]) with B-block i-1 (tokens m*(i-1)+j of stream B, logits gate_b[t] +
 * bias_b[j]); entry 0 merges its A-block alone.  Per gate channel (G == 1: one gate for
 * all dims; G == D: one per dim) the weights are the softmax over the candidates; the
 * entry is the weighted sum of the candidate rows.  Then, if apply_rope, the last R dims
 * are rotated (interleaved pairs, inv_freq_j = theta^(-2j/R)) at position m*i, and the
 * entry is written in the output's format.
 *   kv_a, kv_b  [n_seq][n_tok][D] (device, f32 or bf16 per in_t); row r of sequence s is
 *               its token tok0 + r (all n_seq sequences share tok0 and the entry range)
 *   gate_a, gate_b [n_seq][n_tok][G] f32 (device); bias_a, bias_b [m][G] f32 (device)
 *   Writes entries first_entry .. first_entry+n_entries-1 of slots b0 .. b0+n_seq-1 (which
 *   must exist in the output) of exactly one of
 *   out_kv (records; D == out_kv->D, R == out_kv->R) or out_idx (indexer keys;
 *   D == out_idx->d, no RoPE).  The rows must cover every block these entries read:
 *   tok0 <= m*(first_entry-1) (or tok0 <= 0 when first_entry == 0) and
 *   m*(first_entry+n_entries) <= tok0 + n_tok; tok0 must be a multiple of m.
 *   norm_w: NULL, or [D] f32 (device) RMSNorm weights: [cyqw] section 2.3 (RMSNorm acts
 *   directly on the KV entries).  Each merged entry x becomes x_d * norm_w[d] /
 *   sqrt(mean(x^2) + 1e-6) before RoPE and encoding.
 *   Supports m in [1, 128], G in {1, D}, D in {32, 128, 512}. */
V4A_API v4a_status v4a_compress_csa(const void *kv_a, const void *kv_b, v4a_float in_t, int32_t D,
                            const float *gate_a, const float *gate_b, int32_t G,
                            const float *bias_a, const float *bias_b, int64_t tok0,
                            int64_t n_tok, int32_t m, int64_t first_entry, int64_t n_entries,
                            int32_t apply_rope, float rope_theta, const float *norm_w,
                            const v4a_kv *out_kv, const v4a_idx *out_idx, int32_t b0,
                            int32_t n_seq, void *stream);

/* HCA compressor ([cyqw] section 2.2, [firecat] item 2: every m' = 128 tokens become one
 * entry, no overlap, no sparse selection).  Entry i merges tokens m*i .. m*i+m-1 of kv
 * with logits gate[t] + bias[j]; RoPE at m*i and output as for the CSA compressor.
 * kv [n_seq][n_tok][D], gate [n_seq][n_tok][G]; writes slots b0 .. b0+n_seq-1.
 * Requires tok0 <= m*first_entry, m*(first_entry+n_entries) <= tok0 + n_tok. */
V4A_API v4a_status v4a_compress_hca(const void *kv, v4a_float in_t, int32_t D, const float *gate,
                            int32_t G, const float *bias, int64_t tok0, int64_t n_tok,
                            int32_t m, int64_t first_entry, int64_t n_entries,
                            int32_t apply_rope, float rope_theta, const float *norm_w,
                            const v4a_kv *out_kv, int32_t b0, int32_t n_seq, void *stream);

/* ------------------------------------------------ a4/a5: lightning indexer + top-k ----
 * [cyqw] section 2.2 (a low-rank, low-precision multi-head indexer scores compressed
 * entries; each query keeps its top-k entries; k = 1024 for Pro) and section 3.4 (QK in
 * FP4); [chooseai] section 1 (k = 512 for Flash).
 * For query j of sequence b (position q_pos[b*Q+j]) and each visible key i < n_vis with
 * n_vis = min(n_entries[b], (q_pos+1)/m):
 *   s_h   = q_h . key_i per head h (MXFP4: the exact dot rounded once to fp32; F32: an
 *           fp32 fma chain over ascending dims),
 *   score = sum_h w_h * ReLU(s_h), evaluated as four fp32 fma chains (chain (h>>2)&3,
 *           ascending h), combined as ((c0+c1)+c2)+c3, with -0 turned into +0.
 * The selection is the k_eff = min(k, n_vis) best keys under (score descending, index
 * ascending), written to out_idx[b][j][0..k) in ascending index order, padded with -1.
 *   keys   [B][cap][..] (device; keys->fmt == q_idx->fmt, keys->d == q_idx->d)
 *   q_idx  rows [B*Q*H_I] (device; slot stride cap >= Q*H_I, i.e. one slot per sequence)
 *   w      [B][Q][H_I] f32 (device); n_entries [B], q_pos [B*Q] (host)
 *   out_idx [B][Q][k] int32 (device)
 * Supports H_I a multiple of 4 up to 64, d in {32, 128} (MXFP4: d == 128), k <= 2048,
 * Q*H_I <= q_idx->cap. */
V4A_API v4a_status v4a_indexer_topk(const v4a_idx *keys, const int64_t *n_entries, int32_t m,
                            const v4a_idx *q_idx, const float *w, int32_t B, int32_t Q,
                            int32_t H_I, const int64_t *q_pos, int32_t k, int32_t *out_idx,
                            void *ws, size_t ws_bytes, void *stream);
V4A_API size_t v4a_indexer_topk_workspace(int32_t B, int32_t Q, int64_t n_max, int32_t k);
/* The workspace holds, per query: its score keys (4 bytes per key up to n_max, padded), two
 * 4096-bin histograms and a candidate list sized for the worst case, in which every key of an
 * 8192-key slice ties in the threshold bin (8 bytes per key of every slice).  Examples: 12.7 MB
 * for 4 sequences over 262,144 entries (B = 4, Q = 1), 1.16 GB for a 4096-query prefill chunk
 * over 17,408 entries (B = 1, Q = 4096), of which 805 MB is the candidate list. */

/* The same call with the scores held in BF16 for the selection ([cyqw] section 3.4: the
 * index score is kept in BF16 instead of FP32, which halves the selector's score bytes).
 * Each fp32 score defined above is rounded to the nearest BF16 value (ties to the even
 * one; a -0 result counts as +0), and the k_eff best keys are chosen under (BF16 score
 * descending, index ascending), so scores that round to the same value are taken lowest
 * index first.  Arguments, layouts, limits, errors and the workspace size
 * (v4a_indexer_topk_workspace) are those of v4a_indexer_topk. */
V4A_API v4a_status v4a_indexer_topk_bf16(const v4a_idx *keys, const int64_t *n_entries, int32_t m,
                                 const v4a_idx *q_idx, const float *w, int32_t B, int32_t Q,
                                 int32_t H_I, const int64_t *q_pos, int32_t k, int32_t *out_idx,
                                 void *ws, size_t ws_bytes, void *stream);

/* The scores alone (same definition as above), for inspection: out_scores [B][Q][n_max]
 * f32 (device), -inf at positions that are not visible. */
V4A_API v4a_status v4a_indexer_scores(const v4a_idx *keys, const int64_t *n_entries, int32_t m,
                              const v4a_idx *q_idx, const float *w, int32_t B, int32_t Q,
                              int32_t H_I, const int64_t *q_pos, int64_t n_max,
                              float *out_scores, void *stream);

/* ---------------------------------------- a6/a7: shared-KV MQA with window and sink ----
 * [firecat] item 2 (multi-query attention over the selected compressed entries, head dim
 * 512, partial RoPE on the last 64 dims, a 128-token sliding window, a learnable sink
 * logit so the attention mass may be below one); [cyqw] section 2.2 (the window branch
 * joins the core attention; the sink adds a learnable term to the softmax denominator);
 * [mewclaw] "Partial RoPE" (the output is treated so values carry no absolute position).
 * For sequence b and head h, with keys = the selected (CSA) or all visible (HCA) entries
 * followed by the win_len[b] window tokens, each key also its own value (all D dims):
 *   z_j = softmax_scale * q_h . key_j,   M = max(sink_h, max_j z_j),
 *   out_h = sum_j exp(z_j - M) key_j / (exp(sink_h - M) + sum_j exp(z_j - M)),
 * then, if out_rope_inverse, the last R dims of out_h are rotated by -q_pos[b] (interleaved
 * pairs, inv_freq_j = theta^(-2j/R)).  Queries and window tokens arrive already rotated.
 *   q    [B][H][D] (device, q_t);  sink [H] f32 (device)
 *   win  [B][W][D] (device, win_t): the last win_len[b] <= W tokens, oldest first
 *   win_len [B], q_pos [B] (host)
 *   out  [B][H][D] (device, out_t)
 * decode_csa: topk_idx [B][k] int32 (device), ascending entry indices, -1 padding (the
 *   output of v4a_indexer_topk with Q = 1); every index must be < kv->cap.
 * decode_hca: n_entries [B] (host): entries min(n_entries[b], (q_pos+1)/m) are attended.
 * Supports D in {128, 512}, R even and < D, H a multiple of 16 up to 128 for
 * V4A_KV_FP8_BF16 (BF16 MFMA) and H <= 128 for V4A_KV_F32, W <= 128, k <= 2048. */
V4A_API v4a_status v4a_decode_csa(const void *q, v4a_float q_t, int32_t B, int32_t H, const v4a_kv *kv,
                          const int32_t *topk_idx, int32_t k, const void *win, v4a_float win_t,
                          const int32_t *win_len, int32_t W, const float *sink,
                          const int64_t *q_pos, float softmax_scale, int32_t out_rope_inverse,
                          float rope_theta, void *out, v4a_float out_t, void *ws,
                          size_t ws_bytes, void *stream);
V4A_API v4a_status v4a_decode_hca(const void *q, v4a_float q_t, int32_t B, int32_t H, const v4a_kv *kv,
                          const int64_t *n_entries, int32_t m, const void *win,
                          v4a_float win_t, const int32_t *win_len, int32_t W, const float *sink,
                          const int64_t *q_pos, float softmax_scale, int32_t out_rope_inverse,
                          float rope_theta, void *out, v4a_float out_t, void *ws,
                          size_t ws_bytes, void *stream);
/* Workspace for either decode call: n_keys_max = k (CSA) or max entries (HCA), plus W.  It
 * bounds every sequence of at most n_keys_max keys (a short key list takes more, smaller
 * splits than a long one, so the bound can exceed what one long sequence needs). */
V4A_API size_t v4a_decode_workspace(int32_t B, int32_t H, int32_t D, int64_t n_keys_max, int32_t W);

/* ------------------------------------------------------ grouped output projection ----
 * [cyqw] section 2.2 "Grouped Output Projection" (with many query heads, 128 for V4-Pro, the
 * head outputs are first reduced per group, then concatenated and projected, which cuts the
 * output projection's parameters and FLOPs) and [firecat] item 2 (head dim 512 with a grouped
 * projection).  For every token t (a row of the attention output o) and group g of H/G
 * consecutive heads (Kg = H*D/G values):
 *   y[t][g*r + j] = bf16( sum_{c < Kg} o[t][g*Kg + c] * wg[g][j][c] )   (fp32 accumulation, RNE)
 *   out[t][n]     = sum_{c < G*r} y[t][c] * wf[n][c]                    (fp32, then out_t)
 *   o   [T][H][D] bf16 (device), e.g. the output of the decode or prefill calls
 *   wg  [G][r][Kg] bf16 (device): the group weights, out-feature major
 *   wf  [d][G*r] bf16 (device): the final weights, out-feature major
 *   out [T][d] (device, out_t)
 *   ws: y [T][G*r] bf16, v4a_output_projection_workspace(T, G, r) bytes, 256-byte aligned.
 * Supports G dividing H, Kg and G*r multiples of 128, r and d multiples of 16, 16-byte aligned
 * pointers; T >= 0. */
V4A_API v4a_status v4a_output_projection(const void *o, int32_t T, int32_t H, int32_t D, int32_t G, int32_t r,
                                 const void *wg, const void *wf, int32_t d, void *out, v4a_float out_t,
                                 void *ws, size_t ws_bytes, void *stream);
V4A_API size_t v4a_output_projection_workspace(int32_t T, int32_t G, int32_t r);

/* -------------------------------------------------------------- a8: prefill chunk ----
 * One chunk of C consecutive tokens of one sequence (positions tok0 .. tok0+C-1) through
 * one attention layer of either kind, as C causal queries.  [cyqw] section 3.5 "KV cache
 * layering" and [mewclaw] "State cache" / "Compressed cache": a sequence's state is the
 * cache of compressed entries plus the raw tail (the 128-token window and the tokens of a
 * block not yet complete); a chunk appends its complete blocks to the entry cache.
 * The call
 *   1. compresses every block that ends inside the chunk (entries tok0/m ..
 *      (tok0+C)/m - 1) into the entry cache `kv` and, for CSA, the indexer key cache
 *      `keys` (the compressors above; CSA entry tok0/m also reads the B-block before tok0);
 *   2. CSA: selects, for every query t, the top-k of its visible entries (i < (t+1)/m)
 *      exactly as v4a_indexer_topk (score_bf16: v4a_indexer_topk_bf16) does with Q = C and
 *      q_pos = tok0 + j;
 *   3. attends, for query t = tok0 + j and every head, over its selected entries (CSA) or
 *      all its visible entries (HCA) plus the window tokens max(0, t-W+1) .. t (rows of
 *      stream kv_a), with the sink, exactly as the decode calls define it, and writes
 *      out[j].
 * Every query runs as one split, so its output equals the decode output at q_pos = t on
 * the same cache within rounding (not bitwise: decode splits its keys).
 * Stream rows: every stream holds n_prev + C rows; row r is position tok0 - n_prev + r.
 * Requirements: tok0 a multiple of m; entries [0, tok0/m) already in the caches;
 * n_prev <= tok0 and n_prev >= min(tok0, W-1); CSA with tok0 > 0 also n_prev >= m.
 * Supports the shapes of the calls it composes, C <= 65535, and for CSA the MXFP4 or fp32
 * indexer as in v4a_indexer_topk. */
typedef enum { V4A_LAYER_CSA = 0, V4A_LAYER_HCA = 1 } v4a_layer;

typedef struct {
    int64_t tok0;            /* position of the chunk's first token                      */
    int32_t C;               /* tokens (= queries) in the chunk                           */
    int32_t n_prev;          /* stream rows before tok0 (the raw state)                   */
    int32_t m;               /* compression ratio of this layer (CSA 4, HCA 128)          */
    v4a_float in_t;          /* element type of every raw stream                          */
    int32_t G;               /* gate width of the KV streams (1 or D)                     */
    const void *kv_a;        /* [n_prev+C][D] (device) CSA stream A or the HCA stream; the
                                window tokens are its rows                                */
    const void *kv_b;        /* [n_prev+C][D] (device) CSA stream B; NULL for HCA         */
    const float *gate_a;     /* [n_prev+C][G] f32 (device)                                */
    const float *gate_b;     /* CSA only                                                  */
    const float *bias_a;     /* [m][G] f32 (device)                                       */
    const float *bias_b;     /* CSA only                                                  */
    int32_t apply_rope;      /* rotate the entries' last R dims at their block start      */
    float rope_theta;
    const v4a_kv *kv;        /* entry cache; the sequence lives in slot `slot`            */
    int32_t slot;
    /* CSA indexer */
    int32_t idx_G;           /* gate width of the indexer streams (1 or d)                */
    const void *idx_a;       /* [n_prev+C][d] (device, in_t) indexer stream A             */
    const void *idx_b;       /* [n_prev+C][d] indexer stream B                            */
    const float *idx_gate_a, *idx_gate_b;   /* [n_prev+C][idx_G] f32 (device)             */
    const float *idx_bias_a, *idx_bias_b;   /* [m][idx_G] f32 (device)                    */
    const v4a_idx *keys;     /* indexer key cache, slot `slot`                            */
    const v4a_idx *q_idx;    /* [C*H_I] rows (device): the chunk queries' indexer heads   */
    const float *w;          /* [C][H_I] f32 (device)                                     */
    int32_t H_I, k;
    /* attention */
    const void *q;           /* [C][H][D] (device, q_t)                                   */
    v4a_float q_t;
    int32_t H, W;
    const float *sink;       /* [H] f32 (device)                                          */
    float softmax_scale;
    int32_t out_rope_inverse;
    void *out;               /* [C][H][D] (device, out_t)                                 */
    v4a_float out_t;
    int32_t score_bf16;      /* CSA: nonzero selects as v4a_indexer_topk_bf16 does         */
    const float *norm_w;     /* [D] f32 (device): RMSNorm of the new entries, or NULL      */
    const float *idx_norm_w; /* [d] f32 (device): RMSNorm of the new indexer keys, or NULL */
    const float *q_norm_w;   /* [D] f32 (device, 16-byte aligned) or NULL: queries arrive
                                projected only, as in v4a_decode_step_csa                 */
} v4a_prefill_args;

V4A_API v4a_status v4a_prefill_chunk(v4a_layer kind, const v4a_prefill_args *args, void *ws,
                             size_t ws_bytes, void *stream);
/* Workspace of v4a_prefill_chunk for these arguments (0 for HCA; 0 if they are invalid). */
V4A_API size_t v4a_prefill_workspace(v4a_layer kind, const v4a_prefill_args *args);

/* ------------------------------------------------- fused CSA decode step (one token) ----
 * One decode step of B sequences in one call, equal to v4a_compress_csa (records, then keys)
 * + v4a_indexer_topk (Q = 1) + v4a_decode_csa with the same arguments.  For every sequence b
 * whose newest token t = q_pos[b] completes a block ((t+1) % m == 0), entry (t+1)/m - 1 is
 * compressed into the record cache and the key cache; then the top-k of its visible entries
 * (n_entries[b] cached) are selected and attended over with the window and the sink.  MXFP4
 * keys of d = 128 from BF16 streams with one gate per token and 2m <= 8 are compressed by the
 * scoring kernel itself (bitwise the key v4a_compress_csa writes); other keys by a first
 * launch.  The record compression runs in the final selection's launch, which also clears the
 * selection's histograms for the next call (see ws_clean).
 * [cyqw] section 3.5 (the state cache keeps the incomplete block; a completed block becomes a
 * compressed entry) and the sections cited at the calls it composes.
 * Stream rows: every stream holds [B][2m] rows per sequence, the B-block before the completed
 * block and the completed block itself (positions t+1-2m .. t; for the first block only the
 * last m rows are read).  Sequences whose newest token completes no block read no rows.
 * With ring != 0 the per-token state is kept in rings the caller writes each token into
 * ([cyqw] section 3.5: the state cache holds the window and the incomplete block): each
 * stream's [B][2m] rows hold position p at row p mod 2m, and win [B][W][D] holds position p
 * at row p mod W; the window tokens are positions t-win_len[b]+1 .. t (win_len[b] <= t+1).
 * Split-free attention (no_split != 0; [cyqw] section 3.3: the attention kernels drop
 * split-KV so that results are bitwise identical whatever the batch, and spread the last
 * partial wave over more compute units in the same order of accumulation): every (sequence,
 * head group) attends over all its keys in one workgroup, full waves of the chip as 64-head
 * workgroups and the rest as 16-head ones, so each head's output is bit for bit the prefill
 * chunk's for the same query and caches.  No workspace is needed for attention then.
 * Query prologue (q_norm_w != NULL; [cyqw] section 2.3: RMSNorm acts directly on the queries):
 * q holds the projected queries before normalisation and rotation; each head's D-vector x
 * becomes x_d * q_norm_w[d] / sqrt(mean(x^2) + 1e-6), its last R dims are rotated at the
 * query position (interleaved pairs, as the entries are), and the result enters the products
 * rounded to BF16 (nearest even).  Without it q arrives normalised and rotated.
 * ws_clean != 0 promises that the workspace's selection histograms are already clear: the
 * workspace was last used by a v4a_decode_step_csa call with the same B and k, and nothing
 * has written it since.  The call then skips clearing them (one launch fewer).  Every call
 * leaves them clear, so a caller that keeps one workspace per (B, k) for its decode loop may
 * pass ws_clean = 1 from the second step on.  With ws_clean = 0 the call clears them itself.
 * Multi-token step (Q > 1; [cyqw] section 2 and the model table of [cyqw] section 4.2 and
 * [firecat]: V4 keeps multi-token prediction at depth 1, so a step may verify Q consecutive
 * tokens per sequence): sequence b's new tokens sit at positions t-Q+1 .. t with t = q_pos[b];
 * query j (0-based) is the token at t_j = t-Q+1+j.  The Q queries are evaluated together and
 * causally, exactly as Q steps of one token taken in order: query j sees the entries whose block
 * ends at or before t_j (so an entry completed by a later token of the step is not visible to
 * it, one completed by an earlier token is) and the window tokens ending at t_j.  At most one
 * block completes per step (Q <= m).  Shapes per sequence: q [B][Q][H][D], q_idx rows
 * [B][Q*H_I] (slot b holds its queries' heads in query order), w [B][Q][H_I], out [B][Q][H][D].
 * Stream rows: the plain layout holds [B][2m] rows, the B-block and the block completed by a
 * token of the step (positions m*(i-1) .. m*(i+1)-1 for entry i); a ring holds [B][2m+Q-1] rows
 * with position p at row p mod (2m+Q-1).  Window: query j's window is the
 * min(win_len[b], t_j+1) tokens ending at t_j; the buffer holds W+Q-1 rows per sequence
 * ([B][W+Q-1][D]): in the plain layout the tokens ending at t from row 0 (positions
 * max(0, t-win_len[b]-Q+2) .. t), in a ring position p at row p mod (W+Q-1).  Q = 1 is the
 * one-token step described above, with its layouts unchanged.  B*Q <= 128.
 * Supports the MFMA shapes: D = 512 records with d_I = 128 MXFP4 keys, or D = 128 with
 * d_I = 32; H a multiple of 16 up to 128; B <= 128; k <= 2048. */
typedef struct {
    int32_t B, m;
    const int64_t *q_pos;        /* host[B]: position of each sequence's newest token         */
    const int64_t *n_entries;    /* host[B]: entries cached after this step (<= cap)          */
    v4a_float in_t;              /* element type of the raw streams                            */
    int32_t G, idx_G;            /* gate widths (1 or D / 1 or d)                              */
    const void *kv_a, *kv_b;     /* [B][2m][D] (device)                                        */
    const float *gate_a, *gate_b, *bias_a, *bias_b;      /* [B][2m][G], [m][G]               */
    const void *idx_a, *idx_b;   /* [B][2m][d] (device)                                        */
    const float *idx_gate_a, *idx_gate_b, *idx_bias_a, *idx_bias_b;
    int32_t apply_rope;
    float rope_theta;
    const v4a_kv *kv;            /* record cache, slot b = sequence b                          */
    const v4a_idx *keys;         /* key cache, slot b = sequence b                             */
    const v4a_idx *q_idx;        /* [B*H_I] rows (device)                                      */
    const float *w;              /* [B][H_I] f32 (device)                                      */
    int32_t H_I, k;
    const void *q;               /* [B][H][D] (device)                                         */
    v4a_float q_t;
    int32_t H;
    const void *win;             /* [B][W][D] (device)                                         */
    v4a_float win_t;
    const int32_t *win_len;      /* host[B]                                                    */
    int32_t W;
    const float *sink;           /* [H] f32 (device)                                           */
    float softmax_scale;
    int32_t out_rope_inverse;
    void *out;                   /* [B][H][D] (device)                                         */
    v4a_float out_t;
    int32_t score_bf16;          /* nonzero: select as v4a_indexer_topk_bf16 does               */
    const float *norm_w;         /* [D] f32 (device): RMSNorm of the new entries, or NULL       */
    const float *idx_norm_w;     /* [d] f32 (device): RMSNorm of the new indexer keys, or NULL  */
    int32_t ring;                /* nonzero: the streams and the window are rings (see above)    */
    int32_t no_split;            /* nonzero: split-free attention (see below)                   */
    const float *q_norm_w;       /* [D] f32 (device, 16-byte aligned) or NULL: see below         */
    int32_t ws_clean;            /* nonzero: the workspace's histograms are clear (see above)   */
    int32_t Q;                   /* new tokens (queries) per sequence, 1..4 (0 means 1): see below */
} v4a_decode_step_args;

V4A_API v4a_status v4a_decode_step_csa(const v4a_decode_step_args *args, void *ws, size_t ws_bytes,
                               void *stream);
/* Workspace of v4a_decode_step_csa for these arguments (0 if they are invalid). */
V4A_API size_t v4a_decode_step_workspace(const v4a_decode_step_args *args);

/* The same step for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): no workspace argument, and the call
 * allocates nothing.  Its scratch is one array of V4A_NOALLOC_SCRATCH_BYTES (64 MiB) per device,
 * a static device variable of the library that each device loading it holds until the process
 * ends; its address is looked up once per device (the stream must belong to the current
 * device).  Arguments needing more scratch than that (v4a_decode_step_workspace(args) >
 * V4A_NOALLOC_SCRATCH_BYTES) are rejected with V4A_EWORKSPACE before any launch; the 1M-context
 * step of 4 sequences with k = 1024 needs about 38 MB.  Every call on a device shares that
 * device's array and finds the previous call's contents: the call clears what must start at
 * zero (the selection histograms) with a fill kernel, and ignores ws_clean.  Calls that overlap
 * on one device (several streams or threads) race on the array and must be serialised by the
 * caller.  Results are bitwise those of v4a_decode_step_csa with the same arguments. */
#define V4A_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
V4A_API v4a_status v4a_decode_step_csa_noalloc(const v4a_decode_step_args *args, void *stream);

/* ------------------------------------------------- fused HCA decode step (one token) ----
 * One decode step of B sequences of an HCA layer in one call, equal to v4a_compress_hca +
 * v4a_decode_hca with the same arguments.  For every sequence b whose newest token t = q_pos[b]
 * completes a block ((t+1) % m == 0), entry (t+1)/m - 1 is compressed into the record cache;
 * then its min(n_entries[b], (t+1)/m) visible entries and the window tokens are attended over
 * with the sink.  [cyqw] section 2.2 (HCA: every m' = 128 tokens become one entry, attended
 * densely) and section 3.5 (the state cache), and the sections cited at the calls it composes.
 * Stream rows: kv_a and gate_a hold [B][m] rows per sequence, the block ending at t (positions
 * t+1-m .. t); sequences whose newest token completes no block read no rows.  With ring != 0,
 * position p sits at row p mod m of its sequence's rows and at row p mod W of the window,
 * whose tokens are positions t-win_len[b]+1 .. t (win_len[b] <= t+1).
 * no_split: the split-free attention of v4a_decode_step_csa.
 * Q > 1: the multi-token step of v4a_decode_step_csa (queries at t-Q+1 .. t, each seeing the
 * entries whose block ends at or before it and the window ending at it).  Stream rows: the
 * plain layout holds the block completed by a token of the step ([B][m] rows, positions m*i ..
 * m*i+m-1), a ring [B][m+Q-1] rows with position p at row p mod (m+Q-1); the window as for CSA.
 * Supports the MFMA attention shapes (FP8/BF16 records with D in {128, 512}, H a multiple of 16
 * up to 128), m <= 128, B <= 128. */
typedef struct {
    int32_t B, m;
    const int64_t *q_pos;        /* host[B]: position of each sequence's newest token          */
    const int64_t *n_entries;    /* host[B]: entries cached after this step (<= cap)           */
    v4a_float in_t;              /* element type of the raw stream                             */
    int32_t G;                   /* gate width (1 or D)                                        */
    const void *kv_a;            /* [B][m][D] (device): the HCA stream                         */
    const float *gate_a;         /* [B][m][G] f32 (device)                                     */
    const float *bias_a;         /* [m][G] f32 (device)                                        */
    int32_t apply_rope;
    float rope_theta;
    const float *norm_w;         /* [D] f32 (device): RMSNorm of the new entries, or NULL       */
    const v4a_kv *kv;            /* record cache, slot b = sequence b                          */
    const void *q;               /* [B][H][D] (device)                                         */
    v4a_float q_t;
    int32_t H;
    const void *win;             /* [B][W][D] (device)                                         */
    v4a_float win_t;
    const int32_t *win_len;      /* host[B]                                                    */
    int32_t W;
    const float *sink;           /* [H] f32 (device)                                           */
    float softmax_scale;
    int32_t out_rope_inverse;
    void *out;                   /* [B][H][D] (device)                                         */
    v4a_float out_t;
    int32_t ring;                /* nonzero: the stream rows and the window are rings          */
    int32_t no_split;            /* nonzero: split-free attention (see below)                  */
    const float *q_norm_w;       /* [D] f32 (device, 16-byte aligned) or NULL: as for CSA       */
    int32_t Q;                   /* new tokens (queries) per sequence, 1..4 (0 means 1)         */
} v4a_decode_step_hca_args;

V4A_API v4a_status v4a_decode_step_hca(const v4a_decode_step_hca_args *args, void *ws, size_t ws_bytes,
                               void *stream);
/* Workspace of v4a_decode_step_hca for these arguments (0 if they are invalid or none is needed). */
V4A_API size_t v4a_decode_step_hca_workspace(const v4a_decode_step_hca_args *args);

/* ------------------------------------------------------------------- kernel timing ----
 * Instrumentation, off by default: each kernel the library launches can be timed on the GPU.
 * v4a_trace_begin arms a trace of at most `capacity` kernel launches (1 .. 2^18): until
 * v4a_trace_end, every kernel launched by any call carries its own start and stop HIP events
 * (hipExtLaunchKernelGGL), which time the dispatch itself; launches past `capacity` run
 * untimed.  v4a_trace_end disarms and returns the number of kernels timed.  After the caller
 * has synchronised the streams, v4a_trace_kernel(i, &kernel, &ms) gives the i-th timed
 * kernel's name (a static string, e.g. "indexer_mxfp4_kernel") and its duration in
 * milliseconds.  The events are the library's, created on the current device at the first
 * v4a_trace_begin and kept until the process ends.  One trace at a time per process; not
 * thread-safe. */
V4A_API v4a_status v4a_trace_begin(int32_t capacity);
V4A_API int32_t v4a_trace_end(void);
V4A_API v4a_status v4a_trace_kernel(int32_t i, const char **kernel, float *ms);

/* ---------------------------------------------------------------------- utilities ---- */
V4A_API const char *v4a_last_error(void);
V4A_API const char *v4a_version(void);

#ifdef __cplusplus
}
#endif
#endif /* V4ATTN_H */
