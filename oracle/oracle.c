/*
 * oracle.c -- plain, slow CPU oracle for the DeepSeek-V4 hybrid-attention
 * (CSA + HCA) hot path: one layer, one query step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file; it is used by tests/, by the smoke check and by the
 * cpu_baseline leg of the benchmark.  It shares no code, header, table or
 * constant with the HIP library.
 *
 * Sources (the pages are cited by site, title and section):
 *   [cyqw]     "DeepSeek-V4 technical report walkthrough" (cyqw.cn/news/842812),
 *              section 2.2 "Hybrid attention CSA+HCA" and section 3.4 "FP4 QAT".
 *   [firecat]  "DeepSeek V4 technical report explained: 484 days ..." (firecat-web.com),
 *              "Core architecture upgrades", item 2 "Hybrid attention".
 *   [chooseai] "DeepSeek V4 preview and technical report" (chooseai.net/news/3476),
 *              section 1 "CSA + HCA hybrid attention", section 2 "FP4 QAT".
 *   [mewclaw]  "DeepSeek-V4: the engineering answer to million-token context"
 *              (tutorial.mewclaw.fun), "Hybrid Attention", "Partial RoPE",
 *              "Attention sink", "Low-precision path".
 *
 * Where the pages leave a step open the reading used here is stated at the
 * function; every such reading is also listed in the design notes.
 *
 * Arithmetic: double precision for every floating stage except where a step is
 * defined in fp32 (the fp32 indexer dot and the fixed-order fp32 head sum, the
 * fp32 product x*inv of the FP8 encoder); exact integer arithmetic for MXFP4
 * dot products.  Built with -O2 -ffp-contract=off and without fast-math, so
 * each C expression rounds exactly as written.
 *
 * Parity pins: every function here is pinned by the CPU tests (reductions to
 * textbook attention, closed forms, exhaustive quantiser sweeps, brute force on
 * tiny inputs, RoPE identities, chunk invariance).  None is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_API __attribute__((visibility("default")))

ORC_API int orc_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* OCP FP8 E4M3FN decode: sign, 4 exponent bits (bias 7), 3 mantissa bits, no
 * infinities, only S.1111.111 is NaN.  Exponent field 0 is subnormal:
 * value = m * 2^-9.  Otherwise value = (8 + m) * 2^(e - 10).
 * Cited: [chooseai] section 1 (KV non-RoPE dims stored in FP8). */
ORC_API double orc_e4m3_decode(uint8_t c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* OCP FP8 E4M3FN encode of a finite fp32 value: round to nearest, ties to
 * even, saturate to +-448 (largest finite).  The sign bit is kept, so a
 * negative value that rounds to zero encodes as 0x80. */
ORC_API uint8_t orc_e4m3_encode(float x) {
    uint8_t s = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (a >= 448.0) return s | 0x7E;
    /* quantum: 2^-9 below the smallest normal 2^-6, else 2^(e-3) for a in [2^e, 2^(e+1)) */
    int e2;
    double q;
    if (a < ldexp(1.0, -6)) {
        q = ldexp(1.0, -9);
    } else {
        frexp(a, &e2);              /* a = f * 2^e2, f in [0.5, 1) -> binade e = e2 - 1 */
        q = ldexp(1.0, (e2 - 1) - 3);
    }
    double n = rint(a / q);         /* default rounding mode: nearest, ties to even */
    double v = n * q;
    if (v >= 448.0) return s | 0x7E;
    if (v == 0.0) return s;
    if (v < ldexp(1.0, -6)) return s | (uint8_t)(v / ldexp(1.0, -9));
    frexp(v, &e2);
    int e = e2 - 1;                 /* v in [2^e, 2^(e+1)) */
    int mant = (int)(v / ldexp(1.0, e) * 8.0) - 8;
    return s | (uint8_t)(((e + 7) << 3) | mant);
}

/* bfloat16: the high 16 bits of an fp32, rounded to nearest even on bit 16. */
ORC_API uint16_t orc_bf16_encode(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

ORC_API double orc_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* FP4 E2M1 magnitudes indexed by the 3-bit code (exponent bias 1, one
 * mantissa bit, no inf/NaN): 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

ORC_API double orc_e2m1_decode(uint8_t c) {
    double v = e2m1_mag[c & 7];
    return (c & 8) ? -v : v;
}

/* E2M1 encode, nearest with ties to the even code (mantissa bit 0), saturate at 6. */
ORC_API uint8_t orc_e2m1_encode(double x) {
    uint8_t s = signbit(x) ? 8 : 0;
    double a = fabs(x);
    if (a >= 6.0) return s | 7;
    int best = 0;
    for (int c = 1; c < 8; c++) {
        double dc = fabs(e2m1_mag[c] - a), db = fabs(e2m1_mag[best] - a);
        if (dc < db || (dc == db && (c & 1) == 0)) best = c;
    }
    return s | (uint8_t)best;
}

/* ------------------------------------------------------------------------ */
/* a3: quantisation of entry records and indexer vectors                     */
/* ------------------------------------------------------------------------ */

/* Entry record: the first D-R dims in FP8 E4M3 with one fp32 scale per entry,
 * the last R (RoPE) dims in BF16.  Cited: [chooseai] section 1 and [mewclaw]
 * "Low-precision path" (RoPE dims BF16, the rest FP8).  Reading: the scale is
 * per entry over the non-RoPE dims; amax = max |x|; amax == 0 gives scale 1
 * and zero codes; otherwise inv = 448/amax and scale = amax/448, both fp32,
 * and each code is the E4M3 encoding of the fp32 product x*inv.
 *   x     [rows][D] fp32
 *   nope  [rows][D-R] codes, rope [rows][R] bf16 bits, scale [rows] fp32 */
ORC_API void orc_quant_kv(const float *x, int64_t rows, int D, int R,
                          uint8_t *nope, uint16_t *rope, float *scale) {
    int Dn = D - R;
    for (int64_t r = 0; r < rows; r++) {
        const float *xr = x + r * D;
        float amax = 0.0f;
        for (int d = 0; d < Dn; d++) amax = fmaxf(amax, fabsf(xr[d]));
        if (amax == 0.0f) {
            scale[r] = 1.0f;
            for (int d = 0; d < Dn; d++) nope[r * Dn + d] = 0;
        } else {
            float inv = 448.0f / amax;
            scale[r] = amax / 448.0f;
            for (int d = 0; d < Dn; d++) {
                float v = xr[d] * inv;
                nope[r * Dn + d] = orc_e4m3_encode(v);
            }
        }
        for (int d = 0; d < R; d++) rope[r * R + d] = orc_bf16_encode(xr[Dn + d]);
    }
}

/* Exact value of an entry record, dims in order (code*scale for the first
 * D-R dims, the BF16 value for the last R). */
ORC_API void orc_dequant_kv(const uint8_t *nope, const uint16_t *rope, const float *scale,
                            int64_t rows, int D, int R, double *out) {
    int Dn = D - R;
    for (int64_t r = 0; r < rows; r++) {
        for (int d = 0; d < Dn; d++)
            out[r * D + d] = orc_e4m3_decode(nope[r * Dn + d]) * (double)scale[r];
        for (int d = 0; d < R; d++) out[r * D + Dn + d] = orc_bf16_decode(rope[r * R + d]);
    }
}

/* MXFP4 per the OCP Microscaling format: blocks of 32 elements share an E8M0
 * power-of-two scale 2^X with X = floor(log2(amax)) - 2 (2 is the largest
 * E2M1 exponent), clamped to [-127, 127]; amax == 0 gives X = -127 and zero
 * codes.  Elements are E2M1 codes of x * 2^-X (an exact scaling), element 2j
 * in the low nibble of byte j.  Scale byte = X + 127.
 * Cited: [cyqw] section 3.4 and [chooseai] section 2 (indexer QK in MXFP4,
 * FP4 E2M1 with 1x32 sub-blocks).
 *   x [rows][d] fp32 -> codes [rows][d/2], scales [rows][d/32] */
ORC_API void orc_quant_mxfp4(const float *x, int64_t rows, int d, uint8_t *codes, uint8_t *scales) {
    for (int64_t r = 0; r < rows; r++) {
        for (int b = 0; b < d / 32; b++) {
            const float *xb = x + r * d + b * 32;
            double amax = 0.0;
            for (int j = 0; j < 32; j++) amax = fmax(amax, fabs((double)xb[j]));
            int X;
            if (amax == 0.0) {
                X = -127;
            } else {
                int e2;
                frexp(amax, &e2);   /* amax in [2^(e2-1), 2^e2) -> floor(log2 amax) = e2 - 1 */
                X = (e2 - 1) - 2;
                if (X < -127) X = -127;
                if (X > 127) X = 127;
            }
            scales[r * (d / 32) + b] = (uint8_t)(X + 127);
            for (int j = 0; j < 32; j += 2) {
                uint8_t lo = amax == 0.0 ? 0 : orc_e2m1_encode(ldexp((double)xb[j], -X));
                uint8_t hi = amax == 0.0 ? 0 : orc_e2m1_encode(ldexp((double)xb[j + 1], -X));
                codes[r * (d / 2) + (b * 32 + j) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
}

ORC_API void orc_dequant_mxfp4(const uint8_t *codes, const uint8_t *scales, int64_t rows, int d,
                               double *out) {
    for (int64_t r = 0; r < rows; r++)
        for (int e = 0; e < d; e++) {
            uint8_t byte = codes[r * (d / 2) + e / 2];
            uint8_t c = (e & 1) ? (byte >> 4) : (byte & 15);
            int X = (int)scales[r * (d / 32) + e / 32] - 127;
            out[r * d + e] = ldexp(orc_e2m1_decode(c), X);
        }
}

/* ------------------------------------------------------------------------ */
/* RoPE on the last R dims (partial RoPE)                                     */
/* ------------------------------------------------------------------------ */

/* Rotary embedding of the RoPE slice at position p, in place.  Cited:
 * [firecat] item 2 (partial RoPE on the last 64 dims) and [mewclaw]
 * "Partial RoPE".  Reading: interleaved pairs (2j, 2j+1) of the slice,
 * inv_freq_j = theta^(-2j/R), angle p*inv_freq_j in double, cos and sin
 * evaluated in double and rounded to fp32, rotation done in double.
 * sign = +1 rotates forward, -1 applies the inverse rotation. */
static void rope_rotate(double *slice, int R, double p, double theta, int sign) {
    for (int j = 0; j < R / 2; j++) {
        double inv_freq = pow(theta, -2.0 * (double)j / (double)R);
        double ang = p * inv_freq;
        double c = (double)(float)cos(ang);
        double s = (double)(float)sin(ang) * (double)sign;
        double x = slice[2 * j], y = slice[2 * j + 1];
        slice[2 * j] = x * c - y * s;
        slice[2 * j + 1] = x * s + y * c;
    }
}

ORC_API void orc_rope(double *x, int64_t rows, int D, int R, const double *pos, double theta, int sign) {
    for (int64_t r = 0; r < rows; r++) rope_rotate(x + r * D + (D - R), R, pos[r], theta, sign);
}

/* ------------------------------------------------------------------------ */
/* a1 / a2: KV compressors                                                    */
/* ------------------------------------------------------------------------ */

/* Softmax-gated merge of a candidate set, per gate channel.  Each candidate c
 * is a token row X_c [D] with gate logits z_c [G] (already including the
 * positional bias).  For channel d (gate g = d when G == D, else 0), the
 * weights are softmax_c(z_c[g]) and the merged value is sum_c w_c * X_c[d].
 * A logit of -inf gets weight exactly 0.  Double precision. */
static void gated_merge(int ncand, const float *const *X, const double *logit /*[ncand][G]*/,
                        int G, int D, double *out) {
    for (int d = 0; d < D; d++) {
        int g = (G == 1) ? 0 : d;
        double mx = -INFINITY;
        for (int c = 0; c < ncand; c++) mx = fmax(mx, logit[c * G + g]);
        double den = 0.0, acc = 0.0;
        for (int c = 0; c < ncand; c++) {
            double w = exp(logit[c * G + g] - mx);
            den += w;
            acc += w * (double)X[c][d];
        }
        out[d] = acc / den;
    }
}

/* RMSNorm of one merged entry: y_d = x_d / sqrt(mean_d(x_d^2) + eps) * w_d.
 * Cited: [cyqw] section 2.3 (V4's attention lets RMSNorm act directly on the
 * queries and the KV entries, in place of QK-Clip).  Reading: the norm acts on
 * the merged fp32 entry before RoPE and quantisation; eps is a parameter. */
static void rms_norm(double *x, int D, const float *w, double eps) {
    double ss = 0.0;
    for (int d = 0; d < D; d++) ss += x[d] * x[d];
    const double r = 1.0 / sqrt(ss / (double)D + eps);
    for (int d = 0; d < D; d++) x[d] = x[d] * r * (double)w[d];
}

/* Query prologue for queries that arrive projected but not normalised or
 * rotated: each head's D-vector q (BF16 values) becomes RMSNorm(q) with the
 * weights w (shared by the heads), then its last R dims are rotated at
 * position pos, and the result is rounded to BF16 (nearest even), the
 * precision the queries enter the products in.  Cited: [cyqw] section 2.3
 * (RMSNorm acts directly on the queries) and [mewclaw] "Partial RoPE".
 *   q [H][D] BF16 bits -> out [H][D] BF16 bits */
ORC_API void orc_query_prologue(const uint16_t *q, int H, int D, const float *w, double eps, int R,
                                double pos, double theta, uint16_t *out) {
    double *x = malloc(sizeof(double) * D);
    for (int h = 0; h < H; h++) {
        for (int d = 0; d < D; d++) x[d] = orc_bf16_decode(q[h * D + d]);
        rms_norm(x, D, w, eps);
        if (R > 0) rope_rotate(x + (D - R), R, pos, theta, +1);
        for (int d = 0; d < D; d++) out[h * D + d] = orc_bf16_encode((float)x[d]);
    }
    free(x);
}

/* CSA compressor (ratio m, two streams with overlap).  Cited: [cyqw]
 * section 2.2 (every m = 4 tokens become one entry; two independent KV
 * sequences merged with softmax-normalised gate weights; adjacent compressed
 * blocks share part of their indices) and [chooseai] section 1 (softmax with
 * positional bias).  Reading: entry i merges A-block i (tokens m*i .. m*i+m-1
 * of stream A, logits gate_a[t] + bias_a[j]) with B-block i-1 (tokens
 * m*(i-1)+j of stream B, logits gate_b[t] + bias_b[j]); entry 0 has no
 * B-block and merges its A-block alone.  After the merge the entry is
 * RMS-normalised with weights norm_w (if not NULL), the RoPE slice is rotated
 * at position m*i (if apply_rope) and the entry is rounded to fp32.
 *   kv_a, kv_b [n_tok][D] fp32, row r holds token tok0 + r
 *   gate_a, gate_b [n_tok][G]; bias_a, bias_b [m][G]
 *   writes out [n_entries][D] fp32 for entries first_entry .. first_entry+n_entries-1.
 * Returns 0, or -1 if the rows do not cover the blocks the entries need. */
ORC_API int orc_compress_csa(const float *kv_a, const float *kv_b, int D, const float *gate_a,
                             const float *gate_b, int G, const float *bias_a, const float *bias_b,
                             int64_t tok0, int64_t n_tok, int m, int64_t first_entry,
                             int64_t n_entries, int apply_rope, int R, double theta,
                             const float *norm_w, double eps, float *out) {
    const float **X = malloc(sizeof(float *) * 2 * m);
    double *logit = malloc(sizeof(double) * 2 * m * G);
    double *tmp = malloc(sizeof(double) * D);
    int rc = 0;
    for (int64_t e = 0; e < n_entries && rc == 0; e++) {
        int64_t i = first_entry + e;
        int nc = 0;
        for (int j = 0; j < m; j++) {                 /* A-block i */
            int64_t r = m * i + j - tok0;
            if (r < 0 || r >= n_tok) { rc = -1; break; }
            X[nc] = kv_a + r * D;
            for (int g = 0; g < G; g++)
                logit[nc * G + g] = (double)gate_a[r * G + g] + (double)bias_a[j * G + g];
            nc++;
        }
        if (rc) break;
        if (i >= 1) {
            for (int j = 0; j < m; j++) {             /* B-block i-1 (the overlap) */
                int64_t r = m * (i - 1) + j - tok0;
                if (r < 0 || r >= n_tok) { rc = -1; break; }
                X[nc] = kv_b + r * D;
                for (int g = 0; g < G; g++)
                    logit[nc * G + g] = (double)gate_b[r * G + g] + (double)bias_b[j * G + g];
                nc++;
            }
        }
        if (rc) break;
        gated_merge(nc, X, logit, G, D, tmp);
        if (norm_w) rms_norm(tmp, D, norm_w, eps);
        if (apply_rope) rope_rotate(tmp + (D - R), R, (double)(m * i), theta, +1);
        for (int d = 0; d < D; d++) out[e * D + d] = (float)tmp[d];
    }
    free(X);
    free(logit);
    free(tmp);
    return rc;
}

/* HCA compressor (ratio m', one stream, no overlap).  Cited: [cyqw]
 * section 2.2 and [firecat] item 2 (every 128 tokens become one entry, no
 * sparse selection) and [chooseai] section 1 (no overlapped compression).
 * Entry i merges tokens m*i .. m*i+m-1 with logits gate[t] + bias[j]; then
 * RMSNorm (if norm_w), RoPE at m*i and rounding to fp32 as for CSA. */
ORC_API int orc_compress_hca(const float *kv, int D, const float *gate, int G, const float *bias,
                             int64_t tok0, int64_t n_tok, int m, int64_t first_entry,
                             int64_t n_entries, int apply_rope, int R, double theta,
                             const float *norm_w, double eps, float *out) {
    const float **X = malloc(sizeof(float *) * m);
    double *logit = malloc(sizeof(double) * m * G);
    double *tmp = malloc(sizeof(double) * D);
    int rc = 0;
    for (int64_t e = 0; e < n_entries && rc == 0; e++) {
        int64_t i = first_entry + e;
        for (int j = 0; j < m; j++) {
            int64_t r = m * i + j - tok0;
            if (r < 0 || r >= n_tok) { rc = -1; break; }
            X[j] = kv + r * D;
            for (int g = 0; g < G; g++)
                logit[j * G + g] = (double)gate[r * G + g] + (double)bias[j * G + g];
        }
        if (rc) break;
        gated_merge(m, X, logit, G, D, tmp);
        if (norm_w) rms_norm(tmp, D, norm_w, eps);
        if (apply_rope) rope_rotate(tmp + (D - R), R, (double)(m * i), theta, +1);
        for (int d = 0; d < D; d++) out[e * D + d] = (float)tmp[d];
    }
    free(X);
    free(logit);
    free(tmp);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* a4: lightning-indexer scores                                               */
/* ------------------------------------------------------------------------ */

/* Fixed-order head combine.  Reading (the pages only say the indexer is
 * multi-head and low precision, [cyqw] section 2.2): score = sum_h w_h *
 * ReLU(s_h) in fp32, with ReLU(s) = s if s > 0 else +0, evaluated as four
 * fma chains: chain g = (h >> 2) & 3 accumulates c_g = fmaf(w_h, r_h, c_g)
 * over ascending h from +0, then score = ((c0 + c1) + c2) + c3, and -0 is
 * replaced by +0. */
static float head_combine(const float *s, const float *w, int H) {
    float c[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int h = 0; h < H; h++) {
        float r = s[h] > 0.0f ? s[h] : 0.0f;
        int g = (h >> 2) & 3;
        c[g] = fmaf(w[h], r, c[g]);
    }
    float score = ((c[0] + c[1]) + c[2]) + c[3];
    if (score == 0.0f) score = 0.0f;
    return score;
}

/* Exact MXFP4 dot of two d-vectors, rounded once to fp32.  Per 32-element
 * block b the product of E2M1 values is an integer multiple of 1/4:
 * P_b = sum (2 q)(2 k) is an integer, and the block contributes
 * P_b * 2^(Xq_b + Xk_b - 2).  The sum over blocks is formed exactly (as an
 * integer times a power of two) and converted once to fp32 (nearest even).
 * *inexact is incremented when the exact value needs more than 24
 * significant bits, i.e. is not an fp32 number. */
/* Twice the E2M1 value of each 4-bit code: an integer (E2M1 values are multiples of 1/2). */
static int twice_e2m1[16];
static void init_twice_e2m1(void) {
    for (int c = 0; c < 16; c++) twice_e2m1[c] = (int)lround(2.0 * orc_e2m1_decode((uint8_t)c));
}

static float mxfp4_dot(const uint8_t *qc, const uint8_t *qs, const uint8_t *kc, const uint8_t *ks,
                       int d, int64_t *inexact) {
    int nb = d / 32;
    int64_t P[8];
    int E[8];
    int emin = 1 << 30;
    for (int b = 0; b < nb; b++) {
        int64_t acc = 0;
        for (int j = 0; j < 32; j++) {
            int e = b * 32 + j;
            uint8_t qb = qc[e / 2], kb = kc[e / 2];
            uint8_t qn = (e & 1) ? (qb >> 4) : (qb & 15);
            uint8_t kn = (e & 1) ? (kb >> 4) : (kb & 15);
            acc += (int64_t)twice_e2m1[qn] * (int64_t)twice_e2m1[kn];
        }
        P[b] = acc;
        E[b] = ((int)qs[b] - 127) + ((int)ks[b] - 127) - 2;
        if (acc != 0 && E[b] < emin) emin = E[b];
    }
    /* exact integer sum: value = T * 2^emin (needs the exponent spread to fit) */
    __int128 T = 0;
    int overflow = 0;
    for (int b = 0; b < nb; b++) {
        if (P[b] == 0) continue;
        int sh = E[b] - emin;
        if (sh > 100) { overflow = 1; break; }
        T += (__int128)P[b] << sh;
    }
    if (overflow) {
        long double v = 0.0L;
        for (int b = 0; b < nb; b++) v += ldexpl((long double)P[b], E[b]);
        (*inexact)++;
        return (float)v;
    }
    if (T == 0) return 0.0f;
    /* count significant bits of |T| after stripping trailing zeros */
    unsigned __int128 a = T < 0 ? (unsigned __int128)(-T) : (unsigned __int128)T;
    int e = emin;
    while ((a & 1) == 0) { a >>= 1; e++; }
    int bits = 0;
    for (unsigned __int128 t = a; t; t >>= 1) bits++;
    if (bits > 24) (*inexact)++;
    if (bits <= 53) {
        double v = ldexp((double)(uint64_t)a, e);   /* exact */
        return (float)(T < 0 ? -v : v);             /* one rounding, nearest even */
    }
    long double v = ldexpl((long double)a, e);       /* 64-bit mantissa; only reached if bits > 53 */
    return (float)(T < 0 ? -v : v);
}

/* MXFP4 indexer scores for one query against keys 0..n_keys-1.
 *   q_codes [H][d/2], q_scales [H][d/32], w [H]
 *   k_codes [n_keys][d/2], k_scales [n_keys][d/32]
 *   scores [n_keys] fp32; *inexact counts dots that are not fp32-exact.
 * Cited: [cyqw] section 2.2 and 3.4; [chooseai] section 1 (indexer QK in FP4);
 * per-head dots accumulate in fp32 (fixed reading). */
ORC_API void orc_indexer_scores_mxfp4(const uint8_t *q_codes, const uint8_t *q_scales, const float *w,
                                      int H, int d, const uint8_t *k_codes, const uint8_t *k_scales,
                                      int64_t n_keys, float *scores, int64_t *inexact) {
    int64_t bad = 0;
    init_twice_e2m1();
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (int64_t i = 0; i < n_keys; i++) {
        float s[256];
        for (int h = 0; h < H; h++)
            s[h] = mxfp4_dot(q_codes + (int64_t)h * (d / 2), q_scales + (int64_t)h * (d / 32),
                             k_codes + i * (d / 2), k_scales + i * (d / 32), d, &bad);
        scores[i] = head_combine(s, w, H);
    }
    *inexact = bad;
}

/* fp32 indexer scores (fp32 keys and queries): per head acc = +0,
 * acc = fmaf(q[e], k[e], acc) over ascending e, then the fixed head combine.
 *   q [H][d], w [H], keys [n_keys][d] */
ORC_API void orc_indexer_scores_f32(const float *q, const float *w, int H, int d, const float *keys,
                                    int64_t n_keys, float *scores) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_keys; i++) {
        float s[256];
        for (int h = 0; h < H; h++) {
            float acc = 0.0f;
            for (int e = 0; e < d; e++) acc = fmaf(q[h * d + e], keys[i * d + e], acc);
            s[h] = acc;
        }
        scores[i] = head_combine(s, w, H);
    }
}

/* ------------------------------------------------------------------------ */
/* a5: top-k                                                                  */
/* ------------------------------------------------------------------------ */

typedef struct { float s; int32_t i; } scored;

static int by_score_desc_index_asc(const void *a, const void *b) {
    const scored *x = a, *y = b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->i > y->i) - (x->i < y->i);
}

static int by_int_asc(const void *a, const void *b) {
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* The k best of scores[0..n_vis) under (score descending, index ascending):
 * the lowest index wins ties.  Cited: [cyqw] section 2.2 (each query picks
 * its top-k compressed entries; k = 1024 for Pro) and [chooseai] section 1
 * (k = 512 for Flash).  k_eff = min(k, n_vis); the chosen indices are
 * written in ascending order, then -1 up to k.  Scores must be finite. */
ORC_API void orc_topk(const float *scores, int64_t n_vis, int k, int32_t *out) {
    scored *v = malloc(sizeof(scored) * (n_vis > 0 ? n_vis : 1));
    for (int64_t i = 0; i < n_vis; i++) { v[i].s = scores[i]; v[i].i = (int32_t)i; }
    qsort(v, (size_t)n_vis, sizeof(scored), by_score_desc_index_asc);
    int64_t ke = n_vis < k ? n_vis : k;
    for (int64_t j = 0; j < ke; j++) out[j] = v[j].i;
    qsort(out, (size_t)ke, sizeof(int32_t), by_int_asc);
    for (int64_t j = ke; j < k; j++) out[j] = -1;
    free(v);
}

/* The same selection over the scores held in BF16: each score is first rounded
 * to the nearest BF16 value (ties to the even one), then the k best are chosen
 * under the same order, so scores that become equal are taken lowest index
 * first.  Cited: [cyqw] section 3.4 (the index score is stored as BF16 rather
 * than FP32, which doubles the speed of the top-k selector at 99.7% KV
 * recall).  Scores must be finite. */
ORC_API void orc_topk_bf16(const float *scores, int64_t n_vis, int k, int32_t *out) {
    float *r = malloc(sizeof(float) * (n_vis > 0 ? n_vis : 1));
    for (int64_t i = 0; i < n_vis; i++) r[i] = (float)orc_bf16_decode(orc_bf16_encode(scores[i]));
    orc_topk(r, n_vis, k, out);
    free(r);
}

/* ------------------------------------------------------------------------ */
/* a6 / a7: shared-KV MQA with sliding window and sink                        */
/* ------------------------------------------------------------------------ */

/* Attention of one query position over a key set.  Cited: [firecat] item 2
 * (multi-query attention over the selected compressed entries; head dim 512;
 * partial RoPE; SWA over the last 128 tokens; a learnable sink logit lets the
 * attention mass be below one), [cyqw] section 2.2 (the 128-token window
 * branch joins the core attention; the sink is a learnable term in the
 * softmax denominator) and [mewclaw] "Partial RoPE" (the output is treated so
 * values carry no absolute position).
 * Keys = entries (n_ent rows of E [n_ent][D]) followed by the window tokens
 * (n_win rows of Wn [n_win][D]); each key is also its value (shared KV, all D
 * dims).  For head h:
 *   z_j = scale * q_h . k_j,  M = max(sink_h, max_j z_j),
 *   den = exp(sink_h - M) + sum_j exp(z_j - M),  o = sum_j exp(z_j - M) k_j / den.
 * If rope_inverse, o's RoPE slice is rotated by -t_q.  Double precision.
 * mass (optional, [H]) receives sum_j p_j, the attention mass on real keys.
 *   q [H][D], sink [H], out [H][D] */
ORC_API void orc_attend(const double *q, int H, int D, const double *E, int64_t n_ent,
                        const double *Wn, int64_t n_win, const float *sink, double scale,
                        int rope_inverse, int R, double theta, double t_q, double *out,
                        double *mass) {
    int64_t n = n_ent + n_win;
#pragma omp parallel for schedule(static)
    for (int h = 0; h < H; h++) {
        double *z = malloc(sizeof(double) * (n > 0 ? n : 1));
        const double *qh = q + (int64_t)h * D;
        double M = (double)sink[h];
        for (int64_t j = 0; j < n; j++) {
            const double *k = j < n_ent ? E + j * D : Wn + (j - n_ent) * D;
            double acc = 0.0;
            for (int d = 0; d < D; d++) acc += qh[d] * k[d];
            z[j] = scale * acc;
            if (z[j] > M) M = z[j];
        }
        double den = exp((double)sink[h] - M), msum = 0.0;
        for (int64_t j = 0; j < n; j++) { z[j] = exp(z[j] - M); den += z[j]; msum += z[j]; }
        double *o = out + (int64_t)h * D;
        for (int d = 0; d < D; d++) o[d] = 0.0;
        for (int64_t j = 0; j < n; j++) {
            const double *k = j < n_ent ? E + j * D : Wn + (j - n_ent) * D;
            for (int d = 0; d < D; d++) o[d] += z[j] * k[d];
        }
        for (int d = 0; d < D; d++) o[d] /= den;
        if (mass) mass[h] = msum / den;
        if (rope_inverse) rope_rotate(o + (D - R), R, t_q, theta, -1);
        free(z);
    }
}

/* Grouped output projection: [cyqw] section 2.2 "Grouped Output Projection" (the head outputs
 * are reduced group by group, then concatenated and projected) and [firecat] item 2.  Reading:
 * G groups of H/G consecutive heads; each group's Kg = H*D/G values are projected to r values
 * by its own weights, the result is held as BF16 (the precision of activations), the G*r
 * values are concatenated and projected to d values by the final weights.  Double precision,
 * products and sums in plain loops. */

/* x rounded to the nearest BF16 value (8 significant bits), ties to even, from double directly
 * (no intermediate fp32 rounding); finite, normal-range inputs. */
ORC_API double orc_round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    const double m = frexp(x, &e);             /* x = m * 2^e, 0.5 <= |m| < 1 */
    const double r = nearbyint(ldexp(m, 8));   /* 8 significant bits, ties to even */
    return ldexp(r, e - 8);
}

/* y [T][G*r] (BF16 values, as double) of the attention output o [T][H*D] (BF16 bits) and the
 * group weights wg [G][r][Kg] (BF16 bits). */
ORC_API void orc_group_reduce(const uint16_t *o, int64_t T, int H, int D, int G, int r, const uint16_t *wg,
                              double *y) {
    const int64_t Kg = (int64_t)H * D / G;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; t++) {
        for (int g = 0; g < G; g++) {
            const uint16_t *x = o + t * (int64_t)H * D + g * Kg;
            for (int j = 0; j < r; j++) {
                const uint16_t *w = wg + ((int64_t)g * r + j) * Kg;
                double acc = 0.0;
                for (int64_t c = 0; c < Kg; c++) acc += orc_bf16_decode(x[c]) * orc_bf16_decode(w[c]);
                y[t * (int64_t)G * r + (int64_t)g * r + j] = orc_round_bf16(acc);
            }
        }
    }
}

/* out [T][N] = x [T][K] (double values) times the rows of w [N][K] (BF16 bits). */
ORC_API void orc_project(const double *x, int64_t T, int64_t K, const uint16_t *w, int64_t N, double *out) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t t = 0; t < T; t++) {
        for (int64_t n = 0; n < N; n++) {
            const uint16_t *wn = w + n * K;
            double acc = 0.0;
            for (int64_t c = 0; c < K; c++) acc += x[t * K + c] * orc_bf16_decode(wn[c]);
            out[t * N + n] = acc;
        }
    }
}
