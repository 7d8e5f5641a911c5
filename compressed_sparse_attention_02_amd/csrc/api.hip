// api.hip -- the C ABI of the hot path (declared in include/v4attn.h): host-side argument
// validation (always before any launch), workspace layout, and kernel dispatch.  No device
// memory is allocated here; scratch lives in the caller's workspace.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "compress.hpp"

namespace v4a {

static thread_local std::string g_err;

void set_error(const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

static v4a_status fail(v4a_status st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

static v4a_status hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return V4A_OK;
    return fail(V4A_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Kernel timing: while armed, every kernel launch takes the next start/stop event pair.
struct KernelTrace {
    std::vector<hipEvent_t> start, stop;
    std::vector<const char *> kernel;
    int n = 0;
    bool armed = false;
};
static KernelTrace g_trace;

bool trace_claim(const char *kernel, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_trace.armed || g_trace.n >= (int)g_trace.start.size()) return false;
    *start = g_trace.start[g_trace.n];
    *stop = g_trace.stop[g_trace.n];
    g_trace.kernel[g_trace.n++] = kernel;
    return true;
}

void fill_rope_table(RopeTable &t, int R, double theta) {
    for (int j = 0; j < kMaxRopePairs; j++)
        t.inv_freq[j] = (2 * j < R) ? pow(theta, -2.0 * (double)j / (double)R) : 0.0;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }
static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

static v4a_status check_kv(const v4a_kv *kv, const char *name) {
    if (!kv) return fail(V4A_EINVAL, "%s is NULL", name);
    if (kv->cap < 1) return fail(V4A_EINVAL, "%s->cap must be >= 1", name);
    if (kv->D < 2 || kv->D > 512 || kv->R < 0 || kv->R > kv->D || (kv->R & 1))
        return fail(V4A_EUNSUPPORTED, "%s: D=%d R=%d not supported", name, kv->D, kv->R);
    if (!kv->nope) return fail(V4A_EINVAL, "%s->nope is NULL", name);
    if (kv->fmt == V4A_KV_FP8_BF16) {
        if (!kv->scale || (kv->R > 0 && !kv->rope))
            return fail(V4A_EINVAL, "%s: FP8 records need rope and scale arrays", name);
        if (((kv->D - kv->R) % 8) != 0 || (kv->R % 4) != 0)
            return fail(V4A_EUNSUPPORTED, "%s: D-R must be a multiple of 8 and R of 4", name);
        if (!aligned(kv->nope, 16) || !aligned(kv->rope, 16) || !aligned(kv->scale, 4))
            return fail(V4A_EINVAL, "%s: record arrays must be 16-byte aligned", name);
    } else if (kv->fmt == V4A_KV_F32) {
        if (!aligned(kv->nope, 16)) return fail(V4A_EINVAL, "%s->nope must be 16-byte aligned", name);
    } else {
        return fail(V4A_EUNSUPPORTED, "%s: unknown record format %d", name, (int)kv->fmt);
    }
    return V4A_OK;
}

static v4a_status check_idx(const v4a_idx *x, const char *name) {
    if (!x) return fail(V4A_EINVAL, "%s is NULL", name);
    if (x->cap < 1) return fail(V4A_EINVAL, "%s->cap must be >= 1", name);
    if (!x->codes) return fail(V4A_EINVAL, "%s->codes is NULL", name);
    if (x->fmt == V4A_IDX_MXFP4) {
        // the scoring kernel addresses one slot's rows with 32-bit byte offsets
        if (x->cap > ((int64_t)1 << 26)) return fail(V4A_EUNSUPPORTED, "%s->cap: at most 2^26 MXFP4 rows per slot", name);
        if (x->d % 32 != 0 || x->d < 32 || x->d > 512)
            return fail(V4A_EUNSUPPORTED, "%s: MXFP4 needs d a multiple of 32 up to 512", name);
        if (!x->scales) return fail(V4A_EINVAL, "%s->scales is NULL", name);
        if (!aligned(x->codes, 16) || !aligned(x->scales, 4))
            return fail(V4A_EINVAL, "%s: codes must be 16-byte and scales 4-byte aligned", name);
    } else if (x->fmt == V4A_IDX_F32) {
        if (x->d < 1 || x->d > 512) return fail(V4A_EUNSUPPORTED, "%s: d=%d", name, x->d);
        if (!aligned(x->codes, 4)) return fail(V4A_EINVAL, "%s->codes misaligned", name);
    } else {
        return fail(V4A_EUNSUPPORTED, "%s: unknown format %d", name, (int)x->fmt);
    }
    return V4A_OK;
}

// ------------------------------------------------------------- indexer workspace ----
struct TopkWs {
    size_t keys, hist, list, counts, meta, total;
};

// Workspace of the indexer + top-k call: the per-query histograms (first, so that their place
// depends on B and Q only), orderable score keys, the per-slice ordered lists of keys at or
// above the threshold bin, their counts, and the per-query threshold.
static TopkWs topk_layout(int B, int Q, int64_t n_max, int k) {
    (void)k;
    TopkWs L{};
    const size_t BQ = (size_t)B * (size_t)Q;
    const size_t slices = (size_t)select_slices(n_max);
    size_t off = 0;
    L.hist = off;
    off = round_up(off + BQ * hist_copies((int64_t)BQ) * kHistBins * 4, 256);
    L.keys = off;
    off = round_up(off + BQ * (size_t)score_key_stride(n_max) * 4, 256);
    L.list = off;
    off = round_up(off + BQ * slices * kSelSlice * 8, 256);
    L.counts = off;
    off = round_up(off + BQ * slices * 4, 256);
    L.meta = off;
    off = round_up(off + BQ * 8, 256);
    L.total = off;
    return L;
}

static v4a_status fill_query_pos(QueryPos &qp, int B, int Q, int m, const int64_t *n_entries,
                                 const int64_t *q_pos, int64_t cap, int64_t *n_max) {
    if (B > kMaxSeq) return fail(V4A_EUNSUPPORTED, "B=%d exceeds %d sequences per call", B, kMaxSeq);
    memset(&qp, 0, sizeof qp);
    qp.Q = Q;
    qp.m = m;
    bool consecutive = true;
    for (int b = 0; b < B; b++) {
        if (n_entries[b] < 0) return fail(V4A_EINVAL, "n_entries[%d] < 0", b);
        if (n_entries[b] > cap) return fail(V4A_EINVAL, "n_entries[%d]=%lld exceeds keys->cap", b, (long long)n_entries[b]);
        qp.n_ent[b] = n_entries[b];
        for (int j = 0; j < Q; j++) {
            int64_t p = q_pos[(int64_t)b * Q + j];
            if (p < 0) return fail(V4A_EINVAL, "q_pos[%d] < 0", b * Q + j);
            if (p != q_pos[(int64_t)b * Q] + j) consecutive = false;
        }
    }
    if (consecutive) {
        qp.mode = 1;
        for (int b = 0; b < B; b++) qp.pos[b] = q_pos[(int64_t)b * Q];
    } else {
        if ((int64_t)B * Q > kMaxSeq)
            return fail(V4A_EUNSUPPORTED, "non-consecutive query positions need B*Q <= %d", kMaxSeq);
        qp.mode = 0;
        for (int i = 0; i < B * Q; i++) qp.pos[i] = q_pos[i];
    }
    int64_t mx = 0;
    for (int i = 0; i < B * Q; i++) {
        int64_t v = visible_keys(qp, i);
        if (v > mx) mx = v;
    }
    *n_max = mx;
    return V4A_OK;
}

static v4a_status check_indexer_args(const v4a_idx *keys, const int64_t *n_entries, int32_t m,
                                     const v4a_idx *q_idx, const float *w, int32_t B, int32_t Q,
                                     int32_t H_I, const int64_t *q_pos) {
    v4a_status st;
    if ((st = check_idx(keys, "keys")) != V4A_OK) return st;
    if ((st = check_idx(q_idx, "q_idx")) != V4A_OK) return st;
    if (!n_entries || !q_pos || !w) return fail(V4A_EINVAL, "n_entries, q_pos and w are required");
    if (keys->fmt != q_idx->fmt || keys->d != q_idx->d)
        return fail(V4A_EINVAL, "keys and q_idx must share format and d");
    if (keys->fmt == V4A_IDX_MXFP4 && keys->d != 128)
        return fail(V4A_EUNSUPPORTED, "the MXFP4 indexer supports d = 128");
    if (keys->fmt == V4A_IDX_F32 && (keys->d > 128))
        return fail(V4A_EUNSUPPORTED, "the fp32 indexer supports d <= 128");
    if (B < 1 || Q < 1) return fail(V4A_EINVAL, "B and Q must be >= 1");
    if (H_I < 4 || H_I > 64 || (H_I % 4) != 0)
        return fail(V4A_EUNSUPPORTED, "H_I=%d: need a multiple of 4 in [4, 64]", H_I);
    if ((int64_t)Q * H_I > q_idx->cap) return fail(V4A_EINVAL, "Q*H_I exceeds q_idx->cap");
    if (m < 1 || m > 128) return fail(V4A_EUNSUPPORTED, "m=%d not in [1, 128]", m);
    if (!aligned(w, 4)) return fail(V4A_EINVAL, "w misaligned");
    return V4A_OK;
}

}  // namespace v4a

using namespace v4a;

extern "C" {

size_t v4a_output_projection_workspace(int32_t T, int32_t G, int32_t r) {
    if (T < 0 || G < 1 || r < 1) return 0;
    return round_up((size_t)T * G * r * 2, 256);
}

v4a_status v4a_output_projection(const void *o, int32_t T, int32_t H, int32_t D, int32_t G, int32_t r,
                                 const void *wg, const void *wf, int32_t d, void *out, v4a_float out_t,
                                 void *ws, size_t ws_bytes, void *stream) {
    const char *name = "v4a_output_projection";
    if (T < 0) return fail(V4A_EINVAL, "%s: T < 0", name);
    if (H < 1 || D < 1 || G < 1 || r < 1 || d < 1 || H % G != 0)
        return fail(V4A_EUNSUPPORTED, "%s: H=%d D=%d G=%d r=%d d=%d (G must divide H)", name, H, D, G, r, d);
    const int64_t Kg = (int64_t)H * D / G;
    if (Kg % 128 != 0 || ((int64_t)G * r) % 128 != 0 || r % 16 != 0 || d % 16 != 0)
        return fail(V4A_EUNSUPPORTED, "%s: H*D/G and G*r must be multiples of 128, r and d of 16", name);
    if (Kg > (1 << 30) || (int64_t)G * r > (1 << 30)) return fail(V4A_EUNSUPPORTED, "%s: too large", name);
    if (out_t != V4A_F32 && out_t != V4A_BF16) return fail(V4A_EINVAL, "%s: bad out_t", name);
    if (T == 0) return V4A_OK;
    if (!o || !wg || !wf || !out) return fail(V4A_EINVAL, "%s: o, wg, wf and out are required", name);
    if (!aligned(o, 16) || !aligned(wg, 16) || !aligned(wf, 16) || !aligned(out, 16))
        return fail(V4A_EINVAL, "%s: o, wg, wf and out must be 16-byte aligned", name);
    const size_t need = v4a_output_projection_workspace(T, G, r);
    if (!ws || ws_bytes < need || !aligned(ws, 256))
        return fail(V4A_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", name, need, ws_bytes);
    OutProjArgs a{};
    a.o = o; a.T = T; a.H = H; a.D = D; a.G = G; a.r = r; a.d = d;
    a.wg = wg; a.wf = wf; a.y = ws; a.out = out; a.out_bf16 = out_t == V4A_BF16;
    g_err.clear();
    return hip_status(launch_output_projection(a, (hipStream_t)stream), name);
}

const char *v4a_last_error(void) { return g_err.c_str(); }

const char *v4a_version(void) { return "v4attn 0.1.0 (gfx950)"; }

v4a_status v4a_quantize_kv(const float *x, int64_t rows, const v4a_kv *out, int64_t row0, void *stream) {
    v4a_status st = check_kv(out, "out");
    if (st != V4A_OK) return st;
    if (rows < 0 || row0 < 0) return fail(V4A_EINVAL, "rows and row0 must be >= 0");
    if (rows > 0 && !x) return fail(V4A_EINVAL, "x is NULL");
    if (x && !aligned(x, 16)) return fail(V4A_EINVAL, "x must be 16-byte aligned");
    if (out->D != 32 && out->D != 64 && out->D != 128 && out->D != 256 && out->D != 512)
        return fail(V4A_EUNSUPPORTED, "D=%d: need 32, 64, 128, 256 or 512", out->D);
    const int vpt = out->D >= 64 ? out->D / 64 : 1;
    if (((out->D - out->R) % vpt) != 0) return fail(V4A_EUNSUPPORTED, "D-R must be a multiple of D/64");
    g_err.clear();
    return hip_status(launch_quantize_kv(x, rows, *out, row0, (hipStream_t)stream), "v4a_quantize_kv");
}

v4a_status v4a_quantize_mxfp4(const float *x, int64_t rows, const v4a_idx *out, int64_t row0, void *stream) {
    v4a_status st = check_idx(out, "out");
    if (st != V4A_OK) return st;
    if (rows < 0 || row0 < 0) return fail(V4A_EINVAL, "rows and row0 must be >= 0");
    if (rows > 0 && !x) return fail(V4A_EINVAL, "x is NULL");
    if (out->d != 32 && out->d != 64 && out->d != 128 && out->d != 256 && out->d != 512)
        return fail(V4A_EUNSUPPORTED, "d=%d: need 32, 64, 128, 256 or 512", out->d);
    g_err.clear();
    return hip_status(launch_quantize_mxfp4(x, rows, *out, row0, (hipStream_t)stream), "v4a_quantize_mxfp4");
}

static v4a_status compress_check(CompressArgs &a, const float *norm_w) {
    if (norm_w && !aligned(norm_w, 4)) return fail(V4A_EINVAL, "norm_w is misaligned");
    a.norm_w = norm_w;
    if (a.D != 32 && a.D != 64 && a.D != 128 && a.D != 256 && a.D != 512)
        return fail(V4A_EUNSUPPORTED, "D=%d: need 32, 64, 128, 256 or 512", a.D);
    if (a.G != 1 && a.G != a.D) return fail(V4A_EUNSUPPORTED, "G must be 1 or D");
    if (a.m < 1 || a.m > 128) return fail(V4A_EUNSUPPORTED, "m=%d not in [1, 128]", a.m);
    if (a.n_entries < 0 || a.first_entry < 0 || a.n_tok < 0) return fail(V4A_EINVAL, "negative size");
    if (a.tok0 % a.m != 0) return fail(V4A_EINVAL, "tok0 must be a multiple of m");
    if (a.b0 < 0 || a.n_seq < 0) return fail(V4A_EINVAL, "b0 and n_seq must be >= 0");
    if (a.n_seq > 65535) return fail(V4A_EUNSUPPORTED, "n_seq > 65535");
    for (int s = 0; s < a.n_streams; s++)
        if (a.n_entries > 0 && (!a.x[s] || !a.gate[s] || !a.bias[s]))
            return fail(V4A_EINVAL, "stream, gate and bias pointers are required");
    if (a.n_entries > 0) {
        const int64_t need_lo = a.n_streams == 2 ? (a.first_entry >= 1 ? a.m * (a.first_entry - 1) : 0)
                                                 : a.m * a.first_entry;
        const int64_t need_hi = a.m * (a.first_entry + a.n_entries);
        if (a.tok0 > need_lo || a.tok0 + a.n_tok < need_hi)
            return fail(V4A_EINVAL, "rows [%lld, %lld) do not cover tokens [%lld, %lld)", (long long)a.tok0,
                        (long long)(a.tok0 + a.n_tok), (long long)need_lo, (long long)need_hi);
    }
    if (a.kv) {
        v4a_status st = check_kv(a.kv, "out_kv");
        if (st != V4A_OK) return st;
        if (a.kv->D != a.D) return fail(V4A_EINVAL, "out_kv->D != D");
        if (a.first_entry + a.n_entries > a.kv->cap) return fail(V4A_EINVAL, "entries exceed out_kv->cap");
        if (a.rope && (a.kv->R < 2)) return fail(V4A_EINVAL, "apply_rope needs R >= 2");
        if (a.rope && a.kv->R > 2 * kMaxRopePairs) return fail(V4A_EUNSUPPORTED, "apply_rope supports R <= 64");
        a.R = a.kv->R;
        const int vpt = a.D >= 64 ? a.D / 64 : 1;
        if (((a.D - a.R) % vpt) != 0) return fail(V4A_EUNSUPPORTED, "D-R must be a multiple of D/64");
    } else {
        v4a_status st = check_idx(a.idx, "out_idx");
        if (st != V4A_OK) return st;
        if (a.idx->d != a.D) return fail(V4A_EINVAL, "out_idx->d != D");
        if (a.first_entry + a.n_entries > a.idx->cap) return fail(V4A_EINVAL, "entries exceed out_idx->cap");
        a.rope = false;
        a.R = 0;
    }
    return V4A_OK;
}

static v4a_status compress_common(CompressArgs &a, const float *norm_w, void *stream) {
    v4a_status st = compress_check(a, norm_w);
    if (st != V4A_OK) return st;
    g_err.clear();
    return hip_status(launch_compress(a, (hipStream_t)stream), "compress");
}

v4a_status v4a_compress_csa(const void *kv_a, const void *kv_b, v4a_float in_t, int32_t D, const float *gate_a,
                            const float *gate_b, int32_t G, const float *bias_a, const float *bias_b, int64_t tok0,
                            int64_t n_tok, int32_t m, int64_t first_entry, int64_t n_entries, int32_t apply_rope,
                            float rope_theta, const float *norm_w, const v4a_kv *out_kv, const v4a_idx *out_idx,
                            int32_t b0, int32_t n_seq, void *stream) {
    if ((out_kv == nullptr) == (out_idx == nullptr))
        return fail(V4A_EINVAL, "exactly one of out_kv and out_idx must be given");
    if (in_t != V4A_F32 && in_t != V4A_BF16) return fail(V4A_EINVAL, "in_t");
    CompressArgs a{};
    a.x[0] = kv_a;
    a.x[1] = kv_b;
    a.gate[0] = gate_a;
    a.gate[1] = gate_b;
    a.bias[0] = bias_a;
    a.bias[1] = bias_b;
    a.n_streams = 2;
    a.bf16_in = in_t == V4A_BF16;
    a.D = D;
    a.G = G;
    a.m = m;
    a.tok0 = tok0;
    a.n_tok = n_tok;
    a.first_entry = first_entry;
    a.n_entries = n_entries;
    a.rope = apply_rope != 0;
    a.theta = rope_theta;
    a.kv = out_kv;
    a.idx = out_idx;
    a.b0 = b0;
    a.n_seq = n_seq;
    return compress_common(a, norm_w, stream);
}

v4a_status v4a_compress_hca(const void *kv, v4a_float in_t, int32_t D, const float *gate, int32_t G,
                            const float *bias, int64_t tok0, int64_t n_tok, int32_t m, int64_t first_entry,
                            int64_t n_entries, int32_t apply_rope, float rope_theta, const float *norm_w,
                            const v4a_kv *out_kv, int32_t b0, int32_t n_seq, void *stream) {
    if (!out_kv) return fail(V4A_EINVAL, "out_kv is NULL");
    if (in_t != V4A_F32 && in_t != V4A_BF16) return fail(V4A_EINVAL, "in_t");
    CompressArgs a{};
    a.x[0] = kv;
    a.x[1] = kv;
    a.gate[0] = gate;
    a.gate[1] = gate;
    a.bias[0] = bias;
    a.bias[1] = bias;
    a.n_streams = 1;
    a.bf16_in = in_t == V4A_BF16;
    a.D = D;
    a.G = G;
    a.m = m;
    a.tok0 = tok0;
    a.n_tok = n_tok;
    a.first_entry = first_entry;
    a.n_entries = n_entries;
    a.rope = apply_rope != 0;
    a.theta = rope_theta;
    a.kv = out_kv;
    a.b0 = b0;
    a.n_seq = n_seq;
    return compress_common(a, norm_w, stream);
}

size_t v4a_indexer_topk_workspace(int32_t B, int32_t Q, int64_t n_max, int32_t k) {
    if (B < 0 || Q < 0 || n_max < 0 || k < 0) return 0;
    return topk_layout(B, Q, n_max, k).total;
}

}  // extern "C"

namespace v4a {

// Launches of the indexer + top-k call once every argument has been checked.
static v4a_status indexer_topk_launch(const v4a_idx *keys, const QueryPos &qp, int64_t n_max, const v4a_idx *q_idx,
                                      const float *w, int32_t B, int32_t Q, int32_t H_I, int32_t k, int32_t *out_idx,
                                      void *ws, hipStream_t s, bool clear_hist = true, bool key16 = false,
                                      const CompressArgs *rec = nullptr, const CompressArgs *key_rec = nullptr,
                                      bool clear_after = false) {
    const TopkWs L = topk_layout(B, Q, n_max, k);
    char *base = (char *)ws;
    const size_t BQ = (size_t)B * Q;
    hipError_t e = hipSuccess;
    if (clear_hist) {
        e = launch_zero(base + L.hist, BQ * hist_copies((int64_t)BQ) * kHistBins * 4, s);
        if (e != hipSuccess) return hip_status(e, "v4a_indexer_topk: clear");
    }
    IndexerArgs ia{};
    ia.keys = keys;
    ia.q = q_idx;
    ia.w = w;
    ia.B = B;
    ia.Q = Q;
    ia.H_I = H_I;
    ia.n_max = n_max;
    ia.key_stride = score_key_stride(n_max);
    ia.score_keys = base + L.keys;
    ia.key16 = key16;
    ia.hist = (uint32_t *)(base + L.hist);
    ia.hist_copies = hist_copies((int64_t)BQ);
    ia.key_rec = key_rec;
    if ((e = launch_indexer(ia, qp, s)) != hipSuccess) return hip_status(e, "v4a_indexer_topk: scores");
    SelectArgs sa{};
    sa.score_keys = ia.score_keys;
    sa.key_stride = ia.key_stride;
    sa.key16 = key16;
    sa.hist = ia.hist;
    sa.hist_copies = ia.hist_copies;
    sa.n_max = n_max;
    sa.BQ = (int)BQ;
    sa.k = k;
    sa.list = (uint32_t *)(base + L.list);
    sa.counts = (uint32_t *)(base + L.counts);
    sa.meta = (int32_t *)(base + L.meta);
    sa.out = out_idx;
    sa.rec = rec;
    sa.hist_clear = clear_after ? ia.hist : nullptr;
    return hip_status(launch_select(sa, qp, s), "v4a_indexer_topk: select");
}

}  // namespace v4a

extern "C" {

}  // extern "C"

namespace v4a {

static v4a_status indexer_topk_entry(const v4a_idx *keys, const int64_t *n_entries, int32_t m, const v4a_idx *q_idx,
                                     const float *w, int32_t B, int32_t Q, int32_t H_I, const int64_t *q_pos,
                                     int32_t k, int32_t *out_idx, void *ws, size_t ws_bytes, void *stream,
                                     bool key16) {
    v4a_status st = check_indexer_args(keys, n_entries, m, q_idx, w, B, Q, H_I, q_pos);
    if (st != V4A_OK) return st;
    if (k < 1 || k > 2048) return fail(V4A_EUNSUPPORTED, "k=%d not in [1, 2048]", k);
    if (!out_idx || !aligned(out_idx, 4)) return fail(V4A_EINVAL, "out_idx is NULL or misaligned");
    QueryPos qp;
    int64_t n_max = 0;
    if ((st = fill_query_pos(qp, B, Q, m, n_entries, q_pos, keys->cap, &n_max)) != V4A_OK) return st;
    if (n_max > (int64_t)1024 * kSelSlice) return fail(V4A_EUNSUPPORTED, "more than %d visible keys per query", 1024 * kSelSlice);
    const TopkWs L = topk_layout(B, Q, n_max, k);
    if (!ws || ws_bytes < L.total || !aligned(ws, 256))
        return fail(V4A_EWORKSPACE, "workspace needs %zu bytes, 256-byte aligned (got %zu)", L.total, ws_bytes);
    g_err.clear();
    return indexer_topk_launch(keys, qp, n_max, q_idx, w, B, Q, H_I, k, out_idx, ws, (hipStream_t)stream, true, key16);
}

}  // namespace v4a

extern "C" {

v4a_status v4a_indexer_topk(const v4a_idx *keys, const int64_t *n_entries, int32_t m, const v4a_idx *q_idx,
                            const float *w, int32_t B, int32_t Q, int32_t H_I, const int64_t *q_pos, int32_t k,
                            int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    return indexer_topk_entry(keys, n_entries, m, q_idx, w, B, Q, H_I, q_pos, k, out_idx, ws, ws_bytes, stream, false);
}

v4a_status v4a_indexer_topk_bf16(const v4a_idx *keys, const int64_t *n_entries, int32_t m, const v4a_idx *q_idx,
                                 const float *w, int32_t B, int32_t Q, int32_t H_I, const int64_t *q_pos, int32_t k,
                                 int32_t *out_idx, void *ws, size_t ws_bytes, void *stream) {
    return indexer_topk_entry(keys, n_entries, m, q_idx, w, B, Q, H_I, q_pos, k, out_idx, ws, ws_bytes, stream, true);
}

v4a_status v4a_indexer_scores(const v4a_idx *keys, const int64_t *n_entries, int32_t m, const v4a_idx *q_idx,
                              const float *w, int32_t B, int32_t Q, int32_t H_I, const int64_t *q_pos,
                              int64_t n_max, float *out_scores, void *stream) {
    v4a_status st = check_indexer_args(keys, n_entries, m, q_idx, w, B, Q, H_I, q_pos);
    if (st != V4A_OK) return st;
    if (!out_scores) return fail(V4A_EINVAL, "out_scores is NULL");
    QueryPos qp;
    int64_t vis_max = 0;
    if ((st = fill_query_pos(qp, B, Q, m, n_entries, q_pos, keys->cap, &vis_max)) != V4A_OK) return st;
    if (n_max < vis_max) return fail(V4A_EINVAL, "n_max=%lld is below the visible count %lld", (long long)n_max,
                                     (long long)vis_max);
    g_err.clear();
    IndexerArgs ia{};
    ia.keys = keys;
    ia.q = q_idx;
    ia.w = w;
    ia.B = B;
    ia.Q = Q;
    ia.H_I = H_I;
    ia.n_max = n_max;
    ia.key_stride = score_key_stride(n_max);
    ia.scores = out_scores;
    return hip_status(launch_indexer(ia, qp, (hipStream_t)stream), "v4a_indexer_scores");
}

}  // extern "C"

// ------------------------------------------------------------------- decode ----------
namespace v4a {

constexpr int kDecodeSplitTarget = 16;

// The most splits any sequence of at most n_keys_max keys gets (the plan is not monotonic in the
// key count: short lists take at most two tiles per split).
static int decode_split_cap(int64_t n_keys_max) {
    int cap = 1;
    const int64_t n = n_keys_max < (int64_t)kAttnTile * 4096 ? n_keys_max : (int64_t)kAttnTile * 4096;
    for (int64_t tiles = 1; tiles * kAttnTile <= n + kAttnTile - 1; tiles++) {
        int tps, sp;
        split_plan_host((int)(tiles * kAttnTile), kDecodeSplitTarget, &tps, &sp);
        if (sp > cap) cap = sp;
    }
    return cap;
}

static size_t decode_ws_bytes(int B, int H, int D, int split_cap) {
    if (split_cap <= 1) return 0;
    // BF16 partial sums, then fp32 (m, l) per head
    return round_up((size_t)B * split_cap * H * D * 2 + (size_t)B * split_cap * H * 2 * 4, 256);
}

// Checks a decode call's attention arguments, fills the per-sequence window lengths and
// positions and the split plan, and returns the workspace it needs; launches nothing.
static v4a_status decode_prepare(AttnArgs &a, SeqInfo &sq, const int32_t *win_len, const int64_t *q_pos,
                                 v4a_float q_t, v4a_float win_t, v4a_float out_t, size_t *ws_need,
                                 const char *name, bool no_split = false) {
    if (!a.q || !a.out || !a.sink || !q_pos) return fail(V4A_EINVAL, "%s: q, out, sink and q_pos are required", name);
    if (a.B < 1 || a.B > kMaxSeq) return fail(V4A_EUNSUPPORTED, "%s: B=%d not in [1, %d]", name, a.B, kMaxSeq);
    if (a.H < 1 || a.H > 128) return fail(V4A_EUNSUPPORTED, "%s: H=%d not in [1, 128]", name, a.H);
    if (a.W < 0 || a.W > 128) return fail(V4A_EUNSUPPORTED, "%s: W=%d not in [0, 128]", name, a.W);
    if (a.W > 0 && (!a.win || !win_len)) return fail(V4A_EINVAL, "%s: win and win_len are required", name);
    if ((q_t != V4A_F32 && q_t != V4A_BF16) || (win_t != V4A_F32 && win_t != V4A_BF16) ||
        (out_t != V4A_F32 && out_t != V4A_BF16))
        return fail(V4A_EINVAL, "%s: bad element type", name);
    a.q_bf16 = q_t == V4A_BF16;
    a.win_bf16 = win_t == V4A_BF16;
    a.out_bf16 = out_t == V4A_BF16;
    a.D = a.kv->D;
    a.R = a.kv->R;
    if (a.D % 2 != 0 || (a.rope_inv && (a.R < 2 || a.R > 2 * kMaxRopePairs)))
        return fail(V4A_EUNSUPPORTED, "%s: odd D, or R not in [2, 64] with out_rope_inverse", name);
    if (!aligned(a.q, 16) || !aligned(a.out, 16) || (a.win && !aligned(a.win, 16)))
        return fail(V4A_EINVAL, "%s: q, win and out must be 16-byte aligned", name);
    int64_t n_keys_max = 0;
    for (int b = 0; b < a.B; b++) {
        const int wl = a.W > 0 ? win_len[b] : 0;
        if (wl < 0 || wl > a.W) return fail(V4A_EINVAL, "%s: win_len[%d]=%d not in [0, W]", name, b, wl);
        if (q_pos[b] < 0) return fail(V4A_EINVAL, "%s: q_pos[%d] < 0", name, b);
        sq.win_len[b] = wl;
        sq.q_pos[b] = q_pos[b];
        if ((int64_t)sq.n_ent[b] + wl > n_keys_max) n_keys_max = (int64_t)sq.n_ent[b] + wl;
    }
    const bool mfma = attn_uses_mfma(a);
    if (!mfma && n_keys_max > 8192 + 2048)
        return fail(V4A_EUNSUPPORTED, "%s: this format/shape uses the fp32 kernel, limited to %d keys", name, 8192 + 2048);
    a.no_split = mfma && no_split;
    if (mfma && no_split) {
        if (a.H % 16 != 0) return fail(V4A_EUNSUPPORTED, "%s: the split-free attention needs H a multiple of 16", name);
        a.target_splits = 1;
        a.split_cap = 1;
        *ws_need = 0;
    } else if (mfma) {
        a.target_splits = kDecodeSplitTarget;
        int cap = 1;
        for (int b = 0; b < a.B; b++) {
            int tps, sp;
            split_plan_host(sq.n_ent[b] + sq.win_len[b], kDecodeSplitTarget, &tps, &sp);
            if (sp > cap) cap = sp;
        }
        a.split_cap = cap;
        *ws_need = decode_ws_bytes(a.B, a.H, a.D, cap);
    } else {
        a.target_splits = 1;
        a.split_cap = 1;
        *ws_need = 0;
    }
    a.partial = nullptr;
    return V4A_OK;
}

static v4a_status decode_common(AttnArgs &a, SeqInfo &sq, const int32_t *win_len, const int64_t *q_pos,
                                v4a_float q_t, v4a_float win_t, v4a_float out_t, void *ws, size_t ws_bytes,
                                void *stream, const char *name) {
    size_t need = 0;
    v4a_status st = decode_prepare(a, sq, win_len, q_pos, q_t, win_t, out_t, &need, name);
    if (st != V4A_OK) return st;
    if (need > 0 && (!ws || ws_bytes < need || !aligned(ws, 256)))
        return fail(V4A_EWORKSPACE, "%s: workspace needs %zu bytes, 256-byte aligned (got %zu)", name, need, ws_bytes);
    a.partial = need > 0 ? (float *)ws : nullptr;
    g_err.clear();
    return hip_status(launch_attention(a, sq, (hipStream_t)stream), name);
}

}  // namespace v4a

extern "C" {

size_t v4a_decode_workspace(int32_t B, int32_t H, int32_t D, int64_t n_keys_max, int32_t W) {
    if (B < 0 || H < 0 || D < 0 || n_keys_max < 0 || W < 0) return 0;
    return decode_ws_bytes(B, H, D, decode_split_cap(n_keys_max + W));
}

v4a_status v4a_decode_csa(const void *q, v4a_float q_t, int32_t B, int32_t H, const v4a_kv *kv,
                          const int32_t *topk_idx, int32_t k, const void *win, v4a_float win_t,
                          const int32_t *win_len, int32_t W, const float *sink, const int64_t *q_pos,
                          float softmax_scale, int32_t out_rope_inverse, float rope_theta, void *out,
                          v4a_float out_t, void *ws, size_t ws_bytes, void *stream) {
    v4a_status st = check_kv(kv, "kv");
    if (st != V4A_OK) return st;
    if (!topk_idx || !aligned(topk_idx, 4)) return fail(V4A_EINVAL, "v4a_decode_csa: topk_idx is NULL or misaligned");
    if (k < 1 || k > 2048) return fail(V4A_EUNSUPPORTED, "v4a_decode_csa: k=%d not in [1, 2048]", k);
    AttnArgs a{};
    SeqInfo sq;
    memset(&sq, 0, sizeof sq);
    a.q = q;
    a.B = B;
    a.H = H;
    a.kv = kv;
    a.kv_bstride = kv->cap;
    a.topk = topk_idx;
    a.k = k;
    a.win = win;
    a.W = W;
    a.sink = sink;
    a.scale = softmax_scale;
    a.rope_inv = out_rope_inverse != 0;
    a.theta = rope_theta;
    a.out = out;
    if (B >= 1 && B <= kMaxSeq)
        for (int b = 0; b < B; b++) sq.n_ent[b] = k;
    return decode_common(a, sq, win_len, q_pos, q_t, win_t, out_t, ws, ws_bytes, stream, "v4a_decode_csa");
}

v4a_status v4a_decode_hca(const void *q, v4a_float q_t, int32_t B, int32_t H, const v4a_kv *kv,
                          const int64_t *n_entries, int32_t m, const void *win, v4a_float win_t,
                          const int32_t *win_len, int32_t W, const float *sink, const int64_t *q_pos,
                          float softmax_scale, int32_t out_rope_inverse, float rope_theta, void *out,
                          v4a_float out_t, void *ws, size_t ws_bytes, void *stream) {
    v4a_status st = check_kv(kv, "kv");
    if (st != V4A_OK) return st;
    if (!n_entries || !q_pos) return fail(V4A_EINVAL, "v4a_decode_hca: n_entries and q_pos are required");
    if (m < 1) return fail(V4A_EINVAL, "v4a_decode_hca: m < 1");
    if (B < 1 || B > kMaxSeq) return fail(V4A_EUNSUPPORTED, "v4a_decode_hca: B=%d not in [1, %d]", B, kMaxSeq);
    AttnArgs a{};
    SeqInfo sq;
    memset(&sq, 0, sizeof sq);
    for (int b = 0; b < B; b++) {
        if (n_entries[b] < 0 || n_entries[b] > kv->cap)
            return fail(V4A_EINVAL, "v4a_decode_hca: n_entries[%d] not in [0, cap]", b);
        if (q_pos[b] < 0) return fail(V4A_EINVAL, "v4a_decode_hca: q_pos[%d] < 0", b);
        int64_t vis = (q_pos[b] + 1) / m;
        if (vis > n_entries[b]) vis = n_entries[b];
        if (vis > (1 << 30)) return fail(V4A_EUNSUPPORTED, "v4a_decode_hca: too many entries");
        sq.n_ent[b] = (int32_t)vis;
    }
    a.q = q;
    a.B = B;
    a.H = H;
    a.kv = kv;
    a.kv_bstride = kv->cap;
    a.topk = nullptr;
    a.k = 0;
    a.win = win;
    a.W = W;
    a.sink = sink;
    a.scale = softmax_scale;
    a.rope_inv = out_rope_inverse != 0;
    a.theta = rope_theta;
    a.out = out;
    return decode_common(a, sq, win_len, q_pos, q_t, win_t, out_t, ws, ws_bytes, stream, "v4a_decode_hca");
}

}  // extern "C"

// ------------------------------------------------------------------- prefill ---------
namespace v4a {

struct PrefillPlan {
    bool csa;
    int64_t first, n_new, n_total;   // entries written, entries in the cache afterwards
    CompressArgs ckv, cidx;
    v4a_kv kv;                       // the sequence's slot (record rows 0 .. cap-1)
    v4a_idx keys;
    QueryPos qp;
    size_t idx_bytes, topk_bytes, ws_total;
};

static const char *ptr_at(const void *p, int64_t elems, size_t esz) {
    return p ? (const char *)p + elems * (int64_t)esz : nullptr;
}

// Checks every argument of a prefill chunk and lays out its launches; launches nothing.
static v4a_status prefill_plan(v4a_layer kind, const v4a_prefill_args *a, PrefillPlan &pl) {
    if (!a) return fail(V4A_EINVAL, "v4a_prefill_chunk: args is NULL");
    if (kind != V4A_LAYER_CSA && kind != V4A_LAYER_HCA) return fail(V4A_EINVAL, "v4a_prefill_chunk: kind=%d", (int)kind);
    pl = PrefillPlan{};
    pl.csa = kind == V4A_LAYER_CSA;
    v4a_status st = check_kv(a->kv, "kv");
    if (st != V4A_OK) return st;
    const int D = a->kv->D;
    if (a->C < 0 || a->C > 65535) return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: C=%d not in [0, 65535]", a->C);
    if (a->tok0 < 0) return fail(V4A_EINVAL, "v4a_prefill_chunk: tok0 < 0");
    if (a->m < 1 || a->m > 128) return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: m=%d not in [1, 128]", a->m);
    if (a->tok0 % a->m != 0) return fail(V4A_EINVAL, "v4a_prefill_chunk: tok0 must be a multiple of m");
    if (a->W < 0 || a->W > 128) return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: W=%d not in [0, 128]", a->W);
    if (a->n_prev < 0 || a->n_prev > a->tok0) return fail(V4A_EINVAL, "v4a_prefill_chunk: n_prev not in [0, tok0]");
    int64_t need_prev = a->W > 0 ? (a->tok0 < a->W - 1 ? a->tok0 : a->W - 1) : 0;
    if (pl.csa && a->tok0 > 0 && need_prev < a->m) need_prev = a->m;
    if (a->n_prev < need_prev)
        return fail(V4A_EINVAL, "v4a_prefill_chunk: n_prev=%d, the window and blocks need %lld rows before tok0",
                    a->n_prev, (long long)need_prev);
    if (a->slot < 0) return fail(V4A_EINVAL, "v4a_prefill_chunk: slot < 0");
    if (a->in_t != V4A_F32 && a->in_t != V4A_BF16) return fail(V4A_EINVAL, "v4a_prefill_chunk: in_t");
    if ((a->q_t != V4A_F32 && a->q_t != V4A_BF16) || (a->out_t != V4A_F32 && a->out_t != V4A_BF16))
        return fail(V4A_EINVAL, "v4a_prefill_chunk: q_t / out_t");
    if (a->H < 1 || a->H > 128) return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: H=%d not in [1, 128]", a->H);
    if (!a->q || !a->out || !a->sink || !a->kv_a) return fail(V4A_EINVAL, "v4a_prefill_chunk: q, out, sink and kv_a are required");
    if (!aligned(a->q, 16) || !aligned(a->out, 16) || !aligned(a->kv_a, 16))
        return fail(V4A_EINVAL, "v4a_prefill_chunk: q, out and kv_a must be 16-byte aligned");
    if (D % 2 != 0 || (a->out_rope_inverse && (a->kv->R < 2 || a->kv->R > 2 * kMaxRopePairs)))
        return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: odd D, or R not in [2, 64] with out_rope_inverse");
    pl.first = a->tok0 / a->m;
    pl.n_total = (a->tok0 + a->C) / a->m;
    pl.n_new = pl.n_total - pl.first;
    if (pl.n_total > a->kv->cap) return fail(V4A_EINVAL, "v4a_prefill_chunk: %lld entries exceed kv->cap", (long long)pl.n_total);
    const size_t esz = a->in_t == V4A_BF16 ? 2 : 4;
    // the compressor reads from row n_prev - mneed: CSA also needs the B-block before tok0
    const int mneed = (pl.csa && a->tok0 > 0) ? a->m : 0;
    const int64_t r0 = a->n_prev - mneed;
    CompressArgs &c = pl.ckv;
    c.n_streams = pl.csa ? 2 : 1;
    c.x[0] = ptr_at(a->kv_a, r0 * D, esz);
    c.x[1] = pl.csa ? ptr_at(a->kv_b, r0 * D, esz) : c.x[0];
    c.gate[0] = (const float *)ptr_at(a->gate_a, r0 * a->G, 4);
    c.gate[1] = pl.csa ? (const float *)ptr_at(a->gate_b, r0 * a->G, 4) : c.gate[0];
    c.bias[0] = a->bias_a;
    c.bias[1] = pl.csa ? a->bias_b : a->bias_a;
    c.bf16_in = a->in_t == V4A_BF16;
    c.D = D;
    c.G = a->G;
    c.m = a->m;
    c.tok0 = a->tok0 - mneed;
    c.n_tok = mneed + a->C;
    c.first_entry = pl.first;
    c.n_entries = pl.n_new;
    c.rope = a->apply_rope != 0;
    c.theta = a->rope_theta;
    c.kv = a->kv;
    c.b0 = a->slot;
    c.n_seq = 1;
    if ((st = compress_check(c, a->norm_w)) != V4A_OK) return st;
    if ((int64_t)(a->slot + 1) * a->kv->cap < 0) return fail(V4A_EINVAL, "v4a_prefill_chunk: slot");
    pl.kv = *a->kv;
    {
        const int64_t base = (int64_t)a->slot * a->kv->cap;
        const int Dn = D - a->kv->R;
        if (a->kv->fmt == V4A_KV_FP8_BF16) {
            pl.kv.nope = (char *)a->kv->nope + base * Dn;
            pl.kv.rope = (char *)a->kv->rope + base * a->kv->R * 2;
            pl.kv.scale = a->kv->scale + base;
        } else {
            pl.kv.nope = (char *)a->kv->nope + base * D * 4;
        }
    }
    AttnArgs probe{};
    probe.kv = &pl.kv;
    probe.q_bf16 = a->q_t == V4A_BF16;
    probe.win_bf16 = a->in_t == V4A_BF16;
    probe.H = a->H;
    probe.D = D;
    probe.R = a->kv->R;
    const int64_t ent_max = pl.csa ? a->k : pl.n_total;
    if (!attn_uses_mfma(probe) && ent_max + a->W > 8192 + 2048)
        return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: this format/shape uses the fp32 kernel, limited to %d keys",
                    8192 + 2048);
    if (a->q_norm_w && (!attn_uses_mfma(probe) || !aligned(a->q_norm_w, 16)))
        return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: q_norm_w needs the MFMA attention shapes and 16-byte alignment");
    pl.ws_total = 0;
    if (pl.csa) {
        if (!a->kv_b) return fail(V4A_EINVAL, "v4a_prefill_chunk: kv_b is required for CSA");
        if ((st = check_idx(a->keys, "keys")) != V4A_OK) return st;
        if (a->k < 1 || a->k > 2048) return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: k=%d not in [1, 2048]", a->k);
        const int d = a->keys->d;
        CompressArgs &ci = pl.cidx;
        ci.n_streams = 2;
        ci.x[0] = ptr_at(a->idx_a, r0 * d, esz);
        ci.x[1] = ptr_at(a->idx_b, r0 * d, esz);
        ci.gate[0] = (const float *)ptr_at(a->idx_gate_a, r0 * a->idx_G, 4);
        ci.gate[1] = (const float *)ptr_at(a->idx_gate_b, r0 * a->idx_G, 4);
        ci.bias[0] = a->idx_bias_a;
        ci.bias[1] = a->idx_bias_b;
        ci.bf16_in = c.bf16_in;
        ci.D = d;
        ci.G = a->idx_G;
        ci.m = a->m;
        ci.tok0 = c.tok0;
        ci.n_tok = c.n_tok;
        ci.first_entry = pl.first;
        ci.n_entries = pl.n_new;
        ci.idx = a->keys;
        ci.b0 = a->slot;
        ci.n_seq = 1;
        if ((st = compress_check(ci, a->idx_norm_w)) != V4A_OK) return st;
        pl.keys = *a->keys;
        const int64_t base = (int64_t)a->slot * a->keys->cap;
        if (a->keys->fmt == V4A_IDX_MXFP4) {
            pl.keys.codes = (char *)a->keys->codes + base * (d / 2);
            pl.keys.scales = a->keys->scales + base * (d / 32);
        } else {
            pl.keys.codes = (char *)a->keys->codes + base * d * 4;
        }
        const int64_t n_ent1 = pl.n_total;
        const int64_t pos0 = a->tok0;
        if ((st = check_indexer_args(&pl.keys, &n_ent1, a->m, a->q_idx, a->w, 1, a->C > 0 ? a->C : 1, a->H_I, &pos0)) != V4A_OK)
            return st;
        if (pl.n_total > (int64_t)1024 * kSelSlice)
            return fail(V4A_EUNSUPPORTED, "v4a_prefill_chunk: more than %d entries", 1024 * kSelSlice);
        memset(&pl.qp, 0, sizeof pl.qp);
        pl.qp.mode = 1;
        pl.qp.Q = a->C;
        pl.qp.m = a->m;
        pl.qp.pos[0] = a->tok0;
        pl.qp.n_ent[0] = pl.n_total;
        pl.idx_bytes = round_up((size_t)a->C * a->k * 4, 256);
        pl.topk_bytes = topk_layout(1, a->C, pl.n_total, a->k).total;
        pl.ws_total = pl.idx_bytes + pl.topk_bytes;
    }
    return V4A_OK;
}

}  // namespace v4a

extern "C" {

size_t v4a_prefill_workspace(v4a_layer kind, const v4a_prefill_args *args) {
    PrefillPlan pl;
    if (prefill_plan(kind, args, pl) != V4A_OK) return 0;
    return pl.ws_total;
}

v4a_status v4a_prefill_chunk(v4a_layer kind, const v4a_prefill_args *a, void *ws, size_t ws_bytes, void *stream) {
    PrefillPlan pl;
    v4a_status st = prefill_plan(kind, a, pl);
    if (st != V4A_OK) return st;
    if (pl.ws_total > 0 && (!ws || ws_bytes < pl.ws_total || !aligned(ws, 256)))
        return fail(V4A_EWORKSPACE, "v4a_prefill_chunk: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                    pl.ws_total, ws_bytes);
    g_err.clear();
    if (a->C == 0) return V4A_OK;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_compress(pl.ckv, s);
    if (e != hipSuccess) return hip_status(e, "v4a_prefill_chunk: compress");
    int32_t *sel = nullptr;
    if (pl.csa) {
        if ((e = launch_compress(pl.cidx, s)) != hipSuccess) return hip_status(e, "v4a_prefill_chunk: compress keys");
        sel = (int32_t *)ws;
        st = indexer_topk_launch(&pl.keys, pl.qp, pl.n_total, a->q_idx, a->w, 1, a->C, a->H_I, a->k, sel,
                                 (char *)ws + pl.idx_bytes, s, true, a->score_bf16 != 0);
        if (st != V4A_OK) return st;
    }
    AttnArgs at{};
    at.q = a->q;
    at.q_bf16 = a->q_t == V4A_BF16;
    at.B = a->C;
    at.H = a->H;
    at.D = pl.kv.D;
    at.R = pl.kv.R;
    at.kv = &pl.kv;
    at.kv_bstride = 0;
    at.topk = sel;
    at.k = pl.csa ? a->k : 0;
    at.win = a->kv_a;
    at.win_bf16 = a->in_t == V4A_BF16;
    at.W = a->W;
    at.sink = a->sink;
    at.scale = a->softmax_scale;
    at.rope_inv = a->out_rope_inverse != 0;
    at.q_norm_w = a->q_norm_w;
    at.theta = a->rope_theta;
    at.out = a->out;
    at.out_bf16 = a->out_t == V4A_BF16;
    at.partial = nullptr;
    at.target_splits = 1;
    at.split_cap = 1;
    SeqInfo sq;
    memset(&sq, 0, sizeof sq);
    sq.mode = 1;
    sq.tok0 = a->tok0;
    sq.n_prev = a->n_prev;
    sq.W = a->W;
    sq.m = a->m;
    sq.fixed_ent = pl.csa ? a->k : 0;
    sq.n_total = pl.n_total;
    return hip_status(launch_attention(at, sq, s), "v4a_prefill_chunk: attention");
}

}  // extern "C"

// ----------------------------------------------------------- fused CSA decode step ----
namespace v4a {

struct StepPlan {
    CompressArgs rec, key;
    int64_t entry[kMaxSeq];
    QueryPos qp;
    int64_t n_max;
    AttnArgs at;
    SeqInfo sq;
    v4a_kv kv;
    int Q;
    size_t sel_bytes, topk_bytes, attn_bytes, total;
};

// The queries of a decode step with Q new tokens per sequence (the newest at q_pos[b]): query
// b*Q + j is the token at t_j = q_pos[b] - Q + 1 + j.  Fills their positions (qpos), window
// lengths (wl: win_len[b], and for Q > 1 at most t_j + 1), the window rows of the plain layout
// (the buffer's W + Q - 1 rows per sequence hold the tokens ending at q_pos[b], oldest first)
// and the entry each sequence's tokens complete (at most one, since Q <= m).
static v4a_status step_queries(int B, int Q, int m, int W, const int64_t *q_pos, const int32_t *win_len, bool ring,
                               int64_t *qpos, int32_t *wl, int64_t *entry, SeqInfo &sq, const char *name) {
    if (W > 0 && !win_len) return fail(V4A_EINVAL, "%s: win_len is required", name);
    for (int b = 0; b < B; b++) {
        const int64_t t = q_pos[b];
        if (t < Q - 1) return fail(V4A_EINVAL, "%s: q_pos[%d]=%lld is before the step's first token", name, b, (long long)t);
        const int wlb = W > 0 ? win_len[b] : 0;
        if (wlb < 0 || wlb > W) return fail(V4A_EINVAL, "%s: win_len[%d]=%d not in [0, W]", name, b, wlb);
        const int64_t p_lo = std::max<int64_t>(0, t - wlb - Q + 2);  // the plain buffer's row 0
        entry[b] = -1;
        for (int j = 0; j < Q; j++) {
            const int64_t tj = t - Q + 1 + j;
            const int qi = b * Q + j;
            const int w = Q > 1 ? (int)std::min<int64_t>(wlb, tj + 1) : wlb;
            qpos[qi] = tj;
            wl[qi] = w;
            sq.win_off[qi] = (Q > 1 && !ring) ? (int32_t)(tj - w + 1 - p_lo) : 0;
            if ((tj + 1) % m == 0) entry[b] = (tj + 1) / m - 1;
        }
    }
    sq.qps = Q;
    sq.win_stride = Q > 1 ? W + Q - 1 : 0;
    return V4A_OK;
}

static v4a_status step_plan(const v4a_decode_step_args *a, StepPlan &pl) {
    if (!a) return fail(V4A_EINVAL, "v4a_decode_step_csa: args is NULL");
    pl = StepPlan{};
    if (a->B < 1 || a->B > kMaxSeq) return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: B=%d not in [1, %d]", a->B, kMaxSeq);
    if (!a->q_pos || !a->n_entries) return fail(V4A_EINVAL, "v4a_decode_step_csa: q_pos and n_entries are required");
    v4a_status st;
    if ((st = check_kv(a->kv, "kv")) != V4A_OK) return st;
    if ((st = check_idx(a->keys, "keys")) != V4A_OK) return st;
    if (a->in_t != V4A_F32 && a->in_t != V4A_BF16) return fail(V4A_EINVAL, "v4a_decode_step_csa: in_t");
    const int D = a->kv->D, d = a->keys->d, m = a->m;
    if (!((D == 512 && d == 128) || (D == 128 && d == 32)))
        return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: needs D=512 with d=128 or D=128 with d=32");
    const int Q = a->Q > 0 ? a->Q : 1;
    if (Q > 4 || Q > m || a->B * Q > kMaxSeq)
        return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: Q=%d needs Q <= 4, Q <= m and B*Q <= %d", Q, kMaxSeq);
    pl.Q = Q;
    // compressor arguments, checked as one entry at rows [0, 2m) (the per-sequence entries and
    // row origins are set at launch)
    auto fill = [&](CompressArgs &c, const void *xa, const void *xb, const float *ga, const float *gb,
                     const float *ba, const float *bb, int Dd, int G) {
        c.x[0] = xa; c.x[1] = xb; c.gate[0] = ga; c.gate[1] = gb; c.bias[0] = ba; c.bias[1] = bb;
        c.n_streams = 2; c.bf16_in = a->in_t == V4A_BF16; c.D = Dd; c.G = G; c.m = m;
        c.tok0 = 0; c.n_tok = 2 * m + (a->ring ? Q - 1 : 0); c.first_entry = 1; c.n_entries = 1;
        c.theta = a->rope_theta; c.b0 = 0; c.n_seq = a->B;
    };
    fill(pl.rec, a->kv_a, a->kv_b, a->gate_a, a->gate_b, a->bias_a, a->bias_b, D, a->G);
    pl.rec.ring = a->ring != 0;
    pl.rec.rope = a->apply_rope != 0;
    pl.rec.kv = a->kv;
    if ((st = compress_check(pl.rec, a->norm_w)) != V4A_OK) return st;
    if (a->G == 1 && m >= 64)  // the records are compressed one wavefront per entry here
        return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: m=%d with one gate per token", m);
    fill(pl.key, a->idx_a, a->idx_b, a->idx_gate_a, a->idx_gate_b, a->idx_bias_a, a->idx_bias_b, d, a->idx_G);
    pl.key.ring = a->ring != 0;
    pl.key.idx = a->keys;
    if ((st = compress_check(pl.key, a->idx_norm_w)) != V4A_OK) return st;
    memset(&pl.sq, 0, sizeof pl.sq);
    int64_t qpos[kMaxSeq];
    int32_t wl[kMaxSeq];
    if ((st = step_queries(a->B, Q, m, a->W, a->q_pos, a->win_len, a->ring != 0, qpos, wl, pl.entry, pl.sq,
                           "v4a_decode_step_csa")) != V4A_OK)
        return st;
    for (int b = 0; b < a->B; b++) {
        const int64_t i = pl.entry[b];
        if (i >= a->n_entries[b])
            return fail(V4A_EINVAL, "v4a_decode_step_csa: n_entries[%d] does not include the entry this step completes", b);
        if (i >= a->kv->cap || i >= a->keys->cap)
            return fail(V4A_EINVAL, "v4a_decode_step_csa: entry %lld of sequence %d exceeds the cache", (long long)i, b);
    }
    // selection
    if ((st = check_indexer_args(a->keys, a->n_entries, m, a->q_idx, a->w, a->B, Q, a->H_I, qpos)) != V4A_OK)
        return st;
    if (a->k < 1 || a->k > 2048) return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: k=%d not in [1, 2048]", a->k);
    if ((st = fill_query_pos(pl.qp, a->B, Q, m, a->n_entries, qpos, a->keys->cap, &pl.n_max)) != V4A_OK) return st;
    if (pl.n_max > (int64_t)1024 * kSelSlice) return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: too many entries");
    // attention
    AttnArgs &at = pl.at;
    const int BQ = a->B * Q;
    at.q = a->q;
    at.B = BQ;
    at.H = a->H;
    at.kv = a->kv;
    at.kv_bstride = a->kv->cap;
    at.k = a->k;
    at.win = a->win;
    at.W = a->W;
    at.sink = a->sink;
    at.scale = a->softmax_scale;
    at.rope_inv = a->out_rope_inverse != 0;
    at.theta = a->rope_theta;
    at.out = a->out;
    for (int qi = 0; qi < BQ; qi++) pl.sq.n_ent[qi] = a->k;
    size_t attn_need = 0;
    if ((st = decode_prepare(at, pl.sq, wl, qpos, a->q_t, a->win_t, a->out_t, &attn_need,
                             "v4a_decode_step_csa", a->no_split != 0)) != V4A_OK)
        return st;
    if (a->ring) {
        for (int qi = 0; qi < BQ; qi++)
            if (pl.sq.win_len[qi] > pl.sq.q_pos[qi] + 1)
                return fail(V4A_EINVAL, "v4a_decode_step_csa: win_len[%d] exceeds the tokens so far", qi / Q);
        pl.sq.ring = 1;
    }
    if (!attn_uses_mfma(at)) return fail(V4A_EUNSUPPORTED, "v4a_decode_step_csa: needs the MFMA attention shapes");
    if (a->q_norm_w && !aligned(a->q_norm_w, 16))
        return fail(V4A_EINVAL, "v4a_decode_step_csa: q_norm_w must be 16-byte aligned");
    pl.at.q_norm_w = a->q_norm_w;
    pl.sel_bytes = round_up((size_t)BQ * a->k * 4, 256);
    pl.topk_bytes = topk_layout(a->B, Q, pl.n_max, a->k).total;
    pl.attn_bytes = round_up(attn_need, 256);
    pl.total = pl.sel_bytes + pl.topk_bytes + pl.attn_bytes;
    return V4A_OK;
}

}  // namespace v4a

extern "C" {

size_t v4a_decode_step_workspace(const v4a_decode_step_args *args) {
    StepPlan pl;
    if (step_plan(args, pl) != V4A_OK) return 0;
    return pl.total;
}

}  // extern "C"

namespace v4a {

// The launches of one fused CSA decode step on a checked plan and a workspace of pl.total bytes.
static v4a_status decode_step_run(const v4a_decode_step_args *a, StepPlan &pl, void *ws, hipStream_t s) {
    v4a_status st;
    char *base = (char *)ws;
    int32_t *sel = (int32_t *)base;
    char *tws = base + pl.sel_bytes;
    const int Q = pl.Q, BQ = a->B * pl.Q;
    const TopkWs L = topk_layout(a->B, Q, pl.n_max, a->k);
    const size_t hist_bytes = (size_t)BQ * hist_copies(BQ) * kHistBins * 4;
    // MXFP4 keys of d = 128 from short gate-per-token blocks are compressed inside the scoring
    // kernel (its latency hidden behind the scan; one query per sequence); otherwise the
    // prologue compresses them
    const bool key_in_scoring = Q == 1 && a->keys->fmt == V4A_IDX_MXFP4 && a->keys->d == 128 &&
                                entry_two_phase(compress_params(pl.key));
    // the histograms: cleared here unless the caller vouches that the previous call left them
    // clear (the final selection's launch clears them for the next call)
    const size_t clear_bytes = a->ws_clean ? 0 : hist_bytes;
    hipError_t e = hipSuccess;
    if (!key_in_scoring)
        e = launch_decode_prologue(pl.key, 1, a->B, pl.entry, tws + L.hist, clear_bytes, s);
    else if (clear_bytes)
        e = launch_zero(tws + L.hist, clear_bytes, s);
    if (e != hipSuccess) return hip_status(e, "v4a_decode_step_csa: compress");
    st = indexer_topk_launch(a->keys, pl.qp, pl.n_max, a->q_idx, a->w, a->B, Q, a->H_I, a->k, sel, tws, s, false,
                             a->score_bf16 != 0, &pl.rec, key_in_scoring ? &pl.key : nullptr, true);
    if (st != V4A_OK) return st;
    pl.at.topk = sel;
    pl.at.partial = pl.attn_bytes > 0 ? (float *)(tws + pl.topk_bytes) : nullptr;
    return hip_status(launch_attention(pl.at, pl.sq, s), "v4a_decode_step_csa: attention");
}

// Scratch of the entry point that allocates nothing: one array per device (each device that
// loads the library holds its own copy until the process ends).  Host code must not pass the
// array's name to a kernel (in host code it is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kNoAllocScratchBytes = V4A_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array; checks that `stream` belongs to that
// device.
static v4a_status scratch_address(hipStream_t s, void **out, const char *name) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, name);
    if (dev < 0 || dev >= kMaxDevices) return fail(V4A_EUNSUPPORTED, "%s: device %d", name, dev);
    if (s) {
        hipDevice_t sdev = -1;
        e = hipStreamGetDevice(s, &sdev);
        if (e != hipSuccess) return hip_status(e, name);
        if ((int)sdev != dev)
            return fail(V4A_EINVAL, "%s: the stream belongs to device %d, the current device is %d", name, (int)sdev, dev);
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, name);
        if (!p || !aligned(p, 256)) return fail(V4A_EHIP, "%s: scratch address not 256-byte aligned", name);
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return V4A_OK;
}

}  // namespace v4a

extern "C" {

v4a_status v4a_decode_step_csa(const v4a_decode_step_args *a, void *ws, size_t ws_bytes, void *stream) {
    StepPlan pl;
    v4a_status st = step_plan(a, pl);
    if (st != V4A_OK) return st;
    if (!ws || ws_bytes < pl.total || !aligned(ws, 256))
        return fail(V4A_EWORKSPACE, "v4a_decode_step_csa: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                    pl.total, ws_bytes);
    g_err.clear();
    return decode_step_run(a, pl, ws, (hipStream_t)stream);
}

v4a_status v4a_decode_step_csa_noalloc(const v4a_decode_step_args *args, void *stream) {
    const char *name = "v4a_decode_step_csa_noalloc";
    if (!args) return fail(V4A_EINVAL, "%s: args is NULL", name);
    // the scratch keeps whatever the last call on this device left: the histograms are always
    // cleared by this call (a fill kernel, no runtime memset)
    v4a_decode_step_args a = *args;
    a.ws_clean = 0;
    StepPlan pl;
    v4a_status st = step_plan(&a, pl);
    if (st != V4A_OK) return st;
    if (pl.total > kNoAllocScratchBytes)
        return fail(V4A_EWORKSPACE, "%s: these arguments need %zu bytes of scratch, more than the %zu the library holds",
                    name, pl.total, (size_t)kNoAllocScratchBytes);
    hipStream_t s = (hipStream_t)stream;
    void *ws = nullptr;
    if ((st = scratch_address(s, &ws, name)) != V4A_OK) return st;
    g_err.clear();
    return decode_step_run(&a, pl, ws, s);
}

}  // extern "C"

extern "C" {

v4a_status v4a_trace_begin(int32_t capacity) {
    using namespace v4a;
    if (capacity < 1 || capacity > (1 << 18)) return fail(V4A_EINVAL, "v4a_trace_begin: capacity=%d", capacity);
    if (g_trace.armed) return fail(V4A_EINVAL, "v4a_trace_begin: a trace is already armed");
    while ((int)g_trace.start.size() < capacity) {
        hipEvent_t a, b;
        if (hipEventCreate(&a) != hipSuccess) return fail(V4A_EHIP, "v4a_trace_begin: hipEventCreate failed");
        if (hipEventCreate(&b) != hipSuccess) {
            (void)hipEventDestroy(a);
            return fail(V4A_EHIP, "v4a_trace_begin: hipEventCreate failed");
        }
        g_trace.start.push_back(a);
        g_trace.stop.push_back(b);
        g_trace.kernel.push_back(nullptr);
    }
    g_trace.n = 0;
    g_trace.armed = true;
    return V4A_OK;
}

int32_t v4a_trace_end(void) {
    v4a::g_trace.armed = false;
    return v4a::g_trace.n;
}

v4a_status v4a_trace_kernel(int32_t i, const char **kernel, float *ms) {
    using namespace v4a;
    if (g_trace.armed) return fail(V4A_EINVAL, "v4a_trace_kernel: the trace is still armed");
    if (i < 0 || i >= g_trace.n) return fail(V4A_EINVAL, "v4a_trace_kernel: kernel %d of %d", i, g_trace.n);
    if (kernel) *kernel = g_trace.kernel[i];
    if (ms) {
        hipError_t e = hipEventElapsedTime(ms, g_trace.start[i], g_trace.stop[i]);
        if (e != hipSuccess) return hip_status(e, "v4a_trace_kernel");
    }
    return V4A_OK;
}

}  // extern "C"

// ------------------------------------------------------------ fused HCA decode step --------
namespace v4a {

struct StepHcaPlan {
    CompressArgs rec;
    int64_t entry[kMaxSeq];
    AttnArgs at;
    SeqInfo sq;
    size_t attn_bytes;
};

static v4a_status step_hca_plan(const v4a_decode_step_hca_args *a, StepHcaPlan &pl) {
    const char *name = "v4a_decode_step_hca";
    if (!a) return fail(V4A_EINVAL, "%s: args is NULL", name);
    pl = StepHcaPlan{};
    if (a->B < 1 || a->B > kMaxSeq) return fail(V4A_EUNSUPPORTED, "%s: B=%d not in [1, %d]", name, a->B, kMaxSeq);
    if (!a->q_pos || !a->n_entries) return fail(V4A_EINVAL, "%s: q_pos and n_entries are required", name);
    v4a_status st;
    if ((st = check_kv(a->kv, "kv")) != V4A_OK) return st;
    if (a->in_t != V4A_F32 && a->in_t != V4A_BF16) return fail(V4A_EINVAL, "%s: in_t", name);
    const int D = a->kv->D, m = a->m;
    const int Q = a->Q > 0 ? a->Q : 1;
    if (m < 1 || Q > 4 || Q > m || a->B * Q > kMaxSeq)
        return fail(V4A_EUNSUPPORTED, "%s: Q=%d needs Q <= 4, Q <= m and B*Q <= %d", name, Q, kMaxSeq);
    // compressor arguments, checked as one entry at rows [0, m) (entries and row origins are set
    // per sequence at launch)
    CompressArgs &c = pl.rec;
    c.x[0] = a->kv_a; c.gate[0] = a->gate_a; c.bias[0] = a->bias_a;
    c.n_streams = 1; c.bf16_in = a->in_t == V4A_BF16; c.D = D; c.G = a->G; c.m = m;
    c.tok0 = 0; c.n_tok = m + (a->ring ? Q - 1 : 0); c.first_entry = 0; c.n_entries = 1;
    c.rope = a->apply_rope != 0; c.theta = a->rope_theta; c.kv = a->kv; c.b0 = 0; c.n_seq = a->B;
    c.ring = a->ring != 0;
    if ((st = compress_check(c, a->norm_w)) != V4A_OK) return st;
    memset(&pl.sq, 0, sizeof pl.sq);
    int64_t qpos[kMaxSeq];
    int32_t wl[kMaxSeq];
    if ((st = step_queries(a->B, Q, m, a->W, a->q_pos, a->win_len, a->ring != 0, qpos, wl, pl.entry, pl.sq, name)) !=
        V4A_OK)
        return st;
    for (int b = 0; b < a->B; b++) {
        if (a->n_entries[b] < 0 || a->n_entries[b] > a->kv->cap)
            return fail(V4A_EINVAL, "%s: n_entries[%d] not in [0, cap]", name, b);
        if (pl.entry[b] >= a->n_entries[b])
            return fail(V4A_EINVAL, "%s: n_entries[%d] does not include the entry this step completes", name, b);
        for (int j = 0; j < Q; j++) {
            int64_t vis = (qpos[b * Q + j] + 1) / m;
            if (vis > a->n_entries[b]) vis = a->n_entries[b];
            if (vis > (1 << 30)) return fail(V4A_EUNSUPPORTED, "%s: too many entries", name);
            pl.sq.n_ent[b * Q + j] = (int32_t)vis;
        }
    }
    const int BQ = a->B * Q;
    AttnArgs &at = pl.at;
    at.q = a->q;
    at.B = BQ;
    at.H = a->H;
    at.kv = a->kv;
    at.kv_bstride = a->kv->cap;
    at.win = a->win;
    at.W = a->W;
    at.sink = a->sink;
    at.scale = a->softmax_scale;
    at.rope_inv = a->out_rope_inverse != 0;
    at.theta = a->rope_theta;
    at.out = a->out;
    size_t need = 0;
    if ((st = decode_prepare(at, pl.sq, wl, qpos, a->q_t, a->win_t, a->out_t, &need, name, a->no_split != 0)) != V4A_OK)
        return st;
    if (!attn_uses_mfma(at)) return fail(V4A_EUNSUPPORTED, "%s: needs the MFMA attention shapes", name);
    if (a->q_norm_w && !aligned(a->q_norm_w, 16)) return fail(V4A_EINVAL, "%s: q_norm_w must be 16-byte aligned", name);
    at.q_norm_w = a->q_norm_w;
    if (a->ring) {
        for (int qi = 0; qi < BQ; qi++)
            if (pl.sq.win_len[qi] > pl.sq.q_pos[qi] + 1)
                return fail(V4A_EINVAL, "%s: win_len[%d] exceeds the tokens so far", name, qi / Q);
        pl.sq.ring = 1;
    }
    pl.attn_bytes = round_up(need, 256);
    return V4A_OK;
}

}  // namespace v4a

extern "C" {

size_t v4a_decode_step_hca_workspace(const v4a_decode_step_hca_args *args) {
    v4a::StepHcaPlan pl;
    if (v4a::step_hca_plan(args, pl) != V4A_OK) return 0;
    return pl.attn_bytes;
}

v4a_status v4a_decode_step_hca(const v4a_decode_step_hca_args *a, void *ws, size_t ws_bytes, void *stream) {
    using namespace v4a;
    StepHcaPlan pl;
    v4a_status st = step_hca_plan(a, pl);
    if (st != V4A_OK) return st;
    if (pl.attn_bytes > 0 && (!ws || ws_bytes < pl.attn_bytes || !aligned(ws, 256)))
        return fail(V4A_EWORKSPACE, "v4a_decode_step_hca: workspace needs %zu bytes, 256-byte aligned (got %zu)",
                    pl.attn_bytes, ws_bytes);
    g_err.clear();
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = launch_decode_prologue(pl.rec, 0, a->B, pl.entry, nullptr, 0, s);
    if (e != hipSuccess) return hip_status(e, "v4a_decode_step_hca: compress");
    pl.at.partial = pl.attn_bytes > 0 ? (float *)ws : nullptr;
    return hip_status(launch_attention(pl.at, pl.sq, s), "v4a_decode_step_hca: attention");
}

}  // extern "C"
