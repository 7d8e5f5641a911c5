// compress.hip -- a1/a2: the KV compressors.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2: CSA turns every 4
// tokens into one entry by merging two independent KV sequences with softmax-normalised
// gate weights, adjacent compressed blocks sharing indices; HCA turns every 128 tokens into
// one entry with no overlap.  "DeepSeek V4 preview and technical report" (chooseai.net),
// section 1: the merge is a softmax with positional bias.
//
// Entry i of the CSA compressor merges A-block i with B-block i-1 (entry 0: A-block only);
// HCA entry i merges its own block of one stream.  Per gate channel the weights are the
// softmax of (gate logit + positional bias) over the candidate tokens.  The merged entry is
// rotated on its last R dims at position m*i (interleaved pairs) and encoded in the output
// format (entry record or MXFP4 indexer key) by the same row encoders as the quantisers.
//
// One wavefront per entry; each lane owns VPT = D/64 consecutive dims (D = 32 uses one dim
// per lane on half the wavefront).  With one gate per token (G = 1) the candidate weights
// are computed once per wavefront (one candidate per lane) and broadcast through LDS; with
// a gate per dim (G = D) each lane runs an online softmax for its own dims.  All row
// reads are 64-lane contiguous; the work is HBM-bound.
#include <algorithm>

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

// Entry i of sequence seq, computed by one whole wavefront; row 0 of the sequence's streams
// is position tok0 (its streams and gates start n_tok rows further per sequence); wsh is the
// wavefront's scratch for the candidate weights.
template <int VPT>
__device__ __forceinline__ void compress_entry(const CompressParams &P, float *wsh, int64_t seq, int64_t i,
                                               int64_t tok0) {
    const int lane = threadIdx.x & 63;
    const int64_t x_off = seq * P.n_tok * P.D, g_off = seq * P.n_tok * P.G;
    const int m = P.m, D = P.D;
    const int d0 = lane * VPT;
    const bool active = d0 < D;
    // candidate c: stream s = c / m (0: own block i, 1: B-block i-1), position j = c % m
    const int n_cand = (P.n_streams == 2 && i >= 1) ? 2 * m : m;

    float acc[VPT];
#pragma unroll
    for (int v = 0; v < VPT; v++) acc[v] = 0.0f;

    if (P.G == 1) {
        // candidate rows are loaded in batches of kRowBatch; the first batch is issued before the
        // gate logits so the two memory round trips overlap
        constexpr int kRowBatch = 8;
        float xb[kRowBatch][VPT];
        auto load_batch = [&](int c0) {
#pragma unroll
            for (int u = 0; u < kRowBatch; u++) {
                const int c = min(c0 + u, n_cand - 1);
                const int s = c / m, j = c % m;
                const int64_t r = (s == 0 ? m * i : m * (i - 1)) + j - tok0;
                load_row<VPT>(s == 0 ? P.x0 : P.x1, P.bf16_in, r, D, d0, active, xb[u], x_off);
            }
        };
        load_batch(0);
        // weights once per wavefront: lane c holds candidate c (and c + 64, ...)
        float zmax = -INFINITY;
        for (int c = lane; c < n_cand; c += 64) {
            int s = c / m, j = c % m;
            int64_t r = (s == 0 ? m * i : m * (i - 1)) + j - tok0;
            float z = (s == 0 ? P.g0 : P.g1)[g_off + r] + (s == 0 ? P.b0 : P.b1)[j];
            wsh[c] = z;
            zmax = fmaxf(zmax, z);
        }
        zmax = wave_max(zmax);
        float den = 0.0f;
        for (int c = lane; c < n_cand; c += 64) {
            float ex = expf(wsh[c] - zmax);
            wsh[c] = ex;
            den += ex;
        }
        den = wave_sum(den);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        for (int c0 = 0; c0 < n_cand; c0 += kRowBatch) {
            float cur[kRowBatch][VPT];
#pragma unroll
            for (int u = 0; u < kRowBatch; u++)
#pragma unroll
                for (int v = 0; v < VPT; v++) cur[u][v] = xb[u][v];
            if (c0 + kRowBatch < n_cand) load_batch(c0 + kRowBatch);  // next batch in flight
#pragma unroll
            for (int u = 0; u < kRowBatch; u++) {
                if (c0 + u < n_cand) {
                    const float wgt = wsh[c0 + u];
#pragma unroll
                    for (int v = 0; v < VPT; v++) acc[v] = fmaf(wgt, cur[u][v], acc[v]);
                }
            }
        }
#pragma unroll
        for (int v = 0; v < VPT; v++) acc[v] = acc[v] / den;
    } else {
        // per-channel gates: online softmax over the candidates for each of this lane's dims
        float mx[VPT], l[VPT];
#pragma unroll
        for (int v = 0; v < VPT; v++) { mx[v] = -INFINITY; l[v] = 0.0f; }
        for (int c = 0; c < n_cand; c++) {
            int s = c / m, j = c % m;
            int64_t r = (s == 0 ? m * i : m * (i - 1)) + j - tok0;
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

    // partial RoPE on the last R dims at position m*i (interleaved pairs); lane j < R/2
    // evaluates pair j's cos/sin and the owning lanes read them across the wavefront
    if (P.rope) {
        const int rs = D - P.R, npairs = P.R / 2;
        RopeLanes rl;
        rl.eval(P.rt, npairs, (double)(m * i));
        if constexpr (VPT >= 2) {
#pragma unroll
            for (int v = 0; v < VPT; v += 2) {
                const int j = min(max((d0 - rs + v) / 2, 0), npairs - 1);
                const float2 cs = rl.get(j);
                if (active && d0 >= rs) {
                    const float x = acc[v], y = acc[v + 1];
                    acc[v] = x * cs.x - y * cs.y;
                    acc[v + 1] = x * cs.y + y * cs.x;
                }
            }
        } else {
            const float partner = __shfl_xor(acc[0], 1);
            const int j = min(max((d0 - rs) / 2, 0), npairs - 1);
            const float2 cs = rl.get(j);
            if (active && d0 >= rs) {
                const bool even = ((d0 - rs) & 1) == 0;
                const float x = even ? acc[0] : partner, y = even ? partner : acc[0];
                acc[0] = even ? (x * cs.x - y * cs.y) : (x * cs.y + y * cs.x);
            }
        }
    }

    const int64_t orow = P.out_row0 + seq * P.cap + i;
    if (P.to_idx)
        store_mxfp4<VPT>(acc, lane, active, D, P.idx, orow);
    else
        store_record<VPT>(acc, d0, active, D, P.R, P.kv, orow);
}

template <int VPT>
__global__ void __launch_bounds__(256) compress_kernel(CompressParams P) {
    __shared__ float wsh[4][kMaxCand];
    const int wv = threadIdx.x >> 6;
    const int64_t e = (int64_t)blockIdx.x * 4 + wv;
    if (e >= P.n_entries) return;  // the whole wavefront leaves together
    compress_entry<VPT>(P, wsh[wv], blockIdx.y, P.first_entry + e, P.tok0);
}

// Decode-step prologue, one launch: row y < B compresses the entry record of sequence y, row
// B <= y < 2B its indexer key (each where the sequence's newest token completes a block:
// entry[seq] >= 0, the sequence's 2m stream rows starting at the block before it), and row 2B
// clears the selection's histogram region.
struct PrologueParams {
    CompressParams rec, key;
    int B;
    int64_t entry[kMaxSeq];
    uint4 *zero;
    size_t zero_n16;
};

template <int VR, int VK>
__global__ void __launch_bounds__(256) decode_prologue_kernel(PrologueParams P) {
    __shared__ float wsh[kMaxCand];
    const int y = blockIdx.y;
    if (y == 2 * P.B) {
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < P.zero_n16; i += (size_t)gridDim.x * blockDim.x)
            P.zero[i] = make_uint4(0, 0, 0, 0);
        return;
    }
    if (blockIdx.x != 0 || threadIdx.x >= 64) return;  // one wavefront per entry
    const int seq = y < P.B ? y : y - P.B;
    const int64_t i = P.entry[seq];
    if (i < 0) return;
    if (y < P.B)
        compress_entry<VR>(P.rec, wsh, seq, i, (int64_t)P.rec.m * (i - 1));
    else
        compress_entry<VK>(P.key, wsh, seq, i, (int64_t)P.key.m * (i - 1));
}

static CompressParams compress_params(const CompressArgs &a) {
    CompressParams P;
    P.x0 = a.x[0];
    P.x1 = a.x[1];
    P.g0 = a.gate[0];
    P.g1 = a.gate[1];
    P.b0 = a.bias[0];
    P.b1 = a.bias[1];
    P.n_streams = a.n_streams;
    P.D = a.D;
    P.G = a.G;
    P.m = a.m;
    P.R = a.R;
    P.bf16_in = a.bf16_in;
    P.rope = a.rope;
    P.tok0 = a.tok0;
    P.first_entry = a.first_entry;
    P.n_entries = a.n_entries;
    if (a.rope) fill_rope_table(P.rt, a.R, a.theta);
    P.to_idx = a.idx != nullptr;
    if (a.kv) P.kv = *a.kv; else P.kv = v4a_kv{};
    if (a.idx) P.idx = *a.idx; else P.idx = v4a_idx{};
    P.cap = a.idx ? a.idx->cap : a.kv->cap;
    P.out_row0 = (int64_t)a.b0 * P.cap;
    P.n_tok = a.n_tok;
    return P;
}

hipError_t launch_compress(const CompressArgs &a, hipStream_t s) {
    if (a.n_entries == 0 || a.n_seq == 0) return hipSuccess;
    const CompressParams P = compress_params(a);
    dim3 grid((unsigned)((a.n_entries + 3) / 4), (unsigned)a.n_seq), block(256);
    switch (a.D) {
        case 32: case 64: hipLaunchKernelGGL(compress_kernel<1>, grid, block, 0, s, P); break;
        case 128: hipLaunchKernelGGL(compress_kernel<2>, grid, block, 0, s, P); break;
        case 256: hipLaunchKernelGGL(compress_kernel<4>, grid, block, 0, s, P); break;
        default: hipLaunchKernelGGL(compress_kernel<8>, grid, block, 0, s, P); break;
    }
    return hipGetLastError();
}

}  // namespace v4a

namespace v4a {

hipError_t launch_decode_prologue(const CompressArgs &rec, const CompressArgs &key, int B, const int64_t *entry,
                                  void *zero, size_t zero_bytes, hipStream_t s) {
    PrologueParams P;
    P.rec = compress_params(rec);
    P.key = compress_params(key);
    P.B = B;
    for (int b = 0; b < kMaxSeq; b++) P.entry[b] = b < B ? entry[b] : -1;
    P.zero = (uint4 *)zero;
    P.zero_n16 = zero_bytes / 16;
    const unsigned zx = (unsigned)std::min<size_t>((P.zero_n16 + 255) / 256, 1024);
    dim3 grid(zx > 0 ? zx : 1, (unsigned)(2 * B + 1));
    if (rec.D == 512 && key.D == 128)
        hipLaunchKernelGGL((decode_prologue_kernel<8, 2>), grid, dim3(256), 0, s, P);
    else if (rec.D == 128 && key.D == 32)
        hipLaunchKernelGGL((decode_prologue_kernel<2, 1>), grid, dim3(256), 0, s, P);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace v4a
