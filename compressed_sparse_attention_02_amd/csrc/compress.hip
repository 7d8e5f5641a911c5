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

#include "compress.hpp"

namespace v4a {

// 2 * kEntryWaves entries per workgroup, two consecutive ones per wavefront, whose RoPE cos/sin
// (R/2 <= 32 pairs each) one pass of the wavefront's 64 lanes evaluates; or, for the long
// gate-per-token blocks (HCA), one entry per workgroup shared by its kEntryWaves wavefronts.
// PK: BF16 streams read with one vector load per lane and row (rows kept as packed pairs).
template <int VPT, bool PK>
__global__ void __launch_bounds__(64 * kEntryWaves) compress_kernel(CompressParams P) {
    __shared__ float wsh[kEntryWaves][kMaxCand];
    __shared__ float red[kEntryWaves * 64 * VPT];
    if (entry_uses_workgroup(P)) {
        const int64_t e = blockIdx.x;
        if (e >= P.n_entries) return;  // the whole workgroup leaves together
        compress_entry_wg<VPT, PK>(P, &wsh[0][0], red, blockIdx.y, P.first_entry + e, P.tok0);
        return;
    }
    const int wv = threadIdx.x >> 6;
    const int64_t e = ((int64_t)blockIdx.x * kEntryWaves + wv) * 2;
    if (e >= P.n_entries) return;  // the whole wavefront leaves together
    const int64_t i0 = P.first_entry + e;
    const bool two = e + 1 < P.n_entries;  // uniform
    if constexpr (VPT % 2 == 0) {
        if (entry_two_phase(P) && P.D == 64 * VPT) {
            // both entries' rows, gate logits and biases requested before either is merged
            KeyPrefetch<VPT> ka, kb;
            key_prefetch<VPT>(P, blockIdx.y, i0, P.tok0, ka);
            if (two) key_prefetch<VPT>(P, blockIdx.y, i0 + 1, P.tok0, kb);
            RopeLanes rl;
            const bool shared = P.rope && P.R / 2 <= 32;
            if (shared) rl.eval2(P.rt, P.R / 2, (double)(P.m * i0), (double)(P.m * (two ? i0 + 1 : i0)));
            prefetched_entry_finish<VPT>(P, ka, blockIdx.y, i0, shared ? &rl : nullptr, 0);
            if (two) prefetched_entry_finish<VPT>(P, kb, blockIdx.y, i0 + 1, shared ? &rl : nullptr, 32);
            return;
        }
    }
    if (P.rope && P.R / 2 <= 32) {
        RopeLanes rl;
        rl.eval2(P.rt, P.R / 2, (double)(P.m * i0), (double)(P.m * (two ? i0 + 1 : i0)));
        compress_entry<VPT, PK>(P, wsh[wv], blockIdx.y, i0, P.tok0, &rl, 0);
        if (two) compress_entry<VPT, PK>(P, wsh[wv], blockIdx.y, i0 + 1, P.tok0, &rl, 32);
    } else {
        compress_entry<VPT, PK>(P, wsh[wv], blockIdx.y, i0, P.tok0);
        if (two) compress_entry<VPT, PK>(P, wsh[wv], blockIdx.y, i0 + 1, P.tok0);
    }
}

// Decode-step prologue, one launch: row y < B compresses one entry of sequence y (where the
// sequence's newest token completes a block: entry[seq] >= 0; the sequence's stream rows start
// blocks_before blocks before the entry's own block), and row B clears zero_n16 16-byte words.
// The CSA step compresses the indexer keys here (its entry records follow in the final
// selection's launch, since only attention reads them); the HCA step its entry records.
struct PrologueParams {
    CompressParams key;
    int blocks_before;
    int B;
    int64_t entry[kMaxSeq];
    uint4 *zero;
    size_t zero_n16;
};

template <int VK, bool PK>
__global__ void __launch_bounds__(64 * kEntryWaves) decode_prologue_kernel(PrologueParams P) {
    __shared__ float wsh[kEntryWaves * kMaxCand];
    __shared__ float red[kEntryWaves * 64 * VK];
    const int y = blockIdx.y;
    if (y == P.B) {
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < P.zero_n16; i += (size_t)gridDim.x * blockDim.x)
            P.zero[i] = make_uint4(0, 0, 0, 0);
        return;
    }
    if (blockIdx.x != 0) return;
    const int64_t i = P.entry[y];
    if (i < 0) return;  // the whole workgroup leaves together
    const int64_t tok0 = (int64_t)P.key.m * (i - P.blocks_before);
    if (entry_uses_workgroup(P.key)) {
        compress_entry_wg<VK, PK>(P.key, wsh, red, y, i, tok0);
        return;
    }
    if (threadIdx.x >= 64) return;  // one wavefront per entry
    compress_entry<VK, PK>(P.key, wsh, y, i, tok0);
}

CompressParams compress_params(const CompressArgs &a) {
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
    P.norm_w = a.norm_w;
    P.ring = a.ring;
    // one vector load per lane and row needs the streams aligned to the lane's VPT values
    const int vpt = a.D >= 64 ? a.D / 64 : 1;
    const uintptr_t need = (uintptr_t)std::min(16, vpt * (a.bf16_in ? 2 : 4));
    P.vec_in = ((uintptr_t)a.x[0] % need) == 0 && (a.n_streams < 2 || ((uintptr_t)a.x[1] % need) == 0);
    return P;
}

hipError_t launch_compress(const CompressArgs &a, hipStream_t s) {
    if (a.n_entries == 0 || a.n_seq == 0) return hipSuccess;
    const CompressParams P = compress_params(a);
    const int64_t per_wg = entry_uses_workgroup(P) ? 1 : 2 * kEntryWaves;
    dim3 grid((unsigned)((a.n_entries + per_wg - 1) / per_wg), (unsigned)a.n_seq), block(64 * kEntryWaves);
    const bool pk = P.bf16_in && P.vec_in;
    switch (a.D) {
        case 32: case 64: V4A_LAUNCH("compress_kernel", (compress_kernel<1, false>), grid, block, 0, s, P); break;
        case 128:
            if (pk) V4A_LAUNCH("compress_kernel", (compress_kernel<2, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("compress_kernel", (compress_kernel<2, false>), grid, block, 0, s, P);
            break;
        case 256:
            if (pk) V4A_LAUNCH("compress_kernel", (compress_kernel<4, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("compress_kernel", (compress_kernel<4, false>), grid, block, 0, s, P);
            break;
        default:
            if (pk) V4A_LAUNCH("compress_kernel", (compress_kernel<8, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("compress_kernel", (compress_kernel<8, false>), grid, block, 0, s, P);
            break;
    }
    return hipGetLastError();
}

}  // namespace v4a

namespace v4a {

hipError_t launch_decode_prologue(const CompressArgs &key, int blocks_before, int B, const int64_t *entry,
                                  void *zero, size_t zero_bytes, hipStream_t s) {
    PrologueParams P;
    P.key = compress_params(key);
    P.blocks_before = blocks_before;
    P.B = B;
    for (int b = 0; b < kMaxSeq; b++) P.entry[b] = b < B ? entry[b] : -1;
    P.zero = (uint4 *)zero;
    P.zero_n16 = zero_bytes / 16;
    const unsigned zx = (unsigned)std::min<size_t>((P.zero_n16 + 64 * kEntryWaves - 1) / (64 * kEntryWaves), 1024);
    dim3 grid(zx > 0 ? zx : 1, (unsigned)(B + 1));
    const bool pk = P.key.bf16_in && P.key.vec_in;
    const dim3 block(64 * kEntryWaves);
    switch (key.D) {
        case 32: case 64: V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<1, false>), grid, block, 0, s, P); break;
        case 128:
            if (pk) V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<2, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<2, false>), grid, block, 0, s, P);
            break;
        case 256:
            if (pk) V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<4, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<4, false>), grid, block, 0, s, P);
            break;
        case 512:
            if (pk) V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<8, true>), grid, block, 0, s, P);
            else V4A_LAUNCH("decode_prologue_kernel", (decode_prologue_kernel<8, false>), grid, block, 0, s, P);
            break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace v4a
