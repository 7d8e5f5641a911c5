// projection.hip -- the grouped output projection after the attention.
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 2.2, "Grouped Output Projection":
// with many query heads (128 for V4-Pro) the head outputs are first reduced group by group, then
// the reduced groups are concatenated and projected, which cuts the output projection's
// parameters and FLOPs; "DeepSeek V4 technical report explained" (firecat-web.com), item 2: head
// dim 512 with a grouped projection to lower the cost.
//
// Two BF16 GEMMs with fp32 accumulation, both of the form C[M][N] = A[M][K] . W[N][K]^T (rows of
// activations times the rows of a weight matrix stored out-feature major):
//   grouped: for group g, y[t][g*r .. g*r+r) = bf16(o[t][g*Kg .. g*Kg+Kg) . wg[g]^T), Kg = H*D/G;
//   final:   out[t] = y[t] . wf^T.
// On the MFMA unit the weight rows are the A operand (its rows are output features) and the
// tokens the B operand, so each lane ends up holding 4 consecutive output features of one token
// and writes them with one store.
//   GEMV kernel (M <= 8, decode): as the skinny kernel below, but the weight and token rows
//     travel through LDS by direct loads of 256 contiguous bytes per row;
//   skinny kernel (M <= 64, decode): one workgroup per 16 output features; its four wavefronts
//     stream disjoint quarters of K (the weights are read once, straight from HBM, in 16-byte
//     loads, 8 or 16 k-steps in flight), each holding every token as MFMA B operands, and add
//     their partial sums in a fixed order through LDS;
//   tiled kernel (large M, prefill): 256 x 128 output tiles, K in chunks of 64 through three LDS
//     stages filled by direct loads two chunks ahead, four wavefronts of 128 x 64 each on
//     v_mfma_f32_32x32x16_bf16.
#include "common.hpp"

namespace v4a {

struct GemmParams {
    const uint16_t *A;   // [batch][M][lda] bf16 (activations)
    const uint16_t *W;   // [batch][N][ldw] bf16 (weights, out-feature major)
    void *C;             // [batch][M][ldc] bf16 or fp32
    int M, N, K;
    int64_t lda, ldw, ldc;
    int64_t sa, sw, sc;  // batch strides (elements)
    bool c_bf16;
};

typedef float v16f __attribute__((ext_vector_type(16)));

__device__ __forceinline__ v8bf as_bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// A streamed (read-once) 16-byte weight load.
__device__ __forceinline__ uint4 load_nt16(const uint16_t *p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Stores 4 consecutive output features n0..n0+3 of token m (n0 a multiple of 4).
__device__ __forceinline__ void store4(const GemmParams &P, int64_t cbase, int m, int n0, float a, float b, float c,
                                       float d) {
    const int64_t off = cbase + (int64_t)m * P.ldc + n0;
    if (P.c_bf16) {
        const uint32_t lo = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(c) | ((uint32_t)f32_to_bf16(d) << 16);
        *(uint2 *)((uint16_t *)P.C + off) = make_uint2(lo, hi);
    } else {
        *(float4 *)((float *)P.C + off) = make_float4(a, b, c, d);
    }
}

// ---------------------------------------------------------------- skinny kernel ----
constexpr int kSkinnyTokens = 64;  // M limit of the skinny kernel (four 16-token MFMA columns)

// MT: 16-token column tiles held per wavefront (M <= 16 * MT); UNROLL: k-steps of 32 whose
// weight loads are in flight together (16 with one token tile measured 3-4% faster than 8).
template <int MT, int UNROLL>
__global__ void __launch_bounds__(256) gemm_skinny_kernel(GemmParams P) {
    __shared__ float red[3][MT][64][4];  // partial sums of wavefronts 1..3
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int n0 = blockIdx.x * 16, bt = blockIdx.y;
    const uint16_t *A = P.A + (int64_t)bt * P.sa;
    const uint16_t *W = P.W + (int64_t)bt * P.sw + (int64_t)(n0 + col) * P.ldw;  // the lane's weight row
    const int kq = P.K / 4;                     // this wavefront's quarter of K (a multiple of 32)
    const int kb = wv * kq;
    v4f acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // token rows of the B operand: lane holds token 16t + col (rows past M read row 0, masked
    // at the store)
    int64_t arow[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) arow[t] = (int64_t)(16 * t + col < P.M ? 16 * t + col : 0) * P.lda;
    for (int k0 = kb; k0 < kb + kq; k0 += 32 * UNROLL) {
        const int nk = min(UNROLL, (kb + kq - k0) / 32);  // uniform
        uint4 wr[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; u++)
            if (u < nk) wr[u] = load_nt16(W + k0 + 32 * u + 8 * grp);
#pragma unroll
        for (int u = 0; u < UNROLL; u++) {
            if (u >= nk) continue;  // uniform; a predicated step keeps the loop unrolled
            uint4 ar[MT];
#pragma unroll
            for (int t = 0; t < MT; t++) ar[t] = *(const uint4 *)(A + arow[t] + k0 + 32 * u + 8 * grp);
#pragma unroll
            for (int t = 0; t < MT; t++)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(wr[u]), as_bf(ar[t]), acc[t], 0, 0, 0);
        }
    }
    // fixed-order sum over the four K quarters: ((w0 + w1) + w2) + w3
    if (wv > 0) {
#pragma unroll
        for (int t = 0; t < MT; t++) *(v4f *)red[wv - 1][t][lane] = acc[t];
    }
    __syncthreads();
    if (wv != 0) return;
    const int64_t cbase = (int64_t)bt * P.sc;
#pragma unroll
    for (int t = 0; t < MT; t++) {
        v4f s = acc[t];
#pragma unroll
        for (int w = 0; w < 3; w++) s += *(const v4f *)red[w][t][lane];
        const int m = 16 * t + col;
        if (m < P.M) store4(P, cbase, m, n0 + 4 * grp, s[0], s[1], s[2], s[3]);
    }
}

// ----------------------------------------------------------------- tiled kernel ----
// Output tile: 256 features x 128 tokens; wavefront (wn, wm) of four owns 128 features x 64 tokens
// (4 x 2 MFMA tiles of 32 x 32).  K runs in chunks of 64 through a ring of three LDS stages,
// filled by direct-to-LDS loads two chunks ahead (no register staging).  An LDS row is one
// feature's (or token's) 64 K values, 128 bytes in eight 16-byte slots; slot c of row r holds K
// chunk c ^ ((r >> 1) & 7), so the 16 rows read by one quarter-wavefront hit 16 different
// 4-bank groups.  Tiles are numbered so that the workgroups resident on one XCD (linear ids
// congruent mod 8) take consecutive tile numbers, which cover blocks of 4 feature tiles by 8 token
// tiles and share their operands through that XCD's L2.
constexpr int kTN = 256;            // tile features
constexpr int kTM = 128;            // tile tokens
constexpr int kTK = 64;             // K per stage
constexpr int kGroupM = 8;          // token tiles per tile group
constexpr int kStageW = kTN * kTK;  // bf16 elements of one stage's weight tile
constexpr int kStageA = kTM * kTK;
constexpr int kStage = kStageW + kStageA;

typedef __attribute__((address_space(3))) void *gemm_lds_ptr_t;
typedef __attribute__((address_space(1))) void *gemm_glb_ptr_t;

struct TiledMap {
    int nN, nM, per_batch, batch, per_xcd;
};

__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One chunk: the direct loads of chunk k_next into stage `next` (when issue), then the MFMAs of the
// chunk held in stage `cur`.  The two stages are distinct restrict pointers: the loads into one
// never hold up the operand reads of the other.
__device__ __forceinline__ void tiled_chunk(const uint16_t *__restrict__ cur, uint16_t *__restrict__ next, bool issue,
                                            int k_next, const uint16_t *const (&wsrc)[8],
                                            const uint16_t *const (&asrc)[4], int wv_u, const int (&wrow)[4],
                                            const int (&arow)[2], int kh, v16f (&acc)[4][2]) {
    if (issue) {
#pragma unroll
        for (int i = 0; i < 8; i++)
            lds_copy16(wsrc[i] + k_next, lds_addr(next + (64 * wv_u + 8 * i) * kTK));
#pragma unroll
        for (int i = 0; i < 4; i++)
            lds_copy16(asrc[i] + k_next, lds_addr(next + kStageW + (32 * wv_u + 8 * i) * kTK));
    }
    const uint16_t *__restrict__ sa = cur + kStageW;
#pragma unroll
    for (int ks = 0; ks < kTK / 16; ks++) {
        const int ch = 2 * ks + kh;  // this lane's 16-byte K chunk
        v8bf wa[4], ab[2];
#pragma unroll
        for (int i = 0; i < 4; i++) wa[i] = as_bf(*(const uint4 *)(cur + wrow[i] * kTK + 8 * swz(wrow[i], ch)));
#pragma unroll
        for (int j = 0; j < 2; j++) ab[j] = as_bf(*(const uint4 *)(sa + arow[j] * kTK + 8 * swz(arow[j], ch)));
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[i], ab[j], acc[i][j], 0, 0, 0);
    }
}

__global__ void __launch_bounds__(256, 1) gemm_tiled_kernel(GemmParams P, TiledMap TM) {
    __shared__ __attribute__((aligned(16))) uint16_t smem[3 * kStage];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    // tile of this workgroup: XCD-contiguous numbering, then (batch, group of kGroupM token tiles)
    const int L = blockIdx.x;
    const int T = (L & 7) * TM.per_xcd + (L >> 3);
    if (T >= TM.per_batch * TM.batch) return;  // uniform
    const int bt = T / TM.per_batch, loc = T % TM.per_batch;
    const int gsz = kGroupM * TM.nN, grp = loc / gsz, in = loc % gsz;
    const int gm = min(kGroupM, TM.nM - grp * kGroupM);  // token tiles in this (last) group
    const int tn = in / gm, tm = grp * kGroupM + in % gm;
    const int n0 = tn * kTN, m0 = tm * kTM;
    const uint16_t *W = P.W + (int64_t)bt * P.sw;
    const uint16_t *A = P.A + (int64_t)bt * P.sa;

    // direct loads: one instruction moves 8 rows x 128 bytes (lane l -> row l / 8, slot l % 8, which
    // holds K chunk swz(row, l % 8)); wavefront w takes weight rows 64 w .. 64 w + 63 and token
    // rows 32 w .. 32 w + 31
    const int lrow = lane >> 3, slot = lane & 7;
    const uint16_t *wsrc[8];
    const uint16_t *asrc[4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int r = 64 * wv + 8 * i + lrow;
        wsrc[i] = W + (int64_t)min(n0 + r, P.N - 1) * P.ldw + 8 * swz(r, slot);
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int r = 32 * wv + 8 * i + lrow;
        asrc[i] = A + (int64_t)min(m0 + r, P.M - 1) * P.lda + 8 * swz(r, slot);  // rows past M: valid, never stored
    }
    const int wv_u = __builtin_amdgcn_readfirstlane(wv);
    const int wn = wv & 1, wm = wv >> 1;
    const int r32 = lane & 31, kh = lane >> 5;
    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] = 0.0f;
    int wrow[4], arow[2];
#pragma unroll
    for (int i = 0; i < 4; i++) wrow[i] = 128 * wn + 32 * i + r32;
#pragma unroll
    for (int j = 0; j < 2; j++) arow[j] = 64 * wm + 32 * j + r32;

    const int nch = P.K / kTK;
    // chunks 0 and 1 travel first; chunk c is computed from stage c % 3 while chunk c+1 (issued
    // earlier) and c+2 (issued at its start, into the stage chunk c-1 used) travel
    for (int c = 0; c < 2 && c < nch; c++) {
#pragma unroll
        for (int i = 0; i < 8; i++)
            lds_copy16(wsrc[i] + c * kTK, lds_addr(smem + c * kStage + (64 * wv_u + 8 * i) * kTK));
#pragma unroll
        for (int i = 0; i < 4; i++)
            lds_copy16(asrc[i] + c * kTK, lds_addr(smem + c * kStage + kStageW + (32 * wv_u + 8 * i) * kTK));
    }
    for (int c = 0; c < nch; c++) {
        // this wavefront's loads of chunk c have landed (chunk c+1's may still travel); after the
        // barrier every wavefront's have, and chunk c-1's readers are done with its stage
        if (c + 1 < nch) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        asm volatile("s_barrier" ::: "memory");
        tiled_chunk(smem + (c % 3) * kStage, smem + ((c + 2) % 3) * kStage, c + 2 < nch, (c + 2) * kTK, wsrc, asrc, wv_u,
                    wrow, arow, kh, acc);
    }
    // lane holds token 64 wm + 32 j + r32 and, per register e, feature 128 wn + 32 i + 8 (e / 4) + 4 kh + e % 4
    const int64_t cbase = (int64_t)bt * P.sc;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int m = m0 + 64 * wm + 32 * j + r32;
        if (m >= P.M) continue;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
            for (int g = 0; g < 4; g++) {
                const int n = n0 + 128 * wn + 32 * i + 8 * g + 4 * kh;
                if (n < P.N)
                    store4(P, cbase, m, n, acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]);
            }
    }
}

// C = A . W^T over `batch` independent problems: the skinny kernel for a few tokens, else the tiled one.
// ------------------------------------------------------------------- GEMV kernel ----
// M <= 8 tokens (decode): one workgroup per 16 output features, its four wavefronts each
// streaming a quarter of K.  A wavefront moves its 16 weight rows and the 8 token rows through
// its own ring of three LDS stages in chunks of 128 K, two chunks ahead of the MFMAs, with
// direct-to-LDS loads only (one instruction carries four rows x 256 contiguous bytes).  In a
// row, 16-byte slot s holds K chunk s ^ (row & 15), so the A-operand reads of 16 weight rows
// hit 16 different 4-bank groups (token rows past M repeat row M-1 and are never stored).
constexpr int kGvK = 128;                 // K per chunk
constexpr int kGvRow = 2 * kGvK;          // bytes of one row's chunk
constexpr int kGvTok = 8;                 // token rows per stage (M limit of this kernel)
constexpr int kGvStage = (16 + kGvTok) * kGvRow;
constexpr int kGvLoads = (16 + kGvTok) / 4;  // direct loads per chunk

// The MFMAs of one chunk held in stage `cur` (a restrict pointer: its reads are ordered after
// the chunk's direct loads by the caller's explicit wait, not by the compiler's).
__device__ __forceinline__ void gemv_compute(const uint8_t *__restrict__ cur, int col, int grp, v4f &acc) {
    const int tr = 16 + (col & (kGvTok - 1));  // this lane's token row
#pragma unroll
    for (int ks = 0; ks < kGvK / 32; ks++) {
        const int ch = 4 * ks + grp;
        const uint4 w = *(const uint4 *)(cur + col * kGvRow + 16 * (ch ^ col));
        const uint4 a = *(const uint4 *)(cur + tr * kGvRow + 16 * (ch ^ (tr & 15)));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf(w), as_bf(a), acc, 0, 0, 0);
    }
}

__global__ void __launch_bounds__(256) gemm_gemv_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(16))) uint8_t buf[4][3][kGvStage];
    __shared__ float red[3][64][4];  // partial sums of wavefronts 1..3
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int wvu = __builtin_amdgcn_readfirstlane(wv);
    const int col = lane & 15, grp = lane >> 4;
    const int n0 = blockIdx.x * 16, bt = blockIdx.y;
    const uint16_t *A = P.A + (int64_t)bt * P.sa;
    const uint16_t *W = P.W + (int64_t)bt * P.sw;
    const int kq = P.K / 4, kb = wvu * kq;  // this wavefront's quarter of K
    const int nch = kq / kGvK;
    // direct load i carries rows 4i .. 4i+3 of the stage: lane l -> row 4i + l/16, slot l%16
    // (K chunk slot ^ (row & 15)); rows 0..15 are weight rows, 16.. token rows
    const int qr = lane >> 4, slot = lane & 15;
    const uint16_t *src[kGvLoads];
#pragma unroll
    for (int i = 0; i < kGvLoads; i++) {
        const int r = 4 * i + qr;
        const int ks = slot ^ (r & 15);
        src[i] = r < 16 ? W + (int64_t)(n0 + r) * P.ldw + kb + 8 * ks
                        : A + (int64_t)min(r - 16, P.M - 1) * P.lda + kb + 8 * ks;
    }
    uint8_t *const base = &buf[wvu][0][0];  // stage j at base + j * kGvStage (kept in LDS arithmetic)
    v4f acc = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // step c loads chunk c + 2 (past the end the last chunk again, into a stage nobody reads, so
    // every step issues the same loads and the wait needs no branch) and, for c >= 0, computes
    // chunk c once its loads have landed (the next two chunks' may travel)
#pragma clang loop unroll(disable)
    for (int c = -2; c < nch; c++) {
        uint8_t *next = base + ((c + 2) % 3) * kGvStage;
#pragma unroll
        for (int i = 0; i < kGvLoads; i++)
            lds_copy16(src[i], lds_addr(next + 4 * i * kGvRow));
        if (c + 3 < nch) {  // uniform
#pragma unroll
            for (int i = 0; i < kGvLoads; i++) src[i] += kGvK;
        }
        if (c >= 0) {  // uniform
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kGvLoads) : "memory");
            gemv_compute(base + (c % 3) * kGvStage, col, grp, acc);
        }
    }
    // fixed-order sum over the four K quarters: ((w0 + w1) + w2) + w3
    if (wv > 0) *(v4f *)red[wv - 1][lane] = acc;
    __syncthreads();
    if (wv != 0) return;
    v4f s4 = acc;
#pragma unroll
    for (int w = 0; w < 3; w++) s4 += *(const v4f *)red[w][lane];
    if (col < P.M) store4(P, (int64_t)bt * P.sc, col, n0 + 4 * grp, s4[0], s4[1], s4[2], s4[3]);
}

hipError_t launch_gemm(const GemmParams &P, int batch, hipStream_t s) {
    if (P.M <= 0 || P.N <= 0 || batch <= 0) return hipSuccess;
    if (P.K % 128 != 0 || P.N % 16 != 0) return hipErrorInvalidValue;
    if (P.M <= kSkinnyTokens) {
        dim3 grid((unsigned)(P.N / 16), (unsigned)batch);
        if (P.M <= kGvTok && P.K % (4 * kGvK) == 0)
            V4A_LAUNCH("gemm_gemv_kernel", gemm_gemv_kernel, grid, dim3(256), 0, s, P);
        else if (P.M <= 16)
            V4A_LAUNCH("gemm_skinny_kernel", (gemm_skinny_kernel<1, 16>), grid, dim3(256), 0, s, P);
        else if (P.M <= 32)
            V4A_LAUNCH("gemm_skinny_kernel", (gemm_skinny_kernel<2, 8>), grid, dim3(256), 0, s, P);
        else
            V4A_LAUNCH("gemm_skinny_kernel", (gemm_skinny_kernel<4, 8>), grid, dim3(256), 0, s, P);
    } else {
        if (P.K % kTK != 0 || P.N % 8 != 0) return hipErrorInvalidValue;
        TiledMap TM;
        TM.nN = (P.N + kTN - 1) / kTN;
        TM.nM = (P.M + kTM - 1) / kTM;
        TM.per_batch = TM.nN * TM.nM;
        TM.batch = batch;
        TM.per_xcd = (TM.per_batch * batch + 7) / 8;
        V4A_LAUNCH("gemm_tiled_kernel", gemm_tiled_kernel, dim3((unsigned)(8 * TM.per_xcd)), dim3(256), 0, s, P, TM);
    }
    return hipGetLastError();
}

hipError_t launch_output_projection(const OutProjArgs &a, hipStream_t s) {
    const int Kg = a.H * a.D / a.G;
    GemmParams g{};
    g.A = (const uint16_t *)a.o;
    g.W = (const uint16_t *)a.wg;
    g.C = a.y;
    g.M = a.T;
    g.N = a.r;
    g.K = Kg;
    g.lda = (int64_t)a.H * a.D;
    g.ldw = Kg;
    g.ldc = (int64_t)a.G * a.r;
    g.sa = Kg;                   // group g reads columns g*Kg .. of every token row
    g.sw = (int64_t)a.r * Kg;
    g.sc = a.r;                  // and writes columns g*r .. of y
    g.c_bf16 = true;
    hipError_t e = launch_gemm(g, a.G, s);
    if (e != hipSuccess) return e;
    GemmParams f{};
    f.A = (const uint16_t *)a.y;
    f.W = (const uint16_t *)a.wf;
    f.C = a.out;
    f.M = a.T;
    f.N = a.d;
    f.K = a.G * a.r;
    f.lda = (int64_t)a.G * a.r;
    f.ldw = (int64_t)a.G * a.r;
    f.ldc = a.d;
    f.c_bf16 = a.out_bf16;
    return launch_gemm(f, 1, s);
}

}  // namespace v4a
