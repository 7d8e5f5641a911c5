// quant.hip -- a3: entry-record quantisation (FP8 E4M3 non-RoPE dims with a per-entry
// fp32 scale, BF16 RoPE dims) and MXFP4 quantisation of indexer vectors.
// "DeepSeek V4 preview and technical report" (chooseai.net), section 1: KV stored with the
// RoPE dims in BF16 and the rest in FP8.  "DeepSeek-V4 technical report walkthrough"
// (cyqw.cn), section 3.4: the indexer QK path uses MXFP4 (E2M1 with 1x32 blocks).
//
// One wavefront per row, each lane owning VPT = D/64 consecutive dims (one lane per dim,
// the upper lanes idle, when D < 64).  Reads are fp32 rows, writes are the packed codes;
// both are contiguous per wavefront.
#include "encoders.hpp"

namespace v4a {

template <int VPT>
__global__ void __launch_bounds__(256) quantize_kv_kernel(const float *__restrict__ x, int64_t rows,
                                                          v4a_kv out, int64_t row0) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;  // whole wavefront leaves together
    const int D = out.D;
    const bool active = lane * VPT < D;
    float v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; i++) v[i] = active ? x[r * D + lane * VPT + i] : 0.0f;
    store_record<VPT>(v, lane * VPT, active, D, out.R, out, row0 + r);
}

template <int VPT>
__global__ void __launch_bounds__(256) quantize_mxfp4_kernel(const float *__restrict__ x, int64_t rows,
                                                             v4a_idx out, int64_t row0) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    const int d = out.d;
    const bool active = lane * VPT < d;
    float v[VPT];
#pragma unroll
    for (int i = 0; i < VPT; i++) v[i] = active ? x[r * d + lane * VPT + i] : 0.0f;
    store_mxfp4<VPT>(v, lane, active, d, out, row0 + r);
}

hipError_t launch_quantize_kv(const float *x, int64_t rows, const v4a_kv &out, int64_t row0,
                              hipStream_t s) {
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    switch (out.D) {
        case 32: case 64: V4A_LAUNCH("quantize_kv_kernel", quantize_kv_kernel<1>, grid, block, 0, s, x, rows, out, row0); break;
        case 128: V4A_LAUNCH("quantize_kv_kernel", quantize_kv_kernel<2>, grid, block, 0, s, x, rows, out, row0); break;
        case 256: V4A_LAUNCH("quantize_kv_kernel", quantize_kv_kernel<4>, grid, block, 0, s, x, rows, out, row0); break;
        default: V4A_LAUNCH("quantize_kv_kernel", quantize_kv_kernel<8>, grid, block, 0, s, x, rows, out, row0); break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp4(const float *x, int64_t rows, const v4a_idx &out, int64_t row0,
                                 hipStream_t s) {
    if (rows == 0) return hipSuccess;
    dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    switch (out.d) {
        case 32: case 64: V4A_LAUNCH("quantize_mxfp4_kernel", quantize_mxfp4_kernel<1>, grid, block, 0, s, x, rows, out, row0); break;
        case 128: V4A_LAUNCH("quantize_mxfp4_kernel", quantize_mxfp4_kernel<2>, grid, block, 0, s, x, rows, out, row0); break;
        case 256: V4A_LAUNCH("quantize_mxfp4_kernel", quantize_mxfp4_kernel<4>, grid, block, 0, s, x, rows, out, row0); break;
        default: V4A_LAUNCH("quantize_mxfp4_kernel", quantize_mxfp4_kernel<8>, grid, block, 0, s, x, rows, out, row0); break;
    }
    return hipGetLastError();
}

}  // namespace v4a
