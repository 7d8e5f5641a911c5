// encoders.hpp -- row encoders shared by the quantisers and the compressors: a row held
// VPT values per lane of one wavefront is written as an entry record (FP8 E4M3 non-RoPE dims
// with a per-entry fp32 scale, BF16 RoPE dims, or plain fp32) or as an MXFP4 indexer vector.
// "DeepSeek V4 preview and technical report" (chooseai.net), section 1 (KV precision split);
// "DeepSeek-V4 technical report walkthrough" (cyqw.cn), section 3.4 (MXFP4 indexer QK).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace v4a {

// Shared by the quantiser and the compressors: encode one row held VPT values per lane.
// `lane_dim0` is the first dim of this lane; `active` is false for lanes past D.
template <int VPT>
__device__ __forceinline__ void store_record(const float (&x)[VPT], int lane_dim0, bool active,
                                             int D, int R, const v4a_kv &out, int64_t row) {
    const int Dn = D - R;
    if (out.fmt == V4A_KV_F32) {
        if (active) {
            float *dst = (float *)out.nope + row * D + lane_dim0;
#pragma unroll
            for (int v = 0; v < VPT; v++) dst[v] = x[v];
        }
        return;
    }
    // FP8 part: amax over the first Dn dims (each lane's dims are all nope or all rope).
    const bool is_nope = active && lane_dim0 < Dn;
    float amax = 0.0f;
    if (is_nope) {
#pragma unroll
        for (int v = 0; v < VPT; v++) amax = fmaxf(amax, fabsf(x[v]));
    }
    amax = wave_max(amax);
    if (is_nope) {
        uint8_t *dst = (uint8_t *)out.nope + row * Dn + lane_dim0;
        if (amax == 0.0f) {
#pragma unroll
            for (int v = 0; v < VPT; v++) dst[v] = 0;
        } else {
            float inv = __fdiv_rn(448.0f, amax);
            uint32_t packed[(VPT + 3) / 4] = {};
            if constexpr (VPT % 4 == 0) {
#pragma unroll
                for (int i = 0; i < VPT / 4; i++)
                    packed[i] = e4m3_encode4(x[4 * i] * inv, x[4 * i + 1] * inv, x[4 * i + 2] * inv, x[4 * i + 3] * inv);
            } else if constexpr (VPT == 2) {
                packed[0] = e4m3_encode2(x[0] * inv, x[1] * inv);
            } else {
                packed[0] = e4m3_encode2(x[0] * inv, 0.0f) & 0xFFu;
            }
            if constexpr (VPT % 4 == 0) {
#pragma unroll
                for (int i = 0; i < VPT / 4; i++) ((uint32_t *)dst)[i] = packed[i];
            } else {
#pragma unroll
                for (int v = 0; v < VPT; v++) dst[v] = (uint8_t)(packed[v / 4] >> (8 * (v % 4)));
            }
        }
        if (lane_dim0 == 0) out.scale[row] = amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
    } else if (active) {
        uint16_t *dst = (uint16_t *)out.rope + row * R + (lane_dim0 - Dn);
#pragma unroll
        for (int v = 0; v < VPT; v++) dst[v] = f32_to_bf16(x[v]);
    }
}

// MXFP4 encoding of one row held VPT values per lane (d = 64*VPT, or d = 32 with VPT = 1).
// With `mirror` (LDS) the row's d/2 code bytes and d/32 scale bytes are also written there,
// in the same order as in the cache row.
template <int VPT>
__device__ __forceinline__ void store_mxfp4(const float (&x)[VPT], int lane, bool active, int d,
                                            const v4a_idx &out, int64_t row, uint8_t *mirror = nullptr,
                                            bool to_global = true) {
    if (out.fmt == V4A_IDX_F32) {
        if (active) {
            float *dst = (float *)out.codes + row * d + lane * VPT;
#pragma unroll
            for (int v = 0; v < VPT; v++) dst[v] = x[v];
        }
        return;
    }
    constexpr int group = 32 / VPT;  // lanes per 32-element block
    float amax = 0.0f;
    if (active) {
#pragma unroll
        for (int v = 0; v < VPT; v++) amax = fmaxf(amax, fabsf(x[v]));
    }
    if constexpr (group == 16) {
        // a block is one 16-lane row: its maximum by row rotations of 8, 4, 2, 1 lanes
        // (exact in any order)
        auto ror_max = [](float a, auto ctrl) {
            return fmaxf(a, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                0, __builtin_bit_cast(int, a), decltype(ctrl)::value, 0xF, 0xF, false)));
        };
        amax = ror_max(amax, std::integral_constant<int, 0x128>{});
        amax = ror_max(amax, std::integral_constant<int, 0x124>{});
        amax = ror_max(amax, std::integral_constant<int, 0x122>{});
        amax = ror_max(amax, std::integral_constant<int, 0x121>{});
    } else {
        for (int o = group / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    }
    int X = mx_block_exp(amax);
    uint32_t codes = 0;  // VPT nibbles, element order = nibble order
#pragma unroll
    for (int v = 0; v < VPT; v++) {
        uint32_t c = amax == 0.0f ? 0u : e2m1_encode(ldexpf(x[v], -X));
        codes |= c << (4 * v);
    }
    uint8_t *dst = (uint8_t *)out.codes + row * (d / 2);
    if constexpr (VPT == 1) {
        uint32_t hi = __shfl_down(codes, 1);
        if (active && (lane & 1) == 0) dst[lane / 2] = (uint8_t)(codes | (hi << 4));
    } else {
        if (active) {
#pragma unroll
            for (int i = 0; i < VPT / 2; i++) {
                if (to_global) dst[lane * VPT / 2 + i] = (uint8_t)(codes >> (8 * i));
                if (mirror) mirror[lane * VPT / 2 + i] = (uint8_t)(codes >> (8 * i));
            }
        }
    }
    if (active && (lane % group) == 0) {
        if (to_global) out.scales[row * (d / 32) + lane / group] = (uint8_t)(X + 127);
        if (mirror) mirror[d / 2 + lane / group] = (uint8_t)(X + 127);
    }
}

}  // namespace v4a
