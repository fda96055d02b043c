// NVFP4 quantization of one 128-element vector by one 64-lane wavefront, and its placement in
// a head page; shared by the insert kernel and the fused insert + indexer kernel.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "TL;DR", its item on fusing the QKV
// GEMM, norm, RoPE and KV insert: K, V and the index key are quantized to NVFP4 when they are
// written to their caches.
// "MiniMax-M3.1-Flash serving notes", section "The capacity numbers": 4-bit E2M1 values and one
// E4M3 scale per 16 values.
//
// Lane l owns elements 2l and 2l+1; eight lanes form one 16-element scale group. The rounding
// rule (msa.h) is evaluated in fp32 exactly as stated: no FP contraction in these functions.
#pragma once

#include "device_common.hpp"

namespace msa {

// Round a non-negative fp32 value to the nearest E4M3 (OCP "FN") code, ties to even, values
// at or above 448 saturating to 448 (code 0x7E). Integer construction from the fp32 bits.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float s) {
#pragma clang fp contract(off)
    if (!(s < 448.0f)) return 0x7Eu;
    const uint32_t bits = __float_as_uint(s);
    const int e = (int)(bits >> 23) - 127;  // unbiased exponent; very small s lands below -6
    if (e < -6) {
        // E4M3 subnormal range: a multiple of 2^-9; 8 * 2^-9 is the smallest normal (code 8)
        return (uint32_t)rintf(s * 512.0f);
    }
    const float m = rintf(ldexpf(s, 3 - e));  // 8..16 quanta of 2^(e-3); 16 carries into e+1
    return (uint32_t)((e + 7) << 3) + (uint32_t)m - 8u;
}

// E2M1 magnitude code of the fp32 ratio r = |x| / s: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
// the even code, saturating at 6. Each comparison is against an exact midpoint; ">" at a
// midpoint whose lower neighbour has the even code, ">=" where the upper one does.
__device__ __forceinline__ uint32_t e2m1_magnitude(float r) {
    return (uint32_t)(r > 0.25f) + (uint32_t)(r >= 0.75f) + (uint32_t)(r > 1.25f) +
           (uint32_t)(r >= 1.75f) + (uint32_t)(r > 2.5f) + (uint32_t)(r >= 3.5f) +
           (uint32_t)(r > 5.0f);
}

// Maximum of v over the 8 lanes of this lane's scale group (lanes 8g .. 8g + 7), with DPP lane
// moves: swap neighbours, swap pairs within the quad, then the mirrored lane of the other quad.
__device__ __forceinline__ float max_over_group(float v) {
    constexpr int kQuadSwap1 = 0xB1;   // quad_perm [1, 0, 3, 2]
    constexpr int kQuadSwap2 = 0x4E;   // quad_perm [2, 3, 0, 1]
    constexpr int kHalfMirror = 0x141; // lane i of each 8-lane half row reads lane 7 - i
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kQuadSwap2, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kHalfMirror, 0xF, 0xF, false)));
    return v;
}

// Quantize the two elements (x0, x1) owned by this lane; returns the byte of their two
// nibbles (x0 low) and the group's scale byte. Every lane of the wavefront takes part.
__device__ __forceinline__ void quantize_pair(float x0, float x1, uint32_t& byte, uint32_t& scale) {
#pragma clang fp contract(off)
    const float amax = max_over_group(fmaxf(fabsf(x0), fabsf(x1)));
    const float s32 = amax / 6.0f;
    scale = e4m3_encode_rne_sat(s32);
    const float s = __builtin_amdgcn_cvt_f32_fp8(scale, 0);
    uint32_t m0 = 0, m1 = 0;
    if (s > 0.0f) {
        m0 = e2m1_magnitude(fabsf(x0) / s);
        m1 = e2m1_magnitude(fabsf(x1) / s);
    }
    const uint32_t n0 = m0 | ((__float_as_uint(x0) >> 31) << 3);
    const uint32_t n1 = m1 | ((__float_as_uint(x1) >> 31) << 3);
    byte = n0 | (n1 << 4);
}

// Store the byte and scale that quantize_pair gave this lane into token t of the head page
// dst: row-operand layout (K, index keys) with plain byte stores, or column-operand layout (V),
// whose code bytes hold two tokens, with an atomic and/or pair per nibble so that a neighbour
// token written concurrently keeps its nibble.
__device__ __forceinline__ void store_quantized(uint32_t byte, uint32_t scale, uint8_t* dst, int t,
                                                bool column_layout, int lane) {
    const int e = 2 * lane;   // first of the lane's two elements
    const int g = lane >> 3;  // its scale group
    if (!column_layout) {
        dst[row_chunk_offset(t, e >> 5) + ((e & 31) >> 1)] = (uint8_t)byte;
        if ((lane & 7) == 0) dst[row_scale_offset(t, g)] = (uint8_t)scale;
    } else {
        const int shift = 8 * ((t >> 1) & 3) + 4 * (t & 1);
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const uint32_t nib = (byte >> (4 * h)) & 15u;
            const int off = col_code_byte(e + h, t) & ~3;
            uint32_t* word = reinterpret_cast<uint32_t*>(dst + off);
            atomicAnd(word, ~(15u << shift));
            atomicOr(word, nib << shift);
        }
        if ((lane & 7) == 0) dst[col_scale_offset(t, g)] = (uint8_t)scale;
    }
}

// Quantize the 128-element vector this wavefront's lanes hold (x = elements 2l, 2l+1) into
// token t of the head page dst.
__device__ __forceinline__ void quantize_store_vector(f32x2 x, uint8_t* dst, int t,
                                                      bool column_layout, int lane) {
    uint32_t byte, scale;
    quantize_pair(x[0], x[1], byte, scale);
    store_quantized(byte, scale, dst, t, column_layout, lane);
}

}  // namespace msa
