// NVFP4 quantize-and-insert of K, V and index keys into their paged caches.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "QKV GEMM + norm + RoPE + KV insert
// fusion": K, V and the index key are quantized to NVFP4 when they are written to their caches.
// "MiniMax-M3.1-Flash serving notes", section "The capacity numbers": 4-bit E2M1 values and one
// E4M3 scale per 16 values.
//
// One 64-lane wavefront quantizes one 128-element vector: lane l owns elements 2l and 2l+1,
// eight lanes form one 16-element scale group. The rounding rule (msa.h) is evaluated in fp32
// exactly as stated, so FP contraction is off in this file.
#include "device_common.hpp"
#include "kernels.hpp"

#pragma clang fp contract(off)

namespace msa {
namespace {

// Round a non-negative fp32 value to the nearest E4M3 (OCP "FN") code, ties to even, values
// at or above 448 saturating to 448 (code 0x7E). Integer construction from the fp32 bits.
__device__ __forceinline__ uint32_t e4m3_encode_rne_sat(float s) {
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

// Quantize the two elements (x0, x1) owned by this lane; returns the byte of their two
// nibbles (x0 low) and the group's scale byte.
__device__ __forceinline__ void quantize_pair(float x0, float x1, uint32_t& byte, uint32_t& scale) {
    float amax = fmaxf(fabsf(x0), fabsf(x1));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
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

// grid.x = tokens, block = 9 wavefronts: waves 0-3 quantize K heads 0-3, waves 4-7 V heads
// 0-3, wave 8 the index key.
__global__ __launch_bounds__(576) void insert_kernel(uint8_t* __restrict__ k_pool,
                                                     uint8_t* __restrict__ v_pool,
                                                     uint8_t* __restrict__ ik_pool,
                                                     int64_t num_pages,
                                                     const int64_t* __restrict__ slots,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ ik) {
    const int token = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const float* src;
    if (wave < 4) {
        if (!k) return;
        src = k + ((int64_t)token * kKvHeads + wave) * kDim;
    } else if (wave < 8) {
        if (!v) return;
        src = v + ((int64_t)token * kKvHeads + (wave - 4)) * kDim;
    } else {
        if (!ik) return;
        src = ik + (int64_t)token * kDim;
    }
    // the values and the slot are requested together: one memory round trip before quantizing
    f32x2 x = *reinterpret_cast<const f32x2*>(src + 2 * lane);
    int64_t slot = slots[token];
    asm volatile("" : "+v"(x));
    if (slot < 0) return;
    const int64_t page = slot >> 7;
    const int t = (int)(slot & 127);
    if (page >= num_pages) return;
    uint8_t* dst;
    bool column_layout = false;
    if (wave < 4) {
        dst = k_pool + (page * kKvHeads + wave) * kHeadPageBytes;
    } else if (wave < 8) {
        dst = v_pool + (page * kKvHeads + (wave - 4)) * kHeadPageBytes;
        column_layout = true;
    } else {
        dst = ik_pool + page * kHeadPageBytes;
    }
    uint32_t byte, scale;
    quantize_pair(x[0], x[1], byte, scale);
    const int e = 2 * lane;   // first of the lane's two elements
    const int g = lane >> 3;  // its scale group
    if (!column_layout) {
        dst[row_chunk_offset(t, e >> 5) + ((e & 31) >> 1)] = (uint8_t)byte;
        if ((lane & 7) == 0) dst[row_scale_offset(t, g)] = (uint8_t)scale;
    } else {
        // Each code byte of a V page holds two tokens of one element: replace this token's
        // nibble with an atomic and/or pair so a neighbour token inserted concurrently keeps its
        // nibble.
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

}  // namespace

hipError_t launch_insert(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool, int64_t num_pages,
                         const int64_t* slots, const float* k, const float* v, const float* ik,
                         int n, hipStream_t stream) {
    hipLaunchKernelGGL(insert_kernel, dim3(n), dim3(576), 0, stream, k_pool, v_pool, ik_pool,
                       num_pages, slots, k, v, ik);
    return hipGetLastError();
}

}  // namespace msa
