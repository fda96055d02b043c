// Device-side building blocks of the MSA decode kernels for gfx950 (CDNA4).
//
// Page layouts follow include/msa.h. Matrix-core operand layouts (64-lane wavefront, lane l,
// n = l % 16, c = l / 16), as used throughout:
//   v_mfma_f32_16x16x32_bf16 : A[m][k] in lane (m, c) holds k = 8c..8c+7;  B[k][n] in lane
//                              (n, c) holds k = 8c..8c+7;  D[m][n] in lane (n, c) holds
//                              m = 4c..4c+3.
//   v_mfma_f32_16x16x16_f16  : the same with k = 4c..4c+3.
// The reduction index k may be permuted freely as long as A and B agree; the page layouts
// pick the permutation that makes every operand a single 16-byte load per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kBlock = 128;        // tokens per block / page
constexpr int kDim = 128;          // head dim = index dim
constexpr int kKvHeads = 4;
constexpr int kQHeads = 64;
constexpr int kGroupHeads = 16;
constexpr int kTopk = 16;
constexpr int kCodeBytes = 8192;   // E2M1 codes of one head page
constexpr int kHeadPageBytes = 9216;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- page layouts (msa.h)
// K / index-key pages: 16-byte code chunk (token t, elements 32c..32c+31).
__device__ __forceinline__ int row_chunk_offset(int t, int c) {
    return ((t & 31) >> 2) * 1024 + (16 * c + 4 * (t >> 5) + (t & 3)) * 16;
}
// K / index-key pages: scale byte of (token t, group g).
__device__ __forceinline__ int row_scale_offset(int t, int g) {
    return kCodeBytes + (g >> 1) * 256 + (t >> 5) * 64 + (t & 3) * 16 + ((t & 31) >> 2) * 2 + (g & 1);
}
// V pages: byte holding tokens (t & ~1, t | 1) of element e; scale byte of (token t, group g).
__device__ __forceinline__ int col_code_byte(int e, int t) { return e * 64 + (t >> 1); }
__device__ __forceinline__ int col_scale_offset(int t, int g) { return kCodeBytes + g * 128 + t; }

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 load16(const uint8_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// ---------------------------------------------------------------- NVFP4 dequantization
// Two E4M3 scale bytes (byte pair HI of `w`) -> two fp32 values (exact).
template <bool HI>
__device__ __forceinline__ f32x2 e4m3_pair_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i) times the fp32
// scale s -> eight bf16 values. The conversion instruction yields the unscaled E2M1 value
// exactly (its scale operand only carries a power of two, so 1.0 is passed) and the E4M3
// scale is applied by an fp32 multiply; every product E2M1 x E4M3 is exact in fp32 and in bf16.
__device__ __forceinline__ bf16x8 dequant8_bf16(uint32_t w, float s) {
    const f32x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const f32x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const f32x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const f32x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    bf16x8 r;
    r[0] = (__bf16)(p0[0] * s);
    r[1] = (__bf16)(p0[1] * s);
    r[2] = (__bf16)(p1[0] * s);
    r[3] = (__bf16)(p1[1] * s);
    r[4] = (__bf16)(p2[0] * s);
    r[5] = (__bf16)(p2[1] * s);
    r[6] = (__bf16)(p3[0] * s);
    r[7] = (__bf16)(p3[1] * s);
    return r;
}

// Four E2M1 codes (bytes SEL, SEL+1 of `w`) times four per-code scales, given in fp16 as the
// pairs (s0, s1) and (s2, s3) -> four fp16 values, exact: E2M1 and E4M3 values are exact in fp16
// and so is their product (at most 6 significant bits, magnitude within [2^-10, 2688]). The
// conversion carries a power-of-two scale operand only, so 1.0 is passed and the E4M3 scale is
// applied by one packed fp16 multiply per pair.
template <int SEL>
__device__ __forceinline__ f16x4 dequant4_f16_scaled(uint32_t w, uint32_t s01, uint32_t s23) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL) * __builtin_bit_cast(f16x2, s01);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL + 1) * __builtin_bit_cast(f16x2, s23);
    return f16x4{a[0], a[1], b[0], b[1]};
}

// Eight E2M1 codes (one 32-bit word) times the scale pair {s, s} -> eight fp16 values, exact
// (see dequant4_f16_scaled): the conversion gives the unscaled E2M1 values, one packed fp16
// multiply per pair applies the E4M3 scale.
__device__ __forceinline__ f16x8 dequant8_f16(uint32_t w, f16x2 ss) {
    const f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return f16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Two E4M3 scale bytes (byte pair HI of `w`) -> fp16 pairs {s0, s0} and {s1, s1} (exact).
template <bool HI>
__device__ __forceinline__ void e4m3_pair_f16(uint32_t w, f16x2& s0, f16x2& s1) {
    const f16x2 s = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
    s0 = f16x2{s[0], s[0]};
    s1 = f16x2{s[1], s[1]};
}

// ---------------------------------------------------------------- cross-lane
// Max and sum over the four lanes n, n + 16, n + 32, n + 48 (the four lane groups c of one
// matrix-core row), in every one of them, by the lane swaps of gfx950: v_permlane32_swap gives
// each lane the values of lanes l and l ^ 32, v_permlane16_swap those of l and l ^ 16 (no LDS
// round trip, unlike a shuffle).
__device__ __forceinline__ float max_over_c(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_c(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Query operands in fp16. A query row (one index query, or one attention head) of 128 bf16
// values is spread over the four lanes n, n+16, n+32, n+48 (32 values each, as 4 x bf16x8).
// Multiplying the row by 2^k (k chosen so the row's largest magnitude lands in [2^14, 2^15))
// keeps every value of a usual row exactly representable in fp16; the caller then divides the
// fp32 result by 2^k, which is exact. Returns false on any lane whose values did not convert
// exactly (the caller keeps the bf16 path for that wavefront).
__device__ __forceinline__ bool query_to_f16(const bf16x8 (&qb)[4], f16x8 (&qh)[4], float& inv_scale) {
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
        for (int i = 0; i < 8; i++) mx = fmaxf(mx, fabsf((float)qb[m][i]));
    mx = max_over_c(mx);
    int e = 0;
    if (mx > 0.f) (void)frexpf(mx, &e);  // mx in [2^(e-1), 2^e)
    const int k = 15 - e;
    inv_scale = ldexpf(1.0f, -k);
    // a value converted exactly when its fp16 value widens back to the same bits: the OR of
    // the differences is zero for a row that converts exactly (bitwise vector operations only,
    // no per-value lane-mask updates)
    uint32_t diff = 0;
#pragma unroll
    for (int m = 0; m < 4; m++)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const float f = ldexpf((float)qb[m][i], k);  // exact: no intermediate 2^k
            const _Float16 h = (_Float16)f;
            diff |= __float_as_uint((float)h) ^ __float_as_uint(f);
            qh[m][i] = h;
        }
    asm volatile("" : "+v"(diff));  // keeps the test one comparison (not one per value)
    return inv_scale > 0.f && diff == 0u;  // k beyond the fp32 range: keep the bf16 path
}

// Exact fp16 -> bf16 of eight dequantized values (E2M1 x E4M3 products fit both formats).
__device__ __forceinline__ bf16x8 f16x8_to_bf16x8(const f16x8& h) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; i++) r[i] = (__bf16)(float)h[i];
    return r;
}

// ---------------------------------------------------------------- matrix cores
__device__ __forceinline__ f32x4 mfma_bf16_k32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k32(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k16(const f16x4& a, const f16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- checked build
// Compiled with -DMSA_CHECKED (libmsa_checked.so), the kernels check the values they read from
// device memory against their contract (context lengths, page ids, block ids, slots: every
// build clamps or skips values outside it) and the indexes they compute against the extents of
// their arguments. A failed check adds 1 to this file's device counter and lowers its lowest
// failing site (the site codes of include/msa_debug.h); the kernel goes on. msa_debug_checks
// reads and resets the counters of every file. In the normal build a check compiles to nothing.
#ifdef MSA_CHECKED
static __device__ uint32_t g_checks[2] = {0u, 0xFFFFFFFFu};  // failures, lowest failing site
__device__ __forceinline__ void check_site(bool ok, uint32_t site) {
    if (!ok) {
        atomicAdd(&g_checks[0], 1u);
        atomicMin(&g_checks[1], site);
    }
}
#define MSA_CHECK(ok, site) ::msa::check_site((ok), (site))
// The host reader of this file's counters (one per .hip file with kernels): adds the failures
// to *count, lowers *site, and resets both.
#define MSA_DEFINE_CHECKS_READER(NAME)                                                   \
    hipError_t NAME(uint32_t* count, uint32_t* site) {                                   \
        uint32_t v[2];                                                                   \
        hipError_t e = hipMemcpyFromSymbol(v, HIP_SYMBOL(g_checks), sizeof(v), 0,        \
                                           hipMemcpyDeviceToHost);                       \
        if (e != hipSuccess) return e;                                                   \
        *count += v[0];                                                                  \
        if (v[1] < *site) *site = v[1];                                                  \
        const uint32_t init[2] = {0u, 0xFFFFFFFFu};                                      \
        return hipMemcpyToSymbol(HIP_SYMBOL(g_checks), init, sizeof(init), 0,            \
                                 hipMemcpyHostToDevice);                                 \
    }
#else
#define MSA_CHECK(ok, site) ((void)0)
#endif

// Check sites (the codes of include/msa_debug.h): a value read from device memory outside its
// contract, then invariants of the kernels' own index arithmetic.
constexpr uint32_t kCheckCtxLen = 1;       // a context length outside q_len .. max_blocks * 128
constexpr uint32_t kCheckSelection = 101;  // a selection not ascending, not within the eligible
                                           // blocks, or without the block of the query token
constexpr uint32_t kCheckWorkspace = 102;  // a split partial or counter past the call's workspace
constexpr uint32_t kCheckLds = 103;        // an LDS list or table index past its array
constexpr uint32_t kCheckOutput = 104;     // a score, id, cache or output index past its array

__device__ __forceinline__ int clamp_ctx(int T, int max_blocks) {
    const int cap = max_blocks * kBlock;
    return T < 0 ? 0 : (T > cap ? cap : T);
}

}  // namespace msa
