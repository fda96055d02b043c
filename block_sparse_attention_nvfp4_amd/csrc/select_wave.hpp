// Block selection of one (sequence, query token, group) row by one 64-lane wavefront, shared by
// the selection kernel and the fused selection + attention kernel.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": the 16 best blocks are
// kept and the most recent block always stays (at most 2,048 keys). "MiniMax M3 on vLLM",
// section "MSA mechanism": local_blocks = 1, init_blocks = 0, the local block is not counted
// twice. Ties go to the lower block index.
//
// The row's scores become order-preserving integer keys in registers (block i in lane i % 64,
// slot i / 64). The 15th-largest of the 64 per-lane maxima, found by a bitwise search with
// ballot counts (two bits per step), is a lower bound of the 15th-largest key (at least 15 keys
// reach it), so the selection lies among the keys at or above it. Those few candidates are
// compacted into LDS in ascending block order as (key, inverted block index) composites and each
// is ranked exactly against the others by reading them back as LDS broadcasts; the 15 best,
// already in ascending block order, are written with the forced block last. When more than 64
// candidates reach the bound (heavy ties), the wavefront extracts the 15 best one by one instead.
#pragma once

#include "device_common.hpp"

namespace msa {

constexpr int kSelectScratch = 64;  // LDS entries per wavefront: up to 64 candidates

// Order-preserving map of a non-NaN float to uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Population count of a lane mask as two 32-bit counts: the result stays a 32-bit scalar, so
// comparisons of it are scalar instructions (a 64-bit count is compared on the vector unit).
__device__ __forceinline__ int popc64(uint64_t x) {
    return (int)(__builtin_popcount((uint32_t)x) + __builtin_popcount((uint32_t)(x >> 32)));
}

// Lane mask of x >= c, written to a scalar register pair by an explicit compare: several such
// compares issue back to back, and the scalar unit then waits once for all of their results
// (through the condition register the compiler would chain them, one wait each).
__device__ __forceinline__ uint64_t ge_mask(uint32_t x, uint32_t c) {
    uint64_t m;
    asm("v_cmp_le_u32_e64 %0, %1, %2" : "=s"(m) : "s"(c), "v"(x));
    return m;
}

// Number of lanes before this one whose bit is set.
__device__ __forceinline__ int lanes_before(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// Eligible blocks of a query token at position p (blocks 0..n-1; the last one, n - 1, holds the
// token and is forced); 0 when the token has no position.
__device__ __forceinline__ int eligible_blocks(int p, int max_blocks) {
    return p < 0 ? 0 : min(p / kBlock + 1, max_blocks);
}

// Scores of blocks lane + 64 k of a row: every load is issued before any is used (an index past
// the row reads its last score, which the selection ignores).
template <int KPL>
__device__ __forceinline__ void load_row_scores(const float* s, int max_blocks, int lane,
                                                float (&v)[KPL]) {
#pragma unroll
    for (int k = 0; k < KPL; k++) v[k] = s[min(lane + 64 * k, max_blocks - 1)];
}

// Select the row's blocks from its scores v (as load_row_scores holds them) and its n eligible
// blocks: out[0..15] gets the selected block ids in ascending order, padded with -1. `cand` is
// this wavefront's kSelectScratch entries of LDS; `out` may point to global memory or LDS.
template <int KPL>
__device__ __forceinline__ void select_row(const float (&v)[KPL], int n, int lane, uint64_t* cand,
                                           int32_t* out) {
    if (n <= kTopk) {
        if (lane < kTopk) out[lane] = lane < n ? lane : -1;
        return;
    }
    const int m = n - 1;  // candidates 0..m-1 compete for 15 places
    uint32_t key[KPL];  // 0 marks "no candidate": every real key is above it
    uint32_t lmax = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) {
        const int i = lane + 64 * k;
        key[k] = i < m ? order_key(v[k]) : 0u;
        lmax = max(lmax, key[k]);
    }
    // bound: the 15th-largest per-lane maximum (bitwise search, most significant bits first, two
    // bits per step: the three candidate values of a step are tested by independent ballots, and
    // the count of maxima at or above a value falls as the value grows)
    uint32_t bound = 0;
#pragma unroll
    for (int bit = 30; bit >= 0; bit -= 2) {
        const uint32_t c3 = bound | (3u << bit), c2 = bound | (2u << bit), c1 = bound | (1u << bit);
        const uint64_t m3 = ge_mask(lmax, c3), m2 = ge_mask(lmax, c2), m1 = ge_mask(lmax, c1);
        const int n3 = popc64(m3), n2 = popc64(m2), n1 = popc64(m1);
        bound = n3 >= kTopk - 1 ? c3 : (n2 >= kTopk - 1 ? c2 : (n1 >= kTopk - 1 ? c1 : bound));
    }
    // candidates: the keys at or above the bound (all slots' masks first, then their counts)
    uint64_t cmask[KPL];
#pragma unroll
    for (int k = 0; k < KPL; k++) cmask[k] = ge_mask(key[k], bound);
    int base[KPL + 1];
    base[0] = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) base[k + 1] = base[k] + popc64(cmask[k]);
    const int count = base[KPL];
    if (count <= 64) {
        // compact the candidates in ascending block order (k-major, lane-minor) as composites
        // (key, inverted block index): a larger composite ranks first, and equal keys rank by
        // the lower block; only candidate lanes store
#pragma unroll
        for (int k = 0; k < KPL; k++) {
            if (key[k] >= bound)
                cand[base[k] + lanes_before(cmask[k])] =
                    ((uint64_t)key[k] << 32) | (uint32_t)~(uint32_t)(lane + 64 * k);
        }
        __builtin_amdgcn_wave_barrier();
        // candidate t of lane t counts the candidates ranked before it, reading them eight at a
        // time as LDS broadcasts
        const uint64_t mine = lane < count ? cand[lane] : 0u;
        int rank = 0;
        for (int t0 = 0; t0 < count; t0 += 8) {
            uint64_t o[8];
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = cand[t0 + i];
#pragma unroll
            for (int i = 0; i < 8; i++) rank += (t0 + i < count) && o[i] > mine;
        }
        const bool sel = lane < count && rank < kTopk - 1;
        const uint64_t smask = __ballot(sel);
        if (sel) out[lanes_before(smask)] = (int)~(uint32_t)mine;
    } else {
        // heavy ties: take the best remaining (key, lowest index) 15 times
        uint32_t taken[(KPL + 31) / 32] = {};
        for (int r = 0; r < kTopk - 1; r++) {
            uint32_t bk = 0;
            int bi = 0x7fffffff;
#pragma unroll
            for (int k = 0; k < KPL; k++) {
                const int i = lane + 64 * k;
                const bool avail = !((taken[k >> 5] >> (k & 31)) & 1u) && key[k] != 0u;
                if (avail && (key[k] > bk || (key[k] == bk && i < bi))) {
                    bk = key[k];
                    bi = i;
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const uint32_t ok = __shfl_xor(bk, d, 64);
                const int oi = __shfl_xor(bi, d, 64);
                if (ok > bk || (ok == bk && oi < bi)) {
                    bk = ok;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) {
                const int k = bi >> 6;
                taken[k >> 5] |= 1u << (k & 31);
            }
        }
        int base = 0;
#pragma unroll
        for (int k = 0; k < KPL; k++) {
            const bool sel = (taken[k >> 5] >> (k & 31)) & 1u;
            const uint64_t mask = __ballot(sel);
            if (sel) out[base + lanes_before(mask)] = lane + 64 * k;
            base += popc64(mask);
        }
    }
    if (lane == 0) out[kTopk - 1] = m;  // the forced block of the query token, the largest id
}

}  // namespace msa
