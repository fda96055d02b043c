// Block selection of one (sequence, query token, group) row by one 64-lane wavefront, shared by
// the selection kernel and the fused selection + attention kernel.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": the 16 best blocks are
// kept and the most recent block always stays (at most 2,048 keys). "MiniMax M3 on vLLM",
// section "MSA mechanism": local_blocks = 1, init_blocks = 0, the local block is not counted
// twice. Ties go to the lower block index.
//
// The row's scores become order-preserving integer keys in registers (block i in lane i % 64,
// slot i / 64). The 15th-largest of the 64 per-lane maxima is a lower bound of the 15th-largest
// key (at least 15 keys reach it), so the selection lies among the keys at or above it. It is
// found without a serial search: every lane counts the maxima above its own (all 64 read back
// from LDS as broadcasts), and the bound is the smallest maximum that fewer than 15 others
// exceed. The few candidates are compacted into LDS in ascending block order as (key, inverted
// block index) composites, without branches, and each is ranked exactly against the others by
// reading them back as LDS broadcasts; the 15 best, already in ascending block order, are written
// with the forced block last. When more than 64 candidates reach the bound (heavy ties), the
// wavefront extracts the 15 best one by one instead.
#pragma once

#include "device_common.hpp"

namespace msa {

// LDS entries (8 bytes) per wavefront: candidates [0, 64), writes of non-candidates [64, 128),
// the 64 lane maxima as 4-byte words [128, 160).
constexpr int kSelectScratch = 160;

// Order-preserving map of a non-NaN float to uint32 (larger float -> larger key); -0 == +0
// (adding +0 turns -0 into +0).
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f + 0.0f);
    return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
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

// if_set in the lanes whose bit of mask is set, if_clear elsewhere: the lane mask (a scalar
// register pair) selects directly. The two wait states cover a mask just written by a compare.
__device__ __forceinline__ uint32_t select_by_mask(uint64_t mask, uint32_t if_set, uint32_t if_clear) {
    uint32_t r;
    asm("s_nop 1\n\tv_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(if_clear), "v"(if_set), "s"(mask));
    return r;
}

// acc plus the number of the four values above x: four compares into scalar register pairs, then
// four carry additions (each compare's result is read three instructions after it is written).
__device__ __forceinline__ int add_count_above(const u32x4& w, uint32_t x, int acc) {
    uint64_t c0, c1, c2, c3, dummy;
    asm("v_cmp_gt_u32_e64 %1, %6, %10\n\t"
        "v_cmp_gt_u32_e64 %2, %7, %10\n\t"
        "v_cmp_gt_u32_e64 %3, %8, %10\n\t"
        "v_cmp_gt_u32_e64 %4, %9, %10\n\t"
        "v_addc_co_u32_e64 %0, %5, %0, 0, %1\n\t"
        "v_addc_co_u32_e64 %0, %5, %0, 0, %2\n\t"
        "v_addc_co_u32_e64 %0, %5, %0, 0, %3\n\t"
        "v_addc_co_u32_e64 %0, %5, %0, 0, %4"
        : "+v"(acc), "=&s"(c0), "=&s"(c1), "=&s"(c2), "=&s"(c3), "=&s"(dummy)
        : "v"(w[0]), "v"(w[1]), "v"(w[2]), "v"(w[3]), "v"(x));
    return acc;
}

// Minimum over the wavefront's 64 lanes, in every lane of the last row (lane 63 is read):
// within each row of 16 by quad swaps and mirrors, then across rows by the row broadcasts.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));  // row 0 -> 1, 2 -> 3
    v = min(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));  // row 1 -> 2, 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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
    const uint8_t* row = reinterpret_cast<const uint8_t*>(s);  // 32-bit byte offsets from it
#pragma unroll
    for (int k = 0; k < KPL; k++)
        v[k] = *reinterpret_cast<const float*>(row + 4u * (uint32_t)min(lane + 64 * k, max_blocks - 1));
}

// Select the `pick` best of a row's keys (position i in lane i % 64, slot i / 64; key 0 marks
// "no candidate"; a larger key ranks first, equal keys by the lower position) and write
// id_of(position) for each in ascending position order to out[0..pick-1], and their keys to
// key_out when it is given. With fewer than `pick` candidates the remaining entries are -1
// (keys 0). 0 <= pick <= 64, wavefront-uniform (a constant where the caller has one). `cand` is
// this wavefront's kSelectScratch entries of LDS; `out` and `key_out` may point to global
// memory or LDS.
template <int KPL, class IdOf>
__device__ __forceinline__ void select_top(const uint32_t (&key)[KPL], int lane, uint64_t* cand,
                                           int32_t* out, uint32_t* key_out, IdOf id_of, int pick) {
    uint32_t lmax = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) lmax = max(lmax, key[k]);
    // bound: the pick-th largest per-lane maximum, the smallest maximum that fewer than `pick`
    // others exceed (each lane counts the maxima above its own, read back as LDS broadcasts),
    // and at least 1 (never a non-candidate). The candidate area is cleared in the same pass:
    // entries past the candidate count read as 0, below every candidate.
    uint32_t* lane_max = reinterpret_cast<uint32_t*>(cand + 128);
    lane_max[lane] = lmax;
    cand[lane] = 0;
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");  // the reads below follow these stores
    u32x4 w[16];
#pragma unroll
    for (int r = 0; r < 16; r++) w[r] = reinterpret_cast<const u32x4*>(lane_max)[r];
    int above = 0;
#pragma unroll
    for (int r = 0; r < 16; r++) above = add_count_above(w[r], lmax, above);
    const uint32_t bound = max(wave_min_u32(above < pick ? lmax : 0xFFFFFFFFu), 1u);
    // candidates: the keys at or above the bound (all slots' masks first, then their counts)
    uint64_t cmask[KPL];
#pragma unroll
    for (int k = 0; k < KPL; k++) cmask[k] = ge_mask(key[k], bound);
    int base[KPL + 1];
    base[0] = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) base[k + 1] = base[k] + popc64(cmask[k]);
    const int count = __builtin_amdgcn_readfirstlane(base[KPL]);  // uniform: a scalar loop bound
    int n_sel;
    if (count <= 64) {
        // compact the candidates in ascending block order (k-major, lane-minor) as composites
        // (key, inverted block index): a larger composite ranks first, and equal keys rank by
        // the lower block. Every lane stores; a non-candidate's store goes to its own entry of
        // the discard area.
        const uint32_t inv_lane = ~(uint32_t)lane;
#pragma unroll
        for (int k = 0; k < KPL; k++) {
            const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(cmask[k] >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)cmask[k], base[k]));
            cand[select_by_mask(cmask[k], pos, 64 + lane)] =
                ((uint64_t)key[k] << 32) | (inv_lane - 64u * k);
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // candidate t of lane t counts the candidates ranked before it, reading them eight at a
        // time as LDS broadcasts (the cleared entries past the count never rank before it)
        const uint64_t mine = cand[lane];
        int rank = 0;
        for (int t0 = 0; t0 < count; t0 += 8) {
            uint64_t o[8];
#pragma unroll
            for (int i = 0; i < 8; i++) o[i] = cand[t0 + i];
#pragma unroll
            for (int i = 0; i < 8; i++) rank += (int)(o[i] > mine);
        }
        const bool sel = lane < count && rank < pick;
        const uint64_t smask = __ballot(sel);
        if (sel) {
            const int at = lanes_before(smask);
            out[at] = id_of((int)~(uint32_t)mine);
            if (key_out) key_out[at] = (uint32_t)(mine >> 32);
        }
        n_sel = popc64(smask);
    } else {
        // heavy ties: take the best remaining (key, lowest index) `pick` times
        uint32_t taken[(KPL + 31) / 32] = {};
        for (int r = 0; r < pick; r++) {
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
            if (bk != 0u && (bi & 63) == lane) {  // (more than 64 candidates: never empty)
                const int k = bi >> 6;
                taken[k >> 5] |= 1u << (k & 31);
            }
        }
        int at = 0;
#pragma unroll
        for (int k = 0; k < KPL; k++) {
            const bool sel = (taken[k >> 5] >> (k & 31)) & 1u;
            const uint64_t mask = __ballot(sel);
            if (sel) {
                out[at + lanes_before(mask)] = id_of(lane + 64 * k);
                if (key_out) key_out[at + lanes_before(mask)] = key[k];
            }
            at += popc64(mask);
        }
        n_sel = at;
    }
    if (lane >= n_sel && lane < pick) {
        out[lane] = -1;
        if (key_out) key_out[lane] = 0u;
    }
}

// select_top for picks above 16 (the window knobs' top-k up to 64), where the lane-maxima bound
// would leave far more than 64 candidates: t, the pick-th largest key (counted with
// multiplicity, the zero keys of non-candidates included), is found one byte at a time from the
// top: a 256-bin histogram in LDS (`hist`, 256 words of this wavefront's scratch) of the next
// byte of the keys that share the bytes found so far, then the bin in which the pick-th largest
// lies. Every key above t and the first keys equal to t in position order (equal keys rank by
// the lower position) are then written in ascending position order; t = 0 (fewer than `pick`
// candidates) takes every candidate. The same contract as select_top.
static_assert(kSelectScratch * 8 >= 256 * 4, "the byte histogram fits a wavefront's scratch");
template <int KPL, class IdOf>
__device__ __forceinline__ void select_top_radix(const uint32_t (&key)[KPL], int lane,
                                                 uint32_t* hist, int32_t* out, uint32_t* key_out,
                                                 IdOf id_of, int pick) {
    uint32_t t = 0, known = 0;  // the bytes of t found so far, and their mask
    int need = pick;            // rank of t among the keys that share those bytes
#pragma unroll
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; i++) hist[lane + 64 * i] = 0u;
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < KPL; k++)
            if ((key[k] & known) == t) atomicAdd(&hist[(key[k] >> shift) & 0xFFu], 1u);
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // lane l holds bins 4l .. 4l + 3; keys in the bins of higher lanes come first
        uint32_t cb[4];
#pragma unroll
        for (int i = 0; i < 4; i++) cb[i] = hist[4 * lane + i];
        const int own = (int)(cb[0] + cb[1] + cb[2] + cb[3]);
        int incl = own;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_down(incl, d, 64);
            if (lane + d < 64) incl += y;
        }
        int cum = incl - own;  // keys in higher bins
        int found = -1, rest = 0;
#pragma unroll
        for (int i = 3; i >= 0; i--) {
            if (cum < need && cum + (int)cb[i] >= need) {
                found = 4 * lane + i;
                rest = need - cum;
            }
            cum += (int)cb[i];
        }
        // exactly one lane holds the bin (the keys that share the bytes found so far number at
        // least `need`)
        const int src = __builtin_ctzll(__ballot(found >= 0));
        t |= (uint32_t)__builtin_amdgcn_readlane(found, src) << shift;
        need = __builtin_amdgcn_readlane(rest, src);
        known |= 0xFFu << shift;
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
    }
    int above = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) above += popc64(__ballot(key[k] > t));
    int take_eq = t == 0u ? 0 : pick - above;  // keys equal to t still to take (none: t = 0)
    int at = 0;
#pragma unroll
    for (int k = 0; k < KPL; k++) {
        const bool eq = t != 0u && key[k] == t;
        const uint64_t eqm = __ballot(eq);
        const bool sel = key[k] > t || (eq && lanes_before(eqm) < take_eq);
        const uint64_t sm = __ballot(sel);
        if (sel) {
            out[at + lanes_before(sm)] = id_of(lane + 64 * k);
            if (key_out) key_out[at + lanes_before(sm)] = key[k];
        }
        at += popc64(sm);
        take_eq -= min(take_eq, popc64(eqm));
    }
    if (lane >= at && lane < pick) {
        out[lane] = -1;
        if (key_out) key_out[lane] = 0u;
    }
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
    uint32_t key[KPL];    // 0 marks "no candidate": every real key is above it
#pragma unroll
    for (int k = 0; k < KPL; k++) {
        const int i = lane + 64 * k;
        key[k] = i < m ? order_key(v[k]) : 0u;
    }
    select_top<KPL>(key, lane, cand, out, nullptr, [](int i) { return i; }, kTopk - 1);
    if (lane == 0) out[kTopk - 1] = m;  // the forced block of the query token, the largest id
}

// The selection with the window knobs ("MiniMax M3 on vLLM", section "MSA mechanism": init
// blocks and local blocks): of the row's n eligible blocks the first `init` and the last
// `local` are kept, and the best others fill the rest of the `topk` places; out[0..topk-1]
// gets the ids in ascending order, padded with -1. init + local <= topk <= 64.
template <int KPL>
__device__ __forceinline__ void select_row_window(const float (&v)[KPL], int n, int lane,
                                                  uint64_t* cand, int32_t* out, int topk,
                                                  int init, int local) {
    if (n <= topk) {
        if (lane < topk) out[lane] = lane < n ? lane : -1;
        return;
    }
    const int lo = min(init, n);              // blocks 0..lo-1: forced
    const int hi = max(n - local, lo);        // blocks hi..n-1: forced
    uint32_t key[KPL];
#pragma unroll
    for (int k = 0; k < KPL; k++) {
        const int i = lane + 64 * k;
        key[k] = (i >= lo && i < hi) ? order_key(v[k]) : 0u;
    }
    // the picks lie between the two forced ranges, so the ascending order is kept
    const int pick = topk - lo - (n - hi);
    if (pick > kTopk)
        select_top_radix<KPL>(key, lane, reinterpret_cast<uint32_t*>(cand), out + lo, nullptr,
                              [](int i) { return i; }, pick);
    else
        select_top<KPL>(key, lane, cand, out + lo, nullptr, [](int i) { return i; }, pick);
    if (lane < lo) out[lane] = lane;
    if (lane < n - hi) out[topk - (n - hi) + lane] = hi + lane;
}

}  // namespace msa
