// MSA sparse GQA attention over the selected blocks, split over workgroups, with an
// online-softmax merge of the partial results.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer" and its Figure 1: every
// query head of a GQA group attends exactly, but only to the blocks its group's indexer kept;
// section "NVFP4 MSA kernel": the kernel reads the NVFP4 pages directly and dequantizes them
// on the fly. "MiniMax M3 on vLLM", section "MiniMax sparse attention backend": the decode GQA
// kernel consumes the selected block pages and merges partial attention outputs; section
// "Prefill execution": the result equals dense attention restricted to the selected set.
//
// Work: a row group is (sequence b, query token j, KV group g) = 16 query heads with its 16
// selected blocks. Each workgroup (4 wavefronts) takes 16 / n_split of them; each wavefront
// streams whole blocks: the K and V pages of a block are copied into the wavefront's LDS
// buffer with direct global->LDS loads (the next block's while the current one computes).
// Per block and wavefront (lane l, n = l % 16, c = l / 16):
//   S^T = K Q^T on the matrix cores (A = keys dequantized exactly to fp16, B = the 16 heads as
//   fp16 after a per-head power-of-two scaling, or bf16 when a head does not convert exactly),
//   so lane (n, c) holds the logits of head n for tokens 32c + 4s + i (slab s, i = 0..3);
//   fp32 online softmax per head, probabilities in fp16;
//   O^T += V^T P^T on fp16 matrix cores: P^T in the same lanes is already the B operand and V^T
//   (A operand, dims x tokens) is the exact fp16 dequantization of the column-layout V page.
// The wavefronts merge through LDS. With one split the workgroup writes the bf16 output;
// otherwise each wavefront writes the fp32 partial (max, sum, output) of four heads with
// agent-coherent stores and counts itself finished on their counter; the wavefront that
// finishes last reads the other splits' partials, merges them by log-sum-exp and writes the
// output, so no second launch (and no second kernel boundary) is needed. Workgroup ids map all work of one (sequence, group) pair
// to one XCD, so the blocks that the query tokens of a pair share are read from HBM once and
// then hit that XCD's L2.
#include "device_common.hpp"
#include "kernels.hpp"
#include "select_wave.hpp"

namespace msa {
namespace {

constexpr int kWaves = 4;
constexpr int kPartStride = 132;  // floats per (row group, split, head): m, l, 2 pad, 128 out
constexpr int kMaxSplits = 4;     // attn_num_splits returns 1, 2 or 4
constexpr int kBlockBytes = 2 * kHeadPageBytes;  // K page then V page of one (block, group)
constexpr int kMergeStride = kDim + 4;           // LDS row of the wavefront merge
// Cache policy of the page loads: the default (0). The query tokens of one (sequence, group)
// pair read mostly the same blocks on the same XCD, and the later reads hit its L2; the
// non-temporal hint measured 0.25 us slower.
constexpr int kPagePolicy = 0;
// Lazy rescaling: a row keeps its running maximum until a block's maximum exceeds it by more
// than this (log2 units); probabilities then stay below 2^kTau, well inside fp16, and the
// accumulators are rescaled only when the maximum jumps.
constexpr float kTau = 8.0f;

// 2^x by the hardware instruction (results below 2^-126 flush to zero, which a softmax weight
// next to a weight of at least 1 cannot notice).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ uint16_t bf16_bits_rne(float x) {
    const __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

// A mask of the first n bytes of a 32-bit word (all four for n >= 4, none for n <= 0): applied to
// four consecutive E4M3 scale bytes, it zeroes the scales of the tokens past the last valid one.
__device__ __forceinline__ uint32_t keep_bytes(int n) {
    return n >= 4 ? 0xFFFFFFFFu : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
}

// Copy the K and V pages of one (block, group) into an LDS buffer: 18 direct 16-byte loads.
__device__ __forceinline__ void block_to_lds(const uint8_t* kp, const uint8_t* vp, uint8_t* buf,
                                             int lane) {
#pragma unroll
    for (int s = 0; s < 9; s++)
        __builtin_amdgcn_global_load_lds(kp + s * 1024 + lane * 16, (lds_void*)(buf + s * 1024), 16,
                                         0, kPagePolicy);
#pragma unroll
    for (int s = 0; s < 9; s++)
        __builtin_amdgcn_global_load_lds(vp + s * 1024 + lane * 16,
                                         (lds_void*)(buf + kHeadPageBytes + s * 1024), 16, 0,
                                         kPagePolicy);
}

// Agent-coherent 16-byte store and load (cache policy sc1): written through to, and read from,
// the point where every XCD sees the same data, without flushing or invalidating the whole L2
// as a device-scope fence would. Used only for the split partials that one workgroup hands to
// another within a launch.
__device__ __forceinline__ void store16_coherent(float* p, const f32x4& v) {
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(p), "v"(v) : "memory");
}
// The three agent-coherent 16-byte loads of each of kMaxSplits partials, all in flight
// together and waited for within the one asm statement.
__device__ __forceinline__ void load_partials_coherent(const float* const (&p)[4][3],
                                                       f32x4 (&v)[4][3]) {
    asm volatile(
        "global_load_dwordx4 %0, %12, off sc1\n\t"
        "global_load_dwordx4 %1, %13, off sc1\n\t"
        "global_load_dwordx4 %2, %14, off sc1\n\t"
        "global_load_dwordx4 %3, %15, off sc1\n\t"
        "global_load_dwordx4 %4, %16, off sc1\n\t"
        "global_load_dwordx4 %5, %17, off sc1\n\t"
        "global_load_dwordx4 %6, %18, off sc1\n\t"
        "global_load_dwordx4 %7, %19, off sc1\n\t"
        "global_load_dwordx4 %8, %20, off sc1\n\t"
        "global_load_dwordx4 %9, %21, off sc1\n\t"
        "global_load_dwordx4 %10, %22, off sc1\n\t"
        "global_load_dwordx4 %11, %23, off sc1\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0][0]), "=&v"(v[0][1]), "=&v"(v[0][2]), "=&v"(v[1][0]), "=&v"(v[1][1]),
          "=&v"(v[1][2]), "=&v"(v[2][0]), "=&v"(v[2][1]), "=&v"(v[2][2]), "=&v"(v[3][0]),
          "=&v"(v[3][1]), "=&v"(v[3][2])
        : "v"(p[0][0]), "v"(p[0][1]), "v"(p[0][2]), "v"(p[1][0]), "v"(p[1][1]), "v"(p[1][2]),
          "v"(p[2][0]), "v"(p[2][1]), "v"(p[2][2]), "v"(p[3][0]), "v"(p[3][1]), "v"(p[3][2])
        : "memory");
}

// LDS reads as explicit instructions (the compiler would otherwise wait for every page load in
// flight before any LDS read), each group issued and waited for within one asm statement: no
// register written by a read the compiler does not see is live outside it, so the compiler can
// never copy one before its data has arrived.
__device__ __forceinline__ void lds_read16x9(u32x4 (&v)[8], u32x4& w, uint32_t a, uint32_t aw) {
    asm volatile("ds_read_b128 %0, %9\n\t"
                 "ds_read_b128 %1, %9 offset:1024\n\t"
                 "ds_read_b128 %2, %9 offset:2048\n\t"
                 "ds_read_b128 %3, %9 offset:3072\n\t"
                 "ds_read_b128 %4, %9 offset:4096\n\t"
                 "ds_read_b128 %5, %9 offset:5120\n\t"
                 "ds_read_b128 %6, %9 offset:6144\n\t"
                 "ds_read_b128 %7, %9 offset:7168\n\t"
                 "ds_read_b128 %8, %10\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
                   "=&v"(v[6]), "=&v"(v[7]), "=&v"(w)
                 : "v"(a), "v"(aw)
                 : "memory");
}
__device__ __forceinline__ void lds_read16x5(u32x4& v, u32x4 (&w)[4], uint32_t a, uint32_t aw) {
    asm volatile("ds_read_b128 %0, %5\n\t"
                 "ds_read_b128 %1, %6\n\t"
                 "ds_read_b128 %2, %6 offset:16\n\t"
                 "ds_read_b128 %3, %6 offset:32\n\t"
                 "ds_read_b128 %4, %6 offset:48\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v), "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
                 : "v"(a), "v"(aw)
                 : "memory");
}
__device__ __forceinline__ u32x4 lds_read16(uint32_t a) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(a) : "memory");
    return v;
}
// Two 16-byte LDS writes, complete when the statement ends (reads that follow see them).
__device__ __forceinline__ void lds_write32(uint32_t a, const u32x4& v0, const u32x4& v1) {
    asm volatile("ds_write_b128 %0, %1\n\t"
                 "ds_write_b128 %0, %2 offset:16\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 :: "v"(a), "v"(v0), "v"(v1)
                 : "memory");
}

// A block's logits sv (lane (n, c): head n, tokens tok0 + 32c + 4s + i, unscaled) -> tokens past
// the query position masked, the online-softmax state (m_run, l_run, o) updated, and the
// block's probabilities in fp16, slabs 2h and 2h + 1 in pt[h] (the B operand of one 32-token
// step of O^T += V^T P^T).
__device__ __forceinline__ void softmax_block(f32x4 (&sv)[8], int c, int tok0, int p,
                                              float logit_scale, float& m_run, float& l_run,
                                              f32x4 (&o)[8], f16x8 (&pt)[4]) {
    // tokens past the query position: only in the block that holds it, a scalar branch that
    // every other block skips (kept a branch: folded into the selects, the wavefront-uniform
    // condition cost a vector-to-scalar round trip per value)
    if (tok0 + kBlock - 1 > p) {
        asm volatile("");
        const int last = p - tok0 - 32 * c;  // values 4s + i <= last are visible
#pragma unroll
        for (int s = 0; s < 8; s++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // all ones past the position: vector bit operations, no lane-mask updates
                uint32_t past = (uint32_t)((last - (4 * s + i)) >> 31);
                asm("" : "+v"(past));
                sv[s][i] = __uint_as_float((__float_as_uint(sv[s][i]) & ~past) | (0xFF800000u & past));
            }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
        for (int i = 0; i < 4; i++) mb = fmaxf(mb, sv[s][i]);
    mb = max_over_c(mb) * logit_scale;  // finite (token tok0 <= p is valid); scaling keeps order
    const float m_new = (mb > m_run + kTau) ? mb : m_run;  // m_run = -inf -> m_new = mb
    if (__any(m_new != m_run)) {
        const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf (o, l are 0)
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
        m_run = m_new;
    }
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float e = fast_exp2(fmaf(sv[s][i], logit_scale, -m_new));
            pt[s >> 1][4 * (s & 1) + i] = (_Float16)e;
        }
    // (the block's sum of these probabilities is added to l_run by the caller, on the matrix
    // cores, from the same fp16 values the output uses)
}

// One block of one wavefront: logits, online-softmax update, output accumulation. The K page
// is in LDS on entry; the V page may still be arriving (NEXT: the next block's 18 loads were
// issued after it) and is waited for only before its first read. (The softmax step is written
// out here rather than calling softmax_block: the shared helper changed this kernel's register
// allocation, 48 more accumulator-register reads per block.)
template <bool F16, bool NEXT>
__device__ __forceinline__ void attend_block(const uint8_t* buf, int lane, int c, int tok0, int p,
                                             const u32x4 (&qop)[4], float logit_scale,
                                             float& m_run, float& l_run, f32x4 (&o)[8]) {
    const uint32_t kbase = (uint32_t)(uintptr_t)buf;
    const uint32_t vbase = kbase + kHeadPageBytes;
    // ---- logits S^T (log2 domain)
    u32x4 kc[8], ksc;
    lds_read16x9(kc, ksc, kbase + lane * 16, kbase + kCodeBytes + lane * 16);
    f32x4 sv[8];
#pragma unroll
    for (int s = 0; s < 8; s++) {
        const u32x4 code = kc[s];
        f16x2 s0, s1;
        if (s & 1) e4m3_pair_f16<true>(ksc[s >> 1], s0, s1);
        else e4m3_pair_f16<false>(ksc[s >> 1], s0, s1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const f16x8 a = dequant8_f16(code[m], m < 2 ? s0 : s1);
            if constexpr (F16)
                acc = mfma_f16_k32(a, __builtin_bit_cast(f16x8, qop[m]), acc);
            else
                acc = mfma_bf16_k32(f16x8_to_bf16x8(a), __builtin_bit_cast(bf16x8, qop[m]), acc);
        }
        sv[s] = acc;  // unscaled: the scale (> 0) is applied inside the exponent below
    }
    // tokens past the query position: only in the block that holds it, a scalar branch that
    // every other block skips (kept a branch: folded into the selects, the wavefront-uniform
    // condition cost a vector-to-scalar round trip per value)
    if (tok0 + kBlock - 1 > p) {
        asm volatile("");
        const int last = p - tok0 - 32 * c;  // values 4s + i <= last are visible
#pragma unroll
        for (int s = 0; s < 8; s++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                // all ones past the position: vector bit operations, no lane-mask updates
                uint32_t past = (uint32_t)((last - (4 * s + i)) >> 31);
                asm("" : "+v"(past));
                sv[s][i] = __uint_as_float((__float_as_uint(sv[s][i]) & ~past) | (0xFF800000u & past));
            }
    }
    float mb = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
        for (int i = 0; i < 4; i++) mb = fmaxf(mb, sv[s][i]);
    mb = max_over_c(mb) * logit_scale;  // finite (token tok0 <= p is valid); scaling keeps order
    const float m_new = (mb > m_run + kTau) ? mb : m_run;  // m_run = -inf -> m_new = mb
    if (__any(m_new != m_run)) {
        const float alpha = fast_exp2(m_run - m_new);  // 0 when m_run = -inf (o, l are 0)
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
        m_run = m_new;
    }
    f16x4 pt[8];
#pragma unroll
    for (int s = 0; s < 8; s++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const float e = fast_exp2(fmaf(sv[s][i], logit_scale, -m_new));
            pt[s][i] = (_Float16)e;
        }

    // ---- the V page's 9 loads (issued after the K page's 9) complete here
    if constexpr (NEXT) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // ---- the block's 1,024 V scales as fp16, [group][token], written over the K codes (read
    // into registers above and not needed again): lane l converts the 16 scale bytes of group
    // l / 8, tokens 16 (l % 8) .. +15. Each lane then reads its scales ready for the packed
    // multiply instead of converting 256 of them.
    {
        // (with no later page in flight, ordinary LDS reads: the compiler overlaps them with
        // the work before their use; otherwise statements that wait for their own reads only)
        u32x4 raw;
        if constexpr (NEXT) raw = lds_read16(vbase + kCodeBytes + lane * 16);
        else raw = *reinterpret_cast<const u32x4*>(buf + kHeadPageBytes + kCodeBytes + lane * 16);
        // in the block of the query position, the scales of later tokens read as 0: their slots
        // may hold any bytes (an E4M3 NaN among them), and a zero probability times a NaN value
        // would still reach the output through P.V
        if (tok0 + kBlock - 1 > p) {
            asm volatile("");
            const int first = tok0 + 16 * (lane & 7);
#pragma unroll
            for (int i = 0; i < 4; i++) raw[i] &= keep_bytes(p + 1 - (first + 4 * i));
        }
        u32x4 h0, h1;
#pragma unroll
        for (int i = 0; i < 2; i++) {
            h0[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i], 1.0f, false));
            h0[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i], 1.0f, true));
            h1[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i + 2], 1.0f, false));
            h1[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i + 2], 1.0f, true));
        }
        lds_write32(kbase + lane * 32, h0, h1);
    }

    // ---- O^T += V^T P^T, one 16-dim tile (= one scale group) at a time
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
        const int d = 16 * dt + (lane & 15);
        // codes of tokens 32c..32c+31 and their fp16 scales of group dt
        u32x4 vc, sc[4];
        if constexpr (NEXT) {
            lds_read16x5(vc, sc, vbase + d * 64 + 16 * c, kbase + dt * 256 + 64 * c);
        } else {
            vc = *reinterpret_cast<const u32x4*>(buf + kHeadPageBytes + d * 64 + 16 * c);
#pragma unroll
            for (int w = 0; w < 4; w++)
                sc[w] = *reinterpret_cast<const u32x4*>(buf + dt * 256 + 64 * c + 16 * w);
        }
#pragma unroll
        for (int h = 0; h < 4; h++) {
            // tokens 32c + 8h .. +7 (slabs 2h, 2h + 1) in one 32-token step: scale pairs
            // (8h, 8h+1), (8h+2, 8h+3) and (8h+4, 8h+5), (8h+6, 8h+7)
            const f16x4 a0 = dequant4_f16_scaled<0>(vc[h], sc[h][0], sc[h][1]);
            const f16x4 a1 = dequant4_f16_scaled<2>(vc[h], sc[h][2], sc[h][3]);
            const f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const f16x8 pp = {pt[2 * h][0], pt[2 * h][1], pt[2 * h][2], pt[2 * h][3],
                              pt[2 * h + 1][0], pt[2 * h + 1][1], pt[2 * h + 1][2], pt[2 * h + 1][3]};
            o[dt] = mfma_f16_k32(a, pp, o[dt]);
        }
    }
    // each head's sum of the block's probabilities on the matrix cores (an all-ones A operand),
    // from the same fp16 values the output uses
    const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                        (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
    f32x4 ls = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 4; h++) {
        const f16x8 pp = {pt[2 * h][0], pt[2 * h][1], pt[2 * h][2], pt[2 * h][3],
                          pt[2 * h + 1][0], pt[2 * h + 1][1], pt[2 * h + 1][2], pt[2 * h + 1][3]};
        ls = mfma_f16_k32(ones, pp, ls);
    }
    l_run += ls[0];
}

// SELECT: the row's blocks are selected here from its block scores (wavefront 0 of every
// workgroup of the row, or with LONG, rows of up to kSelectLongMaxBlocks blocks, all four
// wavefronts; the first split also writes them to block_ids) instead of being read
// from block_ids.
// VAR_IDS: rows of ids_per_row (1..64) ids instead of 16: each wavefront takes
// ceil(ids_per_row / (4 NSPLIT)) consecutive slots (up to 16; BPW then only sets the page
// buffers: two for BPW > 1, else one), the selection sizes of the window knobs ("MiniMax M3 on
// vLLM", section "MSA mechanism": the top-k count is a knob).
template <int BPW, bool SELECT, bool LONG = false, int NSPLIT = kMaxSplits / BPW, bool VAR_IDS = false>
__global__ __launch_bounds__(kWaves * 64) void attention_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int batch,
    int max_blocks, int q_len, const uint16_t* __restrict__ q, int32_t* __restrict__ block_ids,
    const float* __restrict__ scores, float scale_log2, uint16_t* __restrict__ out,
    int32_t* __restrict__ counters, float* __restrict__ partials, int ids_per_row) {
    constexpr int kBufs = BPW > 1 ? 2 : 1;
    constexpr int n_split = NSPLIT;  // workgroups per row group
    static_assert(VAR_IDS ? !SELECT : BPW * kWaves * NSPLIT == kTopk,
                  "16 ids per row fill the slots exactly; other counts come from block_ids");
    // blocks per wavefront (a constant unless the row length is a call argument)
    const int bpw = VAR_IDS ? (ids_per_row + kWaves * NSPLIT - 1) / (kWaves * NSPLIT) : BPW;
    static_assert(kWaves * kBufs * kBlockBytes >= kWaves * kGroupHeads * kMergeStride * 4,
                  "merge area must fit in the page buffers");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves][kBufs][kBlockBytes];
    __shared__ float sh_m[kWaves][kGroupHeads];
    __shared__ float sh_l[kWaves][kGroupHeads];
    __shared__ int sh_sel[SELECT ? kTopk : 1];
    static_assert(kSelectScratch * 8 <= kBlockBytes, "selection scratch must fit in a page buffer");
    __shared__ int sh_tbl[SELECT ? (LONG ? kSelectLongMaxBlocks : kSelectFusedMaxBlocks) : 1];  // the sequence's block table
    __shared__ int sh_lid[LONG ? kWaves : 1][kTopk];
    __shared__ uint32_t sh_lkey[LONG ? kWaves : 1][kTopk];

    const int lane = threadIdx.x & 63;
    // wavefront-uniform (a scalar value): the per-wavefront roles below are scalar branches, so
    // no wavefront waits for memory that only another role's code path requested
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    // XCD-aware work mapping: pair = (b, g) -> XCD pair % 8. With an even number of query
    // tokens, drafts 2i and 2i + 1 of one (pair, split) take the XCD's workgroups L and
    // L + NL / 2 (NL workgroups per XCD): when the grid holds two workgroups per compute unit,
    // the dispatcher places those two on one compute unit, and the pages of two drafts mostly
    // coincide (measured 0.15-0.35 us faster at 8 sequences x 4 drafts; any mapping gives the
    // same results)
    const int per_pair = q_len * n_split;
    const int local = blockIdx.x >> 3;
    int pair, j, split;
    if ((q_len & 1) == 0) {
        const int half = (int)(gridDim.x >> 4);  // NL / 2
        const int hi = local >= half ? 1 : 0;
        const int r = local - hi * half;
        const int pp = per_pair >> 1;
        pair = (r / pp) * 8 + (blockIdx.x & 7);
        const int within = r - (r / pp) * pp;
        const int jl = within / n_split;
        split = within - jl * n_split;
        j = 2 * jl + hi;
    } else {
        pair = (local / per_pair) * 8 + (blockIdx.x & 7);
        const int within = local - (local / per_pair) * per_pair;
        j = within / n_split;
        split = within - j * n_split;
    }
    if (pair >= batch * kKvHeads) return;
    const int b = pair >> 2;
    const int g = pair & 3;
    const int bq = b * q_len + j;
    const int rg = bq * kKvHeads + g;  // row group
    // the B operand of S^T is requested first (head 16g + n, dims 32c + 8m .. +7): it arrives
    // during the selection, and no later wait for it also waits for the page loads
    bf16x8 qb[4];
    {
        const uint16_t* qp = q + ((int64_t)bq * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
        for (int m = 0; m < 4; m++) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
    }
    // the context length, requested with the query: every wavefront needs it once its blocks
    // are known
    const int T_raw = ctx_lens[b];
    // this wavefront's blocks (id and page, or -1 when the id is not selected, has no visible
    // token or maps to a page out of range), lane k holding its k-th block, read once: a table
    // load issued between page loads would make the in-order memory counter wait for every
    // page in flight.
    int id;
    if constexpr (SELECT && LONG) {
        // rows of up to kSelectLongMaxBlocks blocks: every wavefront selects the best 15 of a
        // quarter of the row (blocks 1024 wave + lane + 64 k) and copies a quarter of the
        // block-table row; wavefront 0 then ranks the 60 candidates exactly (the top 15 of the
        // row lie among the best 15 of their quarters)
        constexpr int kThr = kWaves * 64;
        constexpr int kPer = (kSelectLongMaxBlocks + kThr - 1) / kThr;
        const int32_t* trow = block_table + (int64_t)b * max_blocks;
        const float* srow = scores + (int64_t)rg * max_blocks;
        float sv[16];
#pragma unroll
        for (int k = 0; k < 16; k++) sv[k] = srow[min(1024 * wave + lane + 64 * k, max_blocks - 1)];
        int tv[kPer];
#pragma unroll
        for (int r = 0; r < kPer; r++) tv[r] = trow[min((int)threadIdx.x + r * kThr, max_blocks - 1)];
        int t_sel = T_raw;
        asm volatile("" : "+v"(t_sel));
#pragma unroll
        for (int r = 0; r < kPer; r++) sh_tbl[min((int)threadIdx.x + r * kThr, max_blocks - 1)] = tv[r];
        const int n_el = eligible_blocks(clamp_ctx(t_sel, max_blocks) - q_len + j, max_blocks);
        if (n_el > kTopk) {
            const int m = n_el - 1;  // candidates 0..m-1 compete for 15 places
            uint32_t key[16];
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int i = 1024 * wave + lane + 64 * k;
                key[k] = i < m ? order_key(sv[k]) : 0u;
            }
            const int base = 1024 * wave;
            select_top<16>(key, lane, reinterpret_cast<uint64_t*>(&lds[wave][0][0]), sh_lid[wave],
                           sh_lkey[wave], [base](int i) { return base + i; }, kTopk - 1);
        }
        __syncthreads();
        if (wave == 0) {
            if (n_el > kTopk) {
                // the 60 candidates in ascending block order (list w holds quarter w's blocks,
                // ascending), each ranked against the others read back as LDS broadcasts
                constexpr int kCand = kWaves * (kTopk - 1);
                uint64_t* cand = reinterpret_cast<uint64_t*>(&lds[0][0][0]);
                const int li = lane < kCand ? lane : 0;
                const uint32_t ky = lane < kCand ? sh_lkey[li / (kTopk - 1)][li % (kTopk - 1)] : 0u;
                const int cid = sh_lid[li / (kTopk - 1)][li % (kTopk - 1)];
                const uint64_t mine = ky ? (((uint64_t)ky << 32) | (uint32_t)~(uint32_t)lane) : 0ull;
                cand[lane] = mine;
                __builtin_amdgcn_wave_barrier();
                asm volatile("" ::: "memory");
                int rank = 0;
#pragma unroll
                for (int t0 = 0; t0 < 64; t0 += 8) {
                    uint64_t o[8];
#pragma unroll
                    for (int i = 0; i < 8; i++) o[i] = cand[t0 + i];
#pragma unroll
                    for (int i = 0; i < 8; i++) rank += (int)(o[i] > mine);
                }
                const bool sel = ky != 0u && rank < kTopk - 1;
                const uint64_t smask = __ballot(sel);
                if (sel) sh_sel[lanes_before(smask)] = cid;
                const int n_sel = popc64(smask);
                if (lane >= n_sel && lane < kTopk - 1) sh_sel[lane] = -1;
                if (lane == 0) sh_sel[kTopk - 1] = n_el - 1;  // the forced block, the largest id
            } else if (lane < kTopk) {
                sh_sel[lane] = lane < n_el ? lane : -1;
            }
        }
        __syncthreads();
        if (split == 0 && wave == 0 && lane < kTopk) block_ids[(int64_t)rg * kTopk + lane] = sh_sel[lane];
        id = lane < BPW ? sh_sel[(split * kWaves + wave) * BPW + lane] : -1;
    } else if constexpr (SELECT) {
        if (wave == 0) {
            // the row's scores and the context length in one memory round trip, then the
            // selection, exactly as msa_block_topk makes it
            float sv[16];
            load_row_scores<16>(scores + (int64_t)rg * max_blocks, max_blocks, lane, sv);
            int t_sel = T_raw;
#pragma unroll
            for (int k = 0; k < 16; k++) asm volatile("" : "+v"(sv[k]));
            asm volatile("" : "+v"(t_sel));
            const int p_sel = clamp_ctx(t_sel, max_blocks) - q_len + j;
            // scratch: this wavefront's page buffer, not in use before the selection is done
            select_row<16>(sv, eligible_blocks(p_sel, max_blocks), lane,
                           reinterpret_cast<uint64_t*>(&lds[0][0][0]), sh_sel);
            if (split == 0 && lane < kTopk) block_ids[(int64_t)rg * kTopk + lane] = sh_sel[lane];
        } else {
            // meanwhile the other wavefronts copy the sequence's block-table row into LDS (all
            // loads issued before any is stored), so the selected blocks' pages need no further
            // memory round trip
            constexpr int kThr = (kWaves - 1) * 64;
            constexpr int kPer = (kSelectFusedMaxBlocks + kThr - 1) / kThr;
            const int t0 = threadIdx.x - 64;
            const int32_t* trow = block_table + (int64_t)b * max_blocks;
            // (indexes past the row are clamped to its last entry, which they then rewrite with
            // its own value: every store is unconditional and writes the right value)
            int tv[kPer];
#pragma unroll
            for (int r = 0; r < kPer; r++) tv[r] = trow[min(t0 + r * kThr, max_blocks - 1)];
#pragma unroll
            for (int r = 0; r < kPer; r++) sh_tbl[min(t0 + r * kThr, max_blocks - 1)] = tv[r];
        }
        __syncthreads();
        id = lane < BPW ? sh_sel[(split * kWaves + wave) * BPW + lane] : -1;
    } else {
        if constexpr (VAR_IDS) {
            const int slot0 = (split * kWaves + wave) * bpw;
            const int32_t* my_ids = block_ids + (int64_t)rg * ids_per_row + slot0;
            id = (lane < bpw && slot0 + lane < ids_per_row) ? my_ids[lane] : -1;
        } else {
            const int32_t* my_ids = block_ids + (int64_t)rg * kTopk + (split * kWaves + wave) * BPW;
            id = lane < BPW ? my_ids[lane] : -1;
        }
        asm volatile("" : "+v"(id));
    }
    const int T = clamp_ctx(T_raw, max_blocks);
    const int p = T - q_len + j;
    MSA_CHECK(threadIdx.x != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    MSA_CHECK(!SELECT || max_blocks <= (LONG ? kSelectLongMaxBlocks : kSelectFusedMaxBlocks), kCheckLds);
    MSA_CHECK(bq < batch * q_len && rg < batch * q_len * kKvHeads && split < n_split, kCheckOutput);
#ifdef MSA_CHECKED
    if constexpr (SELECT) {
        // the row's ids: ascending within the eligible blocks, the block of the query token last
        if (wave == 0 && lane < kTopk) {
            const int n_el = eligible_blocks(p, max_blocks);
            const int kept = min(kTopk, n_el);
            const int v = sh_sel[lane];
            MSA_CHECK(lane < kept ? (v >= 0 && v < n_el && (lane == 0 || v > sh_sel[lane - 1]) &&
                                     (lane != kept - 1 || v == n_el - 1))
                                  : v == -1,
                      kCheckSelection);
        }
    }
#endif
    int page = -1;
    if (lane < bpw && id >= 0 && id < max_blocks && id * kBlock <= p) {
        const int pg = SELECT ? sh_tbl[id] : block_table[(int64_t)b * max_blocks + id];
        page = (pg >= 0 && pg < num_pages) ? pg : -1;
    }
    const int blk_id = page >= 0 ? id : -1;
    // every load so far is complete (the query's included), and the compiler knows it: it
    // waits for nothing of them after the page loads are issued
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint8_t* kg = k_pool + (int64_t)g * kHeadPageBytes;
    const uint8_t* vg = v_pool + (int64_t)g * kHeadPageBytes;
    constexpr int64_t kPageStride = (int64_t)kKvHeads * kHeadPageBytes;
    int cur_id = __builtin_amdgcn_readlane(blk_id, 0);
    if (cur_id >= 0) {
        const int pg = __builtin_amdgcn_readlane(page, 0);
        block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride, lds[wave][0], lane);
    }
    // the B operand is prepared while the first block streams in
    f16x8 qh[4];
    float q_unscale;
    const bool f16 = __all(query_to_f16(qb, qh, q_unscale));
    u32x4 qop[4];
#pragma unroll
    for (int m = 0; m < 4; m++)
        qop[m] = f16 ? __builtin_bit_cast(u32x4, qh[m]) : __builtin_bit_cast(u32x4, qb[m]);
    // a negative softmax scale is applied as the negated query (an exact sign flip of every
    // fp16 / bf16 value) times its magnitude, so the scale inside the blocks is never negative
    if (scale_log2 < 0.f) {
#pragma unroll
        for (int m = 0; m < 4; m++) qop[m] ^= 0x80008000u;
    }
    const float logit_scale = fabsf(scale_log2) * (f16 ? q_unscale : 1.0f);

    // (left to the compiler: with several blocks per wavefront the unrolled body is too large)
    // Two buffers: the next block's copies are issued before the current block is attended.
    // One buffer (VAR_IDS rows with BPW = 1, which may still give a wavefront several blocks):
    // they are issued once the current block's LDS reads have all returned.
    for (int kb = 0; kb < bpw; kb++) {
        int nxt_id = -1;
        if (kb + 1 < bpw) {
            nxt_id = __builtin_amdgcn_readlane(blk_id, kb + 1);
            if (kBufs > 1 && nxt_id >= 0) {
                const int pg = __builtin_amdgcn_readlane(page, kb + 1);
                block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride,
                             lds[wave][(kb + 1) % kBufs], lane);
            }
        }
        if (cur_id >= 0) {
            // the current block's K page (its first 9 loads) has arrived
            uint8_t* buf = lds[wave][kb % kBufs];
            const int tok0 = cur_id * kBlock;
            if (kBufs > 1 && nxt_id >= 0) {
                asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
                if (f16) attend_block<true, true>(buf, lane, c, tok0, p, qop, logit_scale, m_run, l_run, o);
                else attend_block<false, true>(buf, lane, c, tok0, p, qop, logit_scale, m_run, l_run, o);
            } else {
                asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
                if (f16) attend_block<true, false>(buf, lane, c, tok0, p, qop, logit_scale, m_run, l_run, o);
                else attend_block<false, false>(buf, lane, c, tok0, p, qop, logit_scale, m_run, l_run, o);
            }
        }
        if (kBufs == 1 && nxt_id >= 0) {
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            const int pg = __builtin_amdgcn_readlane(page, kb + 1);
            block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride, lds[wave][0], lane);
        }
        cur_id = nxt_id;
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();  // all page buffers are free: reuse them for the merge

    // ---- merge the 4 wavefronts: lane (n, c) holds o[dt][i] = out(head n, dim 16dt + 4c + i)
    float* sh_o = reinterpret_cast<float*>(&lds[0][0][0]);  // [kWaves][16][kMergeStride]
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            sh_o[(wave * kGroupHeads + n) * kMergeStride + 16 * dt + 4 * c + i] = o[dt][i];
    if (c == 0) {
        sh_m[wave][n] = m_run;
        sh_l[wave][n] = l_run;
    }
    __syncthreads();
    const int h = threadIdx.x >> 4;         // head 0..15
    const int d0 = (threadIdx.x & 15) * 8;  // 8 dims
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, sh_m[w][h]);
    float L = 0.f, acc[8];
    {
        float wt[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; w++) {
            wt[w] = (sh_m[w][h] == -INFINITY) ? 0.f : fast_exp2(sh_m[w][h] - M);
            L += wt[w] * sh_l[w][h];
        }
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; w++) x += wt[w] * sh_o[(w * kGroupHeads + h) * kMergeStride + d0 + e];
            acc[e] = x;
        }
    }
    if (n_split > 1) {
        // hand this split's (max, sum, output) over; the wavefront that finishes last among the
        // splits' wavefronts of the same four heads merges them and writes the output (its
        // counter counts finished wavefronts and is left at zero again for the next launch)
        const int64_t part_base = (int64_t)rg * n_split * kGroupHeads;
        float* pp = partials + ((part_base + (int64_t)split * kGroupHeads) + h) * kPartStride;
        MSA_CHECK(((part_base + (int64_t)split * kGroupHeads) + h + 1) * kPartStride <=
                      (int64_t)batch * q_len * kKvHeads * n_split * kGroupHeads * kPartStride,
                  kCheckWorkspace);
        if (d0 == 0) store16_coherent(pp, f32x4{M, L, 0.f, 0.f});
        store16_coherent(pp + 4 + d0, f32x4{acc[0], acc[1], acc[2], acc[3]});
        store16_coherent(pp + 8 + d0, f32x4{acc[4], acc[5], acc[6], acc[7]});
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stores complete, agent-wide
        // each wavefront counts itself finished on the counter of its four heads: the last of
        // them merges those heads, with no barrier between the wavefronts of a workgroup
        int32_t* counter = counters + (int64_t)rg * kWaves + wave;
        int prior = 0;
        if (lane == 0) prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__builtin_amdgcn_readlane(prior, 0) != n_split - 1) return;
        // every split's values requested before any is used (one memory round trip): splits
        // past n_split read this split's own partial, then every value not from another split
        // is replaced
        static_assert(kMaxSplits == 4, "load_partials_coherent loads four partials");
        const float* pp4[kMaxSplits][3];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; sp++) {
            const int src = sp < n_split ? sp : split;
            const float* qp = partials + ((part_base + (int64_t)src * kGroupHeads) + h) * kPartStride;
            pp4[sp][0] = qp;
            pp4[sp][1] = qp + 4 + d0;
            pp4[sp][2] = qp + 8 + d0;
        }
        f32x4 part[kMaxSplits][3];
        load_partials_coherent(pp4, part);
        f32x4 ml[kMaxSplits], a0[kMaxSplits], a1[kMaxSplits];
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; sp++) {
            const bool other = sp < n_split && sp != split;
            ml[sp] = other ? part[sp][0]
                           : f32x4{sp == split ? M : -INFINITY, sp == split ? L : 0.f, 0.f, 0.f};
            a0[sp] = other ? part[sp][1]
                           : (sp == split ? f32x4{acc[0], acc[1], acc[2], acc[3]} : f32x4{0.f, 0.f, 0.f, 0.f});
            a1[sp] = other ? part[sp][2]
                           : (sp == split ? f32x4{acc[4], acc[5], acc[6], acc[7]} : f32x4{0.f, 0.f, 0.f, 0.f});
        }
        if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        M = -INFINITY;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; sp++) M = fmaxf(M, ml[sp][0]);
        L = 0.f;
#pragma unroll
        for (int e = 0; e < 8; e++) acc[e] = 0.f;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; sp++) {
            const float w = ml[sp][0] == -INFINITY ? 0.f : fast_exp2(ml[sp][0] - M);
            L += w * ml[sp][1];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                acc[e] += w * a0[sp][e];
                acc[4 + e] += w * a1[sp][e];
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; e++)
        packed[e] = (uint32_t)bf16_bits_rne(acc[2 * e] * inv) |
                    ((uint32_t)bf16_bits_rne(acc[2 * e + 1] * inv) << 16);
    uint16_t* op = out + ((int64_t)bq * kQHeads + kGroupHeads * g + h) * kDim + d0;
    *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
}

// ---------------------------------------------------------------- token tiles
// Batches with many query tokens per sequence (prefill chunks): the tokens of one (sequence,
// group) pair select mostly the same blocks, and reading each block once per token makes the
// page traffic, not the arithmetic, the bound. A workgroup of eight wavefronts takes 16
// consecutive query tokens of one pair, two per wavefront. The union of their selected
// blocks streams once, in ascending block order, through two LDS buffers that the workgroup
// shares (the next block's loads spread over the wavefronts and in flight while the current
// block is used). The workgroup dequantizes each block once into fp16 operand tables (one K
// slab and one V dim tile per wavefront), and each wavefront attends exactly the blocks its
// tokens selected, from the tables (each table read serving both tokens), keeping its tokens'
// whole softmax state: no partials and no merge.
// Four 16-byte LDS reads at a, a + 1 KB, a + 2 KB, a + 3 KB, issued and waited for together.
__device__ __forceinline__ void lds_read16x4(u32x4 (&v)[4], uint32_t a) {
    asm volatile("ds_read_b128 %0, %4\n\t"
                 "ds_read_b128 %1, %4 offset:1024\n\t"
                 "ds_read_b128 %2, %4 offset:2048\n\t"
                 "ds_read_b128 %3, %4 offset:3072\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a) : "memory");
}
// Four 16-byte LDS writes at a, a + 1 KB, a + 2 KB, a + 3 KB (waited for by the caller).
__device__ __forceinline__ void lds_write16x4(uint32_t a, const u32x4 (&v)[4]) {
    asm volatile("ds_write_b128 %0, %1\n\t"
                 "ds_write_b128 %0, %2 offset:1024\n\t"
                 "ds_write_b128 %0, %3 offset:2048\n\t"
                 "ds_write_b128 %0, %4 offset:3072"
                 :: "v"(a), "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3])
                 : "memory");
}

// The fp16 operand tables of one block, made once per workgroup from its NVFP4 K and V pages
// (in LDS at `page`): wavefront w dequantizes K slab w and V dims 16w .. 16w + 15, exactly.
//   kf + 4096 s + 1024 m + 16 l : lane l's A operand of S^T step (slab s, k-step m), f16x8
//   vf + 4096 dt + 1024 h + 16 l: lane l's A operands of O^T steps (dim tile dt, token slabs
//                                 2h and 2h + 1), two f16x4
__device__ __forceinline__ void dequant_tables(const uint8_t* page, uint8_t* kf, uint8_t* vf,
                                               int wave, int lane, int valid) {
    const int n = lane & 15, c = lane >> 4;
    const uint32_t pbase = (uint32_t)(uintptr_t)page;
    u32x4 kc[4], vr[4];
    // K codes of slab `wave` and the token row's scale bytes; V codes of dim 16 wave + n (tokens
    // 32c .. 32c + 31) and the raw scales of group `wave` for those tokens
    asm volatile("ds_read_b128 %0, %4\n\t"
                 "ds_read_b128 %1, %5\n\t"
                 "ds_read_b128 %2, %6\n\t"
                 "ds_read_b128 %3, %6 offset:16\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(kc[0]), "=&v"(kc[1]), "=&v"(vr[0]), "=&v"(vr[1])
                 : "v"(pbase + 1024 * wave + 16 * lane), "v"(pbase + kCodeBytes + 16 * lane),
                   "v"(pbase + kHeadPageBytes + kCodeBytes + 128 * wave + 32 * c)
                 : "memory");
    const u32x4 code = kc[0], ksc = kc[1];
    const u32x4 vc = lds_read16(pbase + kHeadPageBytes + (16 * wave + n) * 64 + 16 * c);
    f16x2 s0, s1;
    if (wave & 1) e4m3_pair_f16<true>(ksc[wave >> 1], s0, s1);
    else e4m3_pair_f16<false>(ksc[wave >> 1], s0, s1);
    u32x4 ko[4];
#pragma unroll
    for (int m = 0; m < 4; m++) ko[m] = __builtin_bit_cast(u32x4, dequant8_f16(code[m], m < 2 ? s0 : s1));
    lds_write16x4((uint32_t)(uintptr_t)(kf + 4096 * wave + 16 * lane), ko);
    // V: tokens 32c + 4s .. +3 of slab s take the scale pairs (4s, 4s + 1), (4s + 2, 4s + 3)
    uint32_t raw[8] = {vr[0][0], vr[0][1], vr[0][2], vr[0][3], vr[1][0], vr[1][1], vr[1][2], vr[1][3]};
    // tokens at or past the context length (`valid` tokens of the block are in the cache): their
    // scales read as 0, so bytes never written (an E4M3 NaN among them) cannot reach the output
    // through a zero probability
    if (valid < kBlock) {
#pragma unroll
        for (int sl = 0; sl < 8; sl++) raw[sl] &= keep_bytes(valid - (32 * c + 4 * sl));
    }
    u32x4 vo[4];
#pragma unroll
    for (int h = 0; h < 4; h++) {
        f16x4 a[2];
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const int sl = 2 * h + e;
            const uint32_t s01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[sl], 1.0f, false));
            const uint32_t s23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[sl], 1.0f, true));
            a[e] = e ? dequant4_f16_scaled<2>(vc[h], s01, s23) : dequant4_f16_scaled<0>(vc[h], s01, s23);
        }
        const uint2 lo = __builtin_bit_cast(uint2, a[0]), hi = __builtin_bit_cast(uint2, a[1]);
        vo[h] = u32x4{lo.x, lo.y, hi.x, hi.y};
    }
    lds_write16x4((uint32_t)(uintptr_t)(vf + 4096 * wave + 16 * lane), vo);
}

// One block of one wavefront from the fp16 tables, for the TPW tokens the wavefront holds
// (those with sel[t]): logits, online-softmax update, output accumulation (the arithmetic of
// attend_block, with the dequantization done beforehand). Each 16-byte table read feeds the
// matrix-core steps of every selecting token.
template <bool F16, int TPW>
__device__ __forceinline__ void attend_tables(const uint8_t* kf, const uint8_t* vf, int lane,
                                              int c, int tok0, const int (&p)[TPW],
                                              const bool (&sel)[TPW], const u32x4 (&qop)[TPW][4],
                                              const float (&logit_scale)[TPW],
                                              float (&m_run)[TPW], float (&l_run)[TPW],
                                              f32x4 (&o)[TPW][8]) {
    f32x4 sv[TPW][8];
#pragma unroll
    for (int s = 0; s < 8; s++) {
        u32x4 a[4];
        lds_read16x4(a, (uint32_t)(uintptr_t)(kf + 4096 * s + 16 * lane));
        // (every token's steps run: branches around them cost register copies at every merge;
        // a token that did not select the block gets zero probabilities below)
#pragma unroll
        for (int t = 0; t < TPW; t++) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; m++) {
                if constexpr (F16)
                    acc = mfma_f16_k32(__builtin_bit_cast(f16x8, a[m]), __builtin_bit_cast(f16x8, qop[t][m]), acc);
                else
                    acc = mfma_bf16_k32(f16x8_to_bf16x8(__builtin_bit_cast(f16x8, a[m])),
                                        __builtin_bit_cast(bf16x8, qop[t][m]), acc);
            }
            sv[t][s] = acc;
        }
    }
    f16x8 pt[TPW][4];
#pragma unroll
    for (int t = 0; t < TPW; t++) {
        if (sel[t]) {
            softmax_block(sv[t], c, tok0, p[t], logit_scale[t], m_run[t], l_run[t], o[t], pt[t]);
        } else {
#pragma unroll
            for (int h = 0; h < 4; h++) pt[t][h] = f16x8{};  // adds exactly 0 to the output
        }
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
        u32x4 a[4];
        lds_read16x4(a, (uint32_t)(uintptr_t)(vf + 4096 * dt + 16 * lane));
        // one 32-token step per slab pair: lane (n, c) holds dim 16 dt + n of tokens
        // 32c + 8h .. +7 in A and the same tokens' probabilities of head n in B (any order of
        // the reduction index works when both operands agree)
#pragma unroll
        for (int t = 0; t < TPW; t++)
#pragma unroll
            for (int h = 0; h < 4; h++)
                o[t][dt] = mfma_f16_k32(__builtin_bit_cast(f16x8, a[h]), pt[t][h], o[t][dt]);
    }
    // each head's sum of the block's probabilities: a matrix-core step with an all-ones A
    // operand (every row m of D gets the sum over the tokens of head n), which spares the
    // vector unit 32 additions and a cross-lane sum per token and block
    const f16x8 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f,
                        (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int t = 0; t < TPW; t++) {
        f32x4 ls = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 4; h++) ls = mfma_f16_k32(ones, pt[t][h], ls);
        l_run[t] += ls[0];
    }
}

constexpr int kTileWaves = 8;
constexpr int kTileTpw = 2;                         // tokens per wavefront
constexpr int kTileTokens = kTileWaves * kTileTpw;  // tokens per workgroup
constexpr int kUnionMaxBlocks = 8192;  // rows of up to this many blocks (the union's bitmap)
constexpr int kTileMinQ = 8;           // from this many query tokens per sequence (and no split)

__global__ __launch_bounds__(kTileWaves * 64) void attention_tile_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int batch,
    int max_blocks, int q_len, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ block_ids, float scale_log2, uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t pages[2][kBlockBytes];
    __shared__ __attribute__((aligned(16))) uint8_t kf[8 * 4096];  // fp16 operand tables
    __shared__ __attribute__((aligned(16))) uint8_t vf[8 * 4096];
    __shared__ uint64_t bitmap[kUnionMaxBlocks / 64];
    __shared__ uint64_t tokmap[kTileWaves][kTileTpw][kUnionMaxBlocks / 64];  // per token
    __shared__ int ulist[kTileTokens * kTopk];
    __shared__ int upage[kTileTokens * kTopk];
    __shared__ int ucount;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    // XCD-aware work mapping as in attention_kernel: pair = (b, g) -> XCD pair % 8
    const int tiles = (q_len + kTileTokens - 1) / kTileTokens;
    const int local = blockIdx.x >> 3;
    const int pair = (local / tiles) * 8 + (blockIdx.x & 7);
    if (pair >= batch * kKvHeads) return;  // the whole workgroup
    const int tile = local - (local / tiles) * tiles;
    const int b = pair >> 2;
    const int g = pair & 3;
    // this wavefront's tokens j[t] = tile * 16 + 2 wave + t
    bool has_tok[kTileTpw];
    int bq[kTileTpw], p[kTileTpw];
    bf16x8 qb[kTileTpw][4];
    const int T = clamp_ctx(ctx_lens[b], max_blocks);
#pragma unroll
    for (int t = 0; t < kTileTpw; t++) {
        const int j_raw = tile * kTileTokens + kTileTpw * wave + t;
        has_tok[t] = j_raw < q_len;  // wavefront-uniform
        const int j = min(j_raw, q_len - 1);
        bq[t] = b * q_len + j;
        p[t] = T - q_len + j;
        const uint16_t* qp = q + ((int64_t)bq[t] * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
        for (int m = 0; m < 4; m++) qb[t][m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
    }
    // lanes 16 t .. 16 t + 15 hold token t's ids
    int myid = -1;
    if (lane < kTileTpw * kTopk) {
        const int t = lane >> 4;
        const int id = has_tok[t] ? block_ids[((int64_t)bq[t] * kKvHeads + g) * kTopk + (lane & 15)] : -1;
        // the token's usable blocks (as attention_kernel: in the table and holding a visible key)
        myid = (id >= 0 && id < max_blocks && id * kBlock <= p[t]) ? id : -1;
    }

    // the union: a bitmap over the row's blocks, then its set bits in ascending order
    // (and each token's own bitmap, which the block loop reads instead of keeping the ids)
    const int nwords = (max_blocks + 63) >> 6;
    for (int i = threadIdx.x; i < nwords; i += kTileWaves * 64) bitmap[i] = 0;
    for (int i = lane; i < kTileTpw * nwords; i += 64) tokmap[wave][i / nwords][i % nwords] = 0;
    __syncthreads();
    if (myid >= 0) {
        atomicOr(reinterpret_cast<unsigned long long*>(&bitmap[myid >> 6]), 1ull << (myid & 63));
        atomicOr(reinterpret_cast<unsigned long long*>(&tokmap[wave][lane >> 4][myid >> 6]),
                 1ull << (myid & 63));
    }
    __syncthreads();
    if (wave == 0) {
        int base = 0;
        for (int w0 = 0; w0 < nwords; w0 += 64) {
            const int wi = w0 + lane;
            uint64_t bits = wi < nwords ? bitmap[wi] : 0ull;
            const int cnt = popc64(bits);
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            int at = base + incl - cnt;
            while (bits) {
                ulist[at++] = wi * 64 + __builtin_ctzll(bits);
                bits &= bits - 1;
            }
            base += __shfl(incl, 63, 64);
        }
        if (lane == 0) ucount = base;  // at most 16 x 16 blocks
    }
    __syncthreads();
    const int nu = ucount;
    MSA_CHECK(nu <= kTileTokens * kTopk && max_blocks <= kUnionMaxBlocks, kCheckLds);
    if ((int)threadIdx.x < nu) {
        const int pg = block_table[(int64_t)b * max_blocks + ulist[threadIdx.x]];
        upage[threadIdx.x] = (pg >= 0 && pg < num_pages) ? pg : -1;
    }
    __syncthreads();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    // union entry u (block id, page) read back from LDS as a broadcast, by an explicit read
    // waited for on its own (page loads are in flight from here on)
    auto entry = [&](int u, int& id_u, int& page_u) {
        int a, bb;
        asm volatile("ds_read_b32 %0, %2\n\t"
                     "ds_read_b32 %1, %3\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(a), "=&v"(bb)
                     : "v"((uint32_t)(uintptr_t)&ulist[u]), "v"((uint32_t)(uintptr_t)&upage[u])
                     : "memory");
        id_u = __builtin_amdgcn_readfirstlane(a);
        page_u = __builtin_amdgcn_readfirstlane(bb);
    };

    const uint8_t* kg = k_pool + (int64_t)g * kHeadPageBytes;
    const uint8_t* vg = v_pool + (int64_t)g * kHeadPageBytes;
    constexpr int64_t kPageStride = (int64_t)kKvHeads * kHeadPageBytes;
    // block u's 18 page pieces (1 KB each: 9 of K, then 9 of V) spread over the wavefronts
    auto issue = [&](int u) {
        int bid_u, pg;
        entry(u, bid_u, pg);
        if (pg < 0) return;
        uint8_t* dst = pages[u & 1];
        for (int i = wave; i < 18; i += kTileWaves) {
            const uint8_t* src = i < 9 ? kg + pg * kPageStride + i * 1024
                                       : vg + pg * kPageStride + (i - 9) * 1024;
            __builtin_amdgcn_global_load_lds(src + lane * 16, (lds_void*)(dst + i * 1024), 16, 0,
                                             kPagePolicy);
        }
    };
    if (nu > 0) issue(0);

    float m_run[kTileTpw], l_run[kTileTpw], logit_scale[kTileTpw];
    f32x4 o[kTileTpw][8];
    u32x4 qop[kTileTpw][4];
    f16x8 qh[kTileTpw][4];
    float q_unscale[kTileTpw];
    bool exact = true;
#pragma unroll
    for (int t = 0; t < kTileTpw; t++) exact = query_to_f16(qb[t], qh[t], q_unscale[t]) && exact;
    const bool f16 = __all(exact);  // both tokens in fp16, or both in bf16
#pragma unroll
    for (int t = 0; t < kTileTpw; t++) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            qop[t][m] = f16 ? __builtin_bit_cast(u32x4, qh[t][m]) : __builtin_bit_cast(u32x4, qb[t][m]);
            if (scale_log2 < 0.f) qop[t][m] ^= 0x80008000u;
        }
        logit_scale[t] = fabsf(scale_log2) * (f16 ? q_unscale[t] : 1.0f);
    }

    for (int u = 0; u < nu; u++) {
        // block u has arrived for every wavefront, and every wavefront is done with block u - 1
        // (its page buffer, which the next loads overwrite, and the fp16 tables)
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wavefront's pieces of block u
        __syncthreads();
        if (u + 1 < nu) issue(u + 1);
        int bid, pg;
        entry(u, bid, pg);
        if (pg < 0) continue;  // (uniform: no wavefront reaches the barrier below)
        // the lane's LDS addresses are recomputed in every iteration, not held across the loop
        // (registers are the limit here: held, they were spilled to scratch)
        int lane_i = lane;
        asm volatile("" : "+v"(lane_i));
        dequant_tables(pages[u & 1], kf, vf, wave, lane_i, T - bid * kBlock);
        // the tables are complete for every wavefront (LDS only: the next block's loads stay
        // in flight)
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        // did this wavefront's tokens select block bid (their bitmaps' words, LDS broadcasts)
        static_assert(kTileTpw == 2, "two token bitmaps read below");
        uint64_t w0, w1;
        asm volatile("ds_read_b64 %0, %2\n\t"
                     "ds_read_b64 %1, %3\n\t"
                     "s_waitcnt lgkmcnt(0)"
                     : "=&v"(w0), "=&v"(w1)
                     : "v"((uint32_t)(uintptr_t)&tokmap[wave][0][bid >> 6]),
                       "v"((uint32_t)(uintptr_t)&tokmap[wave][1][bid >> 6])
                     : "memory");
        bool sel[kTileTpw];
        sel[0] = __builtin_amdgcn_readfirstlane((uint32_t)(w0 >> (bid & 63)) & 1u) != 0u;
        sel[1] = __builtin_amdgcn_readfirstlane((uint32_t)(w1 >> (bid & 63)) & 1u) != 0u;
        if (sel[0] || sel[1]) {
            if (f16) attend_tables<true, kTileTpw>(kf, vf, lane_i, c, bid * kBlock, p, sel, qop, logit_scale, m_run, l_run, o);
            else attend_tables<false, kTileTpw>(kf, vf, lane_i, c, bid * kBlock, p, sel, qop, logit_scale, m_run, l_run, o);
        }
    }
#pragma unroll
    for (int t = 0; t < kTileTpw; t++) {
        if (!has_tok[t]) continue;
        // lane (n, c) holds o[dt][i] = out(head n, dim 16 dt + 4 c + i); l_run is the head's sum
        const float inv = l_run[t] > 0.f ? 1.f / l_run[t] : 0.f;
        uint16_t* op = out + ((int64_t)bq[t] * kQHeads + kGroupHeads * g + n) * kDim + 4 * c;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
            const uint32_t lo = (uint32_t)bf16_bits_rne(o[t][dt][0] * inv) | ((uint32_t)bf16_bits_rne(o[t][dt][1] * inv) << 16);
            const uint32_t hi = (uint32_t)bf16_bits_rne(o[t][dt][2] * inv) | ((uint32_t)bf16_bits_rne(o[t][dt][3] * inv) << 16);
            *reinterpret_cast<uint2*>(op + 16 * dt) = uint2{lo, hi};
        }
    }
}

// ---------------------------------------------------------------- shared-prefix pages
// A batch whose requests share the pages of their first prefix_blocks blocks ("vLLM day-0
// support for MiniMax-M3.1-Flash", section "NVFP4 MSA kernel": a page of a shared prefix is
// dequantized once for up to 64 requests that share it). Two launches:
//   shared_block_kernel: one workgroup of eight wavefronts per (shared block, group). It lists
//   every row (query token of any request) whose selection holds the block (a workgroup with
//   none ends there), loads the block's K and V pages once and dequantizes them once into the
//   fp16 operand tables, and then computes the listed rows' attention over that block alone from
//   the tables, two rows per wavefront at a time (each table read serving both), kept as
//   partials: per head the row's maximum and sum (log2 domain) and its output normalized by the
//   sum, in fp16.
//   shared_combine_kernel: one workgroup of eight wavefronts per row group (row, group). Each
//   wavefront takes two of the row's 16 selection slots, folds in the partials of its shared
//   blocks and attends to its private blocks itself (as attention_kernel does), and the eight
//   wavefronts merge by log-sum-exp.
// Rows are held in a workgroup list of at most kSharedMaxRows entries per block.
constexpr int kSharedMaxRows = 1024;
constexpr int kSharedTpw = 2;  // rows per wavefront at a time
constexpr int kSPartBytes = 2 * kGroupHeads * 4 + kGroupHeads * kDim * 2;  // m, l; then o in fp16
constexpr int kCombineWaves = 8;

__global__ __launch_bounds__(kTileWaves * 64) void shared_block_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int batch,
    int max_blocks, int q_len, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ block_ids, float scale_log2, uint8_t* __restrict__ parts) {
    __shared__ __attribute__((aligned(16))) uint8_t page[kBlockBytes];
    __shared__ __attribute__((aligned(16))) uint8_t kf[8 * 4096];  // fp16 operand tables
    __shared__ __attribute__((aligned(16))) uint8_t vf[8 * 4096];
    __shared__ int items[kSharedMaxRows];  // 16 r + k: slot k of row r selected this block
    __shared__ int n_items;
    static_assert(kTileWaves == 8, "dequant_tables: one K slab and one V dim tile per wavefront");

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    // group g on XCDs g and g + 4: the query rows of a group are read from those XCDs' L2
    const int g = blockIdx.x & 3;
    const int blk = blockIdx.x >> 2;
    const int rows = batch * q_len;
    if (threadIdx.x == 0) n_items = 0;
    __syncthreads();
    // the rows that selected the block and see a key of it (the rule of attention_kernel)
    for (int i = threadIdx.x; i < rows * kTopk; i += kTileWaves * 64) {
        const int r = i >> 4;
        if (block_ids[((int64_t)r * kKvHeads + g) * kTopk + (i & 15)] == blk) {
            const int b = r / q_len;
            const int p = clamp_ctx(ctx_lens[b], max_blocks) - q_len + (r - b * q_len);
            if (blk * kBlock <= p) {
                const int at = atomicAdd(&n_items, 1);
                if (at < kSharedMaxRows) items[at] = i;
            }
        }
    }
    __syncthreads();
    const int count = __builtin_amdgcn_readfirstlane(min(n_items, kSharedMaxRows));
    MSA_CHECK(n_items <= kSharedMaxRows, kCheckLds);
    // sequence 0's table entry: the page every request holds for the block
    const int pg = __builtin_amdgcn_readfirstlane(block_table[blk]);
    if (count == 0 || pg < 0 || pg >= num_pages) return;  // the whole workgroup

    // the block's K and V pages (9 + 9 pieces of 1 KB) spread over the wavefronts
    const uint8_t* kp = k_pool + ((int64_t)pg * kKvHeads + g) * kHeadPageBytes;
    const uint8_t* vp = v_pool + ((int64_t)pg * kKvHeads + g) * kHeadPageBytes;
    for (int i = wave; i < 18; i += kTileWaves) {
        const uint8_t* src = i < 9 ? kp + i * 1024 : vp + (i - 9) * 1024;
        __builtin_amdgcn_global_load_lds(src + lane * 16, (lds_void*)(page + i * 1024), 16, 0,
                                         kPagePolicy);
    }
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
    __syncthreads();
    // a shared block lies before every query token: all 128 of its tokens are in the cache
    dequant_tables(page, kf, vf, wave, lane, kBlock);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __syncthreads();

    for (int it0 = kSharedTpw * wave; it0 < count; it0 += kSharedTpw * kTileWaves) {
        int r[kSharedTpw], k[kSharedTpw], p[kSharedTpw];
        bool sel[kSharedTpw];
        bf16x8 qb[kSharedTpw][4];
#pragma unroll
        for (int t = 0; t < kSharedTpw; t++) {
            sel[t] = it0 + t < count;  // wavefront-uniform
            const int code = __builtin_amdgcn_readfirstlane(items[sel[t] ? it0 + t : it0]);
            r[t] = code >> 4;
            k[t] = code & 15;
            const int b = r[t] / q_len;
            p[t] = clamp_ctx(ctx_lens[b], max_blocks) - q_len + (r[t] - b * q_len);
            const uint16_t* qp = q + ((int64_t)r[t] * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
            for (int m = 0; m < 4; m++) qb[t][m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
        }
        f16x8 qh[kSharedTpw][4];
        float q_unscale[kSharedTpw];
        bool exact = true;
#pragma unroll
        for (int t = 0; t < kSharedTpw; t++) exact = query_to_f16(qb[t], qh[t], q_unscale[t]) && exact;
        const bool f16 = __all(exact);  // both rows in fp16, or both in bf16
        u32x4 qop[kSharedTpw][4];
        float logit_scale[kSharedTpw], m_run[kSharedTpw], l_run[kSharedTpw];
        f32x4 o[kSharedTpw][8];
#pragma unroll
        for (int t = 0; t < kSharedTpw; t++) {
#pragma unroll
            for (int m = 0; m < 4; m++) {
                qop[t][m] = f16 ? __builtin_bit_cast(u32x4, qh[t][m]) : __builtin_bit_cast(u32x4, qb[t][m]);
                if (scale_log2 < 0.f) qop[t][m] ^= 0x80008000u;  // as attention_kernel
            }
            logit_scale[t] = fabsf(scale_log2) * (f16 ? q_unscale[t] : 1.0f);
            m_run[t] = -INFINITY;
            l_run[t] = 0.f;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) o[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        int lane_i = lane;  // recomputed addresses (as in attention_tile_kernel)
        asm volatile("" : "+v"(lane_i));
        if (f16) attend_tables<true, kSharedTpw>(kf, vf, lane_i, c, blk * kBlock, p, sel, qop, logit_scale, m_run, l_run, o);
        else attend_tables<false, kSharedTpw>(kf, vf, lane_i, c, blk * kBlock, p, sel, qop, logit_scale, m_run, l_run, o);
        // the partials of (row r, group g, slot k); lane (n, c) holds head n, dims 16 dt + 4c + i
#pragma unroll
        for (int t = 0; t < kSharedTpw; t++) {
            if (!sel[t]) continue;
            uint8_t* dst = parts + (((int64_t)r[t] * kKvHeads + g) * kTopk + k[t]) * kSPartBytes;
            if (c == 0) {
                reinterpret_cast<float*>(dst)[n] = m_run[t];
                reinterpret_cast<float*>(dst)[kGroupHeads + n] = l_run[t];
            }
            const float inv = 1.f / l_run[t];  // >= 1: the block's largest weight is 1
            _Float16* od = reinterpret_cast<_Float16*>(dst + 2 * kGroupHeads * 4) + n * kDim + 4 * c;
#pragma unroll
            for (int dt = 0; dt < 8; dt++)
                *reinterpret_cast<f16x4*>(od + 16 * dt) =
                    f16x4{(_Float16)(o[t][dt][0] * inv), (_Float16)(o[t][dt][1] * inv),
                          (_Float16)(o[t][dt][2] * inv), (_Float16)(o[t][dt][3] * inv)};
        }
    }
}

__global__ __launch_bounds__(kCombineWaves * 64) void shared_combine_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int batch,
    int max_blocks, int q_len, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ block_ids, int prefix_blocks, float scale_log2,
    const uint8_t* __restrict__ parts, uint16_t* __restrict__ out) {
    constexpr int kSlots = kTopk / kCombineWaves;  // selection slots per wavefront
    static_assert(kCombineWaves * kBlockBytes >= kCombineWaves * kGroupHeads * kMergeStride * 4,
                  "merge area must fit in the page buffers");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kCombineWaves][kBlockBytes];
    __shared__ float sh_m[kCombineWaves][kGroupHeads];
    __shared__ float sh_l[kCombineWaves][kGroupHeads];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15;
    const int c = lane >> 4;
    const int rg = blockIdx.x;  // row group: row r, group g
    const int r = rg >> 2;
    const int g = rg & 3;
    const int b = r / q_len;
    bf16x8 qb[4];
    {
        const uint16_t* qp = q + ((int64_t)r * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
        for (int m = 0; m < 4; m++) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
    }
    const int T = clamp_ctx(ctx_lens[b], max_blocks);
    const int p = T - q_len + (r - b * q_len);
    // this wavefront's slots, lane k holding slot kSlots wave + k: the block id and its page
    // (sequence 0's entry for a shared block), or -1 when the slot is unusable
    int id = -1, page = -1;
    if (lane < kSlots) {
        const int v = block_ids[(int64_t)rg * kTopk + kSlots * wave + lane];
        if (v >= 0 && v < max_blocks && v * kBlock <= p) {
            const int pgv = block_table[(int64_t)(v < prefix_blocks ? 0 : b) * max_blocks + v];
            if (pgv >= 0 && pgv < num_pages) {
                id = v;
                page = pgv;
            }
        }
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);
    const uint8_t* kg = k_pool + (int64_t)g * kHeadPageBytes;
    const uint8_t* vg = v_pool + (int64_t)g * kHeadPageBytes;
    constexpr int64_t kPageStride = (int64_t)kKvHeads * kHeadPageBytes;
    // the first private block's pages are requested first, then every shared slot's partial:
    // all of it is in flight together
    int first_priv = kSlots;
    for (int kb = kSlots - 1; kb >= 0; kb--) {
        if (__builtin_amdgcn_readlane(id, kb) >= prefix_blocks) first_priv = kb;
    }
    if (first_priv < kSlots) {
        const int pg = __builtin_amdgcn_readlane(page, first_priv);
        block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride, lds[wave], lane);
    }
    float pm[kSlots], pl[kSlots];
    f16x4 pv[kSlots][8];
#pragma unroll
    for (int kb = 0; kb < kSlots; kb++) {
        const int cid = __builtin_amdgcn_readlane(id, kb);
        pm[kb] = -INFINITY;
        pl[kb] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) pv[kb][dt] = f16x4{};
        if (cid >= 0 && cid < prefix_blocks) {
            const uint8_t* src = parts + ((int64_t)rg * kTopk + kSlots * wave + kb) * kSPartBytes;
            pm[kb] = reinterpret_cast<const float*>(src)[n];
            pl[kb] = reinterpret_cast<const float*>(src)[kGroupHeads + n];
            const _Float16* op = reinterpret_cast<const _Float16*>(src + 2 * kGroupHeads * 4) + n * kDim + 4 * c;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) pv[kb][dt] = *reinterpret_cast<const f16x4*>(op + 16 * dt);
        }
    }
    f16x8 qh[4];
    float q_unscale;
    const bool f16 = __all(query_to_f16(qb, qh, q_unscale));
    u32x4 qop[4];
#pragma unroll
    for (int m = 0; m < 4; m++) {
        qop[m] = f16 ? __builtin_bit_cast(u32x4, qh[m]) : __builtin_bit_cast(u32x4, qb[m]);
        if (scale_log2 < 0.f) qop[m] ^= 0x80008000u;
    }
    const float logit_scale = fabsf(scale_log2) * (f16 ? q_unscale : 1.0f);

    // shared blocks: each partial rescaled to the running maximum and added
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < kSlots; kb++) {
        if (pm[kb] == -INFINITY) continue;  // not a shared slot (every head agrees)
        const float m_new = fmaxf(m_run, pm[kb]);
        const float a = m_run == -INFINITY ? 0.f : fast_exp2(m_run - m_new);
        const float wp = pl[kb] * fast_exp2(pm[kb] - m_new);
        l_run = l_run * a + wp;
#pragma unroll
        for (int dt = 0; dt < 8; dt++)
#pragma unroll
            for (int i = 0; i < 4; i++) o[dt][i] = o[dt][i] * a + wp * (float)pv[kb][dt][i];
        m_run = m_new;
    }
    // private blocks: attended here, as attention_kernel does (the first one's pages requested
    // above)
    for (int kb = first_priv; kb < kSlots; kb++) {
        const int cid = __builtin_amdgcn_readlane(id, kb);
        if (cid < prefix_blocks) continue;  // shared, or unusable (-1)
        if (kb != first_priv) {
            const int pg = __builtin_amdgcn_readlane(page, kb);
            block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride, lds[wave], lane);
        }
        asm volatile("s_waitcnt vmcnt(9)" ::: "memory");  // the K page has arrived
        if (f16) attend_block<true, false>(lds[wave], lane, c, cid * kBlock, p, qop, logit_scale, m_run, l_run, o);
        else attend_block<false, false>(lds[wave], lane, c, cid * kBlock, p, qop, logit_scale, m_run, l_run, o);
    }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();  // every page buffer is free: the merge area

    // ---- merge the wavefronts: lane (n, c) holds o[dt][i] = out(head n, dim 16dt + 4c + i)
    float* sh_o = reinterpret_cast<float*>(&lds[0][0]);  // [kCombineWaves][16][kMergeStride]
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
#pragma unroll
        for (int i = 0; i < 4; i++)
            sh_o[(wave * kGroupHeads + n) * kMergeStride + 16 * dt + 4 * c + i] = o[dt][i];
    if (c == 0) {
        sh_m[wave][n] = m_run;
        sh_l[wave][n] = l_run;
    }
    __syncthreads();
    const int h = threadIdx.x >> 5;         // head 0..15
    const int d0 = (threadIdx.x & 31) * 4;  // 4 dims
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kCombineWaves; w++) M = fmaxf(M, sh_m[w][h]);
    float L = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kCombineWaves; w++) {
        const float wt = sh_m[w][h] == -INFINITY ? 0.f : fast_exp2(sh_m[w][h] - M);
        L += wt * sh_l[w][h];
#pragma unroll
        for (int e = 0; e < 4; e++) acc[e] += wt * sh_o[(w * kGroupHeads + h) * kMergeStride + d0 + e];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const uint32_t lo = (uint32_t)bf16_bits_rne(acc[0] * inv) | ((uint32_t)bf16_bits_rne(acc[1] * inv) << 16);
    const uint32_t hi = (uint32_t)bf16_bits_rne(acc[2] * inv) | ((uint32_t)bf16_bits_rne(acc[3] * inv) << 16);
    uint16_t* op = out + ((int64_t)r * kQHeads + kGroupHeads * g + h) * kDim + d0;
    *reinterpret_cast<uint2*>(op) = uint2{lo, hi};
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_attention)
#endif

int attn_num_splits(int batch, int q_len) {
    const long rows = (long)batch * q_len * kKvHeads;
    // enough workgroups to cover the 256 compute units, at most 4 splits (1 block per wave)
    if (rows >= 1024) return 1;
    if (rows >= 512) return 2;
    return 4;
}

// Workspace with split partials: one int32 counter per (row group, wavefront of four heads),
// zero between launches, padded to 256 bytes, then the partials.
static size_t attn_counter_bytes(int batch, int q_len) {
    return ((size_t)batch * q_len * kKvHeads * kWaves * sizeof(int32_t) + 255) / 256 * 256;
}

// Zeroes n 32-bit words (a plain kernel rather than a memset, so that a captured graph holds no
// memset node).
__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t* __restrict__ p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0u;
}

// Batches that take the union kernel (attention_union.hip): 2 to 4 query tokens per sequence and
// at least kUnionMinBatch sequences. There the attention is bound by page traffic and
// dequantization, which the union does once per (sequence, group) instead of once per token
// (128K context, 4 tokens: 24.7 against 26.3 us at 16 sequences, 31 against 53 us at 32,
// 46 against 70 us at 64). With fewer sequences the launch is bound by the latency of its
// steps, and the union's merge of its 64-row partials across splits costs more than it saves
// (8 sequences: 22.7 against 14.2 us), so the per-token kernel runs.
constexpr int kUnionMinBatch = 16;
static bool use_union(int batch, int q_len, int max_blocks, bool select) {
    return q_len >= 2 && q_len <= 4 && batch >= kUnionMinBatch &&
           max_blocks <= (select ? kSelectFusedMaxBlocks : kUnionAttnMaxBlocks);
}


hipError_t launch_attn_workspace_clear(void* workspace, int batch, int q_len, hipStream_t stream) {
    // the counters of whichever kernel runs sit at the start of the workspace
    size_t bytes = attn_num_splits(batch, q_len) > 1 ? attn_counter_bytes(batch, q_len) : 0;
    if (q_len >= 2 && q_len <= 4 && batch >= kUnionMinBatch && union_num_splits(batch) > 1 &&
        union_counter_bytes(batch) > bytes)
        bytes = union_counter_bytes(batch);
    if (bytes == 0) return hipSuccess;
    const int words = (int)(bytes / sizeof(uint32_t));
    const int grid = (words + 255) / 256 < 64 ? (words + 255) / 256 : 64;
    hipLaunchKernelGGL(clear_words_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<uint32_t*>(workspace), words);
    return hipGetLastError();
}

size_t attn_workspace_bytes(int batch, int q_len) {
    // enough for either kernel a call of this shape may run (the union kernel for 2 to 4 query
    // tokens per sequence, the per-token kernel for longer rows)
    const int ns = attn_num_splits(batch, q_len);
    size_t ws = ns == 1 ? 0
                        : attn_counter_bytes(batch, q_len) +
                              (size_t)batch * q_len * kKvHeads * ns * kGroupHeads * kPartStride * sizeof(float);
    if (q_len >= 2 && q_len <= 4 && batch >= kUnionMinBatch) {
        const size_t u = union_workspace_bytes(batch, q_len);
        if (u > ws) ws = u;
    }
    return ws;
}

namespace {

template <bool SELECT>
hipError_t launch_attention_t(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                              const int32_t* block_table, const int32_t* ctx_lens, int batch,
                              int max_blocks, int q_len, const uint16_t* q, int32_t* ids,
                              const float* scores, float softmax_scale, uint16_t* out,
                              void* workspace, hipStream_t stream) {
    const int ns = attn_num_splits(batch, q_len);
    const int pairs = batch * kKvHeads;
    const int pair_slots = 8 * ((pairs + 7) / 8);
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    if (use_union(batch, q_len, max_blocks, SELECT)) {
        // speculative verify: each (sequence, group) reads the union of its drafts' blocks once
        return launch_attention_union(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                      max_blocks, q_len, q, ids, SELECT ? scores : nullptr,
                                      kTopk, scale_log2, out, workspace, stream);
    }
    if (ns == 1 && q_len >= kTileMinQ && max_blocks <= kUnionMaxBlocks) {
        // many tokens per sequence: token tiles over the union of their blocks (the selection,
        // if asked for, as its own launch first)
        if constexpr (SELECT) {
            const hipError_t err = launch_topk(scores, ctx_lens, batch, max_blocks, q_len, ids, stream);
            if (err != hipSuccess) return err;
        }
        const int tiles = (q_len + kTileTokens - 1) / kTileTokens;
        hipLaunchKernelGGL(attention_tile_kernel, dim3(pair_slots * tiles), dim3(kTileWaves * 64),
                           0, stream, k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                           max_blocks, q_len, q, ids, scale_log2, out);
        return hipGetLastError();
    }
    const dim3 grid(pair_slots * q_len * ns), block(kWaves * 64);
    int32_t* counters = nullptr;
    float* partials = nullptr;
    if (ns > 1) {
        counters = static_cast<int32_t*>(workspace);
        partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                            attn_counter_bytes(batch, q_len));
    }
#define MSA_LAUNCH_ATTN(BPW_)                                                                    \
    hipLaunchKernelGGL((attention_kernel<BPW_, SELECT>), grid, block, 0, stream, k_pool, v_pool, \
                       num_pages, block_table, ctx_lens, batch, max_blocks, q_len, q, ids,       \
                       scores, scale_log2, out, counters, partials, kTopk)
    switch (ns) {
        case 1: MSA_LAUNCH_ATTN(4); break;
        case 2: MSA_LAUNCH_ATTN(2); break;
        default: MSA_LAUNCH_ATTN(1); break;
    }
#undef MSA_LAUNCH_ATTN
    return hipGetLastError();
}

// Rows of kSelectFusedMaxBlocks + 1 .. kSelectLongMaxBlocks blocks with four splits (the
// per-token kernel with one block per wavefront): the selection in the attention launch, shared
// by the workgroup's four wavefronts.
hipError_t launch_attention_long_select(const uint8_t* k_pool, const uint8_t* v_pool,
                                        int64_t num_pages, const int32_t* block_table,
                                        const int32_t* ctx_lens, int batch, int max_blocks,
                                        int q_len, const uint16_t* q, int32_t* ids,
                                        const float* scores, float softmax_scale, uint16_t* out,
                                        void* workspace, hipStream_t stream) {
    const int pairs = batch * kKvHeads;
    const int pair_slots = 8 * ((pairs + 7) / 8);
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    int32_t* counters = static_cast<int32_t*>(workspace);
    float* partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                               attn_counter_bytes(batch, q_len));
    hipLaunchKernelGGL((attention_kernel<1, true, true>), dim3(pair_slots * q_len * kMaxSplits),
                       dim3(kWaves * 64), 0, stream, k_pool, v_pool, num_pages, block_table,
                       ctx_lens, batch, max_blocks, q_len, q, ids, scores, scale_log2, out,
                       counters, partials, kTopk);
    return hipGetLastError();
}

}  // namespace

// Rows of topk (1..64) ids: rows of up to kTopk ids on the union kernel wherever the 16-id call
// runs it, else the per-token kernel with the splits of the 16-id calls and
// ceil(topk / (4 splits)) slots per wavefront, streamed through one page buffer per wavefront:
// 74 KB of LDS per workgroup, so two workgroups share a compute unit and hide each other's
// copies, where two buffers (144 KB) would leave one workgroup per compute unit (at 64 ids,
// 8 sequences of 128K tokens with 4 query tokens: 31.8 against 39.5 us per launch). (The union
// kernel over rows of 64 ids, whose splits each stream a long run of union blocks, is slower
// still there: 62 us.)
hipError_t launch_attention_topk(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                 const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                 int max_blocks, int q_len, const uint16_t* q, const int32_t* ids,
                                 int topk, float softmax_scale, uint16_t* out, void* workspace,
                                 hipStream_t stream) {
    const int ns = attn_num_splits(batch, q_len);
    const int pairs = batch * kKvHeads;
    const int pair_slots = 8 * ((pairs + 7) / 8);
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    if (topk <= kTopk && use_union(batch, q_len, max_blocks, false))
        return launch_attention_union(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                      max_blocks, q_len, q, const_cast<int32_t*>(ids), nullptr,
                                      topk, scale_log2, out, workspace, stream);
    const dim3 grid(pair_slots * q_len * ns), block(kWaves * 64);
    int32_t* counters = nullptr;
    float* partials = nullptr;
    if (ns > 1) {
        counters = static_cast<int32_t*>(workspace);
        partials = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                            attn_counter_bytes(batch, q_len));
    }
    static_assert(kMaxTopkIds <= 16 * kWaves, "one split holds 16 slots per wavefront at most");
#define MSA_LAUNCH_ATTN_VAR(NS_)                                                                 \
    hipLaunchKernelGGL((attention_kernel<1, false, false, NS_, true>), grid, block, 0, stream,   \
                       k_pool, v_pool, num_pages, block_table, ctx_lens, batch, max_blocks,      \
                       q_len, q, const_cast<int32_t*>(ids), nullptr, scale_log2, out, counters,  \
                       partials, topk)
    switch (ns) {
        case 1: MSA_LAUNCH_ATTN_VAR(1); break;
        case 2: MSA_LAUNCH_ATTN_VAR(2); break;
        default: MSA_LAUNCH_ATTN_VAR(4); break;
    }
#undef MSA_LAUNCH_ATTN_VAR
    return hipGetLastError();
}

hipError_t launch_attention(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                            const int32_t* block_table, const int32_t* ctx_lens, int batch,
                            int max_blocks, int q_len, const uint16_t* q, const int32_t* ids,
                            float softmax_scale, uint16_t* out, void* workspace,
                            hipStream_t stream) {
    return launch_attention_t<false>(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                     max_blocks, q_len, q, const_cast<int32_t*>(ids), nullptr,
                                     softmax_scale, out, workspace, stream);
}

hipError_t launch_select_attention(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                   const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                   int max_blocks, int q_len, const float* scores, int32_t* ids,
                                   const uint16_t* q, float softmax_scale, uint16_t* out,
                                   void* workspace, hipStream_t stream) {
    if (max_blocks > kSelectFusedMaxBlocks && max_blocks <= kSelectLongMaxBlocks &&
        attn_num_splits(batch, q_len) == kMaxSplits && !use_union(batch, q_len, max_blocks, false))
        return launch_attention_long_select(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                            max_blocks, q_len, q, ids, scores, softmax_scale, out,
                                            workspace, stream);
    if (max_blocks > kSelectFusedMaxBlocks) {
        // longer rows: the selection kernel for them, then the attention reading its ids
        const hipError_t err = launch_topk(scores, ctx_lens, batch, max_blocks, q_len, ids, stream);
        if (err != hipSuccess) return err;
        return launch_attention(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                max_blocks, q_len, q, ids, softmax_scale, out, workspace, stream);
    }
    return launch_attention_t<true>(k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                                    max_blocks, q_len, q, ids, scores, softmax_scale, out,
                                    workspace, stream);
}

int attn_shared_prefix_max_rows() { return kSharedMaxRows; }

size_t attn_shared_prefix_workspace_bytes(int batch, int q_len) {
    return (size_t)batch * q_len * kKvHeads * kTopk * kSPartBytes;
}

hipError_t launch_attention_shared_prefix(const uint8_t* k_pool, const uint8_t* v_pool,
                                          int64_t num_pages, const int32_t* block_table,
                                          const int32_t* ctx_lens, int batch, int max_blocks,
                                          int q_len, const uint16_t* q, const int32_t* ids,
                                          int prefix_blocks, float softmax_scale, uint16_t* out,
                                          void* workspace, hipStream_t stream) {
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    uint8_t* parts = static_cast<uint8_t*>(workspace);
    if (prefix_blocks > 0) {
        hipLaunchKernelGGL(shared_block_kernel, dim3(prefix_blocks * kKvHeads), dim3(kTileWaves * 64),
                           0, stream, k_pool, v_pool, num_pages, block_table, ctx_lens, batch,
                           max_blocks, q_len, q, ids, scale_log2, parts);
        const hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(shared_combine_kernel, dim3(batch * q_len * kKvHeads), dim3(kCombineWaves * 64), 0,
                       stream, k_pool, v_pool, num_pages, block_table, ctx_lens, batch, max_blocks,
                       q_len, q, ids, prefix_blocks, scale_log2, parts, out);
    return hipGetLastError();
}

}  // namespace msa
