// MSA sparse GQA attention for speculative verify: 2 to 4 query tokens per sequence, the drafts'
// blocks read and dequantized once per (sequence, group).
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": each query head of a GQA
// group attends exactly to the blocks its group's indexer kept; section "Indexer NVFP4 DCP"
// (AMD part): with only a few query rows per group the matrix cores run mostly empty. "MiniMax M3
// on vLLM", section "Speculative decoding in the decode kernels": the draft tokens of a request
// are flattened into query rows with their own causal positions; section "MiniMax sparse
// attention backend": the decode kernel reads the selected pages and merges partial outputs.
//
// The draft tokens of one (sequence b, group g) pair select nearly the same blocks (16 per row,
// or up to 16 with the window knobs). Here the pair's query rows (QL tokens x 16 heads, QL row
// tiles of the matrix cores) are computed together, over the union of the drafts' selections:
// each union block streams into LDS once and is dequantized once for every draft. A draft that
// did not select a union block gets zero probabilities for it, and one whose row lists a block
// several times weights its keys that many times, so each row's result is exactly the attention
// over its own selection.
//
// Work: n_split workgroups per pair take contiguous ranges of the union. A workgroup has eight
// wavefronts, wavefront (w, h) = (token quarter, half of the row tiles): for every block it works
// on tokens 32c + 8w + (0..7) (c = 0..3; K slabs 2w and 2w + 1 of the row-operand layout) for row
// tiles RT h .. RT h + RT - 1, RT = ceil(QL / 2):
//   S^T = K Q^T on v_mfma_f32_16x16x32_f16 (two 16-token tiles per row tile),
//   fp32 online softmax per row over the wavefront's tokens (lazy rescale),
//   O^T += V^T P^T, one 32-token step per row tile and 16-dim tile (lane (n, c) holds dim
//   16 dt + n of its eight tokens: one 32-bit code word and two scale words).
// The block's K and V pages are copied global->LDS by all eight wavefronts (double buffered).
// At the end the four token quarters of each row tile merge in LDS. With several splits each
// wavefront publishes a quarter of the dims of its row tiles (normalized fp16 values and the
// rows' fp32 max and sum) and counts itself on the pair's counter for them; the last of the
// splits to arrive merges all the splits' values by log-sum-exp, in split order, and writes bf16.
#include "device_common.hpp"
#include "kernels.hpp"
#include "select_wave.hpp"

namespace msa {
namespace {

constexpr int kUHalves = 2;                       // wavefronts per token quarter (row-tile halves)
constexpr int kUWaves = 4 * kUHalves;             // 4 token quarters x kUHalves parts of the row tiles
constexpr int kUBlockBytes = 2 * kHeadPageBytes;  // K page then V page of one (block, group)
constexpr int kUMaxSplits = 8;
constexpr int kUMaxQL = 4;
constexpr int kUMaxUnion = kUMaxQL * kTopk;
constexpr int kUMergeStride = kDim + 4;           // floats per LDS row of the wavefront merge
// LDS of the page buffers, reused by the final merge of the token quarters
constexpr int kUMergeBytes = kUHalves * 4 * kGroupHeads * kUMergeStride * 4;
constexpr int kUScratchBytes = kUMergeBytes > 2 * kUBlockBytes ? kUMergeBytes : 2 * kUBlockBytes;
// Lazy rescaling (log2 units): a row keeps its running maximum until a block's maximum exceeds
// it by more than this, so probabilities stay below 2^8 (well inside fp16).
constexpr float kUTau = 8.0f;
// Cache policy of the split partials: sc1, written through to and read from the point where
// every XCD sees the same data.
constexpr int kCoherent = 16;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t bf16_rne(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// First n bytes of a word kept (all for n >= 4, none for n <= 0).
__device__ __forceinline__ uint32_t keep_first_bytes(int n) {
    return n >= 4 ? 0xFFFFFFFFu : (n <= 0 ? 0u : (1u << (8 * n)) - 1u);
}

// The 18 one-kilobyte pieces of a block's K and V pages, copied global->LDS by the eight
// wavefronts together (piece i by wavefront i % 8).
__device__ __forceinline__ void union_block_to_lds(const uint8_t* kp, const uint8_t* vp,
                                                   uint8_t* buf, int wave, int lane) {
#pragma unroll
    for (int r = 0; r < 3; r++) {
        const int i = wave + kUWaves * r;
        if (i < 18) {
            const uint8_t* src = i < 9 ? kp + i * 1024 : vp + (i - 9) * 1024;
            __builtin_amdgcn_global_load_lds(src + lane * 16, (lds_void*)(buf + i * 1024), 16, 0, 0);
        }
    }
}

// LDS reads of page data, each group issued and waited for inside one statement (page copies
// for the next block are in flight meanwhile, and the compiler would otherwise wait for them).
__device__ __forceinline__ void lds_read_k(u32x4& c0, u32x4& c1, uint32_t& sc, uint32_t a,
                                           uint32_t as) {
    asm volatile("ds_read_b128 %0, %3\n\t"
                 "ds_read_b128 %1, %3 offset:1024\n\t"
                 "ds_read_b32 %2, %4\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(c0), "=&v"(c1), "=&v"(sc)
                 : "v"(a), "v"(as)
                 : "memory");
}
// V codes of one dim (8 tokens, one word) for each of the eight 16-dim tiles, and the eight
// tokens' scale bytes (two words) for each tile.
__device__ __forceinline__ void lds_read_v(uint32_t (&code)[8], uint2 (&sc)[8], uint32_t a,
                                           uint32_t as) {
    asm volatile("ds_read_b32 %0, %16\n\t"
                 "ds_read_b32 %1, %16 offset:1024\n\t"
                 "ds_read_b32 %2, %16 offset:2048\n\t"
                 "ds_read_b32 %3, %16 offset:3072\n\t"
                 "ds_read_b32 %4, %16 offset:4096\n\t"
                 "ds_read_b32 %5, %16 offset:5120\n\t"
                 "ds_read_b32 %6, %16 offset:6144\n\t"
                 "ds_read_b32 %7, %16 offset:7168\n\t"
                 "ds_read_b64 %8, %17\n\t"
                 "ds_read_b64 %9, %17 offset:128\n\t"
                 "ds_read_b64 %10, %17 offset:256\n\t"
                 "ds_read_b64 %11, %17 offset:384\n\t"
                 "ds_read_b64 %12, %17 offset:512\n\t"
                 "ds_read_b64 %13, %17 offset:640\n\t"
                 "ds_read_b64 %14, %17 offset:768\n\t"
                 "ds_read_b64 %15, %17 offset:896\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(code[0]), "=&v"(code[1]), "=&v"(code[2]), "=&v"(code[3]),
                   "=&v"(code[4]), "=&v"(code[5]), "=&v"(code[6]), "=&v"(code[7]),
                   "=&v"(sc[0]), "=&v"(sc[1]), "=&v"(sc[2]), "=&v"(sc[3]), "=&v"(sc[4]),
                   "=&v"(sc[5]), "=&v"(sc[6]), "=&v"(sc[7])
                 : "v"(a), "v"(as)
                 : "memory");
}
// A union entry (block id, page, drafts), three 32-bit LDS reads waited for inside the statement.
__device__ __forceinline__ void lds_read_entry(int& x, int& y, int& z, uint32_t ax, uint32_t ay,
                                               uint32_t az) {
    asm volatile("ds_read_b32 %0, %3\n\t"
                 "ds_read_b32 %1, %4\n\t"
                 "ds_read_b32 %2, %5\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(x), "=&v"(y), "=&v"(z)
                 : "v"(ax), "v"(ay), "v"(az)
                 : "memory");
}

// One union block for one wavefront: its quarter w of the block's tokens for its RT row tiles
// (tiles tile0 .. tile0 + RT - 1; a tile at or past QL is never selected). `buf` holds the
// block's K and V pages; tok0 = first token of the block; p = position of each of its tiles'
// drafts (lowest first); dm = how many times each draft's row lists the block, one byte per
// draft, shifted so byte i is tile0 + i (0: not selected; at most 1 unless MULTI); T = context
// length.
template <int RT, bool F16, bool MULTI>
__device__ __forceinline__ void union_attend_block(const uint8_t* buf, int w, int lane, int c,
                                                   int n, int tok0, int T, const int (&p)[RT],
                                                   int dm, const u32x4 (&qop)[RT][4],
                                                   const float (&ls)[RT], float (&m_run)[RT],
                                                   float (&l_run)[RT], f32x4 (&o)[RT][8]) {
    const uint32_t kb = (uint32_t)(uintptr_t)buf;
    // ---- logits: K slabs 2w, 2w + 1 (token 32c' + 8w + 4tt + i in MFMA row 4c' + i)
    u32x4 kc[2];
    uint32_t ksc;
    lds_read_k(kc[0], kc[1], ksc, kb + 2048 * w + 16 * lane, kb + kCodeBytes + 16 * lane + 4 * w);
    f32x4 sv[RT][2];
#pragma unroll
    for (int tt = 0; tt < 2; tt++) {
        f16x2 s0, s1;
        if (tt) e4m3_pair_f16<true>(ksc, s0, s1);
        else e4m3_pair_f16<false>(ksc, s0, s1);
        f16x8 a[4];
#pragma unroll
        for (int m = 0; m < 4; m++) a[m] = dequant8_f16(kc[tt][m], m < 2 ? s0 : s1);
#pragma unroll
        for (int i = 0; i < RT; i++) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; m++) {
                if constexpr (F16)
                    acc = mfma_f16_k32(a[m], __builtin_bit_cast(f16x8, qop[i][m]), acc);
                else
                    acc = mfma_bf16_k32(f16x8_to_bf16x8(a[m]), __builtin_bit_cast(bf16x8, qop[i][m]), acc);
            }
            sv[i][tt] = acc;  // lane (n, c): head n, tokens tok0 + 32c + 8w + 4tt + i
        }
    }
    // ---- causal mask: only in a block that holds a draft's position (a scalar branch)
    if (tok0 + kBlock - 1 > p[0]) {
        asm volatile("");
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const int last = p[i] - tok0 - 32 * c - 8 * w;  // values 4tt + e <= last visible
#pragma unroll
            for (int tt = 0; tt < 2; tt++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    uint32_t past = (uint32_t)((last - (4 * tt + e)) >> 31);
                    asm("" : "+v"(past));
                    sv[i][tt][e] = __uint_as_float((__float_as_uint(sv[i][tt][e]) & ~past) | (0xFF800000u & past));
                }
        }
    }
    // ---- online softmax per row tile; probabilities in the B-operand order of the P.V step
    // (k = 8c + 4tt + e <-> token 32c + 8w + 4tt + e). A tile whose draft did not select the
    // block takes its exponent against +inf: all its probabilities are 0.
    f16x8 pt[RT];
#pragma unroll
    for (int i = 0; i < RT; i++) {
        const int cnt = (dm >> (8 * i)) & 0xFF;  // (wavefront-uniform)
        const bool sel = cnt != 0;
        float mb = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int e = 0; e < 4; e++) mb = fmaxf(mb, sv[i][tt][e]);
        mb = sel ? max_over_c(mb) * ls[i] : -INFINITY;  // -inf: no visible token of this quarter
        const float m_new = (mb > m_run[i] + kUTau) ? mb : m_run[i];
        if (__any(m_new != m_run[i])) {
            const float alpha = exp2_hw(m_run[i] - m_new);  // 0 from -inf (o, l are 0)
            l_run[i] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; dt++) o[i][dt] *= alpha;
            m_run[i] = m_new;
        }
        const float mu = !sel ? INFINITY : (m_new == -INFINITY ? 0.f : m_new);
        float sum = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; tt++)
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float x = exp2_hw(fmaf(sv[i][tt][e], ls[i], -mu));
                sum += x;
                pt[i][4 * tt + e] = (_Float16)x;
            }
        if (MULTI && cnt > 1) {
            // a block listed cnt times in the draft's row: each of its keys counts cnt times
            const float mult = (float)cnt;
            sum *= mult;
#pragma unroll
            for (int e = 0; e < 8; e++) pt[i][e] *= (_Float16)mult;
        }
        l_run[i] += sum;  // this lane's tokens; the four lanes of a row add up at the end
    }
    // ---- O^T += V^T P^T: lane (n, c) holds dim 16 dt + n of tokens 32c + 8w + (0..7)
    uint32_t vcode[8];
    uint2 vsc[8];
    lds_read_v(vcode, vsc, kb + kHeadPageBytes + n * 64 + 16 * c + 4 * w,
               kb + kHeadPageBytes + kCodeBytes + 32 * c + 8 * w);
    if (tok0 + kBlock - 1 >= T) {
        // tokens at or past the context length: scales read as 0, so bytes never written (an
        // E4M3 NaN among them) cannot reach the output through a zero probability
        asm volatile("");
        const int first = tok0 + 32 * c + 8 * w;
        const uint32_t k0 = keep_first_bytes(T - first), k1 = keep_first_bytes(T - first - 4);
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
            vsc[dt].x &= k0;
            vsc[dt].y &= k1;
        }
    }
#pragma unroll
    for (int dt = 0; dt < 8; dt++) {
        const uint32_t s01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc[dt].x, 1.0f, false));
        const uint32_t s23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc[dt].x, 1.0f, true));
        const uint32_t s45 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc[dt].y, 1.0f, false));
        const uint32_t s67 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(vsc[dt].y, 1.0f, true));
        const f16x4 a0 = dequant4_f16_scaled<0>(vcode[dt], s01, s23);
        const f16x4 a1 = dequant4_f16_scaled<2>(vcode[dt], s45, s67);
        const f16x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int i = 0; i < RT; i++) o[i][dt] = mfma_f16_k32(a, pt[i], o[i][dt]);
    }
}

// The union blocks [lo, hi) of one split: double-buffered page copies, a workgroup barrier per
// block, then this wavefront's part of each block (one instantiation per operand type; MULTI:
// a row may list a block more than once).
template <int RT, bool F16, bool MULTI, class Issue, class Entry>
__device__ __forceinline__ void union_loop(uint8_t* pages, int lo, int hi, Issue issue, Entry entry,
                                           int w, int tile0, int lane, int c, int n, int T,
                                           const int (&p)[RT], const u32x4 (&qop)[RT][4],
                                           const float (&ls)[RT], float (&m_run)[RT],
                                           float (&l_run)[RT], f32x4 (&o)[RT][8]) {
    for (int u = lo; u < hi; u++) {
        // block u has landed for every wavefront, and every wavefront is done with block u - 1,
        // whose buffer the next copies overwrite
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int bi = (u - lo) & 1;
        if (u + 1 < hi) issue(u + 1, pages + (bi ^ 1) * kUBlockBytes);
        int id, pg, dm;
        entry(u, id, pg, dm);
        if (pg < 0) continue;  // (uniform)
        union_attend_block<RT, F16, MULTI>(pages + bi * kUBlockBytes, w, lane, c, n, id * kBlock, T, p,
                                    dm >> (8 * tile0), qop, ls, m_run, l_run, o);
    }
}

// Bytes one wavefront publishes per split: RT row tiles x 64 lanes x 16 B of normalized output
// (fp16), then RT x 16 rows x 16 B (max, sum as fp32, two unused words).
template <int RT>
constexpr int union_wave_part_bytes() { return RT * (64 * 16 + 16 * 16); }

template <int QL, bool SELECT>
__global__ __launch_bounds__(kUWaves * 64) void attention_union_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int batch,
    int max_blocks, int n_split, const uint16_t* __restrict__ q, int32_t* __restrict__ block_ids,
    const float* __restrict__ scores, float scale_log2, uint16_t* __restrict__ out,
    int32_t* __restrict__ counters, uint8_t* __restrict__ partials, int ids_per_row) {
    static_assert(QL >= 2 && QL <= kUMaxQL, "2 to 4 query tokens per sequence");
    constexpr int RT = (QL + kUHalves - 1) / kUHalves;  // row tiles per wavefront
    constexpr int kWords = ((SELECT ? kSelectFusedMaxBlocks : kUnionAttnMaxBlocks) + 63) / 64;
    __shared__ __attribute__((aligned(16))) uint8_t scratch[kUScratchBytes];
    static_assert(kUMaxQL * kSelectScratch * 8 <= kUBlockBytes, "selection scratch in a page buffer");
    __shared__ int sh_sel[kUMaxQL][kTopk];
    __shared__ uint64_t sh_bits[kWords];
    __shared__ uint64_t sh_dbits[QL][kWords];
    __shared__ int sh_prefix[kWords];
    __shared__ int sh_ulist[kUMaxUnion];
    __shared__ int sh_upage[kUMaxUnion];
    __shared__ int sh_udm[kUMaxUnion];
    __shared__ int sh_ucount;
    __shared__ int sh_tbl[SELECT ? kSelectFusedMaxBlocks : 1];
    __shared__ float sh_m[kUWaves][RT][kGroupHeads];
    __shared__ float sh_l[kUWaves][RT][kGroupHeads];

    const int lane = threadIdx.x & 63;
    // wavefront-uniform (scalar) roles: w = token quarter, h = half of the row tiles
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = wave & 3;
    const int h = wave >> 2;
    const int tile0 = RT * h;
    const int n = lane & 15;
    const int c = lane >> 4;
    // XCD-aware mapping: pair (b, g) -> XCD pair % 8, all its splits there
    const int local = blockIdx.x >> 3;
    const int pair = (local / n_split) * 8 + (blockIdx.x & 7);
    if (pair >= batch * kKvHeads) return;
    const int split = local - (local / n_split) * n_split;
    const int b = pair >> 2;
    const int g = pair & 3;

    // this wavefront's query rows (the B operand of S^T: head 16g + n, dims 32c + 8m .. +7),
    // requested first (a tile past QL reads the last draft's rows and is never used)
    u32x4 qraw[RT][4];
#pragma unroll
    for (int i = 0; i < RT; i++) {
        const int j = min(tile0 + i, QL - 1);
        const uint16_t* qp = q + ((int64_t)(b * QL + j) * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
        for (int m = 0; m < 4; m++) qraw[i][m] = *reinterpret_cast<const u32x4*>(qp + 8 * m);
    }
    const int T_raw = ctx_lens[b];
    for (int i = threadIdx.x; i < kWords; i += kUWaves * 64) sh_bits[i] = 0ull;
    for (int i = threadIdx.x; i < QL * kWords; i += kUWaves * 64) (&sh_dbits[0][0])[i] = 0ull;
    for (int i = threadIdx.x; i < kUMaxUnion; i += kUWaves * 64) sh_udm[i] = 0;

    // ---- each draft's selection: wavefront j (< QL) selects draft j's row; the others copy the
    // sequence's block-table row into LDS
    if constexpr (SELECT) {
        constexpr int kThr = (kUWaves - QL) * 64;
        constexpr int kPer = (kSelectFusedMaxBlocks + kThr - 1) / kThr;
        if (wave < QL) {
            const int rg = (b * QL + wave) * kKvHeads + g;
            float sv[16];
            load_row_scores<16>(scores + (int64_t)rg * max_blocks, max_blocks, lane, sv);
            const int p_sel = clamp_ctx(T_raw, max_blocks) - QL + wave;
            select_row<16>(sv, eligible_blocks(p_sel, max_blocks), lane,
                           reinterpret_cast<uint64_t*>(scratch + wave * kSelectScratch * 8), sh_sel[wave]);
            if (split == 0 && lane < kTopk) block_ids[(int64_t)rg * kTopk + lane] = sh_sel[wave][lane];
        } else {
            // (indexes past the row are clamped to its last entry and rewrite it with its value)
            const int t0 = threadIdx.x - QL * 64;
            const int32_t* trow = block_table + (int64_t)b * max_blocks;
            int tv[kPer];
#pragma unroll
            for (int r = 0; r < kPer; r++) tv[r] = trow[min(t0 + r * kThr, max_blocks - 1)];
#pragma unroll
            for (int r = 0; r < kPer; r++) sh_tbl[min(t0 + r * kThr, max_blocks - 1)] = tv[r];
        }
    } else {
        // draft j's row of ids_per_row (1 .. kTopk) ids
        if (wave < QL && lane < kTopk) {
            const int32_t* row = block_ids + ((int64_t)(b * QL + wave) * kKvHeads + g) * ids_per_row;
            sh_sel[wave][lane] = lane < ids_per_row ? row[lane] : -1;
        }
    }
    const int T = clamp_ctx(T_raw, max_blocks);
    __syncthreads();

    // ---- the union of the drafts' usable blocks (in range, holding a key visible to the draft),
    // in ascending order, by wavefront 0: candidate l = entry l % 16 of draft l / 16. Every union
    // entry counts, per draft, how many times the draft's row lists it (one byte per draft).
    if (wave == 0) {
        const int jd = lane >> 4;
        int x = -1;
        if (jd < QL) {
            const int id = sh_sel[jd][lane & 15];
            if (id >= 0 && id < max_blocks && id * kBlock <= T - QL + jd) x = id;
        }
        if (x >= 0) {
            atomicOr(reinterpret_cast<unsigned long long*>(&sh_bits[x >> 6]), 1ull << (x & 63));
            atomicOr(reinterpret_cast<unsigned long long*>(&sh_dbits[jd][x >> 6]), 1ull << (x & 63));
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        // exclusive prefix counts of the bitmap words (64 words per pass)
        const int nwords = (max_blocks + 63) >> 6;
        int base = 0;
        for (int w0 = 0; w0 < nwords; w0 += 64) {
            const int wi = w0 + lane;
            const int cnt = wi < nwords ? popc64(sh_bits[wi]) : 0;
            int incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d, 64);
                if (lane >= d) incl += y;
            }
            if (wi < nwords) sh_prefix[wi] = base + incl - cnt;
            base += __shfl(incl, 63, 64);
        }
        __builtin_amdgcn_wave_barrier();
        asm volatile("" ::: "memory");
        if (x >= 0) {
            const int wd = x >> 6;
            const uint64_t below = (1ull << (x & 63)) - 1ull;
            const int r = sh_prefix[wd] + popc64(sh_bits[wd] & below);
            atomicAdd(&sh_udm[r], 1 << (8 * jd));
            int dm = 0;
#pragma unroll
            for (int j = 0; j < QL; j++) dm |= (int)((sh_dbits[j][wd] >> (x & 63)) & 1ull) << j;
            if ((dm & ((1 << jd) - 1)) == 0) {  // the first draft that holds x writes its entry
                sh_ulist[r] = x;
                const int pg = SELECT ? sh_tbl[x] : block_table[(int64_t)b * max_blocks + x];
                sh_upage[r] = (pg >= 0 && pg < num_pages) ? pg : -1;
            }
        }
        if (lane == 0) sh_ucount = base;
    }
    __syncthreads();
    const int U = sh_ucount;
    MSA_CHECK(threadIdx.x != 0 || (T_raw >= QL && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    MSA_CHECK(U <= kUMaxUnion && max_blocks <= kWords * 64, kCheckLds);
    MSA_CHECK(split < n_split && n_split <= kUMaxSplits && b < batch, kCheckWorkspace);
#ifdef MSA_CHECKED
    if constexpr (SELECT) {
        // each draft's ids: ascending within its eligible blocks, the block of its token last
        if (wave < QL && lane < kTopk) {
            const int n_el = eligible_blocks(T - QL + wave, max_blocks);
            const int kept = min(kTopk, n_el);
            const int v = sh_sel[wave][lane];
            MSA_CHECK(lane < kept ? (v >= 0 && v < n_el && (lane == 0 || v > sh_sel[wave][lane - 1]) &&
                                     (lane != kept - 1 || v == n_el - 1))
                                  : v == -1,
                      kCheckSelection);
        }
    }
#endif
    const int lo = (int)(((int64_t)split * U) / n_split);
    const int hi = (int)(((int64_t)(split + 1) * U) / n_split);
    // every load so far is complete, and the compiler knows it (none is waited for between the
    // page copies below)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0);

    const uint8_t* kg = k_pool + (int64_t)g * kHeadPageBytes;
    const uint8_t* vg = v_pool + (int64_t)g * kHeadPageBytes;
    constexpr int64_t kPageStride = (int64_t)kKvHeads * kHeadPageBytes;
    auto entry = [&](int u, int& id_u, int& page_u, int& dm_u) {
        int x, y, z;
        lds_read_entry(x, y, z, (uint32_t)(uintptr_t)&sh_ulist[u], (uint32_t)(uintptr_t)&sh_upage[u],
                       (uint32_t)(uintptr_t)&sh_udm[u]);
        id_u = __builtin_amdgcn_readfirstlane(x);
        page_u = __builtin_amdgcn_readfirstlane(y);
        dm_u = __builtin_amdgcn_readfirstlane(z);
    };
    auto issue = [&](int u, uint8_t* buf) {
        int id_u, pg, dm_u;
        entry(u, id_u, pg, dm_u);
        if (pg >= 0) union_block_to_lds(kg + pg * kPageStride, vg + pg * kPageStride, buf, wave, lane);
    };
    if (lo < hi) issue(lo, scratch);

    // ---- this wavefront's query operand, made while the first block streams in: fp16 after a
    // per-row power-of-two scaling when every row of its tiles converts exactly (every usual
    // row does), else the bf16 values
    u32x4 qop[RT][4];
    float ls[RT];
    int p[RT];
    u32x4 qconv[RT][4];
    float q_unscale[RT];
    bool exact = true;
#pragma unroll
    for (int i = 0; i < RT; i++) {
        bf16x8 t[4];
        f16x8 hq[4];
#pragma unroll
        for (int m = 0; m < 4; m++) t[m] = __builtin_bit_cast(bf16x8, qraw[i][m]);
        exact = query_to_f16(t, hq, q_unscale[i]) && exact;
#pragma unroll
        for (int m = 0; m < 4; m++) qconv[i][m] = __builtin_bit_cast(u32x4, hq[m]);
    }
    const bool f16 = __all(exact);
#pragma unroll
    for (int i = 0; i < RT; i++) {
#pragma unroll
        for (int m = 0; m < 4; m++) {
            qop[i][m] = f16 ? qconv[i][m] : qraw[i][m];
            // a negative softmax scale: the exactly negated query times the scale's magnitude
            if (scale_log2 < 0.f) qop[i][m] ^= 0x80008000u;
        }
        ls[i] = fabsf(scale_log2) * (f16 ? q_unscale[i] : 1.0f);
        p[i] = T - QL + min(tile0 + i, QL - 1);
    }
    float m_run[RT], l_run[RT];
    f32x4 o[RT][8];
#pragma unroll
    for (int i = 0; i < RT; i++) {
        m_run[i] = -INFINITY;
        l_run[i] = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[i][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (f16)
        union_loop<RT, true, !SELECT>(scratch, lo, hi, issue, entry, w, tile0, lane, c, n, T, p, qop, ls, m_run, l_run, o);
    else
        union_loop<RT, false, !SELECT>(scratch, lo, hi, issue, entry, w, tile0, lane, c, n, T, p, qop, ls, m_run, l_run, o);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();  // the page buffers are free: the merge below reuses them

    // ---- merge the four token quarters of each row tile in LDS
#pragma unroll
    for (int i = 0; i < RT; i++) {
        const float lsum = sum_over_c(l_run[i]);
        if (c == 0) {
            sh_m[wave][i][n] = m_run[i];
            sh_l[wave][i][n] = lsum;
        }
    }
    __syncthreads();
    float M[RT], L[RT], own[RT];
#pragma unroll
    for (int i = 0; i < RT; i++) {
        float mx = -INFINITY;
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) mx = fmaxf(mx, sh_m[4 * h + q4][i][n]);
        float l = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const float mw = sh_m[4 * h + q4][i][n];
            l += (mw == -INFINITY) ? 0.f : exp2_hw(mw - mx) * sh_l[4 * h + q4][i][n];
        }
        M[i] = mx;
        L[i] = l;
        own[i] = (m_run[i] == -INFINITY) ? 0.f : exp2_hw(m_run[i] - mx);
    }
    // lane (n, c) of wavefront (w, h) ends with dims 32w + 8c .. +7 of head n of its tiles
    float R[RT][8];
    float* sh_o = reinterpret_cast<float*>(scratch);  // [2 halves][4 quarters][16][kUMergeStride]
#pragma unroll
    for (int i = 0; i < RT; i++) {
#pragma unroll
        for (int dt = 0; dt < 8; dt++)
#pragma unroll
            for (int e = 0; e < 4; e++)
                sh_o[((h * 4 + w) * kGroupHeads + n) * kUMergeStride + 16 * dt + 4 * c + e] = o[i][dt][e] * own[i];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float x = 0.f;
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++)
                x += sh_o[((h * 4 + q4) * kGroupHeads + n) * kUMergeStride + 32 * w + 8 * c + e];
            R[i][e] = x;
        }
        __syncthreads();
    }

    if (n_split > 1) {
        // publish this wavefront's dims of its tiles: normalized fp16 values and the rows' (max,
        // sum), written through to the device coherence point and complete before the counter
        // moves
        const uint32_t part_bytes = (uint32_t)union_wave_part_bytes<RT>();
        const uint32_t pair_bytes = kUWaves * part_bytes;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            partials + (int64_t)pair * n_split * pair_bytes, 0, (int)(n_split * pair_bytes), 0x00020000);
        const uint32_t mine = (uint32_t)split * pair_bytes + wave * part_bytes;
        u32x4 own_h[RT], own_ml[RT];
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const float inv = L[i] > 0.f ? 1.f / L[i] : 0.f;
            f16x8 hv;
#pragma unroll
            for (int e = 0; e < 8; e++) hv[e] = (_Float16)(R[i][e] * inv);
            own_h[i] = __builtin_bit_cast(u32x4, hv);
            own_ml[i] = u32x4{__float_as_uint(M[i]), __float_as_uint(L[i]), 0u, 0u};
            __builtin_amdgcn_raw_buffer_store_b128(own_h[i], rs, mine + (i * 64 + lane) * 16, 0, kCoherent);
            if (c == 0)
                __builtin_amdgcn_raw_buffer_store_b128(own_ml[i], rs, mine + RT * 1024 + (i * 16 + n) * 16, 0, kCoherent);
        }
        // the stores are complete (acknowledged by the coherence point) before the count: the
        // split that sees the final count reads data that has already landed
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int32_t* counter = counters + pair * kUWaves + wave;
        int prior = 0;
        if (lane == 0) prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__builtin_amdgcn_readlane(prior, 0) != n_split - 1) return;
        asm volatile("" ::: "memory");  // (the loads below are issued after the count returned)
        // the last split for these dims: every split's values (this one's from registers),
        // requested together, then merged in split order
        u32x4 hv[kUMaxSplits][RT], mlv[kUMaxSplits][RT];
#pragma unroll
        for (int s = 0; s < kUMaxSplits; s++) {
            const uint32_t src = (uint32_t)min(s, n_split - 1) * pair_bytes + wave * part_bytes;
#pragma unroll
            for (int i = 0; i < RT; i++) {
                if (s < n_split && s != split) {
                    hv[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, src + (i * 64 + lane) * 16, 0, kCoherent);
                    mlv[s][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, src + RT * 1024 + (i * 16 + n) * 16, 0, kCoherent);
                } else {
                    hv[s][i] = own_h[i];
                    mlv[s][i] = own_ml[i];
                }
            }
        }
        if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int i = 0; i < RT; i++) {
            float mx = -INFINITY;
#pragma unroll
            for (int s = 0; s < kUMaxSplits; s++)
                if (s < n_split) mx = fmaxf(mx, __uint_as_float(mlv[s][i][0]));
            float den = 0.f;
            float acc[8] = {};
#pragma unroll
            for (int s = 0; s < kUMaxSplits; s++) {
                if (s < n_split) {
                    const float ms = __uint_as_float(mlv[s][i][0]);
                    const float wgt = (ms == -INFINITY) ? 0.f : exp2_hw(ms - mx) * __uint_as_float(mlv[s][i][1]);
                    den += wgt;
                    const f16x8 hs = __builtin_bit_cast(f16x8, hv[s][i]);
#pragma unroll
                    for (int e = 0; e < 8; e++) acc[e] += wgt * (float)hs[e];
                }
            }
            const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) R[i][e] = acc[e] * inv;
        }
    } else {
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const float inv = L[i] > 0.f ? 1.f / L[i] : 0.f;
#pragma unroll
            for (int e = 0; e < 8; e++) R[i][e] *= inv;
        }
    }
#pragma unroll
    for (int i = 0; i < RT; i++) {
        const int j = tile0 + i;
        if (j >= QL) continue;  // (uniform: the unused slot of an odd tile count)
        uint32_t packed[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
            packed[e] = (uint32_t)bf16_rne(R[i][2 * e]) | ((uint32_t)bf16_rne(R[i][2 * e + 1]) << 16);
        uint16_t* op = out + ((int64_t)(b * QL + j) * kQHeads + kGroupHeads * g + n) * kDim + 32 * w + 8 * c;
        *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    }
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_union)
#endif

int union_num_splits(int batch) {
    const int pairs = batch * kKvHeads;
    const int ns = (256 + pairs - 1) / pairs;
    return ns < 1 ? 1 : (ns > kUMaxSplits ? kUMaxSplits : ns);
}

size_t union_counter_bytes(int batch) {
    return ((size_t)batch * kKvHeads * kUWaves * sizeof(int32_t) + 255) / 256 * 256;
}

size_t union_workspace_bytes(int batch, int q_len) {
    const int ns = union_num_splits(batch);
    if (ns == 1) return 0;
    const size_t rt = (size_t)(q_len + kUHalves - 1) / kUHalves;
    return union_counter_bytes(batch) +
           (size_t)batch * kKvHeads * ns * kUWaves * rt * (64 * 16 + 16 * 16);
}

hipError_t launch_attention_union(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                  const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                  int max_blocks, int q_len, const uint16_t* q, int32_t* ids,
                                  const float* scores, int ids_per_row, float scale_log2,
                                  uint16_t* out, void* workspace, hipStream_t stream) {
    const int ns = union_num_splits(batch);
    const int pairs = batch * kKvHeads;
    const dim3 grid(8 * ((pairs + 7) / 8) * ns), block(kUWaves * 64);
    int32_t* counters = nullptr;
    uint8_t* partials = nullptr;
    if (ns > 1) {
        counters = static_cast<int32_t*>(workspace);
        partials = static_cast<uint8_t*>(workspace) + union_counter_bytes(batch);
    }
#define MSA_LAUNCH_UNION(QL_, SEL_)                                                                  \
    hipLaunchKernelGGL((attention_union_kernel<QL_, SEL_>), grid, block, 0, stream, k_pool, v_pool, \
                       num_pages, block_table, ctx_lens, batch, max_blocks, ns, q, ids, scores,     \
                       scale_log2, out, counters, partials, ids_per_row)
    const bool sel = scores != nullptr;
    switch (q_len) {
        case 2: if (sel) MSA_LAUNCH_UNION(2, true); else MSA_LAUNCH_UNION(2, false); break;
        case 3: if (sel) MSA_LAUNCH_UNION(3, true); else MSA_LAUNCH_UNION(3, false); break;
        default: if (sel) MSA_LAUNCH_UNION(4, true); else MSA_LAUNCH_UNION(4, false); break;
    }
#undef MSA_LAUNCH_UNION
    return hipGetLastError();
}

}  // namespace msa
