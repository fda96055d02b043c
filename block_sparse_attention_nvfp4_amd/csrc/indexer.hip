// MSA indexer: index scores of every cached key against the index queries, max-pooled into one
// score per 128-token block.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": one index query per GQA
// group scores every key of the single shared index-key head; scores are max-pooled per block;
// the scan reads only the index keys of the whole context each step (the term that still grows
// with context). "MiniMax M3 on vLLM", section "Decode indexer score kernel": a dedicated score
// kernel, not a padded dense GEMM, keeping the top-k boundary close to the scores; section "MSA
// mechanism": the partial last block and the causal boundary are masked.
//
// Work split: a workgroup of four wavefront pairs takes 32 consecutive blocks of one sequence;
// a pair takes 8 of them (a block never spans two pages, so the max-pool stays inside the pair),
// and wavefront h of the pair scores the 64 tokens of half h of each page. Pages stream into
// LDS with direct global->LDS loads, one half page ahead of the one being scored, so eight
// wavefronts per CU (two per SIMD) keep the loads in flight while the SIMDs dequantize: the
// dequantization, not the matrix cores, is most of the arithmetic, and a second wavefront per
// SIMD hides its latencies. The two half-page maxima of a block meet in LDS at the end.
// Per 16-token slab a wavefront dequantizes the keys exactly (A operand, tokens x dims) and
// multiplies them with up to 16 index-query rows (B operand, dims x rows; a row is (query
// token j, group g)) on the matrix cores, fp32 accumulate.
// Keys are dequantized to fp16 with one conversion and one packed multiply per pair of values
// (exact); the query rows are scaled by a power of two into fp16 range (exact for any row whose
// values span less than about 2^29) and the block maxima scaled back. A wavefront whose rows do
// not convert exactly takes the bf16 path (exact keys, bf16 queries) instead.
// Rows beyond 16 (q_len > 4) loop over row tiles.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kPairs = 4;            // wavefront pairs per workgroup; a pair shares its blocks
constexpr int kWaves = 2 * kPairs;   // wavefront h of a pair scores the tokens of half h of each page
constexpr int kBufs = 2;             // LDS buffers per wavefront (half pages in flight: kBufs - 1)
constexpr int kPagesPerPair = 8;
static_assert(kPagesPerPair <= 8, "the score write-out covers at most eight blocks per pair");
constexpr int kHalfBytes = 5 * 1024; // four code slabs of a half page + the page's scale chunk

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kNonTemporal = 2;  // cache-policy bits of the DMA loads: stream, each page is read once

// Copy half h of a 9,216-byte page into this wavefront's LDS buffer with five direct
// global->LDS 16-byte loads, without registers: code slabs 4h..4h+3 (tokens with
// (t % 32) / 4 in that range) and the scale kilobyte (lane l's bytes land at buffer + 16 l of
// each kilobyte). Both wavefronts of a pair read the scale kilobyte, the second mostly from the
// L2: four-byte loads of each half's own scale words move the same bytes in more, smaller
// requests and measured slower.
__device__ __forceinline__ void half_to_lds(const uint8_t* pg, int h, uint8_t* buf, int lane) {
#pragma unroll
    for (int s = 0; s < 4; s++)
        __builtin_amdgcn_global_load_lds(pg + (4 * h + s) * 1024 + lane * 16,
                                         (lds_void*)(buf + s * 1024), 16, 0, kNonTemporal);
    __builtin_amdgcn_global_load_lds(pg + 8192 + lane * 16, (lds_void*)(buf + 4096), 16, 0,
                                     kNonTemporal);
}

// Wait until the loads of all but the `after` most recently issued half pages (five loads
// each) have completed.
__device__ __forceinline__ void wait_halves(int after) {
    switch (after) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
    }
}
static_assert(kBufs <= 3, "wait_halves covers at most two half pages in flight");

// The same wait for loads issued before `after` half pages, and the registers those loads
// write: the asm operands keep every use of `v` after the wait.
__device__ __forceinline__ void wait_halves_then(int after, u32x4 (&v)[4]) {
    switch (after) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) :: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(5)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) :: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(10)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]) :: "memory"); break;
    }
}

// This lane's four 16-byte code chunks and the two scale words of its slabs, read from LDS
// with explicit instructions: the compiler would otherwise wait for every DMA load in flight
// before any LDS read, since it cannot tell which buffer the loads write.
struct HalfRegs {
    u32x4 code[4];
    uint32_t scale[2];
};
__device__ __forceinline__ void read_half(HalfRegs& hr, const uint8_t* buf, int h, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(buf + lane * 16);
    const uint32_t as = (uint32_t)(uintptr_t)(buf + 4096 + lane * 16 + h * 8);
#define MSA_DS_READ(dst, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(dst) : "v"(a))
    MSA_DS_READ(hr.code[0], 0);
    MSA_DS_READ(hr.code[1], 1024);
    MSA_DS_READ(hr.code[2], 2048);
    MSA_DS_READ(hr.code[3], 3072);
#undef MSA_DS_READ
    asm volatile("ds_read_b32 %0, %1" : "=v"(hr.scale[0]) : "v"(as));
    asm volatile("ds_read_b32 %0, %1 offset:4" : "=v"(hr.scale[1]) : "v"(as));
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(hr.code[0]), "+v"(hr.code[1]), "+v"(hr.code[2]), "+v"(hr.code[3]),
                   "+v"(hr.scale[0]), "+v"(hr.scale[1]));
}

// Max over this lane's 16 tokens of half h of a page (token 32c + 4s + i for slabs s = 4h..4h+3,
// query row n); masked -> -inf. `qop` holds the query operand as fp16 (F16 path) or as bf16
// bits (fallback); keys are dequantized to fp16 either way and, on the fallback, converted
// exactly to bf16.
template <bool FULL, bool F16>
__device__ __forceinline__ float half_max(const HalfRegs& hr, const u32x4 (&qop)[4], int h,
                                          int tok0, int c, int p_row) {
    float best = -INFINITY;
#pragma unroll
    for (int s2 = 0; s2 < 4; s2++) {
        const int s = 4 * h + s2;
        f16x2 s0, s1;
        if (s2 & 1) e4m3_pair_f16<true>(hr.scale[s2 >> 1], s0, s1);
        else e4m3_pair_f16<false>(hr.scale[s2 >> 1], s0, s1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const f16x8 a = dequant8_f16(hr.code[s2][m], m < 2 ? s0 : s1);
            if constexpr (F16)
                acc = mfma_f16_k32(a, __builtin_bit_cast(f16x8, qop[m]), acc);
            else
                acc = mfma_bf16_k32(f16x8_to_bf16x8(a), __builtin_bit_cast(bf16x8, qop[m]), acc);
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = tok0 + 32 * c + 4 * s + i;
            best = fmaxf(best, (FULL || t <= p_row) ? acc[i] : -INFINITY);
        }
    }
    return best;
}


__global__ __launch_bounds__(kWaves * 64) void indexer_kernel(
    const uint8_t* __restrict__ ik_pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len,
    const uint16_t* __restrict__ q_idx, float* __restrict__ scores) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves][kBufs][kHalfBytes];
    __shared__ int page_ids[kWaves][kPagesPerPair];
    __shared__ float stash[kPairs][kPagesPerPair][2][16];  // half-page maxima of the row tile
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int pair = wave >> 1;
    const int h = wave & 1;
    const int n = lane & 15;  // B/D column: query row within the tile
    const int c = lane >> 4;  // lane group
    const int b = blockIdx.y;
    const int blk0 = (blockIdx.x * kPairs + pair) * kPagesPerPair;
    // a pair past the end still takes part in the workgroup barriers below
    const bool active = blk0 < max_blocks;
    const int32_t* table = block_table + (int64_t)b * max_blocks;
    // the pair's block-table entries and the context length are requested together (the
    // entries do not depend on it): one memory round trip before the first page load
    int pid_raw = -1;
    if (lane < kPagesPerPair && blk0 + lane < max_blocks) pid_raw = table[blk0 + lane];
    int T_raw = ctx_lens[b];
    asm volatile("" : "+v"(pid_raw), "+v"(T_raw));
    const int T = clamp_ctx(T_raw, max_blocks);
    const int rows = 4 * q_len;
    const int64_t row_base = (int64_t)b * rows;
    const int blk_end = active ? min(blk0 + kPagesPerPair, max_blocks) : blk0;
    // blocks past the last query position hold no visible key and are never loaded
    const int n_blocks = T > 0 ? min(max_blocks, (T - 1) / kBlock + 1) : 0;
    // page ids of the pair's blocks, read once into LDS: a block-table load issued between page
    // loads would make the in-order memory counter wait for every page in flight
    if (lane < kPagesPerPair)
        page_ids[wave][lane] = (active && blk0 + lane < n_blocks && pid_raw >= 0 &&
                                pid_raw < num_pages) ? pid_raw : -1;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    for (int rt = 0; rt < rows; rt += 16) {
        const int r = rt + n;
        const int p_row = T - q_len + (r >> 2);                  // position of row r's token
        const int j_hi = min((rt >> 2) + 3, q_len - 1);
        const int p_lo = T - q_len + (rt >> 2);                  // lowest position in the tile
        const int p_hi = T - q_len + j_hi;                       // highest position in the tile
        const int vis_end = min(blk_end, p_hi >= 0 ? p_hi / kBlock + 1 : 0);

        // software pipeline: half pages of blocks blk+1 .. blk+kBufs-1 stream into LDS while
        // block blk is scored. issued: bit i set when block blk0+i had its half page loaded.
        uint32_t issued = 0;
        auto issue = [&](int i) {
            const int blk = blk0 + i;
            const int pid = (i < kPagesPerPair && blk < vis_end)
                                ? __builtin_amdgcn_readfirstlane(page_ids[wave][i]) : -1;
            if (pid >= 0) {
                half_to_lds(ik_pool + (int64_t)pid * kHeadPageBytes, h, lds[wave][i % kBufs], lane);
                issued |= 1u << i;
            }
        };
        // B operand: row r, dims 32c + 8m .. 32c + 8m + 7 for MFMA m = 0..3. The query rows are
        // requested first and the first pages right after; the loads are written out so that
        // the wait for the query (placed here, not by the compiler, which would wait for every
        // page as well) leaves the pages in flight. Every lane loads a valid row (rows past the
        // tile read row rows - 1) and zeroes it after the wait.
        u32x4 qraw[4];
        {
            const uint16_t* qp = q_idx + (row_base + min(r, rows - 1)) * kDim + 32 * c;
            asm volatile(
                "global_load_dwordx4 %0, %4, off\n\t"
                "global_load_dwordx4 %1, %4, off offset:16\n\t"
                "global_load_dwordx4 %2, %4, off offset:32\n\t"
                "global_load_dwordx4 %3, %4, off offset:48"
                : "=&v"(qraw[0]), "=&v"(qraw[1]), "=&v"(qraw[2]), "=&v"(qraw[3])
                : "v"(qp)
                : "memory");
        }
#pragma unroll
        for (int i = 0; i < kBufs - 1; i++) issue(i);
        wait_halves_then(__popc(issued), qraw);
        bf16x8 qb[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            qb[m] = r < rows ? __builtin_bit_cast(bf16x8, qraw[m]) : bf16x8{};
        f16x8 qh[4];
        float out_scale;
        const bool f16 = __all(query_to_f16(qb, qh, out_scale));
        u32x4 qop[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            qop[m] = f16 ? __builtin_bit_cast(u32x4, qh[m]) : __builtin_bit_cast(u32x4, qb[m]);
        if (!f16) out_scale = 1.0f;

#pragma unroll 1
        for (int blk = blk0; blk < blk_end; blk++) {
            const int k = blk - blk0;
            issue(k + kBufs - 1);
            const int tok0 = blk * kBlock;
            float best = -INFINITY;
            if (issued & (1u << k)) {
                wait_halves(__popc(issued >> (k + 1)));
                HalfRegs hr;
                read_half(hr, lds[wave][k % kBufs], h, lane);
                const bool full = tok0 + kBlock - 1 <= p_lo;
                if (f16)
                    best = (full ? half_max<true, true>(hr, qop, h, tok0, c, p_row)
                                 : half_max<false, true>(hr, qop, h, tok0, c, p_row)) * out_scale;
                else
                    best = full ? half_max<true, false>(hr, qop, h, tok0, c, p_row)
                                : half_max<false, false>(hr, qop, h, tok0, c, p_row);
            }
            best = max_over_c(best);
            // kept in LDS until the tile ends: a global store here would join the page loads in
            // the in-order memory counter and make the next wait cover part of a later page
            if (c == 0) {
                const uint32_t a = (uint32_t)(uintptr_t)&stash[pair][k][h][n];
                asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(best) : "memory");
            }
        }
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        // lane (n, c) of wavefront h writes block c + 4h of row rt + n: the max of both halves
        {
            const int k = c + 4 * h;
            if (k < kPagesPerPair && r < rows && blk0 + k < blk_end)
                scores[(row_base + r) * max_blocks + blk0 + k] =
                    fmaxf(stash[pair][k][0][n], stash[pair][k][1][n]);
        }
        __syncthreads();  // the next row tile rewrites the stash
    }
}

}  // namespace

hipError_t launch_indexer(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                          const uint16_t* q_idx, float* scores, hipStream_t stream) {
    const int per_wg = kPairs * kPagesPerPair;
    dim3 grid((max_blocks + per_wg - 1) / per_wg, batch);
    hipLaunchKernelGGL(indexer_kernel, grid, dim3(kWaves * 64), 0, stream, ik_pool,
                       num_pages, block_table, ctx_lens, max_blocks, q_len, q_idx, scores);
    return hipGetLastError();
}

}  // namespace msa
