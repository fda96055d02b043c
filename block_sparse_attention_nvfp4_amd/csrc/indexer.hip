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
// Work split: one 64-lane wavefront owns PPW whole pages (a block never spans two pages, so the
// max-pool needs no cross-wave step) and issues all their loads before computing, so the whole
// context is in flight at once. Per 16-token slab it dequantizes the keys exactly (A operand,
// tokens x dims) and multiplies them with up to 16 index-query rows (B operand, dims x rows; a
// row is (query token j, group g)) on the matrix cores, fp32 accumulate.
// Keys are dequantized to fp16 with one conversion and one packed multiply per pair of values
// (exact); the query rows are scaled by a power of two into fp16 range (exact for any row whose
// values span less than about 2^29) and the block maxima scaled back. A wavefront whose rows do
// not convert exactly takes the bf16 path (exact keys, bf16 queries) instead.
// Rows beyond 16 (q_len > 4) loop over row tiles.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kWaves = 4;          // wavefronts per workgroup
constexpr int kBufs = 3;           // LDS page buffers per wavefront (pages in flight: kBufs - 1)
constexpr int kPagesPerWave = 8;

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kNonTemporal = 2;  // cache-policy bits of the DMA loads: stream, each page is read once

// Copy one 9,216-byte page into this wavefront's LDS buffer with nine direct global->LDS
// 16-byte loads (lane l's bytes land at buffer + 16 l of each kilobyte), without registers.
__device__ __forceinline__ void page_to_lds(const uint8_t* pg, uint8_t* buf, int lane) {
#pragma unroll
    for (int s = 0; s < 9; s++)
        __builtin_amdgcn_global_load_lds(pg + s * 1024 + lane * 16, (lds_void*)(buf + s * 1024), 16,
                                         0, kNonTemporal);
}

// Wait until the loads of all but the `pages_after` most recently issued pages (9 loads each)
// have completed.
__device__ __forceinline__ void wait_pages(int pages_after) {
    switch (pages_after) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(27)" ::: "memory"); break;
    }
}

// This lane's nine 16-byte chunks of a page in LDS (eight code slabs, then the scales), read
// with explicit instructions: the compiler would otherwise wait for every page load in flight
// before any LDS read, since it cannot tell which buffer the loads write.
struct PageRegs {
    u32x4 code[8];
    u32x4 scale;
};
__device__ __forceinline__ void read_page(PageRegs& pr, const uint8_t* buf, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(buf + lane * 16);
#define MSA_DS_READ(dst, off) asm volatile("ds_read_b128 %0, %1 offset:" #off : "=v"(dst) : "v"(a))
    MSA_DS_READ(pr.code[0], 0);
    MSA_DS_READ(pr.code[1], 1024);
    MSA_DS_READ(pr.code[2], 2048);
    MSA_DS_READ(pr.code[3], 3072);
    MSA_DS_READ(pr.code[4], 4096);
    MSA_DS_READ(pr.code[5], 5120);
    MSA_DS_READ(pr.code[6], 6144);
    MSA_DS_READ(pr.code[7], 7168);
    MSA_DS_READ(pr.scale, 8192);
#undef MSA_DS_READ
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(pr.code[0]), "+v"(pr.code[1]), "+v"(pr.code[2]), "+v"(pr.code[3]),
                   "+v"(pr.code[4]), "+v"(pr.code[5]), "+v"(pr.code[6]), "+v"(pr.code[7]),
                   "+v"(pr.scale));
}

// Max over this lane's 32 tokens of one page (token 32c + 4s + i, query row n); masked -> -inf.
// `qop` holds the query operand as fp16 (F16 path) or as bf16 bits (fallback); keys are
// dequantized to fp16 either way and, on the fallback, converted exactly to bf16.
template <bool FULL, bool F16>
__device__ __forceinline__ float page_max(const PageRegs& pr, const u32x4 (&qop)[4], int tok0,
                                          int c, int p_row) {
    float best = -INFINITY;
#pragma unroll
    for (int s = 0; s < 8; s++) {
        f16x2 s0, s1;
        if (s & 1) e4m3_pair_f16<true>(pr.scale[s >> 1], s0, s1);
        else e4m3_pair_f16<false>(pr.scale[s >> 1], s0, s1);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < 4; m++) {
            const f16x8 a = dequant8_f16(pr.code[s][m], m < 2 ? s0 : s1);
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

__device__ __forceinline__ int page_of(const int32_t* table, int blk, int n_blocks,
                                       int64_t num_pages) {
    const int pid = blk < n_blocks ? table[blk] : -1;
    return (pid >= 0 && pid < num_pages) ? pid : -1;
}

__global__ __launch_bounds__(kWaves * 64) void indexer_kernel(
    const uint8_t* __restrict__ ik_pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len,
    const uint16_t* __restrict__ q_idx, float* __restrict__ scores) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves][kBufs][kHeadPageBytes];
    __shared__ int page_ids[kWaves][kPagesPerWave];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;  // B/D column: query row within the tile
    const int c = lane >> 4;  // lane group
    const int b = blockIdx.y;
    const int blk0 = (blockIdx.x * kWaves + wave) * kPagesPerWave;
    if (blk0 >= max_blocks) return;
    const int T = clamp_ctx(ctx_lens[b], max_blocks);
    const int rows = 4 * q_len;
    const int64_t row_base = (int64_t)b * rows;
    const int32_t* table = block_table + (int64_t)b * max_blocks;
    const int blk_end = min(blk0 + kPagesPerWave, max_blocks);
    // blocks past the last query position hold no visible key and are never loaded
    const int n_blocks = T > 0 ? min(max_blocks, (T - 1) / kBlock + 1) : 0;
    // page ids of this wavefront's blocks, read once into LDS: a block-table load issued between
    // page loads would make the in-order memory counter wait for every page in flight
    if (lane < kPagesPerWave) page_ids[wave][lane] = page_of(table, blk0 + lane, n_blocks, num_pages);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");

    for (int rt = 0; rt < rows; rt += 16) {
        const int r = rt + n;
        // B operand: row r, dims 32c + 8m .. 32c + 8m + 7 for MFMA m = 0..3
        bf16x8 qb[4];
        if (r < rows) {
            const uint16_t* qp = q_idx + (row_base + r) * kDim + 32 * c;
#pragma unroll
            for (int m = 0; m < 4; m++) qb[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
        } else {
#pragma unroll
            for (int m = 0; m < 4; m++) qb[m] = bf16x8{};
        }
        f16x8 qh[4];
        float out_scale;
        const bool f16 = __all(query_to_f16(qb, qh, out_scale));
        u32x4 qop[4];
#pragma unroll
        for (int m = 0; m < 4; m++)
            qop[m] = f16 ? __builtin_bit_cast(u32x4, qh[m]) : __builtin_bit_cast(u32x4, qb[m]);
        if (!f16) out_scale = 1.0f;
        const int p_row = T - q_len + (r >> 2);                  // position of row r's token
        const int j_hi = min((rt >> 2) + 3, q_len - 1);
        const int p_lo = T - q_len + (rt >> 2);                  // lowest position in the tile
        const int p_hi = T - q_len + j_hi;                       // highest position in the tile
        const int vis_end = min(blk_end, p_hi >= 0 ? p_hi / kBlock + 1 : 0);

        // software pipeline: blocks blk+1 .. blk+kBufs-1 stream into LDS while block blk is scored.
        // issued: bit i set when block blk0+i had its page loaded.
        uint32_t issued = 0;
        auto issue = [&](int i) {
            const int blk = blk0 + i;
            const int pid = (i < kPagesPerWave && blk < vis_end)
                                ? __builtin_amdgcn_readfirstlane(page_ids[wave][i]) : -1;
            if (pid >= 0) {
                page_to_lds(ik_pool + (int64_t)pid * kHeadPageBytes, lds[wave][i % kBufs], lane);
                issued |= 1u << i;
            }
        };
#pragma unroll
        for (int i = 0; i < kBufs - 1; i++) issue(i);
#pragma unroll 1
        for (int blk = blk0; blk < blk_end; blk++) {
            const int k = blk - blk0;
            issue(k + kBufs - 1);
            const int tok0 = blk * kBlock;
            float best = -INFINITY;
            if (issued & (1u << k)) {
                wait_pages(__popc(issued >> (k + 1)));
                PageRegs pr;
                read_page(pr, lds[wave][k % kBufs], lane);
                const bool full = tok0 + kBlock - 1 <= p_lo;
                if (f16)
                    best = (full ? page_max<true, true>(pr, qop, tok0, c, p_row)
                                 : page_max<false, true>(pr, qop, tok0, c, p_row)) * out_scale;
                else
                    best = full ? page_max<true, false>(pr, qop, tok0, c, p_row)
                                : page_max<false, false>(pr, qop, tok0, c, p_row);
            }
            best = max_over_c(best);
            if (c == 0 && r < rows) scores[(row_base + r) * max_blocks + blk] = best;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

}  // namespace

hipError_t launch_indexer(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                          const uint16_t* q_idx, float* scores, hipStream_t stream) {
    const int per_wg = kWaves * kPagesPerWave;
    dim3 grid((max_blocks + per_wg - 1) / per_wg, batch);
    hipLaunchKernelGGL(indexer_kernel, grid, dim3(kWaves * 64), 0, stream, ik_pool,
                       num_pages, block_table, ctx_lens, max_blocks, q_len, q_idx, scores);
    return hipGetLastError();
}

}  // namespace msa
