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
// Work split: one 64-lane wavefront owns whole pages (a block never spans two pages, so the
// max-pool needs no cross-wave step). Per 16-token slab it dequantizes the keys exactly into
// bf16 (A operand, tokens x dims) and multiplies them with up to 16 index-query rows (B operand,
// dims x rows; a row is (query token j, group g)) on the matrix cores, fp32 accumulate. Rows
// beyond 16 (q_len > 4) loop over row tiles.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kWaves = 4;

template <int PPW>
__global__ __launch_bounds__(kWaves * 64) void indexer_kernel(
    const uint8_t* __restrict__ ik_pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len,
    const uint16_t* __restrict__ q_idx, float* __restrict__ scores) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;  // B/D column: query row within the tile
    const int c = lane >> 4;  // lane group
    const int b = blockIdx.y;
    const int blk0 = (blockIdx.x * kWaves + wave) * PPW;
    if (blk0 >= max_blocks) return;
    const int T = clamp_ctx(ctx_lens[b], max_blocks);
    const int rows = 4 * q_len;
    const int64_t row_base = (int64_t)b * rows;
    const int32_t* table = block_table + (int64_t)b * max_blocks;

    for (int rt = 0; rt < rows; rt += 16) {
        const int r = rt + n;
        // B operand: row r, dims 32c + 8m .. 32c + 8m + 7 for MFMA m = 0..3
        bf16x8 qop[4];
        if (r < rows) {
            const uint16_t* qp = q_idx + (row_base + r) * kDim + 32 * c;
#pragma unroll
            for (int m = 0; m < 4; m++) qop[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
        } else {
#pragma unroll
            for (int m = 0; m < 4; m++) qop[m] = bf16x8{};
        }
        const int p_row = T - q_len + (r >> 2);                  // position of row r's token
        const int j_hi = min((rt >> 2) + 3, q_len - 1);
        const int p_lo = T - q_len + (rt >> 2);                  // lowest position in the tile
        const int p_hi = T - q_len + j_hi;                       // highest position in the tile

        for (int k = 0; k < PPW; k++) {
            const int blk = blk0 + k;
            if (blk >= max_blocks) break;
            const int tok0 = blk * kBlock;
            float best = -INFINITY;
            const int page = (tok0 <= p_hi) ? table[blk] : -1;
            if (page >= 0 && page < num_pages) {
                const uint8_t* pg = ik_pool + (int64_t)page * kHeadPageBytes;
                u32x4 code[8];
#pragma unroll
                for (int s = 0; s < 8; s++) code[s] = load16(pg + s * 1024 + lane * 16);
                const u32x4 sc = load16(pg + kCodeBytes + lane * 16);
                const bool full = tok0 + kBlock - 1 <= p_lo;
#pragma unroll
                for (int s = 0; s < 8; s++) {
                    // scales of this lane's token for groups 2c and 2c+1
                    const f32x2 s2 = (s & 1) ? e4m3_pair_f32<true>(sc[s >> 1])
                                             : e4m3_pair_f32<false>(sc[s >> 1]);
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 4; m++)
                        acc = mfma_bf16_k32(dequant8_bf16(code[s][m], s2[m >> 1]), qop[m], acc);
                    // acc[i]: token 32c + 4s + i of the page, query row n
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int t = tok0 + 32 * c + 4 * s + i;
                        const float v = (full || t <= p_row) ? acc[i] : -INFINITY;
                        best = fmaxf(best, v);
                    }
                }
            }
            best = max_over_c(best);
            if (c == 0 && r < rows) scores[(row_base + r) * max_blocks + blk] = best;
        }
    }
}

}  // namespace

hipError_t launch_indexer(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                          const uint16_t* q_idx, float* scores, hipStream_t stream) {
    constexpr int PPW = 2;
    const int per_wg = kWaves * PPW;
    dim3 grid((max_blocks + per_wg - 1) / per_wg, batch);
    hipLaunchKernelGGL(indexer_kernel<PPW>, grid, dim3(kWaves * 64), 0, stream, ik_pool,
                       num_pages, block_table, ctx_lens, max_blocks, q_len, q_idx, scores);
    return hipGetLastError();
}

}  // namespace msa
