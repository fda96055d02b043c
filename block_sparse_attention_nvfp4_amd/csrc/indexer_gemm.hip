// MSA indexer for many query rows per sequence (prefill chunks, long speculative drafts): the
// block scores as a score GEMM, each index-key page dequantized once and multiplied with every
// query row that can see it.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": one index query per GQA
// group scores every key of the shared index-key head, max-pooled per 128-token block. "MiniMax
// M3 on vLLM", sections "MSA mechanism" and "Prefill execution": the causal boundary inside a
// block is masked and every query token has its own position (a chunk of q tokens scores
// 4 q rows against the whole visible context, a GEMM).
//
// Work split: a workgroup of four wavefronts takes four consecutive blocks of one sequence
// and a range of up to 512 of its query rows; two workgroups share a CU, so one's page load
// and dequantization overlap the other's matrix-core work (one workgroup of eight wavefronts
// per CU measured 12% slower). Each wavefront loads its block's page once into registers and
// dequantizes it exactly to bf16 (E2M1 x E4M3 products have at most 6 significant bits), as
// the A operand of 16x16x32 bf16 matrix-core steps: 128 tokens x 128 dims in 128 registers.
// The query rows stream through LDS in stages of 64 rows, loaded by direct global->LDS copies
// already in operand order and shared by the workgroup's wavefronts (double buffered: the next
// stage loads while this one is multiplied). Per 16-row tile a wavefront runs 32 matrix-core
// steps (8 token slabs x 4 dimension steps, fp32 accumulate), takes each row's max over its
// visible tokens and keeps it in LDS; the workgroup writes its rows' four block scores at the
// end as contiguous 16-byte runs.
// Query rows are bf16 and used as they are: every product is exact in fp32 and the sums are
// fp32, as in the decode indexer's bf16 path.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kGWaves = 4;                   // one block per wavefront
constexpr int kStageRows = 64;               // query rows per LDS stage
constexpr int kTileBytes = 16 * kDim * 2;    // one 16-row tile of bf16 query rows: 4 KB
constexpr int kMaxRowsPerWg = 512;
typedef __attribute__((address_space(3))) void lds_void;

// This lane's B operand of a 16-row tile (dims x rows): piece m holds row n = lane % 16,
// elements 32 c + 8 m .. +7 (c = lane / 16), stored at tile + 1024 m + 16 lane. Read with
// explicit instructions, issued and waited for in one statement: the compiler cannot tell
// which LDS buffer the direct copies in flight write, and would otherwise wait for all of them.
__device__ __forceinline__ void read_tile(u32x4 (&v)[4], const uint8_t* tile, int lane) {
    const uint32_t a = (uint32_t)(uintptr_t)(tile + lane * 16);
    asm volatile("ds_read_b128 %0, %4\n\t"
                 "ds_read_b128 %1, %4 offset:1024\n\t"
                 "ds_read_b128 %2, %4 offset:2048\n\t"
                 "ds_read_b128 %3, %4 offset:3072\n\t"
                 "s_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]) : "v"(a) : "memory");
}

// LSE: the block's log-sum-exp of its token scores instead of their max ("MiniMax M3 on
// vLLM", section "Prefill execution": the block reduction may be max or log-sum-exp).
// The table columns scored are blk_begin .. blk_end - 1; column c holds the page of global
// block g_begin + c * g_stride (a shard of the blocks; 0 and 1 for a whole table) and the
// context is clamped to total_blocks blocks. SHARED: one row space holds every query row of the
// batch (blockIdx.z = 0), scored against the pages of sequence 0's table, which all sequences
// share there and which hold no query token (no mask: every token is visible).
template <bool LSE, bool SHARED>
__global__ __launch_bounds__(kGWaves * 64, 2) void indexer_gemm_kernel(
    const uint8_t* __restrict__ ik_pool, int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len, int rows_per_wg,
    const uint16_t* __restrict__ q_idx, float* __restrict__ scores, int blk_begin, int blk_end,
    int batch, int g_begin, int g_stride, int total_blocks) {
    __shared__ __attribute__((aligned(16))) uint8_t stage[2][kStageRows / 16][kTileBytes];
    __shared__ float best_of[kMaxRowsPerWg][kGWaves];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, c = lane >> 4;
    const int b = blockIdx.z;
    // this sequence's rows (j, g) = 4 j + g (SHARED: the whole batch's rows)
    const int rows = SHARED ? 4 * q_len * batch : 4 * q_len;
    const int r_begin = blockIdx.y * rows_per_wg;
    const int r_end = min(rows, r_begin + rows_per_wg);
    const int blk0 = blk_begin + blockIdx.x * kGWaves;  // this workgroup's first block
    const int blk = blk0 + wave;
    // (SHARED: a context past every block, so that nothing is masked)
    const int T_raw = SHARED ? max_blocks * kBlock : ctx_lens[b];
    const int T = SHARED ? T_raw : clamp_ctx(T_raw, total_blocks);
    MSA_CHECK(SHARED || threadIdx.x != 0 || (T_raw >= q_len && T_raw <= total_blocks * kBlock), kCheckCtxLen);
    const uint8_t* qseq = reinterpret_cast<const uint8_t*>(q_idx + (int64_t)b * rows * kDim);

    // stage loads: copies of 1 KB (tile tt, piece m), kCopies per wavefront; lane
    // (n, c) of copy (tt, m) brings bytes 64 c + 16 m .. +15 of row 16 tt + n (past the range:
    // its last row, never written out)
    constexpr int kCopies = kStageRows / 4 / kGWaves;  // 4 copies per 16-row tile
    auto load_stage = [&](int r0, int buf) {
#pragma unroll
        for (int k = 0; k < kCopies; k++) {
            const int i = kCopies * wave + k, tt = i >> 2, m = i & 3;
            const int r = min(r0 + 16 * tt + n, r_end - 1);
            __builtin_amdgcn_global_load_lds(qseq + (int64_t)r * (kDim * 2) + 64 * c + 16 * m,
                                             (lds_void*)(&stage[buf][tt][1024 * m]), 16, 0, 0);
        }
    };
    load_stage(r_begin, 0);

    // this wavefront's page: lane (m, c) holds, for token slab s, the 32 codes of token
    // 32 (m / 4) + 4 s + m % 4, elements 32 c .. 32 c + 31, and the 16 scale bytes of its
    // token row (bytes 2 s, 2 s + 1: element groups 2 c, 2 c + 1 of slab s)
    const bool in_table = blk < blk_end;
    int page = in_table ? block_table[(int64_t)b * max_blocks + blk] : -1;
    const int tok0 = (g_begin + blk * g_stride) * kBlock;
    const bool has_keys = in_table && tok0 < T && page >= 0 && page < num_pages;
    bf16x8 ka[8][4];
    if (has_keys) {
        const uint8_t* pg = ik_pool + (int64_t)page * kHeadPageBytes;
        u32x4 code[8];
#pragma unroll
        for (int s = 0; s < 8; s++) code[s] = load16(pg + 1024 * s + 16 * lane);
        const u32x4 sc = load16(pg + kCodeBytes + 16 * lane);
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const f32x2 gs = (s & 1) ? e4m3_pair_f32<true>(sc[s >> 1]) : e4m3_pair_f32<false>(sc[s >> 1]);
#pragma unroll
            for (int m = 0; m < 4; m++) ka[s][m] = dequant8_bf16(code[s][m], m < 2 ? gs[0] : gs[1]);
            // one slab at a time: the fp32 products of later slabs are not all made up front
            asm volatile("" : "+v"(ka[s][0]), "+v"(ka[s][1]), "+v"(ka[s][2]), "+v"(ka[s][3]));
        }
    }

    int buf = 0;
    for (int r0 = r_begin; r0 < r_end; r0 += kStageRows, buf ^= 1) {
        // this stage's rows are in LDS for every wavefront, and every wavefront is done with
        // the other buffer: the next stage may overwrite it
        __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0)
        __syncthreads();
        if (r0 + kStageRows < r_end) load_stage(r0 + kStageRows, buf ^ 1);
#pragma unroll 1
        for (int tt = 0; tt < kStageRows / 16; tt++) {
            const int rt = r0 + 16 * tt;  // rows rt .. rt + 15: tokens rt / 4 .. rt / 4 + 3
            if (rt >= r_end) break;
            const int p_lo = SHARED ? T : T - q_len + (rt >> 2);
            const int p_hi = SHARED ? T : T - q_len + min((rt >> 2) + 3, q_len - 1);
            float best = -INFINITY;
            if (has_keys && p_hi >= tok0) {
                u32x4 qv[4];
                read_tile(qv, &stage[buf][tt][0], lane);
                f32x4 acc[8];
#pragma unroll
                for (int s = 0; s < 8; s++) {
                    acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int m = 0; m < 4; m++)
                        acc[s] = mfma_bf16_k32(ka[s][m], __builtin_bit_cast(bf16x8, qv[m]), acc[s]);
                }
                // D of slab s in lane (n, c): tokens 32 c + 4 s + i, i = 0..3, of query row n
                if (p_lo < tok0 + kBlock - 1) {
                    asm volatile("");  // a scalar branch: the mask only where the block is cut
                    const int lim = T - q_len + min((rt + n) >> 2, q_len - 1) - tok0 - 32 * c;
#pragma unroll
                    for (int s = 0; s < 8; s++)
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (4 * s + i > lim) acc[s][i] = -INFINITY;
                }
#pragma unroll
                for (int s = 0; s < 8; s++)
#pragma unroll
                    for (int i = 0; i < 4; i++) best = fmaxf(best, acc[s][i]);
                best = max_over_c(best);
                if constexpr (LSE) {
                    // log-sum-exp about the row's max (masked tokens are -inf: weight 0)
                    float sum = 0.f;
                    if (best > -INFINITY) {
#pragma unroll
                        for (int s = 0; s < 8; s++)
#pragma unroll
                            for (int i = 0; i < 4; i++)
                                sum += exp2f((acc[s][i] - best) * 1.4426950408889634f);
                    }
                    sum = sum_over_c(sum);
                    best = best > -INFINITY ? best + logf(sum) : -INFINITY;
                }
            }
            if (c == 0 && rt + n < r_end) best_of[rt + n - r_begin][wave] = best;
        }
    }
    __syncthreads();
    // row rl's block scores are kGWaves contiguous floats
    const int nr = r_end - r_begin;
    float* out = scores + ((int64_t)b * rows + r_begin) * max_blocks + blk0;
    for (int i = threadIdx.x; i < nr * kGWaves; i += kGWaves * 64) {
        const int rl = i / kGWaves, kb = i % kGWaves;
        if (blk0 + kb < blk_end) out[(int64_t)rl * max_blocks + kb] = best_of[rl][kb];
    }
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_indexer_gemm)
#endif

namespace {

template <bool LSE, bool SHARED>
hipError_t launch_gemm_t(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                         const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                         const uint16_t* q_idx, float* scores, int blk_begin, int blk_end,
                         hipStream_t stream, int g_begin = 0, int g_stride = 1,
                         int total_blocks = -1) {
    if (blk_end <= blk_begin) return hipSuccess;
    const int rows = SHARED ? 4 * q_len * batch : 4 * q_len;
    const int rows_per_wg = min(kMaxRowsPerWg, (rows + 15) / 16 * 16);
    const dim3 grid((blk_end - blk_begin + kGWaves - 1) / kGWaves,
                    (rows + rows_per_wg - 1) / rows_per_wg, SHARED ? 1 : batch);
    hipLaunchKernelGGL((indexer_gemm_kernel<LSE, SHARED>), grid, dim3(kGWaves * 64), 0, stream,
                       ik_pool, num_pages, block_table, ctx_lens, max_blocks, q_len, rows_per_wg,
                       q_idx, scores, blk_begin, blk_end, batch, g_begin, g_stride,
                       total_blocks < 0 ? max_blocks : total_blocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_indexer_gemm(const uint8_t* ik_pool, int64_t num_pages,
                               const int32_t* block_table, const int32_t* ctx_lens, int batch,
                               int max_blocks, int q_len, const uint16_t* q_idx, float* scores,
                               hipStream_t stream, bool lse) {
    if (lse)
        return launch_gemm_t<true, false>(ik_pool, num_pages, block_table, ctx_lens, batch,
                                          max_blocks, q_len, q_idx, scores, 0, max_blocks, stream);
    return launch_gemm_t<false, false>(ik_pool, num_pages, block_table, ctx_lens, batch,
                                       max_blocks, q_len, q_idx, scores, 0, max_blocks, stream);
}

hipError_t launch_indexer_gemm_shard(const uint8_t* ik_pool, int64_t num_pages,
                                     const int32_t* block_table, const int32_t* ctx_lens,
                                     int batch, int max_blocks, int q_len, const uint16_t* q_idx,
                                     float* scores, int block_begin, int block_stride,
                                     int total_blocks, hipStream_t stream) {
    return launch_gemm_t<false, false>(ik_pool, num_pages, block_table, ctx_lens, batch,
                                       max_blocks, q_len, q_idx, scores, 0, max_blocks, stream,
                                       block_begin, block_stride, total_blocks);
}

hipError_t launch_indexer_shared_prefix(const uint8_t* ik_pool, int64_t num_pages,
                                        const int32_t* block_table, const int32_t* ctx_lens,
                                        int batch, int max_blocks, int q_len,
                                        const uint16_t* q_idx, float* scores, int prefix_blocks,
                                        hipStream_t stream) {
    hipError_t err = launch_gemm_t<false, true>(ik_pool, num_pages, block_table, ctx_lens, batch,
                                                max_blocks, q_len, q_idx, scores, 0, prefix_blocks,
                                                stream);
    if (err != hipSuccess) return err;
    return launch_gemm_t<false, false>(ik_pool, num_pages, block_table, ctx_lens, batch,
                                       max_blocks, q_len, q_idx, scores, prefix_blocks, max_blocks,
                                       stream);
}

}  // namespace msa
