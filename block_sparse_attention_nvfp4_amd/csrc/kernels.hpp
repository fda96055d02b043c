// Host-side launchers of the MSA kernels (internal to libmsa.so). Arguments are already
// validated by the C entry points in api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

hipError_t launch_insert(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool, int64_t num_pages,
                         const int64_t* slots, const float* k, const float* v, const float* ik,
                         int n, hipStream_t stream);

hipError_t launch_indexer(const uint8_t* ik_pool, int64_t num_pages, const int32_t* block_table,
                          const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                          const uint16_t* q_idx, float* scores, hipStream_t stream);

// The indexer as a score GEMM (each page dequantized once for all query rows), used by
// launch_indexer from kIndexerGemmMinQ query tokens per sequence on: the decode indexer streams
// the pages once per 16 query rows, and from 3 row tiles (q = 9..12) on the GEMM is faster
// (8 x 131,072 context: 37 against 28 us at q = 12, 99 against 54 us at q = 32; the scores are
// the same bits).
constexpr int kIndexerGemmMinQ = 9;
// lse: the block's log-sum-exp of its token scores instead of their max (any q_len).
hipError_t launch_indexer_gemm(const uint8_t* ik_pool, int64_t num_pages,
                               const int32_t* block_table, const int32_t* ctx_lens, int batch,
                               int max_blocks, int q_len, const uint16_t* q_idx, float* scores,
                               hipStream_t stream, bool lse = false);

// The indexer over a shard of the blocks: the table's column c holds the page of global block
// block_begin + c * block_stride, the context is clamped to total_blocks blocks; the scores'
// column c equals the whole-table indexer's column block_begin + c * block_stride.
hipError_t launch_indexer_shard(const uint8_t* ik_pool, int64_t num_pages,
                                const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                int max_blocks, int q_len, const uint16_t* q_idx, float* scores,
                                int block_begin, int block_stride, int total_blocks,
                                hipStream_t stream);
hipError_t launch_indexer_gemm_shard(const uint8_t* ik_pool, int64_t num_pages,
                                     const int32_t* block_table, const int32_t* ctx_lens,
                                     int batch, int max_blocks, int q_len, const uint16_t* q_idx,
                                     float* scores, int block_begin, int block_stride,
                                     int total_blocks, hipStream_t stream);

// Indexer for a batch whose sequences share their first prefix_blocks pages (sequence 0's
// table entries) with no query token in them: those pages scored once for every query row of
// the batch, the rest per sequence.
hipError_t launch_indexer_shared_prefix(const uint8_t* ik_pool, int64_t num_pages,
                                        const int32_t* block_table, const int32_t* ctx_lens,
                                        int batch, int max_blocks, int q_len,
                                        const uint16_t* q_idx, float* scores, int prefix_blocks,
                                        hipStream_t stream);

// Insert of a decode step's new tokens at their own positions (slots from the block table).
hipError_t launch_insert_at_positions(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool,
                                      int64_t num_pages, const int32_t* block_table,
                                      const int32_t* ctx_lens, int batch, int max_blocks,
                                      int q_len, const float* k, const float* v, const float* ik,
                                      hipStream_t stream);

// Insert of a decode step's new tokens (positions T - q_len .. T - 1 of each sequence, slots
// from the block table) and the indexer, in one launch when q_len <= 8 (two otherwise).
hipError_t launch_insert_indexer(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool,
                                 int64_t num_pages, const int32_t* block_table,
                                 const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                                 const float* new_k, const float* new_v, const float* new_ik,
                                 const uint16_t* q_idx, float* scores, hipStream_t stream);

hipError_t launch_topk(const float* scores, const int32_t* ctx_lens, int batch, int max_blocks,
                       int q_len, int32_t* ids, hipStream_t stream);

// Selection with the window knobs (rows of up to kWindowMaxBlocks blocks).
constexpr int kWindowMaxBlocks = 64 * 64;
hipError_t launch_topk_window(const float* scores, const int32_t* ctx_lens, int batch,
                              int max_blocks, int q_len, int topk, int init, int local,
                              int32_t* ids, hipStream_t stream);

// Context-parallel selection: one shard's local lists (shards of up to kLocalMaxBlocks
// blocks) and the merge of up to kMergeMaxShards shards' lists.
constexpr int kLocalMaxBlocks = 64 * 64;
constexpr int kMergeMaxShards = 16;
hipError_t launch_topk_local(const float* scores, int ld, int begin, int stride, int n_cols,
                             const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                             int32_t* cand_ids, uint32_t* cand_keys, hipStream_t stream);
hipError_t launch_topk_merge(const int32_t* cand_ids, const uint32_t* cand_keys, int n_shards,
                             int batch, int q_len, int32_t* ids, hipStream_t stream);

// Split of the 16 selected blocks of a (sequence, token, group) row over workgroups.
int attn_num_splits(int batch, int q_len);
size_t attn_workspace_bytes(int batch, int q_len);
// Zeroes the part of an attention workspace that must be zero on entry (its counters).
hipError_t launch_attn_workspace_clear(void* workspace, int batch, int q_len, hipStream_t stream);

hipError_t launch_attention(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                            const int32_t* block_table, const int32_t* ctx_lens, int batch,
                            int max_blocks, int q_len, const uint16_t* q, const int32_t* ids,
                            float softmax_scale, uint16_t* out, void* workspace,
                            hipStream_t stream);
// The same over rows of topk (1..kMaxTopkIds) ids each; the workspace of launch_attention.
constexpr int kMaxTopkIds = 64;  // the largest selection of the window knobs
hipError_t launch_attention_topk(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                 const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                 int max_blocks, int q_len, const uint16_t* q, const int32_t* ids,
                                 int topk, float softmax_scale, uint16_t* out, void* workspace,
                                 hipStream_t stream);

// Attention for 2 to 4 query tokens per sequence over the union of their selected blocks
// (attention_union.hip): rows of up to kUnionAttnMaxBlocks blocks; the selection (kTopk ids per
// row) is made in the same launch when `scores` is given (rows of up to kSelectFusedMaxBlocks
// blocks), else ids_per_row (1 .. kTopk) ids per row are read.
// scale_log2 = softmax scale x log2(e).
constexpr int kUnionAttnMaxBlocks = 8192;
int union_num_splits(int batch);
size_t union_counter_bytes(int batch);
size_t union_workspace_bytes(int batch, int q_len);
hipError_t launch_attention_union(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                  const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                  int max_blocks, int q_len, const uint16_t* q, int32_t* ids,
                                  const float* scores, int ids_per_row, float scale_log2,
                                  uint16_t* out, void* workspace, hipStream_t stream);

// Selection fused into the attention (one launch): rows of up to this many blocks, whose
// selection one wavefront holds in 16 keys per lane; longer rows launch the two kernels.
constexpr int kSelectFusedMaxBlocks = 64 * 16 + 1;
// Rows of up to this many blocks keep the selection in the attention launch with its four
// wavefronts sharing it (one quarter of the row each); longer rows launch the two kernels.
constexpr int kSelectLongMaxBlocks = 4 * 64 * 16 + 1;
hipError_t launch_select_attention(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                                   const int32_t* block_table, const int32_t* ctx_lens, int batch,
                                   int max_blocks, int q_len, const float* scores, int32_t* ids,
                                   const uint16_t* q, float softmax_scale, uint16_t* out,
                                   void* workspace, hipStream_t stream);

// Sparse attention for a batch whose requests share their first prefix_blocks pages (sequence
// 0's table entries): each shared (block, group) dequantized once for every row that selected
// it, one partial per (row, group, slot) in the workspace, then a combine launch per row group
// that attends the private blocks and merges. At most attn_shared_prefix_max_rows() rows.
int attn_shared_prefix_max_rows();
size_t attn_shared_prefix_workspace_bytes(int batch, int q_len);
hipError_t launch_attention_shared_prefix(const uint8_t* k_pool, const uint8_t* v_pool,
                                          int64_t num_pages, const int32_t* block_table,
                                          const int32_t* ctx_lens, int batch, int max_blocks,
                                          int q_len, const uint16_t* q, const int32_t* ids,
                                          int prefix_blocks, float softmax_scale, uint16_t* out,
                                          void* workspace, hipStream_t stream);

#ifdef MSA_CHECKED
// The checked build's per-file readers of the failed-check counters (device_common.hpp): each
// adds its failures to *count, lowers *site and resets its counters.
hipError_t checks_take_attention(uint32_t* count, uint32_t* site);
hipError_t checks_take_union(uint32_t* count, uint32_t* site);
hipError_t checks_take_indexer(uint32_t* count, uint32_t* site);
hipError_t checks_take_indexer_gemm(uint32_t* count, uint32_t* site);
hipError_t checks_take_insert(uint32_t* count, uint32_t* site);
hipError_t checks_take_topk(uint32_t* count, uint32_t* site);
#endif

}  // namespace msa
