/*
 * msa.h - C ABI of libmsa.so: the MiniMax Sparse Attention (MSA) decode path with NVFP4 caches
 * on AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title and section):
 *   "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": the KV cache is split
 *   into 128-token blocks; a light indexer scores every cached key with one index query per GQA
 *   group against one shared index-key head and max-pools the scores to one score per block;
 *   exact attention then runs over the 16 best blocks only, the most recent block always kept,
 *   so a query reads at most 2,048 keys.
 *   "MiniMax-M3.1-Flash serving notes", section "The capacity numbers": both caches are NVFP4,
 *   4-bit E2M1 values with one E4M3 scale per 16 values (4.5 bits per element).
 *   "MiniMax M3 on vLLM", sections "MSA mechanism", "Decode execution" and "Speculative
 *   decoding in the decode kernels": blocks are the 128-token pages of the paged cache, main
 *   KV and index-key caches are tracked separately through the same block table, the partial
 *   last block and the causal boundary are masked, and several query tokens per request
 *   (uniform decode_query_len) are flattened request-major, each with its own causal position.
 *
 * A decode step is four calls on one stream, in this order:
 *   msa_kv_insert_nvfp4 -> msa_indexer_score -> msa_block_topk -> msa_sparse_attn_decode
 * or three, with the last two fused:
 *   msa_kv_insert_nvfp4 -> msa_indexer_score -> msa_select_attn_decode
 * or two, msa_insert_indexer_score -> msa_select_attn_decode, which one call, msa_decode_step,
 * also makes.
 *
 * Conventions for every entry point
 *   - All tensor arguments are device pointers owned by the caller. The library allocates
 *     nothing and keeps no state besides a thread-local error message and, for
 *     msa_decode_step_noalloc only, one static device array per GPU (see there).
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only enqueues work on it
 *     and returns; nothing synchronizes. Launch shapes depend only on the scalar arguments,
 *     so a step can be captured in a HIP graph.
 *   - Return value: MSA_OK or a negative MSA_ERR_* code; nothing is launched on an error.
 *     msa_last_error() then describes the failure. Arguments are checked on the host only
 *     where that costs nothing (pointers, sizes, constants). Values that live in device
 *     memory (context lengths, block-table entries, selected ids, slots) are not checked on
 *     the host; the kernels stay in bounds for any value: a page id outside [0, num_pages)
 *     or a negative slot is treated as an absent page or token, and context lengths are
 *     clamped to [0, max_blocks * 128].
 *
 * Shapes (notation): B = batch, q = query tokens per sequence (uniform), T_b = context length
 * of sequence b counting its q query tokens, which are already inserted; query token j of
 * sequence b sits at position p = T_b - q + j. 64 query heads, 4 KV heads, head h belongs to
 * KV group h / 16. head_dim = index dim = 128. bf16 tensors are passed as uint16_t bit patterns.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_BLOCK 128       /* tokens per block = tokens per cache page */
#define MSA_HEAD_DIM 128    /* head_dim of K/V and dimension of index keys/queries */
#define MSA_KV_HEADS 4      /* KV heads = GQA groups = index queries per query token */
#define MSA_Q_HEADS 64      /* query heads, 16 per group */
#define MSA_TOPK 16         /* blocks kept per (query token, group) */

/* NVFP4 page of one head: 128 tokens x 128 elements. 8,192 code bytes + 1,024 scale bytes
 * = 9,216 B (72 B per 128-element vector, 4.5 bits per element). */
#define MSA_HEAD_PAGE_BYTES 9216
#define MSA_KV_PAGE_BYTES (MSA_KV_HEADS * MSA_HEAD_PAGE_BYTES) /* 36,864 B per page of K or V */
#define MSA_IK_PAGE_BYTES MSA_HEAD_PAGE_BYTES                  /* 9,216 B per index-key page */

/* Status codes */
#define MSA_OK 0
#define MSA_ERR_INVALID_ARG (-1) /* null pointer, size out of range */
#define MSA_ERR_UNSUPPORTED (-2) /* a value the library does not implement (e.g. topk != 16) */
#define MSA_ERR_WORKSPACE (-3)   /* workspace pointer null or smaller than required */
#define MSA_ERR_HIP (-4)         /* the HIP runtime reported an error at launch */

/*
 * Paged NVFP4 caches. One page id addresses the same 128 tokens in all three pools.
 *   k  : [num_pages][4 heads][9,216 B]   keys
 *   v  : [num_pages][4 heads][9,216 B]   values
 *   ik : [num_pages][9,216 B]            index keys (one shared head)
 *
 * Within a 9,216 B head page, bytes [0, 8192) hold E2M1 codes (sign bit 3, magnitude bits
 * 2..0: 0, 0.5, 1, 1.5, 2, 3, 4, 6) and bytes [8192, 9216) hold one E4M3 (OCP "FN") scale
 * per 16 consecutive elements of a token's 128-element vector (scale group g = elements
 * 16g..16g+15). A value is E2M1(code) * E4M3(scale). Token t = 0..127 of the page, element
 * e = 0..127, group g = e / 16:
 *
 *   K and index-key pages ("row-operand" layout, a token's elements run along a row):
 *     code byte holding elements e and e+1 (e even; e in the low nibble):
 *         ((t % 32) / 4) * 1024 + 256 * (e / 32) + 64 * (t / 32) + 16 * (t % 4) + (e % 32) / 2
 *       i.e. the 16-byte chunk (t, c = e / 32) starts at
 *         ((t % 32) / 4) * 1024 + (16 c + 4 (t / 32) + t % 4) * 16
 *     scale byte: 8192 + (g / 2) * 256 + (t / 32) * 64 + (t % 4) * 16 + ((t % 32) / 4) * 2 + g % 2
 *
 *   V pages ("column-operand" layout, one element runs along the tokens):
 *     code byte holding tokens t and t+1 (t even; t in the low nibble) of element e:
 *         e * 64 + t / 2
 *     scale byte: 8192 + g * 128 + t
 *
 * These orders let each 64-lane wavefront load, with single 16-byte loads, exactly the
 * operands of its matrix-core instructions. Bytes of a page that no insert touched are left
 * as the caller initialized them (zero-initialize pools to read absent tokens as 0).
 */
typedef struct {
    uint8_t *k;
    uint8_t *v;
    uint8_t *ik;
    int64_t num_pages;
} msa_cache_t;

/*
 * A decode batch.
 *   block_table : device int32 [batch][max_blocks]; entry (b, i) = page id of logical block i
 *                 of sequence b. The whole row, max_blocks entries, must be allocated: entries
 *                 past the sequence may be read (and are then ignored); -1 marks an absent
 *                 page, and so does any id outside [0, num_pages).
 *   ctx_lens    : device int32 [batch]; T_b (tokens in the cache, query tokens included).
 *   q_len       : query tokens per sequence, uniform across the batch (1 for plain decode,
 *                 the draft length for speculative verify, the chunk length for prefill).
 */
typedef struct {
    const int32_t *block_table;
    const int32_t *ctx_lens;
    int32_t batch;
    int32_t max_blocks;
    int32_t q_len;
} msa_batch_t;

/* Bytes of one page of pool `which` (0 = K, 1 = V, 2 = index keys). 0 for other values. */
size_t msa_page_bytes(int which);

/*
 * NVFP4-quantize n tokens and write them into their cache slots. ("vLLM day-0 support for
 * MiniMax-M3.1-Flash", section "TL;DR", its item on fusing the QKV GEMM, norm, RoPE and KV insert:
 * K, V and the index key are quantized to NVFP4 as they are written to their caches.)
 *   slots : device int64 [n]; slot = page * 128 + token offset in the page. A negative slot or
 *           one whose page is outside [0, num_pages) skips that token. Slots must be distinct
 *           within one call (two tokens in one slot race).
 *   k, v  : device fp32 [n][4][128]; ik : device fp32 [n][128]. Any of the three may be NULL
 *           to leave that pool untouched.
 * Quantization of each 16-element group x[0..15] (bit-exact, fp32 as stated):
 *   s32 = max|x| / 6 (IEEE fp32 division); scale = E4M3 round-to-nearest-even of s32,
 *   saturating at 448; s = value of scale; magnitude of x_i = E2M1 nearest-even of the fp32
 *   quotient |x_i| / s (0 if s == 0, saturating at 6); sign bit = sign bit of x_i.
 *   Non-finite inputs give unspecified codes.
 * n == 0 is a no-op. Errors: MSA_ERR_INVALID_ARG (cache or slots NULL, n < 0,
 * num_pages < 1, all three value pointers NULL).
 */
int msa_kv_insert_nvfp4(const msa_cache_t *cache, const int64_t *slots, const float *k,
                        const float *v, const float *ik, int32_t n, void *stream);

/*
 * Indexer: block scores ("vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer";
 * "MiniMax M3 on vLLM", section "Decode indexer score kernel").
 *   q_idx        : device bf16 [batch * q_len][4][128]; row (b * q_len + j, g) is the index
 *                  query of group g for query token j of sequence b.
 *   block_scores : device fp32 [batch * q_len][4][max_blocks], written in full:
 *                  score(b, j, g, i) = max over tokens t of block i with t <= p and t < T_b of
 *                  sum_d q_idx[d] * ik_t[d] (exact NVFP4 values, fp32 accumulation);
 *                  -inf when the block holds no such token or its page id is out of range.
 * Errors: MSA_ERR_INVALID_ARG (NULL pointers, batch/max_blocks/q_len < 1).
 */
int msa_indexer_score(const msa_cache_t *cache, const msa_batch_t *batch, const uint16_t *q_idx,
                      float *block_scores, void *stream);

/*
 * The indexer with a choice of block reduction ("MiniMax M3 on vLLM", section "Prefill
 * execution": the block-level rule may be max or log-sum-exp, depending on the model config).
 *   reduction : MSA_REDUCE_MAX (msa_indexer_score's scores) or MSA_REDUCE_LSE:
 *               score(b, j, g, i) = log(sum over the block's valid tokens t of exp(s_t)), s_t the
 *               token score as above, computed as m + log(sum exp(s_t - m)) with m the max
 *               (fp32 exp and log); -inf when the block holds no valid token.
 * Other arguments, layouts and errors as for msa_indexer_score; MSA_ERR_UNSUPPORTED for another
 * reduction value. The LSE scores feed msa_block_topk like any scores.
 */
#define MSA_REDUCE_MAX 0
#define MSA_REDUCE_LSE 1
int msa_indexer_score_ex(const msa_cache_t *cache, const msa_batch_t *batch,
                         const uint16_t *q_idx, int32_t reduction, float *block_scores,
                         void *stream);

/*
 * The indexer for a batch that shares a prefix (requests over one long common context): every
 * sequence's blocks 0..prefix_blocks-1 are the same pages, and sequence 0's block-table entries
 * are the ones read for them. Each shared page is then dequantized once, for all the batch's
 * query rows together (a score GEMM of batch * q_len * 4 rows), instead of once per sequence
 * ("vLLM day-0 support for MiniMax-M3.1-Flash", section "NVFP4 MSA kernel": a page of a shared
 * prefix is dequantized once for up to 64 requests that share it; here the same reuse in the
 * indexer, which reads every page of every context). Blocks from prefix_blocks on are scored
 * per sequence. Scores, layout and errors as for msa_indexer_score, with the same values.
 * Requirement (not checked: the lengths live in device memory): the shared blocks hold no query
 * token, prefix_blocks * 128 <= T_b - q_len for every b; otherwise their scores for the rows of
 * such a sequence are unspecified (no memory outside the arguments is touched).
 * Errors: as msa_indexer_score, and MSA_ERR_INVALID_ARG for prefix_blocks outside
 * [0, max_blocks].
 */
int msa_indexer_score_shared_prefix(const msa_cache_t *cache, const msa_batch_t *batch,
                                    const uint16_t *q_idx, int32_t prefix_blocks,
                                    float *block_scores, void *stream);

/*
 * Block selection ("vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer"; "MiniMax
 * M3 on vLLM", section "MSA mechanism": local_blocks = 1, init_blocks = 0, the local block is
 * not counted twice). For each row (b, j, g): the eligible blocks are 0..f with
 * f = min(p / 128, max_blocks - 1); block f (the block of the query token) is always kept.
 * If at most `topk` blocks are eligible, all are kept; otherwise f and the best topk - 1 of
 * blocks 0..f-1 by (score descending, block index ascending).
 *   block_ids : device int32 [batch * q_len][4][topk], ascending block ids, padded with -1.
 * Scores must not be NaN. Rows whose token has p < 0 get all -1.
 * Errors: MSA_ERR_INVALID_ARG (NULL pointers, sizes < 1), MSA_ERR_UNSUPPORTED (topk != 16).
 */
int msa_block_topk(const float *block_scores, const msa_batch_t *batch, int32_t topk,
                   int32_t *block_ids, void *stream);

/*
 * Block selection with the window knobs of "MiniMax M3 on vLLM", section "MSA mechanism" (its
 * config exposes init blocks and local blocks; the current recipe, which msa_block_topk
 * implements, uses init_blocks = 0, local_blocks = 1 and topk = 16). For each row (b, j, g)
 * with eligible blocks 0..f (as for msa_block_topk, n = f + 1): if n <= topk all are kept;
 * otherwise blocks 0..init_blocks-1 and n-local_blocks..n-1 are always kept (a block in both
 * ranges once), and the best others by (score descending, block index ascending) fill the rest
 * of the topk places.
 *   block_ids : device int32 [batch * q_len][4][topk], ascending, padded with -1.
 * With topk = 16, init_blocks = 0, local_blocks = 1 the result is msa_block_topk's. Rows of
 * any topk feed msa_sparse_attn_decode_topk (16-id rows also every other attention call).
 * Scores must not be NaN. Errors: MSA_ERR_INVALID_ARG (NULL pointers, sizes < 1, init_blocks
 * or local_blocks < 0, init_blocks + local_blocks > topk), MSA_ERR_UNSUPPORTED (topk outside
 * 1..64, max_blocks > 4096).
 */
int msa_block_topk_window(const float *block_scores, const msa_batch_t *batch, int32_t topk,
                          int32_t init_blocks, int32_t local_blocks, int32_t *block_ids,
                          void *stream);

/*
 * The indexer over one shard of the blocks, as one device of indexer decode context
 * parallelism runs it ("vLLM day-0 support for MiniMax-M3.1-Flash", section "Indexer NVFP4
 * DCP": each device scores every index head on its own share of the context, the scores are
 * bit for bit those of a single device, and the owner of a head selects from them). The shard
 * holds global blocks block_begin + c * block_stride, c = 0..shard->max_blocks - 1 (contiguous
 * shards: stride 1; round-robin shards: begin = shard index, stride = shard count).
 *   cache          : the pool holding the shard's pages (only its index-key pages are read).
 *   shard          : block_table [batch][max_blocks]: column c holds the page of global block
 *                    block_begin + c * block_stride (-1: absent, scored -inf); ctx_lens and
 *                    q_len are the sequences' own (global positions); batch as usual.
 *   total_blocks   : the width of the whole block table the shard is cut from; the context is
 *                    clamped to total_blocks * 128 tokens as msa_indexer_score clamps it.
 *   q_idx          : device bf16 [batch * q_len][4][128], as for msa_indexer_score.
 *   shard_scores   : device fp32 [batch * q_len][4][max_blocks]: column c equals, bit for bit,
 *                    column block_begin + c * block_stride of what msa_indexer_score writes for
 *                    the whole table (-inf where no key of the block is visible to the row).
 * Feed shard_scores to msa_block_topk_local with the same begin and stride (ld = max_blocks),
 * then every shard's list to msa_block_topk_merge: the result is msa_block_topk's.
 * Errors: as msa_indexer_score, and MSA_ERR_INVALID_ARG for block_begin < 0, block_stride < 1,
 * total_blocks < 1 or too large, or a shard block >= total_blocks.
 */
int msa_indexer_score_shard(const msa_cache_t *cache, const msa_batch_t *shard,
                            int32_t block_begin, int32_t block_stride, int32_t total_blocks,
                            const uint16_t *q_idx, float *shard_scores, void *stream);

/*
 * Block selection split over shards of the blocks, as in indexer decode context parallelism
 * ("vLLM day-0 support for MiniMax-M3.1-Flash", section "Indexer NVFP4 DCP": each device
 * scores every index head on its own share of the pages and keeps a local top 16 per head;
 * the device owning the head merges the lists into the final top 16, and the selection stays
 * exact). Here every shard runs on one device: msa_block_topk_local once per shard, then
 * msa_block_topk_merge over all shards' lists gives exactly what msa_block_topk writes.
 *
 * A candidate list entry is (block id, rank key). The rank key is a 32-bit order-preserving
 * code of the score (bits u of the fp32 score with -0 read as +0: u ^ 0x80000000 for a
 * non-negative score, ~u for a negative one), or 0xFFFFFFFF for the forced block of the row
 * (the block of the query token; it outranks every score), or 0 for padding (id -1). A larger
 * key ranks first; equal keys rank by the lower block id.
 *
 * msa_block_topk_local: the shard holds blocks block_begin + c * block_stride, c = 0..n_cols-1.
 *   shard_scores : device fp32 [batch * q_len][4][ld]; column c < n_cols holds the score of the
 *                  shard's block c as msa_indexer_score computes it (other columns unread).
 *   cand_ids     : device int32 [batch * q_len][4][topk]: the best topk of the shard's eligible
 *                  blocks (blocks 0..f as for msa_block_topk, f forced), ascending, -1 padded.
 *   cand_keys    : device uint32, same shape: their rank keys (0 for padding).
 * msa_block_topk_merge: n_shards lists, shard s's at cand_ids + s * (batch * q_len * 4 * topk)
 *   (cand_keys likewise) as msa_block_topk_local writes them, shards disjoint.
 *   block_ids    : device int32 [batch * q_len][4][topk]: the best topk of the union by rank
 *                  key, ascending, -1 padded. Only batch->batch and batch->q_len are read.
 * Scores must not be NaN. Errors: MSA_ERR_INVALID_ARG (NULL pointers, sizes < 1, n_cols >
 * 4096, ld < n_cols, block_begin < 0, block_stride < 1, a shard block >= max_blocks,
 * n_shards > 16), MSA_ERR_UNSUPPORTED (topk != 16).
 */
int msa_block_topk_local(const float *shard_scores, int32_t ld, int32_t block_begin,
                         int32_t block_stride, int32_t n_cols, const msa_batch_t *batch,
                         int32_t topk, int32_t *cand_ids, uint32_t *cand_keys, void *stream);
int msa_block_topk_merge(const int32_t *cand_ids, const uint32_t *cand_keys, int32_t n_shards,
                         const msa_batch_t *batch, int32_t topk, int32_t *block_ids,
                         void *stream);

/* Workspace bytes msa_sparse_attn_decode needs for this batch shape (may be 0). */
size_t msa_sparse_attn_workspace_bytes(const msa_batch_t *batch);

/*
 * Sparse GQA attention over the selected blocks ("vLLM day-0 support for MiniMax-M3.1-Flash",
 * section "MSA primer" and its Figure 1; "MiniMax M3 on vLLM", sections "MiniMax sparse
 * attention backend" (the decode GQA kernel reads the selected pages and merges partial
 * outputs) and "Prefill execution" (the result equals dense attention restricted to the
 * selected set)).
 *   q         : device bf16 [batch * q_len][64][128]
 *   block_ids : device int32 [batch * q_len][4][16] as msa_block_topk writes them (-1 skipped)
 *   out       : device bf16 [batch * q_len][64][128]:
 *               out(b, j, h) = sum_t softmax_t(softmax_scale * q . k_t) v_t over the tokens t of
 *               the selected blocks of (b, j, h / 16) with t <= p, t < T_b (exact NVFP4 values;
 *               fp32 softmax and accumulation); 0 when no key is valid.
 *   workspace : device scratch of at least msa_sparse_attn_workspace_bytes(batch) bytes
 *               (may be NULL when that is 0), 256-byte aligned, ZERO-FILLED before its first
 *               use; every call leaves it zero-filled again where it must be (the per-row-group
 *               counters at its start), so one zero fill at allocation serves all later calls.
 *               It holds the split partial results that the workgroups of one call hand to each
 *               other; calls that share a workspace must not overlap in time (same stream, or
 *               ordered). A call that did not run to completion (a launch error reported after
 *               some of its workgroups ran, a stream torn down mid-call) or two calls that
 *               overlapped can leave counters non-zero; later calls then merge at the wrong
 *               moment and their outputs are unspecified (never a fault: every access stays in
 *               the workspace, and nothing waits on a counter). Zero-fill the workspace again
 *               before reusing it after such an event.
 * Errors: MSA_ERR_INVALID_ARG (NULL pointers, sizes < 1), MSA_ERR_WORKSPACE.
 */
int msa_sparse_attn_decode(const msa_cache_t *cache, const msa_batch_t *batch, const uint16_t *q,
                           const int32_t *block_ids, float softmax_scale, uint16_t *out,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * Sparse attention over rows of any selection size from 1 to 64 blocks, as
 * msa_block_topk_window writes them ("MiniMax M3 on vLLM", section "MSA mechanism": the top-k
 * count, the init blocks and the local blocks are configuration knobs; "vLLM day-0 support for
 * MiniMax-M3.1-Flash", section "MSA primer": exact attention over whatever the selection kept).
 * Arguments, results, workspace and errors as msa_sparse_attn_decode, with:
 *   block_ids : device int32 [batch * q_len][4][topk]; every entry that is >= 0, < max_blocks
 *               and holds a visible key is attended (-1 and other entries are skipped; a block
 *               listed twice counts twice, as the formula then says).
 *   topk      : 1..64. With topk = 16 the output is msa_sparse_attn_decode's bit for bit
 *               wherever that call runs its per-token or union kernel (below 8 query tokens
 *               per sequence or 1,024 rows), and within the attention tolerance of it where
 *               that call runs its token-tile kernel.
 *   workspace : at least msa_sparse_attn_workspace_bytes(batch) bytes, the same contract.
 * Rows of up to 16 ids take the union kernel where the 16-id call does (2-4 query tokens per
 * sequence, 16 sequences and more); every other shape runs the per-token kernel (each wavefront
 * streams ceil(topk / (4 splits)) blocks in turn).
 * Errors: as msa_sparse_attn_decode; MSA_ERR_UNSUPPORTED for topk outside 1..64.
 */
int msa_sparse_attn_decode_topk(const msa_cache_t *cache, const msa_batch_t *batch,
                                const uint16_t *q, const int32_t *block_ids, int32_t topk,
                                float softmax_scale, uint16_t *out, void *workspace,
                                size_t ws_bytes, void *stream);

/*
 * Sparse attention for a batch whose requests share a prefix: every sequence's blocks
 * 0..prefix_blocks-1 are the same pages, and sequence 0's block-table entries are the ones read
 * for them ("vLLM day-0 support for MiniMax-M3.1-Flash", section "NVFP4 MSA kernel": a page of
 * a shared prefix is dequantized once for up to 64 requests that share it). Each shared
 * (block, KV group) that any row selected is loaded and dequantized once, for all the rows of
 * the batch that selected it (one launch, a workgroup per shared block and group), and each
 * row's own blocks are attended per row in a second launch that merges the two by log-sum-exp.
 * Arguments, results and errors as msa_sparse_attn_decode (the same values within its
 * floating-point tolerance; the shared blocks' partial outputs pass through fp16, normalized by
 * their sums, as the selected V values themselves are), with:
 *   prefix_blocks : shared blocks, 0..max_blocks (0: every block is attended per row).
 *   workspace     : device scratch of at least msa_sparse_attn_shared_prefix_workspace_bytes
 *                   (batch) bytes (4,224 per (row, group, slot)), 256-byte aligned; no fill
 *                   needed (every partial read is written by the same call first); calls that
 *                   share it must not overlap in time.
 * Requirement (not checked: the lengths live in device memory): the shared blocks hold no query
 * token, prefix_blocks * 128 <= T_b - q_len for every b, and a row's block ids are distinct (as
 * msa_block_topk writes them). Otherwise the output is unspecified (no memory outside the
 * arguments is touched).
 * Errors: as msa_sparse_attn_decode; MSA_ERR_INVALID_ARG for prefix_blocks outside
 * [0, max_blocks]; MSA_ERR_UNSUPPORTED for batch * q_len above 1,024 rows.
 */
size_t msa_sparse_attn_shared_prefix_workspace_bytes(const msa_batch_t *batch);
int msa_sparse_attn_decode_shared_prefix(const msa_cache_t *cache, const msa_batch_t *batch,
                                         const uint16_t *q, const int32_t *block_ids,
                                         int32_t prefix_blocks, float softmax_scale,
                                         uint16_t *out, void *workspace, size_t ws_bytes,
                                         void *stream);

/*
 * Selection and attention in one launch: the effect of msa_block_topk(block_scores, batch, topk,
 * block_ids) followed by msa_sparse_attn_decode(cache, batch, q, block_ids, softmax_scale, out,
 * workspace, ws_bytes), with the same results bit for bit (block_ids is written as well), but
 * each attention workgroup selects its row's blocks itself from the scores, so the selection
 * needs no launch of its own and its ids no round trip through memory ("MiniMax M3 on vLLM",
 * section "Decode indexer score kernel": the top-k boundary stays close to the scores). Rows of
 * 1,026 to 4,097 blocks keep one launch when the batch has fewer than 128 query tokens in all
 * and does not take the speculative-verify kernel (the four wavefronts of a workgroup then
 * share the selection, a quarter of the row each); longer rows, and those other batches with
 * max_blocks > 1025, run the two steps as two launches, and so do batches of 8 or more query
 * tokens per sequence with at least 1,024 (token, group) rows (prefill chunks), whose
 * attention streams the union of 16 tokens' blocks once per workgroup instead of once per
 * token.
 * Arguments and workspace as for the two calls. Errors: as for the two calls.
 */
int msa_select_attn_decode(const msa_cache_t *cache, const msa_batch_t *batch,
                           const float *block_scores, int32_t topk, int32_t *block_ids,
                           const uint16_t *q, float softmax_scale, uint16_t *out,
                           void *workspace, size_t ws_bytes, void *stream);

/*
 * Insert of the step's new tokens and the indexer in one launch: the effect of
 *   msa_kv_insert_nvfp4(cache, slots, k, v, ik, batch * q_len)
 *   msa_indexer_score(cache, batch, q_idx, block_scores)
 * with the slots of the new tokens' own positions (as msa_decode_step below states), the same
 * results bit for bit, cache bytes included. With more than 8 query tokens per sequence the
 * two run as two launches (the indexer then as a score GEMM, each page dequantized once for
 * all the sequence's query rows; msa_indexer_score does the same from 9 tokens on).
 * Arguments as for msa_decode_step. Errors:
 * MSA_ERR_INVALID_ARG (a NULL pointer, sizes < 1).
 */
int msa_insert_indexer_score(const msa_cache_t *cache, const msa_batch_t *batch, const float *k,
                             const float *v, const float *ik, const uint16_t *q_idx,
                             float *block_scores, void *stream);

/*
 * One whole decode step in two launches (msa_insert_indexer_score, then
 * msa_select_attn_decode): the effect of
 *   msa_kv_insert_nvfp4(cache, slots, k, v, ik, batch * q_len)
 *   msa_indexer_score(cache, batch, q_idx, block_scores)
 *   msa_select_attn_decode(cache, batch, block_scores, topk, block_ids, q, softmax_scale, out,
 *                          workspace, ws_bytes)
 * where the slots are the new tokens' own positions: query token j of sequence b is written at
 * position T_b - q_len + j, into page block_table(b, (T_b - q_len + j) / 128) at token
 * (T_b - q_len + j) % 128 ("MiniMax M3 on vLLM", section "Decode execution": the step's keys,
 * values and index keys are written to the paged caches before the indexer and attention read
 * them). Tokens at negative positions (T_b < q_len) are skipped. Results, cache bytes included,
 * are those of the three calls bit for bit. The insert runs in the indexer's launch: the
 * indexer quantizes the sequence's new index keys itself into its copy of the pages it scores,
 * so it needs no finished insert ("vLLM day-0 support for MiniMax-M3.1-Flash", section "TL;DR",
 * its item on fusing the QKV GEMM, norm, RoPE and KV insert: the insert is fused into the step's
 * first kernel; "MiniMax M3 on vLLM", its roadmap section: fusing the many small indexer, top-k
 * and quantization kernels). With q_len > 8 the insert runs as a launch of its own before the
 * indexer.
 *   k, v : device fp32 [batch * q_len][4][128]; ik : device fp32 [batch * q_len][128]
 *          (request-major, as q); q_idx, q, block_scores, block_ids, out, workspace as for the
 *          calls above.
 * Errors: MSA_ERR_INVALID_ARG (a NULL pointer, sizes < 1), MSA_ERR_UNSUPPORTED (topk != 16),
 * MSA_ERR_WORKSPACE.
 */
int msa_decode_step(const msa_cache_t *cache, const msa_batch_t *batch, const float *k,
                    const float *v, const float *ik, const uint16_t *q_idx, const uint16_t *q,
                    int32_t topk, float softmax_scale, float *block_scores, int32_t *block_ids,
                    uint16_t *out, void *workspace, size_t ws_bytes, void *stream);

/*
 * One whole decode step with the selection's window knobs ("MiniMax M3 on vLLM", section "MSA
 * mechanism": the number of kept blocks and the init and local windows are configuration
 * knobs), in three launches: the effect of
 *   msa_insert_indexer_score(cache, batch, k, v, ik, q_idx, block_scores)
 *   msa_block_topk_window(block_scores, batch, topk, init_blocks, local_blocks, block_ids)
 *   msa_sparse_attn_decode_topk(cache, batch, q, block_ids, topk, softmax_scale, out,
 *                               workspace, ws_bytes)
 * on one stream, with those calls' results bit for bit. Arguments as for msa_decode_step, with:
 *   topk, init_blocks, local_blocks : as msa_block_topk_window takes them (topk 1..64,
 *          init_blocks + local_blocks <= topk); block_ids is [batch * q_len][4][topk].
 * Errors: MSA_ERR_INVALID_ARG (a NULL pointer, sizes < 1, knobs out of range),
 * MSA_ERR_UNSUPPORTED (topk outside 1..64, rows longer than msa_block_topk_window builds),
 * MSA_ERR_WORKSPACE.
 */
int msa_decode_step_window(const msa_cache_t *cache, const msa_batch_t *batch, const float *k,
                           const float *v, const float *ik, const uint16_t *q_idx,
                           const uint16_t *q, int32_t topk, int32_t init_blocks,
                           int32_t local_blocks, float softmax_scale, float *block_scores,
                           int32_t *block_ids, uint16_t *out, void *workspace, size_t ws_bytes,
                           void *stream);

/*
 * msa_decode_step for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, and harnesses that forbid hipMalloc. The same two launches and results,
 * bit for bit, as msa_decode_step with a workspace, preceded by one small kernel that zeroes the
 * workspace's counters. The attention's workspace is instead a static device array of the
 * library, 20 MiB (20,971,520 bytes), one per GPU, held until the process ends; no allocation of
 * any kind happens in this call. Every shape the current kernels run needs at most about
 * 17.3 MB of it (batches with fewer than 1,024 (token, group) rows; larger ones need none); a
 * batch that would need more is rejected with MSA_ERR_WORKSPACE before anything is launched.
 * All calls on one GPU share that array: calls that overlap in time on one GPU (different
 * streams, or threads without ordering) race and give undefined results; calls ordered on one
 * stream are safe. Arguments as for msa_decode_step, without the workspace.
 * Errors: as msa_decode_step; MSA_ERR_HIP if the array's device address cannot be obtained.
 */
int msa_decode_step_noalloc(const msa_cache_t *cache, const msa_batch_t *batch, const float *k,
                            const float *v, const float *ik, const uint16_t *q_idx,
                            const uint16_t *q, int32_t topk, float softmax_scale,
                            float *block_scores, int32_t *block_ids, uint16_t *out, void *stream);

/* Message of the last failed call on this thread ("" if none). */
const char *msa_last_error(void);

/* Library version string. */
const char *msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
