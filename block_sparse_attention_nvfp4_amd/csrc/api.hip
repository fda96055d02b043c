// C entry points of libmsa.so (declared and documented in include/msa.h and include/msa_debug.h): host-side argument
// checks, then asynchronous launches on the caller's stream.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/msa.h"
#include "../../include/msa_debug.h"
#include "kernels.hpp"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_last_error[0] = '\0';
    return MSA_OK;
}

int hip_status(hipError_t err, const char* what) {
    if (err != hipSuccess) return fail(MSA_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
    return ok();
}

int check_batch(const msa_batch_t* batch, const char* fn) {
    if (!batch) return fail(MSA_ERR_INVALID_ARG, "%s: batch is NULL", fn);
    if (!batch->block_table || !batch->ctx_lens)
        return fail(MSA_ERR_INVALID_ARG, "%s: block_table or ctx_lens is NULL", fn);
    if (batch->batch < 1 || batch->max_blocks < 1 || batch->q_len < 1)
        return fail(MSA_ERR_INVALID_ARG, "%s: batch=%d max_blocks=%d q_len=%d must all be >= 1", fn,
                    batch->batch, batch->max_blocks, batch->q_len);
    if (batch->batch > 65535)
        return fail(MSA_ERR_INVALID_ARG, "%s: batch=%d exceeds 65535", fn, batch->batch);
    if ((int64_t)batch->max_blocks * MSA_BLOCK > INT32_MAX / 2)
        return fail(MSA_ERR_INVALID_ARG, "%s: max_blocks=%d too large", fn, batch->max_blocks);
    const int64_t rows = (int64_t)batch->batch * batch->q_len * MSA_KV_HEADS;
    if (rows > INT32_MAX / 64)
        return fail(MSA_ERR_INVALID_ARG, "%s: batch*q_len=%lld too large", fn,
                    (long long)batch->batch * batch->q_len);
    return MSA_OK;
}

int check_cache(const msa_cache_t* cache, const char* fn, bool need_kv, bool need_ik) {
    if (!cache) return fail(MSA_ERR_INVALID_ARG, "%s: cache is NULL", fn);
    if (cache->num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "%s: num_pages must be >= 1", fn);
    if (need_kv && (!cache->k || !cache->v))
        return fail(MSA_ERR_INVALID_ARG, "%s: K or V pool is NULL", fn);
    if (need_ik && !cache->ik) return fail(MSA_ERR_INVALID_ARG, "%s: index-key pool is NULL", fn);
    return MSA_OK;
}

// The attention workspace of msa_decode_step_noalloc: a device array of the library, one copy
// per GPU, which each device keeps until the process ends. Host code never passes the array's
// name to a kernel (on the host it only stands for the symbol); it asks the runtime for the
// array's device address once per device and uses that pointer.
constexpr size_t kNoallocScratchBytes = (size_t)20 << 20;  // 20 MiB
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device (looked up on the first call there).
hipError_t noalloc_scratch(void** ptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t msa_page_bytes(int which) {
    switch (which) {
        case 0:
        case 1:
            return MSA_KV_PAGE_BYTES;
        case 2:
            return MSA_IK_PAGE_BYTES;
        default:
            return 0;
    }
}

const char* msa_last_error(void) { return g_last_error; }

const char* msa_version(void) {
#ifdef MSA_CHECKED
    return "msa-mi355x 0.1 (gfx950, checked)";
#else
    return "msa-mi355x 0.1 (gfx950)";
#endif
}

int msa_debug_checks(uint32_t* count, uint32_t* site) {
    static const char* fn = "msa_debug_checks";
    if (!count || !site) return fail(MSA_ERR_INVALID_ARG, "%s: count or site is NULL", fn);
#ifdef MSA_CHECKED
    uint32_t n = 0, lowest = 0xFFFFFFFFu;
    for (auto take : {msa::checks_take_attention, msa::checks_take_union, msa::checks_take_indexer,
                      msa::checks_take_indexer_gemm, msa::checks_take_insert,
                      msa::checks_take_topk}) {
        const hipError_t e = take(&n, &lowest);
        if (e != hipSuccess)
            return fail(MSA_ERR_HIP, "%s: reading the check counters: %s", fn, hipGetErrorString(e));
    }
    *count = n;
    *site = lowest == 0xFFFFFFFFu ? 0u : lowest;
    return MSA_OK;
#else
    *count = 0;
    *site = 0;
    return fail(MSA_ERR_UNSUPPORTED, "%s: this library is built without the checks (use libmsa_checked.so)", fn);
#endif
}

int msa_kv_insert_nvfp4(const msa_cache_t* cache, const int64_t* slots, const float* k,
                        const float* v, const float* ik, int32_t n, void* stream) {
    static const char* fn = "msa_kv_insert_nvfp4";
    if (!cache) return fail(MSA_ERR_INVALID_ARG, "%s: cache is NULL", fn);
    if (!slots) return fail(MSA_ERR_INVALID_ARG, "%s: slots is NULL", fn);
    if (n < 0) return fail(MSA_ERR_INVALID_ARG, "%s: n=%d < 0", fn, n);
    if (!k && !v && !ik) return fail(MSA_ERR_INVALID_ARG, "%s: k, v and ik are all NULL", fn);
    if (cache->num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "%s: num_pages must be >= 1", fn);
    if ((k && !cache->k) || (v && !cache->v) || (ik && !cache->ik))
        return fail(MSA_ERR_INVALID_ARG, "%s: a pool for supplied values is NULL", fn);
    if (n == 0) return ok();
    return hip_status(msa::launch_insert(cache->k, cache->v, cache->ik, cache->num_pages, slots, k,
                                         v, ik, n, (hipStream_t)stream),
                      fn);
}

int msa_indexer_score(const msa_cache_t* cache, const msa_batch_t* batch, const uint16_t* q_idx,
                      float* block_scores, void* stream) {
    static const char* fn = "msa_indexer_score";
    int rc = check_cache(cache, fn, false, true);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q_idx || !block_scores) return fail(MSA_ERR_INVALID_ARG, "%s: q_idx or block_scores is NULL", fn);
    return hip_status(msa::launch_indexer(cache->ik, cache->num_pages, batch->block_table,
                                          batch->ctx_lens, batch->batch, batch->max_blocks,
                                          batch->q_len, q_idx, block_scores, (hipStream_t)stream),
                      fn);
}

int msa_indexer_score_ex(const msa_cache_t* cache, const msa_batch_t* batch,
                         const uint16_t* q_idx, int32_t reduction, float* block_scores,
                         void* stream) {
    static const char* fn = "msa_indexer_score_ex";
    int rc = check_cache(cache, fn, false, true);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q_idx || !block_scores) return fail(MSA_ERR_INVALID_ARG, "%s: q_idx or block_scores is NULL", fn);
    if (reduction == MSA_REDUCE_MAX)
        return hip_status(msa::launch_indexer(cache->ik, cache->num_pages, batch->block_table,
                                              batch->ctx_lens, batch->batch, batch->max_blocks,
                                              batch->q_len, q_idx, block_scores, (hipStream_t)stream),
                          fn);
    if (reduction != MSA_REDUCE_LSE)
        return fail(MSA_ERR_UNSUPPORTED, "%s: reduction=%d (0 = max, 1 = log-sum-exp)", fn, reduction);
    return hip_status(msa::launch_indexer_gemm(cache->ik, cache->num_pages, batch->block_table,
                                               batch->ctx_lens, batch->batch, batch->max_blocks,
                                               batch->q_len, q_idx, block_scores,
                                               (hipStream_t)stream, true),
                      fn);
}

int msa_indexer_score_shared_prefix(const msa_cache_t* cache, const msa_batch_t* batch,
                                    const uint16_t* q_idx, int32_t prefix_blocks,
                                    float* block_scores, void* stream) {
    static const char* fn = "msa_indexer_score_shared_prefix";
    int rc = check_cache(cache, fn, false, true);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q_idx || !block_scores) return fail(MSA_ERR_INVALID_ARG, "%s: q_idx or block_scores is NULL", fn);
    if (prefix_blocks < 0 || prefix_blocks > batch->max_blocks)
        return fail(MSA_ERR_INVALID_ARG, "%s: prefix_blocks=%d outside [0, max_blocks=%d]", fn,
                    prefix_blocks, batch->max_blocks);
    return hip_status(msa::launch_indexer_shared_prefix(cache->ik, cache->num_pages,
                                                        batch->block_table, batch->ctx_lens,
                                                        batch->batch, batch->max_blocks,
                                                        batch->q_len, q_idx, block_scores,
                                                        prefix_blocks, (hipStream_t)stream),
                      fn);
}

int msa_indexer_score_shard(const msa_cache_t* cache, const msa_batch_t* shard,
                            int32_t block_begin, int32_t block_stride, int32_t total_blocks,
                            const uint16_t* q_idx, float* shard_scores, void* stream) {
    static const char* fn = "msa_indexer_score_shard";
    int rc = check_cache(cache, fn, false, true);
    if (rc) return rc;
    if ((rc = check_batch(shard, fn))) return rc;
    if (!q_idx || !shard_scores) return fail(MSA_ERR_INVALID_ARG, "%s: q_idx or shard_scores is NULL", fn);
    if (block_begin < 0 || block_stride < 1 || total_blocks < 1 ||
        (int64_t)total_blocks * MSA_BLOCK > INT32_MAX / 2)
        return fail(MSA_ERR_INVALID_ARG, "%s: block_begin=%d, block_stride=%d, total_blocks=%d", fn,
                    block_begin, block_stride, total_blocks);
    const int64_t last = (int64_t)block_begin + (int64_t)(shard->max_blocks - 1) * block_stride;
    if (last >= total_blocks)
        return fail(MSA_ERR_INVALID_ARG, "%s: the shard's last block %lld is past total_blocks=%d",
                    fn, (long long)last, total_blocks);
    return hip_status(msa::launch_indexer_shard(cache->ik, cache->num_pages, shard->block_table,
                                                shard->ctx_lens, shard->batch, shard->max_blocks,
                                                shard->q_len, q_idx, shard_scores, block_begin,
                                                block_stride, total_blocks, (hipStream_t)stream),
                      fn);
}

int msa_block_topk(const float* block_scores, const msa_batch_t* batch, int32_t topk,
                   int32_t* block_ids, void* stream) {
    static const char* fn = "msa_block_topk";
    int rc = check_batch(batch, fn);
    if (rc) return rc;
    if (!block_scores || !block_ids)
        return fail(MSA_ERR_INVALID_ARG, "%s: block_scores or block_ids is NULL", fn);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    return hip_status(msa::launch_topk(block_scores, batch->ctx_lens, batch->batch,
                                       batch->max_blocks, batch->q_len, block_ids,
                                       (hipStream_t)stream),
                      fn);
}

int msa_block_topk_window(const float* block_scores, const msa_batch_t* batch, int32_t topk,
                          int32_t init_blocks, int32_t local_blocks, int32_t* block_ids,
                          void* stream) {
    static const char* fn = "msa_block_topk_window";
    int rc = check_batch(batch, fn);
    if (rc) return rc;
    if (!block_scores || !block_ids)
        return fail(MSA_ERR_INVALID_ARG, "%s: block_scores or block_ids is NULL", fn);
    if (topk < 1 || topk > 64)
        return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (1..64 are built)", fn, topk);
    if (init_blocks < 0 || local_blocks < 0 || init_blocks + local_blocks > topk)
        return fail(MSA_ERR_INVALID_ARG,
                    "%s: init_blocks=%d and local_blocks=%d must be >= 0 and sum to at most topk=%d",
                    fn, init_blocks, local_blocks, topk);
    if (batch->max_blocks > msa::kWindowMaxBlocks)
        return fail(MSA_ERR_UNSUPPORTED, "%s: max_blocks=%d (up to %d are built)", fn,
                    batch->max_blocks, msa::kWindowMaxBlocks);
    return hip_status(msa::launch_topk_window(block_scores, batch->ctx_lens, batch->batch,
                                              batch->max_blocks, batch->q_len, topk, init_blocks,
                                              local_blocks, block_ids, (hipStream_t)stream),
                      fn);
}

int msa_block_topk_local(const float* shard_scores, int32_t ld, int32_t block_begin,
                         int32_t block_stride, int32_t n_cols, const msa_batch_t* batch,
                         int32_t topk, int32_t* cand_ids, uint32_t* cand_keys, void* stream) {
    static const char* fn = "msa_block_topk_local";
    int rc = check_batch(batch, fn);
    if (rc) return rc;
    if (!shard_scores || !cand_ids || !cand_keys)
        return fail(MSA_ERR_INVALID_ARG, "%s: shard_scores, cand_ids or cand_keys is NULL", fn);
    if (n_cols < 1 || n_cols > msa::kLocalMaxBlocks || ld < n_cols)
        return fail(MSA_ERR_INVALID_ARG, "%s: n_cols=%d must be in [1, %d] and ld=%d >= n_cols", fn,
                    n_cols, msa::kLocalMaxBlocks, ld);
    if (block_begin < 0 || block_stride < 1 ||
        block_begin + (int64_t)(n_cols - 1) * block_stride >= batch->max_blocks)
        return fail(MSA_ERR_INVALID_ARG,
                    "%s: blocks %d + c * %d (c < %d) must lie in [0, max_blocks=%d)", fn,
                    block_begin, block_stride, n_cols, batch->max_blocks);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    return hip_status(msa::launch_topk_local(shard_scores, ld, block_begin, block_stride, n_cols,
                                             batch->ctx_lens, batch->batch, batch->max_blocks,
                                             batch->q_len, cand_ids, cand_keys,
                                             (hipStream_t)stream),
                      fn);
}

int msa_block_topk_merge(const int32_t* cand_ids, const uint32_t* cand_keys, int32_t n_shards,
                         const msa_batch_t* batch, int32_t topk, int32_t* block_ids,
                         void* stream) {
    static const char* fn = "msa_block_topk_merge";
    if (!batch) return fail(MSA_ERR_INVALID_ARG, "%s: batch is NULL", fn);
    if (batch->batch < 1 || batch->q_len < 1 || batch->batch > 65535 ||
        (int64_t)batch->batch * batch->q_len * MSA_KV_HEADS > INT32_MAX / 1024)
        return fail(MSA_ERR_INVALID_ARG, "%s: batch=%d q_len=%d out of range", fn, batch->batch,
                    batch->q_len);
    if (!cand_ids || !cand_keys || !block_ids)
        return fail(MSA_ERR_INVALID_ARG, "%s: cand_ids, cand_keys or block_ids is NULL", fn);
    if (n_shards < 1 || n_shards > msa::kMergeMaxShards)
        return fail(MSA_ERR_INVALID_ARG, "%s: n_shards=%d must be in [1, %d]", fn, n_shards,
                    msa::kMergeMaxShards);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    return hip_status(msa::launch_topk_merge(cand_ids, cand_keys, n_shards, batch->batch,
                                             batch->q_len, block_ids, (hipStream_t)stream),
                      fn);
}

size_t msa_sparse_attn_workspace_bytes(const msa_batch_t* batch) {
    if (!batch || batch->batch < 1 || batch->q_len < 1) return 0;
    return msa::attn_workspace_bytes(batch->batch, batch->q_len);
}

static int check_workspace(const msa_batch_t* batch, void* workspace, size_t ws_bytes,
                           const char* fn) {
    const size_t need = msa::attn_workspace_bytes(batch->batch, batch->q_len);
    if (need > 0 && (!workspace || ws_bytes < need))
        return fail(MSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? ws_bytes : (size_t)0);
    if (need > 0 && ((uintptr_t)workspace & 255u))
        return fail(MSA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    return MSA_OK;
}

int msa_sparse_attn_decode(const msa_cache_t* cache, const msa_batch_t* batch, const uint16_t* q,
                           const int32_t* block_ids, float softmax_scale, uint16_t* out,
                           void* workspace, size_t ws_bytes, void* stream) {
    static const char* fn = "msa_sparse_attn_decode";
    int rc = check_cache(cache, fn, true, false);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if ((rc = check_workspace(batch, workspace, ws_bytes, fn))) return rc;
    return hip_status(msa::launch_attention(cache->k, cache->v, cache->num_pages,
                                            batch->block_table, batch->ctx_lens, batch->batch,
                                            batch->max_blocks, batch->q_len, q, block_ids,
                                            softmax_scale, out, workspace,
                                            (hipStream_t)stream),
                      fn);
}

int msa_sparse_attn_decode_topk(const msa_cache_t* cache, const msa_batch_t* batch,
                                const uint16_t* q, const int32_t* block_ids, int32_t topk,
                                float softmax_scale, uint16_t* out, void* workspace,
                                size_t ws_bytes, void* stream) {
    static const char* fn = "msa_sparse_attn_decode_topk";
    int rc = check_cache(cache, fn, true, false);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if (topk < 1 || topk > msa::kMaxTopkIds)
        return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (1..%d are built)", fn, topk,
                    msa::kMaxTopkIds);
    if ((rc = check_workspace(batch, workspace, ws_bytes, fn))) return rc;
    return hip_status(msa::launch_attention_topk(cache->k, cache->v, cache->num_pages,
                                                 batch->block_table, batch->ctx_lens,
                                                 batch->batch, batch->max_blocks, batch->q_len, q,
                                                 block_ids, topk, softmax_scale, out, workspace,
                                                 (hipStream_t)stream),
                      fn);
}

size_t msa_sparse_attn_shared_prefix_workspace_bytes(const msa_batch_t* batch) {
    if (!batch || batch->batch < 1 || batch->q_len < 1) return 0;
    return msa::attn_shared_prefix_workspace_bytes(batch->batch, batch->q_len);
}

int msa_sparse_attn_decode_shared_prefix(const msa_cache_t* cache, const msa_batch_t* batch,
                                         const uint16_t* q, const int32_t* block_ids,
                                         int32_t prefix_blocks, float softmax_scale,
                                         uint16_t* out, void* workspace, size_t ws_bytes,
                                         void* stream) {
    static const char* fn = "msa_sparse_attn_decode_shared_prefix";
    int rc = check_cache(cache, fn, true, false);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if (prefix_blocks < 0 || prefix_blocks > batch->max_blocks)
        return fail(MSA_ERR_INVALID_ARG, "%s: prefix_blocks=%d outside [0, max_blocks=%d]", fn,
                    prefix_blocks, batch->max_blocks);
    const int64_t rows = (int64_t)batch->batch * batch->q_len;
    if (rows > msa::attn_shared_prefix_max_rows())
        return fail(MSA_ERR_UNSUPPORTED, "%s: batch*q_len=%lld above %d", fn, (long long)rows,
                    msa::attn_shared_prefix_max_rows());
    const size_t need = msa::attn_shared_prefix_workspace_bytes(batch->batch, batch->q_len);
    if (!workspace || ws_bytes < need)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                    workspace ? ws_bytes : (size_t)0);
    if ((uintptr_t)workspace & 255u)
        return fail(MSA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", fn);
    return hip_status(msa::launch_attention_shared_prefix(
                          cache->k, cache->v, cache->num_pages, batch->block_table,
                          batch->ctx_lens, batch->batch, batch->max_blocks, batch->q_len, q,
                          block_ids, prefix_blocks, softmax_scale, out, workspace,
                          (hipStream_t)stream),
                      fn);
}

int msa_select_attn_decode(const msa_cache_t* cache, const msa_batch_t* batch,
                           const float* block_scores, int32_t topk, int32_t* block_ids,
                           const uint16_t* q, float softmax_scale, uint16_t* out,
                           void* workspace, size_t ws_bytes, void* stream) {
    static const char* fn = "msa_select_attn_decode";
    int rc = check_cache(cache, fn, true, false);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!block_scores || !block_ids || !q || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: block_scores, block_ids, q or out is NULL", fn);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    if ((rc = check_workspace(batch, workspace, ws_bytes, fn))) return rc;
    return hip_status(msa::launch_select_attention(cache->k, cache->v, cache->num_pages,
                                                   batch->block_table, batch->ctx_lens,
                                                   batch->batch, batch->max_blocks, batch->q_len,
                                                   block_scores, block_ids, q, softmax_scale, out,
                                                   workspace, (hipStream_t)stream),
                      fn);
}

static int check_insert_indexer(const msa_cache_t* cache, const msa_batch_t* batch,
                                const float* k, const float* v, const float* ik,
                                const uint16_t* q_idx, const float* block_scores, const char* fn) {
    int rc = check_cache(cache, fn, true, true);
    if (rc) return rc;
    if ((rc = check_batch(batch, fn))) return rc;
    if (!k || !v || !ik || !q_idx || !block_scores)
        return fail(MSA_ERR_INVALID_ARG, "%s: k, v, ik, q_idx or block_scores is NULL", fn);
    return MSA_OK;
}

int msa_insert_indexer_score(const msa_cache_t* cache, const msa_batch_t* batch, const float* k,
                             const float* v, const float* ik, const uint16_t* q_idx,
                             float* block_scores, void* stream) {
    static const char* fn = "msa_insert_indexer_score";
    const int rc = check_insert_indexer(cache, batch, k, v, ik, q_idx, block_scores, fn);
    if (rc) return rc;
    return hip_status(msa::launch_insert_indexer(cache->k, cache->v, cache->ik, cache->num_pages,
                                                 batch->block_table, batch->ctx_lens,
                                                 batch->batch, batch->max_blocks, batch->q_len, k,
                                                 v, ik, q_idx, block_scores, (hipStream_t)stream),
                      fn);
}

int msa_decode_step(const msa_cache_t* cache, const msa_batch_t* batch, const float* k,
                    const float* v, const float* ik, const uint16_t* q_idx, const uint16_t* q,
                    int32_t topk, float softmax_scale, float* block_scores, int32_t* block_ids,
                    uint16_t* out, void* workspace, size_t ws_bytes, void* stream) {
    static const char* fn = "msa_decode_step";
    int rc = check_insert_indexer(cache, batch, k, v, ik, q_idx, block_scores, fn);
    if (rc) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    if ((rc = check_workspace(batch, workspace, ws_bytes, fn))) return rc;
    const hipStream_t s = (hipStream_t)stream;
    rc = hip_status(msa::launch_insert_indexer(cache->k, cache->v, cache->ik, cache->num_pages,
                                               batch->block_table, batch->ctx_lens, batch->batch,
                                               batch->max_blocks, batch->q_len, k, v, ik, q_idx,
                                               block_scores, s),
                    fn);
    if (rc) return rc;
    return hip_status(msa::launch_select_attention(cache->k, cache->v, cache->num_pages,
                                                   batch->block_table, batch->ctx_lens,
                                                   batch->batch, batch->max_blocks, batch->q_len,
                                                   block_scores, block_ids, q, softmax_scale, out,
                                                   workspace, s),
                      fn);
}

int msa_decode_step_window(const msa_cache_t* cache, const msa_batch_t* batch, const float* k,
                           const float* v, const float* ik, const uint16_t* q_idx,
                           const uint16_t* q, int32_t topk, int32_t init_blocks,
                           int32_t local_blocks, float softmax_scale, float* block_scores,
                           int32_t* block_ids, uint16_t* out, void* workspace, size_t ws_bytes,
                           void* stream) {
    static const char* fn = "msa_decode_step_window";
    int rc = check_insert_indexer(cache, batch, k, v, ik, q_idx, block_scores, fn);
    if (rc) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if (topk < 1 || topk > msa::kMaxTopkIds)
        return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (1..%d are built)", fn, topk,
                    msa::kMaxTopkIds);
    if (init_blocks < 0 || local_blocks < 0 || init_blocks + local_blocks > topk)
        return fail(MSA_ERR_INVALID_ARG,
                    "%s: init_blocks=%d and local_blocks=%d must be >= 0 and sum to at most topk=%d",
                    fn, init_blocks, local_blocks, topk);
    if (batch->max_blocks > msa::kWindowMaxBlocks)
        return fail(MSA_ERR_UNSUPPORTED, "%s: max_blocks=%d (up to %d are built)", fn,
                    batch->max_blocks, msa::kWindowMaxBlocks);
    if ((rc = check_workspace(batch, workspace, ws_bytes, fn))) return rc;
    const hipStream_t s = (hipStream_t)stream;
    rc = hip_status(msa::launch_insert_indexer(cache->k, cache->v, cache->ik, cache->num_pages,
                                               batch->block_table, batch->ctx_lens, batch->batch,
                                               batch->max_blocks, batch->q_len, k, v, ik, q_idx,
                                               block_scores, s),
                    fn);
    if (rc) return rc;
    rc = hip_status(msa::launch_topk_window(block_scores, batch->ctx_lens, batch->batch,
                                            batch->max_blocks, batch->q_len, topk, init_blocks,
                                            local_blocks, block_ids, s),
                    fn);
    if (rc) return rc;
    return hip_status(msa::launch_attention_topk(cache->k, cache->v, cache->num_pages,
                                                 batch->block_table, batch->ctx_lens,
                                                 batch->batch, batch->max_blocks, batch->q_len, q,
                                                 block_ids, topk, softmax_scale, out, workspace,
                                                 s),
                      fn);
}

int msa_decode_step_noalloc(const msa_cache_t* cache, const msa_batch_t* batch, const float* k,
                            const float* v, const float* ik, const uint16_t* q_idx,
                            const uint16_t* q, int32_t topk, float softmax_scale,
                            float* block_scores, int32_t* block_ids, uint16_t* out,
                            void* stream) {
    static const char* fn = "msa_decode_step_noalloc";
    int rc = check_insert_indexer(cache, batch, k, v, ik, q_idx, block_scores, fn);
    if (rc) return rc;
    if (!q || !block_ids || !out)
        return fail(MSA_ERR_INVALID_ARG, "%s: q, block_ids or out is NULL", fn);
    if (topk != MSA_TOPK) return fail(MSA_ERR_UNSUPPORTED, "%s: topk=%d (only 16 is built)", fn, topk);
    const size_t need = msa::attn_workspace_bytes(batch->batch, batch->q_len);
    if (need > kNoallocScratchBytes)
        return fail(MSA_ERR_WORKSPACE,
                    "%s: this batch needs %zu bytes of attention workspace; the library's static "
                    "scratch holds %zu (use msa_decode_step with a workspace)",
                    fn, need, kNoallocScratchBytes);
    const hipStream_t s = (hipStream_t)stream;
    void* ws = nullptr;
    if (need > 0) {
        if ((rc = hip_status(noalloc_scratch(&ws), fn))) return rc;
        // the counters must start at zero whatever an earlier call left there
        if ((rc = hip_status(msa::launch_attn_workspace_clear(ws, batch->batch, batch->q_len, s),
                             fn)))
            return rc;
    }
    rc = hip_status(msa::launch_insert_indexer(cache->k, cache->v, cache->ik, cache->num_pages,
                                               batch->block_table, batch->ctx_lens, batch->batch,
                                               batch->max_blocks, batch->q_len, k, v, ik, q_idx,
                                               block_scores, s),
                    fn);
    if (rc) return rc;
    return hip_status(msa::launch_select_attention(cache->k, cache->v, cache->num_pages,
                                                   batch->block_table, batch->ctx_lens,
                                                   batch->batch, batch->max_blocks, batch->q_len,
                                                   block_scores, block_ids, q, softmax_scale, out,
                                                   ws, s),
                      fn);
}

}  // extern "C"
