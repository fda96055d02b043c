// MSA block selection: per (sequence, query token, group) row keep the block of the query token
// plus the best 15 other eligible blocks.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": the 16 best blocks are
// kept and the most recent block always stays (at most 2,048 keys). "MiniMax M3 on vLLM",
// section "MSA mechanism": local_blocks = 1 and init_blocks = 0; the local block is not
// counted twice; section "Decode indexer score kernel": the top-k boundary stays close to the
// scores. Ties go to the lower block index.
//
// Rows of up to 4,096 candidate blocks: one 64-lane wavefront per row, no atomics, the
// selection of select_wave.hpp. The row's scores become order-preserving integer keys in
// registers (candidate i in lane i % 64). The 15th-largest of the 64 per-lane maxima is a lower
// bound of the 15th-largest key (at least 15 keys reach it), so the selection lies among the
// keys at or above it; it is found by ranks, not by a search: each lane counts the maxima above
// its own (all 64 read back from LDS as broadcasts), and the bound is the smallest maximum that
// fewer than 15 others exceed. Those few candidates are compacted into LDS in ascending block
// order as (key, inverted block index) composites and each is ranked exactly against the others
// by reading them back as LDS broadcasts; the 15 best, already in ascending block order, are
// written with the forced block last. When more than 64 candidates reach the bound (heavy
// ties), the wavefront extracts the 15 best one by one instead.
// Longer rows: one 256-thread workgroup per row with a 4-pass radix select (8-bit digits, LDS
// histograms) on the keys, then keys above the found key are kept and keys equal to it are taken
// in ascending block order.
#include "device_common.hpp"
#include "kernels.hpp"
#include "select_wave.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;  // keys held in registers: rows of up to 4,096 candidates


// Inclusive prefix sum over a 64-lane wavefront.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t x) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    return x;
}

struct Shared {
    uint32_t hist[256];
    uint32_t digit_prefix, need;
    uint32_t wave_tot[kThreads / 64];
    int sel[kTopk];
    int sel_count;
};

// Radix-select the key of the `need`-th largest candidate among m (REG: keys from registers).
template <bool REG>
__device__ __forceinline__ void radix_select(Shared& sh, const uint32_t (&keys)[kPerThread],
                                             const float* s, int m, int tid, int lane, int wave,
                                             uint32_t& prefix, uint32_t& need) {
    uint32_t prefix_mask = 0;
    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        sh.hist[tid] = 0;
        __syncthreads();
        if constexpr (REG) {
#pragma unroll
            for (int j = 0; j < kPerThread; j++) {
                const int i = tid + j * kThreads;
                if (i < m && (keys[j] & prefix_mask) == prefix)
                    atomicAdd(&sh.hist[(keys[j] >> shift) & 255u], 1u);
            }
        } else {
            for (int i = tid; i < m; i += kThreads) {
                const uint32_t key = order_key(s[i]);
                if ((key & prefix_mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
            }
        }
        __syncthreads();
        if (wave == 0) {
            // lane L covers digits 255-4L .. 252-4L (descending): the scan counts from the top
            uint32_t cnt[4], tot = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                cnt[i] = sh.hist[255 - 4 * lane - i];
                tot += cnt[i];
            }
            uint32_t before = wave_inclusive_scan(tot, lane) - tot;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (before < need && before + cnt[i] >= need) {
                    sh.digit_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
                    sh.need = need - before;
                }
                before += cnt[i];
            }
        }
        __syncthreads();
        prefix = sh.digit_prefix;
        need = sh.need;
        prefix_mask |= 255u << shift;
    }
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                       const int32_t* __restrict__ ctx_lens,
                                                       int max_blocks, int q_len,
                                                       int32_t* __restrict__ ids) {
    __shared__ Shared sh;
    const int row = blockIdx.x;  // ((b * q_len + j) * 4 + g)
    const int bq = row >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int32_t* out = ids + (int64_t)row * kTopk;

    const int T_raw = ctx_lens[b];
    const int T = clamp_ctx(T_raw, max_blocks);
    MSA_CHECK(tid != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    const int p = T - q_len + j;
    if (p < 0) {
        if (tid < kTopk) out[tid] = -1;
        return;
    }
    const int n = min(p / kBlock + 1, max_blocks);  // eligible blocks 0..n-1, forced n-1
    if (n <= kTopk) {
        if (tid < kTopk) out[tid] = tid < n ? tid : -1;
        return;
    }
    const float* s = scores + (int64_t)row * max_blocks;
    const int m = n - 1;  // candidates 0..m-1 compete for kTopk - 1 places
    const bool in_regs = m <= kThreads * kPerThread;
    uint32_t keys[kPerThread];
    {
        // every load goes out before any is used (one memory round trip; an index past the row
        // reads its last score and is discarded)
        float v[kPerThread] = {};
        if (in_regs) {
#pragma unroll
            for (int q = 0; q < kPerThread; q++) v[q] = s[min(tid + q * kThreads, max_blocks - 1)];
        }
#pragma unroll
        for (int q = 0; q < kPerThread; q++) {
            const int i = tid + q * kThreads;
            keys[q] = (in_regs && i < m) ? order_key(v[q]) : 0u;
        }
    }
    uint32_t prefix = 0, need = kTopk - 1;
    if (in_regs) radix_select<true>(sh, keys, s, m, tid, lane, wave, prefix, need);
    else radix_select<false>(sh, keys, s, m, tid, lane, wave, prefix, need);
    // prefix = key of the 15th largest candidate; every candidate above it is kept, and `need`
    // of the candidates equal to it (the lowest block ids).
    if (tid == 0) sh.sel_count = 0;
    uint32_t eq = 0;
    if (in_regs) {
#pragma unroll
        for (int q = 0; q < kPerThread; q++) eq += (tid + q * kThreads < m) && keys[q] == prefix;
    } else {
        for (int i = tid; i < m; i += kThreads) eq += order_key(s[i]) == prefix;
    }
    const uint32_t eq_w = wave_sum(eq);
    if (lane == 0) sh.wave_tot[wave] = eq_w;
    __syncthreads();
    const uint32_t total_eq = sh.wave_tot[0] + sh.wave_tot[1] + sh.wave_tot[2] + sh.wave_tot[3];
    if (total_eq == need) {
        // no tie straddles the boundary: keep every key >= prefix
        if (in_regs) {
#pragma unroll
            for (int q = 0; q < kPerThread; q++) {
                const int i = tid + q * kThreads;
                if (i < m && keys[q] >= prefix) {
                    const int slot = atomicAdd(&sh.sel_count, 1);
                    if (slot < kTopk - 1) sh.sel[slot] = i;
                }
            }
        } else {
            for (int i = tid; i < m; i += kThreads) {
                if (order_key(s[i]) >= prefix) {
                    const int slot = atomicAdd(&sh.sel_count, 1);
                    if (slot < kTopk - 1) sh.sel[slot] = i;
                }
            }
        }
    } else {
        // ties at the boundary: rank equal keys in ascending block order over contiguous chunks
        const int chunk = (m + kThreads - 1) / kThreads;
        const int lo = tid * chunk;
        const int hi = min(lo + chunk, m);
        uint32_t e = 0;
        for (int i = lo; i < hi; i++) e += order_key(s[i]) == prefix;
        const uint32_t incl = wave_inclusive_scan(e, lane);
        __syncthreads();
        if (lane == 63) sh.wave_tot[wave] = incl;
        __syncthreads();
        uint32_t rank = incl - e;
        for (int w = 0; w < wave; w++) rank += sh.wave_tot[w];
        for (int i = lo; i < hi; i++) {
            const uint32_t key = order_key(s[i]);
            bool take = key > prefix;
            if (key == prefix) {
                take = rank < need;
                rank++;
            }
            if (take) {
                const int slot = atomicAdd(&sh.sel_count, 1);
                if (slot < kTopk - 1) sh.sel[slot] = i;
            }
        }
    }
    __syncthreads();
    if (tid == 0) sh.sel[kTopk - 1] = m;  // the forced block of the query token
    __syncthreads();
    if (tid < kTopk) {
        const int v = sh.sel[tid];
        int pos = 0;
#pragma unroll
        for (int k = 0; k < kTopk; k++) pos += sh.sel[k] < v;
        out[pos] = v;
    }
}

// ---------------------------------------------------------------- one wavefront per row
constexpr int kRowsPerWg = 4;

template <int KPL>  // keys per lane: rows of up to 64 * KPL candidates
__global__ __launch_bounds__(kRowsPerWg * 64) void topk_wave_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_lens, int max_blocks,
    int q_len, int rows, int32_t* __restrict__ ids) {
    __shared__ uint64_t cand[kRowsPerWg][kSelectScratch];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kRowsPerWg + wave;  // ((b * q_len + j) * 4 + g)
    if (row >= rows) return;
    const int bq = row >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    // the row's scores are requested together with the context length, before anything waits
    // for either: one memory round trip
    float v[KPL];
    load_row_scores<KPL>(scores + (int64_t)row * max_blocks, max_blocks, lane, v);
    int T_raw = ctx_lens[b];
    // both loads are needed here, so the compiler issues all of them before its single wait
#pragma unroll
    for (int k = 0; k < KPL; k++) asm volatile("" : "+v"(v[k]));
    asm volatile("" : "+v"(T_raw));
    MSA_CHECK(lane != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    const int p = clamp_ctx(T_raw, max_blocks) - q_len + j;
    select_row<KPL>(v, eligible_blocks(p, max_blocks), lane, cand[wave], ids + (int64_t)row * kTopk);
}

// ---------------------------------------------------------------- window knobs
// One row per workgroup (a wavefront each): the byte histograms of select_top_radix are built
// with LDS atomic adds, which rows sharing a compute unit would queue on its one LDS.
constexpr int kWindowRowsPerWg = 1;
template <int KPL>
__global__ __launch_bounds__(kWindowRowsPerWg * 64) void topk_window_kernel(
    const float* __restrict__ scores, const int32_t* __restrict__ ctx_lens, int max_blocks,
    int q_len, int rows, int topk, int init, int local, int32_t* __restrict__ ids) {
    __shared__ uint64_t cand[kWindowRowsPerWg][kSelectScratch];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kWindowRowsPerWg + wave;
    if (row >= rows) return;
    const int bq = row >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    float v[KPL];
    load_row_scores<KPL>(scores + (int64_t)row * max_blocks, max_blocks, lane, v);
    int T_raw = ctx_lens[b];
#pragma unroll
    for (int k = 0; k < KPL; k++) asm volatile("" : "+v"(v[k]));
    asm volatile("" : "+v"(T_raw));
    MSA_CHECK(lane != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    const int p = clamp_ctx(T_raw, max_blocks) - q_len + j;
    select_row_window<KPL>(v, eligible_blocks(p, max_blocks), lane, cand[wave],
                           ids + (int64_t)row * topk, topk, init, local);
}

// ---------------------------------------------------------------- context-parallel selection
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "Indexer NVFP4 DCP": each device scores
// every index head on its own share of the pages, keeps its local top 16 per head, and the
// device that owns the head merges the lists into the final top 16, which is exact: every
// member of the global selection is among the best 16 of its own shard. Ranks travel as 32-bit
// keys (the order key of the score, the forced block as the largest key), so the merge needs
// neither scores nor context lengths.
constexpr uint32_t kForcedKey = 0xFFFFFFFFu;  // above every order key of a non-NaN score

// One shard's local lists: column c of a row holds block begin + c * stride.
template <int KPL>  // keys per lane: shards of up to 64 * KPL blocks
__global__ __launch_bounds__(kRowsPerWg * 64) void topk_local_kernel(
    const float* __restrict__ scores, int ld, int begin, int stride, int n_cols,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len, int rows,
    int32_t* __restrict__ cand_ids, uint32_t* __restrict__ cand_keys) {
    __shared__ uint64_t cand[kRowsPerWg][kSelectScratch];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kRowsPerWg + wave;  // ((b * q_len + j) * 4 + g)
    if (row >= rows) return;
    const int bq = row >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    float v[KPL];
    load_row_scores<KPL>(scores + (int64_t)row * ld, n_cols, lane, v);
    int T_raw = ctx_lens[b];
#pragma unroll
    for (int k = 0; k < KPL; k++) asm volatile("" : "+v"(v[k]));
    asm volatile("" : "+v"(T_raw));
    MSA_CHECK(lane != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    const int n = eligible_blocks(clamp_ctx(T_raw, max_blocks) - q_len + j, max_blocks);
    uint32_t key[KPL];
#pragma unroll
    for (int k = 0; k < KPL; k++) {
        const int c = lane + 64 * k;
        // (wraps harmlessly past the shard, where the key is 0 anyway)
        const int id = (int)((uint32_t)begin + (uint32_t)c * (uint32_t)stride);
        key[k] = (c < n_cols && id < n) ? (id == n - 1 ? kForcedKey : order_key(v[k])) : 0u;
    }
    // columns ascend with the block ids, so the lowest position is the lowest block
    select_top<KPL>(key, lane, cand[wave], cand_ids + (int64_t)row * kTopk,
                    cand_keys + (int64_t)row * kTopk, [=](int c) { return begin + c * stride; },
                    kTopk);
}

// The owner's merge of n_shards lists per row (shard s at [s][rows][16]): every candidate is
// ranked against all others by (key, then lower block) and the best 16 are written in
// ascending block order.
__global__ __launch_bounds__(kRowsPerWg * 64) void topk_merge_kernel(
    const int32_t* __restrict__ cand_ids, const uint32_t* __restrict__ cand_keys, int n_shards,
    int rows, int32_t* __restrict__ ids) {
    constexpr int kSlots = kMergeMaxShards * kTopk / 64;
    __shared__ uint64_t comp[kRowsPerWg][kMergeMaxShards * kTopk];
    __shared__ int32_t kept[kRowsPerWg][kTopk];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row = blockIdx.x * kRowsPerWg + wave;
    if (row >= rows) return;
    const int n_cand = n_shards * kTopk;
    // candidate c = shard c / 16, entry c % 16, as the composite (key, inverted block id): a
    // larger composite ranks first; padding (key 0) is 0 and ranks below every candidate
    uint64_t mine[kSlots];
#pragma unroll
    for (int k = 0; k < kSlots; k++) {
        const int c = lane + 64 * k;
        mine[k] = 0;
        if (c < n_cand) {
            const int64_t at = ((int64_t)(c / kTopk) * rows + row) * kTopk + c % kTopk;
            const uint32_t key = cand_keys[at];
            if (key != 0u) mine[k] = ((uint64_t)key << 32) | ~(uint32_t)cand_ids[at];
            comp[wave][c] = mine[k];
        }
    }
    if (lane < kTopk) kept[wave][lane] = -1;
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");  // the reads below follow these stores
    int rank[kSlots] = {};
    for (int t = 0; t < n_cand; t++) {
        const uint64_t o = comp[wave][t];  // an LDS broadcast
#pragma unroll
        for (int k = 0; k < kSlots; k++) rank[k] += (int)(o > mine[k]);
    }
#pragma unroll
    for (int k = 0; k < kSlots; k++)
        if (mine[k] != 0 && rank[k] < kTopk) kept[wave][rank[k]] = (int)~(uint32_t)mine[k];
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    if (lane < kTopk) {
        // ascending block order, -1 padding last (as unsigned it is the largest)
        const int v = kept[wave][lane];
        int pos = 0;
#pragma unroll
        for (int i = 0; i < kTopk; i++) {
            const int u = kept[wave][i];
            pos += (int)((uint32_t)u < (uint32_t)v || (u == v && i < lane));
        }
        ids[(int64_t)row * kTopk + pos] = v;
    }
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_topk)
#endif

hipError_t launch_topk_window(const float* scores, const int32_t* ctx_lens, int batch,
                              int max_blocks, int q_len, int topk, int init, int local,
                              int32_t* ids, hipStream_t stream) {
    const int rows = batch * q_len * kKvHeads;
    const dim3 grid((rows + kWindowRowsPerWg - 1) / kWindowRowsPerWg), block(kWindowRowsPerWg * 64);
    if (max_blocks <= 64 * 16)
        hipLaunchKernelGGL(topk_window_kernel<16>, grid, block, 0, stream, scores, ctx_lens,
                           max_blocks, q_len, rows, topk, init, local, ids);
    else
        hipLaunchKernelGGL(topk_window_kernel<64>, grid, block, 0, stream, scores, ctx_lens,
                           max_blocks, q_len, rows, topk, init, local, ids);
    return hipGetLastError();
}

hipError_t launch_topk_local(const float* scores, int ld, int begin, int stride, int n_cols,
                             const int32_t* ctx_lens, int batch, int max_blocks, int q_len,
                             int32_t* cand_ids, uint32_t* cand_keys, hipStream_t stream) {
    const int rows = batch * q_len * kKvHeads;
    const dim3 grid((rows + kRowsPerWg - 1) / kRowsPerWg), block(kRowsPerWg * 64);
    if (n_cols <= 64 * 16)
        hipLaunchKernelGGL(topk_local_kernel<16>, grid, block, 0, stream, scores, ld, begin, stride,
                           n_cols, ctx_lens, max_blocks, q_len, rows, cand_ids, cand_keys);
    else
        hipLaunchKernelGGL(topk_local_kernel<64>, grid, block, 0, stream, scores, ld, begin, stride,
                           n_cols, ctx_lens, max_blocks, q_len, rows, cand_ids, cand_keys);
    return hipGetLastError();
}

hipError_t launch_topk_merge(const int32_t* cand_ids, const uint32_t* cand_keys, int n_shards,
                             int batch, int q_len, int32_t* ids, hipStream_t stream) {
    const int rows = batch * q_len * kKvHeads;
    hipLaunchKernelGGL(topk_merge_kernel, dim3((rows + kRowsPerWg - 1) / kRowsPerWg),
                       dim3(kRowsPerWg * 64), 0, stream, cand_ids, cand_keys, n_shards, rows, ids);
    return hipGetLastError();
}

hipError_t launch_topk(const float* scores, const int32_t* ctx_lens, int batch, int max_blocks,
                       int q_len, int32_t* ids, hipStream_t stream) {
    const int rows = batch * q_len * kKvHeads;
    const dim3 wgrid((rows + kRowsPerWg - 1) / kRowsPerWg), wblock(kRowsPerWg * 64);
    if (max_blocks <= 64 * 16 + 1)
        hipLaunchKernelGGL(topk_wave_kernel<16>, wgrid, wblock, 0, stream, scores, ctx_lens,
                           max_blocks, q_len, rows, ids);
    else if (max_blocks <= 64 * 64 + 1)
        hipLaunchKernelGGL(topk_wave_kernel<64>, wgrid, wblock, 0, stream, scores, ctx_lens,
                           max_blocks, q_len, rows, ids);
    else
        hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, stream, scores, ctx_lens,
                           max_blocks, q_len, ids);
    return hipGetLastError();
}

}  // namespace msa
