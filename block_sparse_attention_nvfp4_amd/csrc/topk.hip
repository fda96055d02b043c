// MSA block selection: per (sequence, query token, group) row keep the block of the query token
// plus the best 15 other eligible blocks.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer": the 16 best blocks are
// kept and the most recent block always stays (at most 2,048 keys). "MiniMax M3 on vLLM",
// section "MSA mechanism": local_blocks = 1 and init_blocks = 0; the local block is not
// counted twice; section "Decode indexer score kernel": the top-k boundary stays close to the
// scores. Ties go to the lower block index.
//
// One 256-thread workgroup per row. The 15th-largest score key is found by a 4-pass radix
// select (8-bit digits, most significant first) over order-preserving integer keys; all keys
// above it are kept and the keys equal to it are taken in ascending block order until 15.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kThreads = 256;

// Order-preserving map of a non-NaN float to uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over a 64-lane wavefront.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores,
                                                       const int32_t* __restrict__ ctx_lens,
                                                       int max_blocks, int q_len,
                                                       int32_t* __restrict__ ids) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t sh_digit_prefix, sh_need;
    __shared__ uint32_t wave_tot[kThreads / 64];
    __shared__ int sel[kTopk];
    __shared__ int sel_count;

    const int row = blockIdx.x;  // ((b * q_len + j) * 4 + g)
    const int bq = row >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    int32_t* out = ids + (int64_t)row * kTopk;

    const int T = clamp_ctx(ctx_lens[b], max_blocks);
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
    uint32_t prefix = 0, prefix_mask = 0, need = kTopk - 1;

    for (int pass = 0; pass < 4; pass++) {
        const int shift = 24 - 8 * pass;
        hist[tid] = 0;
        __syncthreads();
        for (int i = tid; i < m; i += kThreads) {
            const uint32_t key = order_key(s[i]);
            if ((key & prefix_mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (wave == 0) {
            // lane L covers digits 255-4L .. 252-4L (descending), so the scan counts keys from the top
            uint32_t cnt[4], tot = 0;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                cnt[i] = hist[255 - 4 * lane - i];
                tot += cnt[i];
            }
            uint32_t before = wave_inclusive_scan(tot, lane) - tot;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (before < need && before + cnt[i] >= need) {
                    sh_digit_prefix = prefix | ((uint32_t)(255 - 4 * lane - i) << shift);
                    sh_need = need - before;
                }
                before += cnt[i];
            }
        }
        __syncthreads();
        prefix = sh_digit_prefix;
        need = sh_need;
        prefix_mask |= 255u << shift;
    }
    // prefix = key of the 15th largest candidate; `need` of the candidates equal to it are kept
    // (the lowest block ids), every candidate above it is kept.
    if (tid == 0) sel_count = 0;
    const int chunk = (m + kThreads - 1) / kThreads;
    const int lo = tid * chunk;
    const int hi = min(lo + chunk, m);
    uint32_t eq = 0;
    for (int i = lo; i < hi; i++) eq += (order_key(s[i]) == prefix);
    const uint32_t incl = wave_inclusive_scan(eq, lane);
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t rank = incl - eq;
    for (int w = 0; w < wave; w++) rank += wave_tot[w];
    for (int i = lo; i < hi; i++) {
        const uint32_t key = order_key(s[i]);
        bool take = key > prefix;
        if (key == prefix) {
            take = rank < need;
            rank++;
        }
        if (take) {
            const int slot = atomicAdd(&sel_count, 1);
            if (slot < kTopk - 1) sel[slot] = i;
        }
    }
    __syncthreads();
    if (tid == 0) sel[kTopk - 1] = m;  // the forced block of the query token
    __syncthreads();
    if (tid < kTopk) {
        const int v = sel[tid];
        int pos = 0;
#pragma unroll
        for (int k = 0; k < kTopk; k++) pos += sel[k] < v;
        out[pos] = v;
    }
}

}  // namespace

hipError_t launch_topk(const float* scores, const int32_t* ctx_lens, int batch, int max_blocks,
                       int q_len, int32_t* ids, hipStream_t stream) {
    const int rows = batch * q_len * kKvHeads;
    hipLaunchKernelGGL(topk_kernel, dim3(rows), dim3(kThreads), 0, stream, scores, ctx_lens,
                       max_blocks, q_len, ids);
    return hipGetLastError();
}

}  // namespace msa
