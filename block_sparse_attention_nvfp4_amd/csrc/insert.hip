// NVFP4 quantize-and-insert of K, V and index keys into their paged caches.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "TL;DR", its item on fusing the QKV
// GEMM, norm, RoPE and KV insert: K, V and the index key are quantized to NVFP4 when they are
// written to their caches.
// "MiniMax-M3.1-Flash serving notes", section "The capacity numbers": 4-bit E2M1 values and one
// E4M3 scale per 16 values.
//
// One 64-lane wavefront quantizes one 128-element vector (nvfp4_quant.hpp).
#include "device_common.hpp"
#include "kernels.hpp"
#include "nvfp4_quant.hpp"

namespace msa {
namespace {

// grid.x = tokens, block = 9 wavefronts: waves 0-3 quantize K heads 0-3, waves 4-7 V heads
// 0-3, wave 8 the index key. AT_POSITIONS: token n = b q_len + j goes to position
// T_b - q_len + j of sequence b, its slot read from the block table (the new tokens of a decode
// step); otherwise to slots[n].
template <bool AT_POSITIONS>
__global__ __launch_bounds__(576) void insert_kernel(uint8_t* __restrict__ k_pool,
                                                     uint8_t* __restrict__ v_pool,
                                                     uint8_t* __restrict__ ik_pool,
                                                     int64_t num_pages,
                                                     const int64_t* __restrict__ slots,
                                                     const int32_t* __restrict__ block_table,
                                                     const int32_t* __restrict__ ctx_lens,
                                                     int max_blocks, int q_len,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     const float* __restrict__ ik) {
    const int token = blockIdx.x;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const float* src;
    if (wave < 4) {
        if (!k) return;
        src = k + ((int64_t)token * kKvHeads + wave) * kDim;
    } else if (wave < 8) {
        if (!v) return;
        src = v + ((int64_t)token * kKvHeads + (wave - 4)) * kDim;
    } else {
        if (!ik) return;
        src = ik + (int64_t)token * kDim;
    }
    // the values and the slot (or the context length) are requested together: one memory round
    // trip before quantizing
    f32x2 x = *reinterpret_cast<const f32x2*>(src + 2 * lane);
    int64_t page;
    int t;
    if constexpr (AT_POSITIONS) {
        const int b = token / q_len;
        int t_raw = ctx_lens[b];
        asm volatile("" : "+v"(x), "+v"(t_raw));
        const int pos = clamp_ctx(t_raw, max_blocks) - q_len + (token - b * q_len);
        if (pos < 0) return;
        page = block_table[(int64_t)b * max_blocks + (pos >> 7)];
        t = pos & 127;
    } else {
        const int64_t slot = slots[token];
        asm volatile("" : "+v"(x));
        if (slot < 0) return;
        page = slot >> 7;
        t = (int)(slot & 127);
    }
    if (page < 0 || page >= num_pages) return;
    uint8_t* dst;
    bool column_layout = false;
    if (wave < 4) {
        dst = k_pool + (page * kKvHeads + wave) * kHeadPageBytes;
    } else if (wave < 8) {
        dst = v_pool + (page * kKvHeads + (wave - 4)) * kHeadPageBytes;
        column_layout = true;
    } else {
        dst = ik_pool + page * kHeadPageBytes;
    }
    quantize_store_vector(x, dst, t, column_layout, lane);
}

}  // namespace

hipError_t launch_insert(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool, int64_t num_pages,
                         const int64_t* slots, const float* k, const float* v, const float* ik,
                         int n, hipStream_t stream) {
    hipLaunchKernelGGL(insert_kernel<false>, dim3(n), dim3(576), 0, stream, k_pool, v_pool,
                       ik_pool, num_pages, slots, nullptr, nullptr, 0, 1, k, v, ik);
    return hipGetLastError();
}

hipError_t launch_insert_at_positions(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool,
                                      int64_t num_pages, const int32_t* block_table,
                                      const int32_t* ctx_lens, int batch, int max_blocks,
                                      int q_len, const float* k, const float* v, const float* ik,
                                      hipStream_t stream) {
    hipLaunchKernelGGL(insert_kernel<true>, dim3(batch * q_len), dim3(576), 0, stream, k_pool,
                       v_pool, ik_pool, num_pages, nullptr, block_table, ctx_lens, max_blocks,
                       q_len, k, v, ik);
    return hipGetLastError();
}

}  // namespace msa
