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
        MSA_CHECK(threadIdx.x != 0 || (t_raw >= q_len && t_raw <= max_blocks * kBlock), kCheckCtxLen);
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

// Inserts of several new tokens per sequence at positions T - q_len .. T - 1 (prefill chunks,
// long drafts): one workgroup per run of 8 aligned positions of one sequence, the tokens that
// share every 32-bit word of the V pages' column layout (element e's word holds the nibbles of
// tokens 8k .. 8k + 7). The wavefronts take the head vectors as in insert_kernel, each for every
// new token of its run; a V word is written with a plain store when all 8 of its tokens are new,
// and with one atomic and/or pair otherwise (the two ends of the new range), instead of an
// atomic pair per nibble and token.
constexpr int kRun = 8;
constexpr int kSlotsRunMinTokens = 256;  // inserts from this size on take insert_slots_kernel

__global__ __launch_bounds__(576) void insert_run_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, uint8_t* __restrict__ ik_pool,
    int64_t num_pages, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ ctx_lens, int max_blocks, int q_len, int runs_per_seq,
    const float* __restrict__ k, const float* __restrict__ v, const float* __restrict__ ik) {
    const int b = blockIdx.x / runs_per_seq;
    const int r = blockIdx.x - b * runs_per_seq;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const float* base;
    int stride;  // floats from one token's vector of this head to the next token's
    if (wave < 4) {
        if (!k) return;
        base = k + wave * kDim;
        stride = kKvHeads * kDim;
    } else if (wave < 8) {
        if (!v) return;
        base = v + (wave - 4) * kDim;
        stride = kKvHeads * kDim;
    } else {
        if (!ik) return;
        base = ik;
        stride = kDim;
    }
    const int T_raw = ctx_lens[b];
    const int T = clamp_ctx(T_raw, max_blocks);
    MSA_CHECK(threadIdx.x != 0 || (T_raw >= q_len && T_raw <= max_blocks * kBlock), kCheckCtxLen);
    const int p_first = T - q_len;                 // position of new token 0 (may be < 0)
    const int pos0 = ((p_first >> 3) + r) * kRun;  // this run's first position (floor of p / 8)
    const int lo = max(pos0, max(p_first, 0));
    const int hi = min(pos0 + kRun, T);
    if (lo >= hi) return;  // (then pos0 >= 0: a multiple of 8 above -8)
    const int64_t page = block_table[(int64_t)b * max_blocks + (pos0 >> 7)];
    if (page < 0 || page >= num_pages) return;
    const int nt = hi - lo;
    // every token's values requested before any is quantized
    f32x2 x[kRun];
#pragma unroll
    for (int i = 0; i < kRun; i++) {
        const int j = min(lo + i, hi - 1) - p_first;  // new-token index (past nt: a repeat)
        x[i] = *reinterpret_cast<const f32x2*>(base + ((int64_t)b * q_len + j) * stride + 2 * lane);
    }
    uint8_t* dst;
    if (wave < 4) dst = k_pool + (page * kKvHeads + wave) * kHeadPageBytes;
    else if (wave < 8) dst = v_pool + (page * kKvHeads + (wave - 4)) * kHeadPageBytes;
    else dst = ik_pool + page * kHeadPageBytes;
    if (wave < 4 || wave == 8) {
        for (int i = 0; i < nt; i++) quantize_store_vector(x[i], dst, (lo + i) & 127, false, lane);
        return;
    }
    // V: the lane's elements e = 2 lane and e + 1, nibble 4 (p % 8) of their words
    uint32_t w0 = 0, w1 = 0, mask = 0;
    for (int i = 0; i < nt; i++) {
        uint32_t byte, scale;
        quantize_pair(x[i][0], x[i][1], byte, scale);
        const int t = (lo + i) & 127;
        const int sh = 4 * (t & 7);
        w0 |= (byte & 15u) << sh;
        w1 |= (byte >> 4) << sh;
        mask |= 15u << sh;
        if ((lane & 7) == 0) dst[col_scale_offset(t, lane >> 3)] = (uint8_t)scale;
    }
    uint32_t* p0 = reinterpret_cast<uint32_t*>(dst + col_code_byte(2 * lane, pos0 & 127));
    uint32_t* p1 = reinterpret_cast<uint32_t*>(dst + col_code_byte(2 * lane + 1, pos0 & 127));
    if (nt == kRun) {
        *p0 = w0;
        *p1 = w1;
    } else {
        atomicAnd(p0, ~mask);
        atomicOr(p0, w0);
        atomicAnd(p1, ~mask);
        atomicOr(p1, w1);
    }
}

// Inserts at given slots, eight input tokens per workgroup. When the eight slots are one aligned
// run of a page (slot[8r + i] = slot[8r] + i, slot[8r] a multiple of 8) they own whole V words
// (slots are distinct within a call), which are then written with plain stores as in
// insert_run_kernel; otherwise each token is inserted as insert_kernel does (an atomic pair per
// V nibble). Prompt prefill hands over consecutive slots, so nearly every group is a run.
__global__ __launch_bounds__(576) void insert_slots_kernel(
    uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool, uint8_t* __restrict__ ik_pool,
    int64_t num_pages, const int64_t* __restrict__ slots, int n, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ ik) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const float* base;
    int stride;
    if (wave < 4) {
        if (!k) return;
        base = k + wave * kDim;
        stride = kKvHeads * kDim;
    } else if (wave < 8) {
        if (!v) return;
        base = v + (wave - 4) * kDim;
        stride = kKvHeads * kDim;
    } else {
        if (!ik) return;
        base = ik;
        stride = kDim;
    }
    const int t0 = blockIdx.x * kRun;
    const int nt = min(kRun, n - t0);
    // every token's slot and values requested before any is used
    int64_t sl[kRun];
    f32x2 x[kRun];
#pragma unroll
    for (int i = 0; i < kRun; i++) {
        const int t = t0 + min(i, nt - 1);
        sl[i] = slots[t];
        x[i] = *reinterpret_cast<const f32x2*>(base + (int64_t)t * stride + 2 * lane);
    }
    const int64_t page0 = sl[0] >> 7;
    bool run = nt == kRun && sl[0] >= 0 && (sl[0] & 7) == 0 && page0 < num_pages;
#pragma unroll
    for (int i = 1; i < kRun; i++) run = run && sl[i] == sl[0] + i;
    uint8_t* pool = wave < 4 ? k_pool : (wave < 8 ? v_pool : ik_pool);
    const int64_t head_stride = wave < 8 ? (int64_t)kKvHeads * kHeadPageBytes : kHeadPageBytes;
    const int head = wave < 8 ? (wave & 3) : 0;
    if (!run || wave < 4 || wave == 8) {
        // token by token (V with the per-nibble atomics)
        for (int i = 0; i < nt; i++) {
            const int64_t slot = sl[i];
            if (slot < 0 || (slot >> 7) >= num_pages) continue;
            uint8_t* dst = pool + (slot >> 7) * head_stride + (int64_t)head * kHeadPageBytes;
            quantize_store_vector(x[i], dst, (int)(slot & 127), wave >= 4 && wave < 8, lane);
        }
        return;
    }
    // V of a whole aligned run: the lane's elements e = 2 lane, e + 1, nibble i of their words
    uint8_t* dst = pool + page0 * head_stride + (int64_t)head * kHeadPageBytes;
    const int tb = (int)(sl[0] & 127);
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int i = 0; i < kRun; i++) {
        uint32_t byte, scale;
        quantize_pair(x[i][0], x[i][1], byte, scale);
        w0 |= (byte & 15u) << (4 * i);
        w1 |= (byte >> 4) << (4 * i);
        if ((lane & 7) == 0) dst[col_scale_offset(tb + i, lane >> 3)] = (uint8_t)scale;
    }
    *reinterpret_cast<uint32_t*>(dst + col_code_byte(2 * lane, tb)) = w0;
    *reinterpret_cast<uint32_t*>(dst + col_code_byte(2 * lane + 1, tb)) = w1;
}

}  // namespace

#ifdef MSA_CHECKED
MSA_DEFINE_CHECKS_READER(checks_take_insert)
#endif

hipError_t launch_insert(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool, int64_t num_pages,
                         const int64_t* slots, const float* k, const float* v, const float* ik,
                         int n, hipStream_t stream) {
    if (n >= kSlotsRunMinTokens) {
        hipLaunchKernelGGL(insert_slots_kernel, dim3((n + kRun - 1) / kRun), dim3(576), 0, stream,
                           k_pool, v_pool, ik_pool, num_pages, slots, n, k, v, ik);
        return hipGetLastError();
    }
    // a decode step's few tokens: one workgroup each, all in parallel (a group of eight that is
    // no run would take its tokens one after another)
    hipLaunchKernelGGL(insert_kernel<false>, dim3(n), dim3(576), 0, stream, k_pool, v_pool,
                       ik_pool, num_pages, slots, nullptr, nullptr, 0, 1, k, v, ik);
    return hipGetLastError();
}

hipError_t launch_insert_at_positions(uint8_t* k_pool, uint8_t* v_pool, uint8_t* ik_pool,
                                      int64_t num_pages, const int32_t* block_table,
                                      const int32_t* ctx_lens, int batch, int max_blocks,
                                      int q_len, const float* k, const float* v, const float* ik,
                                      hipStream_t stream) {
    if (q_len >= 2) {
        // a range of q_len positions meets at most q_len / 8 + 2 aligned runs of 8
        const int runs = q_len / kRun + 2;
        hipLaunchKernelGGL(insert_run_kernel, dim3(batch * runs), dim3(576), 0, stream, k_pool,
                           v_pool, ik_pool, num_pages, block_table, ctx_lens, max_blocks, q_len,
                           runs, k, v, ik);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(insert_kernel<true>, dim3(batch * q_len), dim3(576), 0, stream, k_pool,
                       v_pool, ik_pool, num_pages, nullptr, block_table, ctx_lens, max_blocks,
                       q_len, k, v, ik);
    return hipGetLastError();
}

}  // namespace msa
