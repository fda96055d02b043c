// MSA sparse GQA attention over the selected blocks, split over workgroups, with an
// online-softmax merge of the partial results.
//
// "vLLM day-0 support for MiniMax-M3.1-Flash", section "MSA primer" and its Figure 1: every
// query head of a GQA group attends exactly, but only to the blocks its group's indexer kept;
// section "NVFP4 MSA kernel": the kernel reads the NVFP4 pages directly and dequantizes them
// on the fly. "MiniMax M3 on vLLM", section "MiniMax sparse attention backend": the decode GQA
// kernel consumes the selected block pages and merges partial attention outputs; section
// "Prefill execution": the result equals dense attention restricted to the selected set.
//
// Per workgroup: one row group (sequence b, query token j, KV group g) = 16 query heads, and a
// share of its 16 selected blocks; 4 wavefronts, each takes whole blocks.
// Per block and wavefront (lane l, n = l % 16, c = l / 16):
//   S^T = K Q^T on bf16 matrix cores (A = keys, exact dequantized; B = the 16 heads), so lane
//   (n, c) holds the logits of head n for tokens 32c + 4s + i (slab s, i = 0..3);
//   fp32 online softmax per head (running max and sum), probabilities in fp16;
//   O^T += V^T P^T on fp16 matrix cores: P^T in the same lanes is already the B operand, V^T
//   (A operand, dims x tokens) is the exact fp16 dequantization of the column-layout V page.
// The 4 wavefronts merge through LDS; with one split the workgroup writes bf16 output,
// otherwise it writes an fp32 partial (max, sum, output) that the combine kernel merges.
#include "device_common.hpp"
#include "kernels.hpp"

namespace msa {
namespace {

constexpr int kWaves = 4;
constexpr int kPartStride = 132;  // floats per (row group, split, head): m, l, 2 pad, 128 out

__device__ __forceinline__ uint16_t bf16_bits_rne(float x) {
    const __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
}

template <int BPW>
__global__ __launch_bounds__(kWaves * 64) void attention_kernel(
    const uint8_t* __restrict__ k_pool, const uint8_t* __restrict__ v_pool, int64_t num_pages,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ ctx_lens, int max_blocks,
    int q_len, const uint16_t* __restrict__ q, const int32_t* __restrict__ block_ids,
    float scale_log2, int n_split, uint16_t* __restrict__ out, float* __restrict__ partials) {
    __shared__ float sh_o[kWaves][kGroupHeads][kDim + 4];
    __shared__ float sh_m[kWaves][kGroupHeads];
    __shared__ float sh_l[kWaves][kGroupHeads];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15;
    const int c = lane >> 4;
    const int rg = blockIdx.x / n_split;  // row group ((b * q_len + j) * 4 + g)
    const int split = blockIdx.x - rg * n_split;
    const int g = rg & 3;
    const int bq = rg >> 2;
    const int b = bq / q_len;
    const int j = bq - b * q_len;
    const int T = clamp_ctx(ctx_lens[b], max_blocks);
    const int p = T - q_len + j;

    // B operand of S^T: head 16g + n, dims 32c + 8m .. +7
    bf16x8 qop[4];
    {
        const uint16_t* qp = q + ((int64_t)bq * kQHeads + kGroupHeads * g + n) * kDim + 32 * c;
#pragma unroll
        for (int m = 0; m < 4; m++) qop[m] = *reinterpret_cast<const bf16x8*>(qp + 8 * m);
    }

    float m_run = -INFINITY, l_run = 0.f;
    f32x4 o[8];
#pragma unroll
    for (int dt = 0; dt < 8; dt++) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int32_t* my_ids = block_ids + (int64_t)rg * kTopk + (split * kWaves + wave) * BPW;
    for (int kb = 0; kb < BPW; kb++) {
        const int id = my_ids[kb];
        if (id < 0 || id >= max_blocks || id * kBlock > p) continue;
        const int page = block_table[(int64_t)b * max_blocks + id];
        if (page < 0 || page >= num_pages) continue;
        const uint8_t* kp = k_pool + ((int64_t)page * kKvHeads + g) * kHeadPageBytes;
        const uint8_t* vp = v_pool + ((int64_t)page * kKvHeads + g) * kHeadPageBytes;

        // ---- logits S^T (log2 domain)
        u32x4 kc[8];
#pragma unroll
        for (int s = 0; s < 8; s++) kc[s] = load16(kp + s * 1024 + lane * 16);
        const u32x4 ksc = load16(kp + kCodeBytes + lane * 16);
        f32x4 sv[8];
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const f32x2 s2 = (s & 1) ? e4m3_pair_f32<true>(ksc[s >> 1])
                                     : e4m3_pair_f32<false>(ksc[s >> 1]);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int m = 0; m < 4; m++)
                acc = mfma_bf16_k32(dequant8_bf16(kc[s][m], s2[m >> 1]), qop[m], acc);
            sv[s] = acc * scale_log2;
        }
        const int tok0 = id * kBlock;
        const bool full = tok0 + kBlock - 1 <= p;
        float mb = -INFINITY;
#pragma unroll
        for (int s = 0; s < 8; s++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (!full && tok0 + 32 * c + 4 * s + i > p) sv[s][i] = -INFINITY;
                mb = fmaxf(mb, sv[s][i]);
            }
        mb = max_over_c(mb);  // finite: token tok0 <= p is valid
        const float m_new = fmaxf(m_run, mb);
        const float alpha = exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 8; dt++) o[dt] *= alpha;
        float ls = 0.f;
        f16x4 pt[8];
#pragma unroll
        for (int s = 0; s < 8; s++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float e = exp2f(sv[s][i] - m_new);
                ls += e;
                pt[s][i] = (_Float16)e;
            }
        l_run += sum_over_c(ls);
        m_run = m_new;

        // ---- O^T += V^T P^T, one 16-dim tile (= one scale group) at a time
#pragma unroll
        for (int dt = 0; dt < 8; dt++) {
            const int d = 16 * dt + n;
            const u32x4 vc = load16(vp + d * 64 + 16 * c);            // tokens 32c..32c+31
            const u32x4 vs0 = load16(vp + kCodeBytes + dt * 128 + 32 * c);
            const u32x4 vs1 = load16(vp + kCodeBytes + dt * 128 + 32 * c + 16);
#pragma unroll
            for (int s = 0; s < 8; s++) {
                const uint32_t sw = s < 4 ? vs0[s] : vs1[s - 4];       // tokens 32c+4s..+3
                const f16x4 a = (s & 1) ? dequant4_f16_percode<2>(vc[s >> 1], sw)
                                        : dequant4_f16_percode<0>(vc[s >> 1], sw);
                o[dt] = mfma_f16_k16(a, pt[s], o[dt]);
            }
        }
    }

    // ---- merge the 4 wavefronts: lane (n, c) holds o[dt][i] = out(head n, dim 16dt + 4c + i)
#pragma unroll
    for (int dt = 0; dt < 8; dt++)
#pragma unroll
        for (int i = 0; i < 4; i++) sh_o[wave][n][16 * dt + 4 * c + i] = o[dt][i];
    if (c == 0) {
        sh_m[wave][n] = m_run;
        sh_l[wave][n] = l_run;
    }
    __syncthreads();
    const int h = threadIdx.x >> 4;         // head 0..15
    const int d0 = (threadIdx.x & 15) * 8;  // 8 dims
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, sh_m[w][h]);
    float wt[kWaves], L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        wt[w] = (sh_m[w][h] == -INFINITY) ? 0.f : exp2f(sh_m[w][h] - M);
        L += wt[w] * sh_l[w][h];
    }
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; w++) x += wt[w] * sh_o[w][h][d0 + e];
        acc[e] = x;
    }
    if (n_split == 1) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
        uint16_t* op = out + ((int64_t)bq * kQHeads + kGroupHeads * g + h) * kDim + d0;
        uint32_t packed[4];
#pragma unroll
        for (int e = 0; e < 4; e++)
            packed[e] = (uint32_t)bf16_bits_rne(acc[2 * e] * inv) |
                        ((uint32_t)bf16_bits_rne(acc[2 * e + 1] * inv) << 16);
        *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    } else {
        float* pp = partials + (((int64_t)rg * n_split + split) * kGroupHeads + h) * kPartStride;
        if (d0 == 0) {
            pp[0] = M;
            pp[1] = L;
        }
        *reinterpret_cast<f32x4*>(pp + 4 + d0) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        *reinterpret_cast<f32x4*>(pp + 8 + d0) = f32x4{acc[4], acc[5], acc[6], acc[7]};
    }
}

// One workgroup per row group: merge its n_split partials per head into bf16 output.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partials,
                                                     int n_split, uint16_t* __restrict__ out) {
    const int rg = blockIdx.x;
    const int g = rg & 3;
    const int bq = rg >> 2;
    const int h = threadIdx.x >> 4;
    const int d0 = (threadIdx.x & 15) * 8;
    const float* base = partials + ((int64_t)rg * n_split * kGroupHeads + h) * kPartStride;
    const int stride = kGroupHeads * kPartStride;
    float M = -INFINITY;
    for (int sp = 0; sp < n_split; sp++) M = fmaxf(M, base[sp * stride]);
    float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int sp = 0; sp < n_split; sp++) {
        const float* pp = base + sp * stride;
        const float w = (pp[0] == -INFINITY) ? 0.f : exp2f(pp[0] - M);
        L += w * pp[1];
        const f32x4 a = *reinterpret_cast<const f32x4*>(pp + 4 + d0);
        const f32x4 bb = *reinterpret_cast<const f32x4*>(pp + 8 + d0);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            acc[e] += w * a[e];
            acc[4 + e] += w * bb[e];
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint32_t packed[4];
#pragma unroll
    for (int e = 0; e < 4; e++)
        packed[e] = (uint32_t)bf16_bits_rne(acc[2 * e] * inv) |
                    ((uint32_t)bf16_bits_rne(acc[2 * e + 1] * inv) << 16);
    uint16_t* op = out + ((int64_t)bq * kQHeads + kGroupHeads * g + h) * kDim + d0;
    *reinterpret_cast<u32x4*>(op) = u32x4{packed[0], packed[1], packed[2], packed[3]};
}

}  // namespace

int attn_num_splits(int batch, int q_len) {
    const long rows = (long)batch * q_len * kKvHeads;
    // enough workgroups to cover the 256 compute units, at most 4 splits (1 block per wave)
    if (rows >= 1024) return 1;
    if (rows >= 512) return 2;
    return 4;
}

size_t attn_workspace_bytes(int batch, int q_len) {
    const int ns = attn_num_splits(batch, q_len);
    if (ns == 1) return 0;
    return (size_t)batch * q_len * kKvHeads * ns * kGroupHeads * kPartStride * sizeof(float);
}

hipError_t launch_attention(const uint8_t* k_pool, const uint8_t* v_pool, int64_t num_pages,
                            const int32_t* block_table, const int32_t* ctx_lens, int batch,
                            int max_blocks, int q_len, const uint16_t* q, const int32_t* ids,
                            float softmax_scale, uint16_t* out, float* workspace,
                            hipStream_t stream) {
    const int ns = attn_num_splits(batch, q_len);
    const int rows = batch * q_len * kKvHeads;
    const float scale_log2 = softmax_scale * 1.4426950408889634f;
    const dim3 grid(rows * ns), block(kWaves * 64);
    switch (ns) {
        case 1:
            hipLaunchKernelGGL(attention_kernel<4>, grid, block, 0, stream, k_pool, v_pool,
                               num_pages, block_table, ctx_lens, max_blocks, q_len, q, ids,
                               scale_log2, ns, out, workspace);
            break;
        case 2:
            hipLaunchKernelGGL(attention_kernel<2>, grid, block, 0, stream, k_pool, v_pool,
                               num_pages, block_table, ctx_lens, max_blocks, q_len, q, ids,
                               scale_log2, ns, out, workspace);
            break;
        default:
            hipLaunchKernelGGL(attention_kernel<1>, grid, block, 0, stream, k_pool, v_pool,
                               num_pages, block_table, ctx_lens, max_blocks, q_len, q, ids,
                               scale_log2, ns, out, workspace);
            break;
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || ns == 1) return err;
    hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(256), 0, stream, workspace, ns, out);
    return hipGetLastError();
}

}  // namespace msa
