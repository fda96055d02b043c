// Streaming-read probe (declared in include/msa_probe.h): the rate at which a plain kernel reads
// a working set from HBM on this GPU, to set the HBM-bound kernels' measured rates against.
// Each of 1,024 workgroups (four per compute unit) of 256 threads streams one contiguous share of
// the buffer, four 16-byte loads per thread in flight per iteration. Contiguous shares measured
// faster than a grid-stride loop over the whole buffer (about 6.3 vs 5.6 TB/s for 76 MB, 7.1 vs
// 6.2 TB/s for 2 GiB), and more workgroups or more loads in flight measured no faster.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/msa_probe.h"

namespace {

constexpr int kProbeWgs = 1024;
constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ p,
                                                                    size_t n,
                                                                    uint32_t* __restrict__ sink) {
    const size_t share = (n + gridDim.x - 1) / gridDim.x;
    const size_t lo = (size_t)blockIdx.x * share;
    const size_t hi = lo + share < n ? lo + share : n;
    u32x4 acc = {0u, 0u, 0u, 0u};
    size_t i = lo + threadIdx.x;
    for (; i + (kProbeUnroll - 1) * kProbeThreads < hi; i += kProbeUnroll * kProbeThreads) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) v[u] = __builtin_nontemporal_load(p + i + u * kProbeThreads);
#pragma unroll
        for (int u = 0; u < kProbeUnroll; u++) acc ^= v[u];
    }
    for (; i < hi; i += kProbeThreads) acc ^= __builtin_nontemporal_load(p + i);
    uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    for (int d = 32; d >= 1; d >>= 1) x ^= __shfl_xor(x, d, 64);
    __shared__ uint32_t part[kProbeThreads / 64];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" {

size_t msa_probe_sink_words(void) { return kProbeWgs; }

int msa_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || (bytes & 15u) || ((uintptr_t)buf & 15u)) return -1;
    if (bytes == 0) return 0;
    hipLaunchKernelGGL(stream_read_kernel, dim3(kProbeWgs), dim3(kProbeThreads), 0,
                       (hipStream_t)stream, static_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
