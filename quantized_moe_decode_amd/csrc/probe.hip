// Streaming-read probe: reads a buffer once with 16-byte non-temporal loads
// and reduces it to one partial sum per workgroup.  It is the measurement aid
// behind the "practical HBM read ceiling" that the decode kernels are compared
// with (meTile PR #30, the GB/s table and its reading: decode GEMVs are judged
// against what plain streaming achieves on the same machine).
#include <hip/hip_runtime.h>

#include "api.hpp"
#include "common.hpp"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;                                       // loads in flight per thread
constexpr size_t kProbeChunk = (size_t)kProbeThreads * kProbeUnroll * 16;  // bytes per block step
constexpr int kProbeMaxBlocks = 4096;

static int probe_blocks(size_t bytes) {
    const size_t steps = (bytes + kProbeChunk - 1) / kProbeChunk;
    return (int)(steps < (size_t)kProbeMaxBlocks ? steps : (size_t)kProbeMaxBlocks);
}

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const f32x4 *p, size_t n16, float *out) {
    float acc = 0.f;
    const size_t stride = (size_t)gridDim.x * kProbeThreads * kProbeUnroll;
    for (size_t base = (size_t)blockIdx.x * kProbeThreads * kProbeUnroll + threadIdx.x; base < n16;
         base += stride) {
        f32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) {
            const size_t i = base + (size_t)u * kProbeThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc += (v[u].x + v[u].y) + (v[u].z + v[u].w);
    }
    __shared__ float s[kProbeThreads];
    s[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kProbeThreads / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) s[threadIdx.x] += s[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) out[blockIdx.x] = s[0];
}

}  // namespace moe

using namespace moe;

extern "C" int32_t moe_decode_read_probe_blocks(size_t bytes) { return bytes ? probe_blocks(bytes) : 0; }

extern "C" moe_status moe_decode_read_probe(const void *data, size_t bytes, float *partial_sums,
                                            int32_t n_partial, void *stream) {
    if (!data || !partial_sums || bytes == 0 || bytes % 16) return MOE_EINVAL;
    if (!aligned16(data)) return MOE_EINVAL;
    const int blocks = probe_blocks(bytes);
    if (n_partial < blocks) return MOE_EINVAL;
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(kProbeThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const f32x4 *>(data),
                       bytes / 16, partial_sums);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP;
}
