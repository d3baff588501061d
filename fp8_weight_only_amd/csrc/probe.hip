// Streaming-read reference kernel: reads a buffer once with the same 128-bit
// non-temporal loads the linear kernels use and folds it into one word, so the
// bandwidth the weight-streaming kernels reach can be read against what a
// kernel that only reads achieves on the same bytes (kernel launch, DRAM
// latency and the memory system's ramp included).
#include "common.hpp"
#include "kernels.hpp"

namespace fp8w {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeLoads = 2;  // 16-byte loads in flight per thread

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t* __restrict__ p, int64_t chunks,
                                                                    uint32_t* __restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
    u32x4 v[kProbeLoads];
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u) {
        const int64_t c = base + u * stride;
        v[u] = c < chunks ? load_stream16(p + c * 16) : u32x4{0u, 0u, 0u, 0u};
    }
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < kProbeLoads; ++u)
        acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    // a data-dependent store the compiler cannot remove; it fires only for one
    // specific fold value, so the kernel writes (almost) nothing
    if (acc == 0x9e3779b9u)
        sink[0] = acc;
}

}  // namespace

hipError_t launch_read_probe(const void* p, size_t bytes, uint32_t* sink, hipStream_t stream)
{
    const int64_t chunks = (int64_t)(bytes / 16);
    if (chunks == 0)
        return hipSuccess;
    const int64_t per_block = (int64_t)kProbeThreads * kProbeLoads;
    const dim3 grid((unsigned)((chunks + per_block - 1) / per_block)), block(kProbeThreads);
    hipLaunchKernelGGL(read_probe_kernel, grid, block, 0, stream, static_cast<const uint8_t*>(p), chunks, sink);
    return hipGetLastError();
}

}  // namespace fp8w
