// Read-bandwidth probe: the cache-stream pattern of the decode kernels
// (LDS-DMA, non-temporal, 16 KB tiles, 5-deep ring) with nothing computed.
#include "common.h"
#include "kernels.h"
#include "mfma_lds.h"

namespace attn {

constexpr int kProbeTile = 16384;
constexpr int kProbeRing = 5;

__global__ __launch_bounds__(256) void stream_probe_kernel(const uint8_t* __restrict__ src, size_t per_wg,
                                                           unsigned* __restrict__ sink)
{
    __shared__ __attribute__((aligned(1024))) uint8_t L[kProbeRing * kProbeTile];
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)L;
    const uint8_t* base = src + (size_t)blockIdx.x * per_wg;
    const int nt = (int)(per_wg / kProbeTile);
    // wavefront w moves bytes 4 KB w .. + 4 KB of every tile, 1 KB per load
    auto issue = [&](int t) {
        const bool ok = t < nt;
        const rsrc_t r = make_rsrc(base + (size_t)(ok ? t : 0) * kProbeTile, ok ? kProbeTile : 0);
        const uint32_t lb = lds0 + (uint32_t)((t % kProbeRing) * kProbeTile);
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const uint32_t off = (uint32_t)((4 * wave + j) * 1024);
            dma16(r, off + 16u * (uint32_t)lane, lb + off);
        }
    };
#pragma unroll
    for (int t = 0; t < kProbeRing - 1; t++) issue(t);
    unsigned acc = 0;
    for (int t = 0; t < nt; t++) {
        wait_vmcnt<4 * (kProbeRing - 2)>();   // tile t has landed
        __syncthreads();
        // an LDS-space read: through a generic pointer it would be a flat
        // load, which the compiler waits for with vmcnt(0), draining the ring
        acc += *(volatile const __attribute__((address_space(3))) unsigned*)(L + (t % kProbeRing) * kProbeTile +
                                                                           threadIdx.x * 4);
        issue(t + kProbeRing - 1);            // refills the buffer read one iteration ago
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup
    if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

hipError_t launch_stream_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t st)
{
    const unsigned grid = kProbeGrid;
    hipLaunchKernelGGL(stream_probe_kernel, dim3(grid), dim3(256), 0, st, (const uint8_t*)src,
                       bytes / grid, sink);
    return hipGetLastError();
}

}  // namespace attn
