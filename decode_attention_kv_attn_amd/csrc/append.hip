// Cache append: write one new token row per sequence at slot pos[b], in a
// contiguous [B, s_max, row] buffer or through a paged block table
// (append-by-concatenation in the absorbed decode module of the llms.blog MLA
// page; paged placement per "What a paged KV cache block holds",
// charlestar.github.io).  A bit copy with 16-byte (or narrower) accesses.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int U>  // bytes per access
__global__ __launch_bounds__(256) void append_kernel(const AppendParams pk, const AppendParams pv)
{
    const AppendParams& p = blockIdx.y == 0 ? pk : pv;
    const int b = blockIdx.x;
    const int t = p.pos[b];
    if (t < 0) return;
    size_t row;
    if (p.bt) {
        if (t >= (p.max_blocks << p.bs_log2)) return;
        const int blk = p.bt[(size_t)b * p.max_blocks + (t >> p.bs_log2)];
        if (blk < 0 || blk >= p.num_blocks) return;
        row = ((size_t)blk << p.bs_log2) + (size_t)(t & ((1 << p.bs_log2) - 1));
    } else {
        if (t >= p.s_max) return;
        row = (size_t)b * p.s_max + t;
    }
    typedef typename std::conditional<U == 16, uint4, typename std::conditional<U == 4, uint32_t, uint16_t>::type>::type W;
    W* dst = (W*)((uint8_t*)p.cache + row * p.row_bytes);
    const W* src = (const W*)((const uint8_t*)p.src + (size_t)b * p.row_bytes);
    const long long nw = p.row_bytes / U;
    for (long long i = threadIdx.x; i < nw; i += blockDim.x) dst[i] = src[i];
}

hipError_t launch_append(const AppendParams& k, const AppendParams* v, int B, hipStream_t st)
{
    if (B == 0) return hipSuccess;
    const long long rb = k.row_bytes;
    auto aligned = [](const void* ptr, int a) { return ((uintptr_t)ptr % a) == 0; };
    bool a16 = rb % 16 == 0 && aligned(k.cache, 16) && aligned(k.src, 16);
    bool a4 = rb % 4 == 0 && aligned(k.cache, 4) && aligned(k.src, 4);
    if (v) {
        a16 = a16 && aligned(v->cache, 16) && aligned(v->src, 16);
        a4 = a4 && aligned(v->cache, 4) && aligned(v->src, 4);
    }
    const dim3 grid(B, v ? 2 : 1);
    const AppendParams& pv = v ? *v : k;
    if (a16) hipLaunchKernelGGL(append_kernel<16>, grid, dim3(256), 0, st, k, pv);
    else if (a4) hipLaunchKernelGGL(append_kernel<4>, grid, dim3(256), 0, st, k, pv);
    else hipLaunchKernelGGL(append_kernel<2>, grid, dim3(256), 0, st, k, pv);
    return hipGetLastError();
}

}  // namespace attn
