// Cache append: write one new token row per sequence at slot pos[b], in a
// contiguous [B, s_max, row] buffer or through a paged block table
// (append-by-concatenation in the absorbed decode module of the llms.blog MLA
// page; paged placement per "What a paged KV cache block holds",
// charlestar.github.io).  A bit copy with 16-byte (or narrower) accesses, or,
// for FP8 caches, a conversion of bf16 rows to E4M3 codes.
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

// OCP E4M3 code of an fp32 value: nearest, ties to even, saturating at
// +-448; NaN gives 0x7F; the sign of zero is kept.  Worked from the fp32
// fields: below 2^-6 the code counts quanta of 2^-9, above it the exponent
// is the fp32 one and the mantissa is |y| / 2^(e - 3) rounded (both scalings
// by powers of two are exact, so rintf takes the one rounding).
__device__ __forceinline__ uint32_t e4m3_code(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return 0x7fu;               // NaN
    if (a >= 0x43e00000u) return sign | 0x7eu;       // |y| >= 448, or infinite
    const float ay = __uint_as_float(a);
    if (a < 0x3c800000u)                              // |y| < 2^-6
        return sign | (uint32_t)__builtin_rintf(ay * 512.0f);   // 0 .. 8 (8 is 2^-6)
    int e = (int)(a >> 23) - 127;                    // -6 .. 8
    int m = (int)__builtin_rintf(__builtin_ldexpf(ay, 3 - e));   // 8 .. 16
    if (m == 16) {
        m = 8;
        e++;
    }
    const uint32_t code = (uint32_t)(((e + 7) << 3) | (m - 8));
    return sign | (code > 0x7eu ? 0x7eu : code);
}

// One workgroup per (sequence, K or V); a thread converts 4 bf16 values to 4
// codes (8 bytes in, one 32-bit word out).
__global__ __launch_bounds__(256) void append_fp8_kernel(const AppendParams pk, const AppendParams pv)
{
    const AppendParams& p = blockIdx.y == 0 ? pk : pv;
    const int b = blockIdx.x;
    const int t = p.pos[b];
    if (t < 0) return;
    size_t row;
    int blk = 0;
    if (p.bt) {
        if (t >= (p.max_blocks << p.bs_log2)) return;
        blk = p.bt[(size_t)b * p.max_blocks + (t >> p.bs_log2)];
        if (blk < 0 || blk >= p.num_blocks) return;
        row = ((size_t)blk << p.bs_log2) + (size_t)(t & ((1 << p.bs_log2) - 1));
    } else {
        if (t >= p.s_max) return;
        row = (size_t)b * p.s_max + t;
    }
    const long long n4 = p.row_bytes / 4;
    uint32_t* dst = (uint32_t*)((uint8_t*)p.cache + row * p.row_bytes);
    const uint2* src = (const uint2*)((const uint16_t*)p.src + (size_t)b * p.row_bytes);
    for (long long i = threadIdx.x; i < n4; i += blockDim.x) {
        const uint2 w = src[i];
        float is = 4 * i < p.split ? p.inv_scale : p.inv_scale2;   // MLA: latent, then rotary part
        if (p.page_scales2)   // MLA latent row: this page's latent, then rotary scale
            is = 1.0f / (4 * i < p.split ? p.page_scales[blk] : p.page_scales2[blk]);
        else if (p.page_scales)   // this page's scale for the KV head of these 4 elements
            is = 1.0f / p.page_scales[(size_t)blk * (p.row_bytes / p.d_h) + (4 * i) / p.d_h];
        const uint32_t c0 = e4m3_code(bf16lo_to_f32(w.x) * is);
        const uint32_t c1 = e4m3_code(bf16hi_to_f32(w.x) * is);
        const uint32_t c2 = e4m3_code(bf16lo_to_f32(w.y) * is);
        const uint32_t c3 = e4m3_code(bf16hi_to_f32(w.y) * is);
        dst[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
    }
}

hipError_t launch_append_fp8(const AppendParams& k, const AppendParams* v, int B, hipStream_t st)
{
    if (B == 0) return hipSuccess;
    const dim3 grid(B, v ? 2 : 1);
    hipLaunchKernelGGL(append_fp8_kernel, grid, dim3(256), 0, st, k, v ? *v : k);
    return hipGetLastError();
}

}  // namespace attn
