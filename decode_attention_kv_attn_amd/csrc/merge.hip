// Merge of decode outputs computed over disjoint token slices of the same
// sequences (the exchange step of context-parallel decode, where each GPU
// holds a slice of every sequence's cache).
//
// Slice k of row r holds o_k (softmax-weighted output over its own tokens)
// and lse_k = ln sum_{t in k} exp(z_t), -inf when the slice is empty.  The
// output over all tokens is o = sum_k exp(lse_k - lse) o_k with
// lse = ln sum_k exp(lse_k): the stable combination of per-block maximum,
// normaliser and output described in "MLA: why one latent can replace a
// multi-head KV cache" (charlestar.github.io), section "What FlashMLA solves
// is not the model formula itself".
//
// One wavefront per row; a lane owns 4 consecutive elements of each 256-wide
// chunk of the row, so a chunk of one slice is one coalesced 512 B (bf16) or
// 1 KB (fp32) read.  Eight slices' chunks are loaded before any is used.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

struct Vec4 {
    float v[4];
};

template <bool F32>
__device__ __forceinline__ Vec4 load4(const void* base, size_t idx)
{
    Vec4 r;
    if (F32) {
        const float4 x = *(const float4*)((const float*)base + idx);
        r.v[0] = x.x, r.v[1] = x.y, r.v[2] = x.z, r.v[3] = x.w;
    } else {
        const uint2 x = *(const uint2*)((const uint16_t*)base + idx);
        r.v[0] = bf16lo_to_f32(x.x), r.v[1] = bf16hi_to_f32(x.x);
        r.v[2] = bf16lo_to_f32(x.y), r.v[3] = bf16hi_to_f32(x.y);
    }
    return r;
}

template <bool F32>
__device__ __forceinline__ void store4(void* base, size_t idx, const float* v)
{
    if (F32) {
        *(float4*)((float*)base + idx) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        *(uint2*)((uint16_t*)base + idx) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    }
}

}  // namespace

// NC = number of 256-element chunks of a row (d <= 256 * NC, d % 4 == 0)
template <int NC, bool IN_F32, bool OUT_F32>
__global__ __launch_bounds__(256) void merge_partials_kernel(const MergeParams p)
{
    constexpr int U = 8;   // slices in flight
    const int lane = threadIdx.x % 64;
    const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    if (row >= p.rows) return;   // wave-uniform
    const int n = p.n;
    const float* __restrict__ ls = p.lse_parts + row;   // slice k at ls[k * rows]

    float M = -INFINITY;
    for (int k = lane; k < n; k += 64) M = fmaxf(M, ls[(size_t)k * p.rows]);
    M = wave_max(M);

    float acc[NC][4];
#pragma unroll
    for (int c = 0; c < NC; c++)
#pragma unroll
        for (int e = 0; e < 4; e++) acc[c][e] = 0.f;
    float L = 0.f;
    if (M != -INFINITY) {
        for (int k0 = 0; k0 < n; k0 += U) {
            Vec4 x[U][NC];
#pragma unroll
            for (int u = 0; u < U; u++) {
                const int k = min(k0 + u, n - 1);   // clamped: the loads stay unconditional
                const size_t base = ((size_t)k * p.rows + row) * p.d;
#pragma unroll
                for (int c = 0; c < NC; c++) {
                    const int col = c * 256 + lane * 4;
                    x[u][c] = Vec4{{0.f, 0.f, 0.f, 0.f}};
                    if (col < p.d) x[u][c] = load4<IN_F32>(p.o_parts, base + col);
                }
            }
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (k0 + u < n) {
                    // the slice holding the maximum gets weight 1 exactly
                    const float w = __builtin_amdgcn_exp2f((ls[(size_t)(k0 + u) * p.rows] - M) * kLog2e);
                    if (w > 0.f) {   // an empty slice (lse = -inf) is never read into the sum
                        L += w;
#pragma unroll
                        for (int c = 0; c < NC; c++)
#pragma unroll
                            for (int e = 0; e < 4; e++) acc[c][e] = fmaf(w, x[u][c].v[e], acc[c][e]);
                    }
                }
            }
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int c = 0; c < NC; c++) {
        const int col = c * 256 + lane * 4;
        if (col < p.d) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] = acc[c][e] * inv;
            store4<OUT_F32>(p.out, (size_t)row * p.d + col, v);
        }
    }
    if (lane == 0 && p.lse) p.lse[row] = L > 0.f ? M + __log2f(L) * kLn2 : -INFINITY;
}

template <int NC>
static void launch_merge_nc(const MergeParams& p, bool in_f32, bool out_f32, unsigned grid,
                            hipStream_t st)
{
    if (in_f32 && out_f32)
        hipLaunchKernelGGL((merge_partials_kernel<NC, true, true>), dim3(grid), dim3(256), 0, st, p);
    else if (in_f32)
        hipLaunchKernelGGL((merge_partials_kernel<NC, true, false>), dim3(grid), dim3(256), 0, st, p);
    else if (out_f32)
        hipLaunchKernelGGL((merge_partials_kernel<NC, false, true>), dim3(grid), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((merge_partials_kernel<NC, false, false>), dim3(grid), dim3(256), 0, st, p);
}

hipError_t launch_merge_partials(const MergeParams& p, bool in_f32, bool out_f32, hipStream_t st)
{
    const unsigned grid = (unsigned)((p.rows + 3) / 4);
    switch ((p.d + 255) / 256) {
    case 1: launch_merge_nc<1>(p, in_f32, out_f32, grid, st); break;
    case 2: launch_merge_nc<2>(p, in_f32, out_f32, grid, st); break;
    case 3: launch_merge_nc<3>(p, in_f32, out_f32, grid, st); break;
    default: launch_merge_nc<4>(p, in_f32, out_f32, grid, st); break;
    }
    return hipGetLastError();
}

}  // namespace attn
