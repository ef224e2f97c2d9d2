// MLA output path: the attention block's output projection and the merged
// weights it can be regrouped into ("Multi-Head Latent Attention (MLA):
// Mathematical Foundations" (llms.blog), section "Value Output Matrix
// Absorption": o_t = sum_i W_O^i u_{t,i} = sum_i (W_O^i W_UV,i) u~_{t,i}).
//
//   proj_gemm_kernel   Y[M, N] = X[M, K] W[N, K]^T, bf16 operands, fp32
//                      accumulation.  Deferred form: X = the heads' outputs
//                      [rows, h d_v], W = W_O.  Merged form: X = the latent
//                      sums u~ [rows, h d_c], W = W_O^i W_UV,i side by side.
//   proj_reduce_kernel sums the K-split partials in a fixed order.
//   premerge_kernel    W_abs[n, i d_c + c] = sum_e W_O[n, i d_v + e] W_UV[i, e, c]
//                      (built once, offline).
//
// At decode M (sequences x new tokens) is small and the kernel is a stream
// over W: HBM-bound.  Each wavefront takes 32 output columns (rows of W) and
// a contiguous K range, on v_mfma_f32_32x32x16_bf16 with X as the A operand
// and W as the B operand.  K is taken in steps of 128: lane l (column
// l % 32, half h = l / 32) loads the 128 contiguous bytes of W's row at
// k0 + 64 h .. k0 + 64 h + 63 and X's rows at the same k, and MFMA j of the
// step uses their j-th 8 elements.  The products are summed over all k in
// any case, so this assignment of k to lanes (not the operand's native one)
// changes no result and gives each lane whole 16-byte pieces of one line.
#include "kernels.h"
#include "mfma_lds.h"

namespace attn {

constexpr int kProjStep = 128;   // K elements per step of a wavefront
constexpr int kProjWaves = 4;

__device__ __forceinline__ f32x16 mfma32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Workgroup = (32-column block nb, K split ks, 32 MT-row block mb); its four
// wavefronts split the split's steps into contiguous runs and their sums
// meet in LDS.
template <int MT>
__global__ __launch_bounds__(64 * kProjWaves) void proj_gemm_kernel(const ProjParams p)
{
    __shared__ __attribute__((aligned(16))) float red[kProjWaves][MT * 16][64];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int nblk = p.N / 32;
    // consecutive work items (same K split) stay on one XCD, whose L2 then
    // holds that split's slice of X
    const int w = xcd_major(blockIdx.x, gridDim.x);
    const int nb = w % nblk, ks = (w / nblk) % p.ks, mb = w / (nblk * p.ks);
    const int steps = p.K / kProjStep;
    // steps of split ks, then of this wavefront (contiguous, as even as possible)
    const int s_lo = (int)((long long)steps * ks / p.ks), s_hi = (int)((long long)steps * (ks + 1) / p.ks);
    const int n = s_hi - s_lo;
    const int w_lo = s_lo + n * wave / kProjWaves, w_hi = s_lo + n * (wave + 1) / kProjWaves;

    const int col = lane % 32, hh = lane / 32;
    const int n0 = nb * 32, m0 = mb * 32 * MT;
    // X rows past M start at the buffer's end and read as zeros (the host
    // keeps M K 2 + 2 K below 2^31, so no offset wraps)
    const uint32_t xend = (uint32_t)p.M * (uint32_t)p.K * 2u;
    const rsrc_t xr = make_rsrc(p.x, (int)xend);
    const rsrc_t wr = make_rsrc(p.w + (size_t)n0 * p.K, 32 * p.K * 2);
    const uint32_t woff = (uint32_t)(col * p.K + 64 * hh) * 2;
    uint32_t xoff[MT];
#pragma unroll
    for (int t = 0; t < MT; t++) {
        const int m = m0 + 32 * t + col;
        xoff[t] = m < p.M ? (uint32_t)(m * p.K + 64 * hh) * 2 : xend;
    }

    f32x16 acc[MT];
#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[t][r] = 0.f;

    uint4 wb[2][8], xb[2][MT][8];
    auto load = [&](int buf, int s) {
        const uint32_t kb = (uint32_t)s * kProjStep * 2;
#pragma unroll
        for (int j = 0; j < 8; j++) wb[buf][j] = buf_load16(wr, woff + kb + 16 * j);
#pragma unroll
        for (int t = 0; t < MT; t++)
#pragma unroll
            for (int j = 0; j < 8; j++) xb[buf][t][j] = buf_load16(xr, xoff[t] + kb + 16 * j);
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 8; j++)
#pragma unroll
            for (int t = 0; t < MT; t++)
                acc[t] = mfma32x16(__builtin_bit_cast(bf16x8, xb[buf][t][j]),
                                   __builtin_bit_cast(bf16x8, wb[buf][j]), acc[t]);
    };
    if (w_lo < w_hi) {
        load(0, w_lo);
        int s = w_lo;
        for (; s + 1 < w_hi; s += 2) {
            load(1, s + 1);
            compute(0);
            if (s + 2 < w_hi) load(0, s + 2);
            compute(1);
        }
        if (s < w_hi) compute(0);
    }

#pragma unroll
    for (int t = 0; t < MT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) red[wave][t * 16 + r][lane] = acc[t][r];
    __syncthreads();
    // thread (lane, q): accumulator registers r = q, q + 4, q + 8, q + 12 of
    // every m tile; register r of lane l is row 8 (r / 4) + 4 (l / 32) + r % 4,
    // column l % 32 of the tile
    const int q = wave;
#pragma unroll
    for (int t = 0; t < MT; t++) {
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
            const int r = q + 4 * rr;
            const float v = (red[0][t * 16 + r][lane] + red[1][t * 16 + r][lane]) +
                            (red[2][t * 16 + r][lane] + red[3][t * 16 + r][lane]);
            const int m = m0 + 32 * t + 8 * (r / 4) + 4 * hh + r % 4;
            if (m < p.M) {
                const size_t o = (size_t)m * p.N + n0 + col;
                if (p.ks > 1) p.part[(size_t)ks * p.M * p.N + o] = v;
                else if (p.y_f32) ((float*)p.y)[o] = v;
                else ((uint16_t*)p.y)[o] = (uint16_t)f32_to_bf16_bits(v);
            }
        }
    }
}

// Y = sum over the K splits, in split order; four elements per thread.
__global__ __launch_bounds__(256) void proj_reduce_kernel(const ProjParams p)
{
    const size_t total = (size_t)p.M * p.N;
    const size_t e = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (e >= total) return;   // N % 32 == 0: a thread's four elements are all in range
    float4 s = *(const float4*)(p.part + e);
    for (int k = 1; k < p.ks; k++) {
        const float4 v = *(const float4*)(p.part + (size_t)k * total + e);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    if (p.y_f32) {
        *(float4*)((float*)p.y + e) = s;
    } else {
        *(uint2*)((uint16_t*)p.y + e) = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
    }
}

hipError_t launch_proj(const ProjParams& p, hipStream_t st)
{
    if (p.N % 32 != 0 || p.K % kProjStep != 0 || p.M <= 0 || p.ks < 1) return hipErrorInvalidValue;
    if ((long long)p.M * p.K * 2 + 2LL * p.K >= (1LL << 31)) return hipErrorInvalidValue;
    const int mt = p.M <= 32 ? 1 : 2;
    const long long mblk = (p.M + 32 * mt - 1) / (32 * mt);
    const long long grid = (long long)(p.N / 32) * p.ks * mblk;
    if (grid >= (1LL << 31)) return hipErrorInvalidValue;
    if (mt == 1)
        hipLaunchKernelGGL(proj_gemm_kernel<1>, dim3((unsigned)grid), dim3(64 * kProjWaves), 0, st, p);
    else
        hipLaunchKernelGGL(proj_gemm_kernel<2>, dim3((unsigned)grid), dim3(64 * kProjWaves), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ks == 1) return e;
    const size_t quads = ((size_t)p.M * p.N) / 4;
    hipLaunchKernelGGL(proj_reduce_kernel, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// W_abs[n, i d_c + c] = sum_e W_O[n, i d_v + e] W_UV[i, e, c], fp32 sums
// rounded to bf16.  Workgroup = (head i, 256 latent columns, 32 rows n):
// thread c keeps column c of W_UV[i] (d_v values) in registers, the 32 W_O
// row pieces sit in LDS and are read as broadcasts.
constexpr int kPmRows = 32;
constexpr int kPmMaxDv = 256;

__global__ __launch_bounds__(256) void premerge_kernel(const PremergeParams p)
{
    __shared__ float wo[kPmRows][kPmMaxDv];
    const int tid = threadIdx.x;
    const int ncb = p.d_c / 256, nrb = p.d_model / kPmRows;
    const int i = blockIdx.x % p.h;
    const int cb = (blockIdx.x / p.h) % ncb;
    const int rb = blockIdx.x / (p.h * ncb);
    if (rb >= nrb) return;
    const int c = cb * 256 + tid;
    const uint16_t* __restrict__ wuv = (const uint16_t*)p.w_uv + (size_t)i * p.d_v * p.d_c + c;
    const uint16_t* __restrict__ wo_g = (const uint16_t*)p.w_o;
    for (int k = tid; k < kPmRows * p.d_v; k += 256) {
        const int r = k / p.d_v, e = k % p.d_v;
        wo[r][e] = bf16lo_to_f32(wo_g[(size_t)(rb * kPmRows + r) * p.h * p.d_v + (size_t)i * p.d_v + e]);
    }
    __syncthreads();
    float acc[kPmRows];
#pragma unroll
    for (int r = 0; r < kPmRows; r++) acc[r] = 0.f;
    for (int e = 0; e < p.d_v; e++) {
        const float x = bf16lo_to_f32(wuv[(size_t)e * p.d_c]);
#pragma unroll
        for (int r = 0; r < kPmRows; r++) acc[r] = fmaf(wo[r][e], x, acc[r]);
    }
    uint16_t* __restrict__ out = (uint16_t*)p.w_abs;
#pragma unroll
    for (int r = 0; r < kPmRows; r++)
        out[(size_t)(rb * kPmRows + r) * p.h * p.d_c + (size_t)i * p.d_c + c] =
            (uint16_t)f32_to_bf16_bits(acc[r]);
}

hipError_t launch_premerge(const PremergeParams& p, hipStream_t st)
{
    if (p.d_c % 256 != 0 || p.d_model % kPmRows != 0 || p.d_v > kPmMaxDv || p.d_v <= 0)
        return hipErrorInvalidValue;
    const long long grid = (long long)p.h * (p.d_c / 256) * (p.d_model / kPmRows);
    if (grid >= (1LL << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(premerge_kernel, dim3((unsigned)grid), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
