// Device helpers shared by the gfx950 decode-attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- bit-level conversions ------------------------------------------------
__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xffffu; }

// (low halves of a, b) and (high halves of a, b), each as one bf16 pair
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 operands, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), acc, false);
}

// ---- wavefront (64-lane) reductions: DPP inside rows of 16, lane swaps across rows
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float xor16(float x)
{
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    // r[0] holds the row-swapped copy in odd rows, r[1] in even rows
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ float row16_max(float x)
{
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return x;
}
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    x += dpp<0x140>(x);
    return x;
}
__device__ __forceinline__ float wave_max(float x)
{
    x = row16_max(x);
    x = fmaxf(x, xor16(x));
    x = fmaxf(x, xor32(x));
    return x;
}
__device__ __forceinline__ float wave_sum(float x)
{
    x = row16_sum(x);
    x += xor16(x);
    x += xor32(x);
    return x;
}
// inclusive prefix sum over the 64 lanes of a wavefront (lane l gets the sum
// of lanes 0 .. l)
__device__ __forceinline__ int wave_scan_incl(int x)
{
    const int lane = threadIdx.x % 64;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int t = __shfl_up(x, d, 64);
        if (lane >= d) x += t;
    }
    return x;
}

__device__ __forceinline__ float uniform(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// ---- buffer loads: SGPR resource + 32-bit VGPR offset; offsets at or past
// num_records return zeros (no memory access), which is how tile tails and
// unmapped pages are kept in bounds.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format
// Every field must be wave-uniform; readfirstlane pins them to SGPRs so the
// compiler never wraps the load in a per-lane (waterfall) loop.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int num_records)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const int nr = __builtin_amdgcn_readfirstlane(num_records > 0 ? num_records : 0);
    void* ub = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, nr, kRsrcFlags);
}
__device__ __forceinline__ uint4 buf_load16(rsrc_t r, uint32_t voff)
{
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// Physical row of token t of sequence b in a paged pool of 2^bs_log2-row
// blocks (one scalar load).  Block numbers are clamped into the pool and the
// logical block into the table, so a bad entry can only misplace rows, never
// address outside the pool.
__device__ __forceinline__ size_t paged_row(const int32_t* __restrict__ btab, int b, int t,
                                            int max_blocks, int bs_log2, int num_blocks)
{
    const int lb = min(t >> bs_log2, max_blocks - 1);
    int blk = __builtin_amdgcn_readfirstlane(btab[(size_t)b * max_blocks + lb]);
    blk = min(max(blk, 0), num_blocks - 1);
    return ((size_t)blk << bs_log2) + (t & ((1 << bs_log2) - 1));
}

// Workgroup j of a launch runs on XCD j % 8 (round-robin dispatch).  This
// renumbering gives each XCD a contiguous run of work items, so that items
// that share data (one sequence's splits or KV heads) run under one L2.  A
// tail of n % 8 workgroups keeps its own numbering.
__device__ __forceinline__ int xcd_major(int j, int n)
{
    const int full = n & ~7;
    return j < full ? (j & 7) * (full >> 3) + (j >> 3) : j;
}

// order LDS traffic between the lanes of one wavefront
__device__ __forceinline__ void wave_lds_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace attn
