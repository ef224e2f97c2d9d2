// Matrix-core and LDS-DMA helpers shared by the gfx950 MFMA decode kernels.
#pragma once

#include "common.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// source lane i = a + 4k supplies 4 consecutive 16-bit values M_i[0..3];
// destination lane 4a + c receives M_{a}[c], M_{a+4}[c], M_{a+8}[c],
// M_{a+12}[c].  Pointing source lane i at row (row0 + i/4), column
// (col0 + 4*(i%4)) of a row-major bf16 matrix therefore hands lane j the
// column col0 + j of rows row0 .. row0+3: an MFMA operand with K along rows.
__device__ __forceinline__ s16x4 lds_read_tr(const uint8_t* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// 16 bytes of LDS as two 8-byte reads (ds_read_b64 x 2).  The volatile
// accesses keep the compiler from fusing them into one 16-byte read.
__device__ __forceinline__ bf16x8 lds_read_16_as_2x8(const uint8_t* p)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) volatile const u32x2 lds_u32x2;
    const u32x2 lo = *(lds_u32x2*)p;
    const u32x2 hi = *(lds_u32x2*)(p + 8);
    return __builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], hi[0], hi[1]));
}

__device__ __forceinline__ bf16x8 cat_tr(s16x4 lo, s16x4 hi)
{
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// 16 bytes per lane from the buffer resource to LDS at m0 + 16 * lane.  Issued
// through asm so that the compiler does not serialise it against every LDS
// read; completion is awaited explicitly with wait_vmcnt<N>().  The cache is
// streamed once per call, so the loads carry the non-temporal hint (nt):
// measured on MI355X, a plain LDS-DMA stream reaches 5.8-6.3 TB/s and the
// same stream with nt 7.2-7.3 TB/s.
__device__ __forceinline__ void dma16(rsrc_t r, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :: "v"(voff), "s"(r), "s"(lds_addr) : "memory");
}
// vmcnt(0) through the builtin, so that the compiler knows its own vector
// loads have completed and inserts no waits for them later
__device__ __forceinline__ void vmem_drain()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0), expcnt and lgkmcnt unconstrained
}
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

}  // namespace attn
