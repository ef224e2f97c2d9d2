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

// 8 bytes of LDS (ds_read_b64)
__device__ __forceinline__ uint2 lds_read_8(const uint8_t* p)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) const u32x2 lds_u32x2;
    const u32x2 v = *(lds_u32x2*)p;
    return make_uint2(v[0], v[1]);
}

// Transposing LDS read of 8-bit elements (ds_read_b64_tr_b8).  Within each
// 16-lane group, source lane i supplies 8 consecutive bytes M_i[0..7];
// destination lane 8a + c receives M_a[c], M_{a+2}[c], ..., M_{a+14}[c].
// Pointing source lane i at row R(i / 2), byte 8 (i % 2) of a 16-byte-wide
// column block therefore hands lane j the column j of rows R(0) .. R(7).
__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* p)
{
    typedef int v2i __attribute__((ext_vector_type(2)));
    typedef __attribute__((address_space(3))) v2i lds_v2i;
    const v2i r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i*)p);
    return make_uint2((uint32_t)r[0], (uint32_t)r[1]);
}

// 8 OCP E4M3 codes (byte k of w is element k) -> 8 bf16, exactly (every E4M3
// value is a bf16 value), with v_cvt_scalef32_pk_bf16_fp8 at scale 1
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint2 w)
{
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, 1.f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, 1.f, true);
    const bf16x8 v = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return v;
}

// 8 bf16 times an fp32 factor, rounded back to bf16 (nearest even)
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 x, float f)
{
    const bf16x8 v = {(__bf16)((float)x[0] * f), (__bf16)((float)x[1] * f), (__bf16)((float)x[2] * f),
                      (__bf16)((float)x[3] * f), (__bf16)((float)x[4] * f), (__bf16)((float)x[5] * f),
                      (__bf16)((float)x[6] * f), (__bf16)((float)x[7] * f)};
    return v;
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
