// MLA decode in the absorbed ("MQA mode") form on gfx950, bf16 MFMA with fp32
// accumulation.
//
// Steps, in the order of "Multi-Head Latent Attention (MLA): Mathematical
// Foundations ..." (llms.blog), sections "Attention Logit Matrix Absorption"
// and "Value Output Matrix Absorption", and "MLA: why one latent can replace a
// multi-head KV cache" (charlestar.github.io), "First matrix absorption" /
// "Second matrix absorption":
//   1. mla_absorb_kernel    q^[b,i] = [bf16(W_UK[i]^T q_nope[b,i]) | q_rope[b,i]]
//   2. mla_decode_kernel    per (b, token split), all heads at once:
//                           S = q^ C^T over the cached rows [c | k_R],
//                           online softmax, u~ += P c  (same LDS tile)
//   3. mla_finish_kernel    merge the splits through their lse -> u~ (fp32),
//                           then out[b,i] = W_UV[i] u~[b,i]
// All h heads share every latent row, so the score [h x 576]x[576 x n] and
// value [h x n]x[n x 512] products are dense and run on the matrix cores;
// each latent row is fetched from HBM once per call.
#include "common.h"
#include "kernels.h"

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

__device__ __forceinline__ bf16x8 cat_tr(s16x4 lo, s16x4 hi)
{
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// 1. absorbed query.  One wavefront per (head i, 128 latent columns); W_UK[i]
//    columns are staged in LDS (row stride 272 B) and read as the MFMA B
//    operand with transposing reads; q_nope rows are the A operand.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;
constexpr int kAbsRowStride = kAbsCols * 2 + 16;

__global__ __launch_bounds__(64) void mla_absorb_kernel(const MlaParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int lane = threadIdx.x, G = lane / 16, li = lane % 16;
    const int nq = p.d_c / kAbsCols;
    const int i = blockIdx.x / nq, cq = blockIdx.x % nq;
    const int c0 = cq * kAbsCols;
    const int W = p.d_c + p.d_R;
    const uint16_t* __restrict__ wuk = (const uint16_t*)p.w_uk + (size_t)i * p.d_nope * p.d_c;
    const uint16_t* __restrict__ qn = (const uint16_t*)p.q_nope;

    // stage W_UK[i][:, c0:c0+128] (d_nope rows x 256 B)
    for (int idx = lane; idx < p.d_nope * (kAbsCols / 8); idx += 64) {
        const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
        *(uint4*)(smem + r * kAbsRowStride + c * 16) = *(const uint4*)(wuk + (size_t)r * p.d_c + c0 + c * 8);
    }
    // the rotary part of q^ is a plain copy (done once per head)
    if (cq == 0) {
        for (int idx = lane; idx < p.B * p.d_R; idx += 64) {
            const int bb = idx / p.d_R, e = idx % p.d_R;
            p.qhat[((size_t)bb * p.h + i) * W + p.d_c + e] =
                ((const uint16_t*)p.q_rope)[((size_t)bb * p.h + i) * p.d_R + e];
        }
    }
    __syncthreads();

    for (int b0 = 0; b0 < p.B; b0 += 16) {
        const int bb = b0 + li;
        for (int nt = 0; nt < kAbsCols / 16; nt++) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            for (int k0 = 0; k0 < p.d_nope; k0 += 32) {
                bf16x8 a;
                if (bb < p.B)
                    a = *(const bf16x8*)(qn + ((size_t)bb * p.h + i) * p.d_nope + k0 + 8 * G);
                else
                    a = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
                const int row = k0 + 8 * G + li / 4;
                const int col = nt * 16 + 4 * (li % 4);
                const s16x4 lo = lds_read_tr(smem + row * kAbsRowStride + col * 2);
                const s16x4 hi = lds_read_tr(smem + (row + 4) * kAbsRowStride + col * 2);
                acc = mfma16(a, cat_tr(lo, hi), acc);
            }
            // lane holds q~[b0 + 4G + e][c0 + 16 nt + li]
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int br = b0 + 4 * G + e;
                if (br < p.B)
                    p.qhat[((size_t)br * p.h + i) * W + c0 + nt * 16 + li] = (uint16_t)f32_to_bf16_bits(acc[e]);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// 2. decode.  Workgroup = (b, split, group of 64 heads), 4 wavefronts of
//    HW = 16 heads.
//    Latent tiles of 32 rows go HBM -> registers (one tile ahead) -> LDS
//    (double buffer, row stride 1168 B: conflict-free 16-byte reads).
//    Per wavefront and tile:
//      S^T[32 tok x HW heads] = C_tile[32 x 576] . q^T       (A: LDS rows, B: q^ in registers)
//      online softmax on S^T (lane = head, 8 tokens per lane)
//      U^T[512 x HW] += C_tile^T[512 x 32] . P^T[32 x HW]    (A: transposing LDS reads, B: P in registers)
//    The token order of the value product's K axis follows the score
//    product's output layout (lane group G holds tokens 4G..4G+3 and
//    16+4G..16+4G+3), so P never leaves the registers.
// ---------------------------------------------------------------------------
constexpr int kT = 32;             // tokens per tile
constexpr int kRow = 576 * 2;      // bytes per cached latent row
constexpr int kRS = kRow + 16;     // LDS row stride

template <int HW, bool PAGED>
__global__ __launch_bounds__(256) void mla_decode_kernel(const MlaParams p, int n_hgrp)
{
    constexpr int NT = HW / 16;     // head tiles per wavefront
    constexpr int KS = 576 / 32;    // score K steps
    constexpr int MC = 512 / 16;    // value M tiles (latent columns)
    __shared__ __attribute__((aligned(16))) uint8_t Cs[2][kT * kRS];

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);   // wave-uniform
    // Workgroup -> (unit u = (b, split), head group hg).  The head groups of
    // one unit get ids 8 apart: same XCD (ids are dealt to the 8 XCDs round
    // robin) and dispatched back to back, so the second read of each latent
    // tile is served by that XCD's L2.
    const int lane8 = blockIdx.x % 8, tq8 = blockIdx.x / 8;
    const int hg = tq8 % n_hgrp;
    const int u = (tq8 / n_hgrp) * 8 + lane8;
    if (u >= p.B * p.n_split) return;
    const int split = u % p.n_split, b = u / p.n_split;
    const int32_t* __restrict__ btab = p.bt;
    const int32_t* __restrict__ s_len = p.s;
    int n = __builtin_amdgcn_readfirstlane(s_len[b]);
    n = min(max(n, 0), p.s_max);
    const int t0 = split * p.chunk;
    const int t1 = min(n, t0 + p.chunk);
    const int head0 = (hg * 4 + wave) * HW;
    const bool active = head0 < p.h;
    const size_t pbase = ((size_t)b * p.n_split + split) * p.h;   // partial row of head 0

    if (t0 >= t1) {
        if (active && G == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                float* ml = p.part_ml + (pbase + head0 + nt * 16 + li) * 2;
                ml[0] = -INFINITY;
                ml[1] = 0.f;
            }
        }
        return;
    }

    // q^ fragments: B operand of the score product
    bf16x8 Qf[NT][KS];
    if (active) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                Qf[nt][ks] = *(const bf16x8*)(p.qhat + ((size_t)b * p.h + head0 + nt * 16 + li) * 576 +
                                              ks * 32 + 8 * G);
    }

    // staging: thread -> row (tid / 8) of the tile, chunks (tid % 8) + 8k
    const uint8_t* __restrict__ cbase = (const uint8_t*)p.cache;
    const uint32_t voff = (uint32_t)(lane / 8) * kRow + (uint32_t)(lane % 8) * 16;
    uint4 st[9];
    auto load_tile = [&](int tb) {
        const int r0 = tb + 8 * wave;   // first of this wavefront's 8 rows
        const uint8_t* base;
        int nrec;
        if (PAGED) {
            const int lb = r0 >> p.bs_log2;
            const int bstart = lb << p.bs_log2;
            int blk = __builtin_amdgcn_readfirstlane(btab[(size_t)b * p.max_blocks + min(lb, p.max_blocks - 1)]);
            blk = min(max(blk, 0), p.num_blocks - 1);
            base = cbase + (((size_t)blk << p.bs_log2) + (r0 - bstart)) * kRow;
        } else {
            base = cbase + ((size_t)b * p.s_max + r0) * kRow;
        }
        nrec = max(0, min(8, t1 - r0)) * kRow;
        const rsrc_t r = make_rsrc(base, nrec);
#pragma unroll
        for (int k = 0; k < 9; k++) st[k] = buf_load16(r, voff + k * 128);
    };
    auto store_tile = [&](int buf) {
        uint8_t* dst = Cs[buf] + (tid / 8) * kRS + (tid % 8) * 16;
#pragma unroll
        for (int k = 0; k < 9; k++) *(uint4*)(dst + k * 128) = st[k];
    };

    f32x4 U[MC][NT];
    float m[NT], lsum[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        m[nt] = -INFINITY;
        lsum[nt] = 0.f;
#pragma unroll
        for (int mc = 0; mc < MC; mc++) U[mc][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    load_tile(t0);
    store_tile(0);
    if (t0 + kT < t1) load_tile(t0 + kT);
    __syncthreads();

    int buf = 0;
    for (int tb = t0; tb < t1; tb += kT, buf ^= 1) {
        const uint8_t* C = Cs[buf];
        if (active) {
            // ---- scores S^T = C . q^T
            f32x4 S[2][NT];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++) S[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
#pragma unroll
                for (int mt = 0; mt < 2; mt++) {
                    const bf16x8 a = *(const bf16x8*)(C + (16 * mt + li) * kRS + (4 * ks + G) * 16);
#pragma unroll
                    for (int nt = 0; nt < NT; nt++) S[mt][nt] = mfma16(a, Qf[nt][ks], S[mt][nt]);
                }
            }
            // keep the LDS reads at most two K steps ahead of the MFMAs
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NT, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            // ---- online softmax: lane holds head (16 nt + li), tokens 16 mt + 4G + e.
            // The reference max m only moves when a tile's max exceeds it by
            // more than 8 (log2 units); otherwise probabilities up to 2^8 are
            // accumulated against the old m, which is exact after the final
            // division and spares rescaling the 512-wide accumulators.
            bf16x8 P[NT];
            bool rescale = false;
            float alpha[NT];
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                float z[2][4];
                float lm = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int tok = tb + 16 * mt + 4 * G + e;
                        z[mt][e] = tok < t1 ? S[mt][nt][e] * p.scale_log2 : -INFINITY;
                        lm = fmaxf(lm, z[mt][e]);
                    }
                lm = fmaxf(lm, xor16(lm));
                lm = fmaxf(lm, xor32(lm));
                const bool move = lm > m[nt] + 8.f;
                const float mn = move ? lm : m[nt];
                alpha[nt] = move ? __builtin_amdgcn_exp2f(m[nt] - mn) : 1.f;
                rescale |= move;
                m[nt] = mn;
                uint32_t pk[4];
                float ps = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(z[mt][e] - mn),
                                                       __builtin_amdgcn_exp2f(z[mt][e + 1] - mn));
                        pk[mt * 2 + e / 2] = w;
                        ps += bf16lo_to_f32(w) + bf16hi_to_f32(w);
                    }
                lsum[nt] = lsum[nt] * alpha[nt] + ps;
                P[nt] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
            if (__builtin_amdgcn_ballot_w64(rescale)) {
#pragma unroll
                for (int mc = 0; mc < MC; mc++) {
#pragma unroll
                    for (int nt = 0; nt < NT; nt++) U[mc][nt] *= alpha[nt];
                    __builtin_amdgcn_sched_barrier(0);   // a few accumulators at a time
                }
            }
            // ---- latent sum U^T += C^T . P^T (transposing reads of the same tile)
            const uint8_t* r0 = C + (4 * G + li / 4) * kRS + 4 * (li % 4) * 2;
            const uint8_t* r1 = r0 + 16 * kRS;
#pragma unroll
            for (int mc = 0; mc < MC; mc++) {
                const bf16x8 a = cat_tr(lds_read_tr(r0 + mc * 32), lds_read_tr(r1 + mc * 32));
#pragma unroll
                for (int nt = 0; nt < NT; nt++) U[mc][nt] = mfma16(a, P[nt], U[mc][nt]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
            for (int mc = 0; mc < MC; mc++) {
                __builtin_amdgcn_sched_group_barrier(0x008, NT, 1);
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
            }
        }
        if (tb + kT < t1) {
            store_tile(buf ^ 1);
            if (tb + 2 * kT < t1) load_tile(tb + 2 * kT);
        }
        __syncthreads();
    }

    if (!active) return;
    // ---- partial state of this split: m, l per head, U^T columns
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        float l = lsum[nt];
        l += xor16(l);
        l += xor32(l);
        const size_t row = pbase + head0 + nt * 16 + li;
        float* pu = p.part_u + row * 512 + 4 * G;
#pragma unroll
        for (int mc = 0; mc < MC; mc++)
            *(float4*)(pu + 16 * mc) = make_float4(U[mc][nt][0], U[mc][nt][1], U[mc][nt][2], U[mc][nt][3]);
        if (G == 0) {
            p.part_ml[row * 2] = m[nt];
            p.part_ml[row * 2 + 1] = l;
        }
    }
}

// ---------------------------------------------------------------------------
// 3. finish.  Workgroup = (head i, 16 sequences).  Merge the split partials
//    into u~ (fp32; written to u_latent and kept in LDS), then
//    out[b, i, :] = W_UV[i] u~[b, i, :] on the matrix cores.  u~ is fed as a
//    bf16 hi/lo pair (u~ = hi + lo exactly to about 2^-16 relative), so the
//    product keeps u~ at fp32-level precision; W_UV rows are the B operand
//    as stored (16 contiguous bytes per lane).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mla_finish_kernel(const MlaParams p)
{
    __shared__ __attribute__((aligned(16))) float Us[16][512 + 4];
    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int i = blockIdx.x % p.h;
    const int b0 = (blockIdx.x / p.h) * 16;

    // merge: wavefront w handles sequences b0 + 4w .. b0 + 4w + 3
    for (int sb = 0; sb < 4; sb++) {
        const int r = 4 * wave + sb, bb = b0 + r;
        if (bb >= p.B) {
            for (int c = lane; c < 512; c += 64) Us[r][c] = 0.f;
            continue;
        }
        const float* __restrict__ ml = p.part_ml;
        float M = -INFINITY;
        for (int k = 0; k < p.n_split; k++) {
            const size_t row = ((size_t)bb * p.n_split + k) * p.h + i;
            if (ml[row * 2 + 1] > 0.f) M = fmaxf(M, ml[row * 2]);
        }
        float L = 0.f;
        float4 acc0 = make_float4(0, 0, 0, 0), acc1 = make_float4(0, 0, 0, 0);
        for (int k = 0; k < p.n_split; k++) {
            const size_t row = ((size_t)bb * p.n_split + k) * p.h + i;
            const float lk = ml[row * 2 + 1];
            if (lk > 0.f) {
                const float wk = __builtin_amdgcn_exp2f(ml[row * 2] - M);
                L = fmaf(wk, lk, L);
                const float4 u0 = *(const float4*)(p.part_u + row * 512 + lane * 4);
                const float4 u1 = *(const float4*)(p.part_u + row * 512 + 256 + lane * 4);
                acc0.x = fmaf(wk, u0.x, acc0.x); acc0.y = fmaf(wk, u0.y, acc0.y);
                acc0.z = fmaf(wk, u0.z, acc0.z); acc0.w = fmaf(wk, u0.w, acc0.w);
                acc1.x = fmaf(wk, u1.x, acc1.x); acc1.y = fmaf(wk, u1.y, acc1.y);
                acc1.z = fmaf(wk, u1.z, acc1.z); acc1.w = fmaf(wk, u1.w, acc1.w);
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        acc0.x *= inv; acc0.y *= inv; acc0.z *= inv; acc0.w *= inv;
        acc1.x *= inv; acc1.y *= inv; acc1.z *= inv; acc1.w *= inv;
        *(float4*)&Us[r][lane * 4] = acc0;
        *(float4*)&Us[r][256 + lane * 4] = acc1;
        const size_t urow = ((size_t)bb * p.h + i) * 512;
        *(float4*)(p.u_latent + urow + lane * 4) = acc0;
        *(float4*)(p.u_latent + urow + 256 + lane * 4) = acc1;
        if (lane == 0 && p.lse) p.lse[(size_t)bb * p.h + i] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
    __syncthreads();

    // out[b0 + m, i, n] = sum_c u~[m][c] W_UV[i][n][c]: M = 16 sequences,
    // N = d_v (wavefront w takes column tiles w, w+4, ...), K = d_c
    const uint16_t* __restrict__ wuv = (const uint16_t*)p.w_uv + (size_t)i * p.d_v * p.d_c;
    for (int nt = wave; nt < p.d_v / 16; nt += 4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* wrow = wuv + (size_t)(nt * 16 + li) * p.d_c + 8 * G;
        for (int k0 = 0; k0 < p.d_c; k0 += 32) {
            const bf16x8 bw = *(const bf16x8*)(wrow + k0);
            const float4 x0 = *(const float4*)&Us[li][k0 + 8 * G];
            const float4 x1 = *(const float4*)&Us[li][k0 + 8 * G + 4];
            const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const uint32_t h2 = pack_bf16x2(xs[e], xs[e + 1]);
                hi[e / 2] = h2;
                lo[e / 2] = pack_bf16x2(xs[e] - bf16lo_to_f32(h2), xs[e + 1] - bf16hi_to_f32(h2));
            }
            acc = mfma16(__builtin_bit_cast(bf16x8, make_uint4(hi[0], hi[1], hi[2], hi[3])), bw, acc);
            acc = mfma16(__builtin_bit_cast(bf16x8, make_uint4(lo[0], lo[1], lo[2], lo[3])), bw, acc);
        }
        // lane holds out[b0 + 4G + e][i][16 nt + li]
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int bb = b0 + 4 * G + e;
            if (bb < p.B)
                ((uint16_t*)p.out)[((size_t)bb * p.h + i) * p.d_v + nt * 16 + li] =
                    (uint16_t)f32_to_bf16_bits(acc[e]);
        }
    }
}

hipError_t launch_mla(const MlaParams& p, bool paged, hipStream_t st)
{
    const unsigned g1 = (unsigned)(p.h * (p.d_c / kAbsCols));
    const size_t smem1 = (size_t)p.d_nope * kAbsRowStride;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t ea = hipFuncSetAttribute((const void*)mla_absorb_kernel,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (ea != hipSuccess) return ea;
        attr_set = true;
    }
    hipLaunchKernelGGL(mla_absorb_kernel, dim3(g1), dim3(64), smem1, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_hgrp = (p.h + 63) / 64;
    const unsigned units8 = (unsigned)((p.B * p.n_split + 7) / 8 * 8);
    const unsigned g2 = units8 * n_hgrp;
    if (paged) hipLaunchKernelGGL((mla_decode_kernel<16, true>), dim3(g2), dim3(256), 0, st, p, n_hgrp);
    else hipLaunchKernelGGL((mla_decode_kernel<16, false>), dim3(g2), dim3(256), 0, st, p, n_hgrp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g3 = (unsigned)(p.h * ((p.B + 15) / 16));
    hipLaunchKernelGGL(mla_finish_kernel, dim3(g3), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
