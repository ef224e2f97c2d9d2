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
#include "mfma_lds.h"

namespace attn {

// ---------------------------------------------------------------------------
// 1. absorbed query.  Workgroup (4 wavefronts) per (head i, 128 latent
//    columns): W_UK[i][:, cols] is staged in LDS (row stride 272 B) with all
//    loads in flight at once and read as the MFMA B operand through
//    transposing reads; q_nope rows are the A operand, fetched up front.
// ---------------------------------------------------------------------------
constexpr int kAbsCols = 128;
constexpr int kAbsRowStride = kAbsCols * 2 + 16;

__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int nq = p.d_c / kAbsCols;
    const int i = blockIdx.x / nq, cq = blockIdx.x % nq;
    const int c0 = cq * kAbsCols;
    const int W = p.d_c + p.d_R;
    const uint16_t* __restrict__ wuk = (const uint16_t*)p.w_uk + (size_t)i * p.d_nope * p.d_c;
    const uint16_t* __restrict__ qn = (const uint16_t*)p.q_nope;

    // q_nope rows of one 16-sequence block: the A operand (rows past B are zero)
    const int ksteps = p.d_nope / 32;
    auto load_a = [&](int b0, bf16x8* a) {
        const int bb = b0 + li;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            if (k < ksteps && bb < p.B)
                a[k] = *(const bf16x8*)(qn + ((size_t)bb * p.h + i) * p.d_nope + k * 32 + 8 * G);
            else
                a[k] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
    };
    bf16x8 a[8];
    load_a(0, a);

    // stage W_UK[i][:, c0:c0+128]: d_nope rows x 16 chunks, 8 loads in flight per thread
    const int nchunk = p.d_nope * (kAbsCols / 8);
    for (int base = 0; base < nchunk; base += 256 * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int idx = base + u * 256 + tid;
            if (idx < nchunk) {
                const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
                v[u] = *(const uint4*)(wuk + (size_t)r * p.d_c + c0 + c * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int idx = base + u * 256 + tid;
            if (idx < nchunk) {
                const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
                *(uint4*)(smem + r * kAbsRowStride + c * 16) = v[u];
            }
        }
    }
    // the rotary part of q^ is a plain copy (done once per head, 16 bytes per
    // lane, four copies in flight); d_R is a multiple of 8
    if (cq == 0) {
        const int per = p.d_R / 8, nv = p.B * per;
        const uint16_t* __restrict__ qr = (const uint16_t*)p.q_rope;
        for (int base = 0; base < nv; base += 4 * 256) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int idx = base + u * 256 + tid;
                if (idx < nv) v[u] = *(const uint4*)(qr + ((size_t)(idx / per) * p.h + i) * p.d_R + 8 * (idx % per));
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int idx = base + u * 256 + tid;
                if (idx < nv) *(uint4*)(p.qhat + ((size_t)(idx / per) * p.h + i) * W + p.d_c + 8 * (idx % per)) = v[u];
            }
        }
    }

    __syncthreads();

    // wavefront w computes column tiles 2w and 2w+1 for every 16-row block of
    // b; the next block's q_nope is fetched while this one is multiplied
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        bf16x8 an[8];
        if (b0 + 16 < p.B) load_a(b0 + 16, an);
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int nt = 2 * wave + t;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < 8; k++) {
                if (k < ksteps) {
                    const int row = k * 32 + 8 * G + li / 4;
                    const int col = nt * 16 + 4 * (li % 4);
                    const s16x4 lo = lds_read_tr(smem + row * kAbsRowStride + col * 2);
                    const s16x4 hi = lds_read_tr(smem + (row + 4) * kAbsRowStride + col * 2);
                    acc = mfma16(a[k], cat_tr(lo, hi), acc);
                }
            }
            // lane holds q~[b0 + 4G + e][c0 + 16 nt + li]
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int br = b0 + 4 * G + e;
                if (br < p.B)
                    p.qhat[((size_t)br * p.h + i) * W + c0 + nt * 16 + li] = (uint16_t)f32_to_bf16_bits(acc[e]);
            }
        }
        if (b0 + 16 < p.B) {
#pragma unroll
            for (int k = 0; k < 8; k++) a[k] = an[k];
        }
    }
}

// ---------------------------------------------------------------------------
// 2. decode.  Workgroup = (b, token split) with all heads, so every latent
//    tile is fetched once: 4 wavefronts x 32 heads in the fast kernel (one
//    wavefront per SIMD, accumulators in AGPRs), 8 x 16 in the rescaling
//    fallback.  Tiles of 32 rows move HBM -> LDS by LDS-DMA (buffer_load ...
//    lds, no staging registers) into a ring of 4 buffers, three tiles ahead
//    of use.  Per wavefront, 16-head block and tile:
//      S^T[32 tok x 16 heads] = C_tile[32 x 576] . q^T     (A: LDS, B: q^ in registers)
//      online softmax on S^T (lane = head, 8 tokens per lane)
//      U^T[512 x 16] += C_tile^T[512 x 32] . P^T[32 x 16]  (A: transposing LDS reads, B: P)
//    The token order of the value product's K axis is the score product's
//    output layout (lane group G holds tokens 4G..4G+3 and 16+4G..16+4G+3),
//    so P never leaves the registers.
//
//    LDS tile layout (one buffer, 36 KB): 9 segments of 128 bytes per row,
//    segment-major: byte (s * 4096 + r * 128 + 16 * p) holds row r, 16-byte
//    chunk 8 s + (p ^ swz(r)).  One DMA instruction fills 8 rows of one
//    segment (1 KB, lane-contiguous as the hardware writes it; each group of 8
//    lanes still reads one 128-byte line).  The XOR swizzle spreads the rows
//    of an operand over the banks; score operands are read as two 8-byte
//    halves, which measured ~1.6x faster than one 16-byte read per lane for
//    this scattered-row pattern.
//
//    Completion of the LDS-DMA is tracked with explicit vmcnt waits, so no
//    other vector-memory instruction may be outstanding inside the tile loop
//    (a compiler-inserted vmcnt(0) for it would also drain the prefetched
//    tiles): q^ is loaded and waited for before the loop, and the loop keeps
//    its state in registers (no spills).  LDS operands are read one K step
//    ahead of the matrix instructions that use them.
// ---------------------------------------------------------------------------
constexpr int kT = 32;             // tokens per tile
constexpr int kRow = 576 * 2;      // bytes per cached latent row
constexpr int kTile = kT * kRow;   // 36,864 bytes
constexpr int kNBuf = 4;           // LDS ring depth
constexpr int kSlots = kTile / 1024;   // 36 DMA instructions per tile

// XOR swizzle of the 16-byte chunk position within a 128-byte row segment:
// s(r) = r0 ^ 2 r1 ^ 5 r2 ^ 7 r3 (r_k the bits of r).  Any 8 consecutive
// rows get distinct positions; among the XOR-linear choices with that
// property this one measured fastest for the mix of score-operand and
// transposing reads below (within a few percent of the others).
__device__ __forceinline__ int swz(int r)
{
    return (r & 1) ^ (r & 2) ^ ((r & 4) ? 5 : 0) ^ ((r & 8) ? 7 : 0);
}
__device__ __forceinline__ int tile_off(int r, int c)   // row r, logical 16-byte chunk c
{
    return (c >> 3) * 4096 + r * 128 + (((c & 7) ^ swz(r)) << 4);
}

// Per-lane byte offsets of the MFMA operands within a tile buffer, split so
// that everything depending on the K step is a compile-time constant (the
// immediate offset of the LDS instruction):
//   score operand, K step ks, row block mt: row 16 mt + li, chunk 4 ks + G
//     = (ks >> 1) * 4096 + mt * 2048 + [li * 128 + ((4 (ks & 1) + G) ^ s) * 16]
//   value operand, column tile mc, token half th: rows 4G + li/4 + 16 th,
//     chunk 2 mc + (li % 4) / 2, byte 8 (li % 2) within it
//     = (mc >> 2) * 4096 + th * 2048 + [row * 128 + ((2 (mc & 3) + cp) ^ s) * 16 + 8 (li % 2)]
// (s = swz(row) is the same for row and row + 16).
struct TileOffsets {
    int sc[2];   // score, by K-step parity
    int tr[4];   // value, by mc % 4
    __device__ __forceinline__ TileOffsets(int li, int G)
    {
        const int ss = swz(li);
        sc[0] = li * 128 + ((G ^ ss) << 4);
        sc[1] = li * 128 + (((4 + G) ^ ss) << 4);
        const int r = 4 * G + li / 4, cp = (li % 4) / 2, st = swz(r);
#pragma unroll
        for (int j = 0; j < 4; j++) tr[j] = r * 128 + (((2 * j + cp) ^ st) << 4) + 8 * (li % 2);
    }
    __device__ __forceinline__ const uint8_t* score(const uint8_t* C, int ks, int mt) const
    {
        return C + sc[ks & 1] + (ks >> 1) * 4096 + mt * 2048;
    }
    __device__ __forceinline__ const uint8_t* value(const uint8_t* C, int mc, int th) const
    {
        return C + tr[mc & 3] + (mc >> 2) * 4096 + th * 2048;
    }
};


template <int HW, bool PAGED>
__global__ __launch_bounds__(64 * (128 / HW)) void mla_decode_fast_kernel(const MlaParams p,
                                                                          const int32_t* __restrict__ btab)
{
    constexpr int NW = 128 / HW;    // wavefronts per workgroup
    constexpr int NT = HW / 16;     // head tiles per wavefront
    constexpr int SPW = kSlots / NW + (kSlots % NW ? 1 : 0);   // DMA slots per wavefront
    constexpr int KS = 576 / 32;    // score K steps
    constexpr int MC = 512 / 16;    // value M tiles (latent columns)
    constexpr int PS = 1;   // score operands are read this many K steps ahead
    constexpr int PV = 1;   // value operands are read this many column tiles ahead
    __shared__ __attribute__((aligned(1024))) uint8_t Cs[kNBuf * kTile];
    __shared__ int ovf;   // some head's scores ran past its reference max + 64

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wg = xcd_major(blockIdx.x, gridDim.x);
    const int split = wg % p.n_split, b = wg / p.n_split;
    const int32_t* __restrict__ s_len = p.s;
    int n = __builtin_amdgcn_readfirstlane(s_len[b]);
    n = min(max(n, 0), p.s_max);
    const int t0 = split * p.chunk;
    const int t1 = min(n, t0 + p.chunk);
    const int head0 = wave * HW;
    const bool active = head0 < p.h;
    const size_t pbase = ((size_t)b * p.n_split + split) * p.h;   // partial row of head 0

    if (t0 >= t1) {
        if (tid == 0) p.flags[wg] = 0;
        if (active && G == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                if (head0 + 16 * nt < p.h) {
                    float* ml = p.part_ml + (pbase + head0 + 16 * nt + li) * 2;
                    ml[0] = -INFINITY;
                    ml[1] = 0.f;
                }
            }
        }
        return;
    }

    // DMA slots of this wavefront: q = wave + NW j (q < 36); slot q fills
    // segment q / 4, rows 8 (q % 4) .. + 7.
    const uint8_t* __restrict__ cbase = (const uint8_t*)p.cache;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Cs;
    const int lr = lane / 8;                      // row within the slot
    const int lp = lane % 8;                      // physical chunk within the segment
    // A tile's two 16-row halves each lie in one block of a paged pool
    // (blocks hold a power of two >= 16 rows); their physical rows are looked
    // up one iteration before the tile is issued.
    auto half_row = [&](int t) -> size_t {   // physical row of token t (a multiple of 16)
        if (PAGED) return paged_row(btab, b, t, p.max_blocks, p.bs_log2, p.num_blocks);
        return (size_t)b * p.s_max + t;
    };
    auto issue_tile = [&](int tb, int buf, size_t row0, size_t row1) {
#pragma unroll
        for (int j = 0; j < SPW; j++) {
            const int q = wave + NW * j;
            if (q < kSlots) {                      // wave-uniform
                const int seg = q >> 2, rb = q & 3;
                const int r0 = tb + 8 * rb;        // first row of the slot
                const size_t row = (rb < 2 ? row0 : row1) + 8 * (rb & 1);
                const rsrc_t rs = make_rsrc(cbase + row * kRow, max(0, min(8, t1 - r0)) * kRow);
                const int c = 8 * seg + (lp ^ swz(8 * rb + lr));
                dma16(rs, (uint32_t)(lr * kRow + c * 16), lds0 + buf * kTile + q * 1024);
            }
        }
    };

    // Per head: m is fixed at the first tile's max (log2 units) and U, lsum
    // accumulate 2^(z - m).  Later tiles may exceed m by up to 64 (p <= 2^64,
    // far from fp32/bf16 overflow); past that the split is handed to the
    // rescaling kernel (flag), which real logits essentially never need.
    f32x4 U[MC][NT];
    float m[NT], lsum[NT];
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        m[nt] = -INFINITY;
        lsum[nt] = 0.f;
#pragma unroll
        for (int mc = 0; mc < MC; mc++) U[mc][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (tid == 0) ovf = 0;

    // first two tiles in flight, then the q^ fragments (B operand of the
    // score product; head tiles past h read as zeros), then the third tile
    {
        const size_t a0 = half_row(t0), a1 = half_row(t0 + 16);
        const size_t b0 = half_row(t0 + kT), b1 = half_row(t0 + kT + 16);
        issue_tile(t0, 0, a0, a1);
        issue_tile(t0 + kT, 1, b0, b1);
    }
    bf16x8 Qf[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; nt++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            Qf[nt][ks] = head0 + 16 * nt < p.h
                ? *(const bf16x8*)(p.qhat + ((size_t)b * p.h + head0 + 16 * nt + li) * 576 + ks * 32 + 8 * G)
                : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    vmem_drain();
    issue_tile(t0 + 2 * kT, 2, half_row(t0 + 2 * kT), half_row(t0 + 2 * kT + 16));

    const TileOffsets to(li, G);
    int buf = 0;
    for (int tb = t0; tb < t1; tb += kT) {
        const size_t nx0 = half_row(tb + 3 * kT), nx1 = half_row(tb + 3 * kT + 16);
        // tiles tb + T and tb + 2T were issued after this one
        if (SPW * NW == kSlots || wave < kSlots % NW) wait_vmcnt<2 * SPW>();
        else wait_vmcnt<2 * (SPW - 1)>();
        __syncthreads();
        if (ovf) break;                      // uniform across the workgroup
        // refill the buffer read in the previous iteration (every wavefront is
        // past it), so that three tiles stay in flight while this one is used
        issue_tile(tb + 3 * kT, (buf + 3) % kNBuf, nx0, nx1);
        const uint8_t* C = Cs + buf * kTile;
        if (active) {
            // ---- scores S^T = C . q^T
            f32x4 S[2][NT];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++) S[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 a[PS + 1][2];   // ring of operands, PS K steps ahead
#pragma unroll
            for (int i = 0; i < PS; i++) {
                a[i][0] = lds_read_16_as_2x8(to.score(C, i, 0));
                a[i][1] = lds_read_16_as_2x8(to.score(C, i, 1));
            }
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                if (ks + PS < KS) {
                    a[(ks + PS) % (PS + 1)][0] = lds_read_16_as_2x8(to.score(C, ks + PS, 0));
                    a[(ks + PS) % (PS + 1)][1] = lds_read_16_as_2x8(to.score(C, ks + PS, 1));
                }
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int nt = 0; nt < NT; nt++)
                        S[mt][nt] = mfma16(a[ks % (PS + 1)][mt], Qf[nt][ks], S[mt][nt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- softmax weights against the fixed per-head reference m
            bf16x8 P[NT];
            bool over = false;
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
                if (m[nt] == -INFINITY) {       // first tile: fix the reference
                    lm = fmaxf(lm, xor16(lm));
                    lm = fmaxf(lm, xor32(lm));
                    m[nt] = lm;
                }
                over |= lm > m[nt] + 64.f;
                uint32_t pk[4];
                float ps = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const uint32_t w = pack_bf16x2(__builtin_amdgcn_exp2f(z[mt][e] - m[nt]),
                                                       __builtin_amdgcn_exp2f(z[mt][e + 1] - m[nt]));
                        pk[mt * 2 + e / 2] = w;
                        ps += bf16lo_to_f32(w) + bf16hi_to_f32(w);
                    }
                lsum[nt] += ps;
                P[nt] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
            if (__builtin_amdgcn_ballot_w64(over) && lane == 0) ovf = 1;
            // ---- latent sum U^T += C^T . P^T (transposing reads of the same tile)
            s16x4 lo[PV + 1], hi[PV + 1];   // ring of operands, PV column tiles ahead
#pragma unroll
            for (int i = 0; i < PV; i++) {
                lo[i] = lds_read_tr(to.value(C, i, 0));
                hi[i] = lds_read_tr(to.value(C, i, 1));
            }
#pragma unroll
            for (int mc = 0; mc < MC; mc++) {
                if (mc + PV < MC) {
                    lo[(mc + PV) % (PV + 1)] = lds_read_tr(to.value(C, mc + PV, 0));
                    hi[(mc + PV) % (PV + 1)] = lds_read_tr(to.value(C, mc + PV, 1));
                }
                const bf16x8 av = cat_tr(lo[mc % (PV + 1)], hi[mc % (PV + 1)]);
#pragma unroll
                for (int nt = 0; nt < NT; nt++) U[mc][nt] = mfma16(av, P[nt], U[mc][nt]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        buf = (buf + 1) % kNBuf;
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup

    __syncthreads();   // ovf from the last tile
    if (tid == 0) p.flags[wg] = ovf;
    if (ovf || !active) return;
    // ---- partial state of this split: m, l per head, U^T columns
#pragma unroll
    for (int nt = 0; nt < NT; nt++) {
        if (head0 + 16 * nt >= p.h) continue;
        float l = lsum[nt];
        l += xor16(l);
        l += xor32(l);
        const size_t row = pbase + head0 + 16 * nt + li;
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

template <bool PAGED>
__global__ __launch_bounds__(512) void mla_decode_safe_kernel(const MlaParams p,
                                                              const int32_t* __restrict__ btab)
{
    constexpr int KS = 576 / 32;    // score K steps
    constexpr int MC = 512 / 16;    // value M tiles (latent columns)
    __shared__ __attribute__((aligned(1024))) uint8_t Cs[kNBuf * kTile];

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int wg = xcd_major(blockIdx.x, gridDim.x);
    const int split = wg % p.n_split, b = wg / p.n_split;
    if (__builtin_amdgcn_readfirstlane(p.flags[wg]) == 0) return;   // fast kernel finished it
    const int32_t* __restrict__ s_len = p.s;
    int n = __builtin_amdgcn_readfirstlane(s_len[b]);
    n = min(max(n, 0), p.s_max);
    const int t0 = split * p.chunk;
    const int t1 = min(n, t0 + p.chunk);
    const int head0 = wave * 16;
    const bool active = head0 < p.h;
    const size_t pbase = ((size_t)b * p.n_split + split) * p.h;   // partial row of head 0

    if (t0 >= t1) {
        if (active && G == 0) {
            float* ml = p.part_ml + (pbase + head0 + li) * 2;
            ml[0] = -INFINITY;
            ml[1] = 0.f;
        }
        return;
    }

    // DMA slots of this wavefront: q = wave + 8 j (j < 5, q < 36); slot q
    // fills segment q / 4, rows 8 (q % 4) .. + 7.
    const uint8_t* __restrict__ cbase = (const uint8_t*)p.cache;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Cs;
    const int lr = lane / 8;                      // row within the slot
    const int lp = lane % 8;                      // physical chunk within the segment
    // A tile's two 16-row halves each lie in one block of a paged pool
    // (blocks hold a power of two >= 16 rows); their physical rows are looked
    // up one iteration before the tile is issued.
    auto half_row = [&](int t) -> size_t {   // physical row of token t (a multiple of 16)
        if (PAGED) return paged_row(btab, b, t, p.max_blocks, p.bs_log2, p.num_blocks);
        return (size_t)b * p.s_max + t;
    };
    auto issue_tile = [&](int tb, int buf, size_t row0, size_t row1) {
#pragma unroll
        for (int j = 0; j < 5; j++) {
            const int q = wave + 8 * j;
            if (q < kSlots) {                      // wave-uniform
                const int seg = q >> 2, rb = q & 3;
                const int r0 = tb + 8 * rb;        // first row of the slot
                const size_t row = (rb < 2 ? row0 : row1) + 8 * (rb & 1);
                const rsrc_t rs = make_rsrc(cbase + row * kRow, max(0, min(8, t1 - r0)) * kRow);
                const int c = 8 * seg + (lp ^ swz(8 * rb + lr));
                dma16(rs, (uint32_t)(lr * kRow + c * 16), lds0 + buf * kTile + q * 1024);
            }
        }
    };

    f32x4 U[MC];
    float m = -INFINITY, lsum = 0.f;
#pragma unroll
    for (int mc = 0; mc < MC; mc++) U[mc] = f32x4{0.f, 0.f, 0.f, 0.f};

    // first two tiles in flight, then the q^ fragments (B operand of the
    // score product; zeros for wavefronts past h), then the third tile
    {
        const size_t a0 = half_row(t0), a1 = half_row(t0 + 16);
        const size_t b0 = half_row(t0 + kT), b1 = half_row(t0 + kT + 16);
        issue_tile(t0, 0, a0, a1);
        issue_tile(t0 + kT, 1, b0, b1);
    }
    bf16x8 Qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
        Qf[ks] = active ? *(const bf16x8*)(p.qhat + ((size_t)b * p.h + head0 + li) * 576 + ks * 32 + 8 * G)
                        : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    vmem_drain();
    issue_tile(t0 + 2 * kT, 2, half_row(t0 + 2 * kT), half_row(t0 + 2 * kT + 16));

    const TileOffsets to(li, G);
    int buf = 0;
    for (int tb = t0; tb < t1; tb += kT) {
        const size_t nx0 = half_row(tb + 3 * kT), nx1 = half_row(tb + 3 * kT + 16);
        // tiles tb + T and tb + 2T were issued after this one
        if (wave < 4) wait_vmcnt<10>();
        else wait_vmcnt<8>();
        __syncthreads();
        // refill the buffer read in the previous iteration (every wavefront is
        // past it), so that three tiles stay in flight while this one is used
        issue_tile(tb + 3 * kT, (buf + 3) % kNBuf, nx0, nx1);
        const uint8_t* C = Cs + buf * kTile;
        if (active) {
            // ---- scores S^T = C . q^T
            f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            bf16x8 a[2][2];   // [K step parity][mt]
            a[0][0] = lds_read_16_as_2x8(to.score(C, 0, 0));
            a[0][1] = lds_read_16_as_2x8(to.score(C, 0, 1));
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                if (ks + 1 < KS) {
                    a[(ks + 1) & 1][0] = lds_read_16_as_2x8(to.score(C, ks + 1, 0));
                    a[(ks + 1) & 1][1] = lds_read_16_as_2x8(to.score(C, ks + 1, 1));
                }
#pragma unroll
                for (int mt = 0; mt < 2; mt++) S[mt] = mfma16(a[ks & 1][mt], Qf[ks], S[mt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- online softmax: lane holds head (head0 + li), tokens 16 mt + 4G + e.
            // The reference max m only moves when a tile's max exceeds it by
            // more than 8 (log2 units); otherwise probabilities up to 2^8 are
            // accumulated against the old m, which is exact after the final
            // division and spares rescaling the 512-wide accumulators.
            float z[2][4];
            float lm = -INFINITY;
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int tok = tb + 16 * mt + 4 * G + e;
                    z[mt][e] = tok < t1 ? S[mt][e] * p.scale_log2 : -INFINITY;
                    lm = fmaxf(lm, z[mt][e]);
                }
            lm = fmaxf(lm, xor16(lm));
            lm = fmaxf(lm, xor32(lm));
            const bool move = lm > m + 8.f;
            const float mn = move ? lm : m;
            const float alpha = move ? __builtin_amdgcn_exp2f(m - mn) : 1.f;
            m = mn;
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
            lsum = lsum * alpha + ps;
            const bf16x8 P = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
                for (int mc = 0; mc < MC; mc++) {
                    U[mc] *= alpha;
                    __builtin_amdgcn_sched_barrier(0);   // a few accumulators at a time
                }
            }
            // ---- latent sum U^T += C^T . P^T (transposing reads of the same tile)
            s16x4 lo[2], hi[2];
            lo[0] = lds_read_tr(to.value(C, 0, 0));
            hi[0] = lds_read_tr(to.value(C, 0, 1));
#pragma unroll
            for (int mc = 0; mc < MC; mc++) {
                if (mc + 1 < MC) {
                    lo[(mc + 1) & 1] = lds_read_tr(to.value(C, mc + 1, 0));
                    hi[(mc + 1) & 1] = lds_read_tr(to.value(C, mc + 1, 1));
                }
                U[mc] = mfma16(cat_tr(lo[mc & 1], hi[mc & 1]), P, U[mc]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        buf = (buf + 1) % kNBuf;
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup

    if (!active) return;
    // ---- partial state of this split: m, l per head, U^T columns
    float l = lsum;
    l += xor16(l);
    l += xor32(l);
    const size_t row = pbase + head0 + li;
    float* pu = p.part_u + row * 512 + 4 * G;
#pragma unroll
    for (int mc = 0; mc < MC; mc++)
        *(float4*)(pu + 16 * mc) = make_float4(U[mc][0], U[mc][1], U[mc][2], U[mc][3]);
    if (G == 0) {
        p.part_ml[row * 2] = m;
        p.part_ml[row * 2 + 1] = l;
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

    // W_UV fragments of this wavefront's first column tile, fetched now so
    // that their latency hides behind the merge
    const uint16_t* __restrict__ wuv = (const uint16_t*)p.w_uv + (size_t)i * p.d_v * p.d_c;
    bf16x8 bws[16];   // d_c = 512: 16 K steps
    if (wave < p.d_v / 16) {
        const uint16_t* wrow = wuv + (size_t)(wave * 16 + li) * p.d_c + 8 * G;
#pragma unroll
        for (int k = 0; k < 16; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
    }

    // merge: thread -> sequence r = tid / 16 of the block, 32 columns at
    // 32 * (tid % 16).  Pass 1 takes the largest split max over the splits
    // that saw tokens; pass 2 adds the partial sums, four splits' loads in
    // flight at once.  An empty split (l = 0) leaves its partial sum
    // unwritten: it is loaded (the workspace holds it) but never used.
    {
        const int r = tid / 16, cseg = (tid % 16) * 32, bb = b0 + r;
        float4 acc[8];
#pragma unroll
        for (int q = 0; q < 8; q++) acc[q] = make_float4(0.f, 0.f, 0.f, 0.f);
        float M = -INFINITY, L = 0.f;
        if (bb < p.B) {
            const float2* __restrict__ ml = (const float2*)p.part_ml;
            const size_t row0 = (size_t)bb * p.n_split * p.h + i;   // split k: row0 + k h
            for (int k0 = 0; k0 < p.n_split; k0 += 8) {
                float2 v[8];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (k0 + u < p.n_split) v[u] = ml[row0 + (size_t)(k0 + u) * p.h];
#pragma unroll
                for (int u = 0; u < 8; u++)
                    if (k0 + u < p.n_split && v[u].y > 0.f) M = fmaxf(M, v[u].x);
            }
            const float4* __restrict__ pu = (const float4*)p.part_u;
            for (int k0 = 0; k0 < p.n_split; k0 += 4) {
                float2 v[4];
                float4 u[4][8];
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (k0 + g < p.n_split) {
                        const size_t row = row0 + (size_t)(k0 + g) * p.h;
                        v[g] = ml[row];
#pragma unroll
                        for (int q = 0; q < 8; q++) u[g][q] = pu[(row * 512 + cseg) / 4 + q];
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; g++) {
                    if (k0 + g < p.n_split && v[g].y > 0.f) {
                        const float wk = __builtin_amdgcn_exp2f(v[g].x - M);
                        L = fmaf(wk, v[g].y, L);
#pragma unroll
                        for (int q = 0; q < 8; q++) {
                            acc[q].x = fmaf(wk, u[g][q].x, acc[q].x);
                            acc[q].y = fmaf(wk, u[g][q].y, acc[q].y);
                            acc[q].z = fmaf(wk, u[g][q].z, acc[q].z);
                            acc[q].w = fmaf(wk, u[g][q].w, acc[q].w);
                        }
                    }
                }
            }
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int q = 0; q < 8; q++) {
                acc[q].x *= inv; acc[q].y *= inv; acc[q].z *= inv; acc[q].w *= inv;
            }
            if (p.u_latent) {
                float4* dst = (float4*)(p.u_latent + ((size_t)bb * p.h + i) * 512 + cseg);
#pragma unroll
                for (int q = 0; q < 8; q++) dst[q] = acc[q];
            }
            if ((tid % 16) == 0 && p.lse)
                p.lse[(size_t)bb * p.h + i] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        }
#pragma unroll
        for (int q = 0; q < 8; q++) *(float4*)&Us[r][cseg + 4 * q] = acc[q];
    }
    __syncthreads();

    // out[b0 + m, i, n] = sum_c u~[m][c] W_UV[i][n][c]: M = 16 sequences,
    // N = d_v (wavefront w takes column tiles w, w+4, ...), K = d_c
    for (int nt = wave; nt < p.d_v / 16; nt += 4) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (nt != wave) {
            const uint16_t* wrow = wuv + (size_t)(nt * 16 + li) * p.d_c + 8 * G;
#pragma unroll
            for (int k = 0; k < 16; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
        }
#pragma unroll
        for (int k = 0; k < 16; k++) {
            const int k0 = 32 * k;
            const bf16x8 bw = bws[k];
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
    hipLaunchKernelGGL(mla_absorb_kernel, dim3(g1), dim3(256), smem1, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = (unsigned)(p.B * p.n_split);
    if (paged) {
        hipLaunchKernelGGL((mla_decode_fast_kernel<32, true>), dim3(g2), dim3(256), 0, st, p, p.bt);
        hipLaunchKernelGGL((mla_decode_safe_kernel<true>), dim3(g2), dim3(512), 0, st, p, p.bt);
    } else {
        hipLaunchKernelGGL((mla_decode_fast_kernel<32, false>), dim3(g2), dim3(256), 0, st, p, p.bt);
        hipLaunchKernelGGL((mla_decode_safe_kernel<false>), dim3(g2), dim3(512), 0, st, p, p.bt);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g3 = (unsigned)(p.h * ((p.B + 15) / 16));
    hipLaunchKernelGGL(mla_finish_kernel, dim3(g3), dim3(256), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
