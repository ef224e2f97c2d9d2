// MLA decode in the absorbed ("MQA mode") form on gfx950, bf16 MFMA with fp32
// accumulation.
//
// Steps, in the order of "Multi-Head Latent Attention (MLA): Mathematical
// Foundations ..." (llms.blog), sections "Attention Logit Matrix Absorption"
// and "Value Output Matrix Absorption", and "MLA: why one latent can replace a
// multi-head KV cache" (charlestar.github.io), "First matrix absorption" /
// "Second matrix absorption":
//   1. mla_absorb_kernel    q^[b,i] = [bf16(W_UK[i]^T q_nope[b,i]) | q_rope[b,i]]
//   2. mla_decode_kernel    per run of 32-token tiles, all heads at once:
//                           S = q^ C^T over the cached rows [c | k_R],
//                           softmax against a per-head reference max,
//                           u~ += P c  (same LDS tile)
//   3. mla_finish_kernel    merge the splits through their lse -> u~ (fp32),
//                           then out[b,i] = W_UV[i] u~[b,i]
// All h heads share every latent row, so the score [h x 576]x[576 x n] and
// value [h x n]x[n x 512] products are dense and run on the matrix cores;
// each latent row is fetched from HBM once per call.
#include <type_traits>

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
// the decode tile schedule (defined with the decode kernels below).  Its
// inputs are passed by value: a reference to the kernel's parameter block
// would force a copy of it into scratch memory for every wavefront.
struct SchedArgs {
    const int32_t* s;
    int32_t* sched;
    int B, s_max, n_wg, min_tiles, q_len;
};

// Query rows: row b is new-token position b % q_len of sequence b / q_len
// (q_len = 1: one row per sequence).  Its cache is that sequence's, and it
// sees the sequence's clamped length less the new tokens after it.
__device__ __forceinline__ int mla_cache_seq(int b, int q_len) { return q_len == 1 ? b : b / q_len; }
__device__ __forceinline__ int mla_seen(int s_b, int b, int q_len, int s_max)
{
    const int n = min(max(s_b, 0), s_max);
    return q_len == 1 ? n : max(n - (q_len - 1 - b % q_len), 0);
}
__device__ __forceinline__ void mla_schedule(SchedArgs p, int tid, int nthr, int* sc);

// q^ is stored in the order the decode kernel reads it as the B operand of
// its score product: wavefront g (heads 32 g .. 32 g + 31), K step ks (16
// dims), lane l (head 32 g + l % 32, dims 16 ks + 8 (l / 32) .. + 7) own
// the 16 bytes at ((b NG + g) 36 + ks) 64 + l, NG = ceil(h / 32).  Each
// 64-lane load is then one contiguous kilobyte; in the row-major
// [B, h, 576] order every load touched 32 rows and each 128-byte line was
// fetched four times.  Returns the bf16 index of dims d .. d + 7 (d a
// multiple of 8) of head i of sequence b.
__device__ __forceinline__ size_t qhat_index(int b, int i, int d, int h)
{
    const int ng = (h + 31) / 32;
    const int lane = i % 32 + 32 * ((d / 8) % 2);
    return ((((size_t)b * ng + i / 32) * 36 + d / 16) * 64 + lane) * 8;
}

constexpr int kAbsCols = 128;
constexpr int kAbsRowStride = kAbsCols * 2 + 16;

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// q_nope rows of one 16-sequence block as the A operand, K steps 0..KS-1.
// The loads are unconditional from clamped addresses and their values are
// not touched until the products use them, so all of them stay in flight
// together: K steps past d_nope / 32 are never multiplied, and rows past B
// (copies of row B - 1) only give result rows that are not stored.
template <int KS>
struct AbsA {
    bf16x8 k[KS];
};
template <int KS>
__device__ __forceinline__ AbsA<KS> absorb_load_a(const uint16_t* __restrict__ qn, int b0, int li, int G,
                                                  int B, int h, int i, int d_nope)
{
    AbsA<KS> a;
    const int ksteps = d_nope / 32;
    const int bc = min(b0 + li, B - 1);
#pragma unroll
    for (int k = 0; k < KS; k++) {
        const int kc = min(k, ksteps - 1);
        a.k[k] = *(const bf16x8*)(qn + ((size_t)bc * h + i) * d_nope + kc * 32 + 8 * G);
    }
    return a;
}

constexpr int kAbsMaxNope = 256;   // largest d_nope the staging area holds

// MAXN: the largest d_nope this instantiation stages (128 or 256).  The
// W_UK staging is a static allocation sized for it, so no per-kernel
// attribute is set at run time; the 128-row instantiation (34 KB) lets four
// workgroups share a CU, the 256-row one (68 KB) two.
template <int MAXN>
__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t smem[MAXN * kAbsRowStride];
    __shared__ __attribute__((aligned(16))) uint16_t ost[4][16][32 + 8];   // per-wavefront output staging
    // one extra workgroup, dispatched first so that its loads of the lengths
    // go out ahead of the W_UK stream: the decode tile schedule
    if (blockIdx.x == 0) {
        __shared__ int sc[256];
        mla_schedule(SchedArgs{p.s, p.sched, p.B, p.s_max, p.n_wg, p.min_tiles, p.q_len}, threadIdx.x, 256,
                     sc);
        return;
    }
    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int nq = p.d_c / kAbsCols;
    const int i = (blockIdx.x - 1) / nq, cq = (blockIdx.x - 1) % nq;
    const int c0 = cq * kAbsCols;
    const uint16_t* __restrict__ wuk = (const uint16_t*)p.w_uk + (size_t)i * p.d_nope * p.d_c;
    const uint16_t* __restrict__ qn = (const uint16_t*)p.q_nope;
    const int ksteps = p.d_nope / 32;
    constexpr int KS = MAXN / 32;

    // the first two 16-sequence blocks of q_nope, in flight with the W_UK
    // staging below (later blocks are fetched two blocks ahead)
    AbsA<KS> a0 = absorb_load_a<KS>(qn, 0, li, G, p.B, p.h, i, p.d_nope);
    AbsA<KS> a1 = absorb_load_a<KS>(qn, 16, li, G, p.B, p.h, i, p.d_nope);   // rows clamped to B - 1

    // stage W_UK[i][:, c0:c0+128]: d_nope rows x 16 chunks, 8 loads in flight
    // per thread; past the end, lanes load and store the last chunk again
    // (same place, same value), so nothing branches and the staging values
    // stay in registers
    const int nchunk = p.d_nope * (kAbsCols / 8);
    for (int base = 0; base < nchunk; base += 256 * 8) {
        u32x4v v[8];
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int idx = min(base + u * 256 + tid, nchunk - 1);
            const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
            v[u] = *(const u32x4v*)(wuk + (size_t)r * p.d_c + c0 + c * 8);
        }
#pragma unroll
        for (int u = 0; u < 8; u++) {
            const int idx = min(base + u * 256 + tid, nchunk - 1);
            const int r = idx / (kAbsCols / 8), c = idx % (kAbsCols / 8);
            *(u32x4v*)(smem + r * kAbsRowStride + c * 16) = v[u];
        }
    }
    // the rotary part of q^ is q_rope times the rotary scale of an FP8 cache
    // (a plain copy for bf16: the scale is 1); once per head, 16 bytes per
    // lane, four copies in flight; d_R is a multiple of 8
    if (cq == 0) {
        const int per = p.d_R / 8, nv = p.B * per;
        const uint16_t* __restrict__ qr = (const uint16_t*)p.q_rope;
        for (int base = 0; base < nv; base += 4 * 256) {
            u32x4v v[4];
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int idx = min(base + u * 256 + tid, nv - 1);
                v[u] = *(const u32x4v*)(qr + ((size_t)(idx / per) * p.h + i) * p.d_R + 8 * (idx % per));
            }
#pragma unroll
            for (int u = 0; u < 4; u++) {
                const int idx = min(base + u * 256 + tid, nv - 1);   // duplicates rewrite the same value
                u32x4v x = v[u];
                if (p.f8) {   // workgroup-uniform
#pragma unroll
                    for (int e = 0; e < 4; e++)
                        x[e] = pack_bf16x2(bf16lo_to_f32(x[e]) * p.r_scale, bf16hi_to_f32(x[e]) * p.r_scale);
                }
                *(u32x4v*)(p.qhat + qhat_index(idx / per, i, p.d_c + 8 * (idx % per), p.h)) = x;
            }
        }
    }

    __syncthreads();

    // wavefront w computes column tiles 2w and 2w+1 (32 columns) for every
    // 16-row block of b.  Blocks go in pairs: each one's registers are
    // refilled with the block two ahead as soon as it has been multiplied,
    // so the next pair's q_nope is in flight during this pair's work and no
    // register copy waits for a load.  The block's 16 x 32 results go through
    // LDS so that each lane stores 16 contiguous bytes.
    auto block = [&](const AbsA<KS>& a, int b0) {
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int nt = 2 * wave + t;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < KS; k++) {
                if (k < ksteps) {
                    const int row = k * 32 + 8 * G + li / 4;
                    const int col = nt * 16 + 4 * (li % 4);
                    const s16x4 lo = lds_read_tr(smem + row * kAbsRowStride + col * 2);
                    const s16x4 hi = lds_read_tr(smem + (row + 4) * kAbsRowStride + col * 2);
                    acc = mfma16(a.k[k], cat_tr(lo, hi), acc);
                }
            }
            // lane holds q~[b0 + 4G + e][c0 + 16 nt + li], times the latent
            // scale of an FP8 cache (1 for bf16)
#pragma unroll
            for (int e = 0; e < 4; e++)
                ost[wave][4 * G + e][16 * t + li] = (uint16_t)f32_to_bf16_bits(acc[e] * p.c_scale);
        }
        __syncthreads();
        {
            const int r = lane / 4, sg = lane % 4;   // row of the block, 16-byte segment
            const u32x4v v = *(const u32x4v*)&ost[wave][r][8 * sg];
            if (b0 + r < p.B)
                *(u32x4v*)(p.qhat + qhat_index(b0 + r, i, c0 + 32 * wave + 8 * sg, p.h)) = v;
        }
        __syncthreads();
    };
    // the first pair outside the loop: straight-line code, so the compiler's
    // waits there cover exactly the loads a block uses (a wait carried round
    // a loop would also drain the stores of the block before it)
    block(a0, 0);
    if (p.B > 32) a0 = absorb_load_a<KS>(qn, 32, li, G, p.B, p.h, i, p.d_nope);   // uniform
    if (p.B > 16) block(a1, 16);
    if (p.B > 48) a1 = absorb_load_a<KS>(qn, 48, li, G, p.B, p.h, i, p.d_nope);
    for (int b0 = 32; b0 < p.B; b0 += 32) {
        block(a0, b0);
        if (b0 + 32 < p.B) a0 = absorb_load_a<KS>(qn, b0 + 32, li, G, p.B, p.h, i, p.d_nope);
        if (b0 + 16 < p.B) block(a1, b0 + 16);
        if (b0 + 48 < p.B) a1 = absorb_load_a<KS>(qn, b0 + 48, li, G, p.B, p.h, i, p.d_nope);
    }
}

// ---------------------------------------------------------------------------
// 2. decode.  Workgroup = a run of tiles with all heads, so every latent
//    tile is fetched once.  Tiles of 32 rows move HBM -> LDS by LDS-DMA
//    (buffer_load ... lds, no staging registers) into a ring of 4 buffers,
//    three tiles ahead of use.  4 wavefronts (one per SIMD; the latent-sum
//    accumulators fill the 256 AGPRs of each):
//      scores   wavefront w, heads 32w .. 32w+31:
//               S^T[32 tok x 32 heads] = C_tile[32 x 576] . q^T
//               (v_mfma_f32_32x32x16_bf16, A: LDS, B: q^ in registers);
//      softmax  lane = head, 16 tokens per lane; P rounded to bf16;
//      exchange P of all heads through LDS (8 KB per tile);
//      latent   wavefront w, latent columns 128w .. 128w+127, all heads:
//               U^T[128 x 128] += C_tile^T[128 x 32] . P^T[32 x 128]
//               (A: transposing LDS reads of a quarter of the tile, B: P).
//    The 32 x 32 x 16 products halve the instruction count of the 16 x 16 x
//    32 ones for the same work, and a wavefront's 16 score registers then
//    cost as much as its 16 heads x 32 tokens did before.  The score chain
//    keeps its accumulator in VGPRs (the AGPRs hold U), which the compiler's
//    MFMA forms cannot express, so it is issued as inline assembly with the
//    wait states the hardware requires around it.
//    The value product's K order is the score product's output order: lane
//    half hh of head j holds tokens 8g + 4hh + e (g < 4, e < 4); K step kk
//    takes g = 2kk, 2kk + 1, so P keeps the layout it was computed in, and
//    the transposing reads of C fetch those two groups of 4 rows.
//
//    LDS tile layout (one buffer, 36 KB): 9 segments of 128 bytes per row,
//    segment-major: byte (s * 4096 + r * 128 + 16 * p) holds row r, 16-byte
//    chunk 8 s + (p ^ swz(r)).  One DMA instruction fills 8 rows of one
//    segment (1 KB, lane-contiguous as the hardware writes it).  The XOR
//    swizzle spreads the rows of an operand over the banks.
//
//    Completion of the LDS-DMA is tracked with explicit vmcnt waits, so no
//    other vector-memory instruction may be outstanding inside the tile loop
//    (a compiler-inserted vmcnt(0) for it would also drain the prefetched
//    tiles): q^ is loaded and waited for before the loop, and the loop keeps
//    its state in registers (no spills).
// ---------------------------------------------------------------------------
constexpr int kT = 32;             // tokens per tile
constexpr int kNBuf = 4;           // LDS ring depth

// Tile geometry by cache format.  bf16: 9 segments of 128 bytes per row,
// one DMA instruction = 8 rows of a segment.  E4M3 (576-byte rows): 9
// segments of 64 bytes, one DMA instruction = 16 rows of a segment.
template <bool F8>
struct MlaTile {
    static constexpr int ROW = F8 ? 576 : 1152;       // bytes per cached row
    static constexpr int TILE = kT * ROW;             // bytes per tile
    static constexpr int SLOTS = TILE / 1024;         // DMA instructions per tile
    static constexpr int SEG = F8 ? 64 : 128;         // bytes per row segment
    static constexpr int RPS = 1024 / SEG;            // rows per DMA instruction
    static constexpr int SPS = kT / RPS;              // DMA instructions per segment
};

// XOR swizzle of the 16-byte chunk position within a 128-byte row segment.
// The LDS has 64 four-byte banks and serves 16 lanes of a 16-byte read (32
// lanes of an 8-byte one) per cycle, so a 16-lane group must cover all 64
// banks: a row's banks start at 32 (r % 2), so the rows of each parity
// among 16 consecutive ones need distinct positions.  With u = (r / 2) mod 8,
// s(r) = 4 (u % 2) + u / 2 does that, and rows 4k and 4k + 2 (4k + 1 and
// 4k + 3) differ in bit 2, so the transposing reads of 4 rows x 32 bytes
// per 32-lane group hit 64 distinct banks too.  Measured with an LDS probe:
// the score pattern under the previous swizzle (any 8 consecutive rows
// distinct) ran at half rate once 8 wavefronts per CU were reading.
__device__ __forceinline__ int swz(int r)
{
    const int u = (r >> 1) & 7;
    return ((u & 1) << 2) | (u >> 1);
}

// Per-lane byte offsets of the MFMA operands within a tile buffer, split so
// that everything depending on the K step or the column tile is a
// compile-time constant (the immediate offset of the LDS instruction).
//   score operand, K step ks: row l % 32, chunk 2 ks + hh (hh = l / 32)
//     = (ks >> 2) * 4096 + [r * 128 + ((2 (ks & 3) + hh) ^ swz(r)) * 16]
//   value operand of wavefront w, column tile mc, K step kk, read t (rows
//     16 kk + 8 t + 4 hh + i / 4 of 16-lane group q, i = l % 16, hh = q / 2):
//     column 128 w + 32 mc + 16 (q % 2) + 4 (i % 4), i.e. chunk
//     16 w + 4 mc + 2 (q % 2) + (i % 4) / 2, byte 8 (i % 2) within it
//     = (2 w + mc / 2) * 4096 + kk * 2048 + [row * 128 + ((4 (mc & 1) + ...) ^ swz(row)) * 16 + 8 (i % 2)]
struct TileOffsets {
    int sc[4];      // score, by ks & 3
    int tr[2][2];   // value, by (mc & 1, t)
    __device__ __forceinline__ TileOffsets(int lane)
    {
        const int r = lane % 32, hh = lane / 32, s = swz(r);
#pragma unroll
        for (int j = 0; j < 4; j++) sc[j] = r * 128 + (((2 * j + hh) ^ s) << 4);
        const int q = lane / 16, i = lane % 16;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const int row = 8 * t + 4 * (q / 2) + i / 4, st = swz(row);
#pragma unroll
            for (int m1 = 0; m1 < 2; m1++)
                tr[m1][t] = row * 128 + (((4 * m1 + 2 * (q % 2) + (i % 4) / 2) ^ st) << 4) + 8 * (i % 2);
        }
    }
    __device__ __forceinline__ const uint8_t* score(const uint8_t* C, int ks) const
    {
        return C + sc[ks & 3] + (ks >> 2) * 4096;
    }
    __device__ __forceinline__ const uint8_t* value(const uint8_t* C, int w, int mc, int kk, int t) const
    {
        return C + tr[mc & 1][t] + (2 * w + (mc >> 1)) * 4096 + kk * 2048;
    }
};

// E4M3 tiles (576-byte rows in 64-byte segments: byte s * 2048 + r * 64 +
// 16 p holds row r, 16-byte chunk 4 s + (p ^ swz8(r))).
//   swz8(r) = (r >> 2) & 3
// Score operands: a lane reads one whole chunk (16 codes) per pair of K
// steps: lane (row r = l % 32, hh = l / 32) reads chunk 2 j + hh, whose
// first 8 codes are its operand of step 2 j and the last 8 of step 2 j + 1
// (the K order inside a step is free as long as q^ follows it).  A row's
// banks start at 16 (r % 4), so the 16 rows of a 16-lane group need distinct
// positions within each residue mod 4: rows c, c + 4, c + 8, c + 12 get
// positions 0 .. 3.
// Value operands: an 8-bit transposing read per (column tile, K step).  In
// 16-lane group q (= l / 16), source lane i reads 8 bytes of row
// 16 kk + tau(q / 2, i / 2), columns 128 w + 32 mc + 16 (q % 2) + 8 (i % 2),
// with tau(hh, k) = 4 hh + k for k < 4 and 4 hh + k + 4 otherwise -- the
// score output's token order; the read hands lane 8 a + c byte c of source
// lanes a, a + 2, .., a + 14, i.e. column 16 (q % 2) + 8 a + c for its 8
// tokens.  Rows {0-3, 8-11} and {4-7, 12-15} each cover the 64 banks (rows r
// and r + 8 differ in bit 1 of their position).
__device__ __forceinline__ int swz8(int r) { return (r >> 2) & 3; }

struct TileOffsets8 {
    int sc[2];   // score, by j & 1
    int tr[2];   // value, by mc & 1
    __device__ __forceinline__ TileOffsets8(int lane)
    {
        const int r = lane % 32, hh = lane / 32, s = swz8(r);
#pragma unroll
        for (int j = 0; j < 2; j++) sc[j] = r * 64 + (((2 * j + hh) ^ s) << 4);
        const int q = lane / 16, i = lane % 16, k = i / 2;
        const int row = 4 * (q / 2) + (k < 4 ? k : k + 4), st = swz8(row);
#pragma unroll
        for (int m1 = 0; m1 < 2; m1++) tr[m1] = row * 64 + (((2 * m1 + q % 2) ^ st) << 4) + 8 * (i % 2);
    }
    __device__ __forceinline__ const uint8_t* score(const uint8_t* C, int j) const
    {
        return C + sc[j & 1] + (j >> 1) * 2048;
    }
    __device__ __forceinline__ const uint8_t* value(const uint8_t* C, int w, int mc, int kk) const
    {
        return C + tr[mc & 1] + (2 * w + (mc >> 1)) * 2048 + kk * 1024;
    }
};

// Score products with the accumulator in VGPRs.  Each instruction is
// preceded by two wait states (a VALU write of an operand register needs
// them before a matrix instruction reads it), and the last one of a chain is
// followed by 20, more than an 8-pass XDL result needs before a VALU reads
// it.  Back-to-back accumulation into the same registers needs none.
__device__ __forceinline__ f32x16 mfma32_first(bf16x8 a, bf16x8 b)
{
    f32x16 d;
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ void mfma32_acc(f32x16& d, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_last(f32x16& d, bf16x8 a, bf16x8 b)
{
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 3"
                 : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Variable-length tile schedule.  The cached tiles of all sequences are laid
// end to end, sequence-major: tile_start[b] is the first tile of sequence b
// and tile_start[B] the total.  Decode workgroup w takes tiles
// [w tpw, (w + 1) tpw), so every workgroup gets the same amount of cache
// whatever the mix of lengths, crossing sequence boundaries where it must.
// It leaves one partial (m, l, u~) per sequence it touches, in slot w + b:
// along the tile order each step to the next (workgroup, sequence) pair
// raises w, b or both, so w + b never repeats and n_wg + B - 1 slots do.
// This is the tile-scheduler metadata that "MLA: why one latent can replace
// a multi-head KV cache" (charlestar.github.io) puts next to the paged
// cache in the section on what FlashMLA solves, computed here on the device
// from the device-resident lengths.
// Workspace layout (int32): tile_start [B + 1], wstart [n_wg] (sequence of
// each workgroup's first tile, -1 when it has none), tpw [1].
// ---------------------------------------------------------------------------
// Read-only views of the lengths and the schedule.  The kernels take them as
// separate restrict parameters, so that these wave-uniform reads become
// scalar loads: a vector load inside the tile loop would make the compiler
// wait for every outstanding vector-memory operation, DMA included.
// Every value taken from the schedule is clamped into range, so that even a
// workspace whose schedule was overwritten cannot steer an access outside the
// lengths, the table, the pool or the partial slots.
struct SchedView {
    const int32_t* __restrict__ s;       // lengths [B / q_len]
    const int32_t* __restrict__ sched;   // tile_start [B + 1], wstart [n_wg], tpw
    int s_max, B, n_wg, q_len;
    __device__ __forceinline__ int len(int b) const
    {
        return mla_seen(__builtin_amdgcn_readfirstlane(s[mla_cache_seq(b, q_len)]), b, q_len, s_max);
    }
    __device__ __forceinline__ int at(int i) const { return __builtin_amdgcn_readfirstlane(sched[i]); }
    __device__ __forceinline__ int total() const
    {
        return min(max(at(B), 0), B * ((s_max + kT - 1) / kT));
    }
    __device__ __forceinline__ int tpw(int tot) const { return min(max(at(B + 1 + n_wg), 1), max(tot, 1)); }
    __device__ __forceinline__ int first_seq(int w) const { return min(max(at(B + 1 + w), 0), B - 1); }
};

// Computed by one workgroup of nthr threads (a multiple of 64, at most 1024);
// sc is nthr ints of LDS.  Thread t takes rows E t .. E t + E - 1 of each
// chunk of E nthr rows, so one round trip to memory brings the lengths of up
// to E nthr rows, which stay in registers for both passes: the first totals
// the tiles (which fixes tpw), the second scans them (within a thread, then
// across wavefronts through LDS) and writes the tile offsets and each
// workgroup's first sequence.  Only longer batches load their lengths again
// per chunk.  No thread reads back what another wrote to global memory.
__device__ __forceinline__ void mla_schedule(SchedArgs p, int tid, int nthr, int* sc)
{
    constexpr int E = 4;
    int32_t* ts = p.sched;
    int32_t* wstart = p.sched + p.B + 1;
    const int lane = tid % 64, wv = tid / 64, nwv = nthr / 64;
    const int per = E * nthr;   // rows per chunk
    auto load = [&](int base, int* tl) {
        int len[E];
#pragma unroll
        for (int k = 0; k < E; k++)   // unconditional, all E loads in flight together
            len[k] = p.s[mla_cache_seq(min(base + E * tid + k, p.B - 1), p.q_len)];
#pragma unroll
        for (int k = 0; k < E; k++) {
            const int i = base + E * tid + k;
            const int t = (mla_seen(len[k], i, p.q_len, p.s_max) + kT - 1) / kT;
            tl[k] = i < p.B ? t : 0;
        }
    };
    // sum over the workgroup (sc[0 .. nwv - 1] hold the wavefront totals)
    auto block_total = [&](int x) {
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
        __syncthreads();
        if (lane == 0) sc[wv] = x;
        __syncthreads();
        int t = 0;
        for (int v = 0; v < nwv; v++) t += sc[v];
        return t;
    };
    int tl[E];
    load(0, tl);
    int part = 0;
#pragma unroll
    for (int k = 0; k < E; k++) part += tl[k];
    for (int base = per; base < p.B; base += per) {   // batches of more than E nthr rows
        int tx[E];
        load(base, tx);
#pragma unroll
        for (int k = 0; k < E; k++) part += tx[k];
    }
    const int total = block_total(part);
    const int tpw = max((total + p.n_wg - 1) / p.n_wg, p.min_tiles);
    // pass 2: offsets; workgroup w starts at tile w tpw, inside exactly one
    // non-empty sequence
    int carry = 0;
    for (int base = 0; base < p.B; base += per) {
        if (base > 0) load(base, tl);
        int mine = 0;
#pragma unroll
        for (int k = 0; k < E; k++) mine += tl[k];
        const int incl = wave_scan_incl(mine);
        __syncthreads();   // sc free again
        if (lane == 63) sc[wv] = incl;
        __syncthreads();
        int before = 0, chunk = 0;
        for (int v = 0; v < nwv; v++) {
            before += v < wv ? sc[v] : 0;
            chunk += sc[v];
        }
        int a = carry + before + incl - mine;
#pragma unroll
        for (int k = 0; k < E; k++) {
            const int i = base + E * tid + k;
            if (i < p.B) {
                ts[i] = a;
                for (int w = (a + tpw - 1) / tpw; w * tpw < a + tl[k]; w++) wstart[w] = i;
            }
            a += tl[k];
        }
        carry += chunk;
    }
    if (tid == 0) {
        ts[p.B] = total;
        wstart[p.n_wg] = tpw;
    }
    for (int w = (total + tpw - 1) / tpw + tid; w < p.n_wg; w += nthr) wstart[w] = -1;
}

// A position in a workgroup's tile stream: sequence b, its tile lt of nt,
// its clamped length n; g is the global tile index, past the stream once
// g >= g1 (tiles issued there move nothing).
struct TileWalk {
    int b, lt, nt, n, g, g1;
    __device__ __forceinline__ TileWalk(const SchedView& v, int b0, int g0, int g1_)
        : b(b0), g(g0), g1(g1_)
    {
        const int s0 = v.at(b0), s1 = v.at(b0 + 1);
        nt = max(s1 - s0, 1);
        lt = min(max(g0 - s0, 0), nt - 1);
        n = v.len(b0);
    }
    __device__ __forceinline__ bool past() const { return g >= g1; }
    __device__ __forceinline__ void next(const SchedView& v)
    {
        ++g;
        if (++lt < nt || g >= g1) return;
        // the next sequence with tiles (one lies ahead while g < g1); never past B - 1
        int s0 = 0, s1 = v.at(b + 1);
        while (b + 1 < v.B) {
            ++b;
            s0 = s1;
            s1 = v.at(b + 1);
            if (s1 != s0) break;
        }
        lt = 0;
        nt = max(s1 - s0, 1);
        n = v.len(b);
    }
};

// DMA of one tile (bf16: 36 slots of 8 rows x 128 bytes, slot q filling
// segment q / 4, rows 8 (q % 4) .. + 7; E4M3: 18 slots of 16 rows x 64
// bytes, slot q filling segment q / 2, rows 16 (q % 2) .. + 15; spread over
// the wavefronts) and the physical rows of its two 16-row halves.  A tile's halves each lie in one
// block of a paged pool (blocks hold a power of two >= 16 rows).  With NW a
// multiple of 4 a wavefront's slots all cover the same rows (q % SPS =
// wave % SPS), so one buffer resource per tile serves all of them and a slot
// differs only in its segment's byte offset and LDS destination.
template <int NW, bool PAGED, bool F8>
struct TileDma {
    using TL = MlaTile<F8>;
    static_assert(NW % TL::SPS == 0, "a wavefront's slots must share their rows");
    static constexpr int kSlots = TL::SLOTS;
    static constexpr int kRow = TL::ROW;
    static constexpr int SPW = kSlots / NW + (kSlots % NW ? 1 : 0);   // slots per wavefront
    const MlaParams& p;
    const int32_t* __restrict__ btab;
    const uint8_t* __restrict__ cbase;
    uint32_t lds0, vbase;
    int wave, rb;
    __device__ __forceinline__ TileDma(const MlaParams& p_, const int32_t* __restrict__ bt,
                                       uint32_t lds, int wave_, int lane)
        : p(p_), btab(bt), cbase((const uint8_t*)p_.cache), lds0(lds), wave(wave_), rb(wave_ % TL::SPS)
    {
        constexpr int PPS = TL::SEG / 16;   // 16-byte positions per segment
        const int lr = lane / PPS, lp = lane % PPS;   // row of the RPS, 16-byte position in the segment
        const int sw = F8 ? swz8(TL::RPS * rb + lr) : swz(TL::RPS * rb + lr);
        vbase = (uint32_t)(lr * kRow + 16 * (lp ^ sw));
    }
    __device__ __forceinline__ size_t half_row(int b, int t) const
    {
        const int cb = mla_cache_seq(b, p.q_len);
        if (PAGED) return paged_row(btab, cb, t, p.max_blocks, p.bs_log2, p.num_blocks);
        return (size_t)cb * p.s_max + t;
    }
    __device__ __forceinline__ void rows(const TileWalk& c, size_t& r0, size_t& r1) const
    {
        if (c.past()) {
            r0 = r1 = 0;
            return;
        }
        const int t0 = c.lt * kT;
        if (PAGED) {   // both table entries requested before either is used: one round trip
            const int32_t* __restrict__ row = btab + (size_t)mla_cache_seq(c.b, p.q_len) * p.max_blocks;
            const int e0 = row[min(t0 >> p.bs_log2, p.max_blocks - 1)];
            const int e1 = row[min((t0 + 16) >> p.bs_log2, p.max_blocks - 1)];
            const int m = (1 << p.bs_log2) - 1;
            const int b0 = min(max(__builtin_amdgcn_readfirstlane(e0), 0), p.num_blocks - 1);
            const int b1 = min(max(__builtin_amdgcn_readfirstlane(e1), 0), p.num_blocks - 1);
            r0 = ((size_t)b0 << p.bs_log2) + (t0 & m);
            r1 = ((size_t)b1 << p.bs_log2) + ((t0 + 16) & m);
            return;
        }
        r0 = half_row(c.b, t0);
        r1 = half_row(c.b, t0 + 16);
    }
    // A tile's DMA, prepared (buffer resource and LDS base, wave-uniform)
    // and then issued one instruction at a time, so that the issue can be
    // spread between other work.
    struct Pending {
        rsrc_t rs;
        uint32_t lb;
    };
    __device__ __forceinline__ Pending prepare(const TileWalk& c, int buf, size_t row0, size_t row1) const
    {
        // first row of this wavefront's RPS rows (a 16-row half lies in one block)
        const size_t row = F8 ? (rb == 0 ? row0 : row1) : (rb < 2 ? row0 : row1) + 8 * (rb & 1);
        const int t0 = c.lt * kT + TL::RPS * rb;                      // its token index
        const int nr = c.past() ? 0 : max(0, min(TL::RPS, c.n - t0)) * kRow;   // rows past the length read 0
        return Pending{make_rsrc(cbase + row * kRow, nr), lds0 + (uint32_t)(buf * TL::TILE)};
    }
    // instruction j < SPW of this wavefront's share
    __device__ __forceinline__ void issue_slot(const Pending& pd, int j) const
    {
        const int q = wave + NW * j;
        if (kSlots % NW == 0 || q < kSlots)   // wave-uniform, static when NW divides the slots
            dma16(pd.rs, vbase + (uint32_t)TL::SEG * (uint32_t)(q / TL::SPS), pd.lb + (uint32_t)q * 1024u);
    }
    __device__ __forceinline__ void issue(const TileWalk& c, int buf, size_t row0, size_t row1) const
    {
        const Pending pd = prepare(c, buf, row0, row1);
#pragma unroll
        for (int j = 0; j < SPW; j++) issue_slot(pd, j);
    }
    // tiles tb + T and tb + 2T were issued after tile tb
    __device__ __forceinline__ void wait_tile() const
    {
        if (SPW * NW == kSlots || wave < kSlots % NW) wait_vmcnt<2 * SPW>();
        else wait_vmcnt<2 * (SPW - 1)>();
    }
};

// PS (E4M3 pages with their own scale pair): the scores are summed as
// q~ . c + rho q_R . k_R with rho = r_scale / c_scale of the token's page
// folded into the widened rotary codes, then scaled by the page's c_scale;
// the probabilities that weight the latent sum carry c_scale too (the sums l
// do not), so U / l comes out in value units.  The scales of a tile's two
// 16-row halves are looked up when its DMA is issued and wait in LDS.
template <bool PAGED, bool F8, bool PS = false>
__global__ __launch_bounds__(256) void mla_decode_kernel(const MlaParams p,
                                                         const int32_t* __restrict__ btab,
                                                         const int32_t* __restrict__ slen,
                                                         const int32_t* __restrict__ sched,
                                                         const float* __restrict__ cscl,
                                                         const float* __restrict__ rscl)
{
    static_assert(!PS || (PAGED && F8), "page scales come with a paged E4M3 pool");
    constexpr int NW = 4;           // wavefronts per workgroup
    constexpr int KS = 576 / 16;    // score K steps
#ifndef MLA_PD
#define MLA_PD 4
#endif
    // score operands read ahead of their product (bf16); one fewer over a
    // paged pool, whose block-table walk needs registers of its own
    constexpr int PD = PAGED ? MLA_PD - 1 : MLA_PD;
#ifndef MLA_NU1
#define MLA_NU1 0
#endif
#ifndef MLA_NU1_F8
#define MLA_NU1_F8 16
#endif
    // latent-sum products of the previous tile issued between the score
    // products (the others run beside the softmax).  bf16 tiles: none -- the
    // score chain then runs alone (1,770 cycles a tile against 2,220 with 16
    // interleaved) and all 32 cover the softmax (1,460 against 1,200 cycles):
    // 5 % fewer cycles a tile.  E4M3 tiles measured faster with 16.
    constexpr int NU1 = F8 ? MLA_NU1_F8 : MLA_NU1;
    constexpr int MCW = 4;          // 32-column tiles of the latent sum per wavefront
    constexpr int NTH = 4;          // 32-head tiles of the latent sum (all heads; zeros past h)
#ifndef MLA_SCH
#define MLA_SCH 1
#endif
    constexpr int SCH = MLA_SCH;    // score accumulation chains (1 or 2)
    static_assert((NU1 == 0 || NU1 == 8 || NU1 == 16 || NU1 == 32) && (SCH == 1 || SCH == 2), "interleave");
    using TL = MlaTile<F8>;
    __shared__ __attribute__((aligned(1024))) uint8_t Cs[kNBuf * TL::TILE];
    // P of every head tile in B-operand layout, for two tiles: the value
    // product of tile g - 1 reads one buffer while the softmax of tile g
    // writes the other, so one barrier per tile orders both
    __shared__ __attribute__((aligned(16))) bf16x8 Pb[2][NTH][2][64];
    // partial-write staging of E4M3 tiles (bf16 tiles use a free ring buffer)
    __shared__ __attribute__((aligned(16))) uint8_t Stg8[F8 ? 4 * 32 * 272 : 16];
    // page scales of the tiles in the ring: [c half 0, c half 1, r half 0, r half 1]
    __shared__ __attribute__((aligned(16))) float Scl[PS ? kNBuf * 4 : 4];

    const int tid = threadIdx.x, lane = tid % 64, hh = lane / 32;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int w = xcd_major(blockIdx.x, gridDim.x);
    const SchedView sv{slen, sched, p.s_max, p.B, p.n_wg, p.q_len};
    const int total = sv.total();
    const int tpw = sv.tpw(total);
    const long long g0l = (long long)w * tpw;
    const int g0 = (int)min(g0l, (long long)total), g1 = min(g0 + tpw, total);
    if (g0 >= g1) {
        if (tid == 0) p.flags[w] = 0;
        return;
    }
    const int hs = 32 * wave + lane % 32;   // this lane's score head
    const bool hv = hs < p.h;

    const TileDma<NW, PAGED, F8> dma(p, btab, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Cs,
                                 wave, lane);
    // the page scales of the tile whose rows are r0, r1, for ring slot `slot`
    // (read by the step that scores it, after a barrier)
    auto note_scales = [&](int slot, bool past, size_t r0, size_t r1) {
        if constexpr (PS) {
            if (!past) {
                const int b0 = (int)(r0 >> p.bs_log2), b1 = (int)(r1 >> p.bs_log2);
                const float4 v = make_float4(cscl[b0], cscl[b1], rscl[b0], rscl[b1]);
                if (tid == 0) *(float4*)&Scl[4 * slot] = v;
            }
        }
    };
    TileWalk ic(sv, sv.first_seq(w), g0, g1);   // issue cursor
    TileWalk cc = ic;                            // compute cursor (the tile being scored)

    // q^ fragments of one sequence: B operand of the score product (heads
    // past h read as zeros)
    // An E4M3 tile feeds steps 2j and 2j + 1 from one chunk per lane (see
    // TileOffsets8): lane half hh takes dims 16 (2j + hh) .. + 7 at step 2j
    // and the next 8 at step 2j + 1, so q^ is read in that order.
    bf16x8 Qf[KS];
    // (dims d = 32 (ks / 2) + 16 hh + 8 (ks % 2): in the q^ layout that is
    // the element at qhat_index(b, i, 16 hh) + 1024 (ks / 2) + 256 (ks % 2))
    auto load_q = [&](int b) {
        const uint16_t* qrow = p.qhat + qhat_index(b, min(hs, p.h - 1), F8 ? 16 * hh : 8 * hh, p.h);
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
            const int off = F8 ? 1024 * (ks / 2) + 256 * (ks % 2) : 512 * ks;
            Qf[ks] = hv ? *(const bf16x8*)(qrow + off) : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
    };

    // Per head and sequence: m is the reference max (log2 units), fixed at
    // the first tile, and U, lsum accumulate 2^(z - m).  A later tile may
    // exceed m by up to 64 (p <= 2^64 stays far from fp32/bf16 overflow);
    // rescaling the AGPR-resident U in place would cost the loop its
    // register allocation, so past that the wavefront only notes it: after
    // the loop the workgroup flags itself, and the merge kernel recomputes
    // all of its partials exactly (the partials it wrote are never read).
    // Real logits essentially never get there.  m and lsum belong to this
    // lane's score head, U to the wavefront's latent columns (all heads).
    f32x16 U[MCW][NTH];
    float m, lsum;
    int ovf_w = 0;   // wave-uniform: some score of this wavefront's heads ran past m + 64
    auto reset = [&]() {
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int mc = 0; mc < MCW; mc++)
#pragma unroll
            for (int nt = 0; nt < NTH; nt++)
#pragma unroll
                for (int v = 0; v < 16; v++) U[mc][nt][v] = 0.f;
    };
    // partial state of sequence b, slot w + b: (m, l) of the score heads and
    // the U^T columns 128 wave .. + 127 of every head.
    // U / l is a weighted mean of cached latents, so it is stored as fp16
    // (2^-11 relative), halving the partial traffic of fp32 sums.  The sums l
    // of all heads go through LDS (the second P buffer) to the wavefronts
    // holding their columns.  Vector arithmetic on the AGPR-resident U would
    // cost the tile loop its register allocation, so U leaves through LDS:
    // per round (a head tile and 64 of the wavefront's columns) each
    // wavefront stores its accumulators as they are into its own staging
    // rows [32 heads][64 columns] fp32 (rows padded to 272 bytes, so that 16
    // lanes' 16-byte accesses fall in distinct banks), reads back 8
    // consecutive columns of one head per lane, scales them by 1 / l,
    // converts them and writes 16 contiguous bytes: 8 lanes cover one head's
    // 128 bytes of the round.  The staging area is the ring buffer of the
    // last scored tile (free once every wavefront has passed the first
    // barrier below; the next refill of it is issued after this returns),
    // or a separate area for E4M3 tiles, which are smaller than it.
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(1))) h8 gh8;
    float* const Lx = (float*)&Pb[1][0][0][0];   // NTH * 32 sums
    constexpr int kStgRow = 272, kStgWave = 32 * kStgRow;
    auto write_partial = [&](int b, uint8_t* stage) {
        const float l = lsum + xor32(lsum);
        __syncthreads();   // every wavefront is done with both P buffers and the staging buffer
        if (hh == 0) {
            Lx[hs] = l;
            if (hv) {
                const size_t row = (size_t)(w + b) * p.h + hs;
                p.part_ml[row * 2] = m;
                p.part_ml[row * 2 + 1] = l;
            }
        }
        __syncthreads();   // Lx written
        uint8_t* const st = stage + wave * kStgWave;
#pragma unroll
        for (int nt = 0; nt < NTH; nt++) {
#pragma unroll
            for (int half = 0; half < 2; half++) {
                // accumulator lane l, register 4 gq + e holds head 32 nt + l % 32,
                // column 32 mc + 8 gq + 4 (l / 32) + e of the wavefront's 128
#pragma unroll
                for (int mm = 0; mm < 2; mm++)
#pragma unroll
                    for (int gq = 0; gq < 4; gq++) {
                        const f32x16& u = U[2 * half + mm][nt];
                        *(float4*)(st + (lane % 32) * kStgRow + (32 * mm + 8 * gq + 4 * hh) * 4) =
                            make_float4(u[4 * gq], u[4 * gq + 1], u[4 * gq + 2], u[4 * gq + 3]);
                    }
                __builtin_amdgcn_sched_barrier(0);
                // the round's output base, opaque to the compiler: computed
                // here, it is not hoisted out of the tile loops into a
                // register that would be spilled and reloaded (a reload
                // waits for every outstanding store of the round before)
                uint64_t obase = (uint64_t)(uintptr_t)(p.part_u + ((size_t)(w + b) * p.h + 32 * nt) * 512 +
                                                       128 * wave + 64 * half);
                asm volatile("" : "+s"(obase));
#pragma unroll 1
                for (int r = 0; r < 4; r++) {
                    const int q = 64 * r + lane, hd = q / 8, c8 = q % 8;
                    const float4 x0 = *(const float4*)(st + hd * kStgRow + c8 * 32);
                    const float4 x1 = *(const float4*)(st + hd * kStgRow + c8 * 32 + 16);
                    const int head = 32 * nt + hd;
                    const float lh = Lx[head];
                    const float il = lh > 0.f ? __builtin_amdgcn_rcpf(lh) : 0.f;
                    const h8 v = {(_Float16)(x0.x * il), (_Float16)(x0.y * il), (_Float16)(x0.z * il),
                                  (_Float16)(x0.w * il), (_Float16)(x1.x * il), (_Float16)(x1.y * il),
                                  (_Float16)(x1.z * il), (_Float16)(x1.w * il)};
                    // a global-space pointer: a generic one would make these
                    // flat stores, and with a flat operation outstanding the
                    // compiler's wait counting cannot tell LDS results apart,
                    // so it drains every LDS read of the score chain
                    if (head < p.h) ((gh8*)(uintptr_t)obase)[hd * 64 + c8] = v;   // 512 halves a row
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();   // P buffers and staging are reused next
    };
    reset();

    // two tiles in flight, then q^ of the first sequence, then the third tile
    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 0, r0, r1);
        note_scales(0, ic.past(), r0, r1);
        ic.next(sv);
        dma.rows(ic, r0, r1);
        dma.issue(ic, 1, r0, r1);
        note_scales(1, ic.past(), r0, r1);
        ic.next(sv);
    }
    load_q(cc.b);
    vmem_drain();
    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 2, r0, r1);
        note_scales(2, ic.past(), r0, r1);
        ic.next(sv);
    }

    const TileOffsets to(lane);
    const TileOffsets8 to8(lane);
    const float sc = p.scale_log2;

    // Latent-sum operands of the last scored tile (its transposing reads,
    // taken right after its scores), used by the next step's value products.
    // E4M3 tiles keep the raw codes (half the registers) and widen them
    // just before each product.
    bf16x8 av[2][F8 ? 1 : MCW];
    uint2 av8[2][F8 ? MCW : 1];

    // The tile ring: wait until this wavefront's share of the tile in
    // buffer `buf` has landed, then a barrier (everyone's share landed, and
    // every wavefront is past the previous step, so the buffer read there
    // can be refilled and the P it wrote is visible), then refill that
    // buffer three tiles ahead.  The refill's instructions go out one by one
    // between the score products of the step, where the wavefront would
    // otherwise wait on the matrix core, instead of stalling here while the
    // load unit takes them.
    using Dma = TileDma<NW, PAGED, F8>;
    typename Dma::Pending pend;
    auto tile_top = [&](int buf) {
        size_t nx0, nx1;   // rows of the tile issued below, looked up early
        dma.rows(ic, nx0, nx1);
        dma.wait_tile();
        __syncthreads();
        pend = dma.prepare(ic, (buf + 3) % kNBuf, nx0, nx1);   // issued during the step's products
        note_scales((buf + 3) % kNBuf, ic.past(), nx0, nx1);
        ic.next(sv);
    };

    // One step of the pipeline.  With DS: the score product of the tile in
    // C (rows from tbase), its softmax into P buffer pw, and its latent-sum
    // operands into av.  With DV: the latent-sum product of the previous
    // tile, from av and P buffer pr.  The two products' instructions are
    // interleaved -- two score accumulation chains alternating, with one
    // value product after every second score product -- so the matrix core
    // always has an independent product to start; the rest of the value
    // products run beside the softmax.
    auto step = [&](auto DS, auto DV, const uint8_t* C, int tbase, int n, int pr, int pw, int slot) {
        constexpr bool do_s = decltype(DS)::value, do_v = decltype(DV)::value;
        // page scales of the scored tile (PS): c of each half, and this
        // lane's rho (its A-operand row is token lane % 32)
        float cs0 = 1.f, cs1 = 1.f, rho = 1.f;
        if constexpr (PS && do_s) {
            const float4 sv4 = *(const float4*)&Scl[4 * slot];
            cs0 = sv4.x;
            cs1 = sv4.y;
            rho = (lane % 32) < 16 ? sv4.z / sv4.x : sv4.w / sv4.y;
        }
        // Value product j of 32: K half kk = j / 16, head tile nt = j / 4 % 4,
        // column tile mc = j % 4.  The P operands of group j / 4 (one K half,
        // one head tile) stream through two slots: group q + 1 is read when
        // group q starts.
        bf16x8 pbr[2];
        auto load_pb = [&](int q) {
            if (q < 8) pbr[q % 2] = Pb[pr][q % 4][q / 4][lane];
        };
        auto vprod = [&](int j) {
            if (j % 4 == 0) load_pb(j / 4 + 1);
            const int kk = j / 16, nt = (j / 4) % 4, mc = j % 4;
            const bf16x8 a = F8 ? fp8x8_to_bf16(av8[kk][F8 ? mc : 0]) : av[kk][F8 ? 0 : mc];
            U[mc][nt] = mfma32(a, pbr[(j / 4) % 2], U[mc][nt]);
        };
        if constexpr (do_v) load_pb(0);
        // in the score phase: value products 0 .. NU1 - 1, one after each
        // score product (NU1 = 32) or after every second one (NU1 = 16)
        auto interleave = [&](int ks) {
            constexpr int IV = NU1 ? 32 / NU1 : 1;   // score products per interleaved value product
            if (NU1 && ks < 32 && ks % IV == IV - 1) vprod(ks / IV);
        };
        // the prepared refill, one instruction every DMA_EVERY score products
        constexpr int DMA_EVERY = KS / Dma::SPW;
        auto dma_slot = [&](int ks) {
            if (ks % DMA_EVERY == 0 && ks / DMA_EVERY < Dma::SPW) dma.issue_slot(pend, ks / DMA_EVERY);
        };
        f32x16 S;
        if constexpr (do_s) {
            f32x16 Sc[SCH];
            if (!F8) {
                bf16x8 a[PD];
#pragma unroll
                for (int ks = 0; ks < PD; ks++) a[ks] = *(const bf16x8*)to.score(C, ks);
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int c = ks % SCH;
                    if (ks < SCH) Sc[c] = mfma32_first(a[ks % PD], Qf[ks]);
                    else if (ks + SCH < KS) mfma32_acc(Sc[c], a[ks % PD], Qf[ks]);
                    else mfma32_last(Sc[c], a[ks % PD], Qf[ks]);
                    if (ks + PD < KS) a[ks % PD] = *(const bf16x8*)to.score(C, ks + PD);
                    if constexpr (do_v) interleave(ks);
                    dma_slot(ks);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                // one 16-byte read per pair of steps, PJ pairs ahead; the codes
                // widen to bf16 exactly just before their product.  With page
                // scales one pair ahead: the scales' registers would otherwise
                // push a q^ fragment out to scratch, and its reload inside the
                // chain makes the compiler wait for all outstanding vector
                // memory operations, the tile DMA included.
#ifndef MLA_PJ8
#define MLA_PJ8 2
#endif
                constexpr int PJ = PS ? 1 : MLA_PJ8, KJ = KS / 2;
                uint4 raw[PJ];
#pragma unroll
                for (int j = 0; j < PJ; j++) raw[j] = *(const uint4*)to8.score(C, j);
                bf16x8 a0, a1;
#pragma unroll
                for (int ks = 0; ks < KS; ks++) {
                    const int c = ks % SCH, j = ks / 2;
                    if (ks % 2 == 0) {
                        a0 = fp8x8_to_bf16(make_uint2(raw[j % PJ].x, raw[j % PJ].y));
                        a1 = fp8x8_to_bf16(make_uint2(raw[j % PJ].z, raw[j % PJ].w));
                        if (PS && j >= 16) {   // rotary dims: times this token's rho
                            a0 = scale_bf16x8(a0, rho);
                            a1 = scale_bf16x8(a1, rho);
                        }
                        if (j + PJ < KJ) raw[j % PJ] = *(const uint4*)to8.score(C, j + PJ);
                    }
                    const bf16x8 av8 = ks % 2 ? a1 : a0;
                    if (ks < SCH) Sc[c] = mfma32_first(av8, Qf[ks]);
                    else if (ks + SCH < KS) mfma32_acc(Sc[c], av8, Qf[ks]);
                    else mfma32_last(Sc[c], av8, Qf[ks]);
                    if constexpr (do_v) interleave(ks);
                    dma_slot(ks);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            S = Sc[0];
            if constexpr (SCH == 2) S += Sc[1];
        } else if constexpr (do_v) {
#pragma unroll
            for (int j = 0; j < NU1; j++) vprod(j);
        }
        // the remaining value products, independent of the softmax below:
        // the wavefront issues the softmax's vector instructions while each
        // product runs on the matrix core
        if constexpr (do_v) {
#pragma unroll
            for (int j = NU1; j < 32; j++) vprod(j);
        }
        if constexpr (do_s) {
            // ---- softmax weights: lane holds head hs, tokens 8 (v / 4) + 4 hh + v % 4;
            // rows past the sequence's length (its last tile) are masked
            // without a branch, so the whole phase is one scheduling region
            float lm = -INFINITY;
            const int nv = n - tbase - 4 * hh;   // this lane's rows r < nv are valid
#pragma unroll
            for (int v = 0; v < 16; v++) {
                if constexpr (PS) S[v] *= v < 8 ? cs0 : cs1;   // rows 0..15, then 16..31
                S[v] = 8 * (v / 4) + v % 4 < nv ? S[v] : -INFINITY;
                lm = fmaxf(lm, S[v]);
            }
            lm = fmaxf(lm, xor32(lm)) * sc;
            m = m == -INFINITY ? lm : m;   // first tile of the sequence: fix the reference
            ovf_w |= __builtin_amdgcn_ballot_w64(lm > m + 64.f) != 0;
            uint32_t pk[8];
            float ps = 0.f;
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const float p0 = __builtin_amdgcn_exp2f(fmaf(S[v], sc, -m));
                const float p1 = __builtin_amdgcn_exp2f(fmaf(S[v + 1], sc, -m));
                ps += p0 + p1;
                if constexpr (PS) {   // the latent sum's weights carry the page's c_scale
                    const float cv = v < 8 ? cs0 : cs1;
                    pk[v / 2] = pack_bf16x2(p0 * cv, p1 * cv);
                } else {
                    pk[v / 2] = pack_bf16x2(p0, p1);
                }
            }
            lsum += ps;
            Pb[pw][wave][0][lane] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            Pb[pw][wave][1][lane] = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
            // this tile's latent-sum operands, for the next step
#pragma unroll
            for (int kk = 0; kk < 2; kk++)
#pragma unroll
                for (int mc = 0; mc < MCW; mc++) {
                    if (F8) av8[kk][F8 ? mc : 0] = lds_read_tr8(to8.value(C, wave, mc, kk));
                    else av[kk][F8 ? 0 : mc] = cat_tr(lds_read_tr(to.value(C, wave, mc, kk, 0)),
                                                      lds_read_tr(to.value(C, wave, mc, kk, 1)));
                }
        }
#ifndef MLA_VPG
#define MLA_VPG 4
#endif
#ifndef MLA_VPG_F8
#define MLA_VPG_F8 6
#endif
        if constexpr (do_s && do_v) {
            // one value product, then VPG vector instructions, and so on
            constexpr int VPG = F8 ? MLA_VPG_F8 : MLA_VPG;
#pragma unroll
            for (int j = NU1; j < 32; j++) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, VPG, 0);
            }
        }
    };

    std::true_type Y;
    std::false_type N;
    int buf = 0;
    int g = g0;
    for (;;) {   // one sequence (or the part of it in this workgroup's range) per pass
        const int gend = min(g1, g + cc.nt - cc.lt);
        // first tile: scores only
        tile_top(buf);
        step(Y, N, Cs + buf * TL::TILE, cc.lt * kT, cc.n, 0, g & 1, buf);
        cc.lt++;
        buf = (buf + 1) % kNBuf;
        // then each tile's scores beside the previous tile's latent sum
        for (++g; g < gend; g++) {
            tile_top(buf);
            step(Y, Y, Cs + buf * TL::TILE, cc.lt * kT, cc.n, (g - 1) & 1, g & 1, buf);
            cc.lt++;
            buf = (buf + 1) % kNBuf;
        }
        // last tile's latent sum
        __syncthreads();   // its P visible
        step(N, Y, Cs, 0, 0, (g - 1) & 1, 0, 0);
        write_partial(cc.b, F8 ? Stg8 : Cs + ((buf + kNBuf - 1) % kNBuf) * TL::TILE);
        if (g >= g1) break;
        // the next sequence: its tile cursor, accumulators and q^
        cc.lt--;
        cc.g = g - 1;
        cc.next(sv);
        reset();
        load_q(cc.b);
        vmem_drain();
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup
    // the workgroup's flag: any wavefront that saw a score past its reference
    int* const ovf_s = (int*)&Pb[1][1][0][0];
    if (lane == 0) ovf_s[wave] = ovf_w;
    __syncthreads();
    if (tid == 0) p.flags[w] = (ovf_s[0] | ovf_s[1] | ovf_s[2] | ovf_s[3]) ? 1 : 0;
}

// The partial (m, l, U columns 8 lane .. 8 lane + 7) of head i over the
// tokens of sequence bb in global tiles [g_lo, g_hi), computed from scratch
// by one wavefront: the path for decode workgroups that stopped early.  An
// E4M3 cache is read as codes (U stays in code units, as in the decode
// kernel; q^ already carries the scales).  An
// online softmax in fp32 with the reference moved on every new maximum;
// the dot products take the stored bf16 q^ and cache bits, lane l holding
// latent dims 8 l .. 8 l + 7 and rotary dim l (d_c = 8 * 64, d_R = 64).
// Tokens go kRcRows at a time so that their row loads are in flight together.
constexpr int kRcRows = 4;   // rows in flight in the exact recompute
__device__ void mla_partial_recompute(const MlaParams& p, int bb, int i, int g_lo, int g_hi, int s0,
                                      int lane, float& M, float& L, float4& u0, float4& u1)
{
    const int cb = mla_cache_seq(bb, p.q_len);
    const int n = mla_seen(p.s[cb], bb, p.q_len, p.s_max);
    const int t_lo = (g_lo - s0) * kT, t_hi = min((g_hi - s0) * kT, n);
    const uint16_t* qc = p.qhat + qhat_index(bb, i, 8 * lane, p.h);
    const uint16_t* qr = p.qhat + qhat_index(bb, i, 512 + 8 * (lane / 8), p.h) + lane % 8;
    float q[9];
    {
        const uint4 v = *(const uint4*)qc;
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; e++) {
            q[2 * e] = bf16lo_to_f32(w4[e]);
            q[2 * e + 1] = bf16hi_to_f32(w4[e]);
        }
        q[8] = bf16lo_to_f32(*qr);
    }
    const uint16_t* cache = (const uint16_t*)p.cache;
    float m = -INFINITY, l = 0.f, u[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int t0 = t_lo; t0 < t_hi; t0 += kRcRows) {
        uint4 c8[kRcRows];
        uint16_t cr[kRcRows];
        float rcs[kRcRows], rrs[kRcRows];   // per-page scales (1: none)
#pragma unroll
        for (int k = 0; k < kRcRows; k++) rcs[k] = rrs[k] = 1.f;
#pragma unroll
        for (int k = 0; k < kRcRows; k++) {
            const int t = min(t0 + k, t_hi - 1);
            const size_t row = p.bt ? paged_row(p.bt, cb, t, p.max_blocks, p.bs_log2, p.num_blocks)
                                    : (size_t)cb * p.s_max + t;
            if (p.f8) {   // E4M3 codes, widened to bf16 exactly
                const uint8_t* c8p = (const uint8_t*)p.cache + row * 576;
                c8[k] = __builtin_bit_cast(uint4, fp8x8_to_bf16(*(const uint2*)(c8p + 8 * lane)));
                cr[k] = (uint16_t)(__builtin_bit_cast(uint4, fp8x8_to_bf16(make_uint2(c8p[512 + lane], 0u))).x & 0xffffu);
                if (p.c_scales) {   // the page's scales
                    const int blk = (int)(row >> p.bs_log2);
                    rcs[k] = p.c_scales[blk];
                    rrs[k] = p.r_scales[blk];
                }
            } else {
                c8[k] = *(const uint4*)(cache + row * 576 + 8 * lane);
                cr[k] = cache[row * 576 + 512 + lane];
            }
        }
#pragma unroll
        for (int k = 0; k < kRcRows; k++) {
            if (t0 + k >= t_hi) break;   // wave-uniform
            const uint32_t w4[4] = {c8[k].x, c8[k].y, c8[k].z, c8[k].w};
            float c[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                c[2 * e] = bf16lo_to_f32(w4[e]) * rcs[k];
                c[2 * e + 1] = bf16hi_to_f32(w4[e]) * rcs[k];
            }
            float z = q[8] * (bf16lo_to_f32(cr[k]) * rrs[k]);
#pragma unroll
            for (int e = 0; e < 8; e++) z = fmaf(q[e], c[e], z);
            z = wave_sum(z) * p.scale_log2;
            const float mn = fmaxf(m, z);
            const float a = __builtin_amdgcn_exp2f(m - mn), pz = __builtin_amdgcn_exp2f(z - mn);
            l = fmaf(l, a, pz);
#pragma unroll
            for (int e = 0; e < 8; e++) u[e] = fmaf(u[e], a, pz * c[e]);
            m = mn;
        }
    }
    M = m;
    L = l;
    u0 = make_float4(u[0], u[1], u[2], u[3]);
    u1 = make_float4(u[4], u[5], u[6], u[7]);
}

// ---------------------------------------------------------------------------
// 3. finish.  Workgroup = (head i, up to 8 sequences), 8 wavefronts.
//    Merge: a wavefront takes one sequence, lane l its columns 8l .. 8l+7
//    (a partial row, U / l in fp16, is one contiguous 1 KB span).  The split
//    maxima and sums are wave-uniform, so they come in as scalar loads, and
//    up to 8 partials are in flight per wavefront; chunks are folded in with
//    a running maximum, each weighted by 2^(m_k - M) l_k.  The partials of a decode workgroup that stopped early
//    are recomputed here instead.  When the block holds fewer than 8 sequences the idle
//    wavefronts take a share of some sequence's partials instead, and the
//    shares are combined through LDS.
//    Product: out[b, i, :] = W_UV[i] u~[b, i, :] on the matrix cores, with
//    u~ fed as a bf16 hi/lo pair (u~ = hi + lo to about 2^-16 relative, so
//    the product keeps u~ at fp32-level precision): A rows 0..7 are the hi
//    parts of the 8 sequences, rows 8..15 their lo parts, and the two halves
//    of the result are added across lanes.  W_UV rows are the B operand as
//    stored (16 contiguous bytes per lane).
// ---------------------------------------------------------------------------
constexpr int kFinSeq = 8;     // sequences (and wavefronts) per workgroup
constexpr int kFinChunk = 8;   // partials in flight per wavefront
constexpr int kAbStride = 512 + 8;   // bf16 per A-operand row in LDS

__global__ __launch_bounds__(64 * kFinSeq, 4) void mla_finish_kernel(const MlaParams p)
{
    __shared__ __attribute__((aligned(16))) float Acc[kFinSeq][512];      // shares, when split
    __shared__ float Mls[kFinSeq][2];
    __shared__ __attribute__((aligned(16))) uint16_t Ab[2 * kFinSeq][kAbStride];
    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int i = blockIdx.x % p.h;
    const int b0 = (blockIdx.x / p.h) * kFinSeq;
    const int nb = min(kFinSeq, p.B - b0);   // >= 1: the grid covers exactly the sequences
    const int sq = wave % nb, sub = wave / nb;
    const int nsub = (kFinSeq - sq + nb - 1) / nb;   // wavefronts sharing sequence sq
    const int bb = b0 + sq;

    // W_UV fragments of this wavefront's first column tile: the first
    // kWuvPre K steps are fetched now, so that their latency hides behind
    // the merge, the rest once the merge is done (all 16 up front would
    // push the kernel past 128 registers, i.e. below two workgroups per CU)
    const uint16_t* __restrict__ wuv = (const uint16_t*)p.w_uv + (size_t)i * p.d_v * p.d_c;
#ifndef MLA_WUV_PRE
#define MLA_WUV_PRE 8
#endif
    constexpr int kWuvPre = MLA_WUV_PRE;
    bf16x8 bws[16];   // d_c = 512: 16 K steps
    const bool up = p.out != nullptr;   // value up-projection wanted (else only u~ leaves)
    if (up && wave < p.d_v / 16) {
        const uint16_t* wrow = wuv + (size_t)(wave * 16 + li) * p.d_c + 8 * G;
#pragma unroll
        for (int k = 0; k < kWuvPre; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
    }

    // the partials of sequence bb: slots w + bb of the workgroups w whose
    // tile ranges overlap its tiles; this wavefront takes k = sub + nsub j
    const int32_t* __restrict__ sched = p.sched;
    const int s0 = max(sched[bb], 0), s1 = sched[bb + 1];
    const int tpw = max(sched[p.B + 1 + p.n_wg], 1);
    const int wf = min(s0 / tpw, p.n_wg - 1);
    const int ns = s1 > s0 ? min(max((s1 - 1) / tpw - wf + 1, 0), p.n_wg - wf) : 0;
    const int nj = ns > sub ? (ns - sub + nsub - 1) / nsub : 0;
    const size_t row0 = (size_t)(wf + bb) * p.h + i;   // partial k: row0 + k h
    const float2* __restrict__ ml = (const float2*)p.part_ml;
    const uint4* __restrict__ pu = (const uint4*)p.part_u;   // 8 fp16 of U / l per lane
    auto unpack = [](uint4 h, float4& lo, float4& hi) {
        typedef _Float16 h2 __attribute__((ext_vector_type(2)));
        const h2 x = __builtin_bit_cast(h2, h.x), y = __builtin_bit_cast(h2, h.y);
        const h2 z = __builtin_bit_cast(h2, h.z), t = __builtin_bit_cast(h2, h.w);
        lo = make_float4((float)x[0], (float)x[1], (float)y[0], (float)y[1]);
        hi = make_float4((float)z[0], (float)z[1], (float)t[0], (float)t[1]);
    };

    float M = -INFINITY, L = 0.f;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    // the first chunk of partials is requested before the flags are read,
    // so that both arrive in one round trip
    float2 v[kFinChunk];
    uint4 uh[kFinChunk];
    auto load_chunk = [&](int j0) {
#pragma unroll
        for (int c = 0; c < kFinChunk; c++) {   // clamped, unconditional loads
            const int jj = min(j0 + c, nj - 1);
            const size_t row = row0 + (size_t)(sub + nsub * jj) * p.h;
            v[c] = ml[row];
            uh[c] = pu[row * 64 + lane];
        }
    };
    if (nj > 0) load_chunk(0);
    // a decode workgroup that stopped early left no partials: recompute them
    bool any_flag = false;
    for (int jj = 0; jj < nj; jj++) any_flag |= p.flags[wf + sub + nsub * jj] != 0;
    if (any_flag) {   // wave-uniform; rare
        for (int jj = 0; jj < nj; jj++) {
            const int wk = wf + sub + nsub * jj;
            float mk, lk;
            float4 k0, k1;
            if (p.flags[wk]) {
                mla_partial_recompute(p, bb, i, max(wk * tpw, s0), min((wk + 1) * tpw, s1), s0, lane, mk, lk, k0, k1);
            } else {
                const size_t row = row0 + (size_t)(sub + nsub * jj) * p.h;
                mk = ml[row].x;
                lk = ml[row].y;
                unpack(pu[row * 64 + lane], k0, k1);
                k0 *= lk;
                k1 *= lk;
            }
            if (!(lk > 0.f)) continue;
            const float Mn = fmaxf(M, mk);
            const float sa = __builtin_amdgcn_exp2f(M - Mn), sb = __builtin_amdgcn_exp2f(mk - Mn);
            L = L * sa + lk * sb;
            a0 = a0 * sa + k0 * sb;
            a1 = a1 * sa + k1 * sb;
            M = Mn;
        }
    } else {   // the chunks already requested stay in registers on this path only
        for (int j0 = 0; j0 < nj; j0 += kFinChunk) {
            if (j0 > 0) load_chunk(j0);
            float Mc = M;
#pragma unroll
            for (int c = 0; c < kFinChunk; c++)
                if (j0 + c < nj && v[c].y > 0.f) Mc = fmaxf(Mc, v[c].x);
            if (Mc == -INFINITY) continue;   // nothing seen yet
            const float sc = __builtin_amdgcn_exp2f(M - Mc);   // 0 while M = -inf
            L *= sc;
            a0 *= sc;
            a1 *= sc;
#pragma unroll
            for (int c = 0; c < kFinChunk; c++) {
                if (j0 + c < nj && v[c].y > 0.f) {   // wave-uniform
                    const float wl = __builtin_amdgcn_exp2f(v[c].x - Mc) * v[c].y;   // weight of U / l
                    float4 u0, u1;
                    unpack(uh[c], u0, u1);
                    L += wl;
                    a0.x = fmaf(wl, u0.x, a0.x); a0.y = fmaf(wl, u0.y, a0.y);
                    a0.z = fmaf(wl, u0.z, a0.z); a0.w = fmaf(wl, u0.w, a0.w);
                    a1.x = fmaf(wl, u1.x, a1.x); a1.y = fmaf(wl, u1.y, a1.y);
                    a1.z = fmaf(wl, u1.z, a1.z); a1.w = fmaf(wl, u1.w, a1.w);
                }
            }
            M = Mc;
        }
    }

    // combine the shares of a sequence split over several wavefronts
    if (nb < kFinSeq) {   // workgroup-uniform
        *(float4*)&Acc[wave][8 * lane] = a0;
        *(float4*)&Acc[wave][8 * lane + 4] = a1;
        if (lane == 0) {
            Mls[wave][0] = M;
            Mls[wave][1] = L;
        }
        __syncthreads();
        if (wave < nb) {
            float Mt = -INFINITY;
            for (int t = 0; t < nsub; t++) Mt = fmaxf(Mt, Mls[wave + nb * t][0]);
            L = 0.f;
            a0 = make_float4(0.f, 0.f, 0.f, 0.f);
            a1 = a0;
            if (Mt != -INFINITY) {
                for (int t = 0; t < nsub; t++) {
                    const int src = wave + nb * t;
                    const float wt = __builtin_amdgcn_exp2f(Mls[src][0] - Mt);   // 0 for an empty share
                    L = fmaf(wt, Mls[src][1], L);
                    const float4 x0 = *(const float4*)&Acc[src][8 * lane];
                    const float4 x1 = *(const float4*)&Acc[src][8 * lane + 4];
                    a0.x = fmaf(wt, x0.x, a0.x); a0.y = fmaf(wt, x0.y, a0.y);
                    a0.z = fmaf(wt, x0.z, a0.z); a0.w = fmaf(wt, x0.w, a0.w);
                    a1.x = fmaf(wt, x1.x, a1.x); a1.y = fmaf(wt, x1.y, a1.y);
                    a1.z = fmaf(wt, x1.z, a1.z); a1.w = fmaf(wt, x1.w, a1.w);
                }
            }
            M = Mt;
        }
    }

    if (up && wave < p.d_v / 16) {
        const uint16_t* wrow = wuv + (size_t)(wave * 16 + li) * p.d_c + 8 * G;
#pragma unroll
        for (int k = kWuvPre; k < 16; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
    }
    // u~ = U / L: written out if asked, and split into the A operand rows
    if (wave < nb) {
        // u~ = U / L, in cache units: times the latent scale of an FP8 cache
        const float inv = L > 0.f ? p.c_scale / L : 0.f;
        a0 *= inv;
        a1 *= inv;
        if (p.u_latent) {
            float4* dst = (float4*)(p.u_latent + ((size_t)bb * p.h + i) * 512) + 2 * lane;
            dst[0] = a0;
            dst[1] = a1;
        }
        if (lane == 0 && p.lse)
            p.lse[(size_t)bb * p.h + i] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
        const float xs[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const uint32_t h2 = pack_bf16x2(xs[e], xs[e + 1]);
            hi[e / 2] = h2;
            lo[e / 2] = pack_bf16x2(xs[e] - bf16lo_to_f32(h2), xs[e + 1] - bf16hi_to_f32(h2));
        }
        if (p.u_bf16)   // bf16 u~, the X operand of the merged output projection
            *(uint4*)(p.u_bf16 + ((size_t)bb * p.h + i) * 512 + 8 * lane) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *(uint4*)&Ab[wave][8 * lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *(uint4*)&Ab[kFinSeq + wave][8 * lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    } else {   // rows of absent sequences: zeros
        *(uint4*)&Ab[wave][8 * lane] = make_uint4(0, 0, 0, 0);
        *(uint4*)&Ab[kFinSeq + wave][8 * lane] = make_uint4(0, 0, 0, 0);
    }
    if (!up) return;   // kernel-uniform
    __syncthreads();

    // out[b0 + r, i, n] = sum_c u~[r][c] W_UV[i][n][c]: wavefront w takes
    // column tiles w, w + 8, ...; result row r (< 8) is hi, r + 8 its lo part
    for (int nt = wave; nt < p.d_v / 16; nt += kFinSeq) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (nt != wave) {
            const uint16_t* wrow = wuv + (size_t)(nt * 16 + li) * p.d_c + 8 * G;
#pragma unroll
            for (int k = 0; k < 16; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
            __builtin_amdgcn_sched_barrier(0);   // all 16 loads in flight before the first use
        }
#pragma unroll
        for (int k = 0; k < 16; k++)
            acc = mfma16(*(const bf16x8*)&Ab[li][32 * k + 8 * G], bws[k], acc);
        // lane (G, li) holds row 4G + e of column 16 nt + li; rows 8.. sit 32 lanes up
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float o = acc[e] + xor32(acc[e]);
            const int r = 4 * G + e;
            if (G < 2 && r < nb)
                ((uint16_t*)p.out)[((size_t)(b0 + r) * p.h + i) * p.d_v + nt * 16 + li] =
                    (uint16_t)f32_to_bf16_bits(o);
        }
    }
}

hipError_t launch_mla(const MlaParams& p, bool paged, hipStream_t st)
{
    // absorb workgroups, plus one that computes the tile schedule
    if (p.d_nope > kAbsMaxNope) return hipErrorInvalidValue;
    const unsigned g1 = (unsigned)(p.h * (p.d_c / kAbsCols)) + 1;
    if (p.d_nope <= 128)
        hipLaunchKernelGGL(mla_absorb_kernel<128>, dim3(g1), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL(mla_absorb_kernel<kAbsMaxNope>, dim3(g1), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = (unsigned)p.n_wg;
    if (p.f8 && p.c_scales) {
        if (!paged || !p.r_scales) return hipErrorInvalidValue;
        hipLaunchKernelGGL((mla_decode_kernel<true, true, true>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched,
                           p.c_scales, p.r_scales);
    } else if (p.f8) {
        if (paged)
            hipLaunchKernelGGL((mla_decode_kernel<true, true>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched,
                               nullptr, nullptr);
        else
            hipLaunchKernelGGL((mla_decode_kernel<false, true>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched,
                               nullptr, nullptr);
    } else {
        if (paged)
            hipLaunchKernelGGL((mla_decode_kernel<true, false>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched,
                               nullptr, nullptr);
        else
            hipLaunchKernelGGL((mla_decode_kernel<false, false>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched,
                               nullptr, nullptr);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g3 = (unsigned)(p.h * ((p.B + kFinSeq - 1) / kFinSeq));
    hipLaunchKernelGGL(mla_finish_kernel, dim3(g3), dim3(64 * kFinSeq), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
