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
// the decode tile schedule (defined with the decode kernels below).  Its
// inputs are passed by value: a reference to the kernel's parameter block
// would force a copy of it into scratch memory for every wavefront.
struct SchedArgs {
    const int32_t* s;
    int32_t* sched;
    int B, s_max, n_wg, min_tiles;
};
__device__ __forceinline__ void mla_schedule(SchedArgs p, int tid, int nthr, int* sc);

constexpr int kAbsCols = 128;
constexpr int kAbsRowStride = kAbsCols * 2 + 16;

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// q_nope rows of one 16-sequence block as the A operand, K steps 0..7 (steps
// past d_nope / 32 and rows past B are zero).  The loads are unconditional
// from clamped addresses and masked afterwards, so all of them are in flight
// together.
struct AbsA {
    bf16x8 k[8];
};
__device__ __forceinline__ AbsA absorb_load_a(const uint16_t* __restrict__ qn, int b0, int li, int G,
                                              int B, int h, int i, int d_nope)
{
    AbsA a;
    const int ksteps = d_nope / 32;
    const int bb = b0 + li, bc = min(bb, B - 1);
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int kc = min(k, ksteps - 1);
        const u32x4v v = *(const u32x4v*)(qn + ((size_t)bc * h + i) * d_nope + kc * 32 + 8 * G);
        const unsigned keep = (k < ksteps && bb < B) ? 0xffffffffu : 0u;   // mask, not a branch
        a.k[k] = __builtin_bit_cast(bf16x8, v & keep);
    }
    return a;
}

__global__ __launch_bounds__(256) void mla_absorb_kernel(const MlaParams p)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    __shared__ __attribute__((aligned(16))) uint16_t ost[4][16][32 + 8];   // per-wavefront output staging
    if (blockIdx.x == gridDim.x - 1) {   // one extra workgroup: the decode tile schedule
        __shared__ int sc[256];
        mla_schedule(SchedArgs{p.s, p.sched, p.B, p.s_max, p.n_wg, p.min_tiles}, threadIdx.x, 256, sc);
        return;
    }
    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int nq = p.d_c / kAbsCols;
    const int i = blockIdx.x / nq, cq = blockIdx.x % nq;
    const int c0 = cq * kAbsCols;
    const int W = p.d_c + p.d_R;
    const uint16_t* __restrict__ wuk = (const uint16_t*)p.w_uk + (size_t)i * p.d_nope * p.d_c;
    const uint16_t* __restrict__ qn = (const uint16_t*)p.q_nope;
    const int ksteps = p.d_nope / 32;

    AbsA a = absorb_load_a(qn, 0, li, G, p.B, p.h, i, p.d_nope);

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
    // the rotary part of q^ is a plain copy (done once per head, 16 bytes per
    // lane, four copies in flight); d_R is a multiple of 8
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
                *(u32x4v*)(p.qhat + ((size_t)(idx / per) * p.h + i) * W + p.d_c + 8 * (idx % per)) = v[u];
            }
        }
    }

    __syncthreads();

    // wavefront w computes column tiles 2w and 2w+1 (32 columns) for every
    // 16-row block of b; the next block's q_nope is fetched while this one
    // is multiplied.  The block's 16 x 32 results go through LDS so that
    // each lane stores 16 contiguous bytes.
    for (int b0 = 0; b0 < p.B; b0 += 16) {
        const AbsA an = absorb_load_a(qn, min(b0 + 16, p.B - 1), li, G, p.B, p.h, i, p.d_nope);
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
                    acc = mfma16(a.k[k], cat_tr(lo, hi), acc);
                }
            }
            // lane holds q~[b0 + 4G + e][c0 + 16 nt + li]
#pragma unroll
            for (int e = 0; e < 4; e++) ost[wave][4 * G + e][16 * t + li] = (uint16_t)f32_to_bf16_bits(acc[e]);
        }
        __syncthreads();
        {
            const int r = lane / 4, sg = lane % 4;   // row of the block, 16-byte segment
            const u32x4v v = *(const u32x4v*)&ost[wave][r][8 * sg];
            if (b0 + r < p.B)
                *(u32x4v*)(p.qhat + ((size_t)(b0 + r) * p.h + i) * W + c0 + 32 * wave + 8 * sg) = v;
        }
        __syncthreads();
        a = an;
    }
}

// ---------------------------------------------------------------------------
// 2. decode.  Workgroup = a run of tiles with all heads, so every latent
//    tile is fetched once.  Tiles of 32 rows move HBM -> LDS by LDS-DMA
//    (buffer_load ... lds, no staging registers) into a ring of 4 buffers,
//    three tiles ahead of use.
//    Fast kernel, 4 wavefronts (one per SIMD, accumulators in AGPRs):
//      scores   wavefront w, heads 32w .. 32w+31, per 16-head block:
//               S^T[32 tok x 16 heads] = C_tile[32 x 576] . q^T  (A: LDS, B: q^ in registers),
//               softmax weights P on S^T (lane = head, 8 tokens per lane);
//      exchange P of all heads through LDS (8 KB per tile);
//      latent   wavefront w, latent columns 128w .. 128w+127, all heads:
//               U^T[128 x 128] += C_tile^T[128 x 32] . P^T[32 x 128]
//               (A: transposing LDS reads of a quarter of the tile, B: P).
//    Splitting the latent sum by columns instead of heads means each latent
//    byte is read from LDS by one wavefront there instead of four; with the
//    score reads this cuts the LDS traffic per tile from 288 KB to 208 KB,
//    and LDS bandwidth (about 100 B/clock per CU for these patterns, as
//    measured) is what bounds this loop alongside the matrix cores.
//    The fallback kernel uses 8 wavefronts x 16 heads for both products.
//    The token order of the value product's K axis is the score product's
//    output layout (lane group G holds tokens 4G..4G+3 and 16+4G..16+4G+3),
//    so P keeps the layout it was computed in.
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
    const int32_t* __restrict__ s;       // lengths [B]
    const int32_t* __restrict__ sched;   // tile_start [B + 1], wstart [n_wg], tpw
    int s_max, B, n_wg;
    __device__ __forceinline__ int len(int b) const
    {
        return min(max(__builtin_amdgcn_readfirstlane(s[b]), 0), s_max);
    }
    __device__ __forceinline__ int at(int i) const { return __builtin_amdgcn_readfirstlane(sched[i]); }
    __device__ __forceinline__ int total() const
    {
        return min(max(at(B), 0), B * ((s_max + kT - 1) / kT));
    }
    __device__ __forceinline__ int tpw(int tot) const { return min(max(at(B + 1 + n_wg), 1), max(tot, 1)); }
    __device__ __forceinline__ int first_seq(int w) const { return min(max(at(B + 1 + w), 0), B - 1); }
};

// Computed by one workgroup of nthr threads (a power of two); sc is nthr
// ints of LDS.  Two passes over the lengths: the first only totals the
// tiles (which fixes tpw), the second scans them again and writes the tile
// offsets and each workgroup's first sequence; no thread reads back what
// another wrote to global memory.
__device__ __forceinline__ void mla_schedule(SchedArgs p, int tid, int nthr, int* sc)
{
    int32_t* ts = p.sched;
    int32_t* wstart = p.sched + p.B + 1;
    auto tiles_of = [&](int i) { return i < p.B ? (min(max(p.s[i], 0), p.s_max) + kT - 1) / kT : 0; };
    // pass 1: total
    int part = 0;
    for (int i = tid; i < p.B; i += nthr) part += tiles_of(i);
    sc[tid] = part;
    __syncthreads();
    for (int off = nthr / 2; off > 0; off >>= 1) {
        if (tid < off) sc[tid] += sc[tid + off];
        __syncthreads();
    }
    const int total = sc[0];
    const int tpw = max((total + p.n_wg - 1) / p.n_wg, p.min_tiles);
    __syncthreads();
    // pass 2: offsets; workgroup w starts at tile w tpw, inside exactly one
    // non-empty sequence
    int carry = 0;
    for (int base = 0; base < p.B; base += nthr) {
        const int i = base + tid;
        const int tl = tiles_of(i);
        sc[tid] = tl;
        __syncthreads();
        for (int off = 1; off < nthr; off <<= 1) {   // inclusive scan
            const int v = tid >= off ? sc[tid - off] : 0;
            __syncthreads();
            sc[tid] += v;
            __syncthreads();
        }
        if (i < p.B) {
            const int a = carry + sc[tid] - tl, e = a + tl;
            ts[i] = a;
            for (int w = (a + tpw - 1) / tpw; w * tpw < e; w++) wstart[w] = i;
        }
        carry += sc[nthr - 1];
        __syncthreads();
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

// DMA of one tile (all 36 slots of 8 rows x 128 bytes, spread over the
// wavefronts; slot q fills segment q / 4, rows 8 (q % 4) .. + 7) and the
// physical rows of its two 16-row halves.  A tile's halves each lie in one
// block of a paged pool (blocks hold a power of two >= 16 rows).  With NW a
// multiple of 4 a wavefront's slots all cover the same 8 rows (q % 4 =
// wave % 4), so one buffer resource per tile serves all of them and a slot
// differs only in its segment's byte offset and LDS destination.
template <int NW, bool PAGED>
struct TileDma {
    static_assert(NW % 4 == 0, "a wavefront's slots must share their rows");
    static constexpr int SPW = kSlots / NW + (kSlots % NW ? 1 : 0);   // slots per wavefront
    const MlaParams& p;
    const int32_t* __restrict__ btab;
    const uint8_t* __restrict__ cbase;
    uint32_t lds0, vbase;
    int wave, rb;
    __device__ __forceinline__ TileDma(const MlaParams& p_, const int32_t* __restrict__ bt,
                                       uint32_t lds, int wave_, int lane)
        : p(p_), btab(bt), cbase((const uint8_t*)p_.cache), lds0(lds), wave(wave_), rb(wave_ & 3)
    {
        const int lr = lane / 8, lp = lane % 8;   // row of the 8, 16-byte position in the segment
        vbase = (uint32_t)(lr * kRow + 16 * (lp ^ swz(8 * rb + lr)));
    }
    __device__ __forceinline__ size_t half_row(int b, int t) const
    {
        if (PAGED) return paged_row(btab, b, t, p.max_blocks, p.bs_log2, p.num_blocks);
        return (size_t)b * p.s_max + t;
    }
    __device__ __forceinline__ void rows(const TileWalk& c, size_t& r0, size_t& r1) const
    {
        if (c.past()) {
            r0 = r1 = 0;
            return;
        }
        r0 = half_row(c.b, c.lt * kT);
        r1 = half_row(c.b, c.lt * kT + 16);
    }
    __device__ __forceinline__ void issue(const TileWalk& c, int buf, size_t row0, size_t row1) const
    {
        const size_t row = (rb < 2 ? row0 : row1) + 8 * (rb & 1);   // first row of this wavefront's 8
        const int t0 = c.lt * kT + 8 * rb;                            // its token index
        const int nr = c.past() ? 0 : max(0, min(8, c.n - t0)) * kRow;   // rows past the length read 0
        const rsrc_t rs = make_rsrc(cbase + row * kRow, nr);
        const uint32_t lb = lds0 + (uint32_t)(buf * kTile);
#pragma unroll
        for (int j = 0; j < SPW; j++) {
            const int q = wave + NW * j;
            if (kSlots % NW == 0 || q < kSlots)   // wave-uniform, static when NW divides the slots
                dma16(rs, vbase + 128u * (uint32_t)(q >> 2), lb + (uint32_t)q * 1024u);
        }
    }
    // tiles tb + T and tb + 2T were issued after tile tb
    __device__ __forceinline__ void wait_tile() const
    {
        if (SPW * NW == kSlots || wave < kSlots % NW) wait_vmcnt<2 * SPW>();
        else wait_vmcnt<2 * (SPW - 1)>();
    }
};

template <bool PAGED>
__global__ __launch_bounds__(256) void mla_decode_fast_kernel(const MlaParams p,
                                                              const int32_t* __restrict__ btab,
                                                              const int32_t* __restrict__ slen,
                                                              const int32_t* __restrict__ sched)
{
    constexpr int NW = 4;           // wavefronts per workgroup
    constexpr int NT = 8 / NW;      // score head tiles per wavefront (32 heads)
    constexpr int KS = 576 / 32;    // score K steps
    constexpr int VMC = 512 / NW / 16;   // latent column tiles per wavefront
    constexpr int VNT = 128 / 16;   // head tiles of the latent sum (all heads; zeros past h)
    __shared__ __attribute__((aligned(1024))) uint8_t Cs[kNBuf * kTile];
    __shared__ __attribute__((aligned(16))) bf16x8 Pb[VNT][64];   // P of every head tile, B-operand layout
    __shared__ int ovf;   // some head's scores ran past its reference max + 64

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int w = xcd_major(blockIdx.x, gridDim.x);
    const SchedView sv{slen, sched, p.s_max, p.B, p.n_wg};
    const int total = sv.total();
    const int tpw = sv.tpw(total);
    const long long g0l = (long long)w * tpw;
    const int g0 = (int)min(g0l, (long long)total), g1 = min(g0 + tpw, total);
    if (g0 >= g1) {
        if (tid == 0) p.flags[w] = 0;
        return;
    }
    const int head0 = wave * 16 * NT;
    const bool active = head0 < p.h;   // this wavefront has score heads

    const TileDma<NW, PAGED> dma(p, btab, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Cs,
                                 wave, lane);
    TileWalk ic(sv, sv.first_seq(w), g0, g1);   // issue cursor
    TileWalk cc = ic;                            // compute cursor

    // q^ fragments of one sequence: B operand of the score product (head
    // tiles past h read as zeros)
    bf16x8 Qf[NT][KS];
    auto load_q = [&](int b) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++)
#pragma unroll
            for (int ks = 0; ks < KS; ks++)
                Qf[nt][ks] = head0 + 16 * nt < p.h
                    ? *(const bf16x8*)(p.qhat + ((size_t)b * p.h + head0 + 16 * nt + li) * 576 + ks * 32 + 8 * G)
                    : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    };

    // Per head and sequence: m is fixed at the first tile's max (log2 units)
    // and U, lsum accumulate 2^(z - m).  Later tiles may exceed m by up to 64
    // (p <= 2^64, far from fp32/bf16 overflow); past that the workgroup is
    // handed to the rescaling kernel (flag), which real logits essentially
    // never need.  m and lsum belong to this wavefront's score heads, U to
    // its latent columns (all heads).
    f32x4 U[VMC][VNT];
    float m[NT], lsum[NT];
    auto reset = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            m[nt] = -INFINITY;
            lsum[nt] = 0.f;
        }
#pragma unroll
        for (int mc = 0; mc < VMC; mc++)
#pragma unroll
            for (int t = 0; t < VNT; t++) U[mc][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // partial state of sequence b, slot w + b: (m, l) of the score heads and
    // the U^T columns 128 wave .. + 127 of every head
    auto write_partial = [&](int b) {
#pragma unroll
        for (int nt = 0; nt < NT; nt++) {
            if (head0 + 16 * nt >= p.h) continue;
            float l = lsum[nt];
            l += xor16(l);
            l += xor32(l);
            const size_t row = (size_t)(w + b) * p.h + head0 + 16 * nt + li;
            if (G == 0) {
                p.part_ml[row * 2] = m[nt];
                p.part_ml[row * 2 + 1] = l;
            }
        }
#pragma unroll
        for (int t = 0; t < VNT; t++) {
            if (16 * t >= p.h) continue;
            const size_t row = (size_t)(w + b) * p.h + 16 * t + li;
            float* pu = p.part_u + row * 512 + (512 / NW) * wave + 4 * G;
#pragma unroll
            for (int mc = 0; mc < VMC; mc++)
                *(float4*)(pu + 16 * mc) = make_float4(U[mc][t][0], U[mc][t][1], U[mc][t][2], U[mc][t][3]);
        }
    };
    reset();
    if (tid == 0) ovf = 0;

    // two tiles in flight, then q^ of the first sequence, then the third tile
    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 0, r0, r1);
        ic.next(sv);
        dma.rows(ic, r0, r1);
        dma.issue(ic, 1, r0, r1);
        ic.next(sv);
    }
    load_q(cc.b);
    vmem_drain();
    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 2, r0, r1);
        ic.next(sv);
    }

    const TileOffsets to(li, G);
    const int cseg = 2 * wave * 4096;   // this wavefront's latent columns: segments 2w, 2w + 1
    int buf = 0;
    int g = g0;
    for (;;) {   // one sequence (or the part of it in this workgroup's range) per pass
      const int gend = min(g1, g + cc.nt - cc.lt);
      for (; g < gend; g++) {
        size_t nx0, nx1;   // rows of the tile issued below, looked up early
        dma.rows(ic, nx0, nx1);
        dma.wait_tile();
        __syncthreads();
        if (ovf) break;                      // uniform across the workgroup
        // refill the buffer read in the previous iteration (every wavefront is
        // past it), so that three tiles stay in flight while this one is used
        dma.issue(ic, (buf + 3) % kNBuf, nx0, nx1);
        ic.next(sv);
        const uint8_t* C = Cs + buf * kTile;
        const int tbase = cc.lt * kT;
        bf16x8 P[NT];
        if (active) {
            // ---- scores S^T = C . q^T, operands read one K step ahead
            f32x4 S[2][NT];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < NT; nt++) S[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            bf16x8 a[2][2];
            a[0][0] = lds_read_16_as_2x8(to.score(C, 0, 0));
            a[0][1] = lds_read_16_as_2x8(to.score(C, 0, 1));
#pragma unroll
            for (int ks = 0; ks < KS; ks++) {
                if (ks + 1 < KS) {
                    a[(ks + 1) & 1][0] = lds_read_16_as_2x8(to.score(C, ks + 1, 0));
                    a[(ks + 1) & 1][1] = lds_read_16_as_2x8(to.score(C, ks + 1, 1));
                }
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int nt = 0; nt < NT; nt++)
                        S[mt][nt] = mfma16(a[ks & 1][mt], Qf[nt][ks], S[mt][nt]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // ---- softmax weights against the fixed per-head reference m
            bool over = false;
#pragma unroll
            for (int nt = 0; nt < NT; nt++) {
                float z[2][4];
                float lm = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int tok = tbase + 16 * mt + 4 * G + e;
                        z[mt][e] = tok < cc.n ? S[mt][nt][e] * p.scale_log2 : -INFINITY;
                        lm = fmaxf(lm, z[mt][e]);
                    }
                if (m[nt] == -INFINITY) {       // first tile of the sequence: fix the reference
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
                        const uint32_t wv = pack_bf16x2(__builtin_amdgcn_exp2f(z[mt][e] - m[nt]),
                                                        __builtin_amdgcn_exp2f(z[mt][e + 1] - m[nt]));
                        pk[mt * 2 + e / 2] = wv;
                        ps += bf16lo_to_f32(wv) + bf16hi_to_f32(wv);
                    }
                lsum[nt] += ps;
                P[nt] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            }
            if (__builtin_amdgcn_ballot_w64(over) && lane == 0) ovf = 1;
        } else {
#pragma unroll
            for (int nt = 0; nt < NT; nt++) P[nt] = __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
#pragma unroll
        for (int nt = 0; nt < NT; nt++) Pb[NT * wave + nt][lane] = P[nt];
        __syncthreads();                     // P of every head visible
        // ---- latent sum U^T += C^T . P^T over this wavefront's columns: the
        // A operands of all its column tiles, then one head tile of P at a time
        bf16x8 av[VMC];
#pragma unroll
        for (int mc = 0; mc < VMC; mc++)
            av[mc] = cat_tr(lds_read_tr(to.value(C + cseg, mc, 0)), lds_read_tr(to.value(C + cseg, mc, 1)));
        bf16x8 Pt[2];
        Pt[0] = Pb[0][lane];
#pragma unroll
        for (int t = 0; t < VNT; t++) {
            if (t + 1 < VNT) Pt[(t + 1) & 1] = Pb[t + 1][lane];
#pragma unroll
            for (int mc = 0; mc < VMC; mc++) U[mc][t] = mfma16(av[mc], Pt[t & 1], U[mc][t]);
            __builtin_amdgcn_sched_barrier(0);
        }
        cc.lt++;
        buf = (buf + 1) % kNBuf;
      }
      if (g < gend) break;                   // left early: flagged for the rescaling kernel
      write_partial(cc.b);
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
    __syncthreads();   // ovf from the last tile
    if (tid == 0) p.flags[w] = ovf;
}

// Fallback for a workgroup whose fast pass was flagged: the same tile range,
// 8 wavefronts x 16 heads, with a lazily moving reference max and in-register
// rescaling.  Unflagged workgroups return at once.
template <bool PAGED>
__global__ __launch_bounds__(512) void mla_decode_safe_kernel(const MlaParams p,
                                                              const int32_t* __restrict__ btab,
                                                              const int32_t* __restrict__ slen,
                                                              const int32_t* __restrict__ sched)
{
    constexpr int KS = 576 / 32;    // score K steps
    constexpr int MC = 512 / 16;    // value M tiles (latent columns)
    __shared__ __attribute__((aligned(1024))) uint8_t Cs[kNBuf * kTile];

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int w = xcd_major(blockIdx.x, gridDim.x);
    if (__builtin_amdgcn_readfirstlane(p.flags[w]) == 0) return;   // the fast kernel finished it
    const SchedView sv{slen, sched, p.s_max, p.B, p.n_wg};
    const int total = sv.total();
    const int tpw = sv.tpw(total);
    const long long g0l = (long long)w * tpw;
    const int g0 = (int)min(g0l, (long long)total), g1 = min(g0 + tpw, total);
    if (g0 >= g1) return;
    const int head0 = wave * 16;
    const bool active = head0 < p.h;

    const TileDma<8, PAGED> dma(p, btab, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Cs,
                                wave, lane);
    TileWalk ic(sv, sv.first_seq(w), g0, g1);
    TileWalk cc = ic;

    bf16x8 Qf[KS];
    auto load_q = [&](int b) {
#pragma unroll
        for (int ks = 0; ks < KS; ks++)
            Qf[ks] = active ? *(const bf16x8*)(p.qhat + ((size_t)b * p.h + head0 + li) * 576 + ks * 32 + 8 * G)
                            : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    };
    f32x4 U[MC];
    float m, lsum;
    auto reset = [&]() {
        m = -INFINITY;
        lsum = 0.f;
#pragma unroll
        for (int mc = 0; mc < MC; mc++) U[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    auto write_partial = [&](int b) {
        float l = lsum;
        l += xor16(l);
        l += xor32(l);
        const size_t row = (size_t)(w + b) * p.h + head0 + li;
        float* pu = p.part_u + row * 512 + 4 * G;
#pragma unroll
        for (int mc = 0; mc < MC; mc++)
            *(float4*)(pu + 16 * mc) = make_float4(U[mc][0], U[mc][1], U[mc][2], U[mc][3]);
        if (G == 0) {
            p.part_ml[row * 2] = m;
            p.part_ml[row * 2 + 1] = l;
        }
    };
    reset();

    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 0, r0, r1);
        ic.next(sv);
        dma.rows(ic, r0, r1);
        dma.issue(ic, 1, r0, r1);
        ic.next(sv);
    }
    load_q(cc.b);
    vmem_drain();
    {
        size_t r0, r1;
        dma.rows(ic, r0, r1);
        dma.issue(ic, 2, r0, r1);
        ic.next(sv);
    }

    const TileOffsets to(li, G);
    int buf = 0;
    for (int g = g0; g < g1; g++) {
        size_t nx0, nx1;
        dma.rows(ic, nx0, nx1);
        dma.wait_tile();
        __syncthreads();
        dma.issue(ic, (buf + 3) % kNBuf, nx0, nx1);
        ic.next(sv);
        if (cc.lt == 0 && g != g0) {
            load_q(cc.b);
            vmem_drain();
        }
        const uint8_t* C = Cs + buf * kTile;
        const int tbase = cc.lt * kT;
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
                    const int tok = tbase + 16 * mt + 4 * G + e;
                    z[mt][e] = tok < cc.n ? S[mt][e] * p.scale_log2 : -INFINITY;
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
                    const uint32_t wv = pack_bf16x2(__builtin_amdgcn_exp2f(z[mt][e] - mn),
                                                    __builtin_amdgcn_exp2f(z[mt][e + 1] - mn));
                    pk[mt * 2 + e / 2] = wv;
                    ps += bf16lo_to_f32(wv) + bf16hi_to_f32(wv);
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
        if (g + 1 == g1 || cc.lt + 1 == cc.nt) {
            if (active) write_partial(cc.b);
            reset();
        }
        cc.next(sv);
        buf = (buf + 1) % kNBuf;
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup
}

// ---------------------------------------------------------------------------
// 3. finish.  Workgroup = (head i, up to 8 sequences), 8 wavefronts.
//    Merge: a wavefront takes one sequence, lane l its columns 8l .. 8l+7
//    (a partial row is read as two contiguous 1 KB spans).  The split maxima
//    and sums are wave-uniform, so they come in as scalar loads, and up to 8
//    partials are in flight per wavefront; chunks are folded in with a
//    running maximum.  When the block holds fewer than 8 sequences the idle
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

__global__ __launch_bounds__(64 * kFinSeq) void mla_finish_kernel(const MlaParams p)
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

    // W_UV fragments of this wavefront's first column tile, fetched now so
    // that their latency hides behind the merge
    const uint16_t* __restrict__ wuv = (const uint16_t*)p.w_uv + (size_t)i * p.d_v * p.d_c;
    bf16x8 bws[16];   // d_c = 512: 16 K steps
    if (wave < p.d_v / 16) {
        const uint16_t* wrow = wuv + (size_t)(wave * 16 + li) * p.d_c + 8 * G;
#pragma unroll
        for (int k = 0; k < 16; k++) bws[k] = *(const bf16x8*)(wrow + 32 * k);
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
    const float4* __restrict__ pu = (const float4*)p.part_u;

    float M = -INFINITY, L = 0.f;
    float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
    for (int j0 = 0; j0 < nj; j0 += kFinChunk) {
        float2 v[kFinChunk];
        float4 u[kFinChunk][2];
#pragma unroll
        for (int c = 0; c < kFinChunk; c++) {   // clamped, unconditional loads
            const int jj = min(j0 + c, nj - 1);
            const size_t row = row0 + (size_t)(sub + nsub * jj) * p.h;
            v[c] = ml[row];
            u[c][0] = pu[row * 128 + 2 * lane];
            u[c][1] = pu[row * 128 + 2 * lane + 1];
        }
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
                const float wk = __builtin_amdgcn_exp2f(v[c].x - Mc);
                L = fmaf(wk, v[c].y, L);
                a0.x = fmaf(wk, u[c][0].x, a0.x); a0.y = fmaf(wk, u[c][0].y, a0.y);
                a0.z = fmaf(wk, u[c][0].z, a0.z); a0.w = fmaf(wk, u[c][0].w, a0.w);
                a1.x = fmaf(wk, u[c][1].x, a1.x); a1.y = fmaf(wk, u[c][1].y, a1.y);
                a1.z = fmaf(wk, u[c][1].z, a1.z); a1.w = fmaf(wk, u[c][1].w, a1.w);
            }
        }
        M = Mc;
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

    // u~ = U / L: written out if asked, and split into the A operand rows
    if (wave < nb) {
        const float inv = L > 0.f ? 1.f / L : 0.f;
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
        *(uint4*)&Ab[wave][8 * lane] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        *(uint4*)&Ab[kFinSeq + wave][8 * lane] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    } else {   // rows of absent sequences: zeros
        *(uint4*)&Ab[wave][8 * lane] = make_uint4(0, 0, 0, 0);
        *(uint4*)&Ab[kFinSeq + wave][8 * lane] = make_uint4(0, 0, 0, 0);
    }
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
    const unsigned g1 = (unsigned)(p.h * (p.d_c / kAbsCols)) + 1;
    const size_t smem1 = (size_t)p.d_nope * kAbsRowStride;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t ea = hipFuncSetAttribute((const void*)mla_absorb_kernel,
                                            hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);   // d_nope <= 256 rows of 272 bytes
        if (ea != hipSuccess) return ea;
        attr_set = true;
    }
    hipLaunchKernelGGL(mla_absorb_kernel, dim3(g1), dim3(256), smem1, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g2 = (unsigned)p.n_wg;
    if (paged) {
        hipLaunchKernelGGL((mla_decode_fast_kernel<true>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched);
        hipLaunchKernelGGL((mla_decode_safe_kernel<true>), dim3(g2), dim3(512), 0, st, p, p.bt, p.s, p.sched);
    } else {
        hipLaunchKernelGGL((mla_decode_fast_kernel<false>), dim3(g2), dim3(256), 0, st, p, p.bt, p.s, p.sched);
        hipLaunchKernelGGL((mla_decode_safe_kernel<false>), dim3(g2), dim3(512), 0, st, p, p.bt, p.s, p.sched);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned g3 = (unsigned)(p.h * ((p.B + kFinSeq - 1) / kFinSeq));
    hipLaunchKernelGGL(mla_finish_kernel, dim3(g3), dim3(64 * kFinSeq), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
