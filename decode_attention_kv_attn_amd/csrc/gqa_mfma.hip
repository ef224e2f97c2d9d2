// Decode attention for GQA / MQA / MHA over bf16 caches on the matrix cores.
//
// out[b,i] = sum_t softmax_t(scale * q[b,i] . K[b,t,j]) V[b,t,j], j = i / g
// ("The KV cache size formula", mlinterviewnotes.com: attention against all
// previous positions; "MHA -> MQA -> GQA -> MLA", opening section: the g
// query heads of a group share one KV head).
//
// The g query heads of one KV head are exactly the "many heads, one shared
// K/V" shape that MLA decode takes in its MQA mode ("MHA -> MQA -> GQA ->
// MLA", the MLA-decode-becomes-MQA remark): per token, one K row and one V
// row serve g dot products each.  The vector form of that work needs about
// 2g FLOP per cached byte of dot-product instructions, which at g >= 8 runs
// into the vector ALU before HBM.  Here the products run as bf16 MFMA with
// the heads padded to 16, so the ALU only carries the softmax:
//
//  * workgroup = (b, KV head j, token split); wavefront w takes query heads
//    16w .. 16w+15 of the group (2 or 4 wavefronts, g <= 64; all of them
//    issue the tile DMA);
//  * K and V tiles of 32 tokens move HBM -> LDS by LDS-DMA (buffer_load ...
//    lds) into a ring of NBUF buffers, NBUF - 1 tiles ahead of use; completion is
//    tracked with explicit vmcnt waits (no other vector-memory instruction is
//    outstanding inside the loop);
//  * S^T[32 tok x 16 heads] = K_tile . q^T   (v_mfma_f32_16x16x32_bf16, K rows
//    from LDS, q in registers);
//  * online softmax per head (log2 domain, lazily rescaled: the reference max
//    moves only when a tile exceeds it by more than 8), P rounded to bf16;
//  * O^T[d_h x 16 heads] += V_tile^T . P^T, the V operand read with
//    transposing LDS reads; the score output layout is the K order of this
//    product, so P stays in registers;
//  * splits write (m, l, o) partials that are combined through their
//    log-sum-exp ("MLA: why one latent can replace a multi-head KV cache",
//    charlestar.github.io, section on what FlashMLA solves): by the last
//    workgroup of the (b, KV head, row block) item to finish, which learns
//    that it is last from an arrival counter, or, without counters, by the
//    separate merge kernel.
#include "common.h"
#include "kernels.h"
#include "mfma_lds.h"

namespace attn {

#ifndef GQA_MFMA_NBUF
#define GQA_MFMA_NBUF 4
#endif
#ifndef GQA_MFMA_NBUF_F8
#define GQA_MFMA_NBUF_F8 4
#endif

template <int D, bool F8>
struct MfmaCfg {
    static constexpr int T = 32;               // tokens per tile
    static constexpr int RB = D * (F8 ? 1 : 2);  // bytes of one row (one KV head)
    static constexpr int NCH = RB / 16;        // 16-byte chunks per row
    static constexpr int KT = T * RB;          // bytes of a K (or V) tile
    static constexpr int RPO = 1024 / RB;      // rows per DMA instruction
    static constexpr int OPS = 2 * KT / 1024;  // DMA instructions per tile (K, then V)
    static constexpr int NBUF = F8 ? GQA_MFMA_NBUF_F8 : GQA_MFMA_NBUF;   // ring depth (NBUF - 1 tiles in flight)
    static constexpr int KS = D / 32;          // score K steps
    static constexpr int MC = D / 16;          // value M tiles (head dimensions)
};

// XOR swizzle of the 16-byte chunk position within a row: logical chunk c of
// tile row r sits at c ^ gswz(r).  Rows r and r + 16 share a value.  For
// 256-byte rows, rows 0..15 get 16 distinct positions (score operands read
// 16 rows at one chunk) and every 4 consecutive rows get distinct aligned
// chunk pairs (the transposing reads take 4 rows x 32 bytes).
// FP8 rows (D bytes, D / 16 chunks): position c ^ ((r / 2) mod (D / 16)).
// The score operands (16 rows, 8 bytes each at one column) then cover every
// (row parity, chunk) pair once, and so do the transposing reads (pairs of
// consecutive rows, 16 bytes each).
template <int D, bool F8>
__device__ __forceinline__ int gswz(int r)
{
    if (F8) return (r >> 1) & (D / 16 - 1);
    r &= 15;
    if (D == 128) return (2 * r + (r >> 3)) & 15;
    return (r & 1) ^ (r & 2) ^ ((r & 4) ? 5 : 0) ^ ((r & 8) ? 7 : 0);
}

// Per-lane byte offsets of the MFMA operands within a K or V tile buffer
// (row block mt = 1 adds 16 rows).
// bf16:
//   score operand (K step ks, row block mt): row 16 mt + li, chunk 4 ks + G
//   value operand (M tile mc, token half th): rows 4G + li/4 + 16 th, chunk
//     2 mc + (li % 4) / 2, byte 8 (li % 2) within it
// FP8 (converted to bf16 after the read):
//   score operand: row 16 mt + li, byte 32 ks + 8 G: chunk 2 ks + G / 2,
//     byte 8 (G % 2) within it
//   value operand (M tile mc): a transposing 8-bit read; source lane li reads
//     row tau(G, li / 2), bytes 16 mc + 8 (li % 2), where tau(G, k) = 4 G + k
//     for k < 4 and 16 + 4 G + k - 4 otherwise -- the token order of the
//     score product's output, which is the K order of the value product
template <int D, bool F8>
struct GTileOffsets {
    int sc[D / 32];
    int tr[D / 16];
    __device__ __forceinline__ GTileOffsets(int li, int G)
    {
        constexpr int RB = D * (F8 ? 1 : 2);
        const int ss = gswz<D, F8>(li);
        if (F8) {
#pragma unroll
            for (int ks = 0; ks < D / 32; ks++) sc[ks] = li * RB + (((2 * ks + G / 2) ^ ss) << 4) + 8 * (G % 2);
            const int k = li / 2, r = k < 4 ? 4 * G + k : 16 + 4 * G + k - 4, st = gswz<D, F8>(r);
#pragma unroll
            for (int mc = 0; mc < D / 16; mc++) tr[mc] = r * RB + ((mc ^ st) << 4) + 8 * (li % 2);
        } else {
#pragma unroll
            for (int ks = 0; ks < D / 32; ks++) sc[ks] = li * RB + (((4 * ks + G) ^ ss) << 4);
            const int r = 4 * G + li / 4, cp = (li % 4) / 2, st = gswz<D, F8>(r);
#pragma unroll
            for (int mc = 0; mc < D / 16; mc++) tr[mc] = r * RB + (((2 * mc + cp) ^ st) << 4) + 8 * (li % 2);
        }
    }
};

// Splits of every sequence for the compacted grid: sequence 64 c + lane has
// nb[c] = max(1, ceil(min(max(s, 0), s_max) / chunk)) splits (an empty
// sequence keeps one workgroup, which writes its zero rows).  All B lengths are
// loaded at once (B <= 64 kMaxChunks), so finding a workgroup's pair costs one
// round trip to memory, as reading its own length would.
constexpr int kMaxChunks = 16;
struct SplitCounts {
    int nb[kMaxChunks];
    int total;   // wave-uniform
    __device__ __forceinline__ SplitCounts(const int32_t* __restrict__ s, int B, int s_max, int chunk)
    {
        const int lane = threadIdx.x % 64;
        int t = 0;
#pragma unroll
        for (int c = 0; c < kMaxChunks; c++) {
            const int i = 64 * c + lane;
            nb[c] = i < B ? max((min(max(s[i], 0), s_max) + chunk - 1) / chunk, 1) : 0;
            t += nb[c];
        }
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) t += __shfl_xor(t, d, 64);
        total = __builtin_amdgcn_readfirstlane(t);
    }
    // the k-th pair (k < total) in sequence-major order: sequence b, split
    __device__ __forceinline__ void locate(int k, int& b, int& split) const
    {
        int carry = 0;
        b = 0;
        split = 0;
#pragma unroll
        for (int c = 0; c < kMaxChunks; c++) {
            const int incl = wave_scan_incl(nb[c]);
            const int lo = carry + incl - nb[c];
            const unsigned long long hit = __builtin_amdgcn_ballot_w64(k >= lo && k < carry + incl);
            if (hit) {
                const int L = __builtin_ctzll(hit);
                b = 64 * c + L;
                split = k - __builtin_amdgcn_readlane(lo, L);
                return;
            }
            carry += __builtin_amdgcn_readlane(incl, 63);
        }
    }
};

// Head order against the XCDs.  Workgroup i runs on XCD i mod 8, so with the
// plain order (KV head fastest, h_kv a multiple of 8) XCD x streams only
// head columns j = x mod 8, and one head's 256-byte column sits at the same
// address bit 8 in every token row once a row (h_kv * row bytes) is a
// multiple of 512.  Measured on the Llama-3 layers: when that address bit
// equals the parity of the XCD reading it, the batch streams 5-6 % slower
// than when the two differ (every odd shift of the heads against the XCDs
// was fast, every even one slow; mixing all heads on every XCD was slower
// still).  pair_head permutes the low bits of j -- a bijection on every
// group of 2 << kb heads, so any dispatch order stays correct -- such that
// the column's address bit 8 is the opposite of bit 0 of the original
// index, which under the plain order is the XCD's parity.  kb is the bit of
// j that moves address bit 8 (256 / row bytes = 2^kb); flip is bit 8 of the
// cache's own address.
template <int RB>
__device__ __forceinline__ int pair_head(int j, int flip)
{
    constexpr int kb = RB >= 256 ? 0 : RB == 128 ? 1 : 2;
    constexpr int msk = (2 << kb) - 1;
    const int lo = j & msk;
    return (j & ~msk) | (((lo & 1) ^ 1 ^ flip) << kb) | (lo >> 1);
}

#ifndef GQA_MERGE_U
#define GQA_MERGE_U 8
#endif
// Buffer stores and loads coherent at device scope (cache policy sc1: they
// pass the XCD's own L2), for the split partials that the last workgroup of
// an item merges, wherever it runs.  Byte offsets into the partials, which
// the host keeps below 2^31 when it enables the merge in the kernel.
constexpr int kPolicyDevice = 16;   // sc1
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
struct PartRsrc {
    rsrc_t o, ml;
    __device__ __forceinline__ PartRsrc(const GqaParams& p, int D)
    {
        const long long rows = (long long)p.B * p.q_len * p.h * p.n_split;
        o = make_rsrc(p.part_o, (int)min(rows * D * 4, 0x7fffffffLL));
        ml = make_rsrc(p.part_ml, (int)min(rows * 8, 0x7fffffffLL));
    }
};
__device__ __forceinline__ void store_dev16(rsrc_t r, uint32_t off, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kPolicyDevice);
}
__device__ __forceinline__ void store_dev8(rsrc_t r, uint32_t off, float2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, off, 0, kPolicyDevice);
}
__device__ __forceinline__ float4 load_dev16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyDevice));
}
__device__ __forceinline__ float2 load_dev8(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicyDevice));
}
// Merge of one item's split partials by its last workgroup: rows r_lo ..
// r_hi - 1 of (b, KV head j), splits 0 .. nsb - 1, in split order (the
// result does not depend on the order of arrival).  m = max m_k over splits
// that saw tokens, l = sum 2^(m_k - m) l_k, o = sum 2^(m_k - m) o_k / l,
// lse = (m + log2 l) ln 2.  D / 8 threads share a row, 8 output elements
// each; a thread keeps U splits' loads in flight.
template <int D, int NT>
__device__ __forceinline__ void merge_item(const GqaParams& p, int b, int j, int r_lo, int r_hi,
                                           int nsb, int tid)
{
    constexpr int TPR = D / 8;     // threads per row
    constexpr int RPP = NT / TPR;  // rows per pass
    constexpr int U = GQA_MERGE_U;
    const int g = p.h / p.h_kv;
    const int e0 = 8 * (tid % TPR);
    const PartRsrc pr(p, D);
    for (int r = r_lo + tid / TPR; r < r_hi; r += RPP) {
        const size_t orow = (size_t)(b * p.q_len + r / g) * p.h + j * g + r % g;
        const uint32_t ml = (uint32_t)(orow * p.n_split * 8);
        const uint32_t po = (uint32_t)((orow * p.n_split * D + e0) * 4);
        float M = -INFINITY, L = 0.f, o[8];
#pragma unroll
        for (int e = 0; e < 8; e++) o[e] = 0.f;
        for (int k0 = 0; k0 < nsb; k0 += U) {
            float2 v[U];
            float4 x[U][2];
#pragma unroll
            for (int u = 0; u < U; u++) {   // clamped, unconditional device-scope loads
                const uint32_t k = min(k0 + u, nsb - 1);
                v[u] = load_dev8(pr.ml, ml + 8 * k);
                x[u][0] = load_dev16(pr.o, po + k * D * 4);
                x[u][1] = load_dev16(pr.o, po + k * D * 4 + 16);
            }
            float Mc = M;
#pragma unroll
            for (int u = 0; u < U; u++)
                if (k0 + u < nsb && v[u].y > 0.f) Mc = fmaxf(Mc, v[u].x);
            if (Mc == -INFINITY) continue;   // nothing seen yet
            const float sc = __builtin_amdgcn_exp2f(M - Mc);   // 0 while M = -inf
            L *= sc;
#pragma unroll
            for (int e = 0; e < 8; e++) o[e] *= sc;
#pragma unroll
            for (int u = 0; u < U; u++) {
                if (k0 + u < nsb && v[u].y > 0.f) {
                    const float w = __builtin_amdgcn_exp2f(v[u].x - Mc);
                    L = fmaf(w, v[u].y, L);
                    o[0] = fmaf(w, x[u][0].x, o[0]); o[1] = fmaf(w, x[u][0].y, o[1]);
                    o[2] = fmaf(w, x[u][0].z, o[2]); o[3] = fmaf(w, x[u][0].w, o[3]);
                    o[4] = fmaf(w, x[u][1].x, o[4]); o[5] = fmaf(w, x[u][1].y, o[5]);
                    o[6] = fmaf(w, x[u][1].z, o[6]); o[7] = fmaf(w, x[u][1].w, o[7]);
                }
            }
            M = Mc;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;   // L = 0: no visible token (0 and -inf)
        *(uint4*)((uint16_t*)p.out + orow * D + e0) =
            make_uint4(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv),
                       pack_bf16x2(o[4] * inv, o[5] * inv), pack_bf16x2(o[6] * inv, o[7] * inv));
        if (tid % TPR == 0 && p.lse) p.lse[orow] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
    }
}

// NI > 0: the last NI wavefronts issue all of the tile DMA and compute
// nothing, and the first NW - NI compute and issue nothing (rows must fit
// them).  Issuing a tile's DMA waits for room in the memory pipeline (about
// 120 cycles an instruction at full stream), which a wavefront that also
// computes would add to its compute time every tile.
template <int D, int NW, bool PAGED, bool F8, int RPW, bool PS = false, int NI = 0>
__global__ __launch_bounds__(64 * NW) void gqa_mfma_kernel(const GqaParams p,
                                                           const int32_t* __restrict__ btab,
                                                           const float* __restrict__ ksp,
                                                           const float* __restrict__ vsp)
{
    using C = MfmaCfg<D, F8>;
    constexpr int NIW = NI ? NI : NW;     // wavefronts that issue DMA
    constexpr int OPW = C::OPS / NIW;     // DMA instructions per issuing wavefront and tile
    static_assert(C::OPS % NIW == 0 && NI < NW, "DMA instructions must split evenly");
    __shared__ __attribute__((aligned(1024))) uint8_t Ls[C::NBUF * 2 * C::KT];

    const int tid = threadIdx.x, lane = tid % 64, G = lane / 16, li = lane % 16;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const bool issuer = NI == 0 || wave >= NW - NI;   // wave-uniform
    const int iw = NI ? wave - (NW - NI) : wave;      // index among the issuing wavefronts
    // work item (b, split, j) with j fastest.  A paged pool is walked
    // XCD-major, so that the KV heads of one sequence, which share every
    // block, run under one L2; a contiguous cache streams faster in plain
    // order (measured).
    // With mixed lengths most (sequence, split) pairs of a grid sized for
    // s_max are empty, and an empty workgroup still holds a slot while it
    // loads its length.  Compacted (the grid then has a multiple of 8
    // workgroups): only the n_real = pairs x KV heads x row blocks items of
    // the non-empty pairs are numbered, XCD-major, and the surplus
    // workgroups, last in every XCD's dispatch order, leave at once (the
    // merge kernel reads only the splits a sequence has).
    // (paged pools only: mixed lengths are their normal case, and the scan
    // costs a contiguous cache's uniform batches more than it saves)
    int w;
    int split = 0, b = 0;
    const bool compact = PAGED && p.compact;
    if (compact) {
        const SplitCounts sc(p.s, p.B, p.s_max, p.chunk);
        const int n_real = sc.total * p.h_kv * p.n_rb;
        const int per = (n_real + 7) / 8, slot = blockIdx.x >> 3;
        w = (blockIdx.x & 7) * per + slot;
        if (slot >= per || w >= n_real) return;   // wave-uniform
        sc.locate(w / (p.h_kv * p.n_rb), b, split);
    } else {
        w = PAGED ? xcd_major(blockIdx.x, gridDim.x) : (int)blockIdx.x;
    }
    const int rb = w % p.n_rb;
    w /= p.n_rb;
    int j = w % p.h_kv;
    w /= p.h_kv;
    if (!PAGED && p.xpair >= 0) j = pair_head<C::RB>(j, p.xpair);
    if (!compact) {
        split = w % p.n_split;
        b = w / p.n_split;
    }
    const int g = p.h / p.h_kv;
    // The rows of a work item are the (query position jq, head of the group)
    // pairs, r = jq * g + gi: g rows for one new token, g * q_len when
    // several new tokens are verified at once.  Row block rb holds rows
    // 64 RPW rb .. + 64 RPW - 1; wavefront w takes the RPW 16-row blocks
    // 16 (k NW + w) .. + 15 of them (k < RPW), all fed by the same LDS
    // operand reads of each tile.
    const int n_rows = g * p.q_len;
    bool act[RPW], hv[RPW];
    size_t orow[RPW];   // row of q, out and lse
    int jq[RPW];
    bool active = false;
#pragma unroll
    for (int k = 0; k < RPW; k++) {
        const int r0 = 64 * RPW * rb + 16 * (k * NW + wave);
        const int nh = min(16, n_rows - r0);        // rows of this block
        act[k] = nh > 0 && (NI == 0 || wave < NW - NI);
        active |= act[k];
        hv[k] = li < nh;                            // this lane's row exists
        const int r = hv[k] ? r0 + li : r0;
        jq[k] = r / g;
        orow[k] = (size_t)(b * p.q_len + jq[k]) * p.h + j * g + r % g;
    }

    const int32_t* __restrict__ s_len = p.s;
    int n = __builtin_amdgcn_readfirstlane(s_len[b]);
    n = min(max(n, 0), p.s_max);
    const int t0 = split * p.chunk;
    const int t1 = min(n, t0 + p.chunk);
    // query position jq sits at cache position n - q_len + jq and sees the
    // tokens before it and itself (causal among the new tokens)
    int tl[RPW];
#pragma unroll
    for (int k = 0; k < RPW; k++) tl[k] = min(t1, n - (p.q_len - 1 - jq[k]));

    // splits of this sequence (>= 1; the merge reads partials 0 .. nsb - 1)
    const int nsb = max((n + p.chunk - 1) / p.chunk, 1);
    if (t0 >= t1) {
        // split 0 of an empty sequence: zero rows and lse = -inf; a split
        // past a sequence's end leaves nothing (the merge does not read it)
        if (split != 0) return;
#pragma unroll
        for (int k = 0; k < RPW; k++) {
            if (!(act[k] && hv[k])) continue;
            uint16_t* o = (uint16_t*)p.out + orow[k] * D;
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++) *(uint2*)(o + 16 * mc + 4 * G) = make_uint2(0, 0);
            if (G == 0 && p.lse) p.lse[orow[k]] = -INFINITY;
        }
        return;
    }

    // DMA instruction q of a tile (q < OPS/2: K, else V) moves tile rows
    // RPO (q % (OPS/2)) .. + RPO-1; lane l writes row l / NCH, physical chunk
    // l % NCH, i.e. logical chunk (l % NCH) ^ gswz(row).  A tile's two
    // 16-token halves each lie in one block of a paged pool (blocks hold a
    // power of two >= 16 of rows), so a tile needs the physical rows of just
    // its two half starts; they are looked up one iteration before the tile
    // is issued, keeping the scalar-load latency off the issue path.  One
    // buffer resource per (K or V, half) covers the rows of that half inside
    // the split (rows past it read as zero); an instruction's lanes reach
    // their row and chunk through a per-lane offset that is the same for
    // every tile.
    const size_t rowstride = (size_t)p.h_kv * C::RB;   // bytes between tokens of one head
    const uint8_t* __restrict__ kb = (const uint8_t*)p.k + (size_t)j * C::RB;
    const uint8_t* __restrict__ vb = (const uint8_t*)p.v + (size_t)j * C::RB;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)Ls;
    uint32_t voff[OPW];
    {
        const int lr = lane / C::NCH, lp = lane % C::NCH;
#pragma unroll
        for (int jj = 0; jj < OPW; jj++) {
            const int q = max(iw, 0) + NIW * jj;
            const int rt = (q % (C::OPS / 2)) * C::RPO;   // first tile row of this instruction
            voff[jj] = (uint32_t)(((rt & 15) + lr) * (int)rowstride + ((lp ^ gswz<D, F8>(rt + lr)) << 4));
        }
    }
    auto half_row = [&](int t) -> size_t {   // physical row of token t (a multiple of 16)
        if (PAGED) return paged_row(btab, b, t, p.max_blocks, p.bs_log2, p.num_blocks);
        return (size_t)b * p.s_max + t;
    };
    auto issue_tile = [&](int tb, int buf, size_t row0, size_t row1) {
        if (!issuer) return;
        const int nv0 = min(max(t1 - tb, 0), 16), nv1 = min(max(t1 - tb - 16, 0), 16);
        const int nr0 = nv0 > 0 ? (nv0 - 1) * (int)rowstride + C::RB : 0;
        const int nr1 = nv1 > 0 ? (nv1 - 1) * (int)rowstride + C::RB : 0;
        const rsrc_t k0 = make_rsrc(kb + row0 * rowstride, nr0), k1 = make_rsrc(kb + row1 * rowstride, nr1);
        const rsrc_t v0 = make_rsrc(vb + row0 * rowstride, nr0), v1 = make_rsrc(vb + row1 * rowstride, nr1);
        const uint32_t lb = lds0 + (uint32_t)(buf * 2 * C::KT);
#pragma unroll
        for (int jj = 0; jj < OPW; jj++) {
            const int q = iw + NIW * jj;
            const bool isv = q >= C::OPS / 2;
            const int rb = isv ? q - C::OPS / 2 : q;
            const bool h1 = rb * C::RPO >= 16;
            const rsrc_t rs = isv ? (h1 ? v1 : v0) : (h1 ? k1 : k0);
            dma16(rs, voff[jj], lb + (isv ? C::KT : 0) + rb * 1024);
        }
    };

    f32x4 O[RPW][C::MC];
    float m[RPW], lsum[RPW];
#pragma unroll
    for (int k = 0; k < RPW; k++) {
#pragma unroll
        for (int mc = 0; mc < C::MC; mc++) O[k][mc] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[k] = -INFINITY;
        lsum[k] = 0.f;
    }

    // two tiles in flight, then q (the B operand of the score product; zero
    // for padding heads), then the third tile
    // NBUF - 2 tiles in flight, then q (the B operand of the score product;
    // zero for padding heads), then one more tile
    // Per-page scales of a paged E4M3 cache (one per page and KV head):
    // a tile's two 16-token halves lie in one page each, so each half has one
    // K and one V scale.  They are read when the tile is issued and carried
    // in a queue of AH entries to its compute iteration.  They come in as
    // restrict parameters with wave-uniform indices, so the reads are scalar
    // loads: a vector load here would make the compiler wait for every
    // outstanding vector-memory operation, the tile DMA included.
    constexpr int AH = C::NBUF - 1;   // tiles in flight ahead of the one in use
    constexpr bool ps = F8 && PAGED && PS;
    float qk[AH][2], qv[AH][2];
    auto page_scales = [&](size_t row0, size_t row1, float* ks, float* vs) {
        const int jj = __builtin_amdgcn_readfirstlane(j);
        const int blk0 = __builtin_amdgcn_readfirstlane((int)(row0 >> p.bs_log2));
        const int blk1 = __builtin_amdgcn_readfirstlane((int)(row1 >> p.bs_log2));
        const size_t i0 = (size_t)blk0 * p.h_kv + jj, i1 = (size_t)blk1 * p.h_kv + jj;
        ks[0] = ksp[i0];
        ks[1] = ksp[i1];
        vs[0] = vsp[i0];
        vs[1] = vsp[i1];
    };
#pragma unroll
    for (int i = 0; i < AH; i++) qk[i][0] = qk[i][1] = qv[i][0] = qv[i][1] = 1.f;
#pragma unroll
    for (int i = 0; i < C::NBUF - 2; i++) {
        const size_t a0 = half_row(t0 + i * C::T), a1 = half_row(t0 + i * C::T + 16);
        issue_tile(t0 + i * C::T, i, a0, a1);
        if (ps) page_scales(a0, a1, qk[i], qv[i]);
    }
    bf16x8 Qf[RPW][C::KS];
#pragma unroll
    for (int k = 0; k < RPW; k++) {
        const uint16_t* qrow = (const uint16_t*)p.q + orow[k] * D + 8 * G;
#pragma unroll
        for (int ks = 0; ks < C::KS; ks++)
            Qf[k][ks] = (act[k] && hv[k]) ? *(const bf16x8*)(qrow + 32 * ks)
                                          : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
    }
    vmem_drain();
    {
        constexpr int L = C::NBUF - 2;
        const size_t a0 = half_row(t0 + L * C::T), a1 = half_row(t0 + L * C::T + 16);
        issue_tile(t0 + L * C::T, L, a0, a1);
        if (ps) page_scales(a0, a1, qk[L], qv[L]);
    }

    const GTileOffsets<D, F8> to(li, G);
    int buf = 0;
    for (int tb = t0; tb < t1; tb += C::T) {
        const size_t nx0 = half_row(tb + AH * C::T), nx1 = half_row(tb + AH * C::T + 16);
        wait_vmcnt<(AH - 1) * OPW>();   // tiles tb + T .. tb + (AH-1) T were issued after this one
        __syncthreads();
        // refill the buffer read in the previous iteration (every wavefront is
        // past it), so that AH tiles stay in flight while this one is used
        issue_tile(tb + AH * C::T, (buf + AH) % C::NBUF, nx0, nx1);
        // this tile's page scales, then the queue moves on by one tile
        float tks[2] = {1.f, 1.f}, tvs[2] = {1.f, 1.f};
        if (ps) {
            tks[0] = qk[0][0], tks[1] = qk[0][1], tvs[0] = qv[0][0], tvs[1] = qv[0][1];
#pragma unroll
            for (int i = 0; i + 1 < AH; i++)
                qk[i][0] = qk[i + 1][0], qk[i][1] = qk[i + 1][1], qv[i][0] = qv[i + 1][0], qv[i][1] = qv[i + 1][1];
            page_scales(nx0, nx1, qk[AH - 1], qv[AH - 1]);
        }
        const uint8_t* Kt = Ls + buf * 2 * C::KT;
        const uint8_t* Vt = Kt + C::KT;
        if (active) {
            // every operand of the tile is read from LDS up front: the K
            // operands of the score product, then the V operands of the value
            // product (which do not depend on P, so their latency hides
            // behind the score products and the softmax)
            bf16x8 ka[C::KS][2];
#pragma unroll
            for (int ks = 0; ks < C::KS; ks++) {
                if (F8) {
                    ka[ks][0] = fp8x8_to_bf16(lds_read_8(Kt + to.sc[ks]));
                    ka[ks][1] = fp8x8_to_bf16(lds_read_8(Kt + to.sc[ks] + 16 * C::RB));
                } else {
                    ka[ks][0] = lds_read_16_as_2x8(Kt + to.sc[ks]);
                    ka[ks][1] = lds_read_16_as_2x8(Kt + to.sc[ks] + 16 * C::RB);
                }
            }
            bf16x8 va[C::MC];
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++)
                va[mc] = F8 ? fp8x8_to_bf16(lds_read_tr8(Vt + to.tr[mc]))
                            : cat_tr(lds_read_tr(Vt + to.tr[mc]), lds_read_tr(Vt + to.tr[mc] + 16 * C::RB));
#pragma unroll
            for (int k = 0; k < RPW; k++) {
                if (RPW > 1 && !act[k]) continue;   // wave-uniform
                // ---- scores S^T = K . q^T
                f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int ks = 0; ks < C::KS; ks++) {
                    S[0] = mfma16(ka[ks][0], Qf[k][ks], S[0]);
                    S[1] = mfma16(ka[ks][1], Qf[k][ks], S[1]);
                }
                // ---- online softmax: lane holds row li, tokens 16 mt + 4G + e
                float z[2][4];
                float lm = -INFINITY;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int tok = tb + 16 * mt + 4 * G + e;
                        z[mt][e] = tok < tl[k] ? S[mt][e] * (p.scale_log2 * tks[mt]) : -INFINITY;
                        lm = fmaxf(lm, z[mt][e]);
                    }
                lm = fmaxf(lm, xor16(lm));
                lm = fmaxf(lm, xor32(lm));
                const bool move = lm > m[k] + 8.f;
                const float mn = move ? lm : m[k];
                const float alpha = move ? __builtin_amdgcn_exp2f(m[k] - mn) : 1.f;
                m[k] = mn;
                // a row that has seen no visible token yet (possible only for
                // the earlier of several query positions) keeps m = -inf:
                // weights 0
                const float mb = mn == -INFINITY ? 0.f : mn;
                uint32_t pk[4];
                float psum = 0.f;
#pragma unroll
                for (int mt = 0; mt < 2; mt++)
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const float e0 = __builtin_amdgcn_exp2f(z[mt][e] - mb);
                        const float e1 = __builtin_amdgcn_exp2f(z[mt][e + 1] - mb);
                        if (ps) {   // the page's V scale rides on P; the sum takes the weights
                            pk[mt * 2 + e / 2] = pack_bf16x2(e0 * tvs[mt], e1 * tvs[mt]);
                            psum += e0 + e1;
                        } else {
                            const uint32_t wv = pack_bf16x2(e0, e1);
                            pk[mt * 2 + e / 2] = wv;
                            psum += bf16lo_to_f32(wv) + bf16hi_to_f32(wv);
                        }
                    }
                lsum[k] = lsum[k] * alpha + psum;
                if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
                    for (int mc = 0; mc < C::MC; mc++) O[k][mc] *= alpha;
                }
                const bf16x8 P = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
                // ---- O^T += V^T . P^T
#pragma unroll
                for (int mc = 0; mc < C::MC; mc++) O[k][mc] = mfma16(va[mc], P, O[k][mc]);
            }
        }
        buf = (buf + 1) % C::NBUF;
    }
    wait_vmcnt<0>();   // no LDS-DMA may outlive the workgroup

    // the only split of its sequence writes the result itself; with arrival
    // counters so does any sequence with one split
    const bool fused = p.arrive != nullptr && nsb > 1;   // workgroup-uniform
    const bool direct = p.n_split == 1 || (p.arrive != nullptr && nsb == 1);
#pragma unroll
    for (int k = 0; k < RPW; k++) {
        if (!act[k]) continue;   // wave-uniform (false on a wavefront without rows)
        float l = lsum[k];
        l += xor16(l);
        l += xor32(l);
        if (!hv[k]) continue;
        if (F8) {   // the V scale of an FP8 cache (the K scale is folded into scale_log2)
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++) O[k][mc] *= p.v_scale;
        }
        if (direct) {
            const float inv = l > 0.f ? 1.f / l : 0.f;   // l = 0: no visible token (0 and -inf)
            uint16_t* o = (uint16_t*)p.out + orow[k] * D + 4 * G;
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++)
                *(uint2*)(o + 16 * mc) = make_uint2(pack_bf16x2(O[k][mc][0] * inv, O[k][mc][1] * inv),
                                                    pack_bf16x2(O[k][mc][2] * inv, O[k][mc][3] * inv));
            if (G == 0 && p.lse) p.lse[orow[k]] = l > 0.f ? (m[k] + __log2f(l)) * kLn2 : -INFINITY;
        } else if (fused) {   // device-scope stores: the merging workgroup may sit on another XCD
            const PartRsrc pr(p, D);
            const uint32_t pi = (uint32_t)(orow[k] * p.n_split + split);
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++)
                store_dev16(pr.o, (pi * D + 16 * mc + 4 * G) * 4,
                            make_float4(O[k][mc][0], O[k][mc][1], O[k][mc][2], O[k][mc][3]));
            if (G == 0) store_dev8(pr.ml, pi * 8, make_float2(m[k], l));
        } else {
            const size_t pi = orow[k] * p.n_split + split;
            float* po = p.part_o + pi * D + 4 * G;
#pragma unroll
            for (int mc = 0; mc < C::MC; mc++)
                *(float4*)(po + 16 * mc) = make_float4(O[k][mc][0], O[k][mc][1], O[k][mc][2], O[k][mc][3]);
            if (G == 0) {
                p.part_ml[pi * 2] = m[k];
                p.part_ml[pi * 2 + 1] = l;
            }
        }
    }
    if (!fused) return;
    // Arrival.  The partials were written with device-scope stores, which
    // pass the XCD's own L2; once every wavefront has seen its stores
    // complete, one lane counts the workgroup in with a device-scope atomic.
    // The workgroup that brings the count to nsb is the last of its item: it
    // reads all partials with device-scope loads, merges them and puts the
    // counter back to zero for the next call.  No workgroup waits for
    // another, and no L2 is written back or invalidated.
    __shared__ int s_last;
    wait_vmcnt<0>();
    __syncthreads();
    int32_t* ctr = p.arrive + ((size_t)b * p.h_kv + j) * p.n_rb + rb;
    if (tid == 0) s_last = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nsb - 1;
    __syncthreads();
    if (!s_last) return;   // workgroup-uniform
    const int r_lo = 64 * RPW * rb;
    merge_item<D, 64 * NW>(p, b, j, r_lo, min(n_rows, r_lo + 64 * RPW), nsb, tid);
    if (tid == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D, int NW, bool F8, int RPW, int NI = 0>
static hipError_t launch_nw(const GqaParams& p, bool paged, unsigned grid, hipStream_t st)
{
    if (F8 && paged && p.k_scales)   // per-page scales
        hipLaunchKernelGGL((gqa_mfma_kernel<D, NW, true, F8, RPW, F8, NI>), dim3(grid), dim3(64 * NW), 0, st, p,
                           p.bt, p.k_scales, p.v_scales);
    else if (paged)
        hipLaunchKernelGGL((gqa_mfma_kernel<D, NW, true, F8, RPW, false, NI>), dim3(grid), dim3(64 * NW), 0, st, p,
                           p.bt, p.k_scales, p.v_scales);
    else
        hipLaunchKernelGGL((gqa_mfma_kernel<D, NW, false, F8, RPW, false, NI>), dim3(grid), dim3(64 * NW), 0, st, p,
                           p.bt, p.k_scales, p.v_scales);
    return hipGetLastError();
}

// (NW, RPW) in {(2, 1), (4, 1), (4, 2)}: 32, 64 or 128 rows per workgroup,
// every wavefront issuing DMA; or (E4M3, ni = 1) two wavefronts, one
// computing (16 rows) and one issuing
template <int D, bool F8>
static hipError_t launch_mfma_d(const GqaParams& p, int NW, int rpw, int ni, bool paged, unsigned grid,
                                hipStream_t st)
{
    if constexpr (F8)
        if (ni > 0) return launch_nw<D, 2, F8, 1, 1>(p, paged, grid, st);
    if (NW == 2) return launch_nw<D, 2, F8, 1>(p, paged, grid, st);
    return rpw == 2 ? launch_nw<D, 4, F8, 2>(p, paged, grid, st) : launch_nw<D, 4, F8, 1>(p, paged, grid, st);
}

hipError_t launch_gqa_mfma(const GqaParams& p, int d_h, int NW, int rpw, int ni, bool paged, bool f8,
                           unsigned grid, hipStream_t st)
{
    hipError_t e;
    if (f8) e = d_h == 64 ? launch_mfma_d<64, true>(p, NW, rpw, ni, paged, grid, st)
                          : launch_mfma_d<128, true>(p, NW, rpw, ni, paged, grid, st);
    else e = d_h == 64 ? launch_mfma_d<64, false>(p, NW, rpw, ni, paged, grid, st)
                       : launch_mfma_d<128, false>(p, NW, rpw, ni, paged, grid, st);
    if (e != hipSuccess || p.n_split == 1 || p.arrive) return e;
    return launch_gqa_combine(p, d_h, false, st);
}

}  // namespace attn
