// Decode attention for MHA / MQA / GQA on gfx950 (vector ALU, no MFMA).
//
// out[b,i] = sum_t softmax_t(scale * q[b,i] . K[b,t,j]) V[b,t,j], j = i / g
// ("The KV cache size formula", mlinterviewnotes.com: attention computes
// softmax(q K^T / sqrt(d_h)) V against all previous positions; "MHA -> MQA
// -> GQA -> MLA", opening section: query heads are broadcast over the
// h_kv shared KV heads).  At decode the intensity is 2g/b FLOP per byte, far
// below any matrix-core ridge, so the kernel is built around HBM streaming:
//
//  * one wavefront per work item (b, KV head j, group of HG query heads,
//    token split); each K/V row of head j is fetched from HBM once per work
//    item and used by all HG query heads of the group;
//  * K and V tiles of 32 tokens are fetched with 16-byte loads, one row per
//    16 (or 8) lanes, fully coalesced, into registers one tile ahead of use;
//  * K goes through LDS (XOR-swizzled 16-byte slots, conflict-free) so that
//    QK runs one token per lane pair with v_dot2_f32_bf16 against q read by
//    broadcast from LDS;
//  * the online softmax keeps a running max per head (wavefront DPP +
//    permlane-swap reductions); probabilities are rounded to bf16 once and
//    PV runs on the V registers with v_dot2_f32_bf16 over token pairs;
//  * long contexts are split across workgroups (split-KV); a second small
//    kernel merges the partial (m, l, o) states through their log-sum-exp,
//    the stable merge of local maxima, normalisers and outputs described in
//    "MLA: why one latent can replace a multi-head KV cache"
//    (charlestar.github.io), section on what FlashMLA solves.
#include "common.h"
#include "kernels.h"

namespace attn {

template <int D, bool F32>
struct GqaCfg {
    static constexpr int EB = F32 ? 4 : 2;   // bytes per element
    static constexpr int RB = D * EB;         // bytes per K/V row of one head
    static constexpr int NC = RB / 16;        // 16-byte chunks per row
    static constexpr int LR = NC;             // lanes per row in a load
    static constexpr int RPI = 64 / LR;       // rows per load instruction
    static constexpr int T = 32;              // tokens per tile
    static constexpr int NI = T / RPI;        // load instructions per tile
    static constexpr int EV = 16 / EB;        // elements per lane in PV
    static constexpr int PB = F32 ? 4 : 2;    // bytes per stored probability
    static constexpr int HC = NC / 2;         // chunks per lane in QK (2 lanes per token)
    static_assert(RPI <= 16 && NI >= 2, "tile shape");
};

template <int D, int HG, bool F32, bool PAGED>
__global__ __launch_bounds__(64) void gqa_decode_kernel(const GqaParams p,
                                                        const int32_t* __restrict__ btab)
{
    using C = GqaCfg<D, F32>;
    __shared__ __attribute__((aligned(16))) uint8_t Ks[C::T * C::RB];
    __shared__ __attribute__((aligned(16))) uint8_t Qs[HG * C::RB];
    __shared__ __attribute__((aligned(16))) uint8_t Ps[HG * C::T * C::PB];

    const int32_t* __restrict__ s_len = p.s;
    const uint8_t* __restrict__ kbase = (const uint8_t*)p.k;
    const uint8_t* __restrict__ vbase = (const uint8_t*)p.v;

    const int lane = threadIdx.x;
    int w = blockIdx.x;
    const int split = w % p.n_split;
    w /= p.n_split;
    const int hgi = w % p.n_hg;
    w /= p.n_hg;
    const int j = w % p.h_kv;
    const int b = w / p.h_kv;
    const int g = p.h / p.h_kv;
    const int head0 = j * g + hgi * HG;

    int n = __builtin_amdgcn_readfirstlane(s_len[b]);
    n = min(max(n, 0), p.s_max);
    const int t0 = split * p.chunk;
    const int t1 = min(n, t0 + p.chunk);

    if (t0 >= t1) {  // nothing to attend to in this split
        if (p.n_split > 1) {
            if (lane < HG) {
                float* ml = p.part_ml + ((size_t)(b * p.h + head0 + lane) * p.n_split + split) * 2;
                ml[0] = -INFINITY;
                ml[1] = 0.f;
            }
        } else {
            for (int gi = 0; gi < HG; gi++) {
                for (int e = lane; e < D; e += 64) {
                    const size_t o = (size_t)(b * p.h + head0 + gi) * D + e;
                    if (F32) ((float*)p.out)[o] = 0.f;
                    else ((uint16_t*)p.out)[o] = 0;
                }
                if (lane == 0 && p.lse) p.lse[b * p.h + head0 + gi] = -INFINITY;
            }
        }
        return;
    }

    // q of the HG heads -> LDS (contiguous HG * RB bytes)
    {
        const uint4* qsrc = (const uint4*)((const uint8_t*)p.q + (size_t)(b * p.h + head0) * C::RB);
        for (int c = lane; c < HG * C::NC; c += 64) ((uint4*)Qs)[c] = qsrc[c];
    }

    const int grp = lane / C::LR;   // row within a load instruction
    const int cl = lane % C::LR;    // 16-byte chunk within the row
    const uint32_t row_stride = (uint32_t)p.h_kv * C::RB;   // bytes between tokens of one head

    // Load the 32-token tile starting at tb (a multiple of 32) with buffer
    // loads: the resource covers only rows < t1, so rows past the end (and
    // whole tiles past it) read as zeros without touching memory.  Paged:
    // the RPI rows of one load instruction share a block (block_size >= 16
    // is a multiple of RPI), so each instruction has a uniform block base.
    const uint32_t voff_lane = (uint32_t)grp * row_stride + (uint32_t)cl * 16;
    auto load_tile = [&](uint4 (&dst)[C::NI], const uint8_t* __restrict__ base, int tb) {
        if (!PAGED) {
            const uint8_t* tbase = base + ((size_t)b * p.s_max + tb) * row_stride + (size_t)j * C::RB;
            const int nrec = (min(t1, tb + C::T) - tb) * (int)row_stride - j * C::RB;
            const rsrc_t r = make_rsrc(tbase, nrec);
#pragma unroll
            for (int k = 0; k < C::NI; k++)
                dst[k] = buf_load16(r, voff_lane + (uint32_t)(k * C::RPI) * row_stride);
        } else {
#pragma unroll
            for (int k = 0; k < C::NI; k++) {
                const int t = tb + k * C::RPI;                       // uniform
                const int lb = t >> p.bs_log2;
                const int bstart = lb << p.bs_log2;
                int blk = __builtin_amdgcn_readfirstlane(btab[(size_t)b * p.max_blocks + min(lb, p.max_blocks - 1)]);
                blk = min(max(blk, 0), p.num_blocks - 1);
                const uint8_t* bbase = base + ((size_t)blk << p.bs_log2) * row_stride + (size_t)j * C::RB;
                const int nrec = (min(t1 - bstart, 1 << p.bs_log2)) * (int)row_stride - j * C::RB;
                const rsrc_t r = make_rsrc(bbase, t < t1 ? nrec : 0);
                dst[k] = buf_load16(r, voff_lane + (uint32_t)(t - bstart) * row_stride);
            }
        }
    };

    float m[HG], lsum[HG], acc[HG][C::EV];
#pragma unroll
    for (int gi = 0; gi < HG; gi++) {
        m[gi] = -INFINITY;
        lsum[gi] = 0.f;
#pragma unroll
        for (int e = 0; e < C::EV; e++) acc[gi][e] = 0.f;
    }

    const int tq = lane % C::T;     // token of this lane in QK
    const int half = lane / C::T;   // which half of the row this lane dots
    const int ppos = (tq % C::RPI) * C::NI + tq / C::RPI;   // token order of PV

    // One tile: K regs -> LDS, refill K regs with tile tb + 2T, QK, online
    // softmax, PV on the V regs, refill V regs with tile tb + 2T.  Two
    // register sets alternate, so two tiles of K and V are in flight.
    auto tile = [&](uint4 (&kr)[C::NI], uint4 (&vr)[C::NI], int tb) {
#pragma unroll
        for (int k = 0; k < C::NI; k++) {
            const int r = k * C::RPI + grp;
            const int slot = cl ^ (r & (C::NC - 1));
            *(uint4*)(Ks + r * C::RB + slot * 16) = kr[k];
        }
        wave_lds_sync();
        // the refills must not be hoisted above the last use of the registers
        // they overwrite (that would double the live tile registers)
        __builtin_amdgcn_sched_barrier(0);
        load_tile(kr, kbase, tb + 2 * C::T);   // zeros once past t1

        // ---- QK: two lanes per token, each over half of the row
        float sc[HG];
#pragma unroll
        for (int gi = 0; gi < HG; gi++) sc[gi] = 0.f;
        {
            // q stays in LDS and is re-read every tile (broadcast reads); the
            // opaque zero offset keeps it from being hoisted into registers.
            int qz = 0;
            asm volatile("" : "+s"(qz));
            const uint8_t* qs = Qs + qz;
            const uint8_t* krow = Ks + tq * C::RB;
            // partial unroll: fully unrolled, the scheduler front-loads every
            // q/K read of the tile and runs out of registers
#pragma unroll 2
            for (int cc = 0; cc < C::HC; cc++) {
                const int c = half * C::HC + cc;
                const uint4 kv = *(const uint4*)(krow + ((c ^ (tq & (C::NC - 1))) * 16));
#pragma unroll
                for (int gi = 0; gi < HG; gi++) {
                    const uint4 qv = *(const uint4*)(qs + gi * C::RB + c * 16);
                    if (F32) {
                        sc[gi] = fmaf(__uint_as_float(kv.x), __uint_as_float(qv.x), sc[gi]);
                        sc[gi] = fmaf(__uint_as_float(kv.y), __uint_as_float(qv.y), sc[gi]);
                        sc[gi] = fmaf(__uint_as_float(kv.z), __uint_as_float(qv.z), sc[gi]);
                        sc[gi] = fmaf(__uint_as_float(kv.w), __uint_as_float(qv.w), sc[gi]);
                    } else {
                        sc[gi] = dot2_bf16(kv.x, qv.x, sc[gi]);
                        sc[gi] = dot2_bf16(kv.y, qv.y, sc[gi]);
                        sc[gi] = dot2_bf16(kv.z, qv.z, sc[gi]);
                        sc[gi] = dot2_bf16(kv.w, qv.w, sc[gi]);
                    }
                }
            }
        }

        // ---- online softmax (log2 domain); P -> LDS in PV order
        const bool valid = tb + tq < t1;
#pragma unroll
        for (int gi = 0; gi < HG; gi++) {
            const float zr = sc[gi] + xor32(sc[gi]);
            const float z = valid ? zr * p.scale_log2 : -INFINITY;
            const float mn = fmaxf(m[gi], uniform(wave_max(z)));
            const float alpha = __builtin_amdgcn_exp2f(m[gi] - mn);
            float pz = __builtin_amdgcn_exp2f(z - mn);
            if (F32) {
                if (half == 0) ((float*)Ps)[gi * C::T + ppos] = pz;
            } else {
                const uint32_t pb = f32_to_bf16_bits(pz);
                if (half == 0) ((uint16_t*)Ps)[gi * C::T + ppos] = (uint16_t)pb;
                pz = __uint_as_float(pb << 16);
            }
            lsum[gi] = lsum[gi] * alpha + (half == 0 ? pz : 0.f);
            m[gi] = mn;
#pragma unroll
            for (int e = 0; e < C::EV; e++) acc[gi][e] *= alpha;
        }
        wave_lds_sync();

        // ---- PV on the V registers: group grp owns tokens k*RPI + grp
        if (F32) {
#pragma unroll
            for (int k4 = 0; k4 < C::NI; k4 += 4) {
#pragma unroll
                for (int gi = 0; gi < HG; gi++) {
                    const float4 pp = *(const float4*)((const float*)Ps + gi * C::T + grp * C::NI + k4);
                    const float pk[4] = {pp.x, pp.y, pp.z, pp.w};
#pragma unroll
                    for (int u = 0; u < 4; u++) {
                        const uint4 vv = vr[k4 + u];
                        acc[gi][0] = fmaf(pk[u], __uint_as_float(vv.x), acc[gi][0]);
                        acc[gi][1] = fmaf(pk[u], __uint_as_float(vv.y), acc[gi][1]);
                        acc[gi][2] = fmaf(pk[u], __uint_as_float(vv.z), acc[gi][2]);
                        acc[gi][3] = fmaf(pk[u], __uint_as_float(vv.w), acc[gi][3]);
                    }
                }
            }
        } else {
            const uint32_t* P32 = (const uint32_t*)Ps;
#pragma unroll
            for (int k2 = 0; k2 < C::NI; k2 += 2) {
                const uint4 va = vr[k2], vb = vr[k2 + 1];
                const uint32_t pr[8] = {pair_lo(va.x, vb.x), pair_hi(va.x, vb.x),
                                        pair_lo(va.y, vb.y), pair_hi(va.y, vb.y),
                                        pair_lo(va.z, vb.z), pair_hi(va.z, vb.z),
                                        pair_lo(va.w, vb.w), pair_hi(va.w, vb.w)};
#pragma unroll
                for (int gi = 0; gi < HG; gi++) {
                    const uint32_t pp = P32[(gi * C::T + grp * C::NI + k2) / 2];
#pragma unroll
                    for (int e = 0; e < 8; e++) acc[gi][e] = dot2_bf16(pr[e], pp, acc[gi][e]);
                }
            }
        }
        wave_lds_sync();  // Ps / Ks reads done before the next tile overwrites them
        __builtin_amdgcn_sched_barrier(0);
        load_tile(vr, vbase, tb + 2 * C::T);
    };

    uint4 kA[C::NI], vA[C::NI], kB[C::NI], vB[C::NI];
    load_tile(kA, kbase, t0);
    load_tile(vA, vbase, t0);
    load_tile(kB, kbase, t0 + C::T);
    load_tile(vB, vbase, t0 + C::T);
    wave_lds_sync();  // Qs visible

    for (int tb = t0; tb < t1; tb += 2 * C::T) {
        tile(kA, vA, tb);
        if (tb + C::T >= t1) break;
        tile(kB, vB, tb + C::T);
    }

    // ---- finish: reduce over lanes, write result or partial
#pragma unroll
    for (int gi = 0; gi < HG; gi++) {
        lsum[gi] = uniform(wave_sum(lsum[gi]));
#pragma unroll
        for (int e = 0; e < C::EV; e++) {
            float x = acc[gi][e];
            if (C::RPI >= 8) x += dpp<0x128>(x);  // row_ror:8 = lane ^ 8 within a row of 16
            x += xor16(x);
            x += xor32(x);
            acc[gi][e] = x;
        }
    }
    if (grp != 0) return;
#pragma unroll
    for (int gi = 0; gi < HG; gi++) {
        const int head = head0 + gi;
        if (p.n_split == 1) {
            const float inv = 1.f / lsum[gi];
            const size_t o = (size_t)(b * p.h + head) * D + cl * C::EV;
            if (F32) {
                *(float4*)((float*)p.out + o) = make_float4(acc[gi][0] * inv, acc[gi][1] * inv,
                                                            acc[gi][2] * inv, acc[gi][3] * inv);
            } else {
                uint4 r;
                r.x = pack_bf16x2(acc[gi][0] * inv, acc[gi][1] * inv);
                r.y = pack_bf16x2(acc[gi][2] * inv, acc[gi][3] * inv);
                r.z = pack_bf16x2(acc[gi][4] * inv, acc[gi][5] * inv);
                r.w = pack_bf16x2(acc[gi][6] * inv, acc[gi][7] * inv);
                *(uint4*)((uint16_t*)p.out + o) = r;
            }
            if (lane == 0 && p.lse) p.lse[b * p.h + head] = (m[gi] + __log2f(lsum[gi])) * kLn2;
        } else {
            const size_t pi = (size_t)(b * p.h + head) * p.n_split + split;
            float* po = p.part_o + pi * D + cl * C::EV;
#pragma unroll
            for (int e = 0; e < C::EV; e += 4)
                *(float4*)(po + e) = make_float4(acc[gi][e], acc[gi][e + 1], acc[gi][e + 2], acc[gi][e + 3]);
            if (lane == 0) {
                p.part_ml[pi * 2] = m[gi];
                p.part_ml[pi * 2 + 1] = lsum[gi];
            }
        }
    }
}

// Merge of the split partials: m = max m_k over splits that saw tokens,
// l = sum 2^(m_k-m) l_k, o = sum 2^(m_k-m) o_k / l, lse = (m + log2 l) ln 2.
// One workgroup of NWV wavefronts per (b, head); each wavefront merges a
// contiguous range of the splits in chunks of 16 with a running maximum
// (lane = D/64 output elements), then the wavefronts' results are merged the
// same way through LDS.  A chunk's (m, l) pairs, its 16 partial rows and the
// sequence's length are loaded together, so a wavefront with at most 16
// splits waits for memory once.  Only the splits that hold tokens of the
// sequence wrote their rows; the others are loaded but not used.
template <int D, bool F32, int NWV>
__global__ __launch_bounds__(64 * NWV) void gqa_combine_kernel(const GqaParams p)
{
    constexpr int PL = D / 64;
    constexpr int U = 16;   // partial rows in flight per wavefront
    __shared__ float sM[NWV], sL[NWV];
    __shared__ float so[NWV][D];
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int bh = blockIdx.x;
    const int ns = p.n_split;
    const int slen = p.s[bh / (p.q_len * p.h)];   // used once the chunk's loads are out
    const int per = (ns + NWV - 1) / NWV;
    const int k_lo = min(wave * per, ns), k_hi = min(k_lo + per, ns);
    const float2* __restrict__ ml = (const float2*)p.part_ml + (size_t)bh * ns;
    const float* __restrict__ po = p.part_o + (size_t)bh * ns * D + lane * PL;
    float M = -INFINITY, L = 0.f, o[PL];
#pragma unroll
    for (int e = 0; e < PL; e++) o[e] = 0.f;
    for (int k0 = k_lo; k0 < k_hi; k0 += U) {
        const int cnt = min(U, k_hi - k0);
        // clamped, unconditional loads: lane u < cnt's pair, and all cnt rows
        const float2 v = ml[k0 + min(lane % U, cnt - 1)];
        float x[U][PL];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int k = k0 + min(u, cnt - 1);
#pragma unroll
            for (int e = 0; e < PL; e++) x[u][e] = po[(size_t)k * D + e];
        }
        const int len = min(max(slen, 0), p.s_max);
        const int nsb = min(ns, (len + p.chunk - 1) / p.chunk);   // splits that were written
        const bool use = lane < cnt && k0 + lane < nsb && v.y > 0.f;
        const float Mc = fmaxf(M, wave_max(use ? v.x : -INFINITY));
        if (Mc == -INFINITY) continue;   // wave-uniform: nothing seen yet
        const float sc = __builtin_amdgcn_exp2f(M - Mc);   // 0 while M = -inf
        const float wk = use ? __builtin_amdgcn_exp2f(v.x - Mc) : 0.f;
        L = fmaf(L, sc, wave_sum(wk * (use ? v.y : 0.f)));
#pragma unroll
        for (int e = 0; e < PL; e++) o[e] *= sc;
#pragma unroll
        for (int u = 0; u < U; u++) {
            const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wk), u));
            if (u < cnt && wu > 0.f) {
#pragma unroll
                for (int e = 0; e < PL; e++) o[e] = fmaf(wu, x[u][e], o[e]);
            }
        }
        M = Mc;
    }
    if (NWV > 1) {
        if (lane == 0) {
            sM[wave] = M;
            sL[wave] = L;
        }
#pragma unroll
        for (int e = 0; e < PL; e++) so[wave][lane * PL + e] = o[e];
        __syncthreads();
        if (wave != 0) return;
        float Mt = -INFINITY;
#pragma unroll
        for (int v = 0; v < NWV; v++)
            if (sL[v] > 0.f) Mt = fmaxf(Mt, sM[v]);
        L = 0.f;
#pragma unroll
        for (int e = 0; e < PL; e++) o[e] = 0.f;
#pragma unroll
        for (int v = 0; v < NWV; v++) {
            const float wv = sL[v] > 0.f ? __builtin_amdgcn_exp2f(sM[v] - Mt) : 0.f;
            L = fmaf(wv, sL[v], L);
#pragma unroll
            for (int e = 0; e < PL; e++) o[e] = fmaf(wv, so[v][lane * PL + e], o[e]);
        }
        M = Mt;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const size_t oo = (size_t)bh * D + lane * PL;
#pragma unroll
    for (int e = 0; e < PL; e++) {
        if (F32) ((float*)p.out)[oo + e] = o[e] * inv;
        else ((uint16_t*)p.out)[oo + e] = (uint16_t)f32_to_bf16_bits(o[e] * inv);
    }
    if (lane == 0 && p.lse) p.lse[bh] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
}

template <int D, bool F32>
static void launch_combine_d(const GqaParams& p, unsigned cg, hipStream_t st)
{
    // more wavefronts per (b, head) when there are many splits to merge, so
    // that each wavefront's share fits one chunk of 16 where it can
    if (p.n_split <= 16)
        hipLaunchKernelGGL((gqa_combine_kernel<D, F32, 1>), dim3(cg), dim3(64), 0, st, p);
    else if (p.n_split <= 64)
        hipLaunchKernelGGL((gqa_combine_kernel<D, F32, 4>), dim3(cg), dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((gqa_combine_kernel<D, F32, 16>), dim3(cg), dim3(1024), 0, st, p);
}

hipError_t launch_gqa_combine(const GqaParams& p, int d_h, bool f32, hipStream_t st)
{
    const unsigned cg = (unsigned)(p.B * p.q_len * p.h);
    if (f32) launch_combine_d<64, true>(p, cg, st);
    else if (d_h == 64) launch_combine_d<64, false>(p, cg, st);
    else launch_combine_d<128, false>(p, cg, st);
    return hipGetLastError();
}

template <int D, int HG, bool F32>
static hipError_t launch_hg(const GqaParams& p, bool paged, unsigned grid, hipStream_t st)
{
    if (paged)
        hipLaunchKernelGGL((gqa_decode_kernel<D, HG, F32, true>), dim3(grid), dim3(64), 0, st, p, p.bt);
    else
        hipLaunchKernelGGL((gqa_decode_kernel<D, HG, F32, false>), dim3(grid), dim3(64), 0, st, p, p.bt);
    return hipGetLastError();
}

template <int D, bool F32>
static hipError_t launch_d(const GqaParams& p, int HG, bool paged, unsigned grid, hipStream_t st)
{
    switch (HG) {
    case 1: return launch_hg<D, 1, F32>(p, paged, grid, st);
    case 2: return launch_hg<D, 2, F32>(p, paged, grid, st);
    case 4: return launch_hg<D, 4, F32>(p, paged, grid, st);
    default: return launch_hg<D, 8, F32>(p, paged, grid, st);
    }
}

hipError_t launch_gqa_decode(const GqaParams& p, int d_h, bool f32, int HG, bool paged,
                             unsigned grid, hipStream_t st)
{
    hipError_t e;
    if (f32) e = launch_d<64, true>(p, HG, paged, grid, st);
    else if (d_h == 64) e = launch_d<64, false>(p, HG, paged, grid, st);
    else e = launch_d<128, false>(p, HG, paged, grid, st);
    if (e != hipSuccess || p.n_split == 1) return e;
    return launch_gqa_combine(p, d_h, f32, st);
}

}  // namespace attn
