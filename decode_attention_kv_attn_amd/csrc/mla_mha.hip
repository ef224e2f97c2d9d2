// MLA in "MHA mode": the per-head keys and values are expanded explicitly
// from the latent cache and attention runs as plain multi-head attention
// ("MLA: why one latent can replace a multi-head KV cache",
// charlestar.github.io, section on MHA mode and MQA mode being execution
// forms (by gloss): expand per-head K/V, then a near-standard multi-head
// kernel, which suits long query blocks; "Multi-Head Latent Attention (MLA):
// Mathematical Foundations" (llms.blog), "Low-Rank Joint Key-Value
// Compression" and "The Decoupled RoPE Solution": k_i = [W_UK,i c ; k_R],
// v_i = W_UV,i c).
//
//   mla_expand_kernel   K_n[b, t, i, :] = W_UK[i] c_{b,t}  (d_nope = 128)
//                       V[b, t, i, :]   = W_UV[i] c_{b,t}  (d_v = 128)
//                       one GEMM over the stacked weights [W_UK ; W_UV]
//                       ([h (d_nope + d_v), d_c] rows), bf16 results.
//   mla_mha_attn_kernel out[b, jq, i] = sum_t softmax_t(scale (q_nope . K_n
//                       + q_rope . k_R)) V over the causal prefix of query
//                       position jq; k_R is read from the cache rows.
//
// The expansion costs 2 d_c h (d_nope + d_v) flops per cached token however
// many queries follow, the attention (d_nope + d_R + d_v) 2 h flops per
// token and query; the absorbed form pays (2 d_c + d_R) 2 h per token and
// query.  The expansion pays for itself only for long query blocks.
#include "kernels.h"
#include "mfma_lds.h"

namespace attn {

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int mha_len(const MhaParams& p, int b)
{
    return min(max(p.s[b], 0), p.s_max);
}

// Cache row of token t of sequence b.  Lanes hold different tokens here, so
// the block number is a per-lane load (clamped into the table and the pool
// like the wave-uniform lookup of the decode kernels).
__device__ __forceinline__ size_t mha_cache_row(const MhaParams& p, int b, int t)
{
    if (!p.bt) return (size_t)b * p.s_max + t;
    const int lb = min(t >> p.bs_log2, p.max_blocks - 1);
    const int blk = min(max(p.bt[(size_t)b * p.max_blocks + lb], 0), p.num_blocks - 1);
    return ((size_t)blk << p.bs_log2) + (t & ((1 << p.bs_log2) - 1));
}

// ---------------------------------------------------------------------------
// Expansion GEMM.  Workgroup = (sequence b, 128 tokens, 128 output columns of
// [K_n | V]); wavefront (wm, wn) takes 64 tokens x 64 columns as 2 x 2
// v_mfma_f32_32x32x16_bf16 tiles, the latent rows as the A operand and the
// weight rows as the B operand.  K = d_c = 512 in steps of 64: each step's
// 128 x 64 slices of both operands move global -> registers -> LDS with
// 16-byte loads, eight lanes per 128-byte row piece (whole lines), one step
// ahead of the products, which read their operands from LDS.  Tokens at or
// past the sequence's length read its last row and store nothing.
constexpr int kExTok = 128, kExCol = 128, kExK = 64;
constexpr int kExRow = kExK + 8;   // bf16 per LDS row (padded: 16 rows hit distinct banks)

__global__ __launch_bounds__(256, 2) void mla_expand_kernel(const MhaParams p)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][kExTok][kExRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kExCol][kExRow];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int wm = wave / 2, wn = wave % 2;
    const int ncol = p.h * 256 / kExCol;                  // column tiles of [K_n | V]
    const int ntok = (p.s_max + kExTok - 1) / kExTok;
    const int ct = blockIdx.x % ncol;
    const int tt = (blockIdx.x / ncol) % ntok;
    const int b = blockIdx.x / (ncol * ntok);
    const int n = mha_len(p, b);
    const int t0 = tt * kExTok;
    if (t0 >= n) return;
    const int hk = p.h * 128;                             // columns of K_n

    // loader: thread tid moves 16-byte piece tid % 8 of rows tid / 8 + 32 u
    const int seg = tid % 8, lrow = tid / 8;
    const uint16_t* ag[4];
    const uint16_t* bg[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
        const int row = lrow + 32 * u;
        const int t = min(t0 + row, n - 1);
        ag[u] = (const uint16_t*)p.cache + mha_cache_row(p, b, t) * 576 + 8 * seg;
        const int f = ct * kExCol + row;
        bg[u] = (f < hk ? (const uint16_t*)p.w_uk + (size_t)f * 512
                        : (const uint16_t*)p.w_uv + (size_t)(f - hk) * 512) + 8 * seg;
    }
    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define EX_GLOAD(k0)                                 \
    ra0 = *(const uint4*)(ag[0] + (k0));             \
    ra1 = *(const uint4*)(ag[1] + (k0));             \
    ra2 = *(const uint4*)(ag[2] + (k0));             \
    ra3 = *(const uint4*)(ag[3] + (k0));             \
    rb0 = *(const uint4*)(bg[0] + (k0));             \
    rb1 = *(const uint4*)(bg[1] + (k0));             \
    rb2 = *(const uint4*)(bg[2] + (k0));             \
    rb3 = *(const uint4*)(bg[3] + (k0));
#define EX_LSTORE(buf)                               \
    *(uint4*)&As[buf][lrow][8 * seg] = ra0;          \
    *(uint4*)&As[buf][lrow + 32][8 * seg] = ra1;     \
    *(uint4*)&As[buf][lrow + 64][8 * seg] = ra2;     \
    *(uint4*)&As[buf][lrow + 96][8 * seg] = ra3;     \
    *(uint4*)&Bs[buf][lrow][8 * seg] = rb0;          \
    *(uint4*)&Bs[buf][lrow + 32][8 * seg] = rb1;     \
    *(uint4*)&Bs[buf][lrow + 64][8 * seg] = rb2;     \
    *(uint4*)&Bs[buf][lrow + 96][8 * seg] = rb3;

    f32x16 acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int nt = 0; nt < 2; nt++)
#pragma unroll
            for (int e = 0; e < 16; e++) acc[mt][nt][e] = 0.f;

    const int r = lane % 32, hh = lane / 32;
    EX_GLOAD(0)
    EX_LSTORE(0)
    __syncthreads();
#pragma unroll 1
    for (int step = 0; step < 512 / kExK; step++) {
        const int buf = step & 1;
        if (step + 1 < 512 / kExK) {
            EX_GLOAD((step + 1) * kExK)
        }
#pragma unroll
        for (int ks = 0; ks < kExK / 16; ks++) {
            bf16x8 av[2], bv[2];
#pragma unroll
            for (int mt = 0; mt < 2; mt++) av[mt] = *(const bf16x8*)&As[buf][64 * wm + 32 * mt + r][16 * ks + 8 * hh];
#pragma unroll
            for (int nt = 0; nt < 2; nt++) bv[nt] = *(const bf16x8*)&Bs[buf][64 * wn + 32 * nt + r][16 * ks + 8 * hh];
#pragma unroll
            for (int mt = 0; mt < 2; mt++)
#pragma unroll
                for (int nt = 0; nt < 2; nt++) acc[mt][nt] = mfma_32x32x16(av[mt], bv[nt], acc[mt][nt]);
        }
        if (step + 1 < 512 / kExK) {
            EX_LSTORE(buf ^ 1)
        }
        __syncthreads();
    }
#undef EX_GLOAD
#undef EX_LSTORE

    // D tile layout: lane l holds column l % 32, rows 8 (e / 4) + 4 (l / 32) + e % 4
#pragma unroll
    for (int nt = 0; nt < 2; nt++) {
        const int f = ct * kExCol + 64 * wn + 32 * nt + r;
        uint16_t* dst;
        size_t stride;
        if (f < hk) {
            dst = p.k_exp + f;
            stride = (size_t)hk;
        } else {
            dst = p.v_exp + (f - hk);
            stride = (size_t)p.h * 128;
        }
#pragma unroll
        for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int e = 0; e < 16; e++) {
                const int t = t0 + 64 * wm + 32 * mt + 8 * (e / 4) + 4 * hh + e % 4;
                if (t < n) dst[((size_t)b * p.s_max + t) * stride] = (uint16_t)f32_to_bf16_bits(acc[mt][nt][e]);
            }
    }
}

// ---------------------------------------------------------------------------
// Attention.  Workgroup = (sequence b, head i, block of 128 query positions),
// eight wavefronts; wavefront w takes positions 16 w .. 16 w + 15 of the
// block.  Key tiles of 32 tokens go through LDS, double-buffered, loaded by
// all 512 threads with 16-byte loads: K rows [K_n (128) | k_R (64)] and V
// rows, both token-major as stored.
//   S^T[32 tokens x 16 queries] = K_tile . Q^T   (v_mfma_f32_16x16x32_bf16:
//     K rows as the A operand, the queries' 192 dims in registers as B)
//   online softmax per query (log2 domain), P rounded to bf16
//   O^T[128 dims x 16 queries] += V_tile^T . P^T: the score output gives
//     lane (query q, G) tokens 4 G .. 4 G + 3 and 16 + 4 G .. 16 + 4 G + 3,
//     the K order this product uses for both operands; the V operand comes
//     from transposing LDS reads (ds_read_b64_tr_b16) of those token rows
constexpr int kMhaW = 8;                   // wavefronts per workgroup
constexpr int kMhaQ = 16 * kMhaW;          // query positions per workgroup
constexpr int kMhaT = 32;                  // tokens per tile
constexpr int kKRow = 192 + 8;             // bf16 per K row in LDS (padded)
constexpr int kVRow = 128 + 16;            // bf16 per V row in LDS (padded)
constexpr int kMhaChunks = kMhaT * 40;     // 16-byte pieces of a tile (16 K_n, 8 k_R, 16 V per row)

__global__ __launch_bounds__(64 * kMhaW) void mla_mha_attn_kernel(const MhaParams p)
{
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kMhaT][kKRow];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kMhaT][kVRow];
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int qi = lane % 16, G = lane / 16;
    const int nqb = (p.q_len + kMhaQ - 1) / kMhaQ;
    const int qb = blockIdx.x % nqb;
    const int i = (blockIdx.x / nqb) % p.h;
    const int b = blockIdx.x / (nqb * p.h);
    const int n = mha_len(p, b);
    const int jq = qb * kMhaQ + 16 * wave + qi;          // this lane's query position
    const bool qv = jq < p.q_len;
    const int last = n - p.q_len + jq;                   // last token it sees (< 0: none)
    // tokens the workgroup needs: up to the last one its last position sees
    const int jmax = min(qb * kMhaQ + kMhaQ, p.q_len) - 1;
    const int t_end = max(min(n, n - p.q_len + jmax + 1), 0);
    const int nt = (t_end + kMhaT - 1) / kMhaT;
    // tokens this wavefront needs (its tiles past that only wait at barriers)
    const int wj = min(qb * kMhaQ + 16 * wave + 15, p.q_len - 1);
    const int w_end = max(min(n, n - p.q_len + wj + 1), 0);

    // this lane's query, dims 32 ks + 8 G .. + 7 (ks < 4: q_nope, else q_rope)
    bf16x8 qf[6];
    {
        const size_t row = ((size_t)b * p.q_len + min(jq, p.q_len - 1)) * p.h + i;
        const uint16_t* qn = (const uint16_t*)p.q_nope + row * 128;
        const uint16_t* qr = (const uint16_t*)p.q_rope + row * 64;
#pragma unroll
        for (int ks = 0; ks < 6; ks++) {
            const uint16_t* src = ks < 4 ? qn + 32 * ks + 8 * G : qr + 32 * (ks - 4) + 8 * G;
            qf[ks] = qv ? *(const bf16x8*)src : __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0));
        }
    }

    // tile loads: thread tid moves pieces tid, tid + 512, tid + 1024 (< 1280)
    uint4 ld0, ld1, ld2;
    auto src_of = [&](int c, int g) -> const uint4* {
        const int row = c / 40, k = c % 40;
        const int t = min(g * kMhaT + row, max(n - 1, 0));
        const size_t tok = (size_t)b * p.s_max + t;
        if (k < 16) return (const uint4*)(p.k_exp + (tok * p.h + i) * 128 + 8 * k);
        if (k < 24) return (const uint4*)((const uint16_t*)p.cache + mha_cache_row(p, b, t) * 576 + 512 + 8 * (k - 16));
        return (const uint4*)(p.v_exp + (tok * p.h + i) * 128 + 8 * (k - 24));
    };
    auto dst_of = [&](int c, int buf) -> uint4* {
        const int row = c / 40, k = c % 40;
        return k < 24 ? (uint4*)&Ks[buf][row][8 * k] : (uint4*)&Vs[buf][row][8 * (k - 24)];
    };
    const bool third = tid + 1024 < kMhaChunks;

    f32x4 o[8];
#pragma unroll
    for (int mc = 0; mc < 8; mc++) o[mc] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, l = 0.f;

    if (nt > 0) {
        ld0 = *src_of(tid, 0);
        ld1 = *src_of(tid + 512, 0);
        if (third) ld2 = *src_of(tid + 1024, 0);
        *dst_of(tid, 0) = ld0;
        *dst_of(tid + 512, 0) = ld1;
        if (third) *dst_of(tid + 1024, 0) = ld2;
    }
    __syncthreads();
    for (int g = 0; g < nt; g++) {
        const int buf = g & 1;
        if (g + 1 < nt) {
            ld0 = *src_of(tid, g + 1);
            ld1 = *src_of(tid + 512, g + 1);
            if (third) ld2 = *src_of(tid + 1024, g + 1);
        }
        if (g * kMhaT < w_end) {   // wave-uniform
            // scores: two 16-token blocks
            f32x4 s[2];
#pragma unroll
            for (int tb = 0; tb < 2; tb++) {
                s[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 6; ks++)
                    s[tb] = mfma16(*(const bf16x8*)&Ks[buf][16 * tb + qi][32 * ks + 8 * G], qf[ks], s[tb]);
            }
            // lane holds query qi of this wavefront, tokens 16 tb + 4 G + e
            float z[8];
            float tm = -INFINITY;
#pragma unroll
            for (int tb = 0; tb < 2; tb++)
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    const int t = g * kMhaT + 16 * tb + 4 * G + e;
                    const float v = t <= last && qv ? s[tb][e] * p.scale_log2 : -INFINITY;
                    z[4 * tb + e] = v;
                    tm = fmaxf(tm, v);
                }
            tm = fmaxf(tm, xor16(tm));
            tm = fmaxf(tm, xor32(tm));
            const float mn = fmaxf(m, tm);
            // rows that have seen nothing yet keep m = -inf and add nothing
            const float alpha = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mn);
            float ps = 0.f;
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float p0 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e] - mn);
                const float p1 = mn == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(z[e + 1] - mn);
                ps += p0 + p1;
                pk[e / 2] = pack_bf16x2(p0, p1);
            }
            ps += xor16(ps);
            ps += xor32(ps);
            l = l * alpha + ps;
            m = mn;
            const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
            // V operand of dims 16 mc .. + 15: source lane qi of group G points
            // at token 4 G + qi / 4 (then 16 + ...), dims 16 mc + 4 (qi % 4) ..
            const uint8_t* vb = (const uint8_t*)&Vs[buf][4 * G + qi / 4][4 * (qi % 4)];
#pragma unroll
            for (int mc = 0; mc < 8; mc++) {
                o[mc] *= alpha;
                const bf16x8 va = cat_tr(lds_read_tr(vb + 32 * mc), lds_read_tr(vb + 32 * mc + 16 * kVRow * 2));
                o[mc] = mfma16(va, pb, o[mc]);
            }
        }
        if (g + 1 < nt) {
            *dst_of(tid, buf ^ 1) = ld0;
            *dst_of(tid + 512, buf ^ 1) = ld1;
            if (third) *dst_of(tid + 1024, buf ^ 1) = ld2;
        }
        __syncthreads();
    }

    // O^T tile mc: lane holds query qi, dims 16 mc + 4 G + e
    if (qv) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
        const size_t row = ((size_t)b * p.q_len + jq) * p.h + i;
        uint16_t* dst = (uint16_t*)p.out + row * 128;
#pragma unroll
        for (int mc = 0; mc < 8; mc++) {
            const uint2 v = make_uint2(pack_bf16x2(o[mc][0] * inv, o[mc][1] * inv),
                                       pack_bf16x2(o[mc][2] * inv, o[mc][3] * inv));
            *(uint2*)(dst + 16 * mc + 4 * G) = v;
        }
        if (G == 0 && p.lse) p.lse[row] = l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
    }
}

hipError_t launch_mla_mha(const MhaParams& p, hipStream_t st)
{
    if (p.h <= 0 || p.B <= 0 || p.q_len <= 0 || p.s_max <= 0) return hipErrorInvalidValue;
    const long long g1 = (long long)p.B * ((p.s_max + kExTok - 1) / kExTok) * (p.h * 256 / kExCol);
    const long long g2 = (long long)p.B * p.h * ((p.q_len + kMhaQ - 1) / kMhaQ);
    if (g1 >= (1LL << 31) || g2 >= (1LL << 31)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mla_expand_kernel, dim3((unsigned)g1), dim3(256), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mla_mha_attn_kernel, dim3((unsigned)g2), dim3(64 * kMhaW), 0, st, p);
    return hipGetLastError();
}

}  // namespace attn
