// Host side of the C ABI declared in include/attn_decode.h: argument checks,
// the split plan, workspace carving and kernel launches.  No allocation; no
// global state except the thread-local error message and, for the no-alloc
// entry point, each device's scratch address (noalloc.hip).
#include "attn_decode.h"
#include "attn_stream_probe.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <string>

#include "kernels.h"

namespace {

thread_local std::string g_err = "no error";

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what)
{
    return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int x)
{
    int r = 0;
    while ((1 << r) < x) r++;
    return r;
}
long long cdiv(long long a, long long b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// ---- GQA split plan ---------------------------------------------------------
// bf16 caches with g <= 64 run on the matrix cores: work item = (b, KV head,
// token split) with all g query heads in one workgroup of 2 or 4 wavefronts
// (16 heads each; a wavefront without heads only issues its share of the
// tile DMA).  A 64 KB LDS ring per workgroup leaves room for two per CU, so
// splits are added until about 512 workgroups exist.
// Otherwise (fp32, or g > 64) the vector kernel runs: work item = (b, KV
// head, group of HG query heads, token split), HG the largest of 8, 4, 2, 1
// dividing g, one wavefront each, about 2048 of them (8 per CU).
// Either way no split is longer than 4096 tokens (with mixed lengths the
// longest sequences would otherwise set the kernel time) or shorter than 512
// tokens, and split lengths are multiples of 64 tokens.
// Several query positions per sequence (q_len > 1) always take the matrix
// cores: the g * q_len rows of a work item fill the 16-row tiles.  Up to 64
// rows take one workgroup of 16-row wavefronts; more take 4 wavefronts of
// two 16-row blocks each (rpw = 2), which read each tile once for 128 rows,
// in n_rb such workgroups.
struct GqaPlan {
    bool mfma;
    int HG, n_hg, NW, n_split, chunk, n_rb, rpw;
    size_t part_o_bytes, part_ml_bytes, ws_bytes;
};

#ifndef GQA_F8_TARGET
#define GQA_F8_TARGET 512
#endif
GqaPlan plan_gqa_path(bool mfma, int B, int s_max, int h, int h_kv, int d_h, bool f8 = false,
                      int q_len = 1)
{
    GqaPlan P{};
    const int g = h / h_kv;
    const int rows = g * q_len;
    P.mfma = mfma;
    P.n_rb = 1;
    P.rpw = 1;
    long long target;
    if (mfma) {
        P.HG = g;
        P.n_hg = 1;
        P.rpw = rows > 64 ? 2 : 1;
        P.n_rb = (rows + 64 * P.rpw - 1) / (64 * P.rpw);
        // two wavefronts at least: both issue the tile DMA, which keeps more
        // loads in flight per CU than one wavefront's counter allows
#ifndef GQA_NW_ROWS
#define GQA_NW_ROWS 32
#endif
#ifndef GQA_BF16_TARGET
#define GQA_BF16_TARGET 512
#endif
        // E4M3 tiles are half the bytes of bf16 ones: four wavefronts, which
        // issue the DMA of a tile in two instructions each, measured 5 % faster
        // than two on the contiguous Llama-3 layers (93.5 against 98.2 us at
        // 8B, 52.6 against 55.3 us at 70B B = 16); deeper rings or more
        // splits gave nothing on top
        P.NW = rows <= GQA_NW_ROWS && !f8 ? 2 : 4;
        target = f8 ? GQA_F8_TARGET : GQA_BF16_TARGET;
    } else {
        P.HG = (g % 8 == 0) ? 8 : (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
        P.n_hg = g / P.HG;
        P.NW = 1;
        target = 2048;
    }
#ifndef GQA_MAX_CHUNK
#define GQA_MAX_CHUNK 4096
#endif
#ifndef GQA_MIN_CHUNK
#define GQA_MIN_CHUNK 512
#endif
    const long long T = 64, min_chunk = GQA_MIN_CHUNK, max_chunk = GQA_MAX_CHUNK;
    const long long units = (long long)B * h_kv * P.n_hg * P.n_rb;
    long long ns = units > 0 ? cdiv(target, units) : 1;
    if (s_max > 0 && ns < cdiv(s_max, max_chunk)) ns = cdiv(s_max, max_chunk);
    const long long ns_max = s_max > 0 ? cdiv(s_max, min_chunk) : 1;
    if (ns > ns_max) ns = ns_max;
    if (ns < 1) ns = 1;
    long long chunk = s_max > 0 ? cdiv(cdiv(s_max, ns), T) * T : T;
    ns = s_max > 0 ? cdiv(s_max, chunk) : 1;
    P.n_split = (int)ns;
    P.chunk = (int)chunk;
    if (P.n_split > 1) {
        P.part_o_bytes = align256((size_t)B * q_len * h * P.n_split * d_h * sizeof(float));
        P.part_ml_bytes = align256((size_t)B * q_len * h * P.n_split * 2 * sizeof(float));
        // the arrival counters (the workspace's first kArriveBytes), then the partials
        P.ws_bytes = attn::kArriveBytes + P.part_o_bytes + P.part_ml_bytes;
    }
    return P;
}

bool gqa_uses_mfma(int h, int h_kv, int b) { return b == 2 && h / h_kv <= 64; }

GqaPlan plan_gqa(int B, int s_max, int h, int h_kv, int d_h, int b, int q_len = 1)
{
    if (b == 1) return plan_gqa_path(true, B, s_max, h, h_kv, d_h, true, q_len);
    if (q_len > 1) return plan_gqa_path(true, B, s_max, h, h_kv, d_h, false, q_len);
    return plan_gqa_path(gqa_uses_mfma(h, h_kv, b), B, s_max, h, h_kv, d_h);
}

// ---- MLA plan ----------------------------------------------------------------
// Decode runs as n_wg = 256 workgroups (one 4-wavefront group per CU), each
// taking an equal share of all cached 32-token tiles (at least 8 tiles);
// the shares are computed on the device from the lengths.  A workgroup
// leaves one partial per sequence it touches, so n_wg + B - 1 partial slots
// cover every schedule.
// new tokens per sequence that one multi-token MLA call takes
constexpr int kMlaMaxQLen = 1024;

struct MlaPlan {
    int n_wg, min_tiles;
    size_t qhat_bytes, part_u_bytes, part_ml_bytes, flag_bytes, sched_bytes, ws_bytes;
};

MlaPlan plan_mla(int B, int h, int d_c, int d_R)
{
    MlaPlan P{};
    P.n_wg = 256;
    P.min_tiles = 8;
    const size_t slots = (size_t)P.n_wg + B - 1;
    P.qhat_bytes = align256((size_t)B * ((h + 31) / 32) * 32 * (d_c + d_R) * 2);
    P.part_u_bytes = align256(slots * h * d_c * 2);   // fp16
    P.part_ml_bytes = align256(slots * h * 2 * sizeof(float));
    P.flag_bytes = align256((size_t)P.n_wg * sizeof(int32_t));
    P.sched_bytes = align256(((size_t)B + 1 + P.n_wg + 1) * sizeof(int32_t));
    // after the arrival-counter prefix that every workspace keeps
    P.ws_bytes = attn::kArriveBytes + P.qhat_bytes + P.part_u_bytes + P.part_ml_bytes + P.flag_bytes +
                 P.sched_bytes;
    return P;
}

int check_table(const int32_t* bt, int max_blocks, int block_size, int num_blocks, int s_max)
{
    if (!bt) {
        if (s_max <= 0) return fail(ATTN_EINVAL, "contiguous cache needs s_max > 0");
        return ATTN_OK;
    }
    if (!pow2(block_size) || block_size < 16)
        return fail(ATTN_EINVAL, "block_size must be a power of two >= 16 (got %d)", block_size);
    if (max_blocks <= 0 || num_blocks <= 0)
        return fail(ATTN_EINVAL, "paged cache needs max_blocks > 0 and num_blocks > 0");
    if ((long long)max_blocks * block_size < s_max)
        return fail(ATTN_EINVAL, "max_blocks * block_size (%lld) < s_max (%d)",
                    (long long)max_blocks * block_size, s_max);
    return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_kv_cell_bytes(int L, int h_kv, int d_h, int b)
{
    if (L < 0 || h_kv < 0 || d_h < 0 || b < 0) return 0;
    return (size_t)2 * (size_t)L * (size_t)h_kv * (size_t)d_h * (size_t)b;
}

size_t attn_mla_cell_bytes(int L, int d_c, int d_R, int b)
{
    if (L < 0 || d_c < 0 || d_R < 0 || b < 0) return 0;
    return (size_t)L * ((size_t)d_c + (size_t)d_R) * (size_t)b;
}

size_t attn_decode_workspace_bytes(int is_mla, int B, int s_max, int h, int h_kv, int d_h_or_dc,
                                   int d_R)
{
    if (B <= 0 || h <= 0 || s_max < 0 || d_h_or_dc <= 0) return 0;
    if (is_mla) return plan_mla(B, h, d_h_or_dc, d_R < 0 ? 0 : d_R).ws_bytes;
    if (h_kv <= 0 || h % h_kv != 0) return 0;
    // the storage type is not an argument: size for whichever kernel runs
    const size_t a = plan_gqa_path(true, B, s_max, h, h_kv, d_h_or_dc).ws_bytes;
    const size_t v = plan_gqa_path(false, B, s_max, h, h_kv, d_h_or_dc).ws_bytes;
    const size_t f = plan_gqa_path(true, B, s_max, h, h_kv, d_h_or_dc, true).ws_bytes;
    return a > v ? (a > f ? a : f) : (v > f ? v : f);
}

const char* attn_last_error(void) { return g_err.c_str(); }

int kv_cache_append(void* cache_k, void* cache_v, const void* k_new, const void* v_new,
                    const int32_t* pos, const int32_t* block_table, int max_blocks,
                    int block_size, int num_blocks, int B, int s_max, int h_kv, int d_h, int b,
                    void* stream)
{
    if (!cache_k || !k_new || !pos) return fail(ATTN_EINVAL, "null cache_k, k_new or pos");
    if ((cache_v == nullptr) != (v_new == nullptr))
        return fail(ATTN_EINVAL, "cache_v and v_new must both be set or both be NULL");
    if (B < 0 || h_kv <= 0 || d_h <= 0) return fail(ATTN_EINVAL, "bad sizes");
    if (b != 2 && b != 4) return fail(ATTN_EINVAL, "b must be 2 (bf16) or 4 (fp32)");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    attn::AppendParams pk{};
    pk.cache = cache_k;
    pk.src = k_new;
    pk.pos = pos;
    pk.bt = block_table;
    pk.max_blocks = max_blocks;
    pk.bs_log2 = block_table ? ilog2(block_size) : 0;
    pk.num_blocks = num_blocks;
    pk.s_max = s_max;
    pk.row_bytes = (long long)h_kv * d_h * b;
    attn::AppendParams pv = pk;
    pv.cache = cache_v;
    pv.src = v_new;
    hipError_t e = attn::launch_append(pk, cache_v ? &pv : nullptr, B, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_cache_append launch");
    return ATTN_OK;
}

}  // extern "C"

namespace {

// Shared body of the GQA entry points.  b = 2 (bf16) or 4 (fp32) caches, or
// b = 1: OCP E4M3 caches with per-tensor scales (q and out bf16).
int decode_gqa(void* out, float* lse, const void* q, const void* cache_k, const void* cache_v,
               const int32_t* s, const int32_t* block_table, int max_blocks, int block_size,
               int num_blocks, int B, int s_max, int h, int h_kv, int d_h, int b, float scale,
               float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
               void* stream, int q_len = 1, const float* k_scales = nullptr,
               const float* v_scales = nullptr, bool noalloc = false)
{
    if (!out || !q || !cache_k || !cache_v || !s)
        return fail(ATTN_EINVAL, "null out, q, cache_k, cache_v or s");
    if (B < 0 || h <= 0 || h_kv <= 0 || d_h <= 0 || s_max < 0)
        return fail(ATTN_EINVAL, "bad sizes (B=%d h=%d h_kv=%d d_h=%d s_max=%d)", B, h, h_kv,
                    d_h, s_max);
    if (h % h_kv != 0)
        return fail(ATTN_EINVAL, "num_heads (%d) is not divisible by num_kv_heads (%d)", h, h_kv);
    if (b != 1 && b != 2 && b != 4) return fail(ATTN_EINVAL, "b must be 2 (bf16) or 4 (fp32)");
    if (!((b <= 2 && (d_h == 64 || d_h == 128)) || (b == 4 && d_h == 64)))
        return fail(ATTN_ENOTSUP, "unsupported (b=%d, d_h=%d)", b, d_h);
    if (b == 1 && h / h_kv > 64)
        return fail(ATTN_ENOTSUP, "FP8 caches support h / h_kv <= 64 (got %d)", h / h_kv);
    if (q_len < 1 || q_len > 64) return fail(ATTN_EINVAL, "q_len must be 1 .. 64 (got %d)", q_len);
    if (q_len > 1 && b == 4) return fail(ATTN_ENOTSUP, "q_len > 1 needs a bf16 or FP8 cache");
    if (block_table || s_max > 0) {
        int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
        if (rc) return rc;
    }
    if (B == 0) return ATTN_OK;
    const GqaPlan P = plan_gqa(B, s_max, h, h_kv, d_h, b, q_len);
    if (noalloc) {   // the fixed per-device scratch replaces the caller's workspace
        if (P.ws_bytes > attn::kNoAllocScratchBytes)
            return fail(ATTN_ENOTSUP,
                        "attn_decode_gqa_noalloc: these sizes need %zu bytes of scratch, more than "
                        "its fixed %zu; use attn_decode_gqa with a workspace",
                        P.ws_bytes, attn::kNoAllocScratchBytes);
        workspace_bytes = attn::kNoAllocScratchBytes;
    }
    if (P.ws_bytes && (!workspace || workspace_bytes < P.ws_bytes))
        return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", P.ws_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    attn::GqaParams p{};
    p.out = out;
    p.lse = lse;
    p.q = q;
    p.k = cache_k;
    p.v = cache_v;
    p.s = s;
    p.bt = block_table;
    p.part_o = (float*)((char*)workspace + attn::kArriveBytes);
    p.part_ml = (float*)((char*)workspace + attn::kArriveBytes + P.part_o_bytes);
    p.max_blocks = max_blocks;
    p.bs_log2 = block_table ? ilog2(block_size) : 0;
    p.num_blocks = num_blocks;
    p.B = B;
    p.s_max = s_max;
    p.h = h;
    p.h_kv = h_kv;
    p.n_hg = P.n_hg;
    p.n_split = P.n_split;
    p.chunk = P.chunk;
    p.q_len = q_len;
    p.n_rb = P.n_rb;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)d_h);
    p.scale_log2 = sc * k_scale * 1.4426950408889634f;
    p.v_scale = v_scale;
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    // Matrix-core kernel with splits: the split partials are merged either
    // by the separate merge kernel (default) or, with ATTN_GQA_MERGE=fused
    // in the environment, inside the decode kernel by the last workgroup of
    // each (b, KV head, row block), which finds out through one arrival
    // counter per item in the workspace's prefix.  Measured on MI355X the
    // in-kernel form is no faster: its last workgroup waits for three
    // device-scope round trips (its stores, the counter, the other
    // partials), about what the second launch costs, and with many splits
    // per item one workgroup merges what the merge kernel spreads over many.
    p.arrive = nullptr;
    const char* mm = getenv("ATTN_GQA_MERGE");
    if (mm && strcmp(mm, "fused") == 0 && P.mfma && P.n_split > 1 &&
        (long long)B * h_kv * P.n_rb <= attn::kArriveCount &&
        P.part_o_bytes < ((size_t)1 << 31))   // 32-bit byte offsets into the partials
        p.arrive = (int32_t*)workspace;
    // matrix-core kernel over a paged pool with splits: workgroups go to the
    // non-empty (b, split) pairs only (each workgroup scans the B lengths to
    // find its pair, so only for moderate B); the grid is then a multiple of 8
    p.compact = P.mfma && block_table != nullptr && P.n_split > 1 && B <= 16 * 64;
    // matrix-core kernel over a contiguous cache: the KV heads are permuted so
    // that the XCD streaming a head column and the column's address bit 8
    // differ in parity (needs one workgroup per (b, head, split), h_kv a
    // multiple of the permuted group, and a 256-byte aligned cache)
    p.xpair = -1;
    {
        const int rbytes = d_h * (b == 1 ? 1 : 2);
        const int group = rbytes >= 256 ? 2 : rbytes == 128 ? 4 : 8;
        if (P.mfma && !block_table && P.n_rb == 1 && h_kv % group == 0 && (uintptr_t)cache_k % 256 == 0)
            p.xpair = (int)(((uintptr_t)cache_k >> 8) & 1);
    }
    long long grid = (long long)B * h_kv * P.n_hg * P.n_split * P.n_rb;
    if (p.compact) grid = (grid + 7) & ~7LL;
    if (grid >= (1LL << 31)) return fail(ATTN_ENOTSUP, "problem too large for one launch");
    // a paged pool's tiles gather 16-row pages: four wavefronts keep more of
    // their DMA in flight than two (measured 1-2 % faster; contiguous
    // caches are faster with two when the group has <= 32 rows)
    int NW = block_table && P.mfma ? 4 : P.NW;
    // E4M3 items of at most 16 rows: one wavefront computes and the other
    // issues all of the tile DMA, whose issue waits for room in the memory
    // pipeline.  Measured against four wavefronts that all issue (and the
    // first also computes): Llama-3-8B 89.9 against 93.1 us, 70B GQA-8 B = 16
    // 51.5 against 53.3 us, paged GQA-8 752 against 767 us; for bf16 the same
    // split was even or 1 % slower
    int ni = 0;
    if (P.mfma && b == 1 && (h / h_kv) * q_len <= 16) {
        NW = 2;
        ni = 1;
    }
    hipError_t e = P.mfma ? attn::launch_gqa_mfma(p, d_h, NW, P.rpw, ni, block_table != nullptr, b == 1,
                                                  (unsigned)grid, (hipStream_t)stream)
                          : attn::launch_gqa_decode(p, d_h, b == 4, P.HG, block_table != nullptr,
                                                    (unsigned)grid, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_gqa launch");
    return ATTN_OK;
}

}  // namespace

extern "C" {

int kv_cache_append_fp8(void* cache_k, void* cache_v, const void* k_new, const void* v_new,
                        float k_scale, float v_scale, const int32_t* pos,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int s_max, int h_kv, int d_h, void* stream)
{
    if (!cache_k || !k_new || !pos) return fail(ATTN_EINVAL, "null cache_k, k_new or pos");
    if ((cache_v == nullptr) != (v_new == nullptr))
        return fail(ATTN_EINVAL, "cache_v and v_new must both be set or both be NULL");
    if (B < 0 || h_kv <= 0 || d_h <= 0 || (h_kv * d_h) % 4 != 0)
        return fail(ATTN_EINVAL, "bad sizes (h_kv * d_h must be a positive multiple of 4)");
    if (!(k_scale > 0.f) || isinf(k_scale) || (cache_v && (!(v_scale > 0.f) || isinf(v_scale))))
        return fail(ATTN_EINVAL, "scales must be positive and finite");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    attn::AppendParams pk{};
    pk.cache = cache_k;
    pk.src = k_new;
    pk.pos = pos;
    pk.bt = block_table;
    pk.max_blocks = max_blocks;
    pk.bs_log2 = block_table ? ilog2(block_size) : 0;
    pk.num_blocks = num_blocks;
    pk.s_max = s_max;
    pk.row_bytes = (long long)h_kv * d_h;   // one byte per code
    pk.inv_scale = 1.0f / k_scale;
    pk.inv_scale2 = pk.inv_scale;
    pk.split = pk.row_bytes;
    attn::AppendParams pv = pk;
    pv.cache = cache_v;
    pv.src = v_new;
    pv.inv_scale = cache_v ? 1.0f / v_scale : 1.0f;
    pv.inv_scale2 = pv.inv_scale;
    hipError_t e = attn::launch_append_fp8(pk, cache_v ? &pv : nullptr, B, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_cache_append_fp8 launch");
    return ATTN_OK;
}

int kv_cache_append_mla_fp8(void* cache, const void* kv_new, float c_scale, float r_scale,
                            const int32_t* pos, const int32_t* block_table, int max_blocks,
                            int block_size, int num_blocks, int B, int s_max, int d_c, int d_R,
                            void* stream)
{
    if (!cache || !kv_new || !pos) return fail(ATTN_EINVAL, "null cache, kv_new or pos");
    if (B < 0 || d_c <= 0 || d_R < 0 || d_c % 4 != 0 || d_R % 4 != 0)
        return fail(ATTN_EINVAL, "bad sizes (d_c and d_R must be multiples of 4)");
    if (!(c_scale > 0.f) || isinf(c_scale) || !(r_scale > 0.f) || isinf(r_scale))
        return fail(ATTN_EINVAL, "scales must be positive and finite");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    attn::AppendParams pk{};
    pk.cache = cache;
    pk.src = kv_new;
    pk.pos = pos;
    pk.bt = block_table;
    pk.max_blocks = max_blocks;
    pk.bs_log2 = block_table ? ilog2(block_size) : 0;
    pk.num_blocks = num_blocks;
    pk.s_max = s_max;
    pk.row_bytes = (long long)d_c + d_R;
    pk.inv_scale = 1.0f / c_scale;
    pk.inv_scale2 = 1.0f / r_scale;
    pk.split = d_c;
    hipError_t e = attn::launch_append_fp8(pk, nullptr, B, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_cache_append_mla_fp8 launch");
    return ATTN_OK;
}

int kv_cache_append_mla_fp8_paged_scales(void* cache, const void* kv_new, const float* c_scales,
                                         const float* r_scales, const int32_t* pos,
                                         const int32_t* block_table, int max_blocks,
                                         int block_size, int num_blocks, int B, int s_max,
                                         int d_c, int d_R, void* stream)
{
    if (!cache || !kv_new || !pos || !c_scales || !r_scales)
        return fail(ATTN_EINVAL, "null cache, kv_new, pos or scales");
    if (!block_table) return fail(ATTN_EINVAL, "per-page scales need a paged cache (block_table)");
    if (B < 0 || d_c <= 0 || d_R < 0 || d_c % 4 != 0 || d_R % 4 != 0)
        return fail(ATTN_EINVAL, "bad sizes (d_c and d_R must be multiples of 4)");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    attn::AppendParams pk{};
    pk.cache = cache;
    pk.src = kv_new;
    pk.pos = pos;
    pk.bt = block_table;
    pk.max_blocks = max_blocks;
    pk.bs_log2 = ilog2(block_size);
    pk.num_blocks = num_blocks;
    pk.s_max = s_max;
    pk.row_bytes = (long long)d_c + d_R;
    pk.inv_scale = pk.inv_scale2 = 1.f;
    pk.split = d_c;
    pk.page_scales = c_scales;
    pk.page_scales2 = r_scales;
    pk.d_h = d_c + d_R;
    hipError_t e = attn::launch_append_fp8(pk, nullptr, B, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_cache_append_mla_fp8_paged_scales launch");
    return ATTN_OK;
}

int attn_decode_gqa(void* out, float* lse, const void* q, const void* cache_k,
                    const void* cache_v, const int32_t* s, const int32_t* block_table,
                    int max_blocks, int block_size, int num_blocks, int B, int s_max, int h,
                    int h_kv, int d_h, int b, float scale, void* workspace,
                    size_t workspace_bytes, void* stream)
{
    if (b != 2 && b != 4) return fail(ATTN_EINVAL, "b must be 2 (bf16) or 4 (fp32)");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, b, scale, 1.f, 1.f, workspace,
                      workspace_bytes, stream);
}

int attn_decode_gqa_noalloc(void* out, float* lse, const void* q, const void* cache_k,
                            const void* cache_v, const int32_t* s, const int32_t* block_table,
                            int max_blocks, int block_size, int num_blocks, int B, int s_max,
                            int h, int h_kv, int d_h, int b, float scale, void* stream)
{
    // the device's scratch address, looked up on the first call on it
    void* ws = nullptr;
    const hipError_t e = attn::noalloc_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_gqa_noalloc scratch lookup");
    if (b != 2 && b != 4) return fail(ATTN_EINVAL, "b must be 2 (bf16) or 4 (fp32)");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, b, scale, 1.f, 1.f, ws, 0, stream, 1,
                      nullptr, nullptr, true);
}

int attn_decode_gqa_fp8(void* out, float* lse, const void* q, const void* cache_k,
                        const void* cache_v, float k_scale, float v_scale, const int32_t* s,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int s_max, int h, int h_kv, int d_h, float scale,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || isinf(k_scale) || isinf(v_scale))
        return fail(ATTN_EINVAL, "k_scale and v_scale must be positive and finite");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, 1, scale, k_scale, v_scale, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Shared body of the MLA entry points: b = 2 (bf16 cache) or b = 1 (E4M3
// cache codes with a latent and a rotary scale); q_len new tokens per
// sequence, each (sequence, position) pair one query row of the kernels.
// out == nullptr (only with u_bf16): no value up-projection; u~ leaves as
// bf16 [B q_len, h, d_c] in u_bf16 and w_uv, d_v are unused.
int decode_mla(void* out, float* u_latent, float* lse, const void* q_nope, const void* q_rope,
               const void* w_uk, const void* w_uv, const void* cache, float c_scale,
               float r_scale, const int32_t* s, const int32_t* block_table, int max_blocks,
               int block_size, int num_blocks, int B, int q_len, int s_max, int h, int d_c,
               int d_R, int d_nope, int d_v, int b, float scale, void* workspace,
               size_t workspace_bytes, void* stream, uint16_t* u_bf16 = nullptr,
               const float* c_scales = nullptr, const float* r_scales = nullptr)
{
    const bool up = out != nullptr;
    if ((!up && !u_bf16) || !q_nope || !q_rope || !w_uk || (up && !w_uv) || !cache || !s)
        return fail(ATTN_EINVAL, "null out, q_nope, q_rope, w_uk, w_uv, cache or s");
    if (!up) d_v = 16;   // unused
    if (B < 0 || h <= 0 || d_c <= 0 || d_R < 0 || d_nope <= 0 || d_v <= 0 || s_max < 0)
        return fail(ATTN_EINVAL, "bad sizes");
    if (q_len < 1 || q_len > kMlaMaxQLen)
        return fail(ATTN_EINVAL, "q_len must be in 1 .. %d (got %d)", kMlaMaxQLen, q_len);
    if (b != 2 && b != 1) return fail(ATTN_ENOTSUP, "MLA supports bf16 storage only (b=2)");
    if (d_c != 512 || d_R != 64)
        return fail(ATTN_ENOTSUP, "MLA supports d_c=512, d_R=64 (got %d, %d)", d_c, d_R);
    if (h % 16 != 0 || h > 128) return fail(ATTN_ENOTSUP, "MLA needs h a multiple of 16, <= 128");
    if ((long long)B * q_len * s_max >= (1LL << 31) || (long long)B * q_len >= (1LL << 24))
        return fail(ATTN_ENOTSUP, "problem too large for one launch");
    if (d_nope % 32 != 0 || d_nope > 256 || d_v % 16 != 0 || d_v > 256)
        return fail(ATTN_ENOTSUP, "MLA needs d_nope a multiple of 32, d_v of 16, both <= 256");
    if (block_table || s_max > 0) {
        int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
        if (rc) return rc;
    }
    if (B == 0) return ATTN_OK;
    const MlaPlan P = plan_mla(B * q_len, h, d_c, d_R);
    if (!workspace || workspace_bytes < P.ws_bytes)
        return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", P.ws_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    attn::MlaParams p{};
    p.out = out;
    p.u_latent = u_latent;
    p.lse = lse;
    p.q_nope = q_nope;
    p.q_rope = q_rope;
    p.w_uk = w_uk;
    p.w_uv = w_uv;
    p.cache = cache;
    p.s = s;
    p.bt = block_table;
    char* ws = (char*)workspace + attn::kArriveBytes;   // past the arrival counters
    p.qhat = (uint16_t*)ws;
    p.part_u = (_Float16*)(ws + P.qhat_bytes);
    p.part_ml = (float*)(ws + P.qhat_bytes + P.part_u_bytes);
    p.flags = (int32_t*)(ws + P.qhat_bytes + P.part_u_bytes + P.part_ml_bytes);
    p.sched = (int32_t*)(ws + P.qhat_bytes + P.part_u_bytes + P.part_ml_bytes + P.flag_bytes);
    p.max_blocks = max_blocks;
    p.bs_log2 = block_table ? ilog2(block_size) : 0;
    p.num_blocks = num_blocks;
    p.B = B * q_len;
    p.q_len = q_len;
    p.s_max = s_max;
    p.h = h;
    p.d_c = d_c;
    p.d_R = d_R;
    p.d_nope = d_nope;
    p.d_v = d_v;
    p.n_wg = P.n_wg;
    p.min_tiles = P.min_tiles;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)(d_nope + d_R));
    p.scale_log2 = sc * 1.4426950408889634f;
    p.f8 = b == 1;
    p.c_scale = c_scale;
    p.r_scale = r_scale;
    p.c_scales = c_scales;
    p.r_scales = r_scales;
    p.u_bf16 = u_bf16;
    hipError_t e = attn::launch_mla(p, block_table != nullptr, (hipStream_t)stream);
    if (e == hipErrorNotSupported) return fail(ATTN_ENOTSUP, "MLA kernels not built");
    if (e != hipSuccess) return hip_fail(e, "attn_decode_mla_absorbed launch");
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla_absorbed(void* out, float* u_latent, float* lse, const void* q_nope,
                             const void* q_rope, const void* w_uk, const void* w_uv,
                             const void* cache, const int32_t* s, const int32_t* block_table,
                             int max_blocks, int block_size, int num_blocks, int B, int s_max,
                             int h, int d_c, int d_R, int d_nope, int d_v, int b, float scale,
                             void* workspace, size_t workspace_bytes, void* stream)
{
    if (b != 2) return fail(ATTN_ENOTSUP, "MLA supports bf16 storage only (b=2)");
    return decode_mla(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1.f, 1.f, s,
                      block_table, max_blocks, block_size, num_blocks, B, 1, s_max, h, d_c, d_R,
                      d_nope, d_v, b, scale, workspace, workspace_bytes, stream);
}

int attn_decode_mla_absorbed_fp8(void* out, float* u_latent, float* lse, const void* q_nope,
                                 const void* q_rope, const void* w_uk, const void* w_uv,
                                 const void* cache, float c_scale, float r_scale,
                                 const int32_t* s, const int32_t* block_table, int max_blocks,
                                 int block_size, int num_blocks, int B, int s_max, int h, int d_c,
                                 int d_R, int d_nope, int d_v, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    if (!(c_scale > 0.f) || isinf(c_scale) || !(r_scale > 0.f) || isinf(r_scale))
        return fail(ATTN_EINVAL, "c_scale and r_scale must be positive and finite");
    return decode_mla(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, c_scale, r_scale, s,
                      block_table, max_blocks, block_size, num_blocks, B, 1, s_max, h, d_c, d_R,
                      d_nope, d_v, 1, scale, workspace, workspace_bytes, stream);
}

int attn_decode_mla_absorbed_fp8_paged_scales(void* out, float* u_latent, float* lse,
                                              const void* q_nope, const void* q_rope,
                                              const void* w_uk, const void* w_uv,
                                              const void* cache, const float* c_scales,
                                              const float* r_scales, const int32_t* s,
                                              const int32_t* block_table, int max_blocks,
                                              int block_size, int num_blocks, int B, int s_max,
                                              int h, int d_c, int d_R, int d_nope, int d_v,
                                              float scale, void* workspace,
                                              size_t workspace_bytes, void* stream)
{
    if (!c_scales || !r_scales) return fail(ATTN_EINVAL, "null c_scales or r_scales");
    if (!block_table) return fail(ATTN_EINVAL, "per-page scales need a paged cache (block_table)");
    return decode_mla(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1.f, 1.f, s,
                      block_table, max_blocks, block_size, num_blocks, B, 1, s_max, h, d_c, d_R,
                      d_nope, d_v, 1, scale, workspace, workspace_bytes, stream, nullptr,
                      c_scales, r_scales);
}

int attn_decode_mla_absorbed_multi(void* out, float* u_latent, float* lse, const void* q_nope,
                                   const void* q_rope, const void* w_uk, const void* w_uv,
                                   const void* cache, const int32_t* s,
                                   const int32_t* block_table, int max_blocks, int block_size,
                                   int num_blocks, int B, int q_len, int s_max, int h, int d_c,
                                   int d_R, int d_nope, int d_v, int b, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream)
{
    if (b != 2) return fail(ATTN_ENOTSUP, "MLA supports bf16 storage only (b=2)");
    return decode_mla(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1.f, 1.f, s,
                      block_table, max_blocks, block_size, num_blocks, B, q_len, s_max, h, d_c,
                      d_R, d_nope, d_v, b, scale, workspace, workspace_bytes, stream);
}

int attn_decode_mla_absorbed_multi_fp8(void* out, float* u_latent, float* lse,
                                       const void* q_nope, const void* q_rope, const void* w_uk,
                                       const void* w_uv, const void* cache, float c_scale,
                                       float r_scale, const int32_t* s,
                                       const int32_t* block_table, int max_blocks,
                                       int block_size, int num_blocks, int B, int q_len,
                                       int s_max, int h, int d_c, int d_R, int d_nope, int d_v,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream)
{
    if (!(c_scale > 0.f) || isinf(c_scale) || !(r_scale > 0.f) || isinf(r_scale))
        return fail(ATTN_EINVAL, "c_scale and r_scale must be positive and finite");
    return decode_mla(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, c_scale, r_scale, s,
                      block_table, max_blocks, block_size, num_blocks, B, q_len, s_max, h, d_c,
                      d_R, d_nope, d_v, 1, scale, workspace, workspace_bytes, stream);
}

size_t attn_decode_mla_multi_workspace_bytes(int B, int q_len, int h, int d_c, int d_R)
{
    if (B <= 0 || q_len < 1 || q_len > kMlaMaxQLen || h <= 0 || d_c <= 0 || d_R < 0) return 0;
    if ((long long)B * q_len >= (1LL << 24)) return 0;
    return plan_mla(B * q_len, h, d_c, d_R).ws_bytes;
}

}  // extern "C"

namespace {

// ---- MLA output projection ------------------------------------------------
// Y [rows, d_model] = X [rows, K] W^T, K = h d_v (deferred: X = the heads'
// outputs, W = W_O) or h d_c (merged: X = bf16 u~, W = W_abs).  The K range
// is split over workgroups until about kProjWgTarget of them exist (4 per
// CU: the stream over W then has enough loads in flight), each wavefront
// keeping at least two 128-wide K steps.
#ifndef ATTN_PROJ_WG_TARGET
#define ATTN_PROJ_WG_TARGET 1024
#endif
constexpr int kProjWgTarget = ATTN_PROJ_WG_TARGET;

int proj_splits(int rows, int d_model, int K)
{
    const long long mblk = rows <= 32 ? 1 : cdiv(rows, 64);
    const long long wg = (long long)(d_model / 32) * mblk;
    const long long steps = K / 128;
    long long ks = cdiv(kProjWgTarget, wg);
    ks = ks < steps / 8 ? ks : steps / 8;
    return (int)(ks < 1 ? 1 : ks);
}

struct OutPlan {
    MlaPlan mla;
    int ks;
    size_t x_bytes, part_bytes, ws_bytes;
};

OutPlan plan_out(bool merged, int rows, int h, int d_c, int d_R, int d_v, int d_model)
{
    OutPlan P{};
    P.mla = plan_mla(rows, h, d_c, d_R);
    const int K = merged ? h * d_c : h * d_v;
    P.ks = proj_splits(rows, d_model, K);
    P.x_bytes = align256((size_t)rows * K * 2);
    P.part_bytes = P.ks > 1 ? align256((size_t)P.ks * rows * d_model * 4) : 0;
    P.ws_bytes = P.mla.ws_bytes + P.x_bytes + P.part_bytes;
    return P;
}

int check_out_sizes(bool merged, int B, int q_len, int h, int d_c, int d_v, int d_model)
{
    if (B < 0 || q_len < 1 || q_len > kMlaMaxQLen || h <= 0 || d_c <= 0 || d_model <= 0 ||
        (!merged && d_v <= 0))
        return fail(ATTN_EINVAL, "bad sizes");
    if (d_model % 32 != 0)
        return fail(ATTN_ENOTSUP, "d_model must be a multiple of 32 (got %d)", d_model);
    const long long K = merged ? (long long)h * d_c : (long long)h * d_v;
    if (K % 128 != 0) return fail(ATTN_ENOTSUP, "h * %s must be a multiple of 128",
                                  merged ? "d_c" : "d_v");
    if ((long long)B * q_len * K * 2 + 2 * K >= (1LL << 31) ||
        (long long)d_model * K * 2 >= (1LL << 32))
        return fail(ATTN_ENOTSUP, "problem too large for one launch");
    return ATTN_OK;
}

// Shared body of the two output-path entry points.
int decode_mla_out(bool merged, void* out, float* lse, const void* q_nope, const void* q_rope,
                   const void* w_uk, const void* w_uv, const void* w_proj, const void* cache,
                   const int32_t* s, const int32_t* block_table, int max_blocks, int block_size,
                   int num_blocks, int B, int q_len, int s_max, int h, int d_c, int d_R,
                   int d_nope, int d_v, int d_model, int b, float scale, void* workspace,
                   size_t workspace_bytes, void* stream)
{
    if (!out || !w_proj) return fail(ATTN_EINVAL, "null out or projection weight");
    if (b != 2) return fail(ATTN_ENOTSUP, "MLA supports bf16 storage only (b=2)");
    int rc = check_out_sizes(merged, B, q_len, h, d_c, d_v, d_model);
    if (rc) return rc;
    if (B == 0) return ATTN_OK;
    const int rows = B * q_len;
    const OutPlan P = plan_out(merged, rows, h, d_c, d_R, d_v, d_model);
    if (!workspace || workspace_bytes < P.ws_bytes)
        return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", P.ws_bytes,
                    workspace ? workspace_bytes : (size_t)0);
    char* ws = (char*)workspace;
    uint16_t* x = (uint16_t*)(ws + P.mla.ws_bytes);
    rc = decode_mla(merged ? nullptr : (void*)x, nullptr, lse, q_nope, q_rope, w_uk,
                    merged ? nullptr : w_uv, cache, 1.f, 1.f, s, block_table, max_blocks,
                    block_size, num_blocks, B, q_len, s_max, h, d_c, d_R, d_nope, d_v, b, scale,
                    workspace, P.mla.ws_bytes, stream, merged ? x : nullptr);
    if (rc) return rc;
    attn::ProjParams pp{};
    pp.x = x;
    pp.w = (const uint16_t*)w_proj;
    pp.y = out;
    pp.part = P.ks > 1 ? (float*)(ws + P.mla.ws_bytes + P.x_bytes) : nullptr;
    pp.M = rows;
    pp.N = d_model;
    pp.K = merged ? h * d_c : h * d_v;
    pp.ks = P.ks;
    pp.y_f32 = 0;
    hipError_t e = attn::launch_proj(pp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "MLA output projection launch");
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_mla_out(void* out, float* lse, const void* q_nope, const void* q_rope,
                        const void* w_uk, const void* w_uv, const void* w_o, const void* cache,
                        const int32_t* s, const int32_t* block_table, int max_blocks,
                        int block_size, int num_blocks, int B, int q_len, int s_max, int h,
                        int d_c, int d_R, int d_nope, int d_v, int d_model, int b, float scale,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    return decode_mla_out(false, out, lse, q_nope, q_rope, w_uk, w_uv, w_o, cache, s,
                          block_table, max_blocks, block_size, num_blocks, B, q_len, s_max, h,
                          d_c, d_R, d_nope, d_v, d_model, b, scale, workspace, workspace_bytes,
                          stream);
}

int attn_decode_mla_out_premerged(void* out, float* lse, const void* q_nope, const void* q_rope,
                                  const void* w_uk, const void* w_absorbed, const void* cache,
                                  const int32_t* s, const int32_t* block_table, int max_blocks,
                                  int block_size, int num_blocks, int B, int q_len, int s_max,
                                  int h, int d_c, int d_R, int d_nope, int d_model, int b,
                                  float scale, void* workspace, size_t workspace_bytes,
                                  void* stream)
{
    return decode_mla_out(true, out, lse, q_nope, q_rope, w_uk, nullptr, w_absorbed, cache, s,
                          block_table, max_blocks, block_size, num_blocks, B, q_len, s_max, h,
                          d_c, d_R, d_nope, 0, d_model, b, scale, workspace, workspace_bytes,
                          stream);
}

size_t attn_decode_mla_out_workspace_bytes(int premerged, int B, int q_len, int h, int d_c,
                                           int d_R, int d_v, int d_model)
{
    const bool merged = premerged != 0;
    if (B <= 0 || d_R < 0) return 0;
    const std::string keep = g_err;   // a size query leaves the error message alone
    const int rc = check_out_sizes(merged, B, q_len, h, d_c, d_v, d_model);
    g_err = keep;
    if (rc) return 0;
    return plan_out(merged, B * q_len, h, d_c, d_R, d_v, d_model).ws_bytes;
}

int attn_mla_premerge_weights(void* w_absorbed, const void* w_o, const void* w_uv, int h,
                              int d_c, int d_v, int d_model, void* stream)
{
    if (!w_absorbed || !w_o || !w_uv) return fail(ATTN_EINVAL, "null weight");
    if (h <= 0 || d_c <= 0 || d_v <= 0 || d_model <= 0) return fail(ATTN_EINVAL, "bad sizes");
    if (d_c % 256 != 0 || d_model % 32 != 0 || d_v > 256)
        return fail(ATTN_ENOTSUP, "premerge needs d_c %% 256 == 0, d_model %% 32 == 0, d_v <= 256");
    if ((long long)d_model * h * d_c >= (1LL << 31))
        return fail(ATTN_ENOTSUP, "merged weight too large");
    attn::PremergeParams pp{w_absorbed, w_o, w_uv, h, d_c, d_v, d_model};
    hipError_t e = attn::launch_premerge(pp, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attn_mla_premerge_weights launch");
    return ATTN_OK;
}

size_t attn_decode_mla_mha_workspace_bytes(int B, int s_max, int h)
{
    if (B <= 0 || s_max <= 0 || h <= 0) return 0;
    // the arrival-counter prefix, then the expanded K and V
    return attn::kArriveBytes + 2 * align256((size_t)B * s_max * h * 128 * 2);
}

int attn_decode_mla_mha(void* out, float* lse, const void* q_nope, const void* q_rope,
                        const void* w_uk, const void* w_uv, const void* cache, const int32_t* s,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int q_len, int s_max, int h, int d_c, int d_R,
                        int d_nope, int d_v, int b, float scale, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    if (!out || !q_nope || !q_rope || !w_uk || !w_uv || !cache || !s)
        return fail(ATTN_EINVAL, "null out, q_nope, q_rope, w_uk, w_uv, cache or s");
    if (B < 0 || q_len < 1 || h <= 0 || s_max <= 0)
        return fail(ATTN_EINVAL, "bad sizes");
    if (b != 2) return fail(ATTN_ENOTSUP, "MHA mode supports bf16 storage only (b=2)");
    if (d_c != 512 || d_R != 64 || d_nope != 128 || d_v != 128)
        return fail(ATTN_ENOTSUP, "MHA mode supports d_c=512, d_R=64, d_nope=d_v=128");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    if ((long long)B * q_len * h >= (1LL << 31) || (long long)B * s_max >= (1LL << 31))
        return fail(ATTN_ENOTSUP, "problem too large for one launch");
    if (B == 0) return ATTN_OK;
    const size_t need = attn_decode_mla_mha_workspace_bytes(B, s_max, h);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_EWORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    attn::MhaParams p{};
    p.out = out;
    p.lse = lse;
    p.q_nope = q_nope;
    p.q_rope = q_rope;
    p.w_uk = w_uk;
    p.w_uv = w_uv;
    p.cache = cache;
    p.s = s;
    p.bt = block_table;
    const size_t half = (need - attn::kArriveBytes) / 2;
    p.k_exp = (uint16_t*)((char*)workspace + attn::kArriveBytes);
    p.v_exp = (uint16_t*)((char*)workspace + attn::kArriveBytes + half);
    p.max_blocks = max_blocks;
    p.bs_log2 = block_table ? ilog2(block_size) : 0;
    p.num_blocks = num_blocks;
    p.B = B;
    p.q_len = q_len;
    p.s_max = s_max;
    p.h = h;
    const float sc = scale > 0.f ? scale : 1.0f / sqrtf((float)(d_nope + d_R));
    p.scale_log2 = sc * 1.4426950408889634f;
    hipError_t e = attn::launch_mla_mha(p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_mla_mha launch");
    return ATTN_OK;
}

int attn_mla_mode(int q_len, int s)
{
    if (q_len < 1 || s < 1) return -1;
    // Per head, with this library's kernels on MI355X (bf16, d_c 512,
    // d_R 64, d_nope = d_v = 128): the absorbed form costs about c_a per
    // (query, token), MHA mode c_e per cached token for the expansion plus
    // c_m per (query, token).  Measured: c_e = 0.64 ns; c_a - c_m = 2.7 ps at
    // s = 2048 and 1.7 ps at s = 8192 (taken linear in log2 s between,
    // constant outside).  MHA mode wins once q_len (c_a - c_m) > c_e.
    const double ls = log2((double)s);
    const double gap = ls <= 11.0 ? 2.7e-12 : ls >= 13.0 ? 1.7e-12 : 2.7e-12 - 0.5e-12 * (ls - 11.0);
    return (double)q_len * gap > 0.64e-9 ? 1 : 0;
}

int attn_mla_out_form(int B, int q_len, int h, int d_c, int d_v, int d_model)
{
    if (B <= 0 || q_len < 1 || h <= 0 || d_c <= 0 || d_v <= 0 || d_model <= 0) return -1;
    const double rows = (double)B * q_len;
    // bytes and matrix-core flops of what differs between the two forms
    const double bd = 2.0 * h * d_v * d_c + 2.0 * d_model * h * d_v + 4.0 * rows * h * d_v;
    const double fd = 2.0 * rows * h * d_v * d_c + 2.0 * rows * d_model * h * d_v;
    const double bm = 2.0 * d_model * h * d_c + 4.0 * rows * h * d_c;
    const double fm = 2.0 * rows * d_model * h * d_c;
    const double hbm = 8.0e12, mfma = 2.5e15;   // MI355X HBM3E bytes/s, dense bf16 flop/s
    const double td = bd / hbm > fd / mfma ? bd / hbm : fd / mfma;
    const double tm = bm / hbm > fm / mfma ? bm / hbm : fm / mfma;
    return tm < td ? 1 : 0;
}

int attn_decode_gqa_multi(void* out, float* lse, const void* q, const void* cache_k,
                          const void* cache_v, const int32_t* s, const int32_t* block_table,
                          int max_blocks, int block_size, int num_blocks, int B, int q_len,
                          int s_max, int h, int h_kv, int d_h, int b, float scale, void* workspace,
                          size_t workspace_bytes, void* stream)
{
    if (b != 2) return fail(ATTN_ENOTSUP, "attn_decode_gqa_multi needs a bf16 cache (b = 2)");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, b, scale, 1.f, 1.f, workspace,
                      workspace_bytes, stream, q_len);
}

int attn_decode_gqa_multi_fp8(void* out, float* lse, const void* q, const void* cache_k,
                              const void* cache_v, float k_scale, float v_scale, const int32_t* s,
                              const int32_t* block_table, int max_blocks, int block_size,
                              int num_blocks, int B, int q_len, int s_max, int h, int h_kv,
                              int d_h, float scale, void* workspace, size_t workspace_bytes,
                              void* stream)
{
    if (!(k_scale > 0.f) || !(v_scale > 0.f) || isinf(k_scale) || isinf(v_scale))
        return fail(ATTN_EINVAL, "k_scale and v_scale must be positive and finite");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, 1, scale, k_scale, v_scale, workspace,
                      workspace_bytes, stream, q_len);
}

int attn_decode_gqa_fp8_paged_scales(void* out, float* lse, const void* q, const void* cache_k,
                                     const void* cache_v, const float* k_scales,
                                     const float* v_scales, const int32_t* s,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, int B, int s_max, int h, int h_kv, int d_h,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     void* stream)
{
    if (!k_scales || !v_scales) return fail(ATTN_EINVAL, "null k_scales or v_scales");
    if (!block_table) return fail(ATTN_EINVAL, "per-page scales need a paged cache (block_table)");
    return decode_gqa(out, lse, q, cache_k, cache_v, s, block_table, max_blocks, block_size,
                      num_blocks, B, s_max, h, h_kv, d_h, 1, scale, 1.f, 1.f, workspace,
                      workspace_bytes, stream, 1, k_scales, v_scales);
}

int kv_cache_append_fp8_paged_scales(void* cache_k, void* cache_v, const void* k_new,
                                     const void* v_new, const float* k_scales,
                                     const float* v_scales, const int32_t* pos,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, int B, int s_max, int h_kv, int d_h,
                                     void* stream)
{
    if (!cache_k || !cache_v || !k_new || !v_new || !pos || !k_scales || !v_scales)
        return fail(ATTN_EINVAL, "null cache, new rows, pos or scales");
    if (!block_table) return fail(ATTN_EINVAL, "per-page scales need a paged cache (block_table)");
    if (B < 0 || h_kv <= 0 || d_h <= 0 || d_h % 4 != 0)
        return fail(ATTN_EINVAL, "bad sizes (d_h must be a positive multiple of 4)");
    int rc = check_table(block_table, max_blocks, block_size, num_blocks, s_max);
    if (rc) return rc;
    attn::AppendParams pk{};
    pk.cache = cache_k;
    pk.src = k_new;
    pk.pos = pos;
    pk.bt = block_table;
    pk.max_blocks = max_blocks;
    pk.bs_log2 = ilog2(block_size);
    pk.num_blocks = num_blocks;
    pk.s_max = s_max;
    pk.row_bytes = (long long)h_kv * d_h;
    pk.inv_scale = pk.inv_scale2 = 1.f;
    pk.split = pk.row_bytes;
    pk.page_scales = k_scales;
    pk.d_h = d_h;
    attn::AppendParams pv = pk;
    pv.cache = cache_v;
    pv.src = v_new;
    pv.page_scales = v_scales;
    hipError_t e = attn::launch_append_fp8(pk, &pv, B, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "kv_cache_append_fp8_paged_scales launch");
    return ATTN_OK;
}

size_t attn_decode_gqa_multi_workspace_bytes(int B, int q_len, int s_max, int h, int h_kv, int d_h)
{
    if (B <= 0 || q_len < 1 || q_len > 64 || h <= 0 || h_kv <= 0 || h % h_kv || d_h <= 0 ||
        s_max < 0)
        return 0;
    const size_t a = plan_gqa_path(true, B, s_max, h, h_kv, d_h, false, q_len).ws_bytes;
    const size_t f = plan_gqa_path(true, B, s_max, h, h_kv, d_h, true, q_len).ws_bytes;
    return a > f ? a : f;
}

int attn_merge_partials(void* out, float* lse, const void* o_parts, const float* lse_parts,
                        int n_parts, int B, int h, int d, int b_parts, int b_out, void* stream)
{
    if (!out || !o_parts || !lse_parts) return fail(ATTN_EINVAL, "out, o_parts and lse_parts must be non-null");
    if (n_parts <= 0 || B < 0 || h <= 0 || d <= 0)
        return fail(ATTN_EINVAL, "n_parts, h and d must be positive, B non-negative");
    if ((b_parts != 2 && b_parts != 4) || (b_out != 2 && b_out != 4))
        return fail(ATTN_ENOTSUP, "b_parts and b_out must be 2 (bf16) or 4 (fp32)");
    if (d % 4 != 0 || d > 1024) return fail(ATTN_ENOTSUP, "d must be a multiple of 4, at most 1024");
    if (((uintptr_t)out | (uintptr_t)o_parts) % 16 != 0 || (uintptr_t)lse_parts % 4 != 0 ||
        (uintptr_t)lse % 4 != 0)
        return fail(ATTN_EINVAL, "out and o_parts must be 16-byte aligned, lse arrays 4-byte aligned");
    if (B == 0) return ATTN_OK;
    if (((long long)B * h + 3) / 4 >= (1LL << 31)) return fail(ATTN_ENOTSUP, "problem too large for one launch");
    attn::MergeParams p{};
    p.out = out;
    p.lse = lse;
    p.o_parts = o_parts;
    p.lse_parts = lse_parts;
    p.rows = (long)B * h;
    p.n = n_parts;
    p.d = d;
    const hipError_t e = attn::launch_merge_partials(p, b_parts == 4, b_out == 4, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "merge launch");
}

int attn_stream_read_probe(const void* src, size_t bytes, unsigned int* sink, void* stream)
{
    if (!src || !sink) return fail(ATTN_EINVAL, "null src or sink");
    const size_t unit = (size_t)attn::kProbeGrid * 16384;
    if (bytes == 0 || bytes % unit != 0)
        return fail(ATTN_EINVAL, "bytes must be a positive multiple of %zu", unit);
    const hipError_t e = attn::launch_stream_probe(src, bytes, sink, (hipStream_t)stream);
    return e == hipSuccess ? ATTN_OK : hip_fail(e, "stream probe launch");
}

}  // extern "C"
