// Kernel parameter blocks and launchers (host <-> device, library-internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct GqaParams {
    void* out;
    float* lse;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* s;
    const int32_t* bt;   // nullptr: contiguous
    float* part_o;       // [B, q_len, h, n_split, d_h]
    float* part_ml;      // [B, q_len, h, n_split, 2]  (m in log2 units, l)
    int max_blocks, bs_log2, num_blocks;
    int B, s_max, h, h_kv;
    int n_hg, n_split, chunk;
    int q_len;           // query positions per sequence (matrix-core kernel only; 1 otherwise)
    int n_rb;            // row blocks (64 or 128 rows) per (b, KV head) work item (matrix-core kernel)
    int compact;         // matrix-core kernel: workgroups map to the non-empty (b, split) pairs only
    int xpair;           // matrix-core kernel, contiguous cache: -1, or bit 8 of the K cache's address
                         // (the KV heads are then permuted against the XCD parity)
    float scale_log2;    // scale * log2(e) (times the K scale of an FP8 cache)
    float v_scale;       // V scale of an FP8 cache (1 otherwise)
    const float* k_scales;   // paged FP8 cache with one scale per page and KV head: [num_blocks, h_kv]
    const float* v_scales;   // (nullptr: the per-tensor scales above)
    int32_t* arrive;         // matrix-core kernel with splits: one arrival counter per (b, KV head,
                             // row block), zero before the call and left zero by it; the last
                             // workgroup of an item to arrive merges its splits (nullptr: the
                             // separate merge kernel does)
};

// Every workspace starts with this many bytes of arrival counters (used by
// the GQA split merge only, zero-filled when the workspace is allocated and
// left zero by every call), so that one buffer may serve all entry points.
constexpr size_t kArriveBytes = (size_t)64 << 10;
constexpr int kArriveCount = (int)(kArriveBytes / sizeof(int32_t));

// vector kernel (any g; fp32 or bf16), then the split merge when n_split > 1
hipError_t launch_gqa_decode(const GqaParams& p, int d_h, bool f32, int HG, bool paged,
                             unsigned grid, hipStream_t st);
// matrix-core kernel (bf16 or FP8 E4M3 caches, g <= 16 NW, NW = 2 or 4), then the split
// merge when n_split > 1
// ni = 1 (E4M3 caches, at most 16 rows): two wavefronts, one computing and one issuing the DMA
hipError_t launch_gqa_mfma(const GqaParams& p, int d_h, int NW, int rpw, int ni, bool paged, bool f8,
                           unsigned grid, hipStream_t st);
hipError_t launch_gqa_combine(const GqaParams& p, int d_h, bool f32, hipStream_t st);

struct AppendParams {
    void* cache;
    const void* src;
    const int32_t* pos;
    const int32_t* bt;
    int max_blocks, bs_log2, num_blocks, s_max;
    long long row_bytes;   // bytes of one cache row (FP8: elements of one row)
    float inv_scale;       // FP8 append: fp32 reciprocal of the tensor's scale
    float inv_scale2;      // FP8 append: reciprocal scale of elements split .. row end
    long long split;       // FP8 append: first element under inv_scale2 (a multiple of 4)
    const float* page_scales;   // FP8 append into a paged pool with one scale per page and
    int d_h;                    // KV head ([num_blocks, row_bytes / d_h]); nullptr: the above
    const float* page_scales2;  // MLA rows with a scale pair per page: page_scales [num_blocks]
                                // for elements before split, this one after; nullptr: unused
};

hipError_t launch_append(const AppendParams& k, const AppendParams* v, int B, hipStream_t st);
// bf16 rows -> OCP E4M3 codes of x * inv_scale (nearest, ties to even, saturating at +-448)
hipError_t launch_append_fp8(const AppendParams& k, const AppendParams* v, int B, hipStream_t st);

// B counts query rows: row b is new-token position b % q_len of sequence
// b / q_len, whose length s and block-table row it reads (q_len = 1: one
// row per sequence)
struct MlaParams {
    void* out;            // [B, h, d_v] bf16, or nullptr: no value up-projection
    float* u_latent;      // [B, h, d_c] fp32 or nullptr
    float* lse;           // [B, h] or nullptr
    const void* q_nope;   // [B, h, d_nope]
    const void* q_rope;   // [B, h, d_R]
    const void* w_uk;     // [h, d_nope, d_c]
    const void* w_uv;     // [h, d_v, d_c]
    const void* cache;    // rows of d_c + d_R
    const int32_t* s;
    const int32_t* bt;
    uint16_t* qhat;       // bf16 absorbed query, B * ceil(h / 32) blocks of 32 heads x 576 in decode-operand order
    _Float16* part_u;     // [n_wg + B - 1, h, d_c]: U / l of (workgroup w, sequence b) in slot w + b
    float* part_ml;       // [n_wg + B - 1, h, 2]
    int32_t* flags;       // [n_wg]: decode workgroup stopped early; its partials are recomputed by the merge
    int32_t* sched;       // tile_start [B + 1], wstart [n_wg], tpw [1]
    int max_blocks, bs_log2, num_blocks;
    int B, s_max, h, d_c, d_R, d_nope, d_v;
    int q_len;            // new tokens per sequence (query rows per sequence)
    int n_wg, min_tiles;  // decode workgroups; fewest 32-token tiles per workgroup
    float scale_log2;
    uint16_t* u_bf16;     // [B, h, d_c] bf16 u~ for the merged output projection, or nullptr
    int f8;               // cache rows are E4M3 codes (else bf16)
    float c_scale;        // FP8: scale of the latent part (1 for bf16); folded into q^ and u~
    float r_scale;        // FP8: scale of the rotary part (1 for bf16); folded into q^
    const float* c_scales;   // paged FP8 pool with a scale pair per page: [num_blocks] latent,
    const float* r_scales;   // [num_blocks] rotary (c_scale = r_scale = 1 then); nullptr: none
};

hipError_t launch_mla(const MlaParams& p, bool paged, hipStream_t st);

// Y[M, N] = X[M, K] W[N, K]^T (bf16 operands, fp32 sums): the MLA output
// projection.  N % 32 == 0, K % 128 == 0, M K 2 + 2 K < 2^31.
struct ProjParams {
    const uint16_t* x;   // [M, K] bf16
    const uint16_t* w;   // [N, K] bf16
    void* y;             // [M, N] bf16, or fp32 when y_f32
    float* part;         // [ks, M, N] fp32 partial sums when ks > 1
    int M, N, K, ks;     // ks: K splits over workgroups
    int y_f32;
};
hipError_t launch_proj(const ProjParams& p, hipStream_t st);

// W_abs[n, i d_c + c] = sum_e W_O[n, i d_v + e] W_UV[i, e, c] (bf16 in and out)
struct PremergeParams {
    void* w_abs;          // [d_model, h d_c]
    const void* w_o;      // [d_model, h d_v]
    const void* w_uv;     // [h, d_v, d_c]
    int h, d_c, d_v, d_model;   // d_c % 256 == 0, d_model % 32 == 0, d_v <= 256
};
hipError_t launch_premerge(const PremergeParams& p, hipStream_t st);

// MLA in MHA mode: explicit per-head K/V (d_c = 512, d_R = 64, d_nope = d_v = 128)
struct MhaParams {
    void* out;             // [B, q_len, h, 128] bf16
    float* lse;            // [B, q_len, h] or nullptr
    const void* q_nope;    // [B, q_len, h, 128]
    const void* q_rope;    // [B, q_len, h, 64]
    const void* w_uk;      // [h, 128, 512]
    const void* w_uv;      // [h, 128, 512]
    const void* cache;     // rows [c (512) | k_R (64)] bf16
    const int32_t* s;
    const int32_t* bt;     // nullptr: contiguous [B, s_max, 576]
    uint16_t* k_exp;       // [B, s_max, h, 128]: W_UK[i] c
    uint16_t* v_exp;       // [B, s_max, h, 128]: W_UV[i] c
    int max_blocks, bs_log2, num_blocks;
    int B, q_len, s_max, h;
    float scale_log2;
};
hipError_t launch_mla_mha(const MhaParams& p, hipStream_t st);

// merge of decode outputs over disjoint token slices
struct MergeParams {
    void* out;               // [rows, d] bf16 or fp32
    float* lse;              // [rows] or null
    const void* o_parts;     // [n, rows, d] bf16 or fp32
    const float* lse_parts;  // [n, rows]
    long rows;               // B * h
    int n, d;                // d % 4 == 0, d <= 1024
};
hipError_t launch_merge_partials(const MergeParams& p, bool in_f32, bool out_f32, hipStream_t st);

// Device scratch of the entry point that allocates nothing: one fixed array
// per GPU (noalloc.hip).  The address of the current device's copy, looked
// up on the first call on that device and kept.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
hipError_t noalloc_scratch(void** out);

// read-bandwidth probe: kProbeGrid workgroups, bytes / kProbeGrid each (a
// multiple of 16 KB)
constexpr unsigned kProbeGrid = 2048;
hipError_t launch_stream_probe(const void* src, size_t bytes, unsigned* sink, hipStream_t st);

}  // namespace attn
