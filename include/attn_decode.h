/*
 * attn_decode.h -- C ABI of the MI355X (gfx950) decode-attention library
 * (libattn_decode.so).
 *
 * Single-token decode attention softmax(q K^T / sqrt(d_h)) V over a stored
 * KV cache, for the four cache layouts of the pages:
 *   MHA, MQA, GQA  -- h_kv = h, 1, h / g; query head i reads KV head
 *                     floor(i / g)   ("MHA -> MQA -> GQA -> MLA",
 *                     mlinterviewnotes.com, opening section; "The KV cache
 *                     size formula", mlinterviewnotes.com, the attention and
 *                     cell-size derivation);
 *   MLA            -- one latent row [c_KV (d_c) | k_R (d_R)] per token,
 *                     decoded with the absorbed query, a latent weighted sum
 *                     and a deferred W_UV ("Multi-Head Latent Attention
 *                     (MLA): Mathematical Foundations ...", llms.blog,
 *                     sections "Attention Logit Matrix Absorption" and
 *                     "Value Output Matrix Absorption").
 *
 * Conventions shared by every call
 * --------------------------------
 * Symbols follow the pages: B sequences, s_i cached tokens of sequence i
 * (s_max an upper bound), L layers, h query heads, h_kv KV heads, d_h head
 * dimension, d_c latent width (kv_lora_rank), d_R decoupled-RoPE key width,
 * b bytes per stored element.
 *
 * Element type: b = 2 -> bf16 storage, b = 4 -> fp32 storage.  Arithmetic
 * accumulates in fp32.  Outputs have the storage type; lse and u_latent are
 * always fp32.
 *
 * Memory: every tensor pointer is device memory owned by the caller; the
 * library never allocates, frees or keeps a pointer after a call returns.
 * Tensors are dense, row-major (last index fastest), naturally aligned and
 * 16-byte aligned at their base.  The library keeps no state apart from a
 * thread-local error message, and, for attn_decode_gqa_noalloc only, a fixed
 * scratch array per GPU and its looked-up address.
 *
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 * stream).  Calls only enqueue work and return; results are ready when the
 * stream reaches them.  Concurrent calls must not share a workspace.
 *
 * Workspaces: every workspace size reported below includes a first 64 KiB
 * of arrival counters, which only the in-kernel split merge of the GQA
 * calls uses (see attn_decode_gqa) and no call leaves non-zero.  Zero-fill a
 * workspace once when it is allocated; after that any call may use it, and
 * one buffer may serve every entry point.  The rest of a workspace needs no
 * initialisation.
 *
 * Cache layouts:
 *   contiguous (block_table == NULL): token t of sequence i is row
 *     i * s_max + t of a [B, s_max, ...] buffer;
 *   paged (block_table != NULL): token t of sequence i is row
 *     block_table[i * max_blocks + t / block_size] * block_size
 *       + t % block_size
 *     of a [num_blocks, block_size, ...] pool (16-token pages in the
 *     engines quoted by "The KV cache size formula", section "vLLM: a
 *     per-layer page, then integer division"; block contents per "MLA: why
 *     one latent can replace a multi-head KV cache", charlestar.github.io,
 *     section "What a paged KV cache block holds").  block_size must be a
 *     power of two >= 16; max_blocks * block_size >= s_max.
 *
 * Device-resident lengths and tables (s, pos, block_table) are never read
 * on the host.  Kernels clamp them so that no access leaves the buffers the
 * host-side sizes describe: a length is clamped to [0, s_max] (paged: to
 * [0, max_blocks * block_size]) and a block id to [0, num_blocks); results
 * for such out-of-range values are unspecified but memory-safe.  A
 * sequence with s_i = 0 yields an all-zero output row and lse = -inf.
 *
 * Return value: ATTN_OK, or a negative status; attn_last_error() then
 * describes it.  Argument checks happen before anything is enqueued, so a
 * rejected call has no effect.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK          0
#define ATTN_EINVAL     (-1) /* null pointer, non-positive size, h % h_kv != 0, bad block_size */
#define ATTN_ENOTSUP    (-2) /* valid but unsupported shape or dtype (see each call) */
#define ATTN_EWORKSPACE (-3) /* workspace missing or smaller than attn_decode_workspace_bytes() */
#define ATTN_EHIP       (-4) /* the HIP runtime reported an error while enqueuing */

/*
 * Bytes per token of a K/V cache over all layers: 2 * L * h_kv * d_h * b
 * ("The KV cache size formula", the cell size c; "MHA -> MQA -> GQA ->
 * MLA", opening section).  The factor 2 is K plus V.  Host-only, pure.
 * Returns 0 if any argument is negative.
 */
size_t attn_kv_cell_bytes(int L, int h_kv, int d_h, int b);

/*
 * Bytes per token of an MLA latent cache over all layers: L * (d_c + d_R) * b
 * -- no factor 2 and no head count ("The KV cache size formula", section
 * "Where MLA breaks the formula").  Host-only, pure.  Returns 0 if any
 * argument is negative.
 */
size_t attn_mla_cell_bytes(int L, int d_c, int d_R, int b);

/*
 * Workspace bytes the next two calls need for these sizes (0 is possible).
 * is_mla = 0: GQA/MQA/MHA, d_h_or_dc = d_h, d_R ignored.
 * is_mla = 1: MLA, h_kv ignored, d_h_or_dc = d_c.
 * The value depends only on the arguments; a buffer of this size (16-byte
 * aligned) may be reused across calls on one stream.
 */
size_t attn_decode_workspace_bytes(int is_mla, int B, int s_max, int h, int h_kv,
                                   int d_h_or_dc, int d_R);

/* Message for the last non-OK status returned on the calling thread. */
const char* attn_last_error(void);

/*
 * kv_cache_append -- write the new token's cache rows at slot pos[i] of each
 * sequence i (the append-by-concatenation step of the absorbed decode module
 * on the llms.blog MLA page; paged placement per "What a paged KV cache
 * block holds").
 *   cache_k, cache_v : [B, s_max, h_kv, d_h] or [num_blocks, block_size,
 *                      h_kv, d_h]; written in place.
 *   k_new, v_new     : [B, h_kv, d_h].
 *   pos              : [B] int32 device; slot to write (normally the current
 *                      s_i).  The caller keeps the lengths: s is not changed.
 * MLA: pass cache_v = v_new = NULL, h_kv = 1 and d_h = d_c + d_R (one latent
 * buffer, no V -- the num_kv_heads = 1, head_size_v = 0 encoding quoted on
 * "The KV cache size formula").  Rows whose pos or block id is out of range
 * are not written.  The copy is bit-exact.
 * Errors: EINVAL (null cache_k/k_new/pos, cache_v and v_new not both null or
 * both set, B < 0, h_kv <= 0, d_h <= 0, b not 2 or 4, bad block_size,
 * s_max <= 0 with no table, num_blocks <= 0 with a table), EHIP.
 */
int kv_cache_append(void* cache_k, void* cache_v, const void* k_new, const void* v_new,
                    const int32_t* pos, const int32_t* block_table, int max_blocks,
                    int block_size, int num_blocks, int B, int s_max, int h_kv, int d_h,
                    int b, void* stream);

/*
 * attn_decode_gqa -- decode attention for MHA / MQA / GQA.
 *   out   : [B, h, d_h], storage type.
 *   lse   : [B, h] fp32, natural-log log-sum-exp of the scaled scores; may be
 *           NULL.
 *   q     : [B, h, d_h], storage type.
 *   cache_k, cache_v : see "Cache layouts", inner shape [h_kv, d_h].
 *   s     : [B] int32 device lengths s_i.
 *   scale : > 0 used as given; <= 0 selects 1 / sqrt(d_h).
 *   workspace : at least attn_decode_workspace_bytes(0, B, s_max, h, h_kv,
 *           d_h, 0) bytes of device memory (may be NULL when that is 0).
 * out[b, i] = sum_t softmax_t(scale * q[b,i] . K[b,t,j]) V[b,t,j],
 * j = floor(i / (h / h_kv)).
 * Long contexts are split over workgroups; the partials are merged through
 * their log-sum-exp ("MLA: why one latent can replace a multi-head KV
 * cache", charlestar.github.io, section on what FlashMLA solves) by a
 * second kernel on the same stream.  With the environment variable
 * ATTN_GQA_MERGE=fused at the time of the call (bf16 and E4M3 caches), the
 * last workgroup of each (sequence, KV head) to finish merges them inside
 * the decode kernel instead, counting arrivals in the workspace's first
 * 64 KiB (which must then hold zeros, as after every call); batches with
 * more than 16,384 (sequence, KV head, 64- or 128-row block) items keep the
 * merge kernel.
 * Supported: (b = 2, d_h in {64, 128}) and (b = 4, d_h = 64); h / h_kv any
 * positive integer.  Other (b, d_h): ENOTSUP.
 * Errors: EINVAL (null out/q/cache/s, non-positive sizes, h % h_kv != 0,
 * bad block_size, max_blocks * block_size < s_max), ENOTSUP, EWORKSPACE,
 * EHIP.
 */
int attn_decode_gqa(void* out, float* lse, const void* q, const void* cache_k,
                    const void* cache_v, const int32_t* s, const int32_t* block_table,
                    int max_blocks, int block_size, int num_blocks, int B, int s_max, int h,
                    int h_kv, int d_h, int b, float scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * attn_decode_gqa_noalloc -- attn_decode_gqa without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  It calls
 * no allocating routine: the split partials go to a fixed scratch array in
 * the library's device memory, 64 MiB per GPU (one copy on every GPU the
 * library runs on, held until the process ends).  Its address on a device is
 * looked up on the first call made with that device current.
 * Arguments, results, supported shapes and errors as attn_decode_gqa, and
 * the outputs are bit-identical to attn_decode_gqa's for the same inputs;
 * plus ENOTSUP when the sizes need more scratch than 64 MiB (the message
 * gives the amount; attn_decode_workspace_bytes() reports it too) and EHIP if
 * the scratch lookup fails.
 * Every call on one GPU shares that GPU's scratch: calls that overlap in time
 * on one GPU (different streams, or host threads) race and give undefined
 * results; calls ordered on one stream are safe.  The scratch's first 64 KiB
 * (the arrival counters of the in-kernel split merge) are zero when the
 * library is loaded and every call leaves them so; nothing else in it has
 * to start at zero.
 */
int attn_decode_gqa_noalloc(void* out, float* lse, const void* q, const void* cache_k,
                            const void* cache_v, const int32_t* s, const int32_t* block_table,
                            int max_blocks, int block_size, int num_blocks, int B, int s_max,
                            int h, int h_kv, int d_h, int b, float scale, void* stream);

/*
 * FP8 caches.  An 8-bit cache halves the bytes per token that decode streams.
 * "Multi-Head Latent Attention (MLA): Mathematical Foundations ...", section
 * "High-Throughput Serving Kernels: FlashMLA and SGLang", names E4M3 codes
 * with scaling factors for a decode cache; "MLA: why one latent can replace a
 * multi-head KV cache", section "MLA and KV-cache quantization stack" (by
 * gloss), treats the element width as independent of the head layout and
 * leaves the scale granularity open.  Reading taken here: OCP E4M3 codes ("e4m3fn": bias 7, subnormals, no
 * infinities, 0x7F / 0xFF NaN, largest finite 448), one byte per element,
 * with one fp32 scale per tensor: element value = code * scale.  The rows and
 * layouts are those of the bf16 caches with b = 1.
 */

/*
 * kv_cache_append_fp8 -- kv_cache_append for FP8 caches: element x of the
 * bf16 rows k_new / v_new ([B, h_kv, d_h]) is stored as the E4M3 code of
 * x * (1 / k_scale) (resp. v_scale), the reciprocal and the product taken in
 * fp32, rounded to nearest with ties to even and saturated at +-448; NaN
 * stores 0x7F.  MLA: cache_v = v_new = NULL, h_kv = 1, d_h = d_c + d_R.
 * Errors: as kv_cache_append, plus EINVAL for a non-positive or infinite
 * scale or h_kv * d_h not a multiple of 4.
 */
int kv_cache_append_fp8(void* cache_k, void* cache_v, const void* k_new, const void* v_new,
                        float k_scale, float v_scale, const int32_t* pos,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int s_max, int h_kv, int d_h, void* stream);

/*
 * attn_decode_gqa_fp8 -- attn_decode_gqa over FP8 caches: q and out bf16
 * [B, h, d_h], cache_k / cache_v E4M3 codes with scales k_scale, v_scale:
 *   out[b, i] = sum_t softmax_t(scale * q[b,i] . k_scale K8[b,t,j])
 *                 v_scale V8[b,t,j].
 * The codes are widened to bf16 exactly in the kernel, products accumulate
 * in fp32; lse is that of the scaled scores.  Workspace as attn_decode_gqa
 * (b = 2).  Supported: d_h in {64, 128}, h / h_kv <= 64.  Others: ENOTSUP.
 * Errors: as attn_decode_gqa, plus EINVAL for a non-positive or infinite
 * scale.
 */
int attn_decode_gqa_fp8(void* out, float* lse, const void* q, const void* cache_k,
                        const void* cache_v, float k_scale, float v_scale, const int32_t* s,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int s_max, int h, int h_kv, int d_h, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_gqa_multi -- decode of q_len new tokens per sequence in one
 * call, as a speculative step verifies several drafted tokens ("MLA: why
 * one latent can replace a multi-head KV cache", section on why prefill
 * need not absorb as decode does (by gloss), counts the tokens one
 * speculative verification checks among what selects a decode kernel).
 * The q_len tokens are already appended, so s[b]
 * counts them; query position jq (0-based) sits at cache position
 * s[b] - q_len + jq and attends causally to the first s[b] - q_len + 1 + jq
 * tokens:
 *   out[b,jq,i] = sum_{t <= s_b - q_len + jq} softmax_t(scale q[b,jq,i] .
 *                 K[b,t,j]) V[b,t,j],  j = floor(i / g).
 * A position that sees no token (s[b] < q_len - jq) gives 0 and lse -inf.
 *   out : [B, q_len, h, d_h] bf16;  lse : [B, q_len, h] fp32, may be NULL.
 *   q   : [B, q_len, h, d_h] bf16.  Caches, table and lengths as
 *         attn_decode_gqa (b = 2 only).
 *   workspace : at least attn_decode_gqa_multi_workspace_bytes(B, q_len,
 *         s_max, h, h_kv, d_h) bytes.
 * Supported: d_h in {64, 128}, 1 <= q_len <= 64 (q_len = 1 equals
 * attn_decode_gqa on the same inputs up to rounding order; any h / h_kv).
 * Errors: as attn_decode_gqa; EINVAL for q_len outside 1 .. 64; ENOTSUP
 * for b != 2.
 */
int attn_decode_gqa_multi(void* out, float* lse, const void* q, const void* cache_k,
                          const void* cache_v, const int32_t* s, const int32_t* block_table,
                          int max_blocks, int block_size, int num_blocks, int B, int q_len,
                          int s_max, int h, int h_kv, int d_h, int b, float scale, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * attn_decode_gqa_multi_fp8 -- attn_decode_gqa_multi over FP8 (E4M3)
 * caches with per-tensor scales, as attn_decode_gqa_fp8.  h / h_kv <= 64.
 */
int attn_decode_gqa_multi_fp8(void* out, float* lse, const void* q, const void* cache_k,
                              const void* cache_v, float k_scale, float v_scale, const int32_t* s,
                              const int32_t* block_table, int max_blocks, int block_size,
                              int num_blocks, int B, int q_len, int s_max, int h, int h_kv,
                              int d_h, float scale, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Workspace bytes for attn_decode_gqa_multi(_fp8); 0 for invalid sizes. */
size_t attn_decode_gqa_multi_workspace_bytes(int B, int q_len, int s_max, int h, int h_kv, int d_h);

/*
 * attn_decode_gqa_fp8_paged_scales -- attn_decode_gqa_fp8 over a paged E4M3
 * cache with one scale per page and KV head instead of one per tensor: the
 * per-block scaling factors that "Multi-Head Latent Attention (MLA):
 * Mathematical Foundations ...", section "High-Throughput Serving Kernels:
 * FlashMLA and SGLang", pairs with an E4M3 cache.  Element (t, j, d) of K
 * is code * k_scales[blk * h_kv + j] with blk = block_table[b][t /
 * block_size] (V likewise with v_scales); k_scales, v_scales are fp32
 * [num_blocks, h_kv] in device memory (their values are not checked; a
 * non-positive or non-finite scale gives an unspecified result, never an
 * access outside the arrays).  block_table is required.  Other arguments,
 * workspace and errors as attn_decode_gqa_fp8; EINVAL for null scales or
 * no block table.
 */
int attn_decode_gqa_fp8_paged_scales(void* out, float* lse, const void* q, const void* cache_k,
                                     const void* cache_v, const float* k_scales,
                                     const float* v_scales, const int32_t* s,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, int B, int s_max, int h, int h_kv, int d_h,
                                     float scale, void* workspace, size_t workspace_bytes,
                                     void* stream);

/*
 * kv_cache_append_fp8_paged_scales -- kv_cache_append_fp8 into a paged pool
 * with one scale per page and KV head: element x of k_new[b, j] is stored as
 * the E4M3 code of x * (1 / k_scales[blk * h_kv + j]), blk the page of slot
 * pos[b] (reciprocal and product in fp32, nearest with ties to even,
 * saturated at +-448, NaN -> 0x7F); V likewise.  The caller sets a page's
 * scales before its first append.  d_h a multiple of 4.  Errors: as
 * kv_cache_append_fp8, plus EINVAL for null scales or no block table.
 */
int kv_cache_append_fp8_paged_scales(void* cache_k, void* cache_v, const void* k_new,
                                     const void* v_new, const float* k_scales,
                                     const float* v_scales, const int32_t* pos,
                                     const int32_t* block_table, int max_blocks, int block_size,
                                     int num_blocks, int B, int s_max, int h_kv, int d_h,
                                     void* stream);

/*
 * attn_decode_mla_absorbed -- MLA decode in the absorbed ("MQA mode") form:
 *   q~[b,i]  = W_UK[i]^T q_nope[b,i]                      (d_c values)
 *   z_t      = scale * (q~ . c_t + q_rope[b,i] . k_R,t)
 *   u~[b,i]  = sum_t softmax_t(z) c_t                     (d_c values)
 *   out[b,i] = W_UV[i] u~[b,i]                            (d_v values)
 * ("Attention Logit Matrix Absorption" and "Value Output Matrix Absorption"
 * on the llms.blog MLA page; "First matrix absorption" and "Second matrix
 * absorption" on the charlestar.github.io MLA page.)
 *   out      : [B, h, d_v] bf16.
 *   u_latent : [B, h, d_c] fp32 latent weighted sum u~; may be NULL.
 *   lse      : [B, h] fp32; may be NULL.
 *   q_nope   : [B, h, d_nope] bf16; q_rope : [B, h, d_R] bf16, already
 *              rotated.
 *   w_uk     : [h, d_nope, d_c] bf16; w_uv : [h, d_v, d_c] bf16.
 *   cache    : rows [c_KV | k_R] of width d_c + d_R, bf16 (see "Cache
 *              layouts").
 *   scale    : > 0 used as given; <= 0 selects 1 / sqrt(d_nope + d_R).
 *   workspace: at least attn_decode_workspace_bytes(1, B, s_max, h, 1, d_c,
 *              d_R) bytes.
 * Supported: b = 2, d_c = 512, d_R = 64, h a multiple of 16 up to 128,
 * d_nope a multiple of 32 up to 256, d_v a multiple of 16 up to 256.
 * Others: ENOTSUP.
 * Errors: EINVAL, ENOTSUP, EWORKSPACE, EHIP as above.
 */
int attn_decode_mla_absorbed(void* out, float* u_latent, float* lse, const void* q_nope,
                             const void* q_rope, const void* w_uk, const void* w_uv,
                             const void* cache, const int32_t* s, const int32_t* block_table,
                             int max_blocks, int block_size, int num_blocks, int B, int s_max,
                             int h, int d_c, int d_R, int d_nope, int d_v, int b, float scale,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_mla_absorbed_fp8 -- attn_decode_mla_absorbed over an FP8
 * latent cache: rows of d_c + d_R E4M3 codes [c_KV | k_R] (one byte each,
 * d_c + d_R bytes per token), element value = code * c_scale in the latent
 * part and code * r_scale in the rotary part.  "Multi-Head Latent Attention
 * (MLA): Mathematical Foundations ...", section "High-Throughput Serving
 * Kernels: FlashMLA and SGLang", describes DeepSeek-V3's latent cache in
 * E4M3 at 576 bytes per token; "MLA: why one latent can replace a
 * multi-head KV cache", section "MLA and KV-cache quantization stack" (by
 * gloss), notes that the latent and rotary parts may need separate scales.
 * Reading taken here: one fp32 scale per part for the whole cache.
 * q_nope, q_rope, W_UK, W_UV, out as attn_decode_mla_absorbed (bf16).  The
 * codes widen to bf16 exactly in the kernel; c_scale is folded into the
 * absorbed query and into u~, r_scale into the rotary query.  Workspace,
 * supported shapes and errors as attn_decode_mla_absorbed, plus EINVAL for a
 * non-positive or infinite scale.
 */
int attn_decode_mla_absorbed_fp8(void* out, float* u_latent, float* lse, const void* q_nope,
                                 const void* q_rope, const void* w_uk, const void* w_uv,
                                 const void* cache, float c_scale, float r_scale,
                                 const int32_t* s, const int32_t* block_table, int max_blocks,
                                 int block_size, int num_blocks, int B, int s_max, int h, int d_c,
                                 int d_R, int d_nope, int d_v, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * attn_decode_mla_absorbed_fp8_paged_scales -- attn_decode_mla_absorbed_fp8
 * over a paged pool whose pages each carry their own scale pair
 * ("Multi-Head Latent Attention (MLA): Mathematical Foundations", llms.blog,
 * section "High-Throughput Serving Kernels: FlashMLA and SGLang": the E4M3
 * latent is stored with per-block scaling factors; a block is a page here).
 * Element e of a row in page blk is code * c_scales[blk] (e < d_c) or
 * code * r_scales[blk].
 *   c_scales, r_scales : [num_blocks] fp32, device, caller-owned, positive
 *                        and finite for every page a sequence reaches.
 *   block_table        : required.  The rest as attn_decode_mla_absorbed_fp8.
 * In the kernel the rotary codes are widened times r/c of their page (to
 * bf16), the scores times the page's c scale, and the latent sum's weights
 * carry the c scale (the sums do not); q^ carries no scale.
 * Errors: as attn_decode_mla_absorbed_fp8, plus EINVAL for null scales or no
 * block table.
 */
int attn_decode_mla_absorbed_fp8_paged_scales(void* out, float* u_latent, float* lse,
                                              const void* q_nope, const void* q_rope,
                                              const void* w_uk, const void* w_uv,
                                              const void* cache, const float* c_scales,
                                              const float* r_scales, const int32_t* s,
                                              const int32_t* block_table, int max_blocks,
                                              int block_size, int num_blocks, int B, int s_max,
                                              int h, int d_c, int d_R, int d_nope, int d_v,
                                              float scale, void* workspace,
                                              size_t workspace_bytes, void* stream);

/*
 * kv_cache_append_mla_fp8_paged_scales -- kv_cache_append_mla_fp8 into a
 * paged pool with a scale pair per page: element x of kv_new[b] is stored as
 * the E4M3 code of x * (1 / c_scales[blk]) (latent part) or
 * x * (1 / r_scales[blk]) (rotary part), blk the page of slot pos[b]
 * (reciprocal and product in fp32, nearest with ties to even, saturated at
 * +-448).  The caller sets a page's scales before its first append.
 * Errors: as kv_cache_append_mla_fp8, plus EINVAL for null scales or no
 * block table.
 */
int kv_cache_append_mla_fp8_paged_scales(void* cache, const void* kv_new, const float* c_scales,
                                         const float* r_scales, const int32_t* pos,
                                         const int32_t* block_table, int max_blocks,
                                         int block_size, int num_blocks, int B, int s_max,
                                         int d_c, int d_R, void* stream);

/*
 * attn_decode_mla_absorbed_multi -- attn_decode_mla_absorbed for q_len new
 * tokens per sequence in one call: the tokens a speculative step verifies
 * ("MLA: why one latent can replace a multi-head KV cache",
 * charlestar.github.io, lists their count and the query length among the
 * inputs of MLA kernel selection, section on why prefill need not absorb as
 * decode does (by gloss); its validation chain's "Kernel" step covers query
 * lengths and speculative tokens).  The q_len tokens are already appended,
 * so s[b] counts them; position jq (0-based) sits at cache position
 * s[b] - q_len + jq and attends to the first s[b] - q_len + 1 + jq tokens
 * (causal among the new tokens).  A position that sees no token gives 0,
 * u~ = 0 and lse -inf.
 *   out      : [B, q_len, h, d_v] bf16;  u_latent : [B, q_len, h, d_c] fp32
 *              or NULL;  lse : [B, q_len, h] fp32 or NULL.
 *   q_nope   : [B, q_len, h, d_nope] bf16;  q_rope : [B, q_len, h, d_R].
 *   Weights, cache, table, lengths, scale: as attn_decode_mla_absorbed.
 *   workspace: at least attn_decode_mla_multi_workspace_bytes(B, q_len, h,
 *              d_c, d_R) bytes.
 * Each (sequence, position) pair is one query row of the kernels, so q_len
 * = 1 is attn_decode_mla_absorbed exactly; each row streams its visible
 * latent rows once (later rows of a sequence mostly from cache).
 * Supported: 1 <= q_len <= 1024 (else EINVAL), B * q_len < 2^24, the rest
 * as attn_decode_mla_absorbed.
 * Errors: as attn_decode_mla_absorbed.
 */
int attn_decode_mla_absorbed_multi(void* out, float* u_latent, float* lse, const void* q_nope,
                                   const void* q_rope, const void* w_uk, const void* w_uv,
                                   const void* cache, const int32_t* s,
                                   const int32_t* block_table, int max_blocks, int block_size,
                                   int num_blocks, int B, int q_len, int s_max, int h, int d_c,
                                   int d_R, int d_nope, int d_v, int b, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_mla_absorbed_multi_fp8 -- attn_decode_mla_absorbed_multi over
 * an FP8 latent cache with the scales of attn_decode_mla_absorbed_fp8.
 */
int attn_decode_mla_absorbed_multi_fp8(void* out, float* u_latent, float* lse,
                                       const void* q_nope, const void* q_rope, const void* w_uk,
                                       const void* w_uv, const void* cache, float c_scale,
                                       float r_scale, const int32_t* s,
                                       const int32_t* block_table, int max_blocks,
                                       int block_size, int num_blocks, int B, int q_len,
                                       int s_max, int h, int d_c, int d_R, int d_nope, int d_v,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* Workspace bytes for attn_decode_mla_absorbed_multi(_fp8); 0 for invalid sizes. */
size_t attn_decode_mla_multi_workspace_bytes(int B, int q_len, int h, int d_c, int d_R);

/*
 * attn_decode_mla_out -- MLA decode through the attention block's output
 * projection ("Multi-Head Latent Attention (MLA): Mathematical Foundations",
 * llms.blog, section "Value Output Matrix Absorption"):
 *   o[b,jq] = sum_i W_O^i u[b,jq,i],  u[b,jq,i] = W_UV[i] u~[b,jq,i],
 * W_O = [W_O^1 .. W_O^h], head i owning columns i d_v .. i d_v + d_v - 1.
 * Deferred form: the heads' outputs u (bf16, as attn_decode_mla_absorbed_multi
 * returns them) are formed in the workspace, then one projection over all
 * h d_v columns.
 *   out  : [B, q_len, d_model] bf16 (q_len = 1: [B, d_model]).
 *   lse  : [B, q_len, h] fp32 or NULL.
 *   w_o  : [d_model, h d_v] bf16 (the layout of a linear layer's weight).
 *   q_nope, q_rope, w_uk, w_uv, cache, table, lengths, q_len, scale: as
 *   attn_decode_mla_absorbed_multi (the new tokens see their causal prefix).
 *   workspace : at least attn_decode_mla_out_workspace_bytes(0, B, q_len, h,
 *         d_c, d_R, d_v, d_model) bytes.
 * Supported: as attn_decode_mla_absorbed_multi, plus d_model a multiple of
 * 32 and h d_v a multiple of 128.  Others: ENOTSUP.
 * Errors: EINVAL, ENOTSUP, EWORKSPACE, EHIP as above.
 */
int attn_decode_mla_out(void* out, float* lse, const void* q_nope, const void* q_rope,
                        const void* w_uk, const void* w_uv, const void* w_o, const void* cache,
                        const int32_t* s, const int32_t* block_table, int max_blocks,
                        int block_size, int num_blocks, int B, int q_len, int s_max, int h,
                        int d_c, int d_R, int d_nope, int d_v, int d_model, int b, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * attn_decode_mla_out_premerged -- the same output in the merged form of
 * the same section: o[b,jq] = sum_i W_abs^i u~[b,jq,i] with the static
 * W_abs^i = W_O^i W_UV[i] (d_model x d_c), built once by
 * attn_mla_premerge_weights.  u~ is rounded to bf16 for the projection; the
 * per-head d_v-wide outputs are never formed.
 *   w_absorbed : [d_model, h d_c] bf16, head i owning columns
 *                i d_c .. i d_c + d_c - 1.
 *   workspace  : at least attn_decode_mla_out_workspace_bytes(1, B, q_len,
 *                h, d_c, d_R, 0, d_model) bytes.
 * The rest as attn_decode_mla_out (no w_uv, no d_v).  Which form moves and
 * computes less for a shape: attn_mla_out_form.
 */
int attn_decode_mla_out_premerged(void* out, float* lse, const void* q_nope, const void* q_rope,
                                  const void* w_uk, const void* w_absorbed, const void* cache,
                                  const int32_t* s, const int32_t* block_table, int max_blocks,
                                  int block_size, int num_blocks, int B, int q_len, int s_max,
                                  int h, int d_c, int d_R, int d_nope, int d_model, int b,
                                  float scale, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Workspace bytes for attn_decode_mla_out (premerged = 0) or
 * attn_decode_mla_out_premerged (premerged = 1); 0 for invalid sizes. */
size_t attn_decode_mla_out_workspace_bytes(int premerged, int B, int q_len, int h, int d_c,
                                           int d_R, int d_v, int d_model);

/*
 * attn_mla_premerge_weights -- w_absorbed[n, i d_c + c] =
 *   sum_e w_o[n, i d_v + e] w_uv[i, e, c]  (fp32 sums rounded to bf16), the
 * static merged weight of the section above, computed on the device in one
 * launch on `stream`.  w_absorbed [d_model, h d_c], w_o [d_model, h d_v],
 * w_uv [h, d_v, d_c], all bf16, caller-owned.  Supported: d_c a multiple of
 * 256, d_model a multiple of 32, d_v <= 256, d_model h d_c < 2^31.
 * Errors: EINVAL (null, bad sizes), ENOTSUP, EHIP.
 */
int attn_mla_premerge_weights(void* w_absorbed, const void* w_o, const void* w_uv, int h,
                              int d_c, int d_v, int d_model, void* stream);

/*
 * attn_decode_mla_mha -- the same result as attn_decode_mla_absorbed_multi
 * (out and lse; no u~) computed in "MHA mode": every cached token's per-head
 * key and value are expanded explicitly, K_n[b,t,i] = W_UK[i] c_t and
 * V[b,t,i] = W_UV[i] c_t (bf16, in the workspace), and attention runs as
 * plain multi-head attention with key [K_n | k_R] ("MLA: why one latent can
 * replace a multi-head KV cache", charlestar.github.io, section on MHA mode
 * and MQA mode being execution forms (by gloss): the form for long query
 * blocks; llms.blog MLA page, "Low-Rank Joint Key-Value Compression" and
 * "The Decoupled RoPE Solution" for the expansion).  The expansion costs
 * 2 d_c h (d_nope + d_v) flops per cached token whatever q_len is, so this
 * form wins only for long query blocks; attn_mla_mode says which.
 *   Arguments as attn_decode_mla_absorbed_multi without u_latent; any
 *   q_len >= 1; s_max bounds every s[b] (paged caches too).
 *   workspace: at least attn_decode_mla_mha_workspace_bytes(B, s_max, h)
 *   bytes (the expanded K_n and V, [B, s_max, h, 128] each).
 * Supported: b = 2, d_c = 512, d_R = 64, d_nope = d_v = 128.  Others:
 * ENOTSUP.  Errors: EINVAL, ENOTSUP, EWORKSPACE, EHIP as above.
 */
int attn_decode_mla_mha(void* out, float* lse, const void* q_nope, const void* q_rope,
                        const void* w_uk, const void* w_uv, const void* cache, const int32_t* s,
                        const int32_t* block_table, int max_blocks, int block_size,
                        int num_blocks, int B, int q_len, int s_max, int h, int d_c, int d_R,
                        int d_nope, int d_v, int b, float scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/* Workspace bytes for attn_decode_mla_mha; 0 for invalid sizes. */
size_t attn_decode_mla_mha_workspace_bytes(int B, int s_max, int h);

/*
 * attn_mla_mode -- which MLA execution form is faster for q_len new tokens
 * over a context of s tokens (the page's kernel selection by query and KV
 * length): 0 the absorbed (MQA) form, attn_decode_mla_absorbed_multi; 1 MHA
 * mode, attn_decode_mla_mha; -1 bad sizes.  A cost model of this library's
 * kernels fitted to MI355X timings: MHA mode from about q_len 240 at
 * s = 2048 and about 380 at s = 8192.
 */
int attn_mla_mode(int q_len, int s);

/*
 * attn_mla_out_form -- which output form is cheaper for a shape, by the
 * bytes and matrix-core work in which the two differ (deferred: W_UV, W_O
 * and the heads' outputs; merged: W_abs and bf16 u~), each priced at the
 * MI355X HBM and dense bf16 peaks: 0 deferred, 1 merged, -1 bad sizes.
 * With d_c > d_v (DeepSeek: 512 vs 128) the merged weight is d_c / d_v
 * times larger than W_O and the deferred form always wins.
 */
int attn_mla_out_form(int B, int q_len, int h, int d_c, int d_v, int d_model);

/*
 * kv_cache_append_mla_fp8 -- append one latent row per sequence to an FP8
 * latent cache: element x of kv_new[b] ([B, d_c + d_R] bf16, [c | k_R]) is
 * stored as the E4M3 code of x * (1 / c_scale) in the latent part and of
 * x * (1 / r_scale) in the rotary part (reciprocal and product in fp32,
 * nearest with ties to even, saturated at +-448, NaN -> 0x7F), at slot
 * pos[b] as kv_cache_append.  d_c and d_R multiples of 4.
 * Errors: as kv_cache_append, plus EINVAL for a non-positive or infinite
 * scale.
 */
int kv_cache_append_mla_fp8(void* cache, const void* kv_new, float c_scale, float r_scale,
                            const int32_t* pos, const int32_t* block_table, int max_blocks,
                            int block_size, int num_blocks, int B, int s_max, int d_c, int d_R,
                            void* stream);

/*
 * attn_merge_partials -- combine decode results computed over disjoint token
 * slices of the same sequences into the result over all their tokens: the
 * exchange step of context-parallel decode, where each GPU holds a slice of
 * every sequence's cache, runs attn_decode_gqa (or _fp8, or
 * attn_decode_mla_absorbed) over it, and the per-slice out and lse are
 * gathered.  "MHA -> MQA -> GQA -> MLA", section "Where the head count
 * becomes bytes", names decode context parallelism (sharding the sequence
 * axis, the route left once heads cannot be split);
 * the combination is the stable merge of per-block maximum, normaliser and
 * output of "MLA: why one latent can replace a multi-head KV cache", section
 * "What FlashMLA solves is not the model formula itself":
 *   lse[r] = ln sum_k exp(lse_parts[k, r]),
 *   out[r] = sum_k exp(lse_parts[k, r] - lse[r]) o_parts[k, r].
 * For MLA the per-slice out (after W_UV) merges the same way as u~, since
 * W_UV is linear.
 *   out       : [B, h, d], dtype b_out (2 = bf16, 4 = fp32).
 *   lse       : [B, h] fp32 (natural log); may be NULL.
 *   o_parts   : [n_parts, B, h, d], dtype b_parts; slice k is one decode's
 *               out.
 *   lse_parts : [n_parts, B, h] fp32, slice k's lse; -inf marks an empty
 *               slice, whose o_parts row is not read into the sum.
 * A row whose slices are all empty gives out = 0 and lse = -inf.  All
 * pointers are device memory owned by the caller; out and o_parts 16-byte
 * aligned.  Accumulation is fp32.  Asynchronous on `stream`.
 * Supported: d a multiple of 4 up to 1024.  Others: ENOTSUP.
 * Errors: EINVAL (null pointer, n_parts <= 0, B < 0, h or d <= 0,
 * misalignment), ENOTSUP (b_parts or b_out not 2 or 4, d), EHIP.
 */
int attn_merge_partials(void* out, float* lse, const void* o_parts, const float* lse_parts,
                        int n_parts, int B, int h, int d, int b_parts, int b_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
