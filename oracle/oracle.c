/*
 * Plain CPU oracle for single-token decode attention over a stored KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the HIP library is checked against.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it; the library
 * never does.  It shares no code, header or table with the HIP path.
 *
 * Arithmetic: every stored element (bf16 bits or fp32) is widened exactly to
 * double; all sums, the softmax and the final division are in double.  The
 * softmax is two-pass (maximum first, then exponentials), not online.
 * OpenMP splits only the independent output rows (b, i); the arithmetic of a
 * row is the plain sequential loop.
 *
 * Sources (cited by page title and section):
 *  - "The KV cache size formula" (mlinterviewnotes.com): attention at decode
 *    computes softmax(q K^T / sqrt(d_h)) V over all previous positions; the
 *    per-token cell 2 * L * h_kv * d_h * b; the MLA cell L * (d_c + d_R) * b
 *    ("Where MLA breaks the formula"); token-major K/V buffers
 *    [rows, h_kv, d_h] and one latent buffer [rows, 1, d_c + d_R] (listing
 *    under "SGLang: one cell size, one division"); 16-token pages
 *    ("vLLM: a per-layer page, then integer division").
 *  - "MHA -> MQA -> GQA -> MLA" (mlinterviewnotes.com), opening section:
 *    query heads are broadcast against the h_kv shared KV heads; MHA, MQA,
 *    GQA are h_kv = h, 1, h/g.
 *  - "Multi-Head Latent Attention (MLA): Mathematical Foundations ..."
 *    (llms.blog): sections "Attention Logit Matrix Absorption" (absorbed
 *    query q~ = W_UK,i^T q^C and score q~^T c + q^R^T k^R) and "Value Output
 *    Matrix Absorption" (softmax scale 1/sqrt(d_h^C + d_r), latent sum
 *    u~ = sum_j A_j c_j, deferred u = W_UV,i u~); "Low-Rank Joint Key-Value
 *    Compression" for the explicit k^C = W_UK c, v^C = W_UV c.
 *  - "MLA: why one latent can replace a multi-head KV cache"
 *    (charlestar.github.io): "First matrix absorption", "Second matrix
 *    absorption", "What a paged KV cache block holds" (row = [c_KV | k_R]),
 *    "Correctness validation ..." (explicit expansion as the slow reference),
 *    "What FlashMLA solves is not the model formula itself" (each block of
 *    keys yields its own maximum, normaliser and output, and the blocks are
 *    combined stably: the merge of ref_merge_partials).
 *
 * Readings where the pages are silent (listed again in the design notes):
 *  - query head i uses KV head floor(i / g) (consecutive heads share);
 *  - MLA weights are per-head slices W_UK[i] : [d_nope, d_c] and
 *    W_UV[i] : [d_v, d_c]; the MLA scale is 1/sqrt(d_nope + d_R);
 *  - s_b = 0 gives an all-zero output row and lse = -inf;
 *  - paged token t of sequence b lives in physical row
 *    block_table[b][t / block_size] * block_size + t % block_size.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_EINVAL (-1)

/* widen one stored element to double; b = 2 -> bf16 bits, b = 4 -> fp32 */
static double ld(const void* p, size_t idx, int b)
{
    if (b == 4) return (double)((const float*)p)[idx];
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[idx]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* physical row of token t of sequence bb */
static size_t row_of(const int32_t* bt, int max_blocks, int block_size, int s_max,
                     int bb, int t)
{
    if (!bt) return (size_t)bb * (size_t)s_max + (size_t)t;
    int blk = bt[(size_t)bb * (size_t)max_blocks + (size_t)(t / block_size)];
    return (size_t)blk * (size_t)block_size + (size_t)(t % block_size);
}

unsigned long long ref_kv_cell_bytes(int L, int h_kv, int d_h, int b)
{
    return 2ULL * (unsigned long long)L * (unsigned long long)h_kv *
           (unsigned long long)d_h * (unsigned long long)b;
}

unsigned long long ref_mla_cell_bytes(int L, int d_c, int d_R, int b)
{
    return (unsigned long long)L * ((unsigned long long)d_c + (unsigned long long)d_R) *
           (unsigned long long)b;
}

/* every logical block a sequence of n tokens touches must be mapped */
static int table_ok(const int32_t* bt, int max_blocks, int block_size, int bb, int n)
{
    if (!bt) return 1;
    for (int blk = 0; blk * block_size < n; blk++)
        if (bt[(size_t)bb * (size_t)max_blocks + (size_t)blk] < 0) return 0;
    return 1;
}

/* Two-pass softmax-weighted sum over n scores z[]: writes p[t] = exp(z_t - m)
 * and returns l = sum p; *m_out = max z. */
static double softmax_weights(const double* z, int n, double* p, double* m_out)
{
    double m = -INFINITY;
    for (int t = 0; t < n; t++)
        if (z[t] > m) m = z[t];
    double l = 0.0;
    for (int t = 0; t < n; t++) {
        p[t] = exp(z[t] - m);
        l += p[t];
    }
    *m_out = m;
    return l;
}

/*
 * GQA / MQA / MHA decode.
 *   out [B, h, d_h] double, lse [B, h] double (nullable)
 *   q   [B, h, d_h]            stored dtype b
 *   k,v [B, s_max, h_kv, d_h]  (block_table == NULL)  or
 *       [N_blk, block_size, h_kv, d_h]                 (paged)
 *   s   [B] host lengths
 * z_t = scale * sum_d q[b,i,d] K(b,t,j,d), j = floor(i / g);
 * o = sum_t softmax(z)_t V(b,t,j,:);  lse = m + ln(sum_t exp(z_t - m)).
 */
int ref_gqa_decode(double* out, double* lse, const void* q, const void* k, const void* v,
                   const int32_t* s, const int32_t* block_table, int max_blocks,
                   int block_size, int B, int s_max, int h, int h_kv, int d_h, int b,
                   double scale)
{
    if (!out || !q || !k || !v || !s) return OR_EINVAL;
    if (B < 0 || h <= 0 || h_kv <= 0 || d_h <= 0 || (h % h_kv) != 0) return OR_EINVAL;
    if (b != 2 && b != 4) return OR_EINVAL;
    if (block_table && (block_size <= 0 || max_blocks <= 0)) return OR_EINVAL;
    const int g = h / h_kv;
    const long rows = (long)B * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / h), i = (int)(r % h), j = i / g;
        const int n = s[bb];
        double* o = out + (size_t)r * d_h;
        if (n < 0 || (!block_table && n > s_max) ||
            (block_table && n > max_blocks * block_size) ||
            !table_ok(block_table, max_blocks, block_size, bb, n)) {
            bad = 1;
            continue;
        }
        if (n == 0) {
            for (int d = 0; d < d_h; d++) o[d] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n * 2);
        double* p = z + n;
        const size_t qoff = (size_t)r * d_h;
        for (int t = 0; t < n; t++) {
            const size_t koff =
                (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) * d_h;
            double acc = 0.0;
            for (int d = 0; d < d_h; d++) acc += ld(q, qoff + d, b) * ld(k, koff + d, b);
            z[t] = scale * acc;
        }
        double m;
        const double l = softmax_weights(z, n, p, &m);
        for (int d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (int t = 0; t < n; t++) {
                const size_t voff =
                    (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) *
                    d_h;
                acc += p[t] * ld(v, voff + d, b);
            }
            o[d] = acc / l;
        }
        if (lse) lse[r] = m + log(l);
        free(z);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/*
 * MLA decode in the absorbed ("MQA mode") form.
 *   out [B, h, d_v] double; u_latent [B, h, d_c] double (nullable);
 *   lse [B, h] double (nullable)
 *   q_nope [B, h, d_nope], q_rope [B, h, d_R] (already rotated)
 *   w_uk [h, d_nope, d_c], w_uv [h, d_v, d_c]
 *   cache rows [c (d_c) | k_R (d_R)]: [B, s_max, d_c + d_R] or paged
 *   [N_blk, block_size, d_c + d_R]
 * Steps in the pages' order: q~ = W_UK,i^T q^C; score_t = q~ . c_t +
 * q^R . k^R_t; A = softmax(scale * score); u~ = sum_t A_t c_t;
 * o = W_UV,i u~.
 */
double ref_fp8_e4m3_decode(int code);
static double ld_fp8(const uint8_t* p, size_t idx, double scale);

/* element e of cached latent row roff: stored bits of dtype cb (2 or 4), or
 * (cb = 1) an E4M3 code times c_scale (latent part, e < d_c) or r_scale
 * (rotary part) */
static double ld_latent(const void* cache, size_t roff, int e, int cb, int d_c, double c_scale,
                        double r_scale)
{
    if (cb == 1) return ld_fp8((const uint8_t*)cache, roff + e, e < d_c ? c_scale : r_scale);
    return ld(cache, roff + e, cb);
}

/* the scale of token t of sequence bb: that of its page (the physical block
 * the table maps it to) when per-page scales are given, else the tensor's */
static double page_scale(const float* scales, double tensor_scale, const int32_t* block_table,
                         int max_blocks, int block_size, int bb, int t)
{
    if (!scales) return tensor_scale;
    const int blk = block_table[(size_t)bb * max_blocks + t / block_size];
    return (double)scales[blk];
}

/*
 * Rows r = (bb, jq, i) of q_len query positions per sequence (q_len = 1:
 * plain single-token decode).  All q_len new tokens are already in the
 * cache, so s_b counts them; position jq sits at cache position
 * s_b - q_len + jq and attends to the tokens up to and including itself
 * (causal among the new tokens, as when a speculative step verifies them).
 */
static int mla_absorbed_impl(double* out, double* u_latent, double* lse, const void* q_nope,
                             const void* q_rope, const void* w_uk, const void* w_uv,
                             const void* cache, int cb, double c_scale, double r_scale,
                             const float* c_scales, const float* r_scales,
                             const int32_t* s, const int32_t* block_table, int max_blocks,
                             int block_size, int B, int q_len, int s_max, int h, int d_c,
                             int d_R, int d_nope, int d_v, int b, double scale)
{
    if (!out || !q_nope || !q_rope || !w_uk || !w_uv || !cache || !s) return OR_EINVAL;
    if (B < 0 || q_len < 1 || h <= 0 || d_c <= 0 || d_R < 0 || d_nope <= 0 || d_v <= 0)
        return OR_EINVAL;
    if (b != 2 && b != 4) return OR_EINVAL;
    if (block_table && (block_size <= 0 || max_blocks <= 0)) return OR_EINVAL;
    if ((c_scales || r_scales) && (!c_scales || !r_scales || !block_table || cb != 1))
        return OR_EINVAL;
    const int W = d_c + d_R;
    const long rows = (long)B * q_len * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / ((long)q_len * h));
        const int jq = (int)((r / h) % q_len), i = (int)(r % h);
        const int sb = s[bb];
        double* o = out + (size_t)r * d_v;
        if (sb < 0 || (!block_table && sb > s_max) ||
            (block_table && sb > max_blocks * block_size) ||
            !table_ok(block_table, max_blocks, block_size, bb, sb)) {
            bad = 1;
            continue;
        }
        /* tokens this position sees (none for an early position of a sequence
           shorter than q_len) */
        const int n = sb - q_len + 1 + jq > 0 ? sb - q_len + 1 + jq : 0;
        double* qt = (double*)malloc(sizeof(double) * ((size_t)d_c * 2 + (size_t)n * 2));
        double* ut = qt + d_c;
        double* z = ut + d_c;
        double* p = z + n;
        /* absorbed query: q~[c] = sum_n W_UK[i][n][c] q_nope[n] */
        for (int c = 0; c < d_c; c++) {
            double acc = 0.0;
            for (int e = 0; e < d_nope; e++)
                acc += ld(w_uk, ((size_t)i * d_nope + e) * d_c + c, b) *
                       ld(q_nope, (size_t)r * d_nope + e, b);
            qt[c] = acc;
        }
        if (n == 0) {
            for (int c = 0; c < d_c; c++) ut[c] = 0.0;
            if (lse) lse[r] = -INFINITY;
        } else {
            /* scores over the latent and the decoupled RoPE key */
            for (int t = 0; t < n; t++) {
                const size_t roff =
                    row_of(block_table, max_blocks, block_size, s_max, bb, t) * W;
                const double cs = page_scale(c_scales, c_scale, block_table, max_blocks,
                                             block_size, bb, t);
                const double rs = page_scale(r_scales, r_scale, block_table, max_blocks,
                                             block_size, bb, t);
                double acc = 0.0;
                for (int c = 0; c < d_c; c++)
                    acc += qt[c] * ld_latent(cache, roff, c, cb, d_c, cs, rs);
                double accr = 0.0;
                for (int e = 0; e < d_R; e++)
                    accr += ld(q_rope, (size_t)r * d_R + e, b) *
                            ld_latent(cache, roff, d_c + e, cb, d_c, cs, rs);
                z[t] = scale * (acc + accr);
            }
            double m;
            const double l = softmax_weights(z, n, p, &m);
            /* latent weighted sum u~ = sum_t A_t c_t */
            for (int c = 0; c < d_c; c++) {
                double acc = 0.0;
                for (int t = 0; t < n; t++) {
                    const size_t roff =
                        row_of(block_table, max_blocks, block_size, s_max, bb, t) * W;
                    const double cs = page_scale(c_scales, c_scale, block_table, max_blocks,
                                                 block_size, bb, t);
                    acc += p[t] * ld_latent(cache, roff, c, cb, d_c, cs, r_scale);
                }
                ut[c] = acc / l;
            }
            if (lse) lse[r] = m + log(l);
        }
        if (u_latent)
            for (int c = 0; c < d_c; c++) u_latent[(size_t)r * d_c + c] = ut[c];
        /* deferred value up-projection o = W_UV[i] u~ */
        for (int e = 0; e < d_v; e++) {
            double acc = 0.0;
            for (int c = 0; c < d_c; c++)
                acc += ld(w_uv, ((size_t)i * d_v + e) * d_c + c, b) * ut[c];
            o[e] = acc;
        }
        free(qt);
    }
    return bad ? OR_EINVAL : OR_OK;
}

int ref_mla_absorbed(double* out, double* u_latent, double* lse, const void* q_nope,
                     const void* q_rope, const void* w_uk, const void* w_uv,
                     const void* cache, const int32_t* s, const int32_t* block_table,
                     int max_blocks, int block_size, int B, int s_max, int h, int d_c,
                     int d_R, int d_nope, int d_v, int b, double scale)
{
    return mla_absorbed_impl(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, b, 1.0, 1.0,
                             NULL, NULL, s, block_table, max_blocks, block_size, B, 1, s_max, h,
                             d_c, d_R, d_nope, d_v, b, scale);
}

/*
 * MLA absorbed decode of q_len new tokens per sequence: the tokens one
 * speculative step verifies.  "MLA: why one latent can replace a multi-head
 * KV cache" (charlestar.github.io) lists that token count and the query
 * length among the inputs of MLA kernel selection (section on why prefill
 * need not absorb as decode does, by gloss), and the "Kernel" step of its
 * validation chain compares outputs and log-sum-exp over query/KV lengths
 * and speculative tokens.  The causal rule among the new tokens is the
 * plainest reading: each sees the cache up to its own position.
 *   out [B, q_len, h, d_v], u_latent [B, q_len, h, d_c] (nullable),
 *   lse [B, q_len, h] (nullable); q_nope [B, q_len, h, d_nope],
 *   q_rope [B, q_len, h, d_R]; weights, cache and lengths as
 *   ref_mla_absorbed.  Position jq sees the first s_b - q_len + 1 + jq
 *   tokens; one that sees none gives 0 and lse = -inf.
 */
int ref_mla_absorbed_multi(double* out, double* u_latent, double* lse, const void* q_nope,
                           const void* q_rope, const void* w_uk, const void* w_uv,
                           const void* cache, const int32_t* s, const int32_t* block_table,
                           int max_blocks, int block_size, int B, int q_len, int s_max, int h,
                           int d_c, int d_R, int d_nope, int d_v, int b, double scale)
{
    return mla_absorbed_impl(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, b, 1.0, 1.0,
                             NULL, NULL, s, block_table, max_blocks, block_size, B, q_len, s_max,
                             h, d_c, d_R, d_nope, d_v, b, scale);
}

/*
 * MLA decode through the attention block's output projection
 * ("Multi-Head Latent Attention (MLA): Mathematical Foundations" (llms.blog),
 * section "Value Output Matrix Absorption"): the heads are aggregated by
 * W_O = [W_O^1, ..., W_O^h], a [d_model, h d_v] matrix whose columns
 * i d_v .. i d_v + d_v - 1 are W_O^i, as
 *   o_t = sum_i W_O^i u_{t,i},   u_{t,i} = W_UV,i u~_{t,i}.
 * Computed in that order (each head's u in double, then the projection);
 * the merged weights W_O^i W_UV,i of the same section are the library's
 * business, and the tests pin that both groupings agree.
 *   o [B, q_len, d_model]; lse [B, q_len, h] (nullable); the rest as
 *   ref_mla_absorbed_multi, w_o [d_model, h d_v] stored with b bytes.
 */
int ref_mla_output(double* o, double* lse, const void* q_nope, const void* q_rope,
                   const void* w_uk, const void* w_uv, const void* w_o, const void* cache,
                   const int32_t* s, const int32_t* block_table, int max_blocks, int block_size,
                   int B, int q_len, int s_max, int h, int d_c, int d_R, int d_nope, int d_v,
                   int d_model, int b, double scale)
{
    if (!o || !w_o || d_model <= 0 || B < 0 || q_len < 1 || h <= 0 || d_v <= 0)
        return OR_EINVAL;
    const size_t rows = (size_t)B * q_len;
    double* u = (double*)malloc(sizeof(double) * (rows * h * (size_t)d_v + 1));
    if (!u) return OR_EINVAL;
    int rc = mla_absorbed_impl(u, NULL, lse, q_nope, q_rope, w_uk, w_uv, cache, b, 1.0, 1.0,
                               NULL, NULL, s, block_table, max_blocks, block_size, B, q_len,
                               s_max, h, d_c, d_R, d_nope, d_v, b, scale);
    if (rc == OR_OK) {
        const size_t hd = (size_t)h * d_v;
#pragma omp parallel for schedule(static)
        for (long r = 0; r < (long)rows; r++) {
            for (int n = 0; n < d_model; n++) {
                double acc = 0.0;
                for (int i = 0; i < h; i++)
                    for (int e = 0; e < d_v; e++)
                        acc += ld(w_o, (size_t)n * hd + (size_t)i * d_v + e, b) *
                               u[((size_t)r * h + i) * d_v + e];
                o[(size_t)r * d_model + n] = acc;
            }
        }
    }
    free(u);
    return rc;
}

/* ref_mla_absorbed_multi over an FP8 latent cache (as ref_mla_absorbed_fp8) */
int ref_mla_absorbed_multi_fp8(double* out, double* u_latent, double* lse, const void* q_nope,
                               const void* q_rope, const void* w_uk, const void* w_uv,
                               const uint8_t* cache, double c_scale, double r_scale,
                               const int32_t* s, const int32_t* block_table, int max_blocks,
                               int block_size, int B, int q_len, int s_max, int h, int d_c,
                               int d_R, int d_nope, int d_v, double scale)
{
    return mla_absorbed_impl(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1, c_scale,
                             r_scale, NULL, NULL, s, block_table, max_blocks, block_size, B, q_len,
                             s_max, h, d_c, d_R, d_nope, d_v, 2, scale);
}

/*
 * MLA decode over an FP8 latent cache: rows of d_c + d_R E4M3 codes, the
 * latent part scaled by c_scale and the rotary part by r_scale (one scale
 * per tensor part; "MLA: why one latent can replace a multi-head KV cache",
 * section "MLA and KV-cache quantization stack" (by gloss), notes the two
 * parts may need separate scales).  q_nope, q_rope, W_UK, W_UV are bf16.
 * Otherwise as ref_mla_absorbed.
 */
int ref_mla_absorbed_fp8(double* out, double* u_latent, double* lse, const void* q_nope,
                         const void* q_rope, const void* w_uk, const void* w_uv,
                         const uint8_t* cache, double c_scale, double r_scale, const int32_t* s,
                         const int32_t* block_table, int max_blocks, int block_size, int B,
                         int s_max, int h, int d_c, int d_R, int d_nope, int d_v, double scale)
{
    return mla_absorbed_impl(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1, c_scale,
                             r_scale, NULL, NULL, s, block_table, max_blocks, block_size, B, 1,
                             s_max, h, d_c, d_R, d_nope, d_v, 2, scale);
}

/*
 * ref_mla_absorbed_fp8 over a paged pool whose pages each carry their own
 * pair of scales ("Multi-Head Latent Attention (MLA): Mathematical
 * Foundations" (llms.blog), section "High-Throughput Serving Kernels:
 * FlashMLA and SGLang": the E4M3 latent is stored with per-block scaling
 * factors; one block = one page here): element e of token t's row is
 * code * c_scales[blk] (e < d_c) or code * r_scales[blk], blk the physical
 * page the table maps t to.  c_scales, r_scales: [num_blocks] fp32.
 */
int ref_mla_absorbed_fp8_paged_scales(double* out, double* u_latent, double* lse,
                                      const void* q_nope, const void* q_rope, const void* w_uk,
                                      const void* w_uv, const uint8_t* cache,
                                      const float* c_scales, const float* r_scales,
                                      const int32_t* s, const int32_t* block_table,
                                      int max_blocks, int block_size, int B, int h, int d_c,
                                      int d_R, int d_nope, int d_v, double scale)
{
    if (!c_scales || !r_scales || !block_table) return OR_EINVAL;
    return mla_absorbed_impl(out, u_latent, lse, q_nope, q_rope, w_uk, w_uv, cache, 1, 1.0, 1.0,
                             c_scales, r_scales, s, block_table, max_blocks, block_size, B, 1, 0,
                             h, d_c, d_R, d_nope, d_v, 2, scale);
}

/*
 * MLA decode by explicit expansion ("MHA mode"): per head and token build
 * k_t = [W_UK[i] c_t ; k_R,t] and v_t = W_UV[i] c_t, then plain attention
 * with q = [q_nope ; q_rope].  Slow reference for the absorption identities.
 */
int ref_mla_explicit(double* out, double* lse, const void* q_nope, const void* q_rope,
                     const void* w_uk, const void* w_uv, const void* cache, const int32_t* s,
                     const int32_t* block_table, int max_blocks, int block_size, int B,
                     int s_max, int h, int d_c, int d_R, int d_nope, int d_v, int b,
                     double scale)
{
    if (!out || !q_nope || !q_rope || !w_uk || !w_uv || !cache || !s) return OR_EINVAL;
    if (B < 0 || h <= 0 || d_c <= 0 || d_R < 0 || d_nope <= 0 || d_v <= 0) return OR_EINVAL;
    if (b != 2 && b != 4) return OR_EINVAL;
    if (block_table && (block_size <= 0 || max_blocks <= 0)) return OR_EINVAL;
    const int W = d_c + d_R;
    const long rows = (long)B * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / h), i = (int)(r % h);
        const int n = s[bb];
        double* o = out + (size_t)r * d_v;
        if (n < 0 || (!block_table && n > s_max) ||
            (block_table && n > max_blocks * block_size) ||
            !table_ok(block_table, max_blocks, block_size, bb, n)) {
            bad = 1;
            continue;
        }
        if (n == 0) {
            for (int e = 0; e < d_v; e++) o[e] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double* kc = (double*)malloc(sizeof(double) *
                                     ((size_t)n * d_nope + (size_t)n * d_v + (size_t)n * 2));
        double* vc = kc + (size_t)n * d_nope;
        double* z = vc + (size_t)n * d_v;
        double* p = z + n;
        for (int t = 0; t < n; t++) {
            const size_t roff = row_of(block_table, max_blocks, block_size, s_max, bb, t) * W;
            for (int e = 0; e < d_nope; e++) {
                double acc = 0.0;
                for (int c = 0; c < d_c; c++)
                    acc += ld(w_uk, ((size_t)i * d_nope + e) * d_c + c, b) * ld(cache, roff + c, b);
                kc[(size_t)t * d_nope + e] = acc;
            }
            for (int e = 0; e < d_v; e++) {
                double acc = 0.0;
                for (int c = 0; c < d_c; c++)
                    acc += ld(w_uv, ((size_t)i * d_v + e) * d_c + c, b) * ld(cache, roff + c, b);
                vc[(size_t)t * d_v + e] = acc;
            }
            double acc = 0.0;
            for (int e = 0; e < d_nope; e++)
                acc += ld(q_nope, (size_t)r * d_nope + e, b) * kc[(size_t)t * d_nope + e];
            for (int e = 0; e < d_R; e++)
                acc += ld(q_rope, (size_t)r * d_R + e, b) * ld(cache, roff + d_c + e, b);
            z[t] = scale * acc;
        }
        double m;
        const double l = softmax_weights(z, n, p, &m);
        for (int e = 0; e < d_v; e++) {
            double acc = 0.0;
            for (int t = 0; t < n; t++) acc += p[t] * vc[(size_t)t * d_v + e];
            o[e] = acc / l;
        }
        if (lse) lse[r] = m + log(l);
        free(kc);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/*
 * Cache append: copy the new token's rows into a host image of the cache at
 * slot pos[b] (contiguous row b * s_max + pos[b], or the paged row through
 * the block table).  cache_v / v_new may be NULL (MLA: one latent buffer,
 * no V).  Row width is h_kv * d_h elements of b bytes.
 */
int ref_kv_append(void* cache_k, void* cache_v, const void* k_new, const void* v_new,
                  const int32_t* pos, const int32_t* block_table, int max_blocks,
                  int block_size, int B, int s_max, int h_kv, int d_h, int b)
{
    if (!cache_k || !k_new || !pos) return OR_EINVAL;
    if ((cache_v == NULL) != (v_new == NULL)) return OR_EINVAL;
    if (B < 0 || h_kv <= 0 || d_h <= 0 || (b != 2 && b != 4)) return OR_EINVAL;
    const size_t rb = (size_t)h_kv * d_h * b;
    for (int bb = 0; bb < B; bb++) {
        const int t = pos[bb];
        if (t < 0 || (!block_table && t >= s_max) ||
            (block_table && t >= max_blocks * block_size))
            return OR_EINVAL;
        if (block_table && block_table[(size_t)bb * max_blocks + t / block_size] < 0)
            return OR_EINVAL;
        const size_t row = row_of(block_table, max_blocks, block_size, s_max, bb, t);
        memcpy((char*)cache_k + row * rb, (const char*)k_new + (size_t)bb * rb, rb);
        if (cache_v) memcpy((char*)cache_v + row * rb, (const char*)v_new + (size_t)bb * rb, rb);
    }
    return OR_OK;
}

/*
 * FP8 caches (the ranked next step after the bf16 path: "MHA -> MQA -> GQA ->
 * MLA" and the charlestar.github.io MLA page both name an 8-bit cache as the
 * way to halve the bytes per token; the scale granularity is left open).
 * Reading taken: OCP E4M3 codes ("e4m3fn": 1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN; no
 * infinities; largest finite 448) with one fp32 scale per tensor, value =
 * code * scale.
 */

/* value of an E4M3 code, by the format's definition */
double ref_fp8_e4m3_decode(int code)
{
    const int c = code & 0xff;
    const int sgn = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return sgn ? -mag : mag;
}

/*
 * E4M3 code of an fp32 value: round to nearest, ties to even, saturating at
 * +-448 (values at or beyond it, and infinities, give the largest finite
 * code); NaN gives 0x7F; the sign of zero is kept.
 */
int ref_fp8_e4m3_encode(float y)
{
    if (isnan(y)) return 0x7f;
    const int sgn = signbit(y) ? 0x80 : 0;
    const double a = fabs((double)y);
    if (a >= 448.0) return sgn | 0x7e;
    if (a == 0.0) return sgn;
    int e = (int)floor(log2(a));
    if (ldexp(1.0, e) > a) e--;          /* guard the log2 rounding */
    if (ldexp(1.0, e + 1) <= a) e++;
    if (e < -6) e = -6;                  /* subnormals share the quantum 2^-9 */
    const double quantum = ldexp(1.0, e - 3);
    double mq = rint(a / quantum);       /* exact quotient; rint rounds half to even */
    int code;
    if (e == -6 && mq < 8.0) {
        code = (int)mq;                  /* subnormal (mq = 8 is the smallest normal) */
    } else {
        if (mq >= 16.0) {                /* rounded up into the next binade */
            mq = 8.0;
            e++;
        }
        code = ((e + 7) << 3) | ((int)mq - 8);
    }
    if (code > 0x7e) code = 0x7e;
    return sgn | code;
}

static double ld_fp8(const uint8_t* p, size_t idx, double scale)
{
    return ref_fp8_e4m3_decode(p[idx]) * scale;
}

/*
 * Decode attention over an FP8 K/V cache: as ref_gqa_decode with bf16 q,
 * K(b,t,j,d) = decode(k code) * k_scale and V likewise with v_scale.
 */
int ref_gqa_decode_fp8(double* out, double* lse, const void* q, const uint8_t* k,
                       const uint8_t* v, double k_scale, double v_scale, const int32_t* s,
                       const int32_t* block_table, int max_blocks, int block_size, int B,
                       int s_max, int h, int h_kv, int d_h, double scale)
{
    if (!out || !q || !k || !v || !s) return OR_EINVAL;
    if (B < 0 || h <= 0 || h_kv <= 0 || d_h <= 0 || (h % h_kv) != 0) return OR_EINVAL;
    if (block_table && (block_size <= 0 || max_blocks <= 0)) return OR_EINVAL;
    const int g = h / h_kv;
    const long rows = (long)B * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / h), i = (int)(r % h), j = i / g;
        const int n = s[bb];
        double* o = out + (size_t)r * d_h;
        if (n < 0 || (!block_table && n > s_max) ||
            (block_table && n > max_blocks * block_size) ||
            !table_ok(block_table, max_blocks, block_size, bb, n)) {
            bad = 1;
            continue;
        }
        if (n == 0) {
            for (int d = 0; d < d_h; d++) o[d] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n * 2);
        double* p = z + n;
        const size_t qoff = (size_t)r * d_h;
        for (int t = 0; t < n; t++) {
            const size_t koff =
                (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) * d_h;
            double acc = 0.0;
            for (int d = 0; d < d_h; d++) acc += ld(q, qoff + d, 2) * ld_fp8(k, koff + d, k_scale);
            z[t] = scale * acc;
        }
        double m;
        const double l = softmax_weights(z, n, p, &m);
        for (int d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (int t = 0; t < n; t++) {
                const size_t voff =
                    (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) *
                    d_h;
                acc += p[t] * ld_fp8(v, voff + d, v_scale);
            }
            o[d] = acc / l;
        }
        if (lse) lse[r] = m + log(l);
        free(z);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/*
 * Append into FP8 caches: each element x of the bf16 rows k_new / v_new
 * becomes encode(x * inv_scale), the product taken in fp32 (inv_scale is the
 * fp32 reciprocal of the tensor's scale), at slot pos[b] as ref_kv_append.
 */
int ref_kv_append_fp8(uint8_t* cache_k, uint8_t* cache_v, const void* k_new, const void* v_new,
                      float k_inv_scale, float v_inv_scale, const int32_t* pos,
                      const int32_t* block_table, int max_blocks, int block_size, int B,
                      int s_max, int h_kv, int d_h)
{
    if (!cache_k || !k_new || !pos) return OR_EINVAL;
    if ((cache_v == NULL) != (v_new == NULL)) return OR_EINVAL;
    if (B < 0 || h_kv <= 0 || d_h <= 0) return OR_EINVAL;
    const size_t n = (size_t)h_kv * d_h;
    for (int bb = 0; bb < B; bb++) {
        const int t = pos[bb];
        if (t < 0 || (!block_table && t >= s_max) ||
            (block_table && t >= max_blocks * block_size))
            return OR_EINVAL;
        if (block_table && block_table[(size_t)bb * max_blocks + t / block_size] < 0)
            return OR_EINVAL;
        const size_t row = row_of(block_table, max_blocks, block_size, s_max, bb, t);
        for (size_t e = 0; e < n; e++) {
            const float xk = (float)ld(k_new, (size_t)bb * n + e, 2);
            cache_k[row * n + e] = (uint8_t)ref_fp8_e4m3_encode(xk * k_inv_scale);
            if (cache_v) {
                const float xv = (float)ld(v_new, (size_t)bb * n + e, 2);
                cache_v[row * n + e] = (uint8_t)ref_fp8_e4m3_encode(xv * v_inv_scale);
            }
        }
    }
    return OR_OK;
}

/*
 * Append into an FP8 latent cache: element e of the bf16 row kv_new[b]
 * ([c | k_R], d_c + d_R wide) becomes encode(x * c_inv) for e < d_c and
 * encode(x * r_inv) after, the products in fp32, at slot pos[b].
 */
int ref_kv_append_mla_fp8(uint8_t* cache, const void* kv_new, float c_inv_scale,
                          float r_inv_scale, const int32_t* pos, const int32_t* block_table,
                          int max_blocks, int block_size, int B, int s_max, int d_c, int d_R)
{
    if (!cache || !kv_new || !pos) return OR_EINVAL;
    if (B < 0 || d_c <= 0 || d_R < 0) return OR_EINVAL;
    const size_t n = (size_t)d_c + d_R;
    for (int bb = 0; bb < B; bb++) {
        const int t = pos[bb];
        if (t < 0 || (!block_table && t >= s_max) ||
            (block_table && t >= max_blocks * block_size))
            return OR_EINVAL;
        if (block_table && block_table[(size_t)bb * max_blocks + t / block_size] < 0)
            return OR_EINVAL;
        const size_t row = row_of(block_table, max_blocks, block_size, s_max, bb, t);
        for (size_t e = 0; e < n; e++) {
            const float x = (float)ld(kv_new, (size_t)bb * n + e, 2);
            cache[row * n + e] =
                (uint8_t)ref_fp8_e4m3_encode(x * ((int)e < d_c ? c_inv_scale : r_inv_scale));
        }
    }
    return OR_OK;
}

/*
 * Append of latent rows into a paged FP8 pool with per-page scales: element
 * x of kv_new[b] becomes encode(x * (1 / c_scales[blk])) in the latent part
 * and encode(x * (1 / r_scales[blk])) in the rotary part, the reciprocal and
 * the product in fp32, blk the page of slot pos[b].
 */
int ref_kv_append_mla_fp8_paged_scales(uint8_t* cache, const void* kv_new, const float* c_scales,
                                       const float* r_scales, const int32_t* pos,
                                       const int32_t* block_table, int max_blocks,
                                       int block_size, int B, int d_c, int d_R)
{
    if (!cache || !kv_new || !c_scales || !r_scales || !pos || !block_table) return OR_EINVAL;
    if (B < 0 || d_c <= 0 || d_R < 0 || block_size <= 0 || max_blocks <= 0) return OR_EINVAL;
    const size_t n = (size_t)d_c + d_R;
    for (int bb = 0; bb < B; bb++) {
        const int t = pos[bb];
        if (t < 0 || t >= max_blocks * block_size) return OR_EINVAL;
        const int blk = block_table[(size_t)bb * max_blocks + t / block_size];
        if (blk < 0) return OR_EINVAL;
        const size_t row = row_of(block_table, max_blocks, block_size, 0, bb, t);
        const float ic = 1.0f / c_scales[blk], ir = 1.0f / r_scales[blk];
        for (size_t e = 0; e < n; e++) {
            const float x = (float)ld(kv_new, (size_t)bb * n + e, 2);
            cache[row * n + e] = (uint8_t)ref_fp8_e4m3_encode(x * ((int)e < d_c ? ic : ir));
        }
    }
    return OR_OK;
}

/*
 * Merge of attention computed over disjoint slices of the same tokens.
 * Slice k of row r (= b * h + i) holds o_k, the softmax-weighted output over
 * its own tokens, and lse_k = ln sum_{t in k} exp(z_t) (-inf for an empty
 * slice).  Because exp(z_t) = exp(lse_k) * (weight of t inside slice k), the
 * output over all tokens is
 *   lse = ln sum_k exp(lse_k),  o = sum_k exp(lse_k - lse) o_k,
 * evaluated with M = max_k lse_k subtracted first.  A row whose slices are
 * all empty gives o = 0 and lse = -inf, as an empty decode does.
 *   out [B, h, d] double, lse [B, h] double (nullable)
 *   o_parts [n, B, h, d] stored dtype b, lse_parts [n, B, h] fp32
 */
int ref_merge_partials(double* out, double* lse, const void* o_parts, const float* lse_parts,
                       int n, int B, int h, int d, int b)
{
    if (!out || !o_parts || !lse_parts) return OR_EINVAL;
    if (n <= 0 || B < 0 || h <= 0 || d <= 0 || (b != 2 && b != 4)) return OR_EINVAL;
    const long rows = (long)B * h;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; r++) {
        double* o = out + (size_t)r * d;
        double M = -INFINITY;
        for (int k = 0; k < n; k++) {
            const double x = (double)lse_parts[(size_t)k * rows + r];
            if (x > M) M = x;
        }
        for (int c = 0; c < d; c++) o[c] = 0.0;
        if (M == -INFINITY) {
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double L = 0.0;
        for (int k = 0; k < n; k++) {
            const double w = exp((double)lse_parts[(size_t)k * rows + r] - M);
            L += w;
            for (int c = 0; c < d; c++) o[c] += w * ld(o_parts, ((size_t)k * rows + r) * d + c, b);
        }
        for (int c = 0; c < d; c++) o[c] /= L;
        if (lse) lse[r] = M + log(L);
    }
    return OR_OK;
}

/* one cache element: b = 1 -> E4M3 code times its scale, else stored bits */
static double ld_cache(const void* p, size_t idx, int b, double scale)
{
    if (b == 1) return ld_fp8((const uint8_t*)p, idx, scale);
    return ld(p, idx, b);
}

/*
 * Decode attention for q_len new tokens per sequence at once (the tokens a
 * speculative step verifies; "MLA: why one latent can replace a multi-head
 * KV cache", section "MHA mode and MQA mode are execution forms" (by gloss),
 * lists their number among what selects a decode kernel).
 * All q_len tokens are already in the cache, so s_b counts them; query
 * position jq (0-based) sits at cache position s_b - q_len + jq and attends
 * to the n = s_b - q_len + 1 + jq tokens up to and including itself (causal
 * among the new tokens).  n <= 0 gives out = 0, lse = -inf.
 *   out [B, q_len, h, d_h] double, lse [B, q_len, h] double (nullable)
 *   q   [B, q_len, h, d_h]   bf16 bits when b = 1, else stored dtype b
 *   k,v as ref_gqa_decode; b = 1: E4M3 codes, element = code * k_scale
 *       (v_scale), else k_scale and v_scale are ignored
 */
int ref_gqa_decode_multi(double* out, double* lse, const void* q, const void* k, const void* v,
                         double k_scale, double v_scale, const int32_t* s,
                         const int32_t* block_table, int max_blocks, int block_size, int B,
                         int q_len, int s_max, int h, int h_kv, int d_h, int b, double scale)
{
    if (!out || !q || !k || !v || !s) return OR_EINVAL;
    if (B < 0 || q_len < 1 || h <= 0 || h_kv <= 0 || d_h <= 0 || (h % h_kv) != 0)
        return OR_EINVAL;
    if (b != 1 && b != 2 && b != 4) return OR_EINVAL;
    if (block_table && (block_size <= 0 || max_blocks <= 0)) return OR_EINVAL;
    const int g = h / h_kv, bq = b == 1 ? 2 : b;
    const long rows = (long)B * q_len * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / ((long)q_len * h));
        const int jq = (int)((r / h) % q_len), i = (int)(r % h), j = i / g;
        const int sb = s[bb];
        double* o = out + (size_t)r * d_h;
        if (sb < 0 || (!block_table && sb > s_max) ||
            (block_table && sb > max_blocks * block_size) ||
            !table_ok(block_table, max_blocks, block_size, bb, sb)) {
            bad = 1;
            continue;
        }
        const int n = sb - (q_len - 1 - jq);   /* visible tokens of this position */
        if (n <= 0) {
            for (int d = 0; d < d_h; d++) o[d] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n * 2);
        double* p = z + n;
        const size_t qoff = (size_t)r * d_h;
        for (int t = 0; t < n; t++) {
            const size_t koff =
                (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) * d_h;
            double acc = 0.0;
            for (int d = 0; d < d_h; d++) acc += ld(q, qoff + d, bq) * ld_cache(k, koff + d, b, k_scale);
            z[t] = scale * acc;
        }
        double m;
        const double l = softmax_weights(z, n, p, &m);
        for (int d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (int t = 0; t < n; t++) {
                const size_t voff =
                    (row_of(block_table, max_blocks, block_size, s_max, bb, t) * h_kv + j) *
                    d_h;
                acc += p[t] * ld_cache(v, voff + d, b, v_scale);
            }
            o[d] = acc / l;
        }
        if (lse) lse[r] = m + log(l);
        free(z);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/*
 * Decode attention over a paged FP8 cache with one scale per page and KV
 * head: K(b,t,j,d) = decode(code) * k_scales[blk * h_kv + j] with blk =
 * block_table[b][t / block_size] (V likewise), the per-block scaling of a
 * quantised cache that "Multi-Head Latent Attention (MLA): Mathematical
 * Foundations ...", section "High-Throughput Serving Kernels: FlashMLA and
 * SGLang", describes.  Otherwise as ref_gqa_decode_fp8 (block_table
 * required).
 */
int ref_gqa_decode_fp8_paged_scales(double* out, double* lse, const void* q, const uint8_t* k,
                                    const uint8_t* v, const float* k_scales,
                                    const float* v_scales, const int32_t* s,
                                    const int32_t* block_table, int max_blocks, int block_size,
                                    int B, int h, int h_kv, int d_h, double scale)
{
    if (!out || !q || !k || !v || !k_scales || !v_scales || !s || !block_table) return OR_EINVAL;
    if (B < 0 || h <= 0 || h_kv <= 0 || d_h <= 0 || (h % h_kv) != 0) return OR_EINVAL;
    if (block_size <= 0 || max_blocks <= 0) return OR_EINVAL;
    const int g = h / h_kv;
    const long rows = (long)B * h;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (long r = 0; r < rows; r++) {
        const int bb = (int)(r / h), i = (int)(r % h), j = i / g;
        const int n = s[bb];
        double* o = out + (size_t)r * d_h;
        if (n < 0 || n > max_blocks * block_size ||
            !table_ok(block_table, max_blocks, block_size, bb, n)) {
            bad = 1;
            continue;
        }
        if (n == 0) {
            for (int d = 0; d < d_h; d++) o[d] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double* z = (double*)malloc(sizeof(double) * (size_t)n * 2);
        double* p = z + n;
        const size_t qoff = (size_t)r * d_h;
        for (int t = 0; t < n; t++) {
            const int blk = block_table[(size_t)bb * max_blocks + t / block_size];
            const double ks = (double)k_scales[(size_t)blk * h_kv + j];
            const size_t koff = (row_of(block_table, max_blocks, block_size, 0, bb, t) * h_kv + j) * d_h;
            double acc = 0.0;
            for (int d = 0; d < d_h; d++) acc += ld(q, qoff + d, 2) * ld_fp8(k, koff + d, ks);
            z[t] = scale * acc;
        }
        double m;
        const double l = softmax_weights(z, n, p, &m);
        for (int d = 0; d < d_h; d++) {
            double acc = 0.0;
            for (int t = 0; t < n; t++) {
                const int blk = block_table[(size_t)bb * max_blocks + t / block_size];
                const double vs = (double)v_scales[(size_t)blk * h_kv + j];
                const size_t voff = (row_of(block_table, max_blocks, block_size, 0, bb, t) * h_kv + j) * d_h;
                acc += p[t] * ld_fp8(v, voff + d, vs);
            }
            o[d] = acc / l;
        }
        if (lse) lse[r] = m + log(l);
        free(z);
    }
    return bad ? OR_EINVAL : OR_OK;
}

/*
 * Append into a paged FP8 cache with per-page scales: element x of the bf16
 * rows becomes encode(x * (1 / scale of its page and KV head)), the
 * reciprocal and the product in fp32, at slot pos[b].
 */
int ref_kv_append_fp8_paged_scales(uint8_t* cache_k, uint8_t* cache_v, const void* k_new,
                                   const void* v_new, const float* k_scales,
                                   const float* v_scales, const int32_t* pos,
                                   const int32_t* block_table, int max_blocks, int block_size,
                                   int B, int h_kv, int d_h)
{
    if (!cache_k || !cache_v || !k_new || !v_new || !k_scales || !v_scales || !pos || !block_table)
        return OR_EINVAL;
    if (B < 0 || h_kv <= 0 || d_h <= 0 || block_size <= 0 || max_blocks <= 0) return OR_EINVAL;
    const size_t n = (size_t)h_kv * d_h;
    for (int bb = 0; bb < B; bb++) {
        const int t = pos[bb];
        if (t < 0 || t >= max_blocks * block_size) return OR_EINVAL;
        const int blk = block_table[(size_t)bb * max_blocks + t / block_size];
        if (blk < 0) return OR_EINVAL;
        const size_t row = row_of(block_table, max_blocks, block_size, 0, bb, t);
        for (size_t e = 0; e < n; e++) {
            const int j = (int)(e / d_h);
            const float ik = 1.0f / k_scales[(size_t)blk * h_kv + j];
            const float iv = 1.0f / v_scales[(size_t)blk * h_kv + j];
            cache_k[row * n + e] = (uint8_t)ref_fp8_e4m3_encode((float)ld(k_new, (size_t)bb * n + e, 2) * ik);
            cache_v[row * n + e] = (uint8_t)ref_fp8_e4m3_encode((float)ld(v_new, (size_t)bb * n + e, 2) * iv);
        }
    }
    return OR_OK;
}
