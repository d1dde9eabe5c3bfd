/*
 * gqa_oracle.c -- plain, slow, obviously correct CPU oracle for grouped-query
 * attention (GQA).  TEST INFRASTRUCTURE ONLY: it is called by tests/, by the
 * smoke check and by the bench's CPU-baseline leg, never by the library.  It
 * shares no source with the HIP path.
 *
 * Everything here is written from the definition on the pages:
 *
 *  - "Grouped-Query Attention" concept page (compassingai.com), section
 *    技术原理 (technical principle), steps 2-4: Q [B,s,H,d] is viewed as
 *    [B,s,K,H/K,d], so query head h belongs to group g = h / (H/K); every head
 *    of group g attends to the one K/V head g with
 *    softmax(Q_group K_g^T / sqrt(d_k)) V_g; the per-group results are put
 *    back in [B,s,H,d].
 *  - same page, section 关键参数 (key parameters) #2: a token of one layer
 *    holds 2*K*d_k cache elements (one K row and one V row per KV head).
 *  - LLM inference-optimisation page (iopencloud.com), §6.1: total KV
 *    memory = 2 * layers * kv_heads * head_dim * seq_len * batch * bytes.
 *  - same page §9.1 / §9.2.1: the standard (non-streaming) softmax takes
 *    three passes over the scores: the max, the sum of exponentials, the
 *    weighted sum of V.  That three-pass form is what this file computes.
 *  - same page §8.2: a paged cache maps logical block t/bs of a sequence to
 *    a physical block through that sequence's block table.
 *
 * Arithmetic is IEEE fp64 on inputs that the caller has already decoded
 * exactly to fp64 (a bf16 or fp32 value converts to fp64 without error).
 * Loops are written in the definition's order; nothing is blocked, fused
 * or reordered.  OpenMP only distributes independent output rows.
 *
 * Parity pins for these functions live in tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------- */
/* Cache-size arithmetic                                                   */
/* ---------------------------------------------------------------------- */

/* Elements one token adds to one layer's cache: a K row and a V row for
 * each of the K KV heads (concept page, 关键参数 #2). */
int64_t oracle_cache_elems_per_token(int64_t kv_heads, int64_t head_dim)
{
    return 2 * kv_heads * head_dim;
}

/* Total KV elements (inference-optimisation page §6.1, without the
 * bytes-per-element factor). */
int64_t oracle_kv_cache_elems(int64_t layers, int64_t kv_heads, int64_t head_dim,
                              int64_t seq_len, int64_t batch)
{
    return 2 * layers * kv_heads * head_dim * seq_len * batch;
}

/* ---------------------------------------------------------------------- */
/* One attention row, three passes (max, sum of exp, weighted V sum)       */
/* ---------------------------------------------------------------------- */

/*
 * q_row: d values of one query head.
 * k_head, v_head: the [S_k, d] rows of that head's KV group (row stride d).
 * n_vis: number of visible keys, keys 0 .. n_vis-1.
 * out_row: d outputs.  Returns 0, or 1 if no key is visible (out = NaN).
 */
static int attend_row(const double *q_row, const double *k_head, const double *v_head,
                      int64_t n_vis, int d, double scale, double *scores, double *out_row)
{
    if (n_vis <= 0) {
        for (int c = 0; c < d; ++c) out_row[c] = NAN;
        return 1;
    }
    /* scores s_j = scale * <q, k_j> */
    for (int64_t j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q_row[c] * k_head[j * d + c];
        scores[j] = scale * dot;
    }
    /* pass 1: the row maximum */
    double m = scores[0];
    for (int64_t j = 1; j < n_vis; ++j)
        if (scores[j] > m) m = scores[j];
    /* pass 2: p_j = exp(s_j - m) and their sum */
    double l = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        scores[j] = exp(scores[j] - m);
        l += scores[j];
    }
    /* pass 3: sum_j p_j v_j / sum_j p_j */
    for (int c = 0; c < d; ++c) out_row[c] = 0.0;
    for (int64_t j = 0; j < n_vis; ++j) {
        const double p = scores[j];
        for (int c = 0; c < d; ++c) out_row[c] += p * v_head[j * d + c];
    }
    for (int c = 0; c < d; ++c) out_row[c] /= l;
    return 0;
}

/* Number of keys visible to query row i of sequence b.
 * The query sits at absolute position qpos = q_start[b] + i.  Keys are
 * 0 .. kv_len[b]-1; with causal != 0 a key j is visible only when j <= qpos
 * (token t attends to itself and every earlier token: inference-optimisation
 * page §5.1). */
static int64_t visible_keys(int64_t qpos, int64_t kv_len, int causal)
{
    int64_t n = kv_len;
    if (causal && qpos + 1 < n) n = qpos + 1;
    return n < 0 ? 0 : n;
}

/*
 * Grouped-query attention over a contiguous head-major cache.
 *   q      [B, Sq, H, d]
 *   k, v   [B, K, Sk, d]
 *   q_start[B]  absolute position of query row 0 of each sequence
 *   kv_len [B]  valid keys of each sequence (<= Sk)
 *   out    [B, Sq, H, d]
 * Query head h reads KV head g = h / (H / K).
 * Returns the number of rows with no visible key (those rows are NaN).
 */
int64_t oracle_gqa_attention(const double *q, const double *k, const double *v,
                             int B, int Sq, int H, int K, int d, int Sk,
                             const int32_t *q_start, const int32_t *kv_len,
                             int causal, double scale, double *out)
{
    if (B <= 0 || Sq <= 0 || H <= 0 || K <= 0 || d <= 0 || Sk < 0 || H % K != 0) return -1;
    const int G = H / K;
    int64_t empty = 0;
    const int64_t n_rows = (int64_t)B * Sq * H;
#pragma omp parallel reduction(+ : empty)
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for schedule(dynamic, 16)
        for (int64_t row = 0; row < n_rows; ++row) {
            const int h = (int)(row % H);
            const int i = (int)((row / H) % Sq);
            const int b = (int)(row / ((int64_t)H * Sq));
            const int g = h / G; /* head -> group map */
            int64_t len = kv_len[b] < Sk ? kv_len[b] : Sk;
            const int64_t n_vis = visible_keys((int64_t)q_start[b] + i, len, causal);
            const double *q_row = q + (((int64_t)b * Sq + i) * H + h) * d;
            const double *k_head = k + ((int64_t)b * K + g) * Sk * d;
            const double *v_head = v + ((int64_t)b * K + g) * Sk * d;
            double *o_row = out + (((int64_t)b * Sq + i) * H + h) * d;
            empty += attend_row(q_row, k_head, v_head, n_vis, d, scale, scores, o_row);
        }
        free(scores);
    }
    return empty;
}

/*
 * The same definition evaluated only at listed rows, so that a large
 * workload can be checked on a sample.  rows[3*r + 0..2] = (b, i, h);
 * out is [n_rows, d].
 */
/*
 * The rows variant with a sliding window (inference-optimisation page
 * §6.4.1: attention kept to the most recent N tokens).  window > 0: the row
 * at position qpos sees only the keys from qpos + 1 - window on (and, as
 * without a window, below its visible end); window <= 0: no window.
 */
int64_t oracle_gqa_attention_rows_window(const double *q, const double *k, const double *v,
                                         int B, int Sq, int H, int K, int d, int Sk,
                                         const int32_t *q_start, const int32_t *kv_len,
                                         int causal, double scale, int window,
                                         int64_t n_rows, const int32_t *rows, double *out);

int64_t oracle_gqa_attention_rows(const double *q, const double *k, const double *v,
                                  int B, int Sq, int H, int K, int d, int Sk,
                                  const int32_t *q_start, const int32_t *kv_len,
                                  int causal, double scale,
                                  int64_t n_rows, const int32_t *rows, double *out)
{
    return oracle_gqa_attention_rows_window(q, k, v, B, Sq, H, K, d, Sk, q_start, kv_len, causal, scale, 0,
                                            n_rows, rows, out);
}

int64_t oracle_gqa_attention_rows_window(const double *q, const double *k, const double *v,
                                         int B, int Sq, int H, int K, int d, int Sk,
                                         const int32_t *q_start, const int32_t *kv_len,
                                         int causal, double scale, int window,
                                         int64_t n_rows, const int32_t *rows, double *out)
{
    if (B <= 0 || Sq <= 0 || H <= 0 || K <= 0 || d <= 0 || Sk < 0 || H % K != 0) return -1;
    const int G = H / K;
    int64_t empty = 0;
#pragma omp parallel reduction(+ : empty)
    {
        double *scores = (double *)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < n_rows; ++r) {
            const int b = rows[3 * r + 0], i = rows[3 * r + 1], h = rows[3 * r + 2];
            if (b < 0 || b >= B || i < 0 || i >= Sq || h < 0 || h >= H) {
                for (int c = 0; c < d; ++c) out[r * d + c] = NAN;
                empty += 1;
                continue;
            }
            const int g = h / G;
            int64_t len = kv_len[b] < Sk ? kv_len[b] : Sk;
            const int64_t qpos = (int64_t)q_start[b] + i;
            const int64_t n_vis = visible_keys(qpos, len, causal);
            /* with a window: keys lo .. n_vis-1 */
            int64_t lo = window > 0 ? qpos + 1 - window : 0;
            if (lo < 0) lo = 0;
            if (lo > n_vis) lo = n_vis;
            const double *q_row = q + (((int64_t)b * Sq + i) * H + h) * d;
            const double *k_head = k + (((int64_t)b * K + g) * Sk + lo) * d;
            const double *v_head = v + (((int64_t)b * K + g) * Sk + lo) * d;
            empty += attend_row(q_row, k_head, v_head, n_vis - lo, d, scale, scores, out + r * d);
        }
        free(scores);
    }
    return empty;
}

/* ---------------------------------------------------------------------- */
/* Cache writes and paged reads: plain indexed copies                      */
/* ---------------------------------------------------------------------- */

/*
 * Append new rows to a contiguous head-major cache (concept page 技术原理:
 * a new token contributes K/V of shape [B, 1, K, d]; here s_new tokens):
 *   cache[b, g, start_pos[b] + t, :] = new_rows[b, t, g, :]
 * cache is [B, K, S_max, d]; new_rows is [B, s_new, K, d]; elem_bytes is the
 * size of one element.  Rows that would land at or beyond S_max are not
 * written; the count of such rows is returned.
 */
int64_t oracle_kv_append(void *cache, const void *new_rows, const int32_t *start_pos,
                         int B, int s_new, int K, int d, int S_max, int elem_bytes)
{
    const size_t row_bytes = (size_t)d * (size_t)elem_bytes;
    int64_t dropped = 0;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < s_new; ++t)
            for (int g = 0; g < K; ++g) {
                const int64_t pos = (int64_t)start_pos[b] + t;
                if (pos < 0 || pos >= S_max) { ++dropped; continue; }
                const char *src = (const char *)new_rows +
                                  (((int64_t)b * s_new + t) * K + g) * row_bytes;
                char *dst = (char *)cache + (((int64_t)b * K + g) * S_max + pos) * row_bytes;
                memcpy(dst, src, row_bytes);
            }
    return dropped;
}

/*
 * Append into a paged pool [num_blocks, K, block_size, d]
 * (inference-optimisation page §8.2: logical block -> physical block through
 * the per-sequence block table):
 *   pos = start_pos[b] + t
 *   pool[block_table[b, pos / block_size], g, pos % block_size, :] = new_rows[b, t, g, :]
 * block_table is [B, max_blocks].  Rows whose logical block is beyond the
 * table or whose physical id is outside [0, num_blocks) are not written and
 * are counted in the return value.
 */
int64_t oracle_kv_append_paged(void *pool, const void *new_rows, const int32_t *start_pos,
                               const int32_t *block_table, int max_blocks, int num_blocks,
                               int block_size, int B, int s_new, int K, int d, int elem_bytes)
{
    const size_t row_bytes = (size_t)d * (size_t)elem_bytes;
    int64_t dropped = 0;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < s_new; ++t)
            for (int g = 0; g < K; ++g) {
                const int64_t pos = (int64_t)start_pos[b] + t;
                const int64_t logical = pos / block_size;
                if (pos < 0 || logical >= max_blocks) { ++dropped; continue; }
                const int32_t phys = block_table[(int64_t)b * max_blocks + logical];
                if (phys < 0 || phys >= num_blocks) { ++dropped; continue; }
                const char *src = (const char *)new_rows +
                                  (((int64_t)b * s_new + t) * K + g) * row_bytes;
                char *dst = (char *)pool +
                            (((int64_t)phys * K + g) * block_size + pos % block_size) * row_bytes;
                memcpy(dst, src, row_bytes);
            }
    return dropped;
}

/*
 * The same gather for raw elements of elem_bytes bytes (no decoding): rows
 * that no valid block provides are left as the caller filled them.
 */
int64_t oracle_gather_paged_raw(const void *pool, int elem_bytes, const int32_t *block_table,
                                int max_blocks, int num_blocks, int block_size,
                                const int32_t *ctx_lens, int B, int K, int d, int S_out, void *out)
{
    const size_t row_bytes = (size_t)d * (size_t)elem_bytes;
    int64_t bad = 0;
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < K; ++g)
            for (int64_t t = 0; t < S_out && t < ctx_lens[b]; ++t) {
                if (t / block_size >= max_blocks) { ++bad; continue; }
                const int32_t phys = block_table[(int64_t)b * max_blocks + t / block_size];
                if (phys < 0 || phys >= num_blocks) { ++bad; continue; }
                const char *src = (const char *)pool +
                                  (((int64_t)phys * K + g) * block_size + t % block_size) * row_bytes;
                char *dst = (char *)out + (((int64_t)b * K + g) * S_out + t) * row_bytes;
                memcpy(dst, src, row_bytes);
            }
    return bad;
}

/*
 * Gather a paged pool into a contiguous [B, K, S_out, d] array of doubles:
 *   out[b, g, t, :] = pool[block_table[b, t / block_size], g, t % block_size, :]
 * for t < min(ctx_lens[b], S_out); other positions are set to NaN.  The
 * paged attention of the oracle is this gather followed by
 * oracle_gqa_attention, so paged and contiguous answers agree exactly.
 */
int64_t oracle_gather_paged(const double *pool, const int32_t *block_table, int max_blocks,
                            int num_blocks, int block_size, const int32_t *ctx_lens,
                            int B, int K, int d, int S_out, double *out)
{
    int64_t bad = 0;
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < K; ++g)
            for (int64_t t = 0; t < S_out; ++t) {
                double *dst = out + (((int64_t)b * K + g) * S_out + t) * d;
                int ok = t < ctx_lens[b] && t / block_size < max_blocks;
                int32_t phys = ok ? block_table[(int64_t)b * max_blocks + t / block_size] : -1;
                if (ok && (phys < 0 || phys >= num_blocks)) { ok = 0; ++bad; }
                if (!ok) {
                    for (int c = 0; c < d; ++c) dst[c] = NAN;
                    continue;
                }
                const double *src = pool + (((int64_t)phys * K + g) * block_size + t % block_size) * d;
                memcpy(dst, src, sizeof(double) * (size_t)d);
            }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* FP8 (E4M3) KV cache with one scale per cached row                      */
/* ---------------------------------------------------------------------- */

/*
 * The inference-optimisation page, §15.5-§15.5.1, lists for K/V quantisation
 * a scale computed for every token (per-token) or every head (per-head), and
 * FP8 E4M3 as the format whose exponent copes with the long-tailed K/V
 * values.  Reading: one fp32 scale per cached row (one token of one KV head),
 * scale = amax / 448 with 448 the largest finite E4M3 value, and every
 * element stored as the E4M3 value nearest to x / scale (ties to the even
 * code).  The decisions are taken in fp32 (the scale and each quotient are
 * IEEE fp32 divisions), the precision the device takes them in, so codes
 * and scales can be compared bit for bit.  A row that is all zero has
 * scale 0 and all-zero codes.
 *
 * E4M3 here is the OCP 8-bit format: 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits; exponent field 0 holds the subnormals m * 2^-9;
 * there are no infinities and S.1111.111 is NaN, so the largest finite
 * magnitude is 1.75 * 2^8 = 448.
 */
double oracle_e4m3_value(uint8_t code)
{
    const int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* The E4M3 code nearest to x (ties to even), saturating at +-448. */
uint8_t oracle_e4m3_from_float(float x)
{
    const uint8_t sign = signbit(x) ? 0x80 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return 0x7F;
    if (a >= 448.0) return sign | 0x7E;   /* satfinite */
    /* the spacing of E4M3 values around a: 2^-9 below 2^-6 (subnormals),
     * else 2^(floor(log2 a) - 3) */
    int ex = 0;
    if (a > 0) frexp(a, &ex);             /* a = f * 2^ex, f in [0.5, 1) */
    const int e_unb = ex - 1;             /* floor(log2 a) */
    const int step_exp = e_unb < -6 ? -9 : e_unb - 3;
    const double n = rint(ldexp(a, -step_exp));   /* round half to even (default mode) */
    double v = ldexp(n, step_exp);
    if (v > 448.0) v = 448.0;
    if (v == 0.0) return sign;
    /* encode v exactly */
    if (v < ldexp(1.0, -6)) return sign | (uint8_t)ldexp(v, 9);
    frexp(v, &ex);
    const int e = ex - 1;                 /* v = (1 + m/8) * 2^e */
    const int m = (int)(ldexp(v, -e) * 8.0) - 8;
    return sign | (uint8_t)(((e + 7) << 3) | m);
}

/*
 * Quantise rows of d fp32 values (bf16 values are exact in fp32):
 * codes[r, i] = E4M3(x[r, i] / scale[r]), scale[r] = amax_r / 448 (fp32).
 */
void oracle_quantize_e4m3_rows(const float *x, int64_t rows, int d, uint8_t *codes, float *scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * d;
        float amax = 0.0f;
        for (int i = 0; i < d; ++i) {
            const float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        const float scale = amax / 448.0f;
        scales[r] = scale;
        for (int i = 0; i < d; ++i) {
            if (amax == 0.0f) { codes[r * d + i] = 0; continue; }
            const float q = xr[i] / scale;
            codes[r * d + i] = oracle_e4m3_from_float(q);
        }
    }
}

/* The values a quantised row stands for: scale[r] * E4M3(codes[r, i]),
 * exact in fp64. */
void oracle_dequantize_e4m3_rows(const uint8_t *codes, const float *scales, int64_t rows, int d, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < d; ++i)
            out[r * d + i] = (double)scales[r] * oracle_e4m3_value(codes[r * d + i]);
}

/* ---------------------------------------------------------------------- */
/* INT8 KV cache with one scale per cached row                            */
/* ---------------------------------------------------------------------- */

/*
 * The inference-optimisation page, §15.5-§15.5.1, names INT8 beside FP8 for
 * K/V quantisation, with a scale per token or per head, and gives no formula.
 * Reading: symmetric INT8 with one fp32 scale per cached row (one token of
 * one KV head), scale = amax / 127, and every element stored as the integer
 * nearest to x * (1 / scale) (ties to even), |code| <= 127.  The reciprocal
 * and the product are IEEE fp32 operations, as in PyTorch's per-channel
 * qint8 quantiser, and the device takes the same decisions in the same
 * precision, so codes and scales compare bit for bit.  A row that is all zero
 * has scale 0 and all-zero codes.  The value a code stands for is
 * scale * code.
 */
void oracle_quantize_i8_rows(const float *x, int64_t rows, int d, int8_t *codes, float *scales)
{
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * d;
        float amax = 0.0f;
        for (int i = 0; i < d; ++i) {
            const float a = fabsf(xr[i]);
            if (a > amax) amax = a;
        }
        const float scale = amax / 127.0f;
        scales[r] = scale;
        const float inv = amax > 0.0f ? 1.0f / scale : 0.0f;
        for (int i = 0; i < d; ++i) {
            const float q = xr[i] * inv;          /* fp32 product */
            float n = rintf(q);                   /* nearest, ties to even (default mode) */
            if (n > 127.0f) n = 127.0f;
            if (!(n >= -127.0f)) n = -127.0f;     /* below, or NaN (a non-finite row): no cast of NaN */
            codes[r * d + i] = (int8_t)n;
        }
    }
}

/* The values a quantised row stands for: scale[r] * codes[r, i], exact in fp64. */
void oracle_dequantize_i8_rows(const int8_t *codes, const float *scales, int64_t rows, int d, double *out)
{
    for (int64_t r = 0; r < rows; ++r)
        for (int i = 0; i < d; ++i)
            out[r * d + i] = (double)scales[r] * (double)codes[r * d + i];
}
