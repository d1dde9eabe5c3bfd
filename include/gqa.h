/*
 * gqa.h -- C ABI of libgqa.so: grouped-query attention on AMD Instinct MI355X
 * (gfx950).
 *
 * The operation (the "Grouped-Query Attention" concept page, compassingai.com,
 * section 技术原理, steps 2-4): the H query heads are split into K groups of
 * G = H / K heads; query head h belongs to group g = h / G and attends to the
 * single K/V head g of the cache:
 *
 *     out[b, i, h, :] = softmax(q[b, i, h, :] . K_g^T * scale) V_g
 *
 * over the keys visible to that query row.  H must be a multiple of K; K = H
 * is multi-head attention and K = 1 multi-query attention (same page, and the
 * inference-optimisation page, iopencloud.com, §7.1).
 *
 * Layouts (all row-major, element type given by gqa_kv_cache.dtype):
 *   queries / outputs   [B, s, H, d]        (concept page, steps 2 and 4)
 *   new keys / values   [B, s_new, K, d]    (concept page, 技术原理: a new token
 *                                            writes K/V of shape [B, 1, K, d])
 *   contiguous cache    [B, K, S_max, d]    for K and for V separately
 *   paged cache pool    [num_blocks, K, block_size, d]; token t of sequence b
 *                       lives in physical block block_table[b, t / block_size],
 *                       slot t % block_size (inference-optimisation page §8.2)
 *
 * Conventions
 *   - Ownership: the caller owns every buffer (queries, cache, block table,
 *     context lengths, outputs, workspace).  The library never allocates or
 *     frees memory and keeps no state besides cached device properties.
 *   - Pointers are device pointers unless stated otherwise; the
 *     gqa_kv_cache descriptor itself is a host struct.
 *   - Asynchrony: every call enqueues its kernels on `stream` (a hipStream_t
 *     passed as void*, NULL = the default stream) and returns; no call
 *     synchronises unless GQA_CHECK=1 is set in the environment.
 *   - Errors: arguments that the host can check are checked before anything
 *     is enqueued; a bad one returns GQA_ERR_INVALID_ARG / GQA_ERR_UNSUPPORTED
 *     / GQA_ERR_WORKSPACE and nothing runs.  A failed launch returns
 *     GQA_ERR_LAUNCH.  Nothing is thrown across the ABI.
 *   - Device-resident integers (start positions, context lengths, block ids)
 *     are the caller's contract.  Kernels never access memory outside the
 *     buffers described by the arguments whatever those integers hold:
 *     positions past the cache capacity and block ids outside
 *     [0, num_blocks) are skipped (append) or read as zeros (attention), and a
 *     context length below 1 yields an all-zero output row.  With GQA_CHECK=1
 *     the host copies them back, validates them and returns
 *     GQA_ERR_DEVICE_ARG before launching if one is out of range.
 *   - Supported: dtype GQA_BF16 or GQA_F32 (and the quantised caches
 *     below), head_dim 64 or 128,
 *     1 <= K <= H, H % K == 0, G = H / K <= 64, block_size a power of two in
 *     [1, 1024].
 *   - The softmax scale must be a positive finite number (normally
 *     1 / sqrt(d), the concept page's 1/sqrt(d_k)); any other value returns
 *     GQA_ERR_INVALID_ARG.
 *   - Environment knobs, read at every call: GQA_CHECK=1 (above);
 *     GQA_DECODE_WGS=n with 1 <= n <= 512 fixes the number of workgroups a
 *     decode launch splits the keys over (flash-decoding's split count,
 *     inference-optimisation page §10.2; the result is the same for every n
 *     up to the rounding of the merge); unset, each kernel picks its own.
 *   - Quantised cache (GQA_FP8_E4M3 or GQA_INT8): K/V rows stored as FP8
 *     E4M3 or INT8 codes with one fp32 scale per cached row (token x KV
 *     head), written by gqa_kv_append, gqa_decode_step and the prefill calls
 *     and read by the decode and prefill calls (inference-optimisation page
 *     §15.5-§15.5.1: per-token / per-head scales, FP8 E4M3 or INT8).
 *     Queries, new K/V rows and outputs are then bf16.  Supported for
 *     head_dim 128; the decode calls need paged blocks of at least 16
 *     tokens.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GQA_ABI_VERSION 3

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1,   /* null pointer, non-positive size, H % K != 0, ... */
    GQA_ERR_UNSUPPORTED = 2,   /* valid but not built: head_dim, dtype, G > 64 */
    GQA_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    GQA_ERR_LAUNCH = 4,        /* a HIP call or kernel launch failed */
    GQA_ERR_DEVICE_ARG = 5     /* GQA_CHECK=1 only: a device-resident integer is out of range */
} gqa_status;

typedef enum {
    GQA_F32 = 0,               /* IEEE binary32 */
    GQA_BF16 = 1,              /* bfloat16 (upper half of a binary32), stored as 16-bit words */
    GQA_FP8_E4M3 = 2,          /* cache only: OCP FP8 E4M3 codes (bias 7, largest finite 448, no
                                * infinities) with one fp32 scale per row: value = scale * E4M3(code) */
    GQA_INT8 = 3               /* cache only: signed 8-bit codes in [-127, 127] with one fp32 scale
                                * per row: value = scale * code */
} gqa_dtype;

/* One layer's KV cache for K KV heads of width head_dim. */
typedef struct {
    void *k;                      /* contiguous: [B, K, S_max, d]; paged: [num_blocks, K, block_size, d] */
    void *v;                      /* same layout and size as k */
    const int32_t *block_table;   /* NULL: contiguous cache; else device [B, max_blocks_per_seq] */
    int32_t max_blocks_per_seq;   /* paged: columns of block_table */
    int32_t block_size;           /* paged: tokens per block (16 in the workloads here) */
    int32_t num_blocks;           /* paged: blocks in the pool */
    int32_t S_max;                /* contiguous: token capacity per sequence */
    int32_t num_kv_heads;         /* K */
    int32_t head_dim;             /* d */
    int32_t dtype;                /* gqa_dtype */
    float *k_scale;               /* GQA_FP8_E4M3 and GQA_INT8 only (else ignored): one scale per cached row,
                                     contiguous [B, K, S_max], paged [num_blocks, K, block_size] */
    float *v_scale;               /* the same for V */
} gqa_kv_cache;

/* ABI version of the loaded library (GQA_ABI_VERSION). */
int32_t gqa_abi_version(void);

/* Short English text for a status code (static storage). */
const char *gqa_status_string(int32_t status);

/*
 * Cache elements one token adds to one layer: a K row and a V row for each
 * KV head, 2 * K * d (concept page, 关键参数 #2).  Returns -1 if K or d is not
 * positive.  Host-only; no GPU needed.
 */
int32_t gqa_cache_elems_per_token(int32_t num_kv_heads, int32_t head_dim);

/*
 * FP8 cache: a row x of d bf16 values is stored as scale = amax(|x|) / 448
 * and codes E4M3(x_i / scale), nearest value with ties to the even code,
 * both divisions in IEEE fp32; an all-zero row has scale 0 and zero codes.
 * INT8 cache: scale = amax(|x|) / 127 and codes the integers nearest to
 * x_i * (1 / scale), ties to even, the reciprocal and the product in IEEE
 * fp32 (|code| <= 127); an all-zero row has scale 0 and zero codes.  Rows
 * are expected to hold finite values (a NaN element is stored as -127).
 *
 * Append s_new tokens to every sequence of the cache:
 *     pos = start_pos[b] + t,  cache row (b, g, pos) <- new row (b, t, g)
 * for t < s_new, g < K (through the block table when the cache is paged).
 * k_new, v_new: device [B, s_new, K, d] in the cache dtype.
 * start_pos: device int32 [B].  The copy is bit-exact.  Rows whose position is
 * past the capacity (S_max, or max_blocks_per_seq * block_size) or whose block
 * id is outside [0, num_blocks) are not written.
 */
gqa_status gqa_kv_append(const gqa_kv_cache *cache, const void *k_new, const void *v_new,
                         const int32_t *start_pos, int32_t B, int32_t s_new, void *stream);

/*
 * Workspace bytes gqa_decode needs for these sizes (a few MB at most; the
 * amount depends on G = H / K and d only, the other sizes are checked).
 * Host-only; no GPU needed.  Returns 0 on invalid sizes.
 * num_kv_heads is an argument beside num_heads because the partial results
 * are kept per KV group (G = H / K rows of d values per split): sized from H
 * alone, the workspace would have to assume the multi-query end (G = H).
 */
size_t gqa_decode_workspace_bytes(int32_t B, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_ctx);

/*
 * One decode step: each sequence's single query row attends to the first
 * ctx_lens[b] cached tokens (the newest token included: append it first).
 *   q:   device [B, 1, H, d];  out: device [B, 1, H, d]  (cache dtype)
 *   ctx_lens: device int32 [B], each in [1, max_ctx]
 *   max_ctx: host upper bound of ctx_lens, used to plan the key splits
 *   scale: the softmax scale, normally 1 / sqrt(d)
 * The (sequence, KV head, 64-key tile) work is split evenly over one
 * workgroup per compute unit (flash-decoding's split of the keys,
 * inference-optimisation page §10.2); every piece keeps an online-softmax
 * state (§9.2.1) and the pieces of one (sequence, KV head) are merged with
 * their global max and sum.  One K/V row read from memory serves all G heads
 * of its group.
 * workspace: device buffer of at least gqa_decode_workspace_bytes(...) bytes
 * (a tile table and two partial results per workgroup; it needs no
 * initialisation).  A (sequence, KV head) whose keys are shared by several
 * workgroups is merged by a second, small kernel on the same stream.  Calls
 * that may run concurrently need separate workspaces.
 */
gqa_status gqa_decode(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens,
                      int32_t max_ctx, int32_t B, int32_t num_heads, float scale, void *out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Prefill: write the new tokens' K/V into the cache (exactly the bytes
 * gqa_kv_append writes) and attend every new query row to the cache.
 *   q: device [B, s, H, d];  k_new, v_new: device [B, s, K, d];  out: device [B, s, H, d]
 *   start_pos: device int32 [B], the position of query row 0 (0 for a fresh
 *              prompt; > 0 continues a sequence whose earlier tokens are
 *              already cached)
 *   causal != 0: row i (position start_pos[b] + i) sees keys 0 .. start_pos[b] + i
 *   causal == 0: every row sees keys 0 .. start_pos[b] + s - 1
 * bf16 runs on the matrix cores (bf16 products, fp32 accumulation and
 * softmax statistics); fp32 runs on the vector ALUs in fp32 throughout.
 * An FP8 cache (chunked prefill over a quantised prefix, inference-
 * optimisation page §11.7 with §15.5.1): the new rows are quantised into the
 * cache as gqa_kv_append does it, and every row, old and new, is read as its
 * scale times its E4M3 value; queries and outputs are bf16.
 */
gqa_status gqa_prefill(const void *q, const void *k_new, const void *v_new,
                       const gqa_kv_cache *cache, const int32_t *start_pos, int32_t B, int32_t s,
                       int32_t num_heads, float scale, int32_t causal, void *out, void *stream);

/*
 * Sliding-window attention (the inference-optimisation page §6.4.1: a model
 * such as Mistral 7B keeps only the most recent N tokens, N = 4096, in its
 * attention window).  With window > 0, the query at position qpos sees only
 * the keys qpos - window + 1 .. qpos (those that exist and that the causal
 * rule or ctx_lens allow); window <= 0 is no window, the same call as
 * gqa_decode / gqa_prefill.  Keys outside the window are not read: whole
 * tiles below it are skipped and a 16-token cache block that lies wholly
 * below it is never touched, so its block-table entry may be stale.
 *   gqa_decode_window: the decode row's position is ctx_lens[b] - 1, so it
 *     sees keys max(0, ctx_lens[b] - window) .. ctx_lens[b] - 1.
 *   gqa_prefill_window: row i is at position start_pos[b] + i.
 * All other arguments, layouts, ownership and errors are those of
 * gqa_decode and gqa_prefill.
 */
gqa_status gqa_decode_window(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens,
                             int32_t max_ctx, int32_t B, int32_t num_heads, float scale, int32_t window,
                             void *out, void *workspace, size_t workspace_bytes, void *stream);
gqa_status gqa_prefill_window(const void *q, const void *k_new, const void *v_new,
                              const gqa_kv_cache *cache, const int32_t *start_pos, int32_t B, int32_t s,
                              int32_t num_heads, float scale, int32_t causal, int32_t window, void *out,
                              void *stream);

/*
 * One whole decode step: append the newest token's K/V and attend to the
 * cache including it.  The result and the cache bytes are exactly those of
 * gqa_kv_append(cache, k_new, v_new, start_pos = ctx_lens - 1, B, 1) followed
 * by gqa_decode_window(...) (the concept page, 技术原理: each new token's
 * K/V joins the cache, then its query attends to all cached keys).
 *   k_new, v_new: device [B, 1, K, d] (the cache dtype; bf16 for an FP8
 *                 cache), the token at position ctx_lens[b] - 1 of sequence b
 *   window: as for gqa_decode_window (<= 0: no window)
 * For a bf16 cache (d = 128, or d = 64 with G <= 8) one kernel does both: it
 * reads the new token from k_new / v_new and writes it into the cache in the
 * same launch; the other cases launch the append first.  A position at or past the cache capacity,
 * or whose block id is outside the pool, is not written (as in
 * gqa_kv_append).  All other arguments, layouts, ownership and errors are
 * those of gqa_decode; k_new and v_new must both be given
 * (GQA_ERR_INVALID_ARG otherwise).
 */
gqa_status gqa_decode_step(const void *q, const void *k_new, const void *v_new, const gqa_kv_cache *cache,
                           const int32_t *ctx_lens, int32_t max_ctx, int32_t B, int32_t num_heads, float scale,
                           int32_t window, void *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * gqa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  This call allocates nothing.
 * The decode's split partials go to a static buffer inside the library,
 * 12 MiB per GPU, held from the first use on that GPU until the process
 * ends.  The buffer is the current device's, so `stream` must belong to the
 * current device.
 *   - A call whose gqa_decode_workspace_bytes(B, H, K, d, max_ctx) exceeds
 *     12 MiB (G * d above 2048, e.g. G = 32 at d = 128) returns
 *     GQA_ERR_WORKSPACE and launches nothing.
 *   - Every call on one GPU shares that GPU's buffer.  Calls on one stream
 *     run in order and are safe.  Calls that may overlap on one GPU (several
 *     streams, or host threads with their own streams) race on it.
 *   - k_new and v_new are both given (the step) or both NULL (a plain
 *     decode, the newest token already appended).
 * Results, cache bytes, arguments and errors are otherwise exactly those of
 * gqa_decode_step.
 */
gqa_status gqa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new, const gqa_kv_cache *cache,
                                   const int32_t *ctx_lens, int32_t max_ctx, int32_t B, int32_t num_heads,
                                   float scale, int32_t window, void *out, void *stream);

/*
 * Decode of several new positions per sequence at once (a block of s
 * speculative tokens verified in one step, inference-optimisation page §14.2;
 * the concept page's rows are [B, s, H, d] for any s): row i of sequence b is
 * at position ctx_lens[b] - s + i and attends, causally, to the keys up to and
 * including its own position (from its position + 1 - window on when
 * window > 0).  The s tokens' K/V must already be in the cache (gqa_kv_append
 * at start_pos = ctx_lens - s), so ctx_lens[b] >= s.
 *   q, out: device [B, s, H, d];  ctx_lens: device int32 [B]
 *   workspace: at least gqa_decode_multi_workspace_bytes(B, H, K, d, s, max_ctx)
 * Each (sequence, KV head) item carries s * G query rows, so every K/V row
 * read from memory serves all of them; the products run on the matrix cores
 * (bf16 in, fp32 accumulate), the keys split over the workgroups as in
 * gqa_decode.  s == 1 is gqa_decode_window.  Supported for s > 1: bf16 or
 * FP8 cache, head_dim 128, s * G <= 64, paged blocks of at least 16 tokens
 * (GQA_ERR_UNSUPPORTED otherwise).  Other arguments, ownership and errors as
 * for gqa_decode.
 */
size_t gqa_decode_multi_workspace_bytes(int32_t B, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t s, int32_t max_ctx);
gqa_status gqa_decode_multi(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens, int32_t max_ctx,
                            int32_t B, int32_t s, int32_t num_heads, float scale, int32_t window, void *out,
                            void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
