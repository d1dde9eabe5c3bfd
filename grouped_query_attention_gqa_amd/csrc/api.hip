// api.hip -- the C ABI declared in include/gqa.h: argument checks, split
// planning and kernel dispatch.  Every check that needs no device runs before
// any HIP call, so invalid calls fail the same way on a machine without a GPU.
#include "../../include/gqa.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "kernels.h"

namespace gqa {

int32_t pow2_at_least(int32_t g)
{
    int32_t p = 1;
    while (p < g) p <<= 1;
    return p;
}

}  // namespace gqa

using namespace gqa;

namespace {

bool check_mode() { return std::getenv("GQA_CHECK") && std::atoi(std::getenv("GQA_CHECK")) != 0; }
bool debug_mode() { return std::getenv("GQA_DEBUG") && std::atoi(std::getenv("GQA_DEBUG")) != 0; }

gqa_status fail(gqa_status s, const char *what)
{
    if (debug_mode()) std::fprintf(stderr, "[gqa] %s: %s\n", gqa_status_string(s), what);
    return s;
}

// The softmax scale must be positive and finite: the kernels take each
// tile's maximum of the raw dot products and scale it afterwards, which
// commutes with the maximum only for a positive scale.
bool scale_ok(float scale) { return std::isfinite(scale) && scale > 0.f; }

// GQA_DECODE_WGS=n (1 .. kStreamWGs): the number of workgroups a decode
// launch splits its keys over, instead of the default for the kernel that
// runs.  The result is the same for every n up to the rounding of the
// merge; 0 (unset) is the default.
int32_t decode_wgs_override()
{
    const char *e = std::getenv("GQA_DECODE_WGS");
    if (!e) return 0;
    const int n = std::atoi(e);
    return n >= 1 && n <= kStreamWGs ? n : 0;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int32_t x)
{
    int r = 0;
    while ((1 << r) < x) ++r;
    return r;
}

// Validates a cache descriptor and fills the kernel view.
gqa_status make_view(const gqa_kv_cache *c, CacheView *out)
{
    if (!c) return fail(GQA_ERR_INVALID_ARG, "cache descriptor is NULL");
    if (!c->k || !c->v) return fail(GQA_ERR_INVALID_ARG, "cache k/v pointer is NULL");
    if (c->num_kv_heads <= 0) return fail(GQA_ERR_INVALID_ARG, "num_kv_heads <= 0");
    if (c->head_dim <= 0) return fail(GQA_ERR_INVALID_ARG, "head_dim <= 0");
    if (c->head_dim != 64 && c->head_dim != 128) return fail(GQA_ERR_UNSUPPORTED, "head_dim not 64 or 128");
    if (c->dtype != GQA_F32 && c->dtype != GQA_BF16 && c->dtype != GQA_FP8_E4M3 && c->dtype != GQA_INT8)
        return fail(GQA_ERR_UNSUPPORTED, "unknown dtype");
    const bool quant = c->dtype == GQA_FP8_E4M3 || c->dtype == GQA_INT8;
    if (quant) {
        if (!c->k_scale || !c->v_scale) return fail(GQA_ERR_INVALID_ARG, "quantised cache without scales");
        if (c->head_dim != 128) return fail(GQA_ERR_UNSUPPORTED, "quantised cache needs head_dim 128");
    }
    CacheView v{};
    v.k = static_cast<char *>(c->k);
    v.v = static_cast<char *>(c->v);
    v.block_table = c->block_table;
    v.K = c->num_kv_heads;
    v.d = c->head_dim;
    v.elem_bytes = quant ? 1 : c->dtype == GQA_BF16 ? 2 : 4;
    v.int8 = c->dtype == GQA_INT8 ? 1 : 0;
    v.k_scale = quant ? c->k_scale : nullptr;
    v.v_scale = quant ? c->v_scale : nullptr;
    if (c->block_table == nullptr) {
        if (c->S_max <= 0) return fail(GQA_ERR_INVALID_ARG, "S_max <= 0");
        v.S_max = c->S_max;
        v.capacity = c->S_max;
    } else {
        if (!is_pow2(c->block_size) || c->block_size > 1024)
            return fail(GQA_ERR_INVALID_ARG, "block_size not a power of two in [1, 1024]");
        if (c->max_blocks_per_seq <= 0) return fail(GQA_ERR_INVALID_ARG, "max_blocks_per_seq <= 0");
        if (c->num_blocks <= 0) return fail(GQA_ERR_INVALID_ARG, "num_blocks <= 0");
        const int64_t cap = (int64_t)c->max_blocks_per_seq * c->block_size;
        if (cap > 0x7fffffffLL) return fail(GQA_ERR_INVALID_ARG, "paged capacity exceeds 2^31-1 tokens");
        v.max_blocks = c->max_blocks_per_seq;
        v.log2_bs = ilog2(c->block_size);
        v.num_blocks = c->num_blocks;
        v.capacity = (int32_t)cap;
    }
    *out = v;
    return GQA_OK;
}

gqa_status check_heads(int32_t H, int32_t K)
{
    if (H <= 0) return fail(GQA_ERR_INVALID_ARG, "num_heads <= 0");
    if (H % K != 0) return fail(GQA_ERR_INVALID_ARG, "num_heads is not a multiple of num_kv_heads");
    if (H / K > 64) return fail(GQA_ERR_UNSUPPORTED, "group size H/K above 64");
    return GQA_OK;
}

gqa_status launch_status(hipError_t e, const char *what)
{
    if (e != hipSuccess) {
        if (debug_mode()) std::fprintf(stderr, "[gqa] %s: %s\n", what, hipGetErrorString(e));
        return GQA_ERR_LAUNCH;
    }
    return GQA_OK;
}

// GQA_CHECK=1: copy a device int32 array back (synchronising) for validation.
bool fetch_i32(const int32_t *dev, size_t n, std::vector<int32_t> &host)
{
    host.resize(n);
    if (n == 0) return true;
    return hipMemcpy(host.data(), dev, n * sizeof(int32_t), hipMemcpyDeviceToHost) == hipSuccess;
}

// Checks that every position in [lo[b], hi[b]) fits the cache, through the
// block table when paged.
gqa_status check_positions(const CacheView &v, const std::vector<int32_t> &lo,
                           const std::vector<int32_t> &hi)
{
    std::vector<int32_t> table;
    if (v.block_table) {
        if (!fetch_i32(v.block_table, (size_t)lo.size() * v.max_blocks, table))
            return fail(GQA_ERR_LAUNCH, "block table copy failed");
    }
    for (size_t b = 0; b < lo.size(); ++b) {
        if (lo[b] < 0 || hi[b] > v.capacity || hi[b] < lo[b])
            return fail(GQA_ERR_DEVICE_ARG, "position outside the cache capacity");
        if (!v.block_table) continue;
        const int bs = 1 << v.log2_bs;
        for (int64_t lb = lo[b] / bs; lb * bs < hi[b]; ++lb) {
            const int32_t blk = table[b * v.max_blocks + lb];
            if (blk < 0 || blk >= v.num_blocks) return fail(GQA_ERR_DEVICE_ARG, "block id out of range");
        }
    }
    return GQA_OK;
}

// Decode workspace: the launch's tile prefix (read by the merge kernel) and
// two partial-result slots per workgroup.
struct DecodeLayout {
    size_t prefix_bytes = 0, o_bytes = 0, ml_bytes = 0, total = 0;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void decode_layout(int32_t G, int32_t d, DecodeLayout *L)
{
    L->prefix_bytes = align256((size_t)(kStreamRows + 1) * sizeof(int32_t));
    L->o_bytes = align256((size_t)kStreamWGs * 2 * G * d * sizeof(float));
    L->ml_bytes = align256((size_t)kStreamWGs * 2 * G * 2 * sizeof(float));
    L->total = L->prefix_bytes + L->o_bytes + L->ml_bytes;
}

}  // namespace

extern "C" {

int32_t gqa_abi_version(void) { return GQA_ABI_VERSION; }

const char *gqa_status_string(int32_t s)
{
    switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
    case GQA_ERR_WORKSPACE: return "workspace missing or too small";
    case GQA_ERR_LAUNCH: return "HIP launch or runtime failure";
    case GQA_ERR_DEVICE_ARG: return "device-resident argument out of range";
    default: return "unknown status";
    }
}

int32_t gqa_cache_elems_per_token(int32_t num_kv_heads, int32_t head_dim)
{
    if (num_kv_heads <= 0 || head_dim <= 0) return -1;
    const int64_t n = 2LL * num_kv_heads * head_dim;
    return n > 0x7fffffffLL ? -1 : (int32_t)n;
}

size_t gqa_decode_workspace_bytes(int32_t B, int32_t num_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_ctx)
{
    if (B <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_ctx <= 0) return 0;
    if (num_heads % num_kv_heads != 0) return 0;
    DecodeLayout L;
    decode_layout(num_heads / num_kv_heads, head_dim, &L);
    return L.total;
}

gqa_status gqa_kv_append(const gqa_kv_cache *cache, const void *k_new, const void *v_new,
                         const int32_t *start_pos, int32_t B, int32_t s_new, void *stream)
{
    CacheView v;
    gqa_status st = make_view(cache, &v);
    if (st != GQA_OK) return st;
    if (B < 0 || s_new < 0) return fail(GQA_ERR_INVALID_ARG, "B or s_new negative");
    if (B == 0 || s_new == 0) return GQA_OK;
    if (!k_new || !v_new || !start_pos) return fail(GQA_ERR_INVALID_ARG, "NULL k_new/v_new/start_pos");
    if (check_mode()) {
        std::vector<int32_t> sp;
        if (!fetch_i32(start_pos, B, sp)) return fail(GQA_ERR_LAUNCH, "start_pos copy failed");
        std::vector<int32_t> hi(B);
        for (int b = 0; b < B; ++b) hi[b] = (int32_t)std::min<int64_t>((int64_t)sp[b] + s_new, 0x7fffffff);
        if ((st = check_positions(v, sp, hi)) != GQA_OK) return st;
    }
    AppendParams p{};
    p.cache = v;
    p.k_new = static_cast<const char *>(k_new);
    p.v_new = static_cast<const char *>(v_new);
    p.start_pos = start_pos;
    p.B = B;
    p.s_new = s_new;
    return launch_status(launch_kv_append(p, static_cast<hipStream_t>(stream)), "kv_append");
}

gqa_status gqa_decode(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens,
                      int32_t max_ctx, int32_t B, int32_t num_heads, float scale, void *out,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    return gqa_decode_window(q, cache, ctx_lens, max_ctx, B, num_heads, scale, 0, out, workspace, workspace_bytes,
                             stream);
}

gqa_status gqa_decode_window(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens,
                             int32_t max_ctx, int32_t B, int32_t num_heads, float scale, int32_t window,
                             void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    return gqa_decode_step(q, nullptr, nullptr, cache, ctx_lens, max_ctx, B, num_heads, scale, window, out,
                           workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_step(const void *q, const void *k_new, const void *v_new, const gqa_kv_cache *cache,
                           const int32_t *ctx_lens, int32_t max_ctx, int32_t B, int32_t num_heads, float scale,
                           int32_t window, void *out, void *workspace, size_t workspace_bytes, void *stream)
{
    return gqa::decode_step(q, k_new, v_new, cache, ctx_lens, max_ctx, B, num_heads, scale, window, out, workspace,
                            workspace_bytes, nullptr, stream);
}

}  // extern "C"

// The decode step behind gqa_decode_step and gqa_decode_step_noalloc: with
// `scratch` given, the workspace is the one it returns for the bytes this
// call needs (asked for only once every host-side check has passed).
gqa_status gqa::decode_step(const void *q, const void *k_new, const void *v_new, const gqa_kv_cache *cache,
                            const int32_t *ctx_lens, int32_t max_ctx, int32_t B, int32_t num_heads, float scale,
                            int32_t window, void *out, void *workspace, size_t workspace_bytes,
                            gqa_status (*scratch)(size_t need, void **ws, size_t *ws_bytes), void *stream)
{
    // k_new == v_new == nullptr: the plain decode (gqa_decode_window)
    const bool step = k_new != nullptr || v_new != nullptr;
    CacheView v;
    gqa_status st = make_view(cache, &v);
    if (st != GQA_OK) return st;
    if ((st = check_heads(num_heads, v.K)) != GQA_OK) return st;
    if (B < 0) return fail(GQA_ERR_INVALID_ARG, "B negative");
    if (B == 0) return GQA_OK;
    if (!q || !out || !ctx_lens) return fail(GQA_ERR_INVALID_ARG, "NULL q/out/ctx_lens");
    if (step && (!k_new || !v_new)) return fail(GQA_ERR_INVALID_ARG, "NULL k_new or v_new");
    if (v.elem_bytes == 1 && v.block_table && v.log2_bs < 4)
        return fail(GQA_ERR_UNSUPPORTED, "quantised cache with blocks below 16 tokens");
    if (max_ctx <= 0) return fail(GQA_ERR_INVALID_ARG, "max_ctx <= 0");
    if (!scale_ok(scale)) return fail(GQA_ERR_INVALID_ARG, "scale not a positive finite number");
    DecodeLayout L;
    decode_layout(num_heads / v.K, v.d, &L);
    if (scratch != nullptr && (st = scratch(L.total, &workspace, &workspace_bytes)) != GQA_OK)
        return fail(st, "the library's static workspace is too small for this call, or unavailable");
    if (!workspace || workspace_bytes < L.total)
        return fail(GQA_ERR_WORKSPACE, "workspace smaller than gqa_decode_workspace_bytes()");
    if (check_mode()) {
        std::vector<int32_t> cl;
        if (!fetch_i32(ctx_lens, B, cl)) return fail(GQA_ERR_LAUNCH, "ctx_lens copy failed");
        std::vector<int32_t> lo(B, 0);
        for (int b = 0; b < B; ++b) {
            if (cl[b] < 1 || cl[b] > max_ctx) return fail(GQA_ERR_DEVICE_ARG, "ctx_lens outside [1, max_ctx]");
            // keys below the window are never read: their blocks may be stale
            if (window > 0) lo[b] = std::max(0, cl[b] - window);
        }
        if ((st = check_positions(v, lo, cl)) != GQA_OK) return st;
    }
    RowAttnParams p{};
    p.cache = v;
    p.q = static_cast<const char *>(q);
    p.out = static_cast<char *>(out);
    p.ctx_lens = ctx_lens;
    char *ws = static_cast<char *>(workspace);
    p.prefix = reinterpret_cast<int32_t *>(ws);
    p.ws_o = reinterpret_cast<float *>(ws + L.prefix_bytes);
    p.ws_ml = reinterpret_cast<float *>(ws + L.prefix_bytes + L.o_bytes);
    p.total_rows = B;
    p.B = B;
    p.Sq = 1;
    p.H = num_heads;
    p.G = num_heads / v.K;
    p.prefill = 0;
    p.causal = 0;
    p.whole_items = 0;
    p.window = window > 0 ? window : 0;
    p.num_wgs = kStreamWGs;
    p.wgs_override = decode_wgs_override();
    p.scale_log2 = scale * 1.4426950408889634f;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    if (step) {
        // the fused kernel writes the new rows itself and reads them from
        // k_new / v_new; every other path appends first
        p.k_new = static_cast<const char *>(k_new);
        p.v_new = static_cast<const char *>(v_new);
        // the matrix-core decode writes the new bf16 rows itself; a quantised
        // (FP8 or INT8) cache is written by the quantising append kernel, and
        // so are the rest
        if (v.elem_bytes != 2 || !decode_mfma_supported(p)) {
            AppendParams ap{};
            ap.cache = v;
            ap.k_new = p.k_new;
            ap.v_new = p.v_new;
            ap.ctx_lens = ctx_lens;
            ap.B = B;
            ap.s_new = 1;
            if ((st = launch_status(launch_kv_append(ap, hs), "decode step append")) != GQA_OK) return st;
            p.k_new = p.v_new = nullptr;
        }
    }
    return launch_status(launch_row_attention(p, pow2_at_least(p.G), hs), "decode");
}

extern "C" {

size_t gqa_decode_multi_workspace_bytes(int32_t B, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                        int32_t s, int32_t max_ctx)
{
    if (B <= 0 || num_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_ctx <= 0 || s <= 0) return 0;
    if (num_heads % num_kv_heads != 0) return 0;
    const int64_t rows = (int64_t)s * (num_heads / num_kv_heads);
    if (rows > 0x7fffffffLL) return 0;
    DecodeLayout L;
    decode_layout((int32_t)rows, head_dim, &L);
    return L.total;
}

gqa_status gqa_decode_multi(const void *q, const gqa_kv_cache *cache, const int32_t *ctx_lens, int32_t max_ctx,
                            int32_t B, int32_t s, int32_t num_heads, float scale, int32_t window, void *out,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    if (s == 1)
        return gqa_decode_window(q, cache, ctx_lens, max_ctx, B, num_heads, scale, window, out, workspace,
                                 workspace_bytes, stream);
    CacheView v;
    gqa_status st = make_view(cache, &v);
    if (st != GQA_OK) return st;
    if ((st = check_heads(num_heads, v.K)) != GQA_OK) return st;
    if (B < 0 || s < 0) return fail(GQA_ERR_INVALID_ARG, "B or s negative");
    if (B == 0 || s == 0) return GQA_OK;
    if (!q || !out || !ctx_lens) return fail(GQA_ERR_INVALID_ARG, "NULL q/out/ctx_lens");
    if (max_ctx <= 0) return fail(GQA_ERR_INVALID_ARG, "max_ctx <= 0");
    if (!scale_ok(scale)) return fail(GQA_ERR_INVALID_ARG, "scale not a positive finite number");
    const int32_t G = num_heads / v.K;
    if ((int64_t)s * G > 64) return fail(GQA_ERR_UNSUPPORTED, "s * G above 64");
    if (v.elem_bytes == 4 || v.d != 128) return fail(GQA_ERR_UNSUPPORTED, "several positions need a bf16, FP8 or INT8 cache, d = 128");
    if (v.block_table && v.log2_bs < 4) return fail(GQA_ERR_UNSUPPORTED, "blocks below 16 tokens");
    DecodeLayout L;
    decode_layout(s * G, v.d, &L);
    if (!workspace || workspace_bytes < L.total)
        return fail(GQA_ERR_WORKSPACE, "workspace smaller than gqa_decode_multi_workspace_bytes()");
    if (check_mode()) {
        std::vector<int32_t> cl;
        if (!fetch_i32(ctx_lens, B, cl)) return fail(GQA_ERR_LAUNCH, "ctx_lens copy failed");
        std::vector<int32_t> lo(B, 0);
        for (int b = 0; b < B; ++b) {
            if (cl[b] < s || cl[b] > max_ctx) return fail(GQA_ERR_DEVICE_ARG, "ctx_lens outside [s, max_ctx]");
            // the oldest row sits at ctx - s; keys below its window are never read
            if (window > 0) lo[b] = (int32_t)std::max<int64_t>(0, (int64_t)cl[b] - s + 1 - window);
        }
        if ((st = check_positions(v, lo, cl)) != GQA_OK) return st;
    }
    RowAttnParams p{};
    p.cache = v;
    p.q = static_cast<const char *>(q);
    p.out = static_cast<char *>(out);
    p.ctx_lens = ctx_lens;
    char *ws = static_cast<char *>(workspace);
    p.prefix = reinterpret_cast<int32_t *>(ws);
    p.ws_o = reinterpret_cast<float *>(ws + L.prefix_bytes);
    p.ws_ml = reinterpret_cast<float *>(ws + L.prefix_bytes + L.o_bytes);
    p.total_rows = B;
    p.B = B;
    p.Sq = 1;
    p.mq = s;
    p.H = num_heads;
    p.G = G;
    p.window = window > 0 ? window : 0;
    p.num_wgs = kStreamWGs;
    p.wgs_override = decode_wgs_override();
    p.scale_log2 = scale * 1.4426950408889634f;
    return launch_status(launch_row_attention(p, pow2_at_least(p.G), static_cast<hipStream_t>(stream)),
                         "decode (several positions)");
}

gqa_status gqa_prefill(const void *q, const void *k_new, const void *v_new,
                       const gqa_kv_cache *cache, const int32_t *start_pos, int32_t B, int32_t s,
                       int32_t num_heads, float scale, int32_t causal, void *out, void *stream)
{
    return gqa_prefill_window(q, k_new, v_new, cache, start_pos, B, s, num_heads, scale, causal, 0, out, stream);
}

gqa_status gqa_prefill_window(const void *q, const void *k_new, const void *v_new,
                              const gqa_kv_cache *cache, const int32_t *start_pos, int32_t B, int32_t s,
                              int32_t num_heads, float scale, int32_t causal, int32_t window, void *out,
                              void *stream)
{
    CacheView v;
    gqa_status st = make_view(cache, &v);
    if (st != GQA_OK) return st;
    if ((st = check_heads(num_heads, v.K)) != GQA_OK) return st;
    if (B < 0 || s < 0) return fail(GQA_ERR_INVALID_ARG, "B or s negative");
    if (B == 0 || s == 0) return GQA_OK;
    if (!q || !k_new || !v_new || !start_pos || !out) return fail(GQA_ERR_INVALID_ARG, "NULL pointer");
    if (!scale_ok(scale)) return fail(GQA_ERR_INVALID_ARG, "scale not a positive finite number");
    const bool bf16 = v.elem_bytes == 2, fp8 = v.elem_bytes == 1;
    if (check_mode()) {
        std::vector<int32_t> sp;
        if (!fetch_i32(start_pos, B, sp)) return fail(GQA_ERR_LAUNCH, "start_pos copy failed");
        std::vector<int32_t> lo(B, 0), hi(B);
        for (int b = 0; b < B; ++b) {
            if (sp[b] < 0) return fail(GQA_ERR_DEVICE_ARG, "start_pos negative");
            hi[b] = (int32_t)std::min<int64_t>((int64_t)sp[b] + s, 0x7fffffff);
            // row 0 (position start_pos) is the oldest; keys below its window are never read
            if (window > 0) lo[b] = (int32_t)std::max<int64_t>(0, (int64_t)sp[b] + 1 - window);
        }
        if ((st = check_positions(v, lo, hi)) != GQA_OK) return st;
    }
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    AppendParams ap{};
    ap.cache = v;
    ap.k_new = static_cast<const char *>(k_new);
    ap.v_new = static_cast<const char *>(v_new);
    ap.start_pos = start_pos;
    ap.B = B;
    ap.s_new = s;
    if ((st = launch_status(launch_kv_append(ap, hs), "prefill append")) != GQA_OK) return st;

    const float scale_log2 = scale * 1.4426950408889634f;
    if (bf16 || fp8) {
        PrefillParams pp{};
        pp.cache = v;
        pp.q = static_cast<const char *>(q);
        pp.out = static_cast<char *>(out);
        pp.start_pos = start_pos;
        pp.B = B;
        pp.s = s;
        pp.H = num_heads;
        pp.G = num_heads / v.K;
        pp.causal = causal != 0;
        pp.window = window > 0 ? window : 0;
        pp.scale_log2 = scale_log2;
        return launch_status(fp8 ? launch_prefill_fp8(pp, hs) : launch_prefill_mfma(pp, hs), "prefill");
    }
    RowAttnParams p{};
    p.cache = v;
    p.q = static_cast<const char *>(q);
    p.out = static_cast<char *>(out);
    p.start_pos = start_pos;
    p.total_rows = (int64_t)B * s;
    p.B = B;
    p.Sq = s;
    p.H = num_heads;
    p.G = num_heads / v.K;
    p.prefill = 1;
    p.causal = causal != 0;
    p.whole_items = 1;   // no workspace here: every item stays in one workgroup
    p.window = window > 0 ? window : 0;
    p.num_wgs = kStreamWGs;
    p.scale_log2 = scale_log2;
    return launch_status(launch_row_attention(p, pow2_at_least(p.G), hs), "prefill (fp32)");
}

}  // extern "C"
