// kernels.h -- launch parameters shared by the C-ABI layer and the kernels
// (internal; the public interface is include/gqa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/gqa.h"

namespace gqa {

// Where the cache rows of one layer live.
struct CacheView {
    char *k;                    // base of the K cache / pool
    char *v;                    // base of the V cache / pool
    const int32_t *block_table; // nullptr: contiguous [B, K, S_max, d]
    int32_t max_blocks;         // paged: columns of block_table
    int32_t log2_bs;            // paged: log2(block_size)
    int32_t num_blocks;         // paged: rows of the pool
    int32_t S_max;              // contiguous capacity per sequence
    int32_t K;                  // KV heads
    int32_t d;                  // head dim
    int32_t elem_bytes;         // bytes of a stored element: 1 (FP8 E4M3 or INT8), 2 (bf16) or 4 (fp32)
    int32_t int8;               // 1: the 1-byte codes are INT8 (else E4M3)
    int32_t capacity;           // tokens a sequence can hold
    float *k_scale;             // FP8 / INT8 only: one scale per cached row, indexed like the rows
    float *v_scale;
};

struct AppendParams {
    CacheView cache;
    const char *k_new;          // [B, s_new, K, d]
    const char *v_new;
    const int32_t *start_pos;   // [B]
    const int32_t *ctx_lens;    // non-null: one token per sequence at position ctx_lens[b] - 1 (start_pos unused)
    int32_t B;
    int32_t s_new;
};

// Row-wise attention on the vector ALUs: decode (one query row per
// sequence, keys [0, ctx)) and the fp32 prefill (s rows per sequence).
constexpr int kStreamRows = 512;    // rows per launch (row tables in LDS)
constexpr int kStreamWGs = 512;     // workgroups per launch: two per MI355X CU

struct RowAttnParams {
    CacheView cache;
    const char *q;              // [B, Sq, H, d]
    char *out;                  // [B, Sq, H, d]
    const int32_t *ctx_lens;    // decode: [B] keys per sequence
    const int32_t *start_pos;   // prefill: [B] position of query row 0
    const char *k_new;          // decode step: [B, 1, K, d] newest token, at position ctx_lens[b] - 1 (or null)
    const char *v_new;
    int32_t *prefix;            // workspace: [kStreamRows + 1] tile prefix of the launch
    float *ws_o;                // workspace: [W, 2, G, d] partial outputs (unnormalised)
    float *ws_ml;               // workspace: [W, 2, G, 2] partial (max, sum), log2 units
    int64_t total_rows;         // B * Sq
    int64_t row0;               // first row of this launch
    int32_t rows;               // rows of this launch
    int32_t B;
    int32_t Sq;                 // query rows per sequence
    int32_t H;
    int32_t G;                  // H / K
    int32_t prefill;            // 0: decode rows; 1: prefill rows
    int32_t causal;
    int32_t whole_items;        // 1: slices snap to item starts (no partial pieces, no workspace)
    int32_t window;             // > 0: a row sees only its `window` most recent positions
    int32_t mq;                 // decode: query positions per sequence, the newest mq (0 or 1: one)
    int32_t num_wgs;            // W
    int32_t wgs_override;       // decode: > 0 fixes the workgroups of the launch (else the kernel's default)
    int32_t kv_split;           // decode: each KV head's G heads form kv_split items of G / kv_split heads (0, 1: one item)
    float scale_log2;           // softmax scale * log2(e)
};

// Causal / full prefill on the matrix cores (bf16).
struct PrefillParams {
    CacheView cache;
    const char *q;              // [B, s, H, d]
    char *out;                  // [B, s, H, d]
    const int32_t *start_pos;   // [B]
    int32_t B;
    int32_t s;
    int32_t H;
    int32_t G;
    int32_t causal;
    int32_t window;             // > 0: a row sees only its `window` most recent positions
    float scale_log2;
};

// Row index of cache entry (b, g, pos) in units of one head row, or -1 when
// the block id the table gives is outside the pool.
__device__ __forceinline__ int64_t cache_row(const CacheView &c, int b, int g, int pos)
{
    if (c.block_table == nullptr) return ((int64_t)b * c.K + g) * c.S_max + pos;
    const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + (pos >> c.log2_bs)];
    if (blk < 0 || blk >= c.num_blocks) return -1;
    return (((int64_t)blk * c.K + g) << c.log2_bs) + (pos & ((1 << c.log2_bs) - 1));
}

// Wave-uniform 32-bit load through the scalar data cache (s_load_dword).  It
// is counted by lgkmcnt, so waiting for it does not wait behind the wave's
// vector-memory loads in flight (a vector load of the same word would need
// vmcnt(0), which drains every load the wave has issued).
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t *p)
{
    // readfirstlane returns a signed int: go through uint32_t so that the
    // low half is zero-extended, not sign-extended, into the 64-bit address
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const uint64_t ua = ((uint64_t)hi << 32) | (uint64_t)lo;
    int32_t v;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ua) : "memory");
#pragma clang diagnostic pop
    return v;
}

// Four consecutive wave-uniform 32-bit values through the scalar data cache
// (s_load_dwordx4), one wait for all four.
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t scalar_load_i32x4(const int32_t *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
    const uint64_t ua = ((uint64_t)hi << 32) | (uint64_t)lo;
    i32x4_t v;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ua) : "memory");
#pragma clang diagnostic pop
    return v;
}

// The blocks of the four 16-key groups of a 64-key tile (keys j0, j0 + 16,
// j0 + 32 and j0 + 48, j0 a multiple of 64) of sequence b, with blocks of at
// least 16 tokens: one scalar load of the table entries from column
// j0 / block_size on.  Returns false (and sets nothing) when those four
// entries would pass the end of the sequence's table row.
__device__ __forceinline__ bool tile_block_ids(const CacheView &c, int b, int j0, int (&id)[4])
{
    const int col = __builtin_amdgcn_readfirstlane(j0) >> c.log2_bs;
    if (col < 0 || col + 4 > c.max_blocks) return false;
    const i32x4_t v = scalar_load_i32x4(c.block_table + (int64_t)b * c.max_blocks + col);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = ((j0 + 16 * q) >> c.log2_bs) - col;   // 0 .. 3
        id[q] = e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
    }
    return true;
}

// The same lookup for loads where all active lanes of a wave ask for
// positions inside one 16-aligned group of 16 tokens.  With blocks of 16 or
// more tokens that group lies in one block, so one wave-uniform scalar
// table read serves the whole wave.
__device__ __forceinline__ int64_t cache_row_wave(const CacheView &c, int b, int g, int pos)
{
    if (c.block_table == nullptr) return ((int64_t)b * c.K + g) * c.S_max + pos;
    if (c.log2_bs < 4) return cache_row(c, b, g, pos);
    // the column is checked so that the scalar load stays inside the table
    // even if it ran for a wave with no active lane
    const int col = __builtin_amdgcn_readfirstlane(pos) >> c.log2_bs;
    if (col < 0 || col >= c.max_blocks) return -1;
    const int32_t blk = scalar_load_i32(c.block_table + (int64_t)b * c.max_blocks + col);
    if (blk < 0 || blk >= c.num_blocks) return -1;
    return (((int64_t)blk * c.K + g) << c.log2_bs) + (pos & ((1 << c.log2_bs) - 1));
}

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream);
hipError_t launch_row_attention(const RowAttnParams &p, int gp, hipStream_t stream);
// decode on the matrix cores (bf16 at d = 128 and 64, FP8 at d = 128): mq query
// positions x G heads per (sequence, KV head), up to 64 rows
bool decode_mfma_supported(const RowAttnParams &p);
hipError_t launch_decode_mfma(const RowAttnParams &p, hipStream_t stream);
// merge of the partial pieces that W workgroup slices of tt-key tiles left in the workspace
hipError_t launch_merge_pieces(const RowAttnParams &p, int tt, int W, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillParams &p, hipStream_t stream);
// the same over an FP8 E4M3 cache with row scales (d = 128)
hipError_t launch_prefill_fp8(const PrefillParams &p, hipStream_t stream);

constexpr int kKeyTile = 64;   // prefill key tile

// gqa_decode_step's body.  scratch == nullptr: the caller's workspace;
// otherwise scratch(need, &ws, &bytes) supplies it once the host-side checks
// have passed (the static buffer of gqa_decode_step_noalloc).
gqa_status decode_step(const void *q, const void *k_new, const void *v_new, const gqa_kv_cache *cache,
                       const int32_t *ctx_lens, int32_t max_ctx, int32_t B, int32_t num_heads, float scale,
                       int32_t window, void *out, void *workspace, size_t workspace_bytes,
                       gqa_status (*scratch)(size_t need, void **ws, size_t *ws_bytes), void *stream);
int32_t pow2_at_least(int32_t g);

}  // namespace gqa
