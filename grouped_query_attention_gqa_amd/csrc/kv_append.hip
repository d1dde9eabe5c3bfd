// kv_append.hip -- write new tokens' K/V rows into the cache.
//
// The cache write a new token makes ("Grouped-Query Attention" concept page,
// 技术原理: the token's K and V are [B, 1, K, d]); for a paged cache the
// position goes through the sequence's block table (inference-optimisation
// page §8.2).  Pure data movement: one thread moves one 16-byte piece, so the
// copy is bit-exact and both the reads (token-major) and the writes (one
// contiguous row per KV head) are coalesced.
#include "common.h"
#include "kernels.h"

namespace gqa {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p)
{
    const CacheView &c = p.cache;
    const int row_bytes = c.d * c.elem_bytes;
    const int cpr = row_bytes >> 4;                       // 16-byte pieces per row
    const int64_t per_tensor = (int64_t)p.B * p.s_new * c.K * cpr;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= 2 * per_tensor) return;
    const int which = idx >= per_tensor;                  // 0: K, 1: V
    int64_t r = which ? idx - per_tensor : idx;
    const int piece = (int)(r % cpr);
    r /= cpr;
    const int g = (int)(r % c.K);
    r /= c.K;
    const int t = (int)(r % p.s_new);
    const int b = (int)(r / p.s_new);

    const int64_t pos = p.ctx_lens != nullptr ? (int64_t)p.ctx_lens[b] - 1 : (int64_t)p.start_pos[b] + t;
    if (pos < 0 || pos >= c.capacity) return;
    int64_t dst_row;
    if (c.block_table == nullptr) {
        dst_row = ((int64_t)b * c.K + g) * c.S_max + pos;
    } else {
        const int32_t blk = c.block_table[(int64_t)b * c.max_blocks + (pos >> c.log2_bs)];
        if (blk < 0 || blk >= c.num_blocks) return;
        dst_row = (((int64_t)blk * c.K + g) << c.log2_bs) + (pos & ((1 << c.log2_bs) - 1));
    }
    const char *src = (which ? p.v_new : p.k_new) +
                      (((int64_t)b * p.s_new + t) * c.K + g) * row_bytes + piece * 16;
    char *dst = (which ? c.v : c.k) + dst_row * row_bytes + piece * 16;
    st16(dst, ld16(src));
}

// FP8 cache: thread (row, 8-element piece) quantises 8 bf16 values of a new
// row.  The row's largest magnitude comes from the 16 lanes that hold it
// (d = 128); scale = amax / 448 and code = E4M3(x / scale) with IEEE fp32
// divisions and the hardware's round-to-nearest-even conversion, so the
// codes are those of the format's definition (inference-optimisation page
// §15.5.1: a scale per token and head, FP8 E4M3).
constexpr int kF8Lanes = 16;   // lanes per 128-element row
__global__ __launch_bounds__(256) void kv_append_fp8_kernel(AppendParams p)
{
    const CacheView &c = p.cache;
    const int64_t rows = (int64_t)p.B * p.s_new * c.K;      // per tensor
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int piece = (int)(idx % kF8Lanes);
    int64_t r = idx / kF8Lanes;
    // every lane of a 16-lane group takes part in the reduction, so the
    // bounds check comes after it (the grid covers whole groups)
    const bool live = r < 2 * rows;
    const int which = live && r >= rows;                    // 0: K, 1: V
    if (which) r -= rows;
    const int g = (int)(r % c.K);
    const int t = (int)((r / c.K) % p.s_new);
    const int b = (int)(r / c.K / p.s_new);
    uint4 x = make_uint4(0u, 0u, 0u, 0u);
    if (live) x = ld16((which ? p.v_new : p.k_new) + (((int64_t)b * p.s_new + t) * c.K + g) * 256 + piece * 16);
    float f[8];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int o = 1; o < kF8Lanes; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, kF8Lanes));
    if (!live) return;
    const int64_t pos = p.ctx_lens != nullptr ? (int64_t)p.ctx_lens[b] - 1 : (int64_t)p.start_pos[b] + t;
    if (pos < 0 || pos >= c.capacity) return;
    const int64_t dst_row = cache_row(c, b, g, (int)pos);
    if (dst_row < 0) return;
    const float scale = amax / 448.0f;
    uint32_t lo = 0, hi = 0;
    if (amax > 0.f) {
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0] / scale, f[1] / scale, 0, false);
        lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[2] / scale, f[3] / scale, (int)lo, true);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[4] / scale, f[5] / scale, 0, false);
        hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[6] / scale, f[7] / scale, (int)hi, true);
    }
    *reinterpret_cast<uint2 *>((which ? c.v : c.k) + dst_row * 128 + piece * 8) = make_uint2(lo, hi);
    if (piece == 0) (which ? c.v_scale : c.k_scale)[dst_row] = scale;
}

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream)
{
    if (p.cache.elem_bytes == 1) {
        if (p.cache.d != 128) return hipErrorInvalidValue;
        const int64_t total = 2LL * p.B * p.s_new * p.cache.K * kF8Lanes;
        if (total == 0) return hipSuccess;
        const int64_t blocks = (total + 255) / 256;
        if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kv_append_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    const int cpr = p.cache.d * p.cache.elem_bytes / 16;
    const int64_t total = 2LL * p.B * p.s_new * p.cache.K * cpr;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gqa
