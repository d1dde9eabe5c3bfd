// kv_append.hip -- write new tokens' K/V rows into the cache.
//
// The cache write a new token makes ("Grouped-Query Attention" concept page,
// 技术原理: the token's K and V are [B, 1, K, d]); for a paged cache the
// position goes through the sequence's block table (inference-optimisation
// page §8.2).  Pure data movement: one thread moves one 16-byte piece, so the
// copy is bit-exact and both the reads (token-major) and the writes (one
// contiguous row per KV head) are coalesced.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace gqa {

// WIDE: 64-bit index arithmetic, for launches of 2^31 pieces or more; the
// usual launch uses 32-bit arithmetic (the divisions are most of the work a
// thread does besides its one load and store).
template <bool WIDE>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p)
{
    typedef typename std::conditional<WIDE, uint64_t, uint32_t>::type I;
    const CacheView &c = p.cache;
    const int row_bytes = c.d * c.elem_bytes;
    const int lcpr = __builtin_ctz((unsigned)row_bytes >> 4);   // 16-byte pieces per row: a power of two
    const I rows = (I)p.B * (I)p.s_new * (I)c.K;                 // rows per tensor
    const I idx = (I)blockIdx.x * (I)blockDim.x + (I)threadIdx.x;
    if (idx >= (rows << (lcpr + 1))) return;
    const int piece = (int)(idx & ((1u << lcpr) - 1));
    I r = idx >> lcpr;
    const int which = r >= rows;                          // 0: K, 1: V
    if (which) r -= rows;
    // rows in (sequence, KV head, position) order: the 64 lanes of a wave
    // write 4 consecutive positions of one head (1 KB of the cache) and read
    // them from 4 rows of k_new / v_new (measured 24.5 -> 23.3 us on a
    // 4 x 4096-token prefill against (sequence, position, head) order)
    const I bg = r / (I)p.s_new;                          // b * K + g
    const int t = (int)(r - bg * (I)p.s_new);
    const I b_ = bg / (I)c.K;
    const int g = (int)(bg - b_ * (I)c.K);
    const int b = (int)b_;
    const I bt = (I)b * (I)p.s_new + (I)t;                // b * s_new + t

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
    const char *src = (which ? p.v_new : p.k_new) + ((int64_t)bt * c.K + g) * row_bytes + piece * 16;
    char *dst = (which ? c.v : c.k) + dst_row * row_bytes + piece * 16;
    st16(dst, ld16(src));
}

// The quantising append of a 1-byte cache with one fp32 scale per row
// (inference-optimisation page §15.5.1): 16 lanes per 128-element row reduce
// its largest magnitude, then each lane stores its 8 codes.  I8: INT8 codes,
// scale = amax / 127 and code = nearest-even of x * (1 / scale); else E4M3,
// scale = amax / 448 and code = E4M3(x / scale).
constexpr int kF8Lanes = 16;   // lanes per 128-element row
template <bool I8>
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
    const float scale = amax / (I8 ? 127.0f : 448.0f);
    uint32_t lo = 0, hi = 0;
    if (I8) {
        if (amax > 0.f) {
            const float inv = 1.0f / scale;
            uint32_t b[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float n = fminf(fmaxf(__builtin_rintf(f[i] * inv), -127.f), 127.f);
                b[i] = (uint32_t)(int)n & 0xFFu;
            }
            lo = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
            hi = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        }
    } else if (amax > 0.f) {
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
        if (p.cache.int8)
            hipLaunchKernelGGL(kv_append_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
        else
            hipLaunchKernelGGL(kv_append_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    const int cpr = p.cache.d * p.cache.elem_bytes / 16;
    if (cpr <= 0 || (cpr & (cpr - 1)) != 0) return hipErrorInvalidValue;
    const int64_t total = 2LL * p.B * p.s_new * p.cache.K * cpr;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (blocks * 256 <= 0x7fffffffLL)
        hipLaunchKernelGGL(kv_append_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(kv_append_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gqa
