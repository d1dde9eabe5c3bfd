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

hipError_t launch_kv_append(const AppendParams &p, hipStream_t stream)
{
    const int cpr = p.cache.d * p.cache.elem_bytes / 16;
    const int64_t total = 2LL * p.B * p.s_new * p.cache.K * cpr;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

}  // namespace gqa
