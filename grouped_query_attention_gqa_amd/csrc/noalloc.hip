// noalloc.hip -- gqa_decode_step_noalloc: the decode step with the library's
// own static workspace, for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// The split partials of the decode (the tile table of the launch and two
// partial results per workgroup) live in `scratch`, a fixed array in the
// library's device code.  Each GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the device symbol): the
// device address is looked up once per device with hipGetSymbolAddress and
// kept.  Nothing here allocates.
#include <mutex>

#include "kernels.h"

namespace gqa {
namespace {

// 12 MiB: the workspace of every decode with G * d <= 2048 (G <= 16 at
// d = 128, G <= 32 at d = 64); the call refuses larger ones.
constexpr size_t kScratchBytes = 12u << 20;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};   // device address of `scratch`, per device

// The workspace for one call on the current device: `need` bytes of the
// device's copy of `scratch`.  No kernel reads a workspace byte the same call
// has not written, so nothing is cleared between calls.
gqa_status static_workspace(size_t need, void **ws, size_t *ws_bytes)
{
    if (need > kScratchBytes) return GQA_ERR_WORKSPACE;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_LAUNCH;
    std::lock_guard<std::mutex> guard(g_lock);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return GQA_ERR_LAUNCH;
        g_scratch[dev] = ptr;
    }
    *ws = g_scratch[dev];
    *ws_bytes = kScratchBytes;
    return GQA_OK;
}

}  // namespace
}  // namespace gqa

extern "C" gqa_status gqa_decode_step_noalloc(const void *q, const void *k_new, const void *v_new,
                                              const gqa_kv_cache *cache, const int32_t *ctx_lens, int32_t max_ctx,
                                              int32_t B, int32_t num_heads, float scale, int32_t window, void *out,
                                              void *stream)
{
    return gqa::decode_step(q, k_new, v_new, cache, ctx_lens, max_ctx, B, num_heads, scale, window, out, nullptr, 0,
                            gqa::static_workspace, stream);
}
