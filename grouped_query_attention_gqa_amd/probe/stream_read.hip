// stream_read.hip -- a measurement aid beside the attention library (built
// into libgqa_probe.so, never linked into libgqa.so): the rate at which the
// device streams bytes from HBM into its compute units when the waves do
// nothing else.  The decode is bound by exactly this traffic; the bench quotes
// it beside the decode's roofline fraction, which stays against the
// published 8 TB/s.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kUnroll = 8;   // 16-byte loads in flight per thread
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Grid-stride over n16 16-byte words: each thread issues kUnroll independent
// loads per pass (NT: non-temporal, the policy of the decode's tile loads),
// then folds them into one word so that the loads stay live.
template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t *__restrict__ in, int64_t n16, uint32_t *sink)
{
    const int64_t stride = (int64_t)gridDim.x * 256 * kUnroll;
    uint32_t acc = 0;
    for (int64_t i = (int64_t)blockIdx.x * 256 * kUnroll + threadIdx.x; i < n16; i += stride) {
        u32x4_t v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t j = i + (int64_t)u * 256;
            v[u] = u32x4_t{0u, 0u, 0u, 0u};
            if (j < n16) v[u] = NT ? __builtin_nontemporal_load(in + j) : in[j];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// One launch reading the first `bytes` (a multiple of 16) of `buf` once, with
// `wgs` workgroups of 256 threads; sink: room for wgs * 256 words.
// nontemporal: 1 for non-temporal loads.  Returns 0, or a HIP error code.
extern "C" int gqa_probe_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, int wgs,
                                     int nontemporal, void *stream)
{
    if (!buf || bytes < 16 || bytes % 16 != 0 || !sink || wgs <= 0 || (size_t)wgs * 256 > sink_words)
        return (int)hipErrorInvalidValue;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4_t *in = static_cast<const u32x4_t *>(buf);
    const int64_t n16 = (int64_t)(bytes / 16);
    if (nontemporal) hipLaunchKernelGGL(stream_read_kernel<true>, dim3(wgs), dim3(256), 0, s, in, n16, sink);
    else hipLaunchKernelGGL(stream_read_kernel<false>, dim3(wgs), dim3(256), 0, s, in, n16, sink);
    return (int)hipGetLastError();
}
