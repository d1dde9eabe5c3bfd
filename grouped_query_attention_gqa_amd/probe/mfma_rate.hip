// mfma_rate.hip -- a measurement aid beside the attention library (built into
// libgqa_probe.so, never linked into libgqa.so): the rate at which the device
// sustains v_mfma_f32_32x32x16_bf16 when its waves do nothing else.  The
// operands come from a caller's buffer, so they carry the values of a real
// workload: the matrix cores' power, and with it the clock they hold, depends
// on the data.  The prefill's roofline fraction is quoted against the
// published peak; this rate is what the same hardware delivers on the same
// operands with no softmax, LDS or memory traffic at all.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;   // independent accumulators per wave
constexpr int kUnroll = 4;   // matrix instructions per chain per iteration

template <int NT>
__global__ __launch_bounds__(NT) void mfma_rate_kernel(const uint4 *in, int64_t n16, float *sink, int iters)
{
    const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
    uint4 a[kChains], b[kChains];
    for (int i = 0; i < kChains; ++i) {
        a[i] = in[(gid * 2 * kChains + i) % n16];
        b[i] = in[(gid * 2 * kChains + kChains + i) % n16];
    }
    f32x16_t c[kChains];
    for (int i = 0; i < kChains; ++i)
        for (int j = 0; j < 16; ++j) c[i][j] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < kUnroll; ++r)
#pragma unroll
            for (int i = 0; i < kChains; ++i)
                c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[(i + r) % kChains]),
                                                               __builtin_bit_cast(bf16x8_t, b[i]), c[i], 0, 0, 0);
    }
    float s = 0.f;
    for (int i = 0; i < kChains; ++i)
        for (int j = 0; j < 16; ++j) s += c[i][j];
    sink[gid] = s;   // keeps the products live
}

}  // namespace

// One launch: one workgroup per compute unit, waves_per_simd (1 or 2) waves on
// each SIMD, each wave issuing iters * 16 matrix instructions.  operands: at
// least 16 bytes of bf16 values (read cyclically); sink: room for
// num_cus * 512 floats.  Returns 0, or a HIP error code.
extern "C" int gqa_probe_mfma_rate(const void *operands, size_t operand_bytes, float *sink, size_t sink_floats,
                                   int waves_per_simd, int iters, void *stream)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return (int)hipErrorInvalidDevice;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return (int)hipErrorInvalidDevice;
    if (!operands || operand_bytes < 16 || !sink || iters <= 0 || (waves_per_simd != 1 && waves_per_simd != 2))
        return (int)hipErrorInvalidValue;
    const int nt = 256 * waves_per_simd;
    if (sink_floats < (size_t)cus * (size_t)nt) return (int)hipErrorInvalidValue;
    const int64_t n16 = (int64_t)(operand_bytes / 16);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const uint4 *in = static_cast<const uint4 *>(operands);
    if (nt == 256) hipLaunchKernelGGL(mfma_rate_kernel<256>, dim3(cus), dim3(256), 0, s, in, n16, sink, iters);
    else hipLaunchKernelGGL(mfma_rate_kernel<512>, dim3(cus), dim3(512), 0, s, in, n16, sink, iters);
    return (int)hipGetLastError();
}

// Matrix instructions one call issues, for the caller's FLOP count
// (each is 32 x 32 x 16 multiply-adds, 32768 FLOP).
extern "C" int64_t gqa_probe_mfma_count(int waves_per_simd, int iters)
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return -1;
    return (int64_t)cus * 4 * waves_per_simd * (int64_t)iters * kChains * kUnroll;
}
