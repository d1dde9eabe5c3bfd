// common.h -- device helpers shared by the libgqa kernels (not a public header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

constexpr int kWave = 64;   // CDNA wavefront width

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bf16 is the upper 16 bits of a binary32)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats to a bf16 pair (lo in the low half), round to nearest even, in
// one v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}

// Four INT8 codes (code i in byte i of w) -> four bf16 values, two per word,
// exactly: a code of magnitude <= 127 has at most 7 significant bits, so
// its fp32 value's upper half is its bf16 value.
__device__ __forceinline__ uint2 i8x4_bf16x4(uint32_t w)
{
    const uint32_t u = w ^ 0x80808080u;   // code + 128 in each byte, in [1, 255]
    const float f0 = (float)(u & 0xFFu) - 128.f, f1 = (float)((u >> 8) & 0xFFu) - 128.f;
    const float f2 = (float)((u >> 16) & 0xFFu) - 128.f, f3 = (float)(u >> 24) - 128.f;
    return make_uint2(__builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u),
                      __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u));
}

// Two bf16 products summed into an fp32 accumulator (v_dot2_f32_bf16).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (lo16(a), lo16(b)) and (hi16(a), hi16(b)): pair element e of two rows.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b)
{
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// All-reduce over aligned groups of `width` lanes (width a power of two <=
// 64); every lane of a group ends with the group's result.  Within a 16-lane
// row the steps are DPP lane permutations fused into the max/add (quad swaps,
// half-row mirror, row mirror: after each step the value is uniform over the
// lanes combined so far, so a mirror pairs complete sub-groups); the steps
// across rows use the permlane swaps above.
template <int ctrl>
__device__ __forceinline__ float dpp_f32(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), ctrl, 0xF, 0xF, false));
}
// Cross-row steps of a reduction without LDS traffic (a ds_bpermute would
// share the LDS counter with the loads a kernel keeps in flight).
// v_permlane32_swap (v_permlane16_swap) of a register with itself leaves each
// lane holding its own value and the value of the lane 32 (16) away; which
// of the two results is which depends on the lane, so they are combined with
// a symmetric operation.
__device__ __forceinline__ float2 swap_pair32(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float2 swap_pair16(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) { const float2 r = swap_pair32(x); return fmaxf(r.x, r.y); }
__device__ __forceinline__ float sum_xor32(float x) { const float2 r = swap_pair32(x); return r.x + r.y; }
// x + (x of the lane M away), for M = 16 or 32 through the swaps, else ds_bpermute
template <int M>
__device__ __forceinline__ float sum_xor(float x)
{
    if constexpr (M == 32) return sum_xor32(x);
    else if constexpr (M == 16) { const float2 r = swap_pair16(x); return r.x + r.y; }
    else return x + __shfl_xor(x, M, kWave);
}

template <int width, bool is_max>
__device__ __forceinline__ float group_reduce(float x)
{
    auto op = [](float a, float b) { return is_max ? fmaxf(a, b) : a + b; };
    if constexpr (width >= 2) x = op(x, dpp_f32<0xB1>(x));    // quad_perm [1,0,3,2]
    if constexpr (width >= 4) x = op(x, dpp_f32<0x4E>(x));    // quad_perm [2,3,0,1]
    if constexpr (width >= 8) x = op(x, dpp_f32<0x141>(x));   // row_half_mirror
    if constexpr (width >= 16) x = op(x, dpp_f32<0x140>(x));  // row_mirror
    if constexpr (width >= 32) { const float2 r = swap_pair16(x); x = op(r.x, r.y); }
    if constexpr (width >= 64) { const float2 r = swap_pair32(x); x = op(r.x, r.y); }
    return x;
}
template <int width>
__device__ __forceinline__ float group_max(float x) { return group_reduce<width, true>(x); }
template <int width>
__device__ __forceinline__ float group_sum(float x) { return group_reduce<width, false>(x); }

// 16-byte global load / store helpers.
__device__ __forceinline__ uint4 ld16(const void *p) { return *reinterpret_cast<const uint4 *>(p); }

// Pointers tagged as global memory.  A pointer picked between two objects
// (a cache row or a zero page) would otherwise be a generic one, and a
// generic (flat) load is also counted by the LDS counter: every wait for an
// LDS read would then wait for the HBM loads in flight as well.
typedef const __attribute__((address_space(1))) char gmem_t;
__device__ __forceinline__ gmem_t *gmem(const void *p) { return (gmem_t *)p; }
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 gld16(gmem_t *p)
{
    return __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4_t *)p);
}
__device__ __forceinline__ uint2 gld8(gmem_t *p)
{
    return __builtin_bit_cast(uint2, *(const __attribute__((address_space(1))) u32x2_t *)p);
}
// Non-temporal (streaming) loads, for cache rows a call reads once: their
// lines are the first the caches give up.
__device__ __forceinline__ uint4 ld16_nt(const void *p)
{
    return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p)));
}
__device__ __forceinline__ uint2 ld8_nt(const void *p)
{
    return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(p)));
}
__device__ __forceinline__ void st16(void *p, uint4 v) { *reinterpret_cast<uint4 *>(p) = v; }

}  // namespace gqa
