// Device-side helpers shared by the liblinattn kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// bf16 storage is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even; NaNs stay NaN (quiet bit forced).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> __device__ __forceinline__ float load_as_f32(const T *p, size_t i);
template <> __device__ __forceinline__ float load_as_f32<float>(const float *p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
}

template <typename T> __device__ __forceinline__ void store_from_f32(T *p, size_t i, float v);
template <> __device__ __forceinline__ void store_from_f32<float>(float *p, size_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
}

// ELU+1 feature map ("Linear Attention", feature-map table): elu(x) + 1 with
// alpha = 1, which is x + 1 for x > 0 and exp(x) otherwise.  Accurate expf.
__device__ __forceinline__ float elu1_accurate(float x) { return x > 0.f ? x + 1.f : expf(x); }

// Power-of-two scale of an ELU+1 query row ("Story of Attention Part 5", 1a:
// the normaliser phi(q)^T z can drift toward zero): with qmax the row's
// largest coordinate, e = floor(qmax log2 e) when qmax <= 0, else 0, and the
// row's features are taken as phi(q) 2^-e.  The largest then lies in [1, 2),
// so the products with the keys' features stay normal fp32 numbers where
// exp(q_f) exp(k_f) would underflow; numerator and denominator scale alike and
// the output does not change.  Rows with a positive coordinate keep e = 0.
__device__ __forceinline__ float elu1_query_shift(float qmax) {
    return qmax > 0.f ? 0.f : floorf(qmax * 1.44269504088896341f);
}

// ELU+1 of x times 2^-e (e <= 0 from elu1_query_shift), accurate expf: the
// exact power-of-two product while exp(x) is a normal number, exp2 of the
// shifted exponent below that.
__device__ __forceinline__ float elu1_accurate_scaled(float x, float e) {
    if (x > 0.f) return x + 1.f;
    if (e == 0.f || x >= -87.f) return ldexpf(expf(x), static_cast<int>(-e));
    return exp2f(fmaf(x, 1.44269504088896341f, -e));
}

// Same map with the hardware exp2 (about 1 ulp); used where the result is
// rounded to bf16 right after.
__device__ __forceinline__ float elu1_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// x plus lane-permuted x (a DPP control word)
template <int CTRL>
__device__ __forceinline__ float add_dpp(float x) {
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 8 lanes of a group (lanes 8c .. 8c + 7), result in all 8:
// swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), then
// add the mirrored half (row_half_mirror: lane i of each 8 takes lane 7 - i).
__device__ __forceinline__ float group8_sum(float x) {
    x = add_dpp<0xB1>(x);
    x = add_dpp<0x4E>(x);
    return add_dpp<0x141>(x);
}

}  // namespace la
