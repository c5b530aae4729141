// Matrix-core building blocks shared by the bf16 forward kernels
// (v_mfma_f32_16x16x32_bf16 operands, bf16 packing, the feature map on packed
// values, raw buffer resources, LDS transpose reads and barriers).
//
// For v_mfma_f32_16x16x32_bf16 lane l supplies A[l%16][k-slots 8(l/16)..+7],
// B[k-slots][l%16] and receives D[4(l/16)+e][l%16], e = 0..3.  Operands that
// contract over tokens use the k-slot order
//     slot 8g+e  <->  token 16*(e/4) + 4g + (e%4)   inside each 32-token block,
// the order in which a lane holds the scores of two consecutive 16x16 P^T
// accumulator tiles, so P becomes an A operand without an LDS round trip.
#pragma once

#include <type_traits>

#include "la_device.h"

namespace la {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

union Op8 {
    bf16x8_t v;
    uint4 u;
    uint2 q[2];
    uint32_t u32[4];
    uint16_t h[8];
};

__device__ __forceinline__ f32x4 mfma(const Op8 &a, const Op8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) { return make_uint2(cvt2(a, b), cvt2(c, d)); }

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// ELU+1 ("Linear Attention", feature-map table): x + 1 for x > 0, else exp(x)
// (hardware exp2, ~1 ulp).  Since 1 + x <= exp(x) <= 1 for x <= 0 and
// 1 < 1 + x < exp(x) for x > 0, the map is the median of {x + 1, exp(x), 1}:
// one v_med3_f32 in place of a compare and a select.
__device__ __forceinline__ float elu1_hw(float x) {
    const float e = __builtin_amdgcn_exp2f(x * 1.44269504088896341f);
    return __builtin_amdgcn_fmed3f(x + 1.f, e, 1.f);
}

// ELU+1 of eight packed bf16 values, rounded back to packed bf16
__device__ __forceinline__ uint4 elu1_bf16x8(uint4 x) {
    uint4 r;
    r.x = cvt2(elu1_hw(lo_bf16(x.x)), elu1_hw(hi_bf16(x.x)));
    r.y = cvt2(elu1_hw(lo_bf16(x.y)), elu1_hw(hi_bf16(x.y)));
    r.z = cvt2(elu1_hw(lo_bf16(x.z)), elu1_hw(hi_bf16(x.z)));
    r.w = cvt2(elu1_hw(lo_bf16(x.w)), elu1_hw(hi_bf16(x.w)));
    return r;
}

// Exponent of the power-of-two scale of an ELU+1 query row whose largest raw
// coordinate is qmax: e = floor(qmax log2 e) when qmax <= 0 (every feature is
// then exp(q_f) <= 1), else 0.  The row's features are taken as phi(q) 2^-e:
// the largest lands in [1, 2), so phi(q).phi(k) stays a normal fp32 number
// where exp(q_f) exp(k_f) alone would underflow ("Story of Attention Part 5",
// 1a, the normaliser phi(q)^T z drifting toward zero).  A power of two scales
// the row's numerator and denominator alike and leaves their ratio, the
// output, unchanged; for every row with a positive coordinate e = 0 and the
// features are bit for bit the plain ones.
__device__ __forceinline__ float elu1_row_shift(float qmax) {
    return qmax > 0.f ? 0.f : floorf(qmax * 1.44269504088896341f);
}

// ELU+1 of x scaled by 2^-e (e from elu1_row_shift of x's row), as a median
// like elu1_hw with cap = 1 when e = 0 and cap = +inf when e < 0: a row with
// e < 0 has every x <= 0, and its scaled exp(x) 2^-e >= exp(x) >= 1 + x, so
// the median {x + 1, exp(x) 2^-e, +inf} is the scaled exponential.
__device__ __forceinline__ float elu1_row_cap(float e) { return e == 0.f ? 1.f : __builtin_huge_valf(); }
__device__ __forceinline__ float elu1_hw_scaled(float x, float e, float cap) {
    const float v = __builtin_amdgcn_exp2f(x * 1.44269504088896341f - e);
    return __builtin_amdgcn_fmed3f(x + 1.f, v, cap);
}

__device__ __forceinline__ float max_bf16x8(uint4 x, float m) {
    m = fmaxf(m, fmaxf(lo_bf16(x.x), hi_bf16(x.x)));
    m = fmaxf(m, fmaxf(lo_bf16(x.y), hi_bf16(x.y)));
    m = fmaxf(m, fmaxf(lo_bf16(x.z), hi_bf16(x.z)));
    return fmaxf(m, fmaxf(lo_bf16(x.w), hi_bf16(x.w)));
}

// ELU+1 of a query row held as MFMA B-operand pieces (lane l: row l % 16,
// eight features per piece, pieces of the row spread over the lanes
// l % 16 + 16 g), with the row's power-of-two scale (elu1_row_shift).
// A row with a coordinate whose sign bit is clear has qmax >= 0 and scale
// exponent 0, so the exact maximum is taken only when some row of the wave
// has every sign bit set (a wave-uniform branch).
template <int NKB>
__device__ __forceinline__ void elu1_query_pieces(const uint4 (&raw)[NKB], uint4 (&out)[NKB]) {
    uint32_t all = ~0u;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) all &= raw[kb].x & raw[kb].y & raw[kb].z & raw[kb].w;
    int neg = (all & 0x80008000u) == 0x80008000u;
    neg &= __shfl_xor(neg, 16, 64);
    neg &= __shfl_xor(neg, 32, 64);
    float e = 0.f, cap = 1.f;
    if (__builtin_amdgcn_ballot_w64(neg) != 0) {
        float m = -__builtin_huge_valf();
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) m = max_bf16x8(raw[kb], m);
        m = fmaxf(m, __shfl_xor(m, 16, 64));
        m = fmaxf(m, __shfl_xor(m, 32, 64));
        e = elu1_row_shift(m);
        cap = elu1_row_cap(e);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
        const uint4 x = raw[kb];
        out[kb].x = cvt2(elu1_hw_scaled(lo_bf16(x.x), e, cap), elu1_hw_scaled(hi_bf16(x.x), e, cap));
        out[kb].y = cvt2(elu1_hw_scaled(lo_bf16(x.y), e, cap), elu1_hw_scaled(hi_bf16(x.y), e, cap));
        out[kb].z = cvt2(elu1_hw_scaled(lo_bf16(x.z), e, cap), elu1_hw_scaled(hi_bf16(x.z), e, cap));
        out[kb].w = cvt2(elu1_hw_scaled(lo_bf16(x.w), e, cap), elu1_hw_scaled(hi_bf16(x.w), e, cap));
    }
}

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor word 3).
// Loads past the range return zero and stores past it are dropped, without
// a memory access, so a partial or empty chunk runs the same unconditional
// instruction stream as a full one.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
}
// The same with the non-temporal cache policy (nt), for data a kernel touches
// exactly once (queries, outputs; the keys and values of a kernel that reads
// them once): it streams past the caches instead of displacing lines that
// are read again.
constexpr int kStream = 2;
__device__ __forceinline__ uint4 bload16_nt(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kStream));
}
__device__ __forceinline__ void bstore16_nt(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, kStream);
}

// Cache policy of the hand-off between workgroups of one launch (they may run
// on different XCDs, whose L2 caches are not coherent with each other): sc1,
// the policy of agent-scope atomics.  Stores write through to the device
// coherence point and loads read from it, so no L2-wide write-back or
// invalidate is needed around them.
constexpr int kCoherent = 16;
// Wait until this wave's stores have completed (reached the coherence point).
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// LDS transpose read: within each 16-lane group, lane i receives element i%4
// of the 8-byte fragments addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ uint2 tr_read(const uint16_t *p) {
    i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(p));
    return __builtin_bit_cast(uint2, v);
}

// Operand whose k-slots run over the 32 tokens of block kt (slot order above)
// and whose 16 rows/columns are the columns cb..cb+15 of a token-major LDS
// array with row stride R: lane i + 16g receives arr[token(g, s)][cb + i].
template <int R>
__device__ __forceinline__ Op8 token_operand(const uint16_t *arr, int kt, int cb, int lane) {
    const int g = lane >> 4, j = lane & 15;
    const uint16_t *p = arr + (32 * kt + 4 * g + (j >> 2)) * R + cb + 4 * (j & 3);
    Op8 o;
    o.q[0] = tr_read(p);
    o.q[1] = tr_read(p + 16 * R);
    return o;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global load and store of the wave (vmcnt(0)), which
// would drain the next chunk's prefetch at each barrier; the cross-wave
// hand-offs in these kernels go through LDS alone.
__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// f(std::integral_constant<int, v>) for a wave-uniform v in [0, N): code that
// depends on v (causal loop bounds, masks) becomes straight-line per value,
// so loads of later blocks can be issued early.  Values past N - 1 take N - 1.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void dispatch_const(int v, F &&f) {
    if constexpr (I + 1 < N) {
        if (v == I) f(std::integral_constant<int, I>{});
        else dispatch_const<N, I + 1>(v, f);
    } else {
        f(std::integral_constant<int, I>{});
    }
}

// MI355X: workgroups go round-robin over 8 XCDs
constexpr int kXcds = 8;

// Workgroup order.  Workgroup b is dispatched to XCD b % 8, so the segments
// of a slice are given workgroup numbers 8 apart: in every complete group of
// eight slices, b = 8P group + 8 seg + slice % 8; the slices past the last
// complete group share the remaining numbers the same way.  Within a slice
// the segment order is the workgroup order (a segment only waits for lower
// workgroups).
__device__ __forceinline__ void seg_of_block(int b, int BH, int P, int &bh, int &seg) {
    const int full = BH / kXcds, gsz = kXcds * P;
    if (b < full * gsz) {
        const int r = b % gsz;
        seg = r / kXcds;
        bh = (b / gsz) * kXcds + r % kXcds;
    } else {
        const int rest = BH % kXcds, r = b - full * gsz;
        seg = r / rest;
        bh = full * kXcds + r % rest;
    }
}

}  // namespace
}  // namespace la
