// Gated delta rule in chunkwise form ("Story of Attention Part 5", section 7
// Gated DeltaNet; "Linear Attention" (aiwiki.ai), the delta-rule update):
//     S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T,   o_t = S_t^T q_t,
// with S [d_k, d_v] feature-major, a_t the scalar forget gate (1 for the plain
// delta rule) and b_t the write strength.
//
// Chunk form (64-token chunks; t, s index the chunk's tokens from 0).  With
// the chunk's cumulative gates g_t = a_0 ... a_t, the state inside a chunk
// that starts from S0 is
//     S_t = g_t S0 + sum_{s <= t} (g_t / g_s) k_s u_s^T
// for write vectors u_s, because each step multiplies the earlier terms by
// a_t and adds k_t u_t^T with u_t = b_t (v_t - a_t S_{t-1}^T k_t).  Writing
// a_t S_{t-1}^T k_t through the same sum gives the unit lower-triangular
// system
//     u_t + b_t sum_{s < t} (g_t / g_s) (k_t . k_s) u_s = b_t v_t - b_t g_t S0^T k_t,
// i.e. (I + M) U = diag(b) V - diag(b g) K S0 with M[t][s] = b_t (g_t/g_s) k_t.k_s
// (s < t).  Its solution splits as U = Ut - W S0, where (I + M) W = diag(b g) K
// and (I + M) Ut = diag(b) V do not depend on S0 (the UT/WY form of the
// delta rule).  Then
//     O  = diag(g) Q S0 + P U,   P[t][s] = (g_t/g_s) q_t . k_s  (s <= t),
//     S_C = g_C S0 + K^T diag(g_C / g) U          (g_C: the chunk's last gate product).
// Every ratio g_t / g_s with s <= t is a product of gates in [0, 1], formed as
// exp2 of a difference of cumulative log2 gates (gates below 2^-80 count as 2^-80).
//
// Substituting U = Ut - W S0 leaves two operators and two S0-free terms per
// chunk:
//     O   = Qt S0 + P Ut,   Qt = diag(g) Q - P W,
//     S_C = A S0 + B,       A = g_C I - KG W,  B = KG Ut,  KG = K^T diag(g_C / g),
// so the step from chunk to chunk is one product (A S0) and the outputs one
// more, off that chain.
//
// Two launches:
//  * k_delta_prep, one workgroup per (slice, chunk), all chunks at once: the
//    Gram matrices K K^T and Q K^T on fp32 matrix instructions, M and P, W and
//    Ut by blocked forward substitution (16-row blocks: the update from the
//    solved blocks on matrix instructions, the diagonal block by substitution
//    with one right-hand column per thread), then P [W | Ut] and
//    KG [W | Ut] on matrix instructions: Qt, A, (P Ut)^T, B^T into the
//    workspace.
//  * k_delta_scan, one workgroup per (slice, 16 value columns), the chunks in
//    order: S <- A S + B and O = Qt S + P Ut, the state in fp32 accumulators.
// All arithmetic is fp32 (v_mfma_f32_16x16x4_f32: lane l supplies A[l%16][l/16]
// and B[l/16][l%16] of a 16x4 by 4x16 step and receives C[4(l/16)+e][l%16]).
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef float f32x4d __attribute__((ext_vector_type(4)));

constexpr int kXC = 64;        // tokens per chunk
constexpr int kXK = 64;        // d_k
constexpr int kXR = kXK + 4;   // row stride of 64-wide fp32 tiles
constexpr int kXT = 256;       // threads (4 waves)
constexpr float kMinLog2Gate = -80.f;

__device__ __forceinline__ f32x4d zero4d() { return f32x4d{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }  // bf16 bits

// bf16 matrix-instruction operands (v_mfma_f32_16x16x32_bf16: lane l supplies
// A[l%16][8(l/16)..+7] and B[8(l/16)..+7][l%16]) and the split of fp32 values
// into bf16 hi and lo parts, x = hi + lo to about 2^-17 relative
typedef __bf16 dbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 dbf16x2 __attribute__((ext_vector_type(2)));
typedef float df32x2 __attribute__((ext_vector_type(2)));
union D8 {
    dbf16x8 v;
    uint32_t u[4];
};
__device__ __forceinline__ uint32_t dbf2(float a, float b) {  // round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(df32x2{a, b}, dbf16x2));
}
__device__ __forceinline__ void dsplit8(const float (&x)[8], D8 &hi, D8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t h = dbf2(x[2 * e], x[2 * e + 1]);
        hi.u[e] = h;
        lo.u[e] = dbf2(x[2 * e] - __uint_as_float(h << 16), x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
    }
}
// a b in three bf16 passes (hi hi + hi lo + lo hi), accumulated in fp32
__device__ __forceinline__ f32x4d mma3(const D8 &ah, const D8 &al, const D8 &bh, const D8 &bl, f32x4d c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah.v, bh.v, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah.v, bl.v, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al.v, bh.v, c, 0, 0, 0);
}

__device__ __forceinline__ void sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// acc[16 rows at m0][16 columns at n0] += A B over K = 4 * KS.
// A(m, k) and B(k, n) are given as functors of LDS reads.
template <int KS, typename FA, typename FB>
__device__ __forceinline__ f32x4d mm4(FA a, FB b, f32x4d acc, int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < 4 * KS; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a(r, k0 + q), b(k0 + q, r), acc, 0, 0, 0);
    return acc;
}

// One output element through a buffer store: an offset past the resource's
// range drops the store in hardware, so partial tiles issue the same
// unconditional stores as full ones (a store under a branch would leave the
// compiler unable to count the stores in flight before the next wait).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, bytes, 0x00020000);  // raw buffer, gfx9 word 3
}
template <typename T>
__device__ __forceinline__ void store_elem(__amdgpu_buffer_rsrc_t r, int off, float v) {
    if constexpr (sizeof(T) == 2) __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
    else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}

// Per-chunk workspace record (floats): Qt [64 tokens][64], A [64][64]
// (P [64][64] while the record is built), (P Ut)^T [dv][64 tokens], B^T [dv][64].
__host__ __device__ inline size_t delta_rec_floats(int dv) { return 2 * kXC * kXK + 2 * (size_t)kXC * dv; }

// DVM: the largest d_v the instance takes (64 or 128); the right-hand sides
// are sized for it, so at d_v <= 64 the workgroup needs 69 KB of LDS and two
// of them share a CU.
template <typename T, int DVM>
__global__ __launch_bounds__(kXT) void k_delta_prep(const T *__restrict__ Q, const T *__restrict__ K,
                                                    const T *__restrict__ V, const float *__restrict__ alpha,
                                                    const float *__restrict__ beta, int N, int dv, int n_chunks,
                                                    float *__restrict__ ws) {
    constexpr int RX = kXK + DVM + 4;  // row stride of the right-hand sides / solution [64][64 + d_v]
    // sQ is only read by the Gram tiles; the right-hand sides reuse its space afterwards
    __shared__ float sK[kXC * kXR], sM[kXC * kXR];
    __shared__ float sQX[kXC * RX];
    float *const sQ = sQX, *const sX = sQX;
    __shared__ float sl[kXC], sb[kXC];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int bh = blockIdx.x / n_chunks, c = blockIdx.x % n_chunks;
    const int t0 = c * kXC, L = min(kXC, N - t0);
    const int ncol = kXK + dv;
    const size_t tok0 = (size_t)bh * N + t0;

    // chunk rows in 16-byte pieces, all in flight at once (rows past the end: zero)
    constexpr int EP = 16 / (int)sizeof(T);                    // elements per piece
    constexpr int QP = kXC * kXK / EP / kXT;                   // pieces of Q (and of K) per thread
    constexpr int VP = kXC * DVM / EP / kXT;                   // pieces of V per thread, at most
    const char *qb = reinterpret_cast<const char *>(Q + tok0 * kXK);
    const char *kb = reinterpret_cast<const char *>(K + tok0 * kXK);
    const char *vb = reinterpret_cast<const char *>(V + tok0 * dv);
    const int qk_bytes = L * kXK * (int)sizeof(T), v_bytes = L * dv * (int)sizeof(T);
    uint4 xq[QP], xk[QP], xv[VP];
    // unconditional loads from clamped offsets (a load under a branch would
    // wait for every outstanding load); pieces past the end become zero on use
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int off = 16 * (tid + i * kXT);
        xq[i] = *reinterpret_cast<const uint4 *>(qb + (off < qk_bytes ? off : 0));
        xk[i] = *reinterpret_cast<const uint4 *>(kb + (off < qk_bytes ? off : 0));
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
        const int off = 16 * (tid + i * kXT);
        xv[i] = *reinterpret_cast<const uint4 *>(vb + (off < v_bytes ? off : 0));
    }
    const uint4 zero = make_uint4(0, 0, 0, 0);
    // piece -> fp32 values at element e0 of a row-major [rows][width] block
    auto unpack = [&](const uint4 &x, float (&o)[EP]) {
        if constexpr (sizeof(T) == 2) {
            const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                o[2 * e] = __uint_as_float(xs[e] << 16);
                o[2 * e + 1] = __uint_as_float(xs[e] & 0xffff0000u);
            }
        } else {
            o[0] = __uint_as_float(x.x); o[1] = __uint_as_float(x.y);
            o[2] = __uint_as_float(x.z); o[3] = __uint_as_float(x.w);
        }
    };

    // gates: cumulative log2 products (one wave, inclusive scan); tokens past
    // the end have gate 1 and strength 0, so they change nothing
    if (w == 0) {
        const float a = lane < L ? (alpha ? alpha[tok0 + lane] : 1.f) : 1.f;
        float l = fmaxf(__builtin_amdgcn_logf(a), kMinLog2Gate);  // log2
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float o = __shfl_up(l, d, 64);
            if (lane >= d) l += o;
        }
        sl[lane] = l;
        sb[lane] = lane < L ? beta[tok0 + lane] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < QP; ++i) {
        const int e0 = EP * (tid + i * kXT), t = e0 / kXK, f = e0 % kXK;
        float o[EP];
        const bool live = 16 * (tid + i * kXT) < qk_bytes;
        unpack(live ? xq[i] : zero, o);
#pragma unroll
        for (int e = 0; e < EP; ++e) sQ[t * kXR + f + e] = o[e];
        unpack(live ? xk[i] : zero, o);
#pragma unroll
        for (int e = 0; e < EP; ++e) sK[t * kXR + f + e] = o[e];
    }
    __syncthreads();

    float *rec = ws + ((size_t)bh * n_chunks + c) * delta_rec_floats(dv);
    float *Qt = rec, *Am = rec + kXC * kXK, *PUT = rec + 2 * kXC * kXK, *BT = PUT + (size_t)kXC * dv;
    float *const P = Am;  // P until the operator A replaces it

    // Gram tiles: K K^T of row block w (strictly lower part -> M) and Q K^T
    // of row block 3 - w (lower part with the diagonal -> P), five tiles per
    // wave; tiles above the diagonal are zero.  bf16 storage: q and k are exact
    // in bf16, so each tile is two bf16 matrix instructions (k-slot 8g + j of
    // step kk = feature 32kk + 8g + j) with no rounding of the operands.
    auto gram = [&](const float *X, int rb, int cb) {
        f32x4d acc = zero4d();
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float *xa = &X[(16 * rb + c16) * kXR + 32 * kk + 8 * g];
                const float *xb = &sK[(16 * cb + c16) * kXR + 32 * kk + 8 * g];
                D8 a8, b8;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a8.u[e] = dbf2(xa[2 * e], xa[2 * e + 1]);
                    b8.u[e] = dbf2(xb[2 * e], xb[2 * e + 1]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8.v, b8.v, acc, 0, 0, 0);
            }
        } else {
            auto bk = [&](int k, int n) { return sK[(16 * cb + n) * kXR + k]; };
            acc = mm4<16>([&](int m, int k) { return X[(16 * rb + m) * kXR + k]; }, bk, acc, lane);
        }
        return acc;
    };
    const int rk = w, rq = 3 - w;
    for (int cb = 0; cb < 4; ++cb) {
        const f32x4d gk = cb <= rk ? gram(sK, rk, cb) : zero4d();
        const f32x4d gq = cb <= rq ? gram(sQ, rq, cb) : zero4d();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int s = 16 * cb + c16;
            const int t = 16 * rk + 4 * g + e;
            const float rat_k = s < t ? __builtin_amdgcn_exp2f(sl[t] - sl[s]) : 0.f;
            sM[t * kXR + s] = s < t ? sb[t] * rat_k * gk[e] : 0.f;
            const int t2 = 16 * rq + 4 * g + e;
            const float rat_q = s <= t2 ? __builtin_amdgcn_exp2f(sl[t2] - sl[s]) : 0.f;
            P[t2 * kXK + s] = rat_q * gq[e];
        }
    }
    __syncthreads();  // every read of sQ done: its space takes the right-hand sides
    // R = [diag(b g) K | diag(b) V]
    for (int u = tid; u < kXC * kXK; u += kXT) {
        const int t = u / kXK, j = u % kXK;
        sX[t * RX + j] = sb[t] * __builtin_amdgcn_exp2f(sl[t]) * sK[t * kXR + j];
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
        const int e0 = EP * (tid + i * kXT);
        if (e0 < kXC * dv) {
            const int t = e0 / dv, j = e0 % dv;
            float o[EP];
            unpack(16 * (tid + i * kXT) < v_bytes ? xv[i] : zero, o);
#pragma unroll
            for (int e = 0; e < EP; ++e) sX[t * RX + kXK + j + e] = sb[t] * o[e];
        }
    }
    __syncthreads();

    // (I + M) X = R by 16-row blocks, in place in sX: block b's right-hand
    // sides lose M[b][0..b) X[0..b) (matrix instructions, 16-column tiles
    // split over the waves), then the 16x16 diagonal block is solved by
    // substitution, one column per thread with its 16 values in registers.
    const int ntile = ncol / 16;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        if (b > 0) {
            for (int n = w; n < ntile; n += 4) {
                f32x4d acc = zero4d();
                const int r = lane & 15, q = lane >> 4;
                for (int k0 = 0; k0 < 16 * b; k0 += 4)
                    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sM[(16 * b + r) * kXR + k0 + q],
                                                                sX[(k0 + q) * RX + 16 * n + r], acc, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 4; ++e) sX[(16 * b + 4 * g + e) * RX + 16 * n + c16] -= acc[e];
            }
            __syncthreads();
        }
        if (tid < ncol) {
            const int j = tid;
            float x[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int t = 16 * b + r;
                float v = sX[t * RX + j];
#pragma unroll
                for (int r2 = 0; r2 < r; ++r2) v -= sM[t * kXR + 16 * b + r2] * x[r2];
                x[r] = v;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sX[(16 * b + r) * RX + j] = x[r];
        }
        __syncthreads();
    }

    // Tiles of the two operator products over X = [W | Ut] (16-column block n:
    // n < 4 the W part, else value columns 16 (n - 4)..), split over the waves.
    // Qt = diag(g) Q - P W and (P Ut)^T: P is lower triangular, so row block m
    // takes key blocks 0..m (k-slot q of step (kb, j) = token 16kb + 4q + j: a
    // lane reads four consecutive entries of its P row).
    const int r = c16, q = g;
    const int nxt = ncol / 16;  // column blocks of X
    const T *Qg = Q + tok0 * kXK;
    // wave w takes column blocks w, w + 4, .. in pairs (two independent
    // accumulation chains sharing the P row operand; a pair's second block
    // past the last is computed on the last block and not stored).  The P row
    // pieces (token 16kb + 4q..+3 of row 16m + r) and the queries of the
    // wave's Qt column block w are loaded before the products, all at once.
    float4 prow[4][4];
    T qv[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
            prow[m][kb] = *reinterpret_cast<const float4 *>(&P[(16 * m + r) * kXK + 16 * kb + 4 * q]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // clamped rows, zero past the end at use
            const int t = 16 * m + 4 * g + e;
            qv[m][e] = Qg[(t < L ? t : 0) * kXK + 16 * w + c16];
        }
    }
    auto store_p = [&](int m, int n, const f32x4d &acc, const T (&qm)[4]) {
        if (n < 4) {  // n == w: the wave's own query column block
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * m + 4 * g + e;
                const float qf = t < L ? to_f32(qm[e]) : 0.f;
                Qt[t * kXK + 16 * n + c16] = __builtin_amdgcn_exp2f(sl[t]) * qf - acc[e];
            }
        } else {
            *reinterpret_cast<float4 *>(&PUT[(size_t)(16 * (n - 4) + c16) * kXC + 16 * m + 4 * g]) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };
    // bf16 storage: both products in three bf16 passes (k-slot 8q + j of key
    // pair hp = token 16(2hp + j/4) + 4q + j%4 for P X, 32h + 4j + q for KG X);
    // fp32 storage keeps fp32 operands, its results being held to fp32 accuracy
    constexpr bool BF = sizeof(T) == 2;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (BF) {
            D8 ah[2], al[2];
#pragma unroll
            for (int hp = 0; 2 * hp <= m; ++hp) {
                const float pa[8] = {prow[m][2 * hp].x,     prow[m][2 * hp].y,     prow[m][2 * hp].z,
                                     prow[m][2 * hp].w,     prow[m][2 * hp + 1].x, prow[m][2 * hp + 1].y,
                                     prow[m][2 * hp + 1].z, prow[m][2 * hp + 1].w};
                dsplit8(pa, ah[hp], al[hp]);
            }
            for (int n = w; n < nxt; n += 4) {
                f32x4d acc = zero4d();
#pragma unroll
                for (int hp = 0; 2 * hp <= m; ++hp) {
                    float xv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) xv[j] = sX[(16 * (2 * hp + j / 4) + 4 * q + j % 4) * RX + 16 * n + c16];
                    D8 xh, xl;
                    dsplit8(xv, xh, xl);
                    acc = mma3(ah[hp], al[hp], xh, xl, acc);
                }
                store_p(m, n, acc, qv[m]);
            }
        } else {
            for (int n0 = w; n0 < nxt; n0 += 8) {
                const int n1 = n0 + 4, n1c = min(n1, nxt - 1);
                f32x4d acc0 = zero4d(), acc1 = zero4d();
#pragma unroll
                for (int kb = 0; kb <= m; ++kb) {
                    const float pav[4] = {prow[m][kb].x, prow[m][kb].y, prow[m][kb].z, prow[m][kb].w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float *xr = &sX[(16 * kb + 4 * q + j) * RX + c16];
                        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(pav[j], xr[16 * n0], acc0, 0, 0, 0);
                        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(pav[j], xr[16 * n1c], acc1, 0, 0, 0);
                    }
                }
                store_p(m, n0, acc0, qv[m]);
                if (n1 < nxt) store_p(m, n1, acc1, qv[m]);
            }
        }
    }
    __syncthreads();  // every read of P done before A takes its place
    // A = g_C I - KG W and B^T = (KG Ut)^T, KG[f][t] = k_t,f g_C / g_t over all tokens
    const float lC = sl[kXC - 1], gC = __builtin_amdgcn_exp2f(lC);
    float gk[16];  // g_C / g_t for this lane's tokens t = 4i + q
#pragma unroll
    for (int i = 0; i < 16; ++i) gk[i] = __builtin_amdgcn_exp2f(lC - sl[4 * i + q]);
    auto store_a = [&](int m, int n, const f32x4d &acc) {
        if (n < 4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 16 * m + 4 * g + e, f2 = 16 * n + c16;
                Am[f * kXK + f2] = (f == f2 ? gC : 0.f) - acc[e];
            }
        } else {
            *reinterpret_cast<float4 *>(&BT[(size_t)(16 * (n - 4) + c16) * kXK + 16 * m + 4 * g]) =
                make_float4(acc[0], acc[1], acc[2], acc[3]);
        }
    };
    for (int m = 0; m < 4; ++m) {
        float ka[16];  // KG[16m + r][t], t = 4i + q
#pragma unroll
        for (int i = 0; i < 16; ++i) ka[i] = sK[(4 * i + q) * kXR + 16 * m + r] * gk[i];
        if constexpr (BF) {
            D8 ah[2], al[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float a8[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) a8[j] = ka[8 * h + j];
                dsplit8(a8, ah[h], al[h]);
            }
            for (int n = w; n < nxt; n += 4) {
                f32x4d acc = zero4d();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    float xv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) xv[j] = sX[(4 * (8 * h + j) + q) * RX + 16 * n + c16];
                    D8 xh, xl;
                    dsplit8(xv, xh, xl);
                    acc = mma3(ah[h], al[h], xh, xl, acc);
                }
                store_a(m, n, acc);
            }
            continue;
        }
        for (int n0 = w; n0 < nxt; n0 += 8) {
            const int n1 = n0 + 4, n1c = min(n1, nxt - 1);
            f32x4d acc0 = zero4d(), acc1 = zero4d();
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float *xr = &sX[(4 * i + q) * RX + c16];
                acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[i], xr[16 * n0], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[i], xr[16 * n1c], acc1, 0, 0, 0);
            }
            store_a(m, n0, acc0);
            if (n1 < nxt) store_a(m, n1, acc1);
        }
    }
}

// The state chain: one workgroup per (slice, 16 value columns), the chunks
// in order.  Wave w owns feature rows 16w..16w+15 of the state (fp32
// accumulators).  Per chunk: the state entering it, S_c, is written over the
// chunk's B^T in the record (same lane, same address, after that lane's read
// of it), then S <- A S + B with the state image as the B operand (k-slot q
// of step j = feature 16q + j, so a lane's A row is a contiguous 16-float run
// read straight from the record into registers four chunks ahead) and B as
// the accumulators' starting value.  The state image alternates between two
// LDS buffers, so one barrier per chunk orders its writes and reads.
__global__ __launch_bounds__(kXT) void k_delta_scan(float *__restrict__ ws, const float *__restrict__ S_in,
                                                    float *__restrict__ S_out, int dv, int n_chunks) {
    __shared__ __align__(16) float sS[2][16 * kXR];  // [value column][feature], transposed
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;
    const int ncb = dv / 16;
    // slice fastest: the column blocks of a slice are B*H workgroups apart, so
    // (B*H a multiple of 8) they run on one XCD and share its L2 copy of the
    // slice's chunk records
    const int BH = gridDim.x / ncb;
    const int bh = blockIdx.x % BH, cb = blockIdx.x / BH;
    const int col0 = 16 * cb;
    const int r = c16, q = g;  // A-operand row and k group of this lane

    // state rows 16w + 4g + e, column col0 + c16
    f32x4d S = zero4d();
    if (S_in) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[e] = S_in[((size_t)bh * kXK + 16 * w + 4 * g + e) * dv + col0 + c16];
    }
    struct Pre {
        float4 a[4], bt;
    };
    const size_t bt_off = 2 * kXC * kXK + (size_t)kXC * dv + (size_t)(col0 + c16) * kXK + 16 * w + 4 * g;
    auto fetch = [&](Pre &f, int c_) {
        const int c = min(c_, n_chunks - 1);  // past the end: a harmless re-read of the last chunk
        const float *rec = ws + ((size_t)bh * n_chunks + c) * delta_rec_floats(dv);
        const float *Ar = rec + kXC * kXK + (16 * w + r) * kXK + 16 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const float4 *>(Ar + 4 * i);
        f.bt = *reinterpret_cast<const float4 *>(rec + bt_off);
    };
    // the records of the next kDepth chunks in flight: chunk c sits in ring
    // slot c % kDepth (the loop runs in groups of kDepth, so every step's slot
    // is a compile-time choice) and is refilled with chunk c + kDepth
    constexpr int kDepth = 4;
    Pre pre[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) fetch(pre[d], d);

    auto step = [&](Pre &p, int c) {
        float *img = sS[c & 1];
        *reinterpret_cast<float4 *>(&img[c16 * kXR + 16 * w + 4 * g]) = make_float4(S[0], S[1], S[2], S[3]);
        float aa[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            aa[4 * i] = p.a[i].x; aa[4 * i + 1] = p.a[i].y; aa[4 * i + 2] = p.a[i].z; aa[4 * i + 3] = p.a[i].w;
        }
        // B joins after the products: as the accumulators' starting value its
        // prefetch would be loaded into accumulator registers, whose moves wait
        // for every load in flight
        const float4 bt = p.bt;
        f32x4d s0 = zero4d(), s1 = zero4d();
        // S_c over this lane's own B^T entries (read above, into bt)
        *reinterpret_cast<float4 *>(ws + ((size_t)bh * n_chunks + c) * delta_rec_floats(dv) + bt_off) =
            make_float4(S[0], S[1], S[2], S[3]);
        sync_lds();
        fetch(p, c + kDepth);
        float sb[16];  // B operands: a lane's 16 features of its column, four 16-byte reads
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 v = *reinterpret_cast<const float4 *>(&img[c16 * kXR + 16 * q + 4 * i]);
            sb[4 * i] = v.x; sb[4 * i + 1] = v.y; sb[4 * i + 2] = v.z; sb[4 * i + 3] = v.w;
        }
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[j], sb[j], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(aa[j + 1], sb[j + 1], s1, 0, 0, 0);
        }
        S = s0 + s1 + f32x4d{bt.x, bt.y, bt.z, bt.w};
    };
    int c = 0;
    for (; c + kDepth <= n_chunks; c += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) step(pre[d], c + d);
    }
#pragma unroll
    for (int d = 0; d < kDepth; ++d)
        if (c + d < n_chunks) step(pre[d], c + d);
    if (S_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S_out[((size_t)bh * kXK + 16 * w + 4 * g + e) * dv + col0 + c16] = S[e];
    }
}

// O = Qt S_c + P Ut, one workgroup per (slice, chunk), every chunk at once;
// wave w owns token rows 16w..16w+15.  A = Qt rows (k-slot q of step j =
// feature 16q + j), B = S_c (a lane's 16 features of one column are one
// contiguous run of the record's S_c^T), C = the P Ut rows; every load of a
// 64-column group is issued before its products.
template <typename T>
__global__ __launch_bounds__(kXT) void k_delta_out(T *__restrict__ O, const float *__restrict__ ws, int N, int dv,
                                                   int n_chunks) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int bh = blockIdx.x / n_chunks, c = blockIdx.x % n_chunks;
    const int t0 = c * kXC, L = min(kXC, N - t0);
    const float *rec = ws + ((size_t)bh * n_chunks + c) * delta_rec_floats(dv);
    const float *Qt = rec, *PUT = rec + 2 * kXC * kXK, *SST = PUT + (size_t)kXC * dv;
    const auto ro = out_rsrc(O + ((size_t)bh * N + t0) * dv, L * dv * (int)sizeof(T));
    float qa[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(Qt + (16 * w + c16) * kXK + 16 * g + 4 * i);
        qa[4 * i] = v.x; qa[4 * i + 1] = v.y; qa[4 * i + 2] = v.z; qa[4 * i + 3] = v.w;
    }
    for (int cb0 = 0; cb0 < dv; cb0 += 64) {
        float sb[4][16];
        float4 pu[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = min(cb0 + 16 * cb, dv - 16);  // past d_v: a re-read, not stored
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float4 v = *reinterpret_cast<const float4 *>(SST + (size_t)(col + c16) * kXK + 16 * g + 4 * i);
                sb[cb][4 * i] = v.x; sb[cb][4 * i + 1] = v.y; sb[cb][4 * i + 2] = v.z; sb[cb][4 * i + 3] = v.w;
            }
            pu[cb] = *reinterpret_cast<const float4 *>(PUT + (size_t)(col + c16) * kXC + 16 * w + 4 * g);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = cb0 + 16 * cb;
            f32x4d o0 = f32x4d{pu[cb].x, pu[cb].y, pu[cb].z, pu[cb].w}, o1 = zero4d();
#pragma unroll
            for (int j = 0; j < 16; j += 2) {
                o0 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[j], sb[cb][j], o0, 0, 0, 0);
                o1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[j + 1], sb[cb][j + 1], o1, 0, 0, 0);
            }
            const f32x4d o = o0 + o1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * w + 4 * g + e, j = col + c16;
                const int off = (t < L && col < dv) ? (t * dv + j) * (int)sizeof(T) : L * dv * (int)sizeof(T);
                store_elem<T>(ro, off, o[e]);
            }
        }
    }
}

}  // namespace

bool delta_chunk_supported(int dk, int dv, int chunk) {
    return dk == kXK && dv >= 16 && dv <= 128 && dv % 16 == 0 && chunk == kXC;
}

size_t delta_chunk_ws_bytes(int BH, int N, int dv) {
    const size_t n_chunks = (size_t)(N + kXC - 1) / kXC;
    return sizeof(float) * (size_t)BH * n_chunks * delta_rec_floats(dv);
}

hipError_t launch_delta_chunk(const GatedArgs &a, int dtype, float *ws, hipStream_t st, KEvents ev_prep,
                              KEvents ev_scan, KEvents ev_out) {
    if (!delta_chunk_supported(a.dk, a.dv, kXC)) return hipErrorNotSupported;
    const int n_chunks = (a.N + kXC - 1) / kXC;
    const dim3 gp((unsigned)((size_t)a.BH * n_chunks)), gs((unsigned)((size_t)a.BH * (a.dv / 16))), blk(kXT);
    hipError_t e;
    if (dtype == kF32) {
        auto *q = static_cast<const float *>(a.Q), *k = static_cast<const float *>(a.K),
             *v = static_cast<const float *>(a.V);
        e = a.dv <= 64 ? launch_kernel_ev(k_delta_prep<float, 64>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                          a.N, a.dv, n_chunks, ws)
                       : launch_kernel_ev(k_delta_prep<float, 128>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                          a.N, a.dv, n_chunks, ws);
        if (e == hipSuccess) e = launch_kernel_ev(k_delta_scan, gs, blk, 0, st, ev_scan, ws, a.S_in, a.S_out, a.dv, n_chunks);
        if (e == hipSuccess)
            e = launch_kernel_ev(k_delta_out<float>, gp, blk, 0, st, ev_out, static_cast<float *>(a.O),
                                 static_cast<const float *>(ws), a.N, a.dv, n_chunks);
        return e;
    }
    auto *q = static_cast<const uint16_t *>(a.Q), *k = static_cast<const uint16_t *>(a.K),
         *v = static_cast<const uint16_t *>(a.V);
    e = a.dv <= 64 ? launch_kernel_ev(k_delta_prep<uint16_t, 64>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                      a.N, a.dv, n_chunks, ws)
                   : launch_kernel_ev(k_delta_prep<uint16_t, 128>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                      a.N, a.dv, n_chunks, ws);
    if (e == hipSuccess) e = launch_kernel_ev(k_delta_scan, gs, blk, 0, st, ev_scan, ws, a.S_in, a.S_out, a.dv, n_chunks);
    if (e == hipSuccess)
        e = launch_kernel_ev(k_delta_out<uint16_t>, gp, blk, 0, st, ev_out, static_cast<uint16_t *>(a.O),
                             static_cast<const float *>(ws), a.N, a.dv, n_chunks);
    return e;
}

}  // namespace la
