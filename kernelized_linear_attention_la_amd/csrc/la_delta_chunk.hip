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
// Two launches:
//  * k_delta_prep, one workgroup per (slice, chunk), all chunks at once: the
//    Gram matrices K K^T and Q K^T on fp32 matrix instructions, M and P, and
//    W, Ut by blocked forward substitution (16-row blocks: the update from the
//    solved blocks on matrix instructions, the diagonal block by substitution
//    with one right-hand column per thread), into the workspace.
//  * k_delta_scan, one workgroup per (slice, 16 value columns), the chunks in
//    order: U = Ut - W S0, O, and the state carried in fp32 accumulators.
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

// Per-chunk workspace record (floats): W [64][64], P [64][64], Ut [64][dv],
// g [64], g_C / g [64].
__host__ __device__ inline size_t delta_rec_floats(int dv) { return 2 * kXC * kXK + (size_t)kXC * dv + 2 * kXC; }

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
    float *W = rec, *P = rec + kXC * kXK, *Ut = rec + 2 * kXC * kXK, *gv = Ut + (size_t)kXC * dv, *gt = gv + kXC;

    // Gram tiles of row block w: K K^T (strictly lower part -> M) and Q K^T
    // (lower part with the diagonal -> P); tiles above the diagonal are zero
    for (int cb = 0; cb < 4; ++cb) {
        f32x4d gk = zero4d(), gq = zero4d();
        if (cb <= w) {
            auto bk = [&](int k, int n) { return sK[(16 * cb + n) * kXR + k]; };
            gk = mm4<16>([&](int m, int k) { return sK[(16 * w + m) * kXR + k]; }, bk, gk, lane);
            gq = mm4<16>([&](int m, int k) { return sQ[(16 * w + m) * kXR + k]; }, bk, gq, lane);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * w + 4 * g + e, s = 16 * cb + c16;
            const float ratio = s <= t ? __builtin_amdgcn_exp2f(sl[t] - sl[s]) : 0.f;
            sM[t * kXR + s] = s < t ? sb[t] * ratio * gk[e] : 0.f;
            P[t * kXK + s] = ratio * gq[e];
        }
    }
    if (tid < kXC) {
        gv[tid] = __builtin_amdgcn_exp2f(sl[tid]);
        gt[tid] = __builtin_amdgcn_exp2f(sl[kXC - 1] - sl[tid]);
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
            for (int r = 0; r < 16; ++r) {
                const int t = 16 * b + r;
                sX[t * RX + j] = x[r];
                if (j < kXK) W[t * kXK + j] = x[r];
                else Ut[(size_t)t * dv + (j - kXK)] = x[r];
            }
        }
        __syncthreads();
    }
}

// One workgroup per (slice, 16 value columns): the chunks in order.  Wave w
// owns token rows 16w..16w+15 of U and O, and feature rows 16w..16w+15 of the
// state (fp32 accumulators for the whole slice).  The row operands of W S0,
// Q S0 and P U come straight from global memory into registers, one chunk
// ahead: for those products k-step j of lane group q = l/16 takes index
// 16q + j (P U: 16kb + 4q + j), so each lane reads contiguous 16-byte runs,
// and the B operands (state image, U) are read from LDS in the same order.
template <typename T>
__global__ __launch_bounds__(kXT) void k_delta_scan(const T *__restrict__ Q, const T *__restrict__ K, T *__restrict__ O,
                                                    const float *__restrict__ ws, const float *__restrict__ S_in,
                                                    float *__restrict__ S_out, int N, int dv, int n_chunks) {
    __shared__ float sK[kXC * kXR];
    __shared__ float sS[kXK * 20], sU[kXC * 20], sUg[kXC * 20], sUt[kXC * 20];
    __shared__ float sg[kXC], sgt[kXC];
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

    constexpr int EP = 16 / (int)sizeof(T);         // elements per 16-byte piece
    constexpr int KP = kXC * kXK / EP / kXT;        // pieces of K per thread
    constexpr int QR = 16 / EP;                     // pieces of this lane's 16 Q values
    struct Pre {
        float4 w[4], p[4], ut, gg;
        uint4 q[QR], k[KP];
    };
    // Every load is unconditional (offsets clamped to valid data; the zero
    // selects happen where the values are used): a load under a branch makes
    // the compiler wait for all outstanding loads right after it, which would
    // turn the prefetch into a synchronous read.
    auto fetch = [&](Pre &f, int c_) {
        const int c = min(c_, n_chunks - 1);  // past the end: a harmless re-read of the last chunk
        const int t0 = c * kXC, L = min(kXC, N - t0);
        const float *rec = ws + ((size_t)bh * n_chunks + c) * delta_rec_floats(dv);
        const float *Wr = rec + (16 * w + r) * kXK + 16 * q;          // W[16w + r][16q ..]
        const float *Pr = rec + kXC * kXK + (16 * w + r) * kXK + 4 * q;  // P[16w + r][16kb + 4q ..]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.w[i] = *reinterpret_cast<const float4 *>(Wr + 4 * i);
            f.p[i] = *reinterpret_cast<const float4 *>(Pr + 16 * i);
        }
        f.ut = *reinterpret_cast<const float4 *>(rec + 2 * kXC * kXK + (size_t)(tid >> 2) * dv + col0 + 4 * (tid & 3));
        f.gg = reinterpret_cast<const float4 *>(rec + 2 * kXC * kXK + (size_t)kXC * dv)[tid & 31];
        const bool qlive = 16 * w + r < L;
        const T *qrow = Q + ((size_t)bh * N + t0 + (qlive ? 16 * w + r : 0)) * kXK + 16 * q;
#pragma unroll
        for (int i = 0; i < QR; ++i) f.q[i] = reinterpret_cast<const uint4 *>(qrow)[i];
        const char *kb = reinterpret_cast<const char *>(K + ((size_t)bh * N + t0) * kXK);
        const int bytes = L * kXK * (int)sizeof(T);
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int off = 16 * (tid + i * kXT);
            f.k[i] = *reinterpret_cast<const uint4 *>(kb + (off < bytes ? off : 0));
        }
    };
    auto unpack = [&](const uint4 &x, float *o) {
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
    Pre pre;
    fetch(pre, 0);

    for (int c = 0; c < n_chunks; ++c) {
        const int t0 = c * kXC, L = min(kXC, N - t0);
        const size_t tok0 = (size_t)bh * N + t0;
        // operands of chunk c in registers; K, Ut, gates and the state image into LDS
        // (query rows and key pieces past the end read as zero)
        const uint4 zero = make_uint4(0, 0, 0, 0);
        const bool qlive = 16 * w + r < L;
        const int kbytes = L * kXK * (int)sizeof(T);
        float wa[16], qa[16], pa[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wa[4 * i] = pre.w[i].x; wa[4 * i + 1] = pre.w[i].y; wa[4 * i + 2] = pre.w[i].z; wa[4 * i + 3] = pre.w[i].w;
            pa[4 * i] = pre.p[i].x; pa[4 * i + 1] = pre.p[i].y; pa[4 * i + 2] = pre.p[i].z; pa[4 * i + 3] = pre.p[i].w;
        }
#pragma unroll
        for (int i = 0; i < QR; ++i) unpack(qlive ? pre.q[i] : zero, &qa[EP * i]);
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const int e0 = EP * (tid + i * kXT), t = e0 / kXK, f = e0 % kXK;
            float o[EP];
            unpack(16 * (tid + i * kXT) < kbytes ? pre.k[i] : zero, o);
#pragma unroll
            for (int e = 0; e < EP; ++e) sK[t * kXR + f + e] = o[e];
        }
        *reinterpret_cast<float4 *>(&sUt[(tid >> 2) * 20 + 4 * (tid & 3)]) = pre.ut;
        if (tid < 32) {
            const float gg[4] = {pre.gg.x, pre.gg.y, pre.gg.z, pre.gg.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * tid + e;  // gate products g, then g_C / g
                if (i < kXC) sg[i] = gg[e];
                else sgt[i - kXC] = gg[e];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) sS[(16 * w + 4 * g + e) * 20 + c16] = S[e];
        sync_lds();
        fetch(pre, c + 1);

        // U = Ut - W S0 and Q S0 for token rows 16w..16w+15 (k = 16q + j); two
        // accumulators per product halve the dependent chains
        float sb[16];  // B operands read from LDS all at once, then the products
#pragma unroll
        for (int j = 0; j < 16; ++j) sb[j] = sS[(16 * q + j) * 20 + c16];
        f32x4d ws0 = zero4d(), o = zero4d(), ws1 = zero4d(), o1 = zero4d();
#pragma unroll
        for (int j = 0; j < 16; j += 2) {
            ws0 = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[j], sb[j], ws0, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[j], sb[j], o, 0, 0, 0);
            ws1 = __builtin_amdgcn_mfma_f32_16x16x4f32(wa[j + 1], sb[j + 1], ws1, 0, 0, 0);
            o1 = __builtin_amdgcn_mfma_f32_16x16x4f32(qa[j + 1], sb[j + 1], o1, 0, 0, 0);
        }
        ws0 += ws1;
        o += o1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * w + 4 * g + e;
            const float u = sUt[t * 20 + c16] - ws0[e];
            sU[t * 20 + c16] = u;
            sUg[t * 20 + c16] = sgt[t] * u;
            o[e] *= sg[t];
        }
        sync_lds();

        // O += P U over the key blocks up to this row block (k = 16kb + 4q + j)
        f32x4d o2 = zero4d();
        for (int kb = 0; kb <= w; ++kb) {
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                o = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * kb + j], sU[(16 * kb + 4 * q + j) * 20 + c16], o, 0, 0, 0);
                o2 = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[4 * kb + j + 1], sU[(16 * kb + 4 * q + j + 1) * 20 + c16], o2,
                                                          0, 0, 0);
            }
        }
        o += o2;
        // S = g_C S0 + K^T diag(g_C / g) U for feature rows 16w..16w+15 (tokens
        // 0..31 and 32..63 in two accumulators)
        auto aK = [&](int m, int k) { return sK[k * kXR + 16 * w + m]; };
        const f32x4d ku = mm4<8>(aK, [&](int k, int n) { return sUg[k * 20 + n]; }, zero4d(), lane) +
                          mm4<8>([&](int m, int k) { return aK(m, k + 32); },
                                 [&](int k, int n) { return sUg[(k + 32) * 20 + n]; }, zero4d(), lane);
        const float gC = sg[kXC - 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) S[e] = gC * S[e] + ku[e];
        const auto ro = out_rsrc(O + tok0 * dv, L * dv * (int)sizeof(T));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * w + 4 * g + e;
            store_elem<T>(ro, t < L ? (t * dv + col0 + c16) * (int)sizeof(T) : L * dv * (int)sizeof(T), o[e]);
        }
        sync_lds();  // every read of this chunk's tiles done before the next staging
    }
    if (S_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S_out[((size_t)bh * kXK + 16 * w + 4 * g + e) * dv + col0 + c16] = S[e];
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
                              KEvents ev_scan) {
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
        if (e != hipSuccess) return e;
        return launch_kernel_ev(k_delta_scan<float>, gs, blk, 0, st, ev_scan, q, k, static_cast<float *>(a.O),
                                static_cast<const float *>(ws), a.S_in, a.S_out, a.N, a.dv, n_chunks);
    }
    auto *q = static_cast<const uint16_t *>(a.Q), *k = static_cast<const uint16_t *>(a.K),
         *v = static_cast<const uint16_t *>(a.V);
    e = a.dv <= 64 ? launch_kernel_ev(k_delta_prep<uint16_t, 64>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                      a.N, a.dv, n_chunks, ws)
                   : launch_kernel_ev(k_delta_prep<uint16_t, 128>, gp, blk, 0, st, ev_prep, q, k, v, a.alpha, a.beta,
                                      a.N, a.dv, n_chunks, ws);
    if (e != hipSuccess) return e;
    return launch_kernel_ev(k_delta_scan<uint16_t>, gs, blk, 0, st, ev_scan, q, k, static_cast<uint16_t *>(a.O),
                            static_cast<const float *>(ws), a.S_in, a.S_out, a.N, a.dv, n_chunks);
}

}  // namespace la
