// Backward of the causal normalised form on the matrix cores: ELU+1,
// d_k = d_v = 64, 64-token chunks, bf16 storage (the derivation and the
// fp32-FMA kernels are in la_backward.hip; this file runs the same chunked
// algebra with v_mfma_f32_16x16x4_f32).
//
// The arithmetic stays fp32 throughout: the normalised backward cancels
// (g_i . v_j + h_i = g_i . (v_j - o_i), and o_i, h_i come from the recomputed
// forward), so operands rounded to bf16 lose several percent of the gradient;
// fp32 matrix instructions keep the fp32 result.  For that instruction lane l
// supplies A[l%16][l/16] and B[l/16][l%16] of a 16x4 by 4x16 step and receives
// C[4(l/16)+e][l%16]; both operands are single fp32 values, so either
// orientation of a tile is read straight from its one row-major copy in LDS.
// Per chunk the tiles are phi(Q), phi(K), [V | 1 | 0], G_aug, the carried
// state image and a score tile; value-column widths are padded to 68 for
// contractions and 80 (five 16-column blocks) for outputs.
//
// Per chunk, wave w owns query rows 16w..16w+15 (dQ pass) or key rows
// (dK/dV pass) for the row products, and feature rows 16w..16w+15 of the
// carried states (S_aug, U in the dQ pass; R_aug in the dK/dV pass), kept in
// fp32 accumulators and mirrored into LDS for the products that read them.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

constexpr int kD = 64;          // d_k = d_v = d'
constexpr int kC = 64;          // tokens per chunk
constexpr int kVK = 68;         // value columns in contractions (v | 1 | 0 0 0)
constexpr int kVN = 80;         // value columns in outputs (five 16-column blocks)
constexpr int kNW = 4;          // waves
constexpr int kThreads = 64 * kNW;
constexpr int kR64 = 64 + 4;    // row stride of 64-wide tiles (floats)
constexpr int kRV = kVN + 4;    // row stride of value-wide tiles
constexpr int kGW = kVK;        // G_aug floats per token in the workspace

// C[16 rows at m0][16 NB columns at n0] += A B over K (a multiple of 4).
// TA: A is given as its transpose (row-major [k][m]); TB: B as its transpose ([n][k]).
template <int K, int NB, bool TA, bool TB>
__device__ __forceinline__ void mm(const float *A, int lda, int m0, const float *B, int ldb, int n0, f32x4 (&acc)[NB],
                                   int lane) {
    const int r = lane & 15, q = lane >> 4;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
        const float a = TA ? A[(k0 + q) * lda + m0 + r] : A[(m0 + r) * lda + k0 + q];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const float b = TB ? B[(n0 + 16 * j + r) * ldb + k0 + q] : B[(k0 + q) * ldb + n0 + 16 * j + r];
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
        }
    }
}

// accumulator block (rows m0 + 4g + e, column n0 + c16) -> row-major tile [m][n]
__device__ __forceinline__ void put_rows(float *T, int ld, int m0, int n0, f32x4 v, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int e = 0; e < 4; ++e) T[(m0 + 4 * g + e) * ld + n0 + c] = v[e];
}

__device__ __forceinline__ float elu1(float x) { return x > 0.f ? x + 1.f : expf(x); }

struct Tiles {
    float P[kC * kR64];  // phi(Q) rows [token][feature]
    float K[kC * kR64];  // phi(K) rows
    float V[kC * kRV];   // [v | 1 | 0] rows
    float G[kC * kRV];   // G_aug rows [token][value column]
    float S[kD * kRV];   // carried state, rows [feature][value column]
    float W[kC * kR64];  // masked scores, rows of the owning wave
};

// phi(X) rows t0.. of one chunk (rows past `rows` are zero)
__device__ void stage_phi(const uint16_t *X, int t0, int rows, float *R, int tid) {
#pragma unroll
    for (int i = 0; i < kC * kD / 8 / kThreads; ++i) {
        const int u = tid + i * kThreads, t = u / (kD / 8), c8 = u % (kD / 8);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (t < rows) x = *reinterpret_cast<const uint4 *>(&X[(size_t)(t0 + t) * kD + 8 * c8]);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        float4 a, b;
        a.x = elu1(lo_bf16(w[0])); a.y = elu1(hi_bf16(w[0])); a.z = elu1(lo_bf16(w[1])); a.w = elu1(hi_bf16(w[1]));
        b.x = elu1(lo_bf16(w[2])); b.y = elu1(hi_bf16(w[2])); b.z = elu1(lo_bf16(w[3])); b.w = elu1(hi_bf16(w[3]));
        if (t >= rows) a = b = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4 *>(&R[t * kR64 + 8 * c8]) = a;
        *reinterpret_cast<float4 *>(&R[t * kR64 + 8 * c8 + 4]) = b;
    }
}

// [v | 1 | 0] rows of one chunk (columns 64..kRV-1 written too)
__device__ void stage_vaug(const uint16_t *V, int t0, int rows, float *R, int tid) {
#pragma unroll
    for (int i = 0; i < kC * kD / 8 / kThreads; ++i) {
        const int u = tid + i * kThreads, t = u / (kD / 8), c8 = u % (kD / 8);
        uint4 x = make_uint4(0, 0, 0, 0);
        if (t < rows) x = *reinterpret_cast<const uint4 *>(&V[(size_t)(t0 + t) * kD + 8 * c8]);
        *reinterpret_cast<float4 *>(&R[t * kRV + 8 * c8]) =
            make_float4(lo_bf16(x.x), hi_bf16(x.x), lo_bf16(x.y), hi_bf16(x.y));
        *reinterpret_cast<float4 *>(&R[t * kRV + 8 * c8 + 4]) =
            make_float4(lo_bf16(x.z), hi_bf16(x.z), lo_bf16(x.w), hi_bf16(x.w));
    }
    for (int u = tid; u < kC * (kRV - kD); u += kThreads) {
        const int t = u / (kRV - kD), c = kD + u % (kRV - kD);
        R[t * kRV + c] = (c == kD && t < rows) ? 1.f : 0.f;
    }
}

// G_aug rows (fp32 in the workspace, kGW per token) of one chunk
__device__ void stage_g(const float *Gw, int t0, int rows, float *R, int tid) {
    for (int u = tid; u < kC * kRV / 4; u += kThreads) {
        const int t = u / (kRV / 4), c4 = u % (kRV / 4);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < rows && 4 * c4 < kGW) x = *reinterpret_cast<const float4 *>(&Gw[(size_t)(t0 + t) * kGW + 4 * c4]);
        *reinterpret_cast<float4 *>(&R[t * kRV + 4 * c4]) = x;
    }
}

// this wave's 16 feature rows of a carried state (5 accumulator blocks) into the LDS image
__device__ __forceinline__ void put_state(const f32x4 (&S)[5], float *T, int w, int lane) {
#pragma unroll
    for (int j = 0; j < 5; ++j) put_rows(T, kRV, 16 * w, 16 * j, S[j], lane);
}

__device__ __forceinline__ void store_rows(const float *T, int ld, int m0, int rows, uint16_t *dst, size_t row0,
                                           int lane) {
    // 16 rows x 64 columns of T (rows m0..) -> bf16 rows of dst, 16 bytes per lane
#pragma unroll
    for (int it = 0; it < 16 * kD / 8 / 64; ++it) {
        const int idx = it * 64 + lane, r = idx / (kD / 8), c8 = idx % (kD / 8);
        if (m0 + r < rows) {
            const float *s = &T[(m0 + r) * ld + 8 * c8];
            uint4 o;
            o.x = f32_to_bf16(s[0]) | (static_cast<uint32_t>(f32_to_bf16(s[1])) << 16);
            o.y = f32_to_bf16(s[2]) | (static_cast<uint32_t>(f32_to_bf16(s[3])) << 16);
            o.z = f32_to_bf16(s[4]) | (static_cast<uint32_t>(f32_to_bf16(s[5])) << 16);
            o.w = f32_to_bf16(s[6]) | (static_cast<uint32_t>(f32_to_bf16(s[7])) << 16);
            *reinterpret_cast<uint4 *>(&dst[(row0 + m0 + r) * kD + 8 * c8]) = o;
        }
    }
}

// ---------------------------------------------------------------------------
// dQ pass.  Chunks in order from the forward prefix [S | z] of the segment:
//   num_aug = (P (.) M) V_aug + phi(Q) S_aug          P = phi(Q) phi(K)^T
//   G_aug   = [dO / den | -(dO . o) / den | 0]
//   dphi(Q) = (A (.) M) phi(K) + G_aug S_aug^T        A = G_aug V_aug^T
//   dQ = dphi(Q) * elu'(q),  elu'(q) = min(phi(q), 1)
//   U      += phi(Q)^T G_aug    (segment sums for the reverse scan)
//   S_aug  += phi(K)^T V_aug
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_bwd_dq_mfma(BwdMfmaArgs a) {
    __shared__ Tiles sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
    const int N = a.N;
    const int c_begin = seg * a.seg_chunks, c_end = min(a.n_chunks, c_begin + a.seg_chunks);
    const uint16_t *Qs = a.Q + (size_t)bh * N * kD;
    const uint16_t *Ks = a.K + (size_t)bh * N * kD;
    const uint16_t *Vs = a.V + (size_t)bh * N * kD;
    const uint16_t *dOs = a.dO + (size_t)bh * N * kD;
    uint16_t *dQs = a.dQ + (size_t)bh * N * kD;
    float *Gw = a.G + (size_t)bh * N * kGW;
    const int m0 = 16 * w;

    // carried state S_aug (feature rows 16w.., value columns 16j + c16) and U
    f32x4 S[5], U[5];
    {
        const float *Sp = a.Spre + ((size_t)bh * a.P + seg) * kD * kD;
        const float *zp = a.zpre + ((size_t)bh * a.P + seg) * kD;
#pragma unroll
        for (int j = 0; j < 5; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = m0 + 4 * g + e, col = 16 * j + c16;
                S[j][e] = col < kD ? Sp[f * kD + col] : (col == kD ? zp[f] : 0.f);
            }
            U[j] = zero4();
        }
    }
    put_state(S, sm.S, w, lane);

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * kC, rows = min(kC, N - t0);
        block_sync_lds();  // the previous chunk's tiles are consumed, the state image is complete
        stage_phi(Qs, t0, rows, sm.P, tid);
        stage_phi(Ks, t0, rows, sm.K, tid);
        stage_vaug(Vs, t0, rows, sm.V, tid);
        block_sync_lds();

        // scores P = phi(Q) phi(K)^T of this wave's queries, masked (key <= query)
        {
            f32x4 p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = zero4();
            mm<kD, 4, false, true>(sm.P, kR64, m0, sm.K, kR64, 0, p, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * j + c16 > m0 + 4 * g + e) p[j][e] = 0.f;
                put_rows(sm.W, kR64, m0, 16 * j, p[j], lane);
            }
        }
        wave_lds_sync();
        // num_aug = (P (.) M) V_aug + phi(Q) S_aug
        f32x4 num[5];
#pragma unroll
        for (int j = 0; j < 5; ++j) num[j] = zero4();
        mm<kC, 5, false, false>(sm.W, kR64, m0, sm.V, kRV, 0, num, lane);
        mm<kD, 5, false, false>(sm.P, kR64, m0, sm.S, kRV, 0, num, lane);
        // G_aug: den is column 64 (block 4, lane c16 = 0 of each row group)
        f32x4 gv[5];
        {
            float rden[4], dot[4];
            f32x4 dov[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rden[e] = 1.f / __shfl(num[4][e], lane & 48, 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot[e] = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = m0 + 4 * g + e;
                    const float d = t < rows ? bf16_to_f32(dOs[(size_t)(t0 + t) * kD + 16 * j + c16]) : 0.f;
                    dov[j][e] = d;
                    dot[e] += d * (num[j][e] * rden[e]);
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // row sums over the 16 lanes of a row group
                float x = dot[e];
                x += __shfl_xor(x, 1, 64);
                x += __shfl_xor(x, 2, 64);
                x += __shfl_xor(x, 4, 64);
                x += __shfl_xor(x, 8, 64);
                dot[e] = x;
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const bool in = m0 + 4 * g + e < rows;
#pragma unroll
                for (int j = 0; j < 4; ++j) gv[j][e] = in ? dov[j][e] * rden[e] : 0.f;
                gv[4][e] = (c16 == 0 && in) ? -dot[e] * rden[e] : 0.f;
            }
        }
#pragma unroll
        for (int j = 0; j < 5; ++j) put_rows(sm.G, kRV, m0, 16 * j, gv[j], lane);
        wave_lds_sync();
        // G_aug rows to the workspace (kGW floats per token) for the dK/dV pass
        for (int idx = lane; idx < 16 * kGW / 4; idx += 64) {
            const int r = idx / (kGW / 4), c4 = idx % (kGW / 4);
            if (m0 + r < rows)
                *reinterpret_cast<float4 *>(&Gw[(size_t)(t0 + m0 + r) * kGW + 4 * c4]) =
                    *reinterpret_cast<const float4 *>(&sm.G[(m0 + r) * kRV + 4 * c4]);
        }
        // A = G_aug V_aug^T, masked; dphi(Q) = (A (.) M) phi(K) + G_aug S_aug^T
        {
            f32x4 s[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) s[j] = zero4();
            mm<kVK, 4, false, true>(sm.G, kRV, m0, sm.V, kRV, 0, s, lane);
            wave_lds_sync();  // every lane has read the scores P before W is overwritten
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * j + c16 > m0 + 4 * g + e) s[j][e] = 0.f;
                put_rows(sm.W, kR64, m0, 16 * j, s[j], lane);
            }
        }
        wave_lds_sync();
        f32x4 dp[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) dp[j] = zero4();
        mm<kC, 4, false, false>(sm.W, kR64, m0, sm.K, kR64, 0, dp, lane);
        mm<kVK, 4, false, true>(sm.G, kRV, m0, sm.S, kRV, 0, dp, lane);
        // dQ = dphi * min(phi(q), 1) (elu'(q): 1 for q > 0, exp(q) = phi(q) otherwise)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[j][e] *= fminf(sm.P[(m0 + 4 * g + e) * kR64 + 16 * j + c16], 1.f);
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) put_rows(sm.W, kR64, m0, 16 * j, dp[j], lane);
        wave_lds_sync();
        store_rows(sm.W, kR64, m0, rows, dQs, t0, lane);
        block_sync_lds();  // every wave's G_aug rows are in LDS, the state image is read
        // U += phi(Q)^T G_aug, S_aug += phi(K)^T V_aug (this wave's feature rows)
        mm<kC, 5, true, false>(sm.P, kR64, m0, sm.G, kRV, 0, U, lane);
        mm<kC, 5, true, false>(sm.K, kR64, m0, sm.V, kRV, 0, S, lane);
        put_state(S, sm.S, w, lane);
    }
    // segment sums U, layout [feature][d_v + 1] (value columns 0..64)
    float *Us = a.U + ((size_t)bh * a.P + seg) * kD * (kD + 1);
#pragma unroll
    for (int j = 0; j < 5; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = m0 + 4 * g + e, col = 16 * j + c16;
            if (col <= kD) Us[f * (kD + 1) + col] = U[j][e];
        }
}

// ---------------------------------------------------------------------------
// dK / dV pass.  Chunks in reverse from R_aug = dS_out_aug + the later
// segments' sums (key rows j of this wave):
//   dphi(K) = (B (.) M') phi(Q) + V_aug R_aug^T       B = V_aug G_aug^T
//   dV      = (P' (.) M') G     + phi(K) R            P' = phi(K) phi(Q)^T
//   (M': query >= key),  dK = dphi(K) * min(phi(k), 1)
//   R_aug  += phi(Q)^T G_aug
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_bwd_dkv_mfma(BwdMfmaArgs a) {
    __shared__ Tiles sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
    const int N = a.N;
    const int c_begin = seg * a.seg_chunks, c_end = min(a.n_chunks, c_begin + a.seg_chunks);
    const uint16_t *Qs = a.Q + (size_t)bh * N * kD;
    const uint16_t *Ks = a.K + (size_t)bh * N * kD;
    const uint16_t *Vs = a.V + (size_t)bh * N * kD;
    uint16_t *dKs = a.dK + (size_t)bh * N * kD;
    uint16_t *dVs = a.dV + (size_t)bh * N * kD;
    const float *Gw = a.G + (size_t)bh * N * kGW;
    const int m0 = 16 * w;

    f32x4 R[5];
    {
        const float *Rs = a.U + ((size_t)bh * a.P + seg) * kD * (kD + 1);
#pragma unroll
        for (int j = 0; j < 5; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = m0 + 4 * g + e, col = 16 * j + c16;
                R[j][e] = col <= kD ? Rs[f * (kD + 1) + col] : 0.f;
            }
    }
    put_state(R, sm.S, w, lane);

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * kC, rows = min(kC, N - t0);
        block_sync_lds();
        stage_phi(Qs, t0, rows, sm.P, tid);
        stage_phi(Ks, t0, rows, sm.K, tid);
        stage_vaug(Vs, t0, rows, sm.V, tid);
        stage_g(Gw, t0, rows, sm.G, tid);
        block_sync_lds();

        // dphi(K): B = V_aug G_aug^T masked (query >= key), times phi(Q); + V_aug R_aug^T
        f32x4 dk[4];
        {
            f32x4 b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = zero4();
            mm<kVK, 4, false, true>(sm.V, kRV, m0, sm.G, kRV, 0, b, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * j + c16 < m0 + 4 * g + e) b[j][e] = 0.f;
                put_rows(sm.W, kR64, m0, 16 * j, b[j], lane);
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) dk[j] = zero4();
        mm<kC, 4, false, false>(sm.W, kR64, m0, sm.P, kR64, 0, dk, lane);
        mm<kVK, 4, false, true>(sm.V, kRV, m0, sm.S, kRV, 0, dk, lane);
        // dV: P' = phi(K) phi(Q)^T masked, times G; + phi(K) R
        f32x4 dv[4];
        {
            f32x4 p[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) p[j] = zero4();
            mm<kD, 4, false, true>(sm.K, kR64, m0, sm.P, kR64, 0, p, lane);
            wave_lds_sync();  // every lane has read the scores B before W is overwritten
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * j + c16 < m0 + 4 * g + e) p[j][e] = 0.f;
                put_rows(sm.W, kR64, m0, 16 * j, p[j], lane);
            }
        }
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) dv[j] = zero4();
        mm<kC, 4, false, false>(sm.W, kR64, m0, sm.G, kRV, 0, dv, lane);
        mm<kD, 4, false, false>(sm.K, kR64, m0, sm.S, kRV, 0, dv, lane);
        // dK = dphi(K) * min(phi(k), 1); dK and dV rows leave through W
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) dk[j][e] *= fminf(sm.K[(m0 + 4 * g + e) * kR64 + 16 * j + c16], 1.f);
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) put_rows(sm.W, kR64, m0, 16 * j, dk[j], lane);
        wave_lds_sync();
        store_rows(sm.W, kR64, m0, rows, dKs, t0, lane);
        wave_lds_sync();
#pragma unroll
        for (int j = 0; j < 4; ++j) put_rows(sm.W, kR64, m0, 16 * j, dv[j], lane);
        wave_lds_sync();
        store_rows(sm.W, kR64, m0, rows, dVs, t0, lane);
        block_sync_lds();  // the state image is no longer read
        // R_aug += phi(Q)^T G_aug (this wave's feature rows)
        mm<kC, 5, true, false>(sm.P, kR64, m0, sm.G, kRV, 0, R, lane);
        put_state(R, sm.S, w, lane);
    }
}

}  // namespace

bool backward_mfma_supported(const Shape &sh, int chunk) {
    return sh.dtype == kBF16 && sh.phi == kElu1 && sh.dk == kD && sh.dv == kD && chunk == kC;
}

size_t backward_mfma_g_floats() { return kGW; }

hipError_t launch_bwd_dq_mfma(const BwdMfmaArgs &a, hipStream_t st, KEvents ev) {
    return launch_kernel_ev(k_bwd_dq_mfma, dim3((unsigned)((size_t)a.BH * a.P)), dim3(kThreads), 0, st, ev, a);
}

hipError_t launch_bwd_dkv_mfma(const BwdMfmaArgs &a, hipStream_t st, KEvents ev) {
    return launch_kernel_ev(k_bwd_dkv_mfma, dim3((unsigned)((size_t)a.BH * a.P)), dim3(kThreads), 0, st, ev, a);
}

}  // namespace la
