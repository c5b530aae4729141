// Chunkwise kernels for fp32 storage on fp32 matrix instructions
// (v_mfma_f32_16x16x4_f32), d_k = d_v = D in {64, 128}: ELU+1 normalised, or
// retention (identity map, decay lambda per head, no normaliser).
//
// The chunkwise causal form ("Linear Attention", chunkwise parallel form;
// "Story of Attention Part 5", section 6 blockwise split with decay 1 and the
// normaliser of 1a) with every product in fp32 (the 1e-4 accuracy of fp32
// storage rules out bf16 operands):
//   P^T   = phi(K_c) phi(Q_c)^T,  masked to keys <= queries
//   out   = (P (.) M) V_aug + phi(Q_c) S_aug        (V_aug = [V | 1 | 0..])
//   O     = out[:, :D] / out[:, D]
//   S_aug += phi(K_c)^T V_aug
// One workgroup of four waves owns one (slice, segment) and walks its tokens
// in 32-token tiles (the chunkwise form gives the same sums for every chunk
// length).  For the instruction lane l supplies A[l%16][l/16] and B[l/16][l%16]
// of a 16x4 by 4x16 step and receives D[4(l/16)+e][l%16]; both operands are
// single fp32 values, so every product reads its operands from one row-major
// fp32 LDS tile in either orientation.  The scores are computed transposed, so
// that a lane's accumulators P^T[4g+e][q] are the A operand of the value
// product for the k-slots t = 4g + e (the value rows are read in the same
// order): P never leaves the registers.
//   * wave w: query block w & 1 (16 rows) and value blocks 0..4 (w < 2) or
//     5..8 (w >= 2, with the normaliser block) for the outputs; feature rows
//     D/4 w .. D/4 w + D/4 - 1 of the fp32 state S_aug in its accumulators,
//     mirrored into an LDS image that the next tile's outputs read.
// Modes as the other chunk kernels: segment sums (kModeState), causal from a
// prefix state (kModeCausal), non-causal read of a fixed state (kModeRead).
// Retention ("Story of Attention Part 5", section 4 and the blockwise split of
// section 6): the scores take lambda^(i-t) inside a tile, the carried state is
// read with lambda^(i+1) for tile row i, and the state moves on as
// S <- lambda^L S + sum_t lambda^(L-1-t) k_t v_t^T; the powers come from a
// table of lambda^0..lambda^32 formed once per workgroup.
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kFT = 32;       // tokens per tile
constexpr int kFW4 = 4;       // waves
constexpr int kFThr = 64 * kFW4;

template <int D, bool RET>
struct F32Cfg {
    static constexpr int NJ = D / 16 + (RET ? 0 : 1);  // value blocks (+ the normaliser block)
    // row strides (floats): 2 mod 32 makes the 16-row x 4-column operand reads
    // of phi(Q), phi(K) conflict free; 4 mod 8 puts the two 16-lane halves of a
    // value-row read in opposite halves of the banks
    static constexpr int RX = D + 2;
    static constexpr int VA = D + 16;        // V_aug columns
    static constexpr int RV = VA + 4;        // V_aug and state image row stride
    static constexpr int SPLIT = (NJ + 1) / 2;  // value blocks of the first half
    static constexpr int FBW = D / 64;       // 16-row feature blocks per wave (D/4 rows)
};

template <int D, bool RET>
struct F32Smem {
    using G = F32Cfg<D, RET>;
    float Q[kFT * G::RX];   // phi(Q) rows (ELU+1: scaled per row by a power of two)
    float K[kFT * G::RX];   // phi(K) rows
    float V[kFT * G::RV];   // [V | 1 | 0..] rows
    float S[D * G::RV];     // image of the carried state S_aug, rows = features
    float DEN[2][16];       // normaliser of each query block, for the waves without it
    float DW[kFT + 1];      // retention: lambda^x, x = 0..32
};

__device__ __forceinline__ f32x4_t z4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4_t mma4(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, int MODE, bool RET>
__global__ __launch_bounds__(kFThr) void k_f32mma(FwdArgs a) {
    using G = F32Cfg<D, RET>;
    constexpr int NJ = G::NJ, RX = G::RX, RV = G::RV, FBW = G::FBW;
    constexpr bool OUT = MODE != kModeState;
    constexpr bool NEED_K = MODE != kModeRead;
    __shared__ F32Smem<D, RET> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    const Segments sg = a.sg;
    const int N = a.sh.N;
    const int seg = blockIdx.x % sg.P, bh = blockIdx.x / sg.P;
    const int t_begin = seg * sg.seg_chunks * sg.chunk;
    const int t_end = min(N, t_begin + sg.seg_chunks * sg.chunk);

    const float *Qs = static_cast<const float *>(a.Q) + (size_t)bh * N * D;
    const float *Ks = static_cast<const float *>(a.K) + (size_t)bh * N * D;
    const float *Vs = static_cast<const float *>(a.V) + (size_t)bh * N * D;
    float *Os = OUT ? static_cast<float *>(a.O) + (size_t)bh * N * D : nullptr;
    if constexpr (RET) {  // ordered before use by the first barrier of the tile loop
        const float l2 = log2f(a.sh.gamma[bh % a.sh.H]);
        if (tid <= kFT) sm.DW[tid] = tid == 0 ? 1.f : exp2f(l2 * (float)tid);
    }

    constexpr int SPLIT = G::SPLIT;
    const int qb = w & 1;                                          // query block of this wave

    // ---- the carried state: rows D/4 w + 16 q + 4g + e, columns 16 nb + c16
    f32x4_t S[FBW][NJ];
    {
        const float *Ssrc = a.st.S_src ? a.st.S_src + bh * a.st.src_slice + seg * a.st.src_seg : nullptr;
        const float *zsrc = a.st.z_src ? a.st.z_src + bh * a.st.zsrc_slice + seg * a.st.zsrc_seg : nullptr;
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = (D / 4) * w + 16 * q + 4 * g + e, j = 16 * nb + c16;
                    S[q][nb][e] = !Ssrc ? 0.f : (j < D ? Ssrc[(size_t)f * D + j] : (j == D ? zsrc[f] : 0.f));
                }
    }
    auto put_image = [&]() {
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.S[((D / 4) * w + 16 * q + 4 * g + e) * RV + 16 * nb + c16] = S[q][nb][e];
    };
    if constexpr (OUT) put_image();
    // normaliser block of V_aug: column D is 1 for every live token, 0 past the end
    // (written per tile below), columns D+1.. are 0
    for (int u = tid; u < kFT * (RV - D); u += kFThr) {
        const int t = u / (RV - D), c = D + u % (RV - D);
        sm.V[t * RV + c] = 0.f;
    }

    // ---- register prefetch of a tile: 32 rows of Q, K, V as float4 pieces
    constexpr int P4 = kFT * D / 4 / kFThr;  // float4 pieces per thread and tensor
    float4 pq[P4], pk[P4], pv[P4];
    auto fetch = [&](int t0, bool live) {
        const int rows = live ? min(kFT, t_end - t0) : 0;
#pragma unroll
        for (int i = 0; i < P4; ++i) {
            const int u = tid + i * kFThr, t = u / (D / 4), c4 = u % (D / 4);
            const bool in = t < rows;
            const size_t off = (size_t)(in ? t0 + t : t_begin) * D + 4 * c4;  // clamped: every load is issued
            if constexpr (OUT) pq[i] = *reinterpret_cast<const float4 *>(Qs + off);
            if constexpr (NEED_K) {
                pk[i] = *reinterpret_cast<const float4 *>(Ks + off);
                pv[i] = *reinterpret_cast<const float4 *>(Vs + off);
            }
        }
    };
    // phi into LDS; rows past the segment's end are zero (phi = 0 adds nothing).
    // Piece i of a thread is row (tid + 256 i) / (D/4): the D/4 pieces of a row
    // sit in consecutive lanes, which also reduce the row's largest query
    // coordinate for its power-of-two scale (it cancels in the division).
    auto stage = [&](int t0) {
        const int rows = min(kFT, t_end - t0);
#pragma unroll
        for (int i = 0; i < P4; ++i) {
            const int u = tid + i * kFThr, t = u / (D / 4), c4 = u % (D / 4);
            const bool in = t < rows;
            if constexpr (OUT) {
                const float4 x = pq[i];
                float2 y0, y1;
                if constexpr (RET) {
                    y0 = make_float2(x.x, x.y);
                    y1 = make_float2(x.z, x.w);
                } else {
                    float m = fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
#pragma unroll
                    for (int o = 1; o < D / 4; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
                    const float e = elu1_query_shift(m);
                    y0 = make_float2(elu1_accurate_scaled(x.x, e), elu1_accurate_scaled(x.y, e));
                    y1 = make_float2(elu1_accurate_scaled(x.z, e), elu1_accurate_scaled(x.w, e));
                }
                if (!in) y0 = y1 = make_float2(0.f, 0.f);
                *reinterpret_cast<float2 *>(&sm.Q[t * RX + 4 * c4]) = y0;
                *reinterpret_cast<float2 *>(&sm.Q[t * RX + 4 * c4 + 2]) = y1;
            }
            if constexpr (NEED_K) {
                const float4 x = pk[i];
                float2 y0 = RET ? make_float2(x.x, x.y) : make_float2(elu1_accurate(x.x), elu1_accurate(x.y));
                float2 y1 = RET ? make_float2(x.z, x.w) : make_float2(elu1_accurate(x.z), elu1_accurate(x.w));
                float4 v = pv[i];
                if (!in) {
                    y0 = y1 = make_float2(0.f, 0.f);
                    v = make_float4(0.f, 0.f, 0.f, 0.f);
                }
                *reinterpret_cast<float2 *>(&sm.K[t * RX + 4 * c4]) = y0;
                *reinterpret_cast<float2 *>(&sm.K[t * RX + 4 * c4 + 2]) = y1;
                *reinterpret_cast<float4 *>(&sm.V[t * RV + 4 * c4]) = v;
            }
        }
        if constexpr (NEED_K)
            if (tid < kFT) sm.V[tid * RV + D] = tid < rows ? 1.f : 0.f;
    };

    fetch(t_begin, t_begin < t_end);
    for (int t0 = t_begin; t0 < t_end; t0 += kFT) {
        __syncthreads();  // the previous tile's tiles and image are no longer read
        stage(t0);
        __syncthreads();
        fetch(t0 + kFT, t0 + kFT < t_end);

        if constexpr (OUT) {
            // the value half is a compile-time property of the wave: with a run-time
            // block count the accumulators rotate through registers
            auto outputs = [&](auto half) {
                constexpr int NB0 = decltype(half)::value ? SPLIT : 0;
                constexpr int NBN = decltype(half)::value ? NJ - SPLIT : SPLIT;
                f32x4_t acc[NBN];
#pragma unroll
                for (int j = 0; j < NBN; ++j) acc[j] = z4();
                // phi(Q) S_aug with the state carried into this tile
                auto inter = [&]() {
#pragma unroll 2
                    for (int k = 0; k < D; k += 4) {
                        const float av = sm.Q[(16 * qb + c16) * RX + k + g];
#pragma unroll
                        for (int j = 0; j < NBN; ++j)
                            acc[j] = mma4(av, sm.S[(k + g) * RV + 16 * (NB0 + j) + c16], acc[j]);
                    }
                };
                if constexpr (RET) {
                    // retention reads the carried state first, lambda^(i+1) for tile row i
                    inter();
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float r = sm.DW[16 * qb + 4 * g + e + 1];
#pragma unroll
                        for (int j = 0; j < NBN; ++j) acc[j][e] *= r;
                    }
                }
                if constexpr (MODE == kModeCausal) {
                    // (P (.) M) V_aug for key blocks tb <= qb: P^T tile (keys x queries)
#pragma unroll
                    for (int tb = 0; tb < 2; ++tb) {
                        if (tb > qb) continue;
                        f32x4_t pt = z4(), pu = z4();  // two chains over the features
#pragma unroll 8
                        for (int k = 0; k < D; k += 8) {
                            // A[t][f] = phi(K), B[f][q] = phi(Q)^T, both from their row-major tiles
                            pt = mma4(sm.K[(16 * tb + c16) * RX + k + g], sm.Q[(16 * qb + c16) * RX + k + g], pt);
                            pu = mma4(sm.K[(16 * tb + c16) * RX + k + 4 + g], sm.Q[(16 * qb + c16) * RX + k + 4 + g], pu);
                        }
                        pt += pu;
                        if constexpr (RET) {  // lambda^(query - key), 0 above the diagonal
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int d = 16 * (qb - tb) + c16 - 4 * g - e;
                                pt[e] = d >= 0 ? pt[e] * sm.DW[d] : 0.f;
                            }
                        } else if (tb == qb) {  // diagonal: key 4g + e <= query c16
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (4 * g + e > c16) pt[e] = 0.f;
                        }
                        // value product, k-slot e of lane group g <-> key 16 tb + 4g + e
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int t = 16 * tb + 4 * g + e;
#pragma unroll
                            for (int j = 0; j < NBN; ++j)
                                acc[j] = mma4(pt[e], sm.V[t * RV + 16 * (NB0 + j) + c16], acc[j]);
                        }
                    }
                }
                const int rows = min(kFT, t_end - t0);
                float rden[4] = {1.f, 1.f, 1.f, 1.f};
                if constexpr (!RET) {
                    inter();
                    // the normaliser (column D: the last block of the second value half, column 0)
                    if constexpr (NB0 != 0) {
                        if (c16 == 0)
#pragma unroll
                            for (int e = 0; e < 4; ++e) sm.DEN[qb][4 * g + e] = acc[NBN - 1][e];
                    }
                    __syncthreads();
#pragma unroll
                    for (int e = 0; e < 4; ++e) rden[e] = 1.0f / sm.DEN[qb][4 * g + e];
                }
#pragma unroll
                for (int j = 0; j < NBN; ++j) {
                    const int col = 16 * (NB0 + j) + c16;
                    if (col < D)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int r = 16 * qb + 4 * g + e;
                            if (r < rows) Os[(size_t)(t0 + r) * D + col] = acc[j][e] * rden[e];
                        }
                }
            };
            if (w < 2)
                outputs(std::integral_constant<int, 0>{});
            else
                outputs(std::integral_constant<int, 1>{});
        }

        if constexpr (NEED_K) {
            // S_aug += phi(K)^T V_aug over the tile's 32 tokens (retention:
            // S = lambda^L S + sum_t lambda^(L-1-t) k_t v_t^T over its L tokens)
            const int L = min(kFT, t_end - t0);
            if constexpr (RET) {
                const float carry = sm.DW[L];
#pragma unroll
                for (int q = 0; q < FBW; ++q)
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) S[q][nb] *= carry;
            }
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int f0 = (D / 4) * w + 16 * q;
#pragma unroll 2
                for (int t = 0; t < kFT; t += 4) {
                    float av = sm.K[(t + g) * RX + f0 + c16];  // A[f][t] = phi(K)^T
                    if constexpr (RET) av *= t + g < L ? sm.DW[L - 1 - t - g] : 0.f;
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) S[q][nb] = mma4(av, sm.V[(t + g) * RV + 16 * nb + c16], S[q][nb]);
                }
            }
            if constexpr (OUT) {
                __syncthreads();  // every wave is done reading the image of the old state
                put_image();
            }
        }
    }

    // ---- final state of the range
    if (NEED_K && a.st.S_dst) {
        float *Sd = a.st.S_dst + bh * a.st.dst_slice + seg * a.st.dst_seg;
        float *zd = a.st.z_dst ? a.st.z_dst + bh * a.st.zdst_slice + seg * a.st.zdst_seg : nullptr;
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = (D / 4) * w + 16 * q + 4 * g + e, j = 16 * nb + c16;
                    if (j < D) Sd[(size_t)f * D + j] = S[q][nb][e];
                    else if (j == D && zd) zd[f] = S[q][nb][e];
                }
    }
}

template <int D, bool RET>
hipError_t launch_d(const FwdArgs &a, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)((size_t)a.sh.BH * a.sg.P)), block(kFThr);
    switch (a.mode) {
        case kModeState: return launch_kernel_ev(k_f32mma<D, kModeState, RET>, grid, block, 0, st, ev, a);
        case kModeCausal: return launch_kernel_ev(k_f32mma<D, kModeCausal, RET>, grid, block, 0, st, ev, a);
        case kModeRead:
            if constexpr (!RET) return launch_kernel_ev(k_f32mma<D, kModeRead, RET>, grid, block, 0, st, ev, a);
            return hipErrorNotSupported;  // retention is causal only
        default: return hipErrorNotSupported;
    }
}

}  // namespace

bool f32mma_supported(const Shape &sh) {
    const bool map = (sh.phi == kElu1 && sh.ret == 0) || (sh.phi == kIdentity && sh.ret != 0);
    return sh.dtype == kF32 && map && sh.dk == sh.dv && (sh.dk == 64 || sh.dk == 128);
}

hipError_t launch_f32mma(const FwdArgs &a, hipStream_t st, KEvents ev) {
    if (!f32mma_supported(a.sh)) return hipErrorNotSupported;
    if (a.sh.ret) return a.sh.dk == 64 ? launch_d<64, true>(a, st, ev) : launch_d<128, true>(a, st, ev);
    return a.sh.dk == 64 ? launch_d<64, false>(a, st, ev) : launch_d<128, false>(a, st, ev);
}

}  // namespace la
