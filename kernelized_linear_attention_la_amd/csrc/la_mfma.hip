// bf16 matrix-core (MFMA) chunkwise kernels for gfx950.
//
// Chunkwise causal linear attention ("Linear Attention", chunkwise parallel
// form; "Story of Attention Part 5", section 6 blockwise split with decay 1,
// plus the normaliser of section 1a).  One workgroup owns one (slice,
// segment) and walks its chunks of C tokens; wave w owns query rows
// 16w..16w+15 of every chunk (C/16 waves).  Per chunk:
//   P^T  = phi(K_c) phi(Q_c)^T          (scores, computed transposed)
//   O    = [(P (.) M) V_aug + phi(Q_c) S_aug]  -> num | den,  O = num / den
//   S_aug += phi(K_c)^T V_aug
// V_aug = [V | 1 | 0...] and S_aug = [S | z | 0...] carry the normaliser z as
// one extra value column (padded to a 16-wide block), so the denominators
// come out of the same matrix products as the numerators.
//
// All products are v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  For
// that instruction lane l supplies A[l%16][k-slots 8(l/16)..8(l/16)+7],
// B[k-slots][l%16] and receives D[4(l/16)+e][l%16], e = 0..3.  Every LDS
// tile is stored pre-swizzled as the exact 16 bytes a lane feeds to the
// instruction, so each operand fetch is one conflict-free 128-bit LDS read.
// Contractions over tokens use the slot order
//     slot 8g+e  <->  token 16*(e/4) + 4g + (e%4)   inside each 32-token block,
// which is the order in which a lane already holds the scores of two
// consecutive 16x16 P^T accumulator tiles: P converts to an A operand in
// registers, without a trip through LDS.
//
// The state S_aug (d' x (d_v+16), fp32) lives in the accumulators of the
// waves that own its 16-row feature blocks for the whole segment; a bf16
// copy in LDS feeds the next chunk's phi(Q) S read.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

union Op8 {
    bf16x8_t v;
    uint4 u;
    uint2 q[2];
    uint16_t h[8];
};

__device__ __forceinline__ f32x4 mfma(const Op8 &a, const Op8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ uint32_t pack_bf16x2(uint16_t lo, uint16_t hi) {
    return static_cast<uint32_t>(lo) | (static_cast<uint32_t>(hi) << 16);
}

__device__ __forceinline__ uint2 pack4(float a, float b, float c, float d) {
    return make_uint2(pack_bf16x2(f32_to_bf16(a), f32_to_bf16(b)), pack_bf16x2(f32_to_bf16(c), f32_to_bf16(d)));
}

// slot (0..31) of index x (0..31) inside a 32-block, for the token order above
__device__ __forceinline__ int slot_of(int x) { return 8 * ((x >> 2) & 3) + 4 * (x >> 4) + (x & 3); }

template <int DK, int DV, int C, int PHI>
struct Cfg {
    static constexpr int NW = C / 16;            // waves
    static constexpr int THREADS = 64 * NW;
    static constexpr int DP = PHI == kFavor ? 256 : DK;  // feature dimension
    static constexpr int M = PHI == kFavor ? 256 : 0;
    static constexpr int NJ = DV / 16 + 1;       // value column blocks incl. the normaliser block
    static constexpr int KBT = C / 32;           // 32-token k-blocks per chunk
    static constexpr int KBF = DP / 32;          // 32-feature k-blocks
    static constexpr int KBD = DK / 32;          // 32-wide k-blocks of the raw input (FAVOR projection)
    static constexpr int FB = DP / 16;           // 16-row feature blocks of the state
    static constexpr int FBW = (FB + NW - 1) / NW;  // feature blocks owned per wave
    // FAVOR+ feature slots follow the token order (they come out of
    // accumulator tiles); ELU+1 features keep natural order (16-byte loads).
    static constexpr bool FEAT_PI = PHI == kFavor;
};

// LDS image, every entry one lane's 16-byte operand.
template <int DK, int DV, int C, int PHI>
struct Smem {
    using G = Cfg<DK, DV, C, PHI>;
    static constexpr bool F = PHI == kFavor;
    uint4 KA[C / 16][G::KBF][64];                       // phi(K) rows: A operand of P^T
    uint4 KTA[F ? 1 : G::FB][F ? 1 : G::KBT][F ? 1 : 64];  // phi(K)^T: A operand of the state update (ELU+1)
    uint4 VTB[G::NJ][G::KBT][64];                       // V_aug: B operand of P V and of the state update
    uint4 STB[G::NJ][G::KBF][64];                       // bf16 S_aug: B operand of phi(Q) S
    uint4 WA[F ? 2 : 1][F ? G::M / 16 : 1][F ? G::KBD : 1][F ? 64 : 1];  // FAVOR+ W rows, bf16 hi and lo parts
    uint4 XA[F ? C / 16 : 1][F ? G::KBD : 1][F ? 64 : 1];     // FAVOR+ raw K rows (bf16)
    float ksq[F ? C : 1];                               // FAVOR+ |k_t|^2
};

// Map an fp32 state row block (16 features) x column block to the B-operand
// image of S_aug: lane l holds S[16fb + 4g + e][16nb + l%16], e = 0..3.
template <typename G>
__device__ __forceinline__ void put_state_block(uint4 (*STB)[G::KBF][64], int fb, int nb, int lane, f32x4 s) {
    const int g = lane >> 4, c = lane & 15;
    uint2 v = pack4(s[0], s[1], s[2], s[3]);
    if (G::FEAT_PI) {
        reinterpret_cast<uint2 *>(&STB[nb][fb >> 1][lane])[fb & 1] = v;
    } else {
        const int x = 16 * (fb & 1) + 4 * g;  // natural order: slot = x
        reinterpret_cast<uint2 *>(&STB[nb][fb >> 1][c + 16 * (x >> 3)])[(x >> 2) & 1] = v;
    }
}

template <int DK, int DV, int C, int PHI, int MODE>
__global__ __launch_bounds__(C / 16 * 64) void k_mfma(FwdArgs a) {
    using G = Cfg<DK, DV, C, PHI>;
    using T = uint16_t;
    __shared__ Smem<DK, DV, C, PHI> sm;
    constexpr int NW = G::NW, NJ = G::NJ, KBT = G::KBT, KBF = G::KBF, FB = G::FB, FBW = G::FBW;
    constexpr bool DO_OUT = MODE != kModeState;
    constexpr bool DO_STATE = MODE != kModeRead;
    constexpr bool DO_INTRA = MODE == kModeCausal;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15;

    const Segments sg = a.sg;
    const int N = a.sh.N;
    const int seg = blockIdx.x % sg.P;
    const int bh = blockIdx.x / sg.P;
    const int c_begin = seg * sg.seg_chunks;
    const int c_end = min(sg.n_chunks, c_begin + sg.seg_chunks);

    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * DK;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * DK;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * DV;
    T *Os = DO_OUT ? static_cast<T *>(a.O) + (size_t)bh * N * DV : nullptr;

    // ---- FAVOR+ projection rows into LDS, once per workgroup.  W is split as
    // W = W_hi + W_lo with both parts bf16 (W_lo = bf16(W - W_hi)); the
    // inputs are exact in bf16, so x . w_r = x . hi_r + x . lo_r is accurate to
    // about 2^-16 relative, where a single bf16 W would shift every exponent
    // of the feature map by ~2^-9 |w_r| |x|.
    if constexpr (PHI == kFavor) {
        for (int u = tid; u < G::M * DK / 8; u += G::THREADS) {
            const int r = u / (DK / 8), d8 = u % (DK / 8);
            const float *src = a.sh.W + (size_t)r * DK + 8 * d8;
            float4 w0 = *reinterpret_cast<const float4 *>(src);
            float4 w1 = *reinterpret_cast<const float4 *>(src + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
            Op8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi.h[e] = f32_to_bf16(wv[e]);
                lo.h[e] = f32_to_bf16(wv[e] - bf16_to_f32(hi.h[e]));
            }
            const int l = (r & 15) + 16 * (d8 & 3);
            sm.WA[0][r >> 4][d8 >> 2][l] = hi.u;
            sm.WA[1][r >> 4][d8 >> 2][l] = lo.u;
        }
    }

    // ---- starting state into the owners' accumulators (+ bf16 image)
    f32x4 S[FBW][NJ];
    {
        const float *Ssrc = a.st.S_src ? a.st.S_src + bh * a.st.src_slice + seg * a.st.src_seg : nullptr;
        const float *zsrc = a.st.z_src ? a.st.z_src + bh * a.st.zsrc_slice + seg * a.st.zsrc_seg : nullptr;
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int fb = w + NW * q;
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) {
                f32x4 v = zero4();
                if (fb < FB && Ssrc) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 16 * fb + 4 * g + e, j = 16 * nb + c16;
                        v[e] = j < DV ? Ssrc[(size_t)f * DV + j] : (j == DV ? zsrc[f] : 0.f);
                    }
                }
                S[q][nb] = v;
                if (DO_OUT && fb < FB) put_state_block<G>(sm.STB, fb, nb, lane, v);
            }
        }
    }
    // normaliser block of V_aug: column d_v is 1 for every token (fixed up
    // per chunk for tokens past the end), the other 15 columns are 0
    if constexpr (DO_OUT || DO_STATE) {
        for (int u = tid; u < KBT * 64; u += G::THREADS) {
            const int l = u & 63;
            const uint32_t one2 = (l & 15) == 0 ? 0x3f803f80u : 0u;
            sm.VTB[NJ - 1][u >> 6][l] = make_uint4(one2, one2, one2, one2);
        }
    }

    const float inv_sqrt_m = PHI == kFavor ? 1.0f / 16.0f : 1.0f;  // m = 256
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        // ---------------- stage K_c, V_c into LDS
        if constexpr (MODE != kModeRead) {
            constexpr int UK = (C / 4) * (DK / 8);  // 4-token x 8-column units
            constexpr int UV = (C / 4) * (DV / 8);
            for (int u = tid; u < UK + UV; u += G::THREADS) {
                const bool isK = u < UK;
                const int uu = isK ? u : u - UK;
                const int W8 = isK ? DK / 8 : DV / 8;
                const int t4 = 4 * (uu / W8), c8 = uu % W8;
                const int D = isK ? DK : DV;
                const T *src = isK ? Ks : Vs;
                Op8 raw[4];
                bool valid[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    valid[r] = t0 + t4 + r < N;
                    raw[r].u = valid[r] ? *reinterpret_cast<const uint4 *>(src + (size_t)(t0 + t4 + r) * D + 8 * c8)
                                        : make_uint4(0, 0, 0, 0);
                }
                const int x = t4 & 31;                       // token offset inside its 32-block
                const int gt = (x >> 2) & 3, ht = x >> 4;    // slot group and half
                if (isK) {
                    if constexpr (PHI == kElu1) {
                        Op8 ph[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                ph[r].h[e] = valid[r] ? f32_to_bf16(elu1_fast(bf16_to_f32(raw[r].h[e]))) : 0;
                        if (DO_INTRA) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const int j = t4 + r;
                                sm.KA[j >> 4][c8 >> 2][(j & 15) + 16 * (c8 & 3)] = ph[r].u;
                            }
                        }
                        if (DO_STATE) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const int f = 8 * c8 + e;
                                uint2 v = make_uint2(pack_bf16x2(ph[0].h[e], ph[1].h[e]),
                                                     pack_bf16x2(ph[2].h[e], ph[3].h[e]));
                                reinterpret_cast<uint2 *>(&sm.KTA[f >> 4][t4 >> 5][(f & 15) + 16 * gt])[ht] = v;
                            }
                        }
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int j = t4 + r;
                            sm.XA[j >> 4][c8 >> 2][(j & 15) + 16 * (c8 & 3)] = raw[r].u;
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int j = 8 * c8 + e;
                        uint2 v = make_uint2(pack_bf16x2(raw[0].h[e], raw[1].h[e]), pack_bf16x2(raw[2].h[e], raw[3].h[e]));
                        reinterpret_cast<uint2 *>(&sm.VTB[j >> 4][t4 >> 5][(j & 15) + 16 * gt])[ht] = v;
                    }
                    if (c8 == 0) {  // normaliser column: 1 for valid tokens, 0 past the end
                        uint2 v = make_uint2(pack_bf16x2(valid[0] ? 0x3f80 : 0, valid[1] ? 0x3f80 : 0),
                                             pack_bf16x2(valid[2] ? 0x3f80 : 0, valid[3] ? 0x3f80 : 0));
                        reinterpret_cast<uint2 *>(&sm.VTB[NJ - 1][t4 >> 5][16 * gt])[ht] = v;
                    }
                }
            }
        }
        // ---------------- this wave's query rows (ELU+1: straight from HBM)
        const int row = 16 * w + c16;             // query row inside the chunk
        const bool qvalid = t0 + row < N;
        Op8 phq[KBF];
        if constexpr (DO_OUT && PHI == kElu1) {
#pragma unroll
            for (int kb = 0; kb < KBF; ++kb) {
                Op8 raw;
                raw.u = qvalid ? *reinterpret_cast<const uint4 *>(Qs + (size_t)(t0 + row) * DK + 32 * kb + 8 * g)
                               : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 8; ++e) phq[kb].h[e] = qvalid ? f32_to_bf16(elu1_fast(bf16_to_f32(raw.h[e]))) : 0;
            }
        }
        __syncthreads();

        // ---------------- FAVOR+: feature maps through projections on the matrix cores
        Op8 kta[FBW][KBT];  // this wave's phi(K)^T operands (FAVOR+)
        if constexpr (PHI == kFavor) {
            if constexpr (DO_OUT) {
                // query rows: U^T = W Q^T for this wave's 16 rows, |q|^2 from the operand lanes
                Op8 xq[G::KBD];
                float sq = 0.f;
#pragma unroll
                for (int kb = 0; kb < G::KBD; ++kb) {
                    xq[kb].u = qvalid ? *reinterpret_cast<const uint4 *>(Qs + (size_t)(t0 + row) * DK + 32 * kb + 8 * g)
                                      : make_uint4(0, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = bf16_to_f32(xq[kb].h[e]);
                        sq += x * x;
                    }
                }
                sq += __shfl_xor(sq, 16, 64);
                sq += __shfl_xor(sq, 32, 64);
#pragma unroll
                for (int kf = 0; kf < KBF; ++kf) {
                    f32x4 u0 = zero4(), u1 = zero4();
#pragma unroll
                    for (int kb = 0; kb < G::KBD; ++kb) {
#pragma unroll
                        for (int part = 0; part < 2; ++part) {
                            Op8 w0, w1;
                            w0.u = sm.WA[part][2 * kf][kb][lane];
                            w1.u = sm.WA[part][2 * kf + 1][kb][lane];
                            u0 = mfma(w0, xq[kb], u0);
                            u1 = mfma(w1, xq[kb], u1);
                        }
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        phq[kf].h[e] = f32_to_bf16(__expf(u0[e] - 0.5f * sq) * inv_sqrt_m);
                        phq[kf].h[4 + e] = f32_to_bf16(__expf(u1[e] - 0.5f * sq) * inv_sqrt_m);
                    }
                }
            }
            if constexpr (MODE != kModeRead) {
                // key rows of token block w: U^T = W K^T -> A operand of P^T; and |k|^2
                const int tb = w;
                Op8 xk[G::KBD];
                float sq = 0.f;
#pragma unroll
                for (int kb = 0; kb < G::KBD; ++kb) {
                    xk[kb].u = sm.XA[tb][kb][lane];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = bf16_to_f32(xk[kb].h[e]);
                        sq += x * x;
                    }
                }
                sq += __shfl_xor(sq, 16, 64);
                sq += __shfl_xor(sq, 32, 64);
                const bool kvalid = t0 + 16 * tb + c16 < N;
                if (g == 0) sm.ksq[16 * tb + c16] = sq;
                if constexpr (DO_INTRA) {
#pragma unroll
                    for (int kf = 0; kf < KBF; ++kf) {
                        f32x4 u0 = zero4(), u1 = zero4();
#pragma unroll
                        for (int kb = 0; kb < G::KBD; ++kb) {
#pragma unroll
                            for (int part = 0; part < 2; ++part) {
                                Op8 w0, w1;
                                w0.u = sm.WA[part][2 * kf][kb][lane];
                                w1.u = sm.WA[part][2 * kf + 1][kb][lane];
                                u0 = mfma(w0, xk[kb], u0);
                                u1 = mfma(w1, xk[kb], u1);
                            }
                        }
                        Op8 o;
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            o.h[e] = kvalid ? f32_to_bf16(__expf(u0[e] - 0.5f * sq) * inv_sqrt_m) : 0;
                            o.h[4 + e] = kvalid ? f32_to_bf16(__expf(u1[e] - 0.5f * sq) * inv_sqrt_m) : 0;
                        }
                        sm.KA[tb][kf][lane] = o.u;
                    }
                }
            }
            __syncthreads();
            if constexpr (DO_STATE) {
                // phi(K)^T for the feature blocks this wave owns: U = K W^T,
                // accumulator rows are tokens in slot order -> A operands
#pragma unroll
                for (int q = 0; q < FBW; ++q) {
                    const int fb = w + NW * q;
#pragma unroll
                    for (int kt = 0; kt < KBT; ++kt) {
                        f32x4 u0 = zero4(), u1 = zero4();
#pragma unroll
                        for (int kb = 0; kb < G::KBD; ++kb) {
                            Op8 x0, x1;
                            x0.u = sm.XA[2 * kt][kb][lane];
                            x1.u = sm.XA[2 * kt + 1][kb][lane];
#pragma unroll
                            for (int part = 0; part < 2; ++part) {
                                Op8 wb;
                                wb.u = sm.WA[part][fb][kb][lane];
                                u0 = mfma(x0, wb, u0);
                                u1 = mfma(x1, wb, u1);
                            }
                        }
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int ta = 32 * kt + 4 * g + e, tb2 = ta + 16;
                            kta[q][kt].h[e] =
                                t0 + ta < N ? f32_to_bf16(__expf(u0[e] - 0.5f * sm.ksq[ta]) * inv_sqrt_m) : 0;
                            kta[q][kt].h[4 + e] =
                                t0 + tb2 < N ? f32_to_bf16(__expf(u1[e] - 0.5f * sm.ksq[tb2]) * inv_sqrt_m) : 0;
                        }
                    }
                }
            }
        }

        // ---------------- outputs of this wave's 16 query rows
        if constexpr (DO_OUT) {
            f32x4 acc[NJ];
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) acc[nb] = zero4();
            if constexpr (DO_INTRA) {
                // (P (.) M) V_aug over the key blocks up to the diagonal
#pragma unroll
                for (int kt = 0; kt < KBT; ++kt) {
                    if (2 * kt <= w) {
                        f32x4 p[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const int jb = 2 * kt + h;
                            p[h] = zero4();
                            if (jb <= w) {
#pragma unroll
                                for (int kf = 0; kf < KBF; ++kf) {
                                    Op8 ka;
                                    ka.u = sm.KA[jb][kf][lane];
                                    p[h] = mfma(ka, phq[kf], p[h]);
                                }
                                if (jb == w) {  // causal mask on the diagonal block: key 4g+e <= query c16
#pragma unroll
                                    for (int e = 0; e < 4; ++e)
                                        if (4 * g + e > c16) p[h][e] = 0.f;
                                }
                            }
                        }
                        Op8 pa;
                        pa.q[0] = pack4(p[0][0], p[0][1], p[0][2], p[0][3]);
                        pa.q[1] = pack4(p[1][0], p[1][1], p[1][2], p[1][3]);
#pragma unroll
                        for (int nb = 0; nb < NJ; ++nb) {
                            Op8 vb;
                            vb.u = sm.VTB[nb][kt][lane];
                            acc[nb] = mfma(pa, vb, acc[nb]);
                        }
                    }
                }
            }
            // phi(Q) S_aug with the state carried into this chunk
#pragma unroll
            for (int kf = 0; kf < KBF; ++kf) {
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) {
                    Op8 sb;
                    sb.u = sm.STB[nb][kf][lane];
                    acc[nb] = mfma(phq[kf], sb, acc[nb]);
                }
            }
            // epilogue: divide by the normaliser column, round, store
            float rden[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rden[e] = 1.0f / __shfl(acc[NJ - 1][e], lane & 48, 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int orow = 16 * w + 4 * g + e;
                if (t0 + orow < N) {
                    T *dst = Os + (size_t)(t0 + orow) * DV + c16;
#pragma unroll
                    for (int nb = 0; nb < NJ - 1; ++nb) dst[16 * nb] = f32_to_bf16(acc[nb][e] * rden[e]);
                }
            }
        }

        // ---------------- state update S_aug += phi(K_c)^T V_aug
        if constexpr (DO_STATE) {
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB) {
#pragma unroll
                    for (int kt = 0; kt < KBT; ++kt) {
                        Op8 ka;
                        if constexpr (PHI == kFavor) ka = kta[q][kt];
                        else ka.u = sm.KTA[fb][kt][lane];
#pragma unroll
                        for (int nb = 0; nb < NJ; ++nb) {
                            Op8 vb;
                            vb.u = sm.VTB[nb][kt][lane];
                            S[q][nb] = mfma(ka, vb, S[q][nb]);
                        }
                    }
                }
            }
        }
        if constexpr (MODE == kModeCausal) {
            __syncthreads();  // every wave is done reading this chunk's tiles and the old state image
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB) {
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) put_state_block<G>(sm.STB, fb, nb, lane, S[q][nb]);
                }
            }
        } else if constexpr (MODE == kModeState) {
            __syncthreads();  // tiles are rewritten by the next chunk
        } else {
            __syncthreads();
        }
    }

    // ---- final state of the range
    if (DO_STATE && a.st.S_dst) {
        float *Sd = a.st.S_dst + bh * a.st.dst_slice + seg * a.st.dst_seg;
        float *zd = a.st.z_dst + bh * a.st.zdst_slice + seg * a.st.zdst_seg;
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int fb = w + NW * q;
            if (fb < FB) {
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 16 * fb + 4 * g + e, j = 16 * nb + c16;
                        if (j < DV) Sd[(size_t)f * DV + j] = S[q][nb][e];
                        else if (j == DV) zd[f] = S[q][nb][e];
                    }
                }
            }
        }
    }
}

template <int DK, int DV, int C, int PHI>
hipError_t launch_variant(const FwdArgs &a, hipStream_t st) {
    const dim3 grid((unsigned)((size_t)a.sh.BH * a.sg.P)), block(C / 16 * 64);
    switch (a.mode) {
        case kModeState: hipLaunchKernelGGL((k_mfma<DK, DV, C, PHI, kModeState>), grid, block, 0, st, a); break;
        case kModeCausal: hipLaunchKernelGGL((k_mfma<DK, DV, C, PHI, kModeCausal>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((k_mfma<DK, DV, C, PHI, kModeRead>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace

bool mfma_supported(const Shape &sh, int chunk) {
    if (sh.dtype != kBF16) return false;
    if (sh.phi == kElu1)
        return ((sh.dk == 64 && sh.dv == 64) || (sh.dk == 128 && sh.dv == 128)) && (chunk == 64 || chunk == 128);
    return sh.dk == 64 && sh.dv == 64 && sh.m == 256 && chunk == 64;
}

hipError_t launch_mfma(const FwdArgs &a, hipStream_t st) {
    const Shape &s = a.sh;
    const int C = a.sg.chunk;
    if (!mfma_supported(s, C)) return hipErrorNotSupported;
    if (s.phi == kFavor) return launch_variant<64, 64, 64, kFavor>(a, st);
    if (s.dk == 64) return C == 64 ? launch_variant<64, 64, 64, kElu1>(a, st) : launch_variant<64, 64, 128, kElu1>(a, st);
    return C == 64 ? launch_variant<128, 128, 64, kElu1>(a, st) : launch_variant<128, 128, 128, kElu1>(a, st);
}

}  // namespace la
