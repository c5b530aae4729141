// Backward of the causal normalised form on the matrix cores: ELU+1,
// d_k = d_v = D, bf16 or fp32 storage, D = 64 on 64-token tiles and D = 128 on
// 32-token tiles (the derivation and the fp32-FMA kernels are in
// la_backward.hip; this file runs the same chunked algebra on the matrix
// cores; the chunkwise form gives the same gradients for every chunk length,
// so a D = 128 call asking for 64- or 128-token chunks runs on 32-token tiles).
//
// The products stay fp32-class throughout: the normalised backward cancels
// (g_i . v_j + h_i = g_i . (v_j - o_i), and o_i, h_i come from the recomputed
// forward), so operands rounded once to bf16 lose several percent of the
// gradient.  fp32 storage runs v_mfma_f32_16x16x4_f32 on fp32 operands; bf16
// storage splits each fp32 operand into bf16 hi and lo parts at the read and
// runs v_mfma_f32_16x16x32_bf16 passes (hi hi + hi lo + lo hi; the lo pass of
// an operand that is exact in bf16 is skipped: V_aug, and the dO columns of
// G'_aug = [dO | -(dO . o)], which bf16 storage keeps in place of G_aug with
// 1/den applied outside the products), about 2^-16 relative.  Every tile has
// one row-major fp32 copy in LDS, read in either orientation: along a row as
// aligned 16-byte pieces, down a column element by element, with the k
// assignment of each instruction chosen so that both kinds of read are free
// of LDS bank conflicts at the 4 mod 16 row strides.
// Per chunk the tiles are phi(Q), phi(K), [V | 1 | 0], G_aug, the carried
// state image and a score tile; value-column widths are padded to D + 4 for
// contractions and D + 16 (whole 16-column blocks) for outputs.
//
// Four waves.  The row products of a chunk (scores, num, dphi(Q); dphi(K),
// dV) are split over (16-row block, column split): with 64-token tiles each
// wave owns one row block and every column, with 32-token tiles the two
// waves of a row block share its columns and exchange the row statistics of
// G_aug (normaliser, dO . o) through LDS.  Wave w also owns feature rows
// 16 (4q + w) .. +15 of the carried states (S_aug, U in the dQ pass; R_aug in
// the dK/dV pass), kept in fp32 accumulators and mirrored into LDS for the
// products that read them.
#include <type_traits>

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

constexpr int kNW = 4;  // waves
constexpr int kThreads = 64 * kNW;

template <int D, int C>
struct BCfg {
    static constexpr int RB = C / 16;               // 16-row blocks of a tile
    static constexpr int CS = kNW / RB;             // waves sharing a row block (column splits)
    static constexpr int VK = D + 4;                // value columns in contractions (v | 1 | 0 0 0)
    static constexpr int NVB = D / 16 + 1;          // 16-column blocks of [v | 1 | 0..] in outputs
    static constexpr int NDB = D / 16;              // 16-column blocks of d-wide outputs
    static constexpr int RX = D + 4;                // row stride of the phi tiles (floats)
    static constexpr int RV = 16 * NVB + 4;         // row stride of value-wide tiles
    static constexpr int RW = C + 4;                // row stride of the score tile
    static constexpr int FBW = D / 16 / kNW;        // 16-row feature blocks of a carried state per wave
    static constexpr int NSB = RB / CS;             // 16-key score blocks per wave
    static constexpr int NDW = NDB / CS;            // d-wide output blocks per wave
    static constexpr int NV0 = (NVB + CS - 1) / CS; // value blocks of split 0 (split 1: the rest)
    static constexpr bool STAGE = RW >= D;          // d-wide rows leave through the score tile
    static_assert(RB * CS == kNW && RB % CS == 0 && NDB % CS == 0 && FBW >= 1, "wave split");
    static_assert(CS <= 2 && (!STAGE || CS == 1), "one or two column splits");
};

template <int D, int C>
struct alignas(16) BTiles {  // every row stride and tile size a multiple of 4 floats
    using B = BCfg<D, C>;
    float P[C * B::RX];    // phi(Q) rows [token][feature]
    float K[C * B::RX];    // phi(K) rows
    float V[C * B::RV];    // [v | 1 | 0] rows
    float G[C * B::RV];    // rows [token][value column]: bf16 storage G'_aug = [dO | -(dO . o) | 0]
                           // (G_aug = G'_aug / den), fp32 storage G_aug
    float S[D * B::RV];    // carried state, rows [feature][value column]
    float W[C * B::RW];    // masked scores of the tile
    float DEN[C];          // normaliser of each query row (dQ pass)
    float DOT[B::CS][C];   // dO . num of each query row over one column split
    float RDEN[C];         // bf16 storage: 1 / normaliser of each query row (0 past the last row)
};

// v = row[k..k+3], row[k+16..k+19] from a 16-byte aligned LDS row, zeros past
// K (a multiple of 4, so each 4-wide piece lies wholly inside or outside)
template <int K>
__device__ __forceinline__ void row8(const float *row, int k, float (&v)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kh = k + 16 * h;
        const float4 x = *reinterpret_cast<const float4 *>(row + (K % 32 == 0 || kh < K ? kh : K - 4));
        const bool in = K % 32 == 0 || kh < K;
        v[4 * h + 0] = in ? x.x : 0.f;
        v[4 * h + 1] = in ? x.y : 0.f;
        v[4 * h + 2] = in ? x.z : 0.f;
        v[4 * h + 3] = in ? x.w : 0.f;
    }
}

// C[16 rows at m0][16 NB columns at n0] += A B over K (a multiple of 4).
// TA: A is given as its transpose (row-major [k][m]); TB: B as its transpose ([n][k]).
// bf16 matrix-instruction operands (v_mfma_f32_16x16x32_bf16: lane l supplies
// A[l%16][8(l/16)..+7] and B[8(l/16)..+7][l%16], and receives the same
// accumulator lanes as the fp32 instruction) and the split of fp32 values
// into bf16 hi and lo parts, x = hi + lo to about 2^-17 relative
typedef __bf16 wbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 wbf16x2 __attribute__((ext_vector_type(2)));
typedef float wf32x2 __attribute__((ext_vector_type(2)));
union W8 {
    wbf16x8 v;
    uint32_t u[4];
};
__device__ __forceinline__ uint32_t wbf2(float a, float b) {  // round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(wf32x2{a, b}, wbf16x2));
}
__device__ __forceinline__ void wsplit8(const float (&x)[8], W8 &hi, W8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t h = wbf2(x[2 * e], x[2 * e + 1]);
        hi.u[e] = h;
        lo.u[e] = wbf2(x[2 * e] - __uint_as_float(h << 16), x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
    }
}

// acc[j] (rows m0.., columns n0 + 16j..) += A B over K, A and B read from
// row-major fp32 LDS tiles, either transposed (TA: A stored [k][m]; TB: B
// stored [n][k]).  W3 (bf16 storage): three bf16 passes (hi hi + hi lo +
// lo hi) per 32-wide k step, k padded with zeros to a multiple of 32; the
// normalised backward cancels, so single bf16 operands would lose several
// percent, while the split keeps about 2^-16.  EA / EB: that operand is exact
// in bf16 (V_aug of bf16 storage), its lo part is zero and its pass is
// skipped (same result); AXK / BXK: the operand is exact for k < AXK / BXK
// (a k step wholly below skips the pass); BXN: B is exact in its columns
// below BXN (whole 16-column blocks).  Otherwise fp32 operands.  AS: A(m, k)
// is multiplied by as[k] as it is read.
template <int K, int NB, bool TA, bool TB, bool W3 = false, bool UNR = false, bool EA = false, bool EB = false,
          int AXK = 0, int BXK = 0, int BXN = 0, bool AS = false>
__device__ __forceinline__ void mm(const float *A, int lda, int m0, const float *B, int ldb, int n0, f32x4 (&acc)[NB],
                                   int lane, const float *as = nullptr) {
    static_assert(K % 4 == 0, "k in pieces of four");
    const int r = lane & 15, q = lane >> 4;
    if constexpr (!W3) {
        // whole 16-wide k groups: lane group q supplies k = kb + 4q + t in step
        // t, so a row-direction operand is one 16-byte piece and a column read
        // puts the four groups on rows 4 apart; a shorter tail takes k0 + q
        constexpr int K16 = K / 16 * 16;
#pragma unroll
        for (int kb = 0; kb < K16; kb += 16) {
            float a[4];
            if constexpr (TA) {
#pragma unroll
                for (int t = 0; t < 4; ++t) a[t] = A[(kb + 4 * q + t) * lda + m0 + r];
            } else {
                const float4 x = *reinterpret_cast<const float4 *>(A + (m0 + r) * lda + kb + 4 * q);
                a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
            }
            if constexpr (AS) {
                const float4 sc = *reinterpret_cast<const float4 *>(as + kb + 4 * q);
                a[0] *= sc.x; a[1] *= sc.y; a[2] *= sc.z; a[3] *= sc.w;
            }
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float b[4];
                if constexpr (TB) {
                    const float4 x = *reinterpret_cast<const float4 *>(B + (n0 + 16 * j + r) * ldb + kb + 4 * q);
                    b[0] = x.x; b[1] = x.y; b[2] = x.z; b[3] = x.w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) b[t] = B[(kb + 4 * q + t) * ldb + n0 + 16 * j + r];
                }
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc[j], 0, 0, 0);
            }
        }
#pragma unroll
        for (int k0 = K16; k0 < K; k0 += 4) {
            float a = TA ? A[(k0 + q) * lda + m0 + r] : A[(m0 + r) * lda + k0 + q];
            if constexpr (AS) a *= as[k0 + q];
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                const float b = TB ? B[(n0 + 16 * j + r) * ldb + k0 + q] : B[(k0 + q) * ldb + n0 + 16 * j + r];
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc[j], 0, 0, 0);
            }
        }
    } else {
        // UNR: the 32-wide steps unrolled (more loads in flight, more registers).
        // Lane group q supplies k = k0 + 4q + {0..3} and k0 + 16 + 4q + {0..3}
        // (the same permutation of k for A and B, so the sum is unchanged): a
        // read across rows then puts the four groups on rows 4 apart, which the
        // row strides (4 mod 16 floats) map to distinct LDS bank windows, and a
        // read along a row is still two 16-byte pieces.
#pragma unroll UNR ? 8 : 1
        for (int k0 = 0; k0 < K; k0 += 32) {
            float av[8];
            if constexpr (TA) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int k = k0 + 4 * q + (e & 3) + 16 * (e >> 2), kc = k < K ? k : K - 1;
                    const float v = A[kc * lda + m0 + r];
                    av[e] = k < K ? v : 0.f;
                }
            } else {
                row8<K>(A + (m0 + r) * lda, k0 + 4 * q, av);
            }
            if constexpr (AS) {
                float sv[8];
                row8<K>(as, k0 + 4 * q, sv);
#pragma unroll
                for (int e = 0; e < 8; ++e) av[e] *= sv[e];
            }
            const bool ax = EA || k0 + 32 <= AXK;  // A exact in bf16 over this k step
            W8 ah, al;
            wsplit8(av, ah, al);
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                float bv[8];
                if constexpr (TB) {
                    row8<K>(B + (n0 + 16 * j + r) * ldb, k0 + 4 * q, bv);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int k = k0 + 4 * q + (e & 3) + 16 * (e >> 2), kc = k < K ? k : K - 1;
                        const float v = B[kc * ldb + n0 + 16 * j + r];
                        bv[e] = k < K ? v : 0.f;
                    }
                }
                const bool bx = EB || k0 + 32 <= BXK || n0 + 16 * j + 16 <= BXN;  // B exact here
                W8 bh, bl;
                wsplit8(bv, bh, bl);
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah.v, bh.v, acc[j], 0, 0, 0);
                if (!bx) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah.v, bl.v, acc[j], 0, 0, 0);
                if (!ax) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al.v, bh.v, acc[j], 0, 0, 0);
            }
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

// eight consecutive stored values (16 bytes of bf16, 32 of fp32) as float4 pairs
__device__ __forceinline__ void load8(const uint16_t *p, float4 &a, float4 &b) {
    const uint4 x = *reinterpret_cast<const uint4 *>(p);
    a = make_float4(lo_bf16(x.x), hi_bf16(x.x), lo_bf16(x.y), hi_bf16(x.y));
    b = make_float4(lo_bf16(x.z), hi_bf16(x.z), lo_bf16(x.w), hi_bf16(x.w));
}
__device__ __forceinline__ void load8(const float *p, float4 &a, float4 &b) {
    a = *reinterpret_cast<const float4 *>(p);
    b = *reinterpret_cast<const float4 *>(p + 4);
}
__device__ __forceinline__ float load1(const uint16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ void store1(uint16_t *p, float v) { *p = f32_to_bf16(v); }
__device__ __forceinline__ void store1(float *p, float v) { *p = v; }
// eight consecutive values to storage (16 bytes of bf16, 32 of fp32)
__device__ __forceinline__ void store8(uint16_t *p, const float *s) {
    uint4 o;
    o.x = f32_to_bf16(s[0]) | (static_cast<uint32_t>(f32_to_bf16(s[1])) << 16);
    o.y = f32_to_bf16(s[2]) | (static_cast<uint32_t>(f32_to_bf16(s[3])) << 16);
    o.z = f32_to_bf16(s[4]) | (static_cast<uint32_t>(f32_to_bf16(s[5])) << 16);
    o.w = f32_to_bf16(s[6]) | (static_cast<uint32_t>(f32_to_bf16(s[7])) << 16);
    *reinterpret_cast<uint4 *>(p) = o;
}
__device__ __forceinline__ void store8(float *p, const float *s) {
    *reinterpret_cast<float4 *>(p) = make_float4(s[0], s[1], s[2], s[3]);
    *reinterpret_cast<float4 *>(p + 4) = make_float4(s[4], s[5], s[6], s[7]);
}

// Staging loads are unconditional (rows clamped to the tile's last valid
// row, zeros selected where the values are used) and a tile's pieces are all
// issued before the first is used: a load under a branch makes the compiler
// wait for every load in flight right after it, one memory round trip per
// piece.

// v where `in`, else zeros, per component (a select of whole float4 values
// can be lowered through scratch memory)
__device__ __forceinline__ float4 keep4(bool in, float4 v) {
    return make_float4(in ? v.x : 0.f, in ? v.y : 0.f, in ? v.z : 0.f, in ? v.w : 0.f);
}

// A tile's rows as 16-byte pieces in registers: loaded for the next chunk
// while the current one computes, written to LDS once its tiles are free.
template <int D, int C>
struct RowPieces {
    static constexpr int NI = C * D / 8 / kThreads;
    float4 a[NI], b[NI];
};
template <int D, int C, typename T>
__device__ __forceinline__ void load_rows(const T *X, int t0, int rows, RowPieces<D, C> &p, int tid) {
#pragma unroll
    for (int i = 0; i < RowPieces<D, C>::NI; ++i) {
        const int u = tid + i * kThreads, t = u / (D / 8), c8 = u % (D / 8);
        load8(&X[(size_t)(t0 + (t < rows ? t : 0)) * D + 8 * c8], p.a[i], p.b[i]);
    }
}
// phi(X) rows of one tile (rows past `rows` are zero)
template <int D, int C>
__device__ __forceinline__ void put_phi(const RowPieces<D, C> &p, int rows, float *R, int tid) {
    constexpr int RX = BCfg<D, C>::RX;
#pragma unroll
    for (int i = 0; i < RowPieces<D, C>::NI; ++i) {
        const int u = tid + i * kThreads, t = u / (D / 8), c8 = u % (D / 8);
        const bool in = t < rows;
        *reinterpret_cast<float4 *>(&R[t * RX + 8 * c8]) =
            keep4(in, make_float4(elu1(p.a[i].x), elu1(p.a[i].y), elu1(p.a[i].z), elu1(p.a[i].w)));
        *reinterpret_cast<float4 *>(&R[t * RX + 8 * c8 + 4]) =
            keep4(in, make_float4(elu1(p.b[i].x), elu1(p.b[i].y), elu1(p.b[i].z), elu1(p.b[i].w)));
    }
}
// [v | 1 | 0] rows of one tile (columns D..RV-1 written too)
template <int D, int C>
__device__ __forceinline__ void put_vaug(const RowPieces<D, C> &p, int rows, float *R, int tid) {
    constexpr int RV = BCfg<D, C>::RV;
#pragma unroll
    for (int i = 0; i < RowPieces<D, C>::NI; ++i) {
        const int u = tid + i * kThreads, t = u / (D / 8), c8 = u % (D / 8);
        const bool in = t < rows;
        *reinterpret_cast<float4 *>(&R[t * RV + 8 * c8]) = keep4(in, p.a[i]);
        *reinterpret_cast<float4 *>(&R[t * RV + 8 * c8 + 4]) = keep4(in, p.b[i]);
    }
    for (int u = tid; u < C * (RV - D); u += kThreads) {
        const int t = u / (RV - D), c = D + u % (RV - D);
        R[t * RV + c] = (c == D && t < rows) ? 1.f : 0.f;
    }
}
// G_aug rows (fp32 in the workspace, VK per token) of one tile
template <int D, int C>
struct GPieces {
    static constexpr int RV = BCfg<D, C>::RV, NU = C * RV / 4, NI = (NU + kThreads - 1) / kThreads;
    float4 x[NI];
};
template <int D, int C>
__device__ __forceinline__ void load_g(const float *Gw, int t0, int rows, GPieces<D, C> &p, int tid) {
    using G = GPieces<D, C>;
    constexpr int VK = BCfg<D, C>::VK;
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
        const int u = min(tid + i * kThreads, G::NU - 1), t = u / (G::RV / 4), c4 = u % (G::RV / 4);
        p.x[i] = *reinterpret_cast<const float4 *>(&Gw[(size_t)(t0 + (t < rows ? t : 0)) * VK + 4 * min(c4, VK / 4 - 1)]);
    }
}
// stored row (bf16 storage): [dO | -(dO . o) | den | 0 0]; the tile gets
// [dO | -(dO . o) | 0 0 0] and RDEN the reciprocal of den (0 past the last
// row).  fp32 storage stores G_aug, whose column D + 1 is zero: RDEN is then
// not read.
template <int D, int C>
__device__ __forceinline__ void put_g(const GPieces<D, C> &p, int rows, float *R, float *RDEN, int tid) {
    using G = GPieces<D, C>;
    constexpr int VK = BCfg<D, C>::VK;
#pragma unroll
    for (int i = 0; i < G::NI; ++i) {
        const int u = tid + i * kThreads, t = u / (G::RV / 4), c4 = u % (G::RV / 4);
        float4 x = keep4(t < rows && 4 * c4 < VK, p.x[i]);
        if (4 * c4 == D) {
            if (u < G::NU) RDEN[t] = t < rows ? 1.f / x.y : 0.f;
            x.y = 0.f;
        }
        if (u < G::NU) *reinterpret_cast<float4 *>(&R[t * G::RV + 4 * c4]) = x;
    }
}

// this wave's feature rows of a carried state into the LDS image
template <int D, int C>
__device__ __forceinline__ void put_state(const f32x4 (&S)[BCfg<D, C>::FBW][BCfg<D, C>::NVB], float *T, int w,
                                          int lane) {
    using B = BCfg<D, C>;
#pragma unroll
    for (int q = 0; q < B::FBW; ++q)
#pragma unroll
        for (int j = 0; j < B::NVB; ++j) put_rows(T, B::RV, 16 * (kNW * q + w), 16 * j, S[q][j], lane);
}

// Carried-state accumulators (feature row 16 (4q + w) + 4g + e, augmented
// column 16j + c16 <= D) += the sums of segments first, first + step, ..
// (count of them), added in that order; at(p, f, col) is a readable address
// for every column (columns past D are loaded and not added).  PB segments'
// loads are in flight at a time.
template <int D, int C, typename Acc, typename At>
__device__ __forceinline__ void add_segments(Acc &S, int first, int count, int step, At at, int w, int lane) {
    using B = BCfg<D, C>;
    constexpr int PER = B::FBW * B::NVB * 4, PB = PER * 8 <= 160 ? 8 : 160 / PER;
    const int g = lane >> 4, c16 = lane & 15;
    for (int i0 = 0; i0 < count; i0 += PB) {
        float v[PB][B::FBW][B::NVB][4];
#pragma unroll
        for (int b = 0; b < PB; ++b) {
            const int p = first + step * (i0 + b < count ? i0 + b : 0);
#pragma unroll
            for (int q = 0; q < B::FBW; ++q)
#pragma unroll
                for (int j = 0; j < B::NVB; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[b][q][j][e] = *at(p, 16 * (kNW * q + w) + 4 * g + e, 16 * j + c16);
        }
#pragma unroll
        for (int b = 0; b < PB; ++b)
            if (i0 + b < count)
#pragma unroll
                for (int q = 0; q < B::FBW; ++q)
#pragma unroll
                    for (int j = 0; j < B::NVB; ++j)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (16 * j + c16 <= D) S[q][j][e] += v[b][q][j][e];
    }
}

// 16 rows x D columns of T (rows m0..) -> rows of dst, 8 values per lane and step
template <int D, typename ST>
__device__ __forceinline__ void store_rows(const float *T, int ld, int m0, int rows, ST *dst, size_t row0, int lane) {
#pragma unroll
    for (int it = 0; it < 16 * D / 8 / 64; ++it) {
        const int idx = it * 64 + lane, r = idx / (D / 8), c8 = idx % (D / 8);
        if (m0 + r < rows) store8(&dst[(row0 + m0 + r) * D + 8 * c8], &T[(m0 + r) * ld + 8 * c8]);
    }
}

// accumulator blocks (rows m0 + 4g + e, columns n0 + 16 j + c16) -> rows of dst
template <int D, int NB, typename ST>
__device__ __forceinline__ void store_acc(const f32x4 (&v)[NB], int m0, int n0, int rows, ST *dst, size_t row0,
                                          int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = m0 + 4 * g + e;
            if (r < rows) store1(&dst[(row0 + r) * D + n0 + 16 * j + c], v[j][e]);
        }
}

// d-wide row blocks of this wave to dst: through the score tile (one column
// split: the wave's own rows of W) or straight from the accumulators
template <int D, int C, typename ST>
__device__ __forceinline__ void store_dwide(const f32x4 (&v)[BCfg<D, C>::NDW], float *W, int m0, int cs, int rows,
                                            ST *dst, size_t row0, int lane) {
    using B = BCfg<D, C>;
    if constexpr (B::STAGE) {
        wave_lds_sync();  // every lane has read this wave's rows of W
#pragma unroll
        for (int j = 0; j < B::NDW; ++j) put_rows(W, B::RW, m0, 16 * j, v[j], lane);
        wave_lds_sync();
        store_rows<D>(W, B::RW, m0, rows, dst, row0, lane);
    } else {
        store_acc<D, B::NDW>(v, m0, 16 * cs * B::NDW, rows, dst, row0, lane);
    }
}

// the row products of a row block are shared by its column splits
template <int CS>
__device__ __forceinline__ void row_sync() {
    if constexpr (CS == 1)
        wave_lds_sync();
    else
        block_sync_lds();
}

// ---------------------------------------------------------------------------
// dQ pass.  Tiles in order from the forward prefix [S | z] of the segment:
//   num_aug = (P (.) M) V_aug + phi(Q) S_aug          P = phi(Q) phi(K)^T
//   G_aug   = [dO / den | -(dO . o) / den | 0]
//   dphi(Q) = (A (.) M) phi(K) + G_aug S_aug^T        A = G_aug V_aug^T
//   dQ = dphi(Q) * elu'(q),  elu'(q) = min(phi(q), 1)
//   U      += phi(Q)^T G_aug    (segment sums for the reverse scan)
//   S_aug  += phi(K)^T V_aug
// ---------------------------------------------------------------------------
template <int D, int C, typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_dq_mfma(BwdMfmaArgs a) {
    using B = BCfg<D, C>;
    // bf16 storage: products in bf16 passes (two where V_aug is an operand),
    // the k steps unrolled; the tile holds G'_aug (GP), whose dO columns are
    // exact in bf16
    constexpr bool W3 = sizeof(T) == 2, UNR = true, GP = W3;
    constexpr int RX = B::RX, RV = B::RV, RW = B::RW, VK = B::VK, NVB = B::NVB, FBW = B::FBW, NSB = B::NSB,
                  NDW = B::NDW, CS = B::CS, RB = B::RB;
    __shared__ BTiles<D, C> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    // row block and column split of the row products (one split: the column
    // offsets stay compile-time constants)
    const int rb = CS == 1 ? w : w % RB, cs = CS == 1 ? 0 : w / RB;
    const int m0 = 16 * rb;
    const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
    const int N = a.N;
    const int c_begin = seg * a.seg_chunks, c_end = min(a.n_chunks, c_begin + a.seg_chunks);
    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * D;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * D;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * D;
    const T *dOs = static_cast<const T *>(a.dO) + (size_t)bh * N * D;
    T *dQs = static_cast<T *>(a.dQ) + (size_t)bh * N * D;
    float *Gw = a.G + (size_t)bh * N * VK;

    // carried state S_aug (feature rows 16 (4q + w) + 4g + e, value columns
    // 16j + c16) entering the segment: [S_in | z_in] (or zero) plus the
    // forward sums of segments 0 .. seg - 1, in that order; and U
    f32x4 S[FBW][NVB], U[FBW][NVB];
    {
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int j = 0; j < NVB; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = 16 * (kNW * q + w) + 4 * g + e, col = 16 * j + c16;
                    float s0 = 0.f;
                    if (a.S_in) {
                        const float x = col < D ? a.S_in[((size_t)bh * D + f) * D + col] : a.z_in[(size_t)bh * D + f];
                        s0 = col <= D ? x : 0.f;
                    }
                    S[q][j][e] = s0;
                }
                U[q][j] = zero4();
            }
        const float *Sg = a.Ssum + (size_t)bh * a.P * D * D, *zg = a.zsum + (size_t)bh * a.P * D;
        add_segments<D, C>(S, 0, seg, 1, [&](int p, int f, int col) {
            return col < D ? Sg + ((size_t)p * D + f) * D + col : zg + (size_t)p * D + f;
        }, w, lane);
    }
    put_state<D, C>(S, sm.S, w, lane);

    // the rows of chunk c are loaded during chunk c - 1 (the last chunk
    // re-reads itself: every load stays unconditional)
    RowPieces<D, C> xq, xk, xv;
    auto fetch = [&](int cc) {
        const int tt0 = cc * C, rr = min(C, N - tt0);
        load_rows<D, C>(Qs, tt0, rr, xq, tid);
        load_rows<D, C>(Ks, tt0, rr, xk, tid);
        load_rows<D, C>(Vs, tt0, rr, xv, tid);
    };
    fetch(c_begin);
    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C, rows = min(C, N - t0);
        block_sync_lds();  // the previous tile's tiles are consumed, the state image is complete
        put_phi<D, C>(xq, rows, sm.P, tid);
        put_phi<D, C>(xk, rows, sm.K, tid);
        put_vaug<D, C>(xv, rows, sm.V, tid);
        fetch(min(c + 1, c_end - 1));
        block_sync_lds();

        // scores P = phi(Q) phi(K)^T of this wave's key blocks, masked (key <= query)
        {
            f32x4 p[NSB];
#pragma unroll
            for (int j = 0; j < NSB; ++j) p[j] = zero4();
            mm<D, NSB, false, true, W3, UNR>(sm.P, RX, m0, sm.K, RX, 16 * cs * NSB, p, lane);
#pragma unroll
            for (int j = 0; j < NSB; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * (cs * NSB + j) + c16 > m0 + 4 * g + e) p[j][e] = 0.f;
                put_rows(sm.W, RW, m0, 16 * (cs * NSB + j), p[j], lane);
            }
        }
        row_sync<CS>();
        // num_aug = (P (.) M) V_aug + phi(Q) S_aug and G_aug over this wave's value
        // blocks (a compile-time range: the accumulators keep fixed registers)
        auto g_aug = [&](auto split) {
            constexpr int SP = decltype(split)::value;
            constexpr int NB0 = SP * B::NV0, NBN = SP == 0 ? B::NV0 : NVB - B::NV0;
            f32x4 num[NBN];
#pragma unroll
            for (int j = 0; j < NBN; ++j) num[j] = zero4();
            mm<C, NBN, false, false, W3, UNR, false, true>(sm.W, RW, m0, sm.V, RV, 16 * NB0, num, lane);
            mm<D, NBN, false, false, W3, UNR>(sm.P, RX, m0, sm.S, RV, 16 * NB0, num, lane);
            // dO of this wave's columns and its share of the row sums dO . num
            f32x4 dov[NBN];
            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < NBN; ++j)  // unconditional loads (clamped), selects at use
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = m0 + 4 * g + e, col = 16 * (NB0 + j) + c16;
                    dov[j][e] = load1(&dOs[(size_t)(t0 + (t < rows ? t : 0)) * D + (col < D ? col : 0)]);
                }
#pragma unroll
            for (int j = 0; j < NBN; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = m0 + 4 * g + e, col = 16 * (NB0 + j) + c16;
                    const float d = (t < rows && col < D) ? dov[j][e] : 0.f;
                    dov[j][e] = d;
                    part[e] += d * num[j][e];
                }
#pragma unroll
            for (int e = 0; e < 4; ++e) {  // row sums over the 16 lanes of a row group
                float x = part[e];
                x += __shfl_xor(x, 1, 64);
                x += __shfl_xor(x, 2, 64);
                x += __shfl_xor(x, 4, 64);
                x += __shfl_xor(x, 8, 64);
                part[e] = x;
            }
            if (c16 == 0) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sm.DOT[SP][m0 + 4 * g + e] = part[e];
                    // the normaliser is column D: column 0 of the last value block
                    if constexpr (NB0 + NBN == NVB) sm.DEN[m0 + 4 * g + e] = num[NBN - 1][e];
                }
            }
            row_sync<CS>();
            float rden[4], dot[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = m0 + 4 * g + e;
                rden[e] = 1.f / sm.DEN[r];
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < CS; ++k) s += sm.DOT[k][r];
                dot[e] = s * rden[e];  // dO . o
            }
            // G'_aug = [dO | -(dO . o) | 0]: its dO columns are the stored values
            // (exact in bf16); the factor 1 / den goes to dphi(Q) and U instead.
            // fp32 storage keeps G_aug = G'_aug / den in the tile.
#pragma unroll
            for (int j = 0; j < NBN; ++j) {
                f32x4 gv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool in = m0 + 4 * g + e < rows;
                    const int col = 16 * (NB0 + j) + c16;
                    if constexpr (GP)
                        gv[e] = !in ? 0.f : (col < D ? dov[j][e] : (col == D ? -dot[e] : 0.f));
                    else
                        gv[e] = !in ? 0.f : (col < D ? dov[j][e] * rden[e] : (col == D ? -dot[e] * rden[e] : 0.f));
                }
                put_rows(sm.G, RV, m0, 16 * (NB0 + j), gv, lane);
            }
            if (GP && SP == 0 && c16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.RDEN[m0 + 4 * g + e] = m0 + 4 * g + e < rows ? rden[e] : 0.f;
        };
        if constexpr (CS == 1) {
            g_aug(std::integral_constant<int, 0>{});
        } else {
            if (cs == 0)
                g_aug(std::integral_constant<int, 0>{});
            else
                g_aug(std::integral_constant<int, 1>{});
        }
        row_sync<CS>();  // G_aug rows of the row block are complete
        // G'_aug rows to the workspace (VK floats per token, den in column D + 1;
        // fp32 storage: G_aug) for the dK/dV pass
        for (int idx = lane + 64 * cs; idx < 16 * VK / 4; idx += 64 * CS) {
            const int r = idx / (VK / 4), c4 = idx % (VK / 4);
            if (m0 + r < rows) {
                float4 x = *reinterpret_cast<const float4 *>(&sm.G[(m0 + r) * RV + 4 * c4]);
                if (GP && 4 * c4 == D) x.y = sm.DEN[m0 + r];
                *reinterpret_cast<float4 *>(&Gw[(size_t)(t0 + m0 + r) * VK + 4 * c4]) = x;
            }
        }
        // A' = G'_aug V_aug^T, masked; dphi(Q) = ((A' (.) M) phi(K) + G'_aug S_aug^T) / den
        // (fp32 storage: G_aug in the tile, no division)
        {
            f32x4 s[NSB];
#pragma unroll
            for (int j = 0; j < NSB; ++j) s[j] = zero4();
            mm<VK, NSB, false, true, W3, UNR, false, true, GP ? D : 0>(sm.G, RV, m0, sm.V, RV, 16 * cs * NSB, s, lane);
#pragma unroll
            for (int j = 0; j < NSB; ++j) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * (cs * NSB + j) + c16 > m0 + 4 * g + e) s[j][e] = 0.f;
                put_rows(sm.W, RW, m0, 16 * (cs * NSB + j), s[j], lane);
            }
        }
        row_sync<CS>();
        f32x4 dp[NDW];
#pragma unroll
        for (int j = 0; j < NDW; ++j) dp[j] = zero4();
        mm<C, NDW, false, false, W3, UNR>(sm.W, RW, m0, sm.K, RX, 16 * cs * NDW, dp, lane);
        mm<VK, NDW, false, true, W3, UNR, false, false, GP ? D : 0>(sm.G, RV, m0, sm.S, RV, 16 * cs * NDW, dp, lane);
        // dQ = dphi * min(phi(q), 1) (elu'(q): 1 for q > 0, exp(q) = phi(q) otherwise)
#pragma unroll
        for (int j = 0; j < NDW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if constexpr (GP) dp[j][e] *= sm.RDEN[m0 + 4 * g + e];
                dp[j][e] *= fminf(sm.P[(m0 + 4 * g + e) * RX + 16 * (cs * NDW + j) + c16], 1.f);
            }
        store_dwide<D, C, T>(dp, sm.W, m0, cs, rows, dQs, t0, lane);
        block_sync_lds();  // every wave's G_aug rows are in LDS, the state image is read
        // U += phi(Q)^T G_aug (bf16 storage: (phi(Q) / den)^T G'_aug), S_aug +=
        // phi(K)^T V_aug (this wave's feature rows)
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int f0 = 16 * (kNW * q + w);
            if constexpr (GP)
                mm<C, NVB, true, false, W3, UNR, false, false, 0, 0, D, true>(sm.P, RX, f0, sm.G, RV, 0, U[q], lane,
                                                                               sm.RDEN);
            else
                mm<C, NVB, true, false, W3, UNR>(sm.P, RX, f0, sm.G, RV, 0, U[q], lane);
            mm<C, NVB, true, false, W3, UNR, false, true>(sm.K, RX, f0, sm.V, RV, 0, S[q], lane);
        }
        put_state<D, C>(S, sm.S, w, lane);
    }
    // segment sums U, layout [feature][d_v + 1] (value columns 0..D)
    float *Us = a.U + ((size_t)bh * a.P + seg) * D * (D + 1);
#pragma unroll
    for (int q = 0; q < FBW; ++q)
#pragma unroll
        for (int j = 0; j < NVB; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 16 * (kNW * q + w) + 4 * g + e, col = 16 * j + c16;
                if (col <= D) Us[f * (D + 1) + col] = U[q][j][e];
            }
}

// ---------------------------------------------------------------------------
// dK / dV pass.  Tiles in reverse from R_aug = dS_out_aug + the later
// segments' sums (key rows of this wave's row block):
//   dphi(K) = (B (.) M') phi(Q) + V_aug R_aug^T       B = V_aug G_aug^T
//   dV      = (P' (.) M') G     + phi(K) R            P' = phi(K) phi(Q)^T
//   (M': query >= key),  dK = dphi(K) * min(phi(k), 1)
//   R_aug  += phi(Q)^T G_aug
// ---------------------------------------------------------------------------
template <int D, int C, typename T>
__global__ __launch_bounds__(kThreads) void k_bwd_dkv_mfma(BwdMfmaArgs a) {
    using B = BCfg<D, C>;
    // bf16 storage: products in bf16 passes (two where V_aug is an operand),
    // the k steps unrolled; the tile holds G'_aug (GP), whose dO columns are
    // exact in bf16
    constexpr bool W3 = sizeof(T) == 2, UNR = true, GP = W3;
    constexpr int RX = B::RX, RV = B::RV, RW = B::RW, VK = B::VK, NVB = B::NVB, FBW = B::FBW, NSB = B::NSB,
                  NDW = B::NDW, CS = B::CS, RB = B::RB;
    __shared__ BTiles<D, C> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int rb = CS == 1 ? w : w % RB, cs = CS == 1 ? 0 : w / RB;
    const int m0 = 16 * rb;
    const int seg = blockIdx.x % a.P, bh = blockIdx.x / a.P;
    const int N = a.N;
    const int c_begin = seg * a.seg_chunks, c_end = min(a.n_chunks, c_begin + a.seg_chunks);
    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * D;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * D;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * D;
    T *dKs = static_cast<T *>(a.dK) + (size_t)bh * N * D;
    T *dVs = static_cast<T *>(a.dV) + (size_t)bh * N * D;
    const float *Gw = a.G + (size_t)bh * N * VK;

    // R_aug entering the segment from above: [dS_out | dz_out] (or zero) plus
    // the sums of segments P - 1 down to seg + 1, in that order; segment 0
    // adds its own sum as well for dS_in, dz_in (the gradient of the starting
    // state)
    f32x4 R[FBW][NVB];
    {
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int j = 0; j < NVB; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = 16 * (kNW * q + w) + 4 * g + e, col = 16 * j + c16;
                    float r0 = 0.f;
                    if (a.dS_out) {
                        const float x =
                            col < D ? a.dS_out[((size_t)bh * D + f) * D + col] : a.dz_out[(size_t)bh * D + f];
                        r0 = col <= D ? x : 0.f;
                    }
                    R[q][j][e] = r0;
                }
        const float *Ug = a.U + (size_t)bh * a.P * D * (D + 1);
        auto at = [&](int p, int f, int col) { return Ug + ((size_t)p * D + f) * (D + 1) + (col < D ? col : D); };
        add_segments<D, C>(R, a.P - 1, a.P - 1 - seg, -1, at, w, lane);
        if (seg == 0 && a.dS_in) {
            f32x4 T0[FBW][NVB];
#pragma unroll
            for (int q = 0; q < FBW; ++q)
#pragma unroll
                for (int j = 0; j < NVB; ++j) T0[q][j] = R[q][j];
            add_segments<D, C>(T0, 0, 1, 1, at, w, lane);
#pragma unroll
            for (int q = 0; q < FBW; ++q)
#pragma unroll
                for (int j = 0; j < NVB; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 16 * (kNW * q + w) + 4 * g + e, col = 16 * j + c16;
                        if (col < D) a.dS_in[((size_t)bh * D + f) * D + col] = T0[q][j][e];
                        else if (col == D) a.dz_in[(size_t)bh * D + f] = T0[q][j][e];
                    }
        }
    }
    put_state<D, C>(R, sm.S, w, lane);

    // the chunks from last to first; the rows of chunk c are loaded during
    // chunk c + 1 (the first chunk re-reads itself: every load stays unconditional)
    RowPieces<D, C> xq, xk, xv;
    GPieces<D, C> xg;
    auto fetch = [&](int cc) {
        const int tt0 = cc * C, rr = min(C, N - tt0);
        load_rows<D, C>(Qs, tt0, rr, xq, tid);
        load_rows<D, C>(Ks, tt0, rr, xk, tid);
        load_rows<D, C>(Vs, tt0, rr, xv, tid);
        load_g<D, C>(Gw, tt0, rr, xg, tid);
    };
    fetch(c_end - 1);
    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * C, rows = min(C, N - t0);
        block_sync_lds();
        put_phi<D, C>(xq, rows, sm.P, tid);
        put_phi<D, C>(xk, rows, sm.K, tid);
        put_vaug<D, C>(xv, rows, sm.V, tid);
        put_g<D, C>(xg, rows, sm.G, sm.RDEN, tid);
        fetch(max(c - 1, c_begin));
        block_sync_lds();

        // dphi(K): B = V_aug G_aug^T masked (query >= key), times phi(Q); + V_aug R_aug^T
        {
            f32x4 b[NSB];
#pragma unroll
            for (int j = 0; j < NSB; ++j) b[j] = zero4();
            mm<VK, NSB, false, true, W3, UNR, true, false, 0, GP ? D : 0>(sm.V, RV, m0, sm.G, RV, 16 * cs * NSB, b, lane);
#pragma unroll
            for (int j = 0; j < NSB; ++j) {
                const float rq = sm.RDEN[16 * (cs * NSB + j) + c16];  // column = query token
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    b[j][e] = 16 * (cs * NSB + j) + c16 < m0 + 4 * g + e ? 0.f : b[j][e] * (GP ? rq : 1.f);
                put_rows(sm.W, RW, m0, 16 * (cs * NSB + j), b[j], lane);
            }
        }
        row_sync<CS>();
        f32x4 dk[NDW];
#pragma unroll
        for (int j = 0; j < NDW; ++j) dk[j] = zero4();
        mm<C, NDW, false, false, W3, UNR>(sm.W, RW, m0, sm.P, RX, 16 * cs * NDW, dk, lane);
        mm<VK, NDW, false, true, W3, UNR, true, false>(sm.V, RV, m0, sm.S, RV, 16 * cs * NDW, dk, lane);
        // dV: P' = phi(K) phi(Q)^T masked, times G; + phi(K) R
        f32x4 dv[NDW];
        {
            f32x4 p[NSB];
#pragma unroll
            for (int j = 0; j < NSB; ++j) p[j] = zero4();
            mm<D, NSB, false, true, W3, UNR>(sm.K, RX, m0, sm.P, RX, 16 * cs * NSB, p, lane);
            row_sync<CS>();  // the row block's waves have read the scores B before W is overwritten
            // P' / den of the query (column), so that P' G_aug = (P' / den) G'_aug
            // (bf16 storage)
#pragma unroll
            for (int j = 0; j < NSB; ++j) {
                const float rq = sm.RDEN[16 * (cs * NSB + j) + c16];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    p[j][e] = 16 * (cs * NSB + j) + c16 < m0 + 4 * g + e ? 0.f : p[j][e] * (GP ? rq : 1.f);
                put_rows(sm.W, RW, m0, 16 * (cs * NSB + j), p[j], lane);
            }
        }
        row_sync<CS>();
#pragma unroll
        for (int j = 0; j < NDW; ++j) dv[j] = zero4();
        mm<C, NDW, false, false, W3, UNR, false, GP>(sm.W, RW, m0, sm.G, RV, 16 * cs * NDW, dv, lane);
        mm<D, NDW, false, false, W3, UNR>(sm.K, RX, m0, sm.S, RV, 16 * cs * NDW, dv, lane);
        // dK = dphi(K) * min(phi(k), 1)
#pragma unroll
        for (int j = 0; j < NDW; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                dk[j][e] *= fminf(sm.K[(m0 + 4 * g + e) * RX + 16 * (cs * NDW + j) + c16], 1.f);
        store_dwide<D, C, T>(dk, sm.W, m0, cs, rows, dKs, t0, lane);
        store_dwide<D, C, T>(dv, sm.W, m0, cs, rows, dVs, t0, lane);
        block_sync_lds();  // the state image is no longer read
        // R_aug += phi(Q)^T G_aug = (phi(Q) / den)^T G'_aug (this wave's feature rows)
#pragma unroll
        for (int q = 0; q < FBW; ++q)
            mm<C, NVB, true, false, W3, UNR, false, false, 0, 0, GP ? D : 0, GP>(sm.P, RX, 16 * (kNW * q + w), sm.G, RV,
                                                                                  0, R[q], lane, sm.RDEN);
        put_state<D, C>(R, sm.S, w, lane);
    }
}

template <int D, int C>
constexpr size_t lds_bytes() {
    return sizeof(BTiles<D, C>);
}
static_assert(lds_bytes<64, 64>() <= 160 * 1024 && lds_bytes<128, 32>() <= 160 * 1024, "tiles fit the LDS");

}  // namespace

bool backward_mfma_supported(const Shape &sh, int chunk) {
    if ((sh.dtype != kBF16 && sh.dtype != kF32) || sh.phi != kElu1 || sh.dk != sh.dv) return false;
    if (sh.dk == 64) return chunk == 64;
    return sh.dk == 128 && chunk % 32 == 0;  // on 32-token tiles
}

int backward_mfma_tile(const Shape &sh) { return sh.dk == 128 ? 32 : 64; }

size_t backward_mfma_g_floats(const Shape &sh) { return (size_t)sh.dk + 4; }

hipError_t launch_bwd_dq_mfma(const BwdMfmaArgs &a, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)((size_t)a.BH * a.P)), block(kThreads);
    if (a.D == 64)
        return a.f32 ? launch_kernel_ev(k_bwd_dq_mfma<64, 64, float>, grid, block, 0, st, ev, a)
                     : launch_kernel_ev(k_bwd_dq_mfma<64, 64, uint16_t>, grid, block, 0, st, ev, a);
    if (a.D == 128)
        return a.f32 ? launch_kernel_ev(k_bwd_dq_mfma<128, 32, float>, grid, block, 0, st, ev, a)
                     : launch_kernel_ev(k_bwd_dq_mfma<128, 32, uint16_t>, grid, block, 0, st, ev, a);
    return hipErrorNotSupported;
}

hipError_t launch_bwd_dkv_mfma(const BwdMfmaArgs &a, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)((size_t)a.BH * a.P)), block(kThreads);
    if (a.D == 64)
        return a.f32 ? launch_kernel_ev(k_bwd_dkv_mfma<64, 64, float>, grid, block, 0, st, ev, a)
                     : launch_kernel_ev(k_bwd_dkv_mfma<64, 64, uint16_t>, grid, block, 0, st, ev, a);
    if (a.D == 128)
        return a.f32 ? launch_kernel_ev(k_bwd_dkv_mfma<128, 32, float>, grid, block, 0, st, ev, a)
                     : launch_kernel_ev(k_bwd_dkv_mfma<128, 32, uint16_t>, grid, block, 0, st, ev, a);
    return hipErrorNotSupported;
}

}  // namespace la
