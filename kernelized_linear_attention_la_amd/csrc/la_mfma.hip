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
// B[k-slots][l%16] and receives D[4(l/16)+e][l%16], e = 0..3.
//
// phi(K_c) and V_aug sit in LDS token-major, exactly as they arrive from HBM
// (16-byte row writes).  Products that contract over features read rows with
// 128-bit loads; products that contract over tokens (P V and the state
// update) read their operands with ds_read_b64_tr_b16, which hands each lane
// a column slice of four token rows, so no transposed copy is ever written.
// Token k-slots follow the order
//     slot 8g+e  <->  token 16*(e/4) + 4g + (e%4)   inside each 32-token block,
// the order in which a lane already holds the scores of two consecutive
// 16x16 P^T accumulator tiles: P becomes an A operand in registers.
//
// The fp32 state S_aug (d' x (d_v+16)) lives in the accumulators of the waves
// that own its 16-row feature blocks for the whole segment; a pre-swizzled
// bf16 image in LDS feeds the next chunk's phi(Q) S read.
#include <type_traits>

#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_ops.h"

namespace la {
namespace {

template <int DK, int DV, int C, int PHI>
struct Cfg {
    static constexpr bool F = PHI == kFavor;
    // cosFormer ("Story of Attention Part 5", section 3): [ReLU(x) cos t, ReLU(x) sin t]
    static constexpr bool CF = PHI == kCosformer;
    // DPFP with one shift ("Linear Attention", feature-map table): r = ReLU([x, -x]), r_j r_{j+1}
    static constexpr bool DPF = PHI == kDpfp;
    // cos/sin projections ("Linear Attention", feature-map table): [cos(W x); sin(W x)], m = d_k rows of W
    static constexpr bool TR = PHI == kTrig;
    static constexpr bool PR = F || TR;          // the map goes through a projection X W^T on the matrix cores
    static constexpr bool XR = PR || DPF;        // raw K, Q rows staged in LDS, the map formed there
    static constexpr int NW = C / 16;            // waves
    static constexpr int THREADS = 64 * NW;
    static constexpr int DP = F ? 256 : ((CF || DPF || TR) ? 2 * DK : DK);  // feature dimension
    static constexpr int M = F ? 256 : (TR ? DK : 0);  // rows of W
    // Retention ("Story of Attention Part 5", sections 4 and 6): raw q and k,
    // decay per head, no normaliser.
    static constexpr bool RET = PHI == kIdentity;
    static constexpr int NJ = DV / 16 + (RET ? 0 : 1);  // value column blocks incl. the normaliser block
    static constexpr int DVA = DV + (RET ? 0 : 16);
    static constexpr int KBT = C / 32;           // 32-token k-blocks per chunk
    static constexpr int KBF = DP / 32;          // 32-feature k-blocks
    static constexpr int KBD = DK / 32;          // 32-wide k-blocks of the raw input (FAVOR+ projection)
    static constexpr int FB = DP / 16;           // 16-row feature blocks of the state
    static constexpr int FBW = (FB + NW - 1) / NW;  // feature blocks owned per wave
    // LDS row strides (bf16 elements).  phi(K): 8 extra elements keep the
    // 16-row 128-bit reads conflict free.  V_aug: a stride of 16 mod 128
    // elements keeps the transpose reads of 8 consecutive rows conflict free
    // (FAVOR+ takes the short stride to stay inside 160 KB).
    static constexpr int RK = DP + 8;
    static constexpr int RV = F ? DVA + 8 : ((DVA + 111) / 128) * 128 + 16;
    static constexpr int RO = DV + 8;
    static constexpr int RX = DK + 8;  // FAVOR+: raw key / query rows (16-row 128-bit reads conflict free)
};

template <int DK, int DV, int C, int PHI, int NKS>
struct Smem {
    using G = Cfg<DK, DV, C, PHI>;
    static constexpr bool F = G::F;
    uint16_t K[NKS][C * G::RK];         // phi(K_c), token-major (NKS chunks when LDS-resident)
    uint16_t V[NKS][C * G::RV];         // V_aug, token-major
    uint4 STB[G::NJ][G::KBF][64];       // bf16 S_aug: B operand of phi(Q) S
    uint16_t O[G::NW][16 * G::RO];      // per-wave output staging for 16-byte stores
    uint16_t XK[G::XR ? C * G::RX : 1];  // FAVOR+, DPFP, cos/sin: raw K_c, token-major
    uint16_t XQ[G::XR ? C * G::RX : 1];  // FAVOR+, DPFP, cos/sin: raw Q_c, token-major
    uint16_t QP[G::PR ? C * G::RK : 1];  // FAVOR+, cos/sin: phi(Q_c), token-major
};

// Store a 16x16 fp32 state tile (lane l holds S[16fb + 4g + e][16nb + l%16])
// into the bf16 B-operand image of S_aug.
template <typename G>
__device__ __forceinline__ void put_state_block(uint4 (*STB)[G::KBF][64], int fb, int nb, int lane, f32x4 s) {
    const int g = lane >> 4, c = lane & 15;
    uint2 v = pack4(s[0], s[1], s[2], s[3]);
    const int x = 16 * (fb & 1) + 4 * g;  // feature slot inside the 32-feature k-block
    reinterpret_cast<uint2 *>(&STB[nb][fb >> 1][c + 16 * (x >> 3)])[(x >> 2) & 1] = v;
}

// cos u and sin u through the hardware's sine and cosine, which take their
// argument in turns: u / 2pi reduced to [-1/2, 1/2] by the period first.
__device__ __forceinline__ void turn_cos_sin(float u, float &c, float &s) {
    constexpr float kInvTwoPi = 0.159154943091895336f;
    float r = u * kInvTwoPi;
    r -= rintf(r);
    c = __builtin_amdgcn_cosf(r);
    s = __builtin_amdgcn_sinf(r);
}

template <int DK, int DV, int C, int PHI, int MODE>
__global__ __launch_bounds__(C / 16 * 64) void k_mfma(FwdArgs a) {
    using G = Cfg<DK, DV, C, PHI>;
    using T = uint16_t;
    // LDS-resident single pass: phase 1 keeps every chunk's phi(K), V_aug of
    // the segment (at most kResChunks) in LDS, phase 3 reads them back.
    constexpr bool RES = MODE == kModeFusedRes;
    constexpr int NKS = RES ? kResChunks : 1;
    __shared__ Smem<DK, DV, C, PHI, NKS> sm;
    constexpr int NW = G::NW, NJ = G::NJ, KBT = G::KBT, KBF = G::KBF, FB = G::FB, FBW = G::FBW;
    constexpr int RK = G::RK, RV = G::RV, RO = G::RO;
    constexpr bool FUSED = MODE == kModeFused || MODE == kModeFusedRes;
    constexpr bool DO_OUT = MODE != kModeState;  // some chunk of the launch writes outputs
    constexpr bool DO_STATE = MODE != kModeRead;
    constexpr bool NEED_K = MODE != kModeRead;
    constexpr bool RET = G::RET;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform across the wave
    const int g = lane >> 4, c16 = lane & 15;

    const Segments sg = a.sg;
    const int N = a.sh.N;
    const int seg = blockIdx.x % sg.P;
    const int bh = blockIdx.x / sg.P;
    const int c_begin = seg * sg.seg_chunks;
    const int c_end = min(sg.n_chunks, c_begin + sg.seg_chunks);

    // retention decay lambda = gamma[h]; lambda^x = exp2(x log2 lambda), 1 at x = 0
    const float l2 = RET ? log2f(a.sh.gamma[bh % a.sh.H]) : 0.f;
    auto dpow = [&](float x) { return x == 0.f ? 1.f : __builtin_amdgcn_exp2f(x * l2); };
    // Most decay powers of the chunk loop are products of one per-lane power
    // and wave-uniform powers (scalar registers), every exponent >= 0, so no
    // factor overflows, lambda = 0 included:
    //   off-diagonal score tile (jb < qb), lambda^(16(qb-jb) + c16 - 4g - e)
    //     = lambda^(16(qb-jb-1)) * lambda^(c16 + 12 - 4g) * lambda^(4 - e);
    //   key weight of slot 4h + j in a full chunk, lambda^(C-1-t) with
    //   t = 32kt + 16h + 4g + j,
    //     = lambda^(C-32-32kt) * lambda^(12 - 4g) * lambda^(16(1-h) + 3 - j).
    // The diagonal tile and a partial last chunk take the exponentials, and
    // so does d = 64 (whose single pass is the whole-segment kernel): there
    // the factored form let the compiler place an accumulating product two
    // registers above its accumulator input, which the assembly test rejects.
    constexpr bool RFAC = RET && DK == 128;
    auto uni = [](float x) { return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x))); };
    float dec_lane = 1.f, kw_lane = 1.f, dec_e[4], kw_slot[8];
    if constexpr (RFAC) {
        dec_lane = dpow((float)(c16 + 12 - 4 * g));
        kw_lane = dpow((float)(12 - 4 * g));
#pragma unroll
        for (int e = 0; e < 4; ++e) dec_e[e] = uni(dpow((float)(4 - e)));
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) kw_slot[sl] = uni(dpow((float)(16 * (1 - (sl >> 2)) + 3 - (sl & 3))));
    }

    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * DK;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * DK;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * DV;
    T *Os = DO_OUT ? static_cast<T *>(a.O) + (size_t)bh * N * DV : nullptr;

    // ---- FAVOR+ projection rows in registers, once per workgroup: wave w
    // owns features 64w..64w+63 and holds their rows of W as MFMA A operands
    // (lane l: row 64w + 16fbl + l%16, columns 32kb + 8(l/16)..+7).  W is
    // split as W = W_hi + W_lo with both parts bf16 (W_lo = bf16(W - W_hi));
    // the inputs are exact in bf16, so x . w_r = x . hi_r + x . lo_r is
    // accurate to about 2^-16 relative, where a single bf16 W would shift
    // every exponent of the feature map by ~2^-9 |w_r| |x|.
    // The cos/sin map takes the same registers with 16 rows of W per wave.
    constexpr int FWB = G::F ? 4 : 1;  // 16-row blocks of W per wave
    static_assert(!G::PR || NW * 16 * FWB == G::M, "one wave per 64 (FAVOR+) or 16 (cos/sin) rows of W");
    Op8 wreg[FWB][G::PR ? G::KBD : 1][2];
    if constexpr (G::PR) {
#pragma unroll
        for (int fbl = 0; fbl < FWB; ++fbl)
#pragma unroll
            for (int kb = 0; kb < G::KBD; ++kb) {
                const float *src = a.sh.W + (size_t)(16 * FWB * w + 16 * fbl + c16) * DK + 32 * kb + 8 * g;
                const float4 w0 = *reinterpret_cast<const float4 *>(src);
                const float4 w1 = *reinterpret_cast<const float4 *>(src + 4);
                const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int e = 0; e < 8; e += 2) {
                    const uint32_t h2 = cvt2(wv[e], wv[e + 1]);
                    wreg[fbl][kb][0].u32[e / 2] = h2;
                    wreg[fbl][kb][1].u32[e / 2] = cvt2(wv[e] - lo_bf16(h2), wv[e + 1] - hi_bf16(h2));
                }
            }
    }

    const float inv_sqrt_m = G::F ? 1.0f / 16.0f : 1.0f;  // m = 256
    // cosFormer reweighting of token t: (cos, sin) of pi (pos0 + t) / 2M, the
    // phase formed in double so that long positions keep their accuracy
    auto cf_phase = [&](int t, float &cw, float &sw) {
        const double ang = 3.14159265358979323846 * (double)(a.sh.pos0 + t) / (2.0 * (double)a.sh.param);
        cw = (float)cos(ang);
        sw = (float)sin(ang);
    };
    // 8 packed bf16 values: ReLU(x) * w, rounded to bf16
    auto relu_scale8 = [](uint4 x, float w) {
        auto f = [&](float v) { return (v > 0.f ? v : 0.f) * w; };
        uint4 r;
        r.x = cvt2(f(lo_bf16(x.x)), f(hi_bf16(x.x)));
        r.y = cvt2(f(lo_bf16(x.y)), f(hi_bf16(x.y)));
        r.z = cvt2(f(lo_bf16(x.z)), f(hi_bf16(x.z)));
        r.w = cvt2(f(lo_bf16(x.w)), f(hi_bf16(x.w)));
        return r;
    };

    // ---- register prefetch of a chunk: K and V rows in 8-column pieces
    // (FAVOR+: also Q), plus, for ELU+1, this wave's query rows.  Chunk
    // c+DEPTH is fetched right after chunk c is staged, so its loads are in
    // flight during the matrix work of chunks c and c+1.
    constexpr int UK = NEED_K ? C * DK / 8 : 0;
    constexpr int UV = NEED_K ? C * DV / 8 : 0;
    constexpr int UQ = (G::XR && DO_OUT) ? C * DK / 8 : 0;
    constexpr int KBQ = G::XR ? 1 : G::KBD;  // 16-byte raw query pieces per lane (the lane's row)
    // prefetch ring: chunks in flight ahead of the one being computed.  Two
    // for the smaller tiles; one for d = 128 with 128-token chunks, whose
    // chunk takes several load latencies to compute and whose registers are
    // needed by the 8-wave tiles.
    constexpr int DEPTH = (DK == 128 && C == 128) ? 1 : 2;
    // ELU+1 with 128-token chunks at d = 128: a prefetched chunk's keys and
    // this lane's query pieces are mapped in registers at the end of the
    // chunk before the one that stages them (pre_map), not while every wave
    // stages at once: a wave that finishes its matrix work early then runs
    // its exponentials while the other wave of its SIMD is still reading LDS
    // and issuing MFMAs.  (The other tilings map while staging; there the
    // exponentials are a smaller share of the chunk.)
    constexpr bool PRE = PHI == kElu1;
    struct Pref {
        Op8 raw[(UK + UV + UQ) / G::THREADS > 0 ? (UK + UV + UQ) / G::THREADS : 1];
        Op8 q[KBQ];
        bool klive, qlive;  // rows loaded (wave-uniform); dead pieces are not mapped
    };
    Pref pf[DEPTH];
    // Query block of this wave.  Waves w and w + 4 share a SIMD; with eight
    // waves the blocks are paired (0,7) (2,5) (4,3) (6,1) so every SIMD gets
    // the same share of the causal triangle.
    const int qb = NW == 8 ? (w < 4 ? 2 * w : 15 - 2 * w) : w;
    const int row = 16 * qb + c16;  // this lane's query (and FAVOR+ key) row inside a chunk

    static_assert(UK % G::THREADS == 0 && UV % G::THREADS == 0 && UQ % G::THREADS == 0,
                  "units must tile the workgroup");
    constexpr int UKT = UK / G::THREADS, UVT = UV / G::THREADS, UQT = UQ / G::THREADS;  // pieces per thread

    // Piece i of a thread is row t = piece / W8, columns 8 * (piece % W8);
    // its byte offset inside the chunk is 16 * piece.  Every chunk index,
    // also one past the segment (an empty range), issues the same loads.
    // A step is a chunk index.  In the single-pass mode steps 0..n-1 are the
    // segment's n chunks for its own sums (keys and values only); the output
    // pass over the same chunks starts at the even step n + (n & 1), so that
    // it always begins on ring slot 0 (step n of an odd segment is empty).
    // Phase 1 of the single pass walks the segment's chunks last to first
    // (the sums do not depend on the order; retention's decayed sums do, so it
    // keeps the forward order): phase 3 then starts on the chunks read last,
    // which are the likeliest to be still in the Infinity Cache.
    auto p1_chunk = [&](int i) { return RET ? i : c_end - c_begin - 1 - i; };
    auto fetch = [&](Pref &p, int s) {
        bool live, qlive;
        int cc;
        if constexpr (FUSED) {
            const int n = c_end - c_begin, cbase = DEPTH == 2 ? n + (n & 1) : n;
            const bool pa = s < n, pc = s >= cbase && s < cbase + n;
            live = pa || pc;
            cc = c_begin + (pa ? p1_chunk(s) : (pc ? s - cbase : 0));
            qlive = pc;
            if (RES && pc) live = false, cc = c_begin + (s - cbase);  // keys, values are in LDS already
        } else {
            live = s < c_end;
            cc = live ? s : c_begin;
            qlive = live;
        }
        const int tt0 = cc * C;
        const int rows = live ? min(C, N - tt0) : 0;
        const int qrows = qlive ? min(C, N - tt0) : 0;
        p.klive = live;
        p.qlive = qlive;
        const auto rk = make_rsrc(Ks + (size_t)tt0 * DK, rows * DK * 2);
        const auto rv = make_rsrc(Vs + (size_t)tt0 * DV, rows * DV * 2);
#pragma unroll
        for (int i = 0; i < UKT; ++i) p.raw[i].u = bload16(rk, 16 * (tid + i * G::THREADS));
#pragma unroll
        for (int i = 0; i < UVT; ++i) p.raw[UKT + i].u = bload16(rv, 16 * (tid + i * G::THREADS));
        if constexpr (DO_OUT) {
            const auto rq = make_rsrc(Qs + (size_t)tt0 * DK, qrows * DK * 2);
            if constexpr (G::XR) {
#pragma unroll
                for (int i = 0; i < UQT; ++i) p.raw[UKT + UVT + i].u = bload16_nt(rq, 16 * (tid + i * G::THREADS));
            } else {
#pragma unroll
                for (int kb = 0; kb < KBQ; ++kb) p.q[kb].u = bload16_nt(rq, 2 * (row * DK + 8 * g + 32 * kb));
            }
        }
    };

    // ---- write one prefetched chunk into LDS (token-major rows)
    auto stage = [&](const Pref &p, int tt0, int ks) {
        const bool full = tt0 + C <= N;
#pragma unroll
        for (int i = 0; i < UKT; ++i) {
            const int u = tid + i * G::THREADS, t = u / (DK / 8), c8 = u % (DK / 8);
            if constexpr (G::XR) {  // raw rows; the feature map is formed after the barrier
                *reinterpret_cast<uint4 *>(&sm.XK[t * G::RX + 8 * c8]) = p.raw[i].u;
            } else if constexpr (G::CF) {  // cos half at column 8c8, sin half at DK + 8c8
                float cw, sw;
                cf_phase(tt0 + t, cw, sw);
                uint4 pc = relu_scale8(p.raw[i].u, cw), ps = relu_scale8(p.raw[i].u, sw);
                if (!full && tt0 + t >= N) pc = ps = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(&sm.K[ks][t * RK + 8 * c8]) = pc;
                *reinterpret_cast<uint4 *>(&sm.K[ks][t * RK + DK + 8 * c8]) = ps;
            } else {
                // ELU+1 on the way in, unless pre_map has applied it (retention:
                // raw keys); tokens past the end get phi = 0, not phi(0) = 1
                uint4 ph;
                if constexpr (RET || PRE) ph = p.raw[i].u;
                else ph = elu1_bf16x8(p.raw[i].u);
                if (!full && tt0 + t >= N) ph = make_uint4(0, 0, 0, 0);
                *reinterpret_cast<uint4 *>(&sm.K[ks][t * RK + 8 * c8]) = ph;
            }
        }
#pragma unroll
        for (int i = 0; i < UQT; ++i) {
            const int u = tid + i * G::THREADS, t = u / (DK / 8), c8 = u % (DK / 8);
            *reinterpret_cast<uint4 *>(&sm.XQ[t * G::RX + 8 * c8]) = p.raw[UKT + UVT + i].u;
        }
#pragma unroll
        for (int i = 0; i < UVT; ++i) {
            const int u = tid + i * G::THREADS, t = u / (DV / 8), c8 = u % (DV / 8);
            *reinterpret_cast<uint4 *>(&sm.V[ks][t * RV + 8 * c8]) = p.raw[UKT + i].u;
        }
    };

    // ELU+1 of a prefetched chunk in registers: keys piece by piece, query
    // pieces with their row's power-of-two scale (cancels in the division)
    auto pre_map = [&](Pref &p) {
        if constexpr (PRE) {
            if (p.klive) {
#pragma unroll
                for (int i = 0; i < UKT; ++i) p.raw[i].u = elu1_bf16x8(p.raw[i].u);
            }
            if constexpr (DO_OUT) {
                if (p.qlive) {
                    uint4 raw[KBQ], ph[KBQ];
#pragma unroll
                    for (int kb = 0; kb < KBQ; ++kb) raw[kb] = p.q[kb].u;
                    elu1_query_pieces<KBQ>(raw, ph);
#pragma unroll
                    for (int kb = 0; kb < KBQ; ++kb) p.q[kb].u = ph[kb];
                }
            }
        }
    };

    // the first chunks' loads go out before the starting state is read
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(pf[d], (FUSED ? 0 : c_begin) + d);
    // ---- starting state into the owners' accumulators (+ bf16 image)
    f32x4 S[FBW][NJ];
    {
        const float *Ssrc = !FUSED && a.st.S_src ? a.st.S_src + bh * a.st.src_slice + seg * a.st.src_seg : nullptr;
        const float *zsrc = !FUSED && a.st.z_src ? a.st.z_src + bh * a.st.zsrc_slice + seg * a.st.zsrc_seg : nullptr;
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
                if (DO_OUT && !FUSED && fb < FB) put_state_block<G>(sm.STB, fb, nb, lane, v);
            }
        }
    }
    // normaliser block of V_aug: column d_v is 1 for every token, the other
    // 15 columns 0.  Tokens past the end of the sequence have phi(k) = 0, so
    // their 1 contributes nothing.
    if constexpr (NEED_K && !RET) {
        for (int u = tid; u < NKS * C * 2; u += G::THREADS) {
            const int ks = u / (C * 2), t = (u >> 1) % C, half = u & 1;
            const uint32_t first = half == 0 ? 0x3f80u : 0u;
            *reinterpret_cast<uint4 *>(&sm.V[ks][t * RV + DV + 8 * half]) = make_uint4(first, 0, 0, 0);
        }
    }
    block_sync_lds();

    // One chunk c (prefetch step `step`).  OUT: the chunk produces outputs;
    // otherwise only its contribution to the state is accumulated.
    auto body = [&](Pref &p, int c, int step, auto out_tag) {
        constexpr bool OUT = decltype(out_tag)::value;
        constexpr bool INTRA = OUT && MODE != kModeRead;  // causal: intra-chunk products
        constexpr bool CARRY = OUT && MODE != kModeRead;  // refresh the state image for the next chunk
        const int t0 = c * C;
        const int ks = RES ? c - c_begin : 0;  // LDS chunk slot
        if (!(RES && OUT)) stage(p, t0, ks);  // the resident phase 3 finds phi(K), V in LDS
        Op8 phq[KBF];
        if constexpr (OUT && G::CF) {  // features 32kf + 8g..: cos half (kf < KBD), then sin half
            float cw, sw;
            cf_phase(t0 + row, cw, sw);
#pragma unroll
            for (int kf = 0; kf < KBF; ++kf) phq[kf].u = relu_scale8(p.q[kf % G::KBD].u, kf < G::KBD ? cw : sw);
        } else if constexpr (OUT && !G::XR && RET) {
#pragma unroll
            for (int kb = 0; kb < KBF; ++kb) phq[kb].u = p.q[kb].u;  // rows past the end are not stored
        } else if constexpr (OUT && !G::XR && PRE) {
#pragma unroll
            for (int kb = 0; kb < KBF; ++kb) phq[kb].u = p.q[kb].u;  // mapped by pre_map
        } else if constexpr (OUT && !G::XR) {
            // ELU+1 with the row's power-of-two scale (cancels in the division)
            uint4 raw[KBF], ph[KBF];
#pragma unroll
            for (int kb = 0; kb < KBF; ++kb) raw[kb] = p.q[kb].u;
            elu1_query_pieces<KBF>(raw, ph);
#pragma unroll
            for (int kb = 0; kb < KBF; ++kb) phq[kb].u = ph[kb];
        }
        block_sync_lds();
        fetch(p, step + DEPTH);

        // ---------------- FAVOR+ and cos/sin: feature maps through projections
        // on the matrix cores.  Wave w forms U = W_w X^T for its 64 (FAVOR+)
        // or 16 (cos/sin) rows of W and all C tokens: the A operands (W) are
        // in registers, the B operands are the raw rows (lane l: token
        // 16tb + l%16, columns 32kb + 8(l/16)..+7), and accumulator lane
        // (4g+e, c16) of tile (fbl, tb) holds row r = 16 FWB w + 16fbl + 4g + e
        // of token 16tb + c16.  FAVOR+: phi_r = exp(u - |x|^2/2)/sqrt(m) at
        // feature r; cos/sin: cos u at feature r, sin u at feature m + r.
        // phi goes to LDS token-major, in natural feature order.
        if constexpr (G::PR) {
            static_assert(C == 64, "projected maps: four 16-token blocks per chunk");
            auto project = [&](const uint16_t *xr, uint16_t *dst, bool mask_tail) {
                Op8 xb[4][G::KBD];
                float shift[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    float sq = 0.f;
#pragma unroll
                    for (int kb = 0; kb < G::KBD; ++kb) {
                        xb[tb][kb].u = *reinterpret_cast<const uint4 *>(&xr[(16 * tb + c16) * G::RX + 32 * kb + 8 * g]);
                        if constexpr (G::F) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const float v0 = lo_bf16(xb[tb][kb].u32[e]), v1 = hi_bf16(xb[tb][kb].u32[e]);
                                sq += v0 * v0 + v1 * v1;
                            }
                        }
                    }
                    if constexpr (G::F) {
                        sq += __shfl_xor(sq, 16, 64);
                        sq += __shfl_xor(sq, 32, 64);
                    }
                    shift[tb] = 0.5f * sq;
                }
#pragma unroll
                for (int fbl = 0; fbl < FWB; ++fbl)
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        f32x4 u = zero4();
#pragma unroll
                        for (int kb = 0; kb < G::KBD; ++kb)
#pragma unroll
                            for (int part = 0; part < 2; ++part) u = mfma(wreg[fbl][kb][part], xb[tb][kb], u);
                        const int t = 16 * tb + c16;
                        const bool dead = mask_tail && t0 + t >= N;  // keys past the end: phi = 0
                        if constexpr (G::F) {
                            uint2 v = pack4(fast_exp(u[0] - shift[tb]) * inv_sqrt_m, fast_exp(u[1] - shift[tb]) * inv_sqrt_m,
                                            fast_exp(u[2] - shift[tb]) * inv_sqrt_m, fast_exp(u[3] - shift[tb]) * inv_sqrt_m);
                            if (dead) v = make_uint2(0, 0);
                            *reinterpret_cast<uint2 *>(&dst[t * RK + 64 * w + 16 * fbl + 4 * g]) = v;
                        } else {
                            float cv[4], sv[4];
#pragma unroll
                            for (int e = 0; e < 4; ++e) turn_cos_sin(u[e], cv[e], sv[e]);
                            uint2 vc = pack4(cv[0], cv[1], cv[2], cv[3]), vs = pack4(sv[0], sv[1], sv[2], sv[3]);
                            if (dead) vc = vs = make_uint2(0, 0);
                            *reinterpret_cast<uint2 *>(&dst[t * RK + 16 * w + 4 * g]) = vc;
                            *reinterpret_cast<uint2 *>(&dst[t * RK + G::M + 16 * w + 4 * g]) = vs;
                        }
                    }
            };
            if constexpr (NEED_K) project(sm.XK, sm.K[ks], true);
            if constexpr (OUT) project(sm.XQ, sm.QP, false);
            block_sync_lds();
            if constexpr (OUT) {
#pragma unroll
                for (int kf = 0; kf < KBF; ++kf) phq[kf].u = *reinterpret_cast<const uint4 *>(&sm.QP[row * RK + 32 * kf + 8 * g]);
            }
        }

        // ---------------- DPFP, one shift: with r = ReLU([x, -x]) (2d entries),
        // feature j = r_j r_{(j+1) mod 2d}.  phi(K) goes to LDS token-major in
        // 8-feature pieces; this lane's query pieces (features 32kf + 8g..)
        // come straight from the raw row.
        if constexpr (G::DPF) {
            auto piece = [&](const uint16_t *xr, int j0) {  // features j0..j0+7 of raw row xr
                float r[9];
#pragma unroll
                for (int e = 0; e < 9; ++e) {
                    const int j = (j0 + e) % (2 * DK);
                    const float x = bf16_to_f32(xr[j % DK]);
                    const float v = j < DK ? x : -x;
                    r[e] = v > 0.f ? v : 0.f;
                }
                uint4 o;
                o.x = cvt2(r[0] * r[1], r[1] * r[2]);
                o.y = cvt2(r[2] * r[3], r[3] * r[4]);
                o.z = cvt2(r[4] * r[5], r[5] * r[6]);
                o.w = cvt2(r[6] * r[7], r[7] * r[8]);
                return o;
            };
            if constexpr (NEED_K) {
                constexpr int PK = C * G::DP / 8 / G::THREADS;  // 8-feature pieces per thread
                static_assert(PK * G::THREADS * 8 == C * G::DP, "DPFP pieces must tile the workgroup");
#pragma unroll
                for (int i = 0; i < PK; ++i) {
                    const int u = tid + i * G::THREADS, t = u / (G::DP / 8), c8 = u % (G::DP / 8);
                    uint4 v = piece(&sm.XK[t * G::RX], 8 * c8);
                    if (t0 + t >= N) v = make_uint4(0, 0, 0, 0);  // keys past the end: phi = 0
                    *reinterpret_cast<uint4 *>(&sm.K[ks][t * RK + 8 * c8]) = v;
                }
            }
            if constexpr (OUT) {
#pragma unroll
                for (int kf = 0; kf < KBF; ++kf) phq[kf].u = piece(&sm.XQ[row * G::RX], 32 * kf + 8 * g);
            }
            block_sync_lds();
        }

        // ---------------- outputs of this wave's 16 query rows
        if constexpr (OUT) {
            f32x4 acc[NJ];
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) acc[nb] = zero4();
            // phi(Q) S_aug with the state carried into this chunk
            auto inter = [&]() {
#pragma unroll
                for (int kf = 0; kf < KBF; ++kf) {
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) {
                        Op8 sb;
                        sb.u = sm.STB[nb][kf][lane];
                        acc[nb] = mfma(phq[kf], sb, acc[nb]);
                    }
                }
            };
            // epilogue: divide by the normaliser column (retention: none), round,
            // stage, store 16 B per lane.  At d = 64 it runs inside each
            // query-block case, so the accumulators never pass a control-flow
            // join: for ELU+1 the compiler otherwise places some accumulating
            // products with the destination two registers above the accumulator
            // input, a placement the matrix cores do not read correctly (the
            // assembly test scans for it), and DPFP and cos/sin measured 0.5 us
            // faster so.  cosFormer (2 us less) and d = 128 (B2 H16 N16384: 182
            // against 192 us) keep one shared copy, which places none.
            constexpr bool EPI_IN_CASE = DK == 64 && PHI != kCosformer;
            auto epilogue = [&]() {
                float rden[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    rden[e] = RET ? 1.f : __builtin_amdgcn_rcpf(__shfl(acc[NJ - 1][e], lane & 48, 64));
                uint16_t *so = sm.O[w];
#pragma unroll
                for (int nb = 0; nb < DV / 16; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; e += 2) {
                        const uint32_t two = RET ? cvt2(acc[nb][e], acc[nb][e + 1])
                                                 : cvt2(acc[nb][e] * rden[e], acc[nb][e + 1] * rden[e + 1]);
                        so[(4 * g + e) * RO + 16 * nb + c16] = static_cast<uint16_t>(two);
                        so[(4 * g + e + 1) * RO + 16 * nb + c16] = static_cast<uint16_t>(two >> 16);
                    }
                wave_lds_sync();
                constexpr int PIECES = 16 * DV / 8;  // 16-byte pieces of the wave's 16 rows
                const auto ro = make_rsrc(Os + (size_t)t0 * DV, min(C, N - t0) * DV * 2);
#pragma unroll
                for (int it = 0; it < PIECES / 64; ++it) {
                    const int idx = it * 64 + lane;
                    const int r = idx / (DV / 8), c8 = idx % (DV / 8);
                    const uint4 val = *reinterpret_cast<const uint4 *>(&so[r * RO + 8 * c8]);
                    bstore16_nt(ro, 2 * ((16 * qb + r) * DV + 8 * c8), val);
                }
            };
            if constexpr (RET) {
                // retention reads the carried state first, scaled per query row by
                // lambda^(i+1) (the Lambda of the blockwise form), then adds the intra part
                inter();
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float r = dpow((float)(16 * qb + 4 * g + e + 1));
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) acc[nb][e] *= r;
                }
                if constexpr (INTRA) {
                    // (P (.) M) V_aug over the key blocks up to the diagonal
#pragma unroll
                    for (int kt = 0; kt < KBT; ++kt) {
                        if (2 * kt <= qb) {
                            f32x4 p[2];
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const int jb = 2 * kt + h;
                                p[h] = zero4();
                                if (jb <= qb) {
                                    const uint16_t *krow = &sm.K[ks][(16 * jb + c16) * RK];
#pragma unroll
                                    for (int kf = 0; kf < KBF; ++kf) {
                                        Op8 ka;
                                        ka.u = *reinterpret_cast<const uint4 *>(krow + 32 * kf + 8 * g);
                                        p[h] = mfma(ka, phq[kf], p[h]);
                                    }
                                    // decay mask lambda^(query - key), 0 above the diagonal
                                    if (jb == qb || !RFAC) {
#pragma unroll
                                        for (int e = 0; e < 4; ++e) {
                                            const int d = 16 * (qb - jb) + c16 - 4 * g - e;
                                            p[h][e] *= d >= 0 ? dpow((float)d) : 0.f;
                                        }
                                    } else {
                                        const float f = uni(dpow((float)(16 * (qb - jb - 1)))) * dec_lane;
#pragma unroll
                                        for (int e = 0; e < 4; ++e) p[h][e] *= f * dec_e[e];
                                    }
                                }
                            }
                            Op8 pa;
                            pa.q[0] = pack4(p[0][0], p[0][1], p[0][2], p[0][3]);
                            pa.q[1] = pack4(p[1][0], p[1][1], p[1][2], p[1][3]);
#pragma unroll
                            for (int nb = 0; nb < NJ; ++nb)
                                acc[nb] = mfma(pa, token_operand<RV>(sm.V[ks], kt, 16 * nb, lane), acc[nb]);
                        }
                    }
                }
                epilogue();
            } else {
                // The normalised maps take the query block as a compile-time
                // constant (qb is wave-uniform): the causal loop becomes straight
                // line and the key blocks' loads can be issued ahead.  Retention
                // keeps the run-time loop above (its decay factors spill the
                // registers of the unrolled form).
                dispatch_const<NW>(qb, [&](auto qbc) {
                    constexpr int QB = decltype(qbc)::value;
                    if constexpr (INTRA) {
                        // (P (.) M) V_aug over the key blocks up to the diagonal
#pragma unroll
                        for (int kt = 0; kt < KBT; ++kt) {
                            if (2 * kt <= QB) {
                                f32x4 p[2];
#pragma unroll
                                for (int h = 0; h < 2; ++h) {
                                    const int jb = 2 * kt + h;
                                    p[h] = zero4();
                                    if (jb <= QB) {
                                        const uint16_t *krow = &sm.K[ks][(16 * jb + c16) * RK];
#pragma unroll
                                        for (int kf = 0; kf < KBF; ++kf) {
                                            Op8 ka;
                                            ka.u = *reinterpret_cast<const uint4 *>(krow + 32 * kf + 8 * g);
                                            p[h] = mfma(ka, phq[kf], p[h]);
                                        }
                                        if (jb == QB) {  // causal mask on the diagonal block: key 4g+e <= query c16
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
                                for (int nb = 0; nb < NJ; ++nb)
                                    acc[nb] = mfma(pa, token_operand<RV>(sm.V[ks], kt, 16 * nb, lane), acc[nb]);
                            }
                        }
                    }
                    inter();
                    if constexpr (EPI_IN_CASE) epilogue();
                });
                if constexpr (!EPI_IN_CASE) epilogue();
            }
        }

        // ---------------- state update S_aug += phi(K_c)^T V_aug
        // (retention: S = lambda^Lc S + sum_t lambda^(Lc-1-t) phi(k_t) v_t^T over
        // the Lc tokens of the chunk; the key weights scale the operand slots)
        if constexpr (DO_STATE) {
            const int Lc = min(C, N - t0);
            if constexpr (RET) {
                const float carry = dpow((float)Lc);
#pragma unroll
                for (int q = 0; q < FBW; ++q)
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) S[q][nb] *= carry;
            }
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB) {
#pragma unroll
                    for (int kt = 0; kt < KBT; ++kt) {
                        Op8 ka = token_operand<RK>(sm.K[ks], kt, 16 * fb, lane);
                        if constexpr (RET) {
                            if (RFAC && Lc == C) {  // full chunk: products of powers
                                const float f = uni(dpow((float)(C - 32 - 32 * kt))) * kw_lane;
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    ka.u32[j] = cvt2(lo_bf16(ka.u32[j]) * (f * kw_slot[2 * j]),
                                                     hi_bf16(ka.u32[j]) * (f * kw_slot[2 * j + 1]));
                            } else {
                                // key weight of slot sl: token 32kt + 16(sl/4) + 4g + sl%4
                                auto kw = [&](int sl) {
                                    const int t = 32 * kt + 16 * (sl >> 2) + 4 * g + (sl & 3);
                                    return t < Lc ? dpow((float)(Lc - 1 - t)) : 0.f;
                                };
#pragma unroll
                                for (int j = 0; j < 4; ++j)
                                    ka.u32[j] = cvt2(lo_bf16(ka.u32[j]) * kw(2 * j), hi_bf16(ka.u32[j]) * kw(2 * j + 1));
                            }
                        }
#pragma unroll
                        for (int nb = 0; nb < NJ; ++nb)
                            S[q][nb] = mfma(ka, token_operand<RV>(sm.V[ks], kt, 16 * nb, lane), S[q][nb]);
                    }
                }
            }
        }
        pre_map(p);        // the chunk fetched above, mapped before the barrier
        block_sync_lds();  // every wave is done with this chunk's tiles and the old state image
        if constexpr (CARRY) {
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB) {
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb) put_state_block<G>(sm.STB, fb, nb, lane, S[q][nb]);
                }
            }
        }
    };
    // Single-pass hand-off between the segments of one slice.  The state is
    // additive over tokens ("Linear Attention", recurrent form), so the state
    // entering segment s is S_in + the sums of segments 0..s-1.
    //  * Segment 0 copies S_in into slot 0 when the launch starts (so no
    //    other workgroup reads S_in, and S_out may alias it).
    //  * Segment s < P-1 stores its sums into slot 1 + s with
    //    device-coherent stores, waits until they (and segment 0's copy of
    //    S_in) have completed, then tags flag s with this launch's tag.
    //  * Segment s > 0: one thread waits for flags 0..s-1 (each wait bounded
    //    in wall-clock time; on expiry the prefix becomes NaN and the error
    //    word is set, so a lost hand-off cannot hang the device), then every
    //    lane adds slots 0..s in ascending order, two slots in flight: S_in
    //    first, then the segments, the order of the separate scan kernel.
    //  * The last segment writes S_out = prefix + its own sums.
    // Slots hold the state in accumulator order: block (fb, nb) of S_aug is
    // 64 lanes x 4 floats, so each lane moves 16 bytes per block.
    constexpr int SLOT = G::DP * (DV + 16);  // floats per slot
    constexpr int PER = FBW * NJ;            // 16-byte pieces per lane per slot
    float *const slots = FUSED ? a.fu.slots + (size_t)bh * (sg.P + 1) * SLOT : nullptr;
    auto slot_rsrc = [&](int i, bool live) { return make_rsrc(slots + (size_t)i * SLOT, live ? SLOT * 4 : 0); };
    // Piece (fb, nb) of this lane.  In the normaliser block only column d_v
    // (lanes with c16 == 0) is data; the other lanes get an offset past the
    // slot, so their loads read zeros and their stores are dropped, moving
    // no bytes.
    auto piece_off = [&](int fb, int nb) {
        return !RET && nb == NJ - 1 && c16 != 0 ? SLOT * 4 : ((fb * NJ + nb) * 64 + lane) * 16;
    };
    auto store_slot = [&](int i) {  // this lane's pieces of S into slot i
        const auto r = slot_rsrc(i, true);
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int fb = w + NW * q;
            if (fb < FB)
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, S[q][nb]), r, piece_off(fb, nb),
                                                           0, kCoherent);
        }
    };
    auto load_slot = [&](f32x4 *dst, int i, bool live) {  // past the used slots: zeros, no access
        const auto r = slot_rsrc(i, live);
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int fb = min(w + NW * q, FB - 1);
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb)
                dst[q * NJ + nb] =
                    __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, piece_off(fb, nb), 0, kCoherent));
        }
    };
    uint32_t tag = 0;  // this launch's flag tag (thread 0)
    auto publish_and_gather = [&]() {
        const int P = sg.P;
        const bool has_in = a.st.S_src != nullptr;
        uint32_t *fl = a.fu.flags + (size_t)bh * P;
        if (seg < P - 1) {
            store_slot(1 + seg);
            wait_stores();  // every wave's stores have reached the coherence point ...
            __syncthreads();
            if (tid == 0)   // ... before the flag is tagged
                __hip_atomic_store(fl + seg, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        const bool last = seg == P - 1 && a.fu.S_out;
        if (last) store_slot(P);  // park the own sums
        // Wave 0 polls every earlier flag at once (lane i reads flag i, one
        // coalesced access per poll) until all carry this launch's tag.
        bool late = false;
        if (w == 0) {
            const uint32_t want = __shfl(tag, 0, 64);  // the tag lives in thread 0
            const long long t_begin = wall_clock64();
            for (int base = 0; base < seg; base += 64) {
                const int i = base + lane;
                while (true) {
                    const bool ok = i >= seg || __hip_atomic_load(fl + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == want;
                    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
                    if (wall_clock64() - t_begin > a.fu.spin_ticks) {
                        late = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(10);
                }
                if (late) break;
            }
        }
        late = __syncthreads_or(late);  // every flag was seen before any slot is read
        if (late && tid == 0) __hip_atomic_store(a.fu.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // prefix = S_in + sums(0) + ... + sums(seg - 1): slots 0..seg (slot 0 only with S_in)
#pragma unroll
        for (int q = 0; q < FBW; ++q)
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) S[q][nb] = zero4();
        // GD slots in flight (as many as the registers allow)
        constexpr int GD = PER > 6 ? 2 : C == 64 ? 8 : 4;
        f32x4 buf[GD][PER];
#pragma unroll
        for (int d = 0; d < GD; ++d) load_slot(buf[d], d, d == 0 ? has_in : d <= seg);
        // retention: the state decays across each segment, so slot j enters as
        // S = lambda^(tokens of segment j-1) S + slot j (Horner form)
        auto seg_len = [&](int k) { return min(sg.seg_chunks * C, N - k * sg.seg_chunks * C); };
        auto add_slot = [&](const f32x4 *src, int j) {
            const float mul = RET && j >= 1 && j <= seg ? dpow((float)seg_len(j - 1)) : 1.f;
#pragma unroll
            for (int q = 0; q < FBW; ++q)
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) {
                    if constexpr (RET) S[q][nb] = S[q][nb] * mul + src[q * NJ + nb];
                    else S[q][nb] += src[q * NJ + nb];
                }
        };
        for (int i = 0; i <= seg; i += GD) {  // a slot read as zeros adds exactly nothing
#pragma unroll
            for (int d = 0; d < GD; ++d) {
                add_slot(buf[d], i + d);
                load_slot(buf[d], i + d + GD, i + d + GD <= seg);
            }
        }
        if (late)
#pragma unroll
            for (int q = 0; q < FBW; ++q)
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) {
                    const float qn = __builtin_nanf("");
                    S[q][nb] = f32x4{qn, qn, qn, qn};
                }
        if (last) {
            float *So = a.fu.S_out + (size_t)bh * DV * G::DP;
            float *zo = a.fu.z_out + (size_t)bh * G::DP;
            f32x4 own[PER];
            load_slot(own, P, true);
            const float tail = RET ? dpow((float)seg_len(seg)) : 1.f;  // decay across the own segment
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB)
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int f = 16 * fb + 4 * g + e, j = 16 * nb + c16;
                            const float tot = RET ? tail * S[q][nb][e] + own[q * NJ + nb][e]
                                                  : S[q][nb][e] + own[q * NJ + nb][e];
                            if (j < DV) So[(size_t)f * DV + j] = tot;
                            else if (j == DV) zo[f] = tot;
                        }
            }
        }
#pragma unroll
        for (int q = 0; q < FBW; ++q) {
            const int fb = w + NW * q;
            if (fb < FB) {
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) put_state_block<G>(sm.STB, fb, nb, lane, S[q][nb]);
            }
        }
    };
    if constexpr (FUSED) {
        if (tid == 0) tag = __hip_atomic_load(a.fu.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
        if (seg == 0 && a.st.S_src) {  // slot 0 = S_in (S is still zero here)
            const float *Sin = a.st.S_src + bh * a.st.src_slice;
            const float *zin = a.st.z_src + bh * a.st.zsrc_slice;
#pragma unroll
            for (int q = 0; q < FBW; ++q) {
                const int fb = w + NW * q;
                if (fb < FB)
#pragma unroll
                    for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int f = 16 * fb + 4 * g + e, j = 16 * nb + c16;
                            S[q][nb][e] = j < DV ? Sin[(size_t)f * DV + j] : (j == DV ? zin[f] : 0.f);
                        }
            }
            store_slot(0);
#pragma unroll
            for (int q = 0; q < FBW; ++q)
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb) S[q][nb] = zero4();
        }
    }

    // Chunks go in pairs, then an odd last one: the loop back edge always
    // sees the same outstanding loads, so the waits stay partial.  Step s
    // uses ring slot s % 2.  (A one-slot ring walks the chunks one by one.)
    static_assert(DEPTH == 1 || DEPTH == 2, "ring of one or two slots");
    using Out = std::integral_constant<bool, DO_OUT>;
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) pre_map(pf[d]);
    if constexpr (DEPTH == 1) {
        if constexpr (!FUSED) {
            for (int c = c_begin; c < c_end; ++c) body(pf[0], c, c, Out{});
        } else {
            const int n = c_end - c_begin;
            for (int i = 0; i < n; ++i) body(pf[0], c_begin + p1_chunk(i), i, std::false_type{});
            publish_and_gather();
            for (int k = 0; k < n; ++k) body(pf[0], c_begin + k, n + k, std::true_type{});
        }
    } else if constexpr (!FUSED) {
        int c = c_begin;
        for (; c + 2 <= c_end; c += 2) {
            body(pf[0], c, c, Out{});
            body(pf[1], c + 1, c + 1, Out{});
        }
        if (c < c_end) body(pf[0], c, c, Out{});
    } else {
        const int n = c_end - c_begin, cbase = n + (n & 1);
        // ---- phase 1: this segment's own sums, S = 0 + sum phi(K)^T V_aug
        int i = 0;
        for (; i + 2 <= n; i += 2) {
            body(pf[0], c_begin + p1_chunk(i), i, std::false_type{});
            body(pf[1], c_begin + p1_chunk(i + 1), i + 1, std::false_type{});
        }
        if (i < n) {
            body(pf[0], c_begin + p1_chunk(i), i, std::false_type{});  // prefetches step cbase into slot 0
            fetch(pf[DEPTH - 1], cbase + 1);                  // slot 1 held the empty step n
        }
        // ---- phase 2: publish the sums, gather the prefix of the earlier segments
        publish_and_gather();
        if (i < n) pre_map(pf[DEPTH - 1]);
        // ---- phase 3: the chunk loop from the prefix state (step cbase + k = chunk k)
        int k = 0;
        for (; k + 2 <= n; k += 2) {
            body(pf[0], c_begin + k, cbase + k, std::true_type{});
            body(pf[1], c_begin + k + 1, cbase + k + 1, std::true_type{});
        }
        if (k < n) body(pf[0], c_begin + k, cbase + k, std::true_type{});
    }

    if constexpr (FUSED) {
        // the last workgroup of the launch to finish (all flag reads done)
        // advances the launch counter and clears the done count
        if (tid == 0) {
            const uint32_t done =
                __hip_atomic_fetch_add(a.fu.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (done == gridDim.x - 1) {
                __hip_atomic_store(a.fu.ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.fu.ctl, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    // ---- final state of the range
    if (!FUSED && DO_STATE && a.st.S_dst) {
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
hipError_t launch_variant(const FwdArgs &a, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)((size_t)a.sh.BH * a.sg.P)), block(C / 16 * 64);
    if (a.mode == kModeFusedRes) {
        if constexpr (DK == 64 && DV == 64 && C == 64 && (PHI == kElu1 || PHI == kIdentity))
            return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeFusedRes>, grid, block, 0, st, ev, a);
        return hipErrorNotSupported;
    }
    if constexpr (PHI == kIdentity) {  // retention: causal only
        if (a.mode == kModeFused)
            return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeFused>, grid, block, 0, st, ev, a);
        if (a.mode == kModeCausal)
            return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeCausal>, grid, block, 0, st, ev, a);
        return hipErrorNotSupported;
    } else {
        switch (a.mode) {
            case kModeState: return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeState>, grid, block, 0, st, ev, a);
            case kModeCausal: return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeCausal>, grid, block, 0, st, ev, a);
            case kModeFused: return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeFused>, grid, block, 0, st, ev, a);
            default: return launch_kernel_ev(k_mfma<DK, DV, C, PHI, kModeRead>, grid, block, 0, st, ev, a);
        }
    }
}

}  // namespace

bool mfma_supported(const Shape &sh, int chunk) {
    if (sh.dtype != kBF16) return false;
    if ((sh.phi == kIdentity) != (sh.ret != 0)) return false;  // identity map <=> retention here
    if (sh.phi == kElu1 || sh.phi == kIdentity)
        return ((sh.dk == 64 && sh.dv == 64) || (sh.dk == 128 && sh.dv == 128)) && (chunk == 64 || chunk == 128);
    if (sh.phi == kFavor) return sh.dk == 64 && sh.dv == 64 && sh.m == 256 && chunk == 64;
    if (sh.phi == kCosformer) return sh.dk == 64 && sh.dv == 64 && chunk == 64;
    if (sh.phi == kDpfp) return sh.dk == 64 && sh.dv == 64 && sh.param == 1 && chunk == 64;
    if (sh.phi == kTrig) return sh.dk == 64 && sh.dv == 64 && sh.m == 64 && chunk == 64;
    return false;  // the other maps run on the fp32-arithmetic kernels
}

hipError_t launch_mfma(const FwdArgs &a, hipStream_t st, KEvents ev) {
    const Shape &s = a.sh;
    const int C = a.sg.chunk;
    if (!mfma_supported(s, C)) return hipErrorNotSupported;
    if (s.phi == kFavor) return launch_variant<64, 64, 64, kFavor>(a, st, ev);
    if (s.phi == kCosformer) return launch_variant<64, 64, 64, kCosformer>(a, st, ev);
    if (s.phi == kDpfp) return launch_variant<64, 64, 64, kDpfp>(a, st, ev);
    if (s.phi == kTrig) return launch_variant<64, 64, 64, kTrig>(a, st, ev);
    if (s.phi == kIdentity) {
        if (s.dk == 64)
            return C == 64 ? launch_variant<64, 64, 64, kIdentity>(a, st, ev)
                           : launch_variant<64, 64, 128, kIdentity>(a, st, ev);
        return C == 64 ? launch_variant<128, 128, 64, kIdentity>(a, st, ev)
                       : launch_variant<128, 128, 128, kIdentity>(a, st, ev);
    }
    if (s.dk == 64)
        return C == 64 ? launch_variant<64, 64, 64, kElu1>(a, st, ev) : launch_variant<64, 64, 128, kElu1>(a, st, ev);
    return C == 64 ? launch_variant<128, 128, 64, kElu1>(a, st, ev) : launch_variant<128, 128, 128, kElu1>(a, st, ev);
}

}  // namespace la
