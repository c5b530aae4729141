// FAVOR+ single pass on the matrix cores: bf16 storage, d_k = d_v = 64,
// m = 256 random features, 64-token chunks, eight waves per workgroup.
//
// Feature map ("Story of Attention Part 5", section 2, Performer positive
// random features): phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), r = 1..m.
// Causal normalised linear attention in chunkwise form ("Linear Attention",
// chunkwise parallel form; "Story of Attention Part 5", section 6 with decay
// 1) with the normaliser carried as an extra value column, and the state
// entering each segment handed on between the segments of a slice through
// the workspace (the state is additive over tokens: "Linear Attention",
// recurrent form).
//
// One workgroup per (slice, segment), 512 threads, two waves per SIMD.
//  * Wave w owns features 32w..32w+31: it holds their rows of W (bf16 hi and
//    lo parts) in registers, projects those features of every token of a
//    chunk, and carries the matching 32 rows of the fp32 state S_aug =
//    [S | z | 0..] in its accumulators.
//  * Phase 1 (the segment's own sums) projects K as X W^T, so a lane's
//    accumulators hold four tokens of one feature: after the exponent they are
//    the A operand of phi(K)^T V_aug as they stand, with no LDS round trip.
//  * Phase 3 (outputs) projects K and Q as W X^T into token-major LDS rows;
//    the outputs of query block qb are split over two waves by feature half
//    (h = 0: features 0..127, h = 1: 128..255): each forms the causal scores,
//    their value product and the read of the carried state over its half, and
//    the h = 1 wave hands its partial sums to the h = 0 wave through LDS,
//    which divides and stores.  The pairs are placed so that every SIMD holds
//    query blocks s and 3 - s (equal shares of the causal triangle).
//  * Between the phases the segment publishes its sums and gathers the sums
//    of the earlier segments of its slice (flags tagged per launch, bounded
//    waits), as in the chunk-loop kernel.
#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_ops.h"

namespace la {
namespace {

constexpr int kFC = 64;                // tokens per chunk
constexpr int kFD = 64;                // d_k = d_v
constexpr int kFM = 256;               // random features m
constexpr int kFW = 8;                 // waves
constexpr int kFT = 64 * kFW;          // threads
constexpr int kFNJ = kFD / 16 + 1;     // value column blocks incl. the normaliser block
constexpr int kFKBF = kFM / 32;        // 32-feature k-blocks
constexpr int kFRK = kFM + 8;          // phi row stride (16-row 128-bit reads conflict free)
constexpr int kFRV = kFD + 16;         // V_aug row stride: 40 dwords (5 x 8 mod 64), the eight rows of a
                                        // transposed read fall on disjoint bank groups
constexpr int kFRX = kFD + 8;          // raw row stride
constexpr int kFRO = kFD + 8;          // output staging row stride
constexpr int kFSlot = kFM * (kFD + 16);  // floats per hand-off slot
static_assert(kFW * 32 == kFM, "one wave per 32 features");
static_assert(4 * 16 * kFRO <= kFC * kFRX, "output staging fits in the raw key rows");

struct FavorSmem {
    uint16_t XK[kFC * kFRX];        // raw K rows; output staging of the h = 0 waves later in the chunk
    uint16_t XQ[kFC * kFRX];        // raw Q rows
    uint16_t K[kFC * kFRK];         // phi(K) token-major
    uint16_t QP[kFC * kFRK];        // phi(Q) token-major
    uint16_t V[kFC * kFRV];         // V_aug token-major
    uint4 STB[kFNJ][kFKBF][64];     // bf16 S_aug: B operand of phi(Q) S
    f32x4 X[4][kFNJ][64];           // partial outputs of the h = 1 waves, per query block
    float SH[2][kFC];               // per token of K, Q: exponent shift (|x|^2 / 2 + ln 16) * log2(e)
};

// 16x16 fp32 state tile (lane l: rows 16fb + 4g + e, column 16nb + l%16)
// into the bf16 B-operand image of S_aug
__device__ __forceinline__ void put_state(uint4 (*STB)[kFKBF][64], int fb, int nb, int lane, f32x4 s) {
    const int g = lane >> 4, c = lane & 15;
    const uint2 v = pack4(s[0], s[1], s[2], s[3]);
    const int x = 16 * (fb & 1) + 4 * g;  // feature slot inside the 32-feature k-block
    reinterpret_cast<uint2 *>(&STB[nb][fb >> 1][c + 16 * (x >> 3)])[(x >> 2) & 1] = v;
}

__global__ __launch_bounds__(kFT) void k_favor(FwdArgs a) {
    __shared__ FavorSmem sm;
    using T = uint16_t;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    const Segments sg = a.sg;
    const int N = a.sh.N, P = sg.P;
    int bh, seg;
    seg_of_block(blockIdx.x, a.sh.BH, P, bh, seg);
    const int c_begin = seg * sg.seg_chunks;
    const int n = min(sg.n_chunks, c_begin + sg.seg_chunks) - c_begin;  // chunks of this segment (>= 1)

    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * kFD;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * kFD;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * kFD;
    T *Os = static_cast<T *>(a.O) + (size_t)bh * N * kFD;

    // W rows of this wave's features 32w + 16fbl + c16, columns 32kb + 8g..+7,
    // split W = W_hi + W_lo with both parts bf16: the inputs are exact in
    // bf16, so x . w_r = x . hi_r + x . lo_r to about 2^-16 relative, where a
    // single bf16 W would move every exponent by ~2^-9 |w_r| |x|.  The same
    // registers serve as the A operand of W X^T and the B operand of X W^T.
    Op8 wr[2][2][2];  // [fbl][kb][hi, lo]
#pragma unroll
    for (int fbl = 0; fbl < 2; ++fbl)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const float *src = a.sh.W + (size_t)(32 * w + 16 * fbl + c16) * kFD + 32 * kb + 8 * g;
            const float4 w0 = *reinterpret_cast<const float4 *>(src);
            const float4 w1 = *reinterpret_cast<const float4 *>(src + 4);
            const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const uint32_t h2 = cvt2(wv[e], wv[e + 1]);
                wr[fbl][kb][0].u32[e / 2] = h2;
                wr[fbl][kb][1].u32[e / 2] = cvt2(wv[e] - lo_bf16(h2), wv[e + 1] - hi_bf16(h2));
            }
        }
    constexpr float kLog2e = 1.44269504088896341f;

    // output role: feature half h, query block qb (SIMD w % 4 holds blocks s and 3 - s)
    const int h = w >> 2;
    const int qb = h == 0 ? w : 7 - w;
    const int row = 16 * qb + c16;

    // ---- prefetch ring: one 16-byte piece of K, V and Q per thread and chunk.
    // Steps 0..n-1 are phase 1 (the segment's chunks, last to first, keys and
    // values only); phase 3 runs chunk k at step cbase + k, cbase even, so it
    // starts on ring slot 0 (step n of an odd segment is empty).
    struct Pref {
        uint4 k, v, q;
    };
    Pref pf[2];
    const int cbase = n + (n & 1);
    auto fetch = [&](Pref &p, int s) {
        const bool pa = s < n, pc = s >= cbase && s < cbase + n;
        const int cc = c_begin + (pa ? n - 1 - s : (pc ? s - cbase : 0));
        const int tt0 = cc * kFC;
        const int rows = (pa || pc) ? min(kFC, N - tt0) : 0;
        const int qrows = pc ? rows : 0;
        p.k = bload16(make_rsrc(Ks + (size_t)tt0 * kFD, rows * kFD * 2), 16 * tid);
        p.v = bload16(make_rsrc(Vs + (size_t)tt0 * kFD, rows * kFD * 2), 16 * tid);
        p.q = bload16_nt(make_rsrc(Qs + (size_t)tt0 * kFD, qrows * kFD * 2), 16 * tid);
    };
    // piece tid of a chunk is row tid / 8, columns 8 (tid % 8).  The eight
    // lanes of a row also form its exponent shift in the log2 domain,
    // (|x|^2 / 2) log2(e) + 4 (the 1/sqrt(m) = 2^-4 factor folded in), so
    // that phi = exp2(u log2(e) - shift) for u = w . x; keys past the end get
    // an infinite shift, i.e. phi = 0.
    const int st_t = tid >> 3, st_c = 8 * (tid & 7);
    auto row_shift = [&](uint4 x, bool valid) {
        float sq = 0.f;
        const uint32_t xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = lo_bf16(xs[e]), v1 = hi_bf16(xs[e]);
            sq = fmaf(v0, v0, sq);
            sq = fmaf(v1, v1, sq);
        }
        sq = group8_sum(sq);
        return valid ? fmaf(sq, 0.5f * kLog2e, 4.0f) : __builtin_inff();
    };
    auto stage = [&](const Pref &p, int t0, bool with_q) {
        *reinterpret_cast<uint4 *>(&sm.XK[st_t * kFRX + st_c]) = p.k;
        *reinterpret_cast<uint4 *>(&sm.V[st_t * kFRV + st_c]) = p.v;
        const float shk = row_shift(p.k, t0 + st_t < N);
        if ((tid & 7) == 0) sm.SH[0][st_t] = shk;
        if (with_q) {
            *reinterpret_cast<uint4 *>(&sm.XQ[st_t * kFRX + st_c]) = p.q;
            const float shq = row_shift(p.q, true);
            if ((tid & 7) == 0) sm.SH[1][st_t] = shq;
        }
    };
    fetch(pf[0], 0);
    fetch(pf[1], 1);

    // normaliser block of V_aug: column d_v is 1 for every token, columns
    // d_v+1..d_v+15 are 0 (tokens past the end have phi(k) = 0)
    for (int u = tid; u < kFC * 2; u += kFT) {
        const int t = u >> 1, half = u & 1;
        *reinterpret_cast<uint4 *>(&sm.V[t * kFRV + kFD + 8 * half]) = make_uint4(half == 0 ? 0x3f80u : 0u, 0, 0, 0);
    }

    f32x4 S[2][kFNJ];  // state rows 32w + 16fbl + 4g + e, columns 16nb + c16
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int nb = 0; nb < kFNJ; ++nb) S[q][nb] = zero4();

    // raw rows of token block tb (A or B operand: row 16tb + c16, columns 32kb + 8g..)
    auto load_rows = [&](const uint16_t *xr, Op8 (&xb)[4][2]) {
#pragma unroll
        for (int tb = 0; tb < 4; ++tb)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
                xb[tb][kb].u = *reinterpret_cast<const uint4 *>(&xr[(16 * tb + c16) * kFRX + 32 * kb + 8 * g]);
    };

    // ---- phase 1 chunk: S += phi(K)^T V_aug over the chunk, phi(K) from
    // the projection accumulators (X W^T: lane holds tokens 16tb + 4g + e of
    // feature 32w + 16fbl + c16).  For k-block kt the two token blocks 2kt,
    // 2kt+1 give slots 8g + e <-> token 32kt + 16(e/4) + 4g + e%4, the order
    // of the transpose-read value operands.
    auto sums_chunk = [&](Pref &p, int c, int step) {
        stage(p, c * kFC, false);
        block_sync_lds();
        fetch(p, step + 2);
        Op8 xb[4][2];
        load_rows(sm.XK, xb);
        float4 shv[4];  // shifts of tokens 16tb + 4g + e
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) shv[tb] = *reinterpret_cast<const float4 *>(&sm.SH[0][16 * tb + 4 * g]);
        Op8 ka[2][2];  // [fbl][kt]
#pragma unroll
        for (int fbl = 0; fbl < 2; ++fbl) {
            f32x4 u[4];  // the four token blocks' chains, issued interleaved
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) u[tb] = zero4();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int part = 0; part < 2; ++part)
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) u[tb] = mfma(xb[tb][kb], wr[fbl][kb][part], u[tb]);
            float ph[4][4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float shf[4] = {shv[tb].x, shv[tb].y, shv[tb].z, shv[tb].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) ph[tb][e] = __builtin_amdgcn_exp2f(fmaf(u[tb][e], kLog2e, -shf[e]));
            }
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                ka[fbl][kt].u32[0] = cvt2(ph[2 * kt][0], ph[2 * kt][1]);
                ka[fbl][kt].u32[1] = cvt2(ph[2 * kt][2], ph[2 * kt][3]);
                ka[fbl][kt].u32[2] = cvt2(ph[2 * kt + 1][0], ph[2 * kt + 1][1]);
                ka[fbl][kt].u32[3] = cvt2(ph[2 * kt + 1][2], ph[2 * kt + 1][3]);
            }
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) {
                const Op8 vo = token_operand<kFRV>(sm.V, kt, 16 * nb, lane);
                S[0][nb] = mfma(ka[0][kt], vo, S[0][nb]);
                S[1][nb] = mfma(ka[1][kt], vo, S[1][nb]);
            }
        block_sync_lds();  // raw keys and values consumed before the next chunk is staged
    };

    // ---- phase 3 chunk: projections into LDS, outputs, state update
    auto out_chunk = [&](Pref &p, int c, int step) {
        const int t0 = c * kFC;
        stage(p, t0, true);
        block_sync_lds();
        fetch(p, step + 2);
        // W X^T: accumulator lane (4g+e, c16) of tile (fbl, tb) holds feature
        // 32w + 16fbl + 4g + e of token 16tb + c16; phi goes to LDS token-major
        auto project = [&](const uint16_t *xr, const float *shift, uint16_t *dst) {
            Op8 xb[4][2];
            load_rows(xr, xb);
            float shv[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) shv[tb] = shift[16 * tb + c16];
#pragma unroll
            for (int fbl = 0; fbl < 2; ++fbl) {
                f32x4 u[4];  // the four token blocks' chains, issued interleaved
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) u[tb] = zero4();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int part = 0; part < 2; ++part)
#pragma unroll
                        for (int tb = 0; tb < 4; ++tb) u[tb] = mfma(wr[fbl][kb][part], xb[tb][kb], u[tb]);
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    auto ph = [&](int e) { return __builtin_amdgcn_exp2f(fmaf(u[tb][e], kLog2e, -shv[tb])); };
                    *reinterpret_cast<uint2 *>(&dst[(16 * tb + c16) * kFRK + 32 * w + 16 * fbl + 4 * g]) =
                        pack4(ph(0), ph(1), ph(2), ph(3));
                }
            }
        };
        project(sm.XK, sm.SH[0], sm.K);
        project(sm.XQ, sm.SH[1], sm.QP);
        block_sync_lds();

        // outputs of query block qb over feature half h: k-blocks 4h..4h+3
        Op8 phq[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) phq[j].u = *reinterpret_cast<const uint4 *>(&sm.QP[row * kFRK + 32 * (4 * h + j) + 8 * g]);
        f32x4 acc[kFNJ];
#pragma unroll
        for (int nb = 0; nb < kFNJ; ++nb) acc[nb] = zero4();
        // the causal structure of query block qb as constants (qb is wave-uniform)
        dispatch_const<4>(qb, [&](auto qbc) {
            constexpr int QB = decltype(qbc)::value;
            // (P (.) M) V_aug, P^T = phi(K) phi(Q)^T computed transposed so that two
            // consecutive accumulator tiles are the A operand of the value product
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) {
                if (2 * kt <= QB) {
                    f32x4 pt[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int jb = 2 * kt + hh;
                        pt[hh] = zero4();
                        if (jb <= QB) {
                            const uint16_t *krow = &sm.K[(16 * jb + c16) * kFRK + 128 * h + 8 * g];
#pragma unroll
                            for (int j = 0; j < 4; ++j) {
                                Op8 ka;
                                ka.u = *reinterpret_cast<const uint4 *>(krow + 32 * j);
                                pt[hh] = mfma(ka, phq[j], pt[hh]);
                            }
                            if (jb == QB) {  // causal mask on the diagonal block: key 4g+e <= query c16
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    if (4 * g + e > c16) pt[hh][e] = 0.f;
                            }
                        }
                    }
                    Op8 pa;
                    pa.q[0] = pack4(pt[0][0], pt[0][1], pt[0][2], pt[0][3]);
                    pa.q[1] = pack4(pt[1][0], pt[1][1], pt[1][2], pt[1][3]);
#pragma unroll
                    for (int nb = 0; nb < kFNJ; ++nb) acc[nb] = mfma(pa, token_operand<kFRV>(sm.V, kt, 16 * nb, lane), acc[nb]);
                }
            }
            // phi(Q) S_aug with the state carried into this chunk
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int nb = 0; nb < kFNJ; ++nb) {
                    Op8 sb;
                    sb.u = sm.STB[nb][4 * h + j][lane];
                    acc[nb] = mfma(phq[j], sb, acc[nb]);
                }
        });
        if (h == 1) {
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) sm.X[qb][nb][lane] = acc[nb];
        }
        block_sync_lds();  // partial sums visible; every read of the state image done

        if (h == 0) {
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) acc[nb] += sm.X[qb][nb][lane];
            // epilogue: divide by the normaliser column (column d_v: lanes with c16 = 0)
            float rden[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) rden[e] = __builtin_amdgcn_rcpf(__shfl(acc[kFNJ - 1][e], lane & 48, 64));
            uint16_t *so = &sm.XK[w * 16 * kFRO];
#pragma unroll
            for (int nb = 0; nb < kFD / 16; ++nb)
#pragma unroll
                for (int e = 0; e < 4; e += 2) {
                    const uint32_t two = cvt2(acc[nb][e] * rden[e], acc[nb][e + 1] * rden[e + 1]);
                    so[(4 * g + e) * kFRO + 16 * nb + c16] = static_cast<uint16_t>(two);
                    so[(4 * g + e + 1) * kFRO + 16 * nb + c16] = static_cast<uint16_t>(two >> 16);
                }
            wave_lds_sync();
            const auto ro = make_rsrc(Os + (size_t)t0 * kFD, min(kFC, N - t0) * kFD * 2);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int idx = it * 64 + lane;
                const int r = idx >> 3, c8 = idx & 7;
                bstore16_nt(ro, 2 * ((16 * qb + r) * kFD + 8 * c8), *reinterpret_cast<const uint4 *>(&so[r * kFRO + 8 * c8]));
            }
        }

        // state update S_aug += phi(K)^T V_aug (transpose reads of phi(K))
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
            const Op8 k0 = token_operand<kFRK>(sm.K, kt, 32 * w, lane);
            const Op8 k1 = token_operand<kFRK>(sm.K, kt, 32 * w + 16, lane);
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) {
                const Op8 vo = token_operand<kFRV>(sm.V, kt, 16 * nb, lane);
                S[0][nb] = mfma(k0, vo, S[0][nb]);
                S[1][nb] = mfma(k1, vo, S[1][nb]);
            }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) put_state(sm.STB, 2 * w + q, nb, lane, S[q][nb]);
        block_sync_lds();  // new state image visible; chunk tiles consumed
    };

    // ---- hand-off.  Slot 0 of a slice holds S_in, slot 1 + s the sums of
    // segment s, slot P the last segment's own sums; a slot is the state in
    // accumulator order (block (fb, nb): 64 lanes x 16 bytes).  In the
    // normaliser block only column d_v (lanes with c16 = 0) is data; the other
    // lanes get an offset past the slot, so their loads read zeros and their
    // stores are dropped.
    float *const slots = a.fu.slots + (size_t)bh * (P + 1) * kFSlot;
    auto slot_rsrc = [&](int i, bool live) { return make_rsrc(slots + (size_t)i * kFSlot, live ? kFSlot * 4 : 0); };
    auto piece_off = [&](int fb, int nb) {
        return nb == kFNJ - 1 && c16 != 0 ? kFSlot * 4 : ((fb * kFNJ + nb) * 64 + lane) * 16;
    };
    auto store_slot = [&](int i) {
        const auto r = slot_rsrc(i, true);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, S[q][nb]), r, piece_off(2 * w + q, nb), 0,
                                                       kCoherent);
    };
    auto load_slot = [&](f32x4 (&dst)[2][kFNJ], int i, bool live) {  // not live: zeros, no access
        const auto r = slot_rsrc(i, live);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb)
                dst[q][nb] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, piece_off(2 * w + q, nb), 0, kCoherent));
    };

    uint32_t tag = 0;  // this launch's flag tag (thread 0)
    if (tid == 0) tag = __hip_atomic_load(a.fu.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    const bool has_in = a.st.S_src != nullptr;
    if (seg == 0 && has_in) {  // slot 0 = S_in, so that only this workgroup reads S_in (S_out may alias it)
        const float *Sin = a.st.S_src + bh * a.st.src_slice;
        const float *zin = a.st.z_src + bh * a.st.zsrc_slice;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int f = 32 * w + 16 * q + 4 * g + e, j = 16 * nb + c16;
                    S[q][nb][e] = j < kFD ? Sin[(size_t)f * kFD + j] : (j == kFD ? zin[f] : 0.f);
                }
        store_slot(0);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) S[q][nb] = zero4();
    }
    block_sync_lds();  // normaliser block of V_aug in place

    // ---- phase 1: this segment's own sums, chunks last to first (phase 3
    // then starts on the chunks read last, the likeliest still in cache)
    {
        int i = 0;
        for (; i + 2 <= n; i += 2) {
            sums_chunk(pf[0], c_begin + n - 1 - i, i);
            sums_chunk(pf[1], c_begin + n - 2 - i, i + 1);
        }
        if (i < n) {
            sums_chunk(pf[0], c_begin + n - 1 - i, i);  // prefetches step cbase into slot 0
            fetch(pf[1], cbase + 1);                    // slot 1 held the empty step n
        }
    }

    // ---- phase 2: publish the sums, gather S_in + the sums of segments 0..seg-1
    {
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
        // wave 0 polls every earlier flag at once (lane i reads flag i)
        bool late = false;
        if (w == 0) {
            const uint32_t want = __shfl(tag, 0, 64);
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
        late = __syncthreads_or(late);  // every flag seen before any slot is read
        if (late && tid == 0) __hip_atomic_store(a.fu.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // prefix in ascending slot order, two slots in flight (a slot read as zeros adds nothing)
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) S[q][nb] = zero4();
        f32x4 buf[2][2][kFNJ];
        load_slot(buf[0], 0, has_in);
        load_slot(buf[1], 1, 1 <= seg);
        for (int i = 0; i <= seg; i += 2) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int nb = 0; nb < kFNJ; ++nb) S[q][nb] += buf[d][q][nb];
                load_slot(buf[d], i + d + 2, i + d + 2 <= seg);
            }
        }
        if (late) {
            const float qn = __builtin_nanf("");
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int nb = 0; nb < kFNJ; ++nb) S[q][nb] = f32x4{qn, qn, qn, qn};
        }
        if (last) {  // S_out = prefix + own sums
            float *So = a.fu.S_out + (size_t)bh * kFD * kFM;
            float *zo = a.fu.z_out + (size_t)bh * kFM;
            f32x4 own[2][kFNJ];
            load_slot(own, P, true);
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int nb = 0; nb < kFNJ; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 32 * w + 16 * q + 4 * g + e, j = 16 * nb + c16;
                        const float tot = S[q][nb][e] + own[q][nb][e];
                        if (j < kFD) So[(size_t)f * kFD + j] = tot;
                        else if (j == kFD) zo[f] = tot;
                    }
        }
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int nb = 0; nb < kFNJ; ++nb) put_state(sm.STB, 2 * w + q, nb, lane, S[q][nb]);
    }

    // ---- phase 3: the chunk loop from the prefix state (step cbase + k = chunk k)
    {
        int k = 0;
        for (; k + 2 <= n; k += 2) {
            out_chunk(pf[0], c_begin + k, cbase + k);
            out_chunk(pf[1], c_begin + k + 1, cbase + k + 1);
        }
        if (k < n) out_chunk(pf[0], c_begin + k, cbase + k);
    }

    // the last workgroup of the launch to finish advances the launch counter
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.fu.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(a.fu.ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.fu.ctl, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

bool favor_supported(const Shape &sh, const Segments &g) {
    return sh.dtype == kBF16 && sh.phi == kFavor && sh.ret == 0 && sh.dk == kFD && sh.dv == kFD && sh.m == kFM &&
           g.chunk == kFC && g.P > 1;
}

hipError_t launch_favor(const FwdArgs &a, hipStream_t st, KEvents ev) {
    if (!favor_supported(a.sh, a.sg) || a.mode != kModeFused) return hipErrorNotSupported;
    const dim3 grid((unsigned)((size_t)a.sh.BH * a.sg.P)), block(kFT);
    return launch_kernel_ev(k_favor, grid, block, 0, st, ev, a);
}

}  // namespace la
