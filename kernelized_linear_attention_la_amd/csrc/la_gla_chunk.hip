// GLA's gated recurrence in chunkwise form ("Linear Attention" (aiwiki.ai),
// gated linear attention; the same recurrence as the token-by-token kernel
// in la_gated.hip, S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t).
//
// Unrolled over a chunk of C tokens that starts from S_0, with the gates'
// cumulative logs l_t = sum_{s <= t} log2 alpha_s (per key channel, from the
// chunk's first token; base 2, the hardware's exp2 and log2):
//   o_i = S_0^T (q_i * 2^{l_i}) + sum_{t <= i} [sum_c q_ic k_tc 2^{l_ic - l_tc}] v_t
//   S_C = diag(2^{l_C}) S_0 + sum_t (k_t * 2^{l_C - l_t}) v_t^T
// Every factor 2^{l_i - l_t} with t <= i is a product of gates, at most 1.
// The pair sum over channels becomes a matrix product once the factor is
// split at a pivot p (per channel): 2^{l_i - p} 2^{p - l_t}.  Query block I
// takes p = l at its own first token: the query part is at most 1 for every
// key block, the key part is at most 1 for the earlier key blocks and at most
// the block's own decay on the diagonal block; when that exceeds 2^86 for
// some channel, the diagonal block is summed element by element instead (the
// exact form, slower), so no value can overflow whatever the gates.
// The sums are kept per 16-token block (local sums from the block's first
// token, plus block totals), and every exponent is formed as a short sum of
// those: a difference of two long cumulative sums would lose the small
// exponents of close pairs once tiny gates have made the sums large.
//
// One workgroup of 4 waves owns 16 value columns of one (b, h) slice and
// walks its chunks in order, the 64 x 16 state slice in accumulators (wave
// w: feature rows 16w..16w+15).  Wave w owns query rows 16w..16w+15 of each
// chunk.  All products are v_mfma_f32_16x16x4_f32 (fp32 operands): for that
// instruction lane l supplies A[l%16][l/16] and B[l/16][l%16] of each
// 16x4 by 4x16 step and receives D[4(l/16)+e][l%16].  In step ks, k-slot g
// is channel (or token) 16g + ks, so each lane walks a contiguous 16-wide
// run of its row and reads it with 16-byte LDS loads.  d_k <= 64 (zero
// padded; gates of padded channels count as 1).
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;       // tokens per chunk
constexpr int kK = 64;       // key channels (d_k padded)
constexpr int kNC = 16;      // value columns per workgroup
constexpr int kNW = 4;       // waves
constexpr int kThreads = 64 * kNW;
constexpr int kRS = kK + 4;  // row stride of the 64-wide tiles (floats)
constexpr float kPivotBound = 86.f;  // largest diagonal-block decay (in log2) taken through the pivot

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }  // v_exp_f32
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }   // v_log_f32

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ f32x4 mma(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// bf16 matrix-instruction operands (v_mfma_f32_16x16x32_bf16: lane l supplies
// A[l%16][8(l/16)..+7] and B[8(l/16)..+7][l%16]) and the split of fp32 values
// into bf16 hi and lo parts, x = hi + lo to about 2^-17 relative
typedef __bf16 gbf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 gbf16x2 __attribute__((ext_vector_type(2)));
typedef float gf32x2 __attribute__((ext_vector_type(2)));
union B8 {
    gbf16x8 v;
    uint32_t u[4];
};
__device__ __forceinline__ uint32_t bf2(float a, float b) {  // round to nearest even
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(gf32x2{a, b}, gbf16x2));
}
__device__ __forceinline__ void split8(const float (&x)[8], B8 &hi, B8 &lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t h = bf2(x[2 * e], x[2 * e + 1]);
        hi.u[e] = h;
        lo.u[e] = bf2(x[2 * e] - __uint_as_float(h << 16), x[2 * e + 1] - __uint_as_float(h & 0xffff0000u));
    }
}
__device__ __forceinline__ f32x4 mma8(const B8 &a, const B8 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

struct GlaSmem {
    float Q[kC][kRS];      // q rows (raw)
    float K[kC][kRS];      // k rows (raw)
    float L[kC][kRS];      // log2 gates summed from the first token of each 16-token block
    float KET[kK][kRS];    // [feature][token]: k_t 2^{l_last - l_t}, the state update's operand
    float VT[kNC][kRS];    // [value column][token]
    float ST[kNC][kRS];    // [value column][feature]: the state entering the chunk
    float W[kNW][16][kRS];  // per-wave scores [query row][token]
    float tot[4][kK];      // per 16-token block: the sum of its log2 gates
    int big[kNW];          // diagonal block b decays by more than 2^86 in some channel
};

// The per-chunk preparation (k_gla_prep) has its own 70 KB layout, so two of
// its workgroups share a CU (the one-launch kernel's layout, 97 KB, allows one).
struct GlaPrepSmem {
    float Q[kC][kRS];   // q rows; later V^T [value column][token]
    float K[kC][kRS];
    float L[kC][kRS];
    float KE[kK][kRS];  // decayed keys [channel][token]
    float tot[4][kK];
    int big[kNW];
};

// 16 consecutive floats of an LDS row (16-byte aligned) into registers
__device__ __forceinline__ void row16(const float *p, float (&r)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 v = *reinterpret_cast<const float4 *>(p + 4 * j);
        r[4 * j] = v.x; r[4 * j + 1] = v.y; r[4 * j + 2] = v.z; r[4 * j + 3] = v.w;
    }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_gla_chunk(GatedArgs a) {
    __shared__ __align__(16) GlaSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int dk = a.dk, dv = a.dv, N = a.N;
    const int bh = blockIdx.x, col0 = kNC * blockIdx.y;
    const int ncol = min(kNC, dv - col0);
    const T *Q = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *K = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *V = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *O = static_cast<T *>(a.O) + (size_t)bh * N * dv;
    const float *Al = a.alpha + (size_t)bh * N * dk;

    // the state slice: wave w holds feature rows 16w + 4g + e, column c16
    f32x4 S = zero4();
    if (a.S_in) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 16 * w + 4 * g + e;
            S[e] = (f < dk && c16 < ncol) ? a.S_in[((size_t)bh * dk + f) * dv + col0 + c16] : 0.f;
        }
    }

    // Per chunk each thread stages 16 (token, channel) elements of q, k and
    // the gates (thread: channel tid % 64, tokens 16 (tid / 64) ..+15) and 4
    // value elements.  The next chunk's raw elements are loaded while this one
    // is computed (out-of-range indices read element 0 and are replaced when
    // staged, so nothing waits for the loads before then).
    const int sc = tid & 63, sq = tid >> 6;
    T pq[16], pk[16], pv[4];
    float pa[16];
    auto fetch = [&](int t0) {
        const int nt = min(kC, N - t0);
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = 16 * sq + j;
            const bool in = t < nt && sc < dk;
            const size_t gi = (size_t)(t0 + (in ? t : 0)) * dk + (in ? sc : 0);
            pq[j] = Q[gi];
            pk[j] = K[gi];
            pa[j] = Al[gi];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + j * kThreads, t = e / kNC, cc = e % kNC;
            const bool in = t < nt && cc < ncol;
            pv[j] = V[(size_t)(t0 + (in ? t : 0)) * dv + col0 + (in ? cc : 0)];
        }
    };
    auto as_f32 = [](T x) {
        if constexpr (sizeof(T) == 2) return bf16_to_f32(x);
        else return static_cast<float>(x);
    };

    fetch(0);
    for (int t0 = 0; t0 < N; t0 += kC) {
        // ---- stage q, k, v (zero past the end and in padded channels); log2
        // gates (1 there) summed within each 16-token quarter
        float kf[16], lf[16];  // this thread's k and (quarter-local) l, kept for the key operand
        {
            const int nt = min(kC, N - t0);
            float acc = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int t = 16 * sq + j;
                const bool in = t < nt && sc < dk;
                sm.Q[t][sc] = in ? as_f32(pq[j]) : 0.f;
                kf[j] = in ? as_f32(pk[j]) : 0.f;
                sm.K[t][sc] = kf[j];
                // a gate of 0 counts as 2^-115 (its factor vanishes in fp32)
                const float al = in ? pa[j] : 1.f;
                acc += al > 0.f ? lg2(al) : -115.f;
                lf[j] = acc;
                sm.L[t][sc] = acc;
            }
            sm.tot[sq][sc] = acc;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = tid + j * kThreads, t = e / kNC, cc = e % kNC;
                sm.VT[cc][t] = (t < nt && cc < ncol) ? as_f32(pv[j]) : 0.f;
            }
        }
        // this wave's part of the state into the LDS image (rows 4g..4g+3 of column c16)
        *reinterpret_cast<float4 *>(&sm.ST[c16][16 * w + 4 * g]) = make_float4(S[0], S[1], S[2], S[3]);
        lds_barrier();
        if (t0 + kC < N) fetch(t0 + kC);  // in flight during this chunk
        // ---- the state update's key operand (a row of 16 tokens per thread):
        // k_t 2^{l_last - l_t}, the exponent being the rest of the token's own
        // block plus the later blocks' totals; the diagonal-block decay check
        {
            float later = 0.f;  // totals of the blocks after this thread's
#pragma unroll
            for (int q = 0; q < 4; ++q) later += q > sq ? sm.tot[q][sc] : 0.f;
            const float own = lf[15];
#pragma unroll
            for (int j = 0; j < 16; j += 4)
                *reinterpret_cast<float4 *>(&sm.KET[sc][16 * sq + j]) =
                    make_float4(kf[j] * ex2((own - lf[j]) + later), kf[j + 1] * ex2((own - lf[j + 1]) + later),
                                kf[j + 2] * ex2((own - lf[j + 2]) + later), kf[j + 3] * ex2((own - lf[j + 3]) + later));
            // decay across block sq: l(first token) - l(last token)
            const float dmax = lf[0] - lf[15];
            const bool over = __builtin_amdgcn_ballot_w64(dmax > kPivotBound) != 0;
            if (lane == 0) sm.big[sq] = over ? 1 : 0;
        }
        lds_barrier();

        // ---- outputs of query block I = w (row i = 16I + c16 as the A operand);
        // pivot: l at block I's first token (local sums: l_i - piv stays in the block)
        const int I = w;
        float qp[16], piv[16];
        {
            float qr[16], lr[16];
            row16(&sm.Q[16 * I + c16][16 * g], qr);
            row16(&sm.L[16 * I + c16][16 * g], lr);
            row16(&sm.L[16 * I][16 * g], piv);
#pragma unroll
            for (int j = 0; j < 16; ++j) qp[j] = qr[j] * ex2(lr[j] - piv[j]);  // at most |q|
        }
        // Independent accumulators keep several matrix-core chains in flight:
        // every wave forms the score tiles of all four key blocks (the ones
        // past its diagonal are dropped; the wave with the most work sets the
        // pace anyway), and the 16-step sums run as two interleaved halves.
        f32x4 o0 = zero4(), o1 = zero4();
        // scores of the four key blocks, last to first: for T < I the key part
        // is 2^{span + piv - l_t}, span = the totals of blocks T..I-1 (summed
        // here, never as a difference), all terms <= 0; for T = I it is
        // 2^{piv - l_t} within the block; past the diagonal the tile is dropped
        // and its exponent is clamped to stay finite
        float span[16];
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) span[ks] = 0.f;
        {
            f32x4 p[4];
            float kb[4][16];
#pragma unroll
            for (int Tb = 3; Tb >= 0; --Tb) {
                if (Tb < I) {
                    float tr[16];
                    row16(&sm.tot[Tb][16 * g], tr);
#pragma unroll
                    for (int ks = 0; ks < 16; ++ks) span[ks] += tr[ks];
                }
                float kr[16], lt[16];
                row16(&sm.K[16 * Tb + c16][16 * g], kr);
                row16(&sm.L[16 * Tb + c16][16 * g], lt);
#pragma unroll
                for (int ks = 0; ks < 16; ++ks)
                    kb[Tb][ks] = kr[ks] * ex2(fminf(span[ks] + (piv[ks] - lt[ks]), kPivotBound));
                p[Tb] = zero4();
            }
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
#pragma unroll
                for (int Tb = 0; Tb < 4; ++Tb) p[Tb] = mma(qp[ks], kb[Tb][ks], p[Tb]);
            const bool big = sm.big[I] != 0;
            f32x4 pd = zero4();
            if (big) {  // diagonal block element by element: sum_c q_ic k_tc 2^{l_ic - l_tc}, t <= i
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 16 * I + 4 * g + e, t = 16 * I + c16;
                    float sacc = 0.f;
                    if (t <= i)
                        for (int c = 0; c < kK; ++c) sacc += sm.Q[i][c] * sm.K[t][c] * ex2(sm.L[i][c] - sm.L[t][c]);
                    pd[e] = sacc;
                }
            }
#pragma unroll
            for (int Tb = 0; Tb < 4; ++Tb) {
                const f32x4 pv4 = (big && Tb == I) ? pd : p[Tb];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sm.W[w][4 * g + e][16 * Tb + c16] = (Tb < I || (Tb == I && 4 * g + e >= c16)) ? pv4[e] : 0.f;
            }
        }
        {
            // inter: sum_c q_ic 2^{l_i - l_start} S_0[c][col]; from the chunk's
            // start, 2^{...} = 2^{l_i - piv} 2^{piv + (totals of blocks 0..I-1)}
            // (span now holds those totals)
            float sr[16];
            row16(&sm.ST[c16][16 * g], sr);
#pragma unroll
            for (int ks = 0; ks < 16; ks += 2) {
                o0 = mma(qp[ks] * ex2(piv[ks] + span[ks]), sr[ks], o0);
                o1 = mma(qp[ks + 1] * ex2(piv[ks + 1] + span[ks + 1]), sr[ks + 1], o1);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        // intra: sum_{t <= i} score(i, t) v_t, and the state update's products
        float vr[16];
        row16(&sm.VT[c16][16 * g], vr);
        {
            float wr[16];
            row16(&sm.W[w][c16][16 * g], wr);
#pragma unroll
            for (int ks = 0; ks < 16; ks += 2) {
                o0 = mma(wr[ks], vr[ks], o0);
                o1 = mma(wr[ks + 1], vr[ks + 1], o1);
            }
        }
        const f32x4 o = o0 + o1;
        const int nt = min(kC, N - t0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = 16 * I + 4 * g + e;
            if (i < nt && c16 < ncol) store_from_f32(O, (size_t)(t0 + i) * dv + col0 + c16, o[e]);
        }

        // ---- state: S = diag(2^{l_last}) S + sum_t KE_t v_t^T (feature rows 16w..)
        {
            float kr[16];
            row16(&sm.KET[16 * w + c16][16 * g], kr);
            f32x4 u0 = zero4(), u1 = zero4();
#pragma unroll
            for (int ks = 0; ks < 16; ks += 2) {
                u0 = mma(kr[ks], vr[ks], u0);
                u1 = mma(kr[ks + 1], vr[ks + 1], u1);
            }
            const f32x4 u = u0 + u1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int f = 16 * w + 4 * g + e;  // decay of the whole chunk: the four block totals
                S[e] = ex2((sm.tot[0][f] + sm.tot[1][f]) + (sm.tot[2][f] + sm.tot[3][f])) * S[e] + u[e];
            }
        }
        lds_barrier();  // every wave is done with this chunk's tiles
    }
    if (a.S_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 16 * w + 4 * g + e;
            if (f < dk && c16 < ncol) a.S_out[((size_t)bh * dk + f) * dv + col0 + c16] = S[e];
        }
    }
}

// ---------------------------------------------------------------------------
// The same chunk form in three launches (la_forward_gla_chunked).  Given the
// state S_c entering chunk c, the chunk's outputs and the next state are
//   O = QD S_c + P V,   S_{c+1} = diag(decay) S_c + KE^T V,
// with the decayed queries QD[i][ch] = q_i,ch 2^{l_i,ch - l_start,ch}, the
// masked pair scores P (pivot split, element-wise diagonal block for extreme
// decays), the decayed keys KE[t][ch] = k_t,ch 2^{l_last,ch - l_t,ch} and the
// chunk decay 2^{l_last - l_start}.  P V and KE^T V do not involve the state,
// so the only serial step from chunk to chunk is element-wise:
//  1. k_gla_prep, one workgroup per (slice, chunk), every chunk at once:
//     gate sums, QD, P, KE, decay, and the products P V and KE^T V, into a
//     workspace record;
//  2. k_gla_chain, one thread per four state entries: S_c for every chunk
//     from S_in by S_{c+1} = decay (.) S_c + (KE^T V)_c (written over the
//     chunk's KE^T V in its record), S_out at the end;
//  3. k_gla_out, one workgroup per (slice, chunk): O = QD S_c + P V.
// ---------------------------------------------------------------------------

// Per-chunk record (floats), dvp = d_v rounded up to 16:
//   QD [64 tokens][64 channels]
//   PVT [dvp][64 tokens]      (P V)^T
//   KST [dvp][64 channels]    (KE^T V)^T; after k_gla_chain S_c^T
//   DEC [64]                  the chunk's decay per channel
__host__ __device__ inline int gla_dvp(int dv) { return (dv + kNC - 1) / kNC * kNC; }
__host__ __device__ inline size_t gla_rec_floats(int dvp) { return (size_t)kC * kK + 2 * (size_t)dvp * kC + kK; }

template <typename T>
__global__ __launch_bounds__(kThreads, 2) void k_gla_prep(GatedArgs a, int n_chunks, float *__restrict__ ws) {
    __shared__ __align__(16) GlaPrepSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int dk = a.dk, dv = a.dv, dvp = gla_dvp(dv), N = a.N;
    const int bh = blockIdx.x / n_chunks, ch = blockIdx.x % n_chunks;
    const int t0 = ch * kC, nt = min(kC, N - t0);
    const T *Q = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *K = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *V = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    const float *Al = a.alpha + (size_t)bh * N * dk;
    float *rec = ws + ((size_t)bh * n_chunks + ch) * gla_rec_floats(dvp);
    float *QD = rec, *PVT = rec + kC * kK, *KST = PVT + (size_t)dvp * kC, *DEC = KST + (size_t)dvp * kK;
    auto as_f32 = [](T x) {
        if constexpr (sizeof(T) == 2) return bf16_to_f32(x);
        else return static_cast<float>(x);
    };

    // stage q, k (zero past the end and in padded channels) and the log2
    // gates (1 there) summed within each 16-token quarter: thread = channel
    // tid % 64, tokens 16 (tid / 64) .. +15
    const int sc = tid & 63, sq = w;  // sq wave-uniform: the token tests below stay scalar
    float kf[16], lf[16];
    {
        // all loads first, unconditional (clamped indices), then the selects
        T rq[16], rk[16];
        float ra[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = 16 * sq + j;
            const bool in = t < nt && sc < dk;
            const size_t gi = (size_t)(t0 + (in ? t : 0)) * dk + (in ? sc : 0);
            rq[j] = Q[gi];
            rk[j] = K[gi];
            ra[j] = Al[gi];
        }
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = 16 * sq + j;
            const bool in = t < nt && sc < dk;
            sm.Q[t][sc] = in ? as_f32(rq[j]) : 0.f;
            kf[j] = in ? as_f32(rk[j]) : 0.f;
            sm.K[t][sc] = kf[j];
            // a gate of 0 counts as 2^-115 (its factor vanishes in fp32)
            const float al = in ? ra[j] : 1.f;
            acc += al > 0.f ? lg2(al) : -115.f;
            lf[j] = acc;
            sm.L[t][sc] = acc;
        }
        sm.tot[sq][sc] = acc;
    }
    lds_barrier();
    // decayed keys k_t 2^{l_last - l_t} ([channel][token]) and the diagonal-block check
    {
        float later = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) later += q > sq ? sm.tot[q][sc] : 0.f;
        const float own = lf[15];
#pragma unroll
        for (int j = 0; j < 16; j += 4)
            *reinterpret_cast<float4 *>(&sm.KE[sc][16 * sq + j]) =
                make_float4(kf[j] * ex2((own - lf[j]) + later), kf[j + 1] * ex2((own - lf[j + 1]) + later),
                            kf[j + 2] * ex2((own - lf[j + 2]) + later), kf[j + 3] * ex2((own - lf[j + 3]) + later));
        const float dmax = lf[0] - lf[15];
        const bool over = __builtin_amdgcn_ballot_w64(dmax > kPivotBound) != 0;
        if (lane == 0) sm.big[sq] = over ? 1 : 0;
        if (sq == 0) DEC[sc] = ex2((sm.tot[0][sc] + sm.tot[1][sc]) + (sm.tot[2][sc] + sm.tot[3][sc]));
    }
    lds_barrier();

    // scores of query block I = w, transposed: accumulator lane (4g+e, c16)
    // of key block Tb holds P[16I + c16][16Tb + 4g + e], which is the B
    // operand of the value product below as it stands (k-slot g of step
    // (Tb, e) = token 16Tb + 4g + e)
    const int I = w;
    float qp[16], piv[16];
    {
        float qr[16], lr[16];
        row16(&sm.Q[16 * I + c16][16 * g], qr);
        row16(&sm.L[16 * I + c16][16 * g], lr);
        row16(&sm.L[16 * I][16 * g], piv);
#pragma unroll
        for (int j = 0; j < 16; ++j) qp[j] = qr[j] * ex2(lr[j] - piv[j]);
    }
    float span[16];
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) span[ks] = 0.f;
    f32x4 pt[4];
    {
        float kb[4][16];
#pragma unroll
        for (int Tb = 3; Tb >= 0; --Tb) {
            if (Tb < I) {
                float tr[16];
                row16(&sm.tot[Tb][16 * g], tr);
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) span[ks] += tr[ks];
            }
            float kr[16], lt[16];
            row16(&sm.K[16 * Tb + c16][16 * g], kr);
            row16(&sm.L[16 * Tb + c16][16 * g], lt);
#pragma unroll
            for (int ks = 0; ks < 16; ++ks)
                kb[Tb][ks] = kr[ks] * ex2(fminf(span[ks] + (piv[ks] - lt[ks]), kPivotBound));
            pt[Tb] = zero4();
        }
        // QD[i][c] = q_ic 2^{l_i - l_start} = qp 2^{piv + totals of blocks 0..I-1}
#pragma unroll
        for (int ks = 0; ks < 16; ks += 4)
            *reinterpret_cast<float4 *>(&QD[(16 * I + c16) * kK + 16 * g + ks]) =
                make_float4(qp[ks] * ex2(piv[ks] + span[ks]), qp[ks + 1] * ex2(piv[ks + 1] + span[ks + 1]),
                            qp[ks + 2] * ex2(piv[ks + 2] + span[ks + 2]), qp[ks + 3] * ex2(piv[ks + 3] + span[ks + 3]));
#pragma unroll
        for (int ks = 0; ks < 16; ++ks)
#pragma unroll
            for (int Tb = 0; Tb < 4; ++Tb) pt[Tb] = mma(kb[Tb][ks], qp[ks], pt[Tb]);
        const bool big = sm.big[I] != 0;
        f32x4 pd = zero4();
        if (big) {  // diagonal block element by element: sum_c q_ic k_tc 2^{l_ic - l_tc}, t <= i
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * I + 4 * g + e, i = 16 * I + c16;
                float sacc = 0.f;
                if (t <= i)
                    for (int c = 0; c < kK; ++c) sacc += sm.Q[i][c] * sm.K[t][c] * ex2(sm.L[i][c] - sm.L[t][c]);
                pd[e] = sacc;
            }
        }
        // causal mask: key 16Tb + 4g + e <= query 16I + c16
#pragma unroll
        for (int Tb = 0; Tb < 4; ++Tb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float v = (big && Tb == I) ? pd[e] : pt[Tb][e];
                pt[Tb][e] = (Tb < I || (Tb == I && 4 * g + e <= c16)) ? v : 0.f;
            }
    }
    // value products, 64 columns at a time: V^T [column][token] goes to the
    // rows of sm.Q; wave w forms (P V)^T for its query block and (KE^T V)^T for
    // channels 16w..16w+15 on bf16 matrix instructions, with A = V^T (lane:
    // column c16) and k-slot 8g + j of half h = token 16(2h + j/4) + 4g + j%4,
    // so the score accumulators are the B operand of (P V)^T as they stand and
    // KE is read as four-token runs.  bf16 storage: P and KE enter as bf16
    // hi + lo parts and V is exact in bf16.  fp32 storage keeps fp32 operands
    // (v_mfma_f32_16x16x4_f32, k-slot g of step (Tb, e) = token 16Tb + 4g + e),
    // as its results are held to fp32 accuracy.
    constexpr bool BF = sizeof(T) == 2;
    B8 ph[2], pl[2];
    if constexpr (BF) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float pp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pp[j] = pt[2 * h + j / 4][j % 4];
            split8(pp, ph[h], pl[h]);
        }
    }
    B8 kh[2], kl[2];
    bool ke_split = !BF;
    for (int cg = 0; cg < dvp; cg += 64) {
        T rv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int t = 16 * sq + j;
            const bool in = t < nt && cg + sc < dv;
            rv[j] = V[(size_t)(t0 + (in ? t : 0)) * dv + (in ? cg + sc : 0)];
        }
        float vr[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) vr[j] = (16 * sq + j < nt && cg + sc < dv) ? as_f32(rv[j]) : 0.f;
        lds_barrier();  // every read of the staged rows (scores, QD; the previous column group) done
#pragma unroll
        for (int j = 0; j < 16; j += 4)
            *reinterpret_cast<float4 *>(&sm.Q[sc][16 * sq + j]) = make_float4(vr[j], vr[j + 1], vr[j + 2], vr[j + 3]);
        lds_barrier();
        if (!ke_split) {  // KE of channels 16w + c16 (first group only; KE does not change)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float kk[8];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const float4 k4 = *reinterpret_cast<const float4 *>(&sm.KE[16 * w + c16][16 * (2 * h + s2) + 4 * g]);
                    kk[4 * s2] = k4.x; kk[4 * s2 + 1] = k4.y; kk[4 * s2 + 2] = k4.z; kk[4 * s2 + 3] = k4.w;
                }
                split8(kk, kh[h], kl[h]);
            }
            ke_split = true;
        }
#pragma unroll 1
        for (int cb = 0; cb < 4; ++cb) {
            const int col = cg + 16 * cb;
            if (col < dvp) {  // wave-uniform
                f32x4 pv = zero4(), kv = zero4();
                if constexpr (BF) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        float vv[8];
#pragma unroll
                        for (int s2 = 0; s2 < 2; ++s2) {
                            const float4 v4 =
                                *reinterpret_cast<const float4 *>(&sm.Q[16 * cb + c16][16 * (2 * h + s2) + 4 * g]);
                            vv[4 * s2] = v4.x; vv[4 * s2 + 1] = v4.y; vv[4 * s2 + 2] = v4.z; vv[4 * s2 + 3] = v4.w;
                        }
                        B8 vh, vl;
                        split8(vv, vh, vl);  // vl = 0: V is exact in bf16
                        pv = mma8(vh, ph[h], pv);
                        kv = mma8(vh, kh[h], kv);
                        pv = mma8(vh, pl[h], pv);
                        kv = mma8(vh, kl[h], kv);
                    }
                } else {
#pragma unroll
                    for (int Tb = 0; Tb < 4; ++Tb) {
                        const float4 va = *reinterpret_cast<const float4 *>(&sm.Q[16 * cb + c16][16 * Tb + 4 * g]);
                        const float4 kk = *reinterpret_cast<const float4 *>(&sm.KE[16 * w + c16][16 * Tb + 4 * g]);
                        pv = mma(va.x, pt[Tb][0], pv);
                        kv = mma(va.x, kk.x, kv);
                        pv = mma(va.y, pt[Tb][1], pv);
                        kv = mma(va.y, kk.y, kv);
                        pv = mma(va.z, pt[Tb][2], pv);
                        kv = mma(va.z, kk.z, kv);
                        pv = mma(va.w, pt[Tb][3], pv);
                        kv = mma(va.w, kk.w, kv);
                    }
                }
                // lane (4g+e, c16): (P V)[16I + c16][col + 4g + e], (KE^T V)[16w + c16][col + 4g + e]
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    PVT[(size_t)(col + 4 * g + e) * kC + 16 * I + c16] = pv[e];
                    KST[(size_t)(col + 4 * g + e) * kK + 16 * w + c16] = kv[e];
                }
            }
        }
    }
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

// The state entering every chunk: S_0 = S_in, S_{c+1} = decay_c (.) S_c +
// (KE^T V)_c, element by element.  Thread: one value column and four
// channels of one slice; the records of the next kRing chunks are in flight
// (their loads do not depend on the state).  S_c overwrites (KE^T V)_c in
// the record once read (same thread, same address: program order).
constexpr int kRing = 8;
__global__ __launch_bounds__(256) void k_gla_chain(GatedArgs a, int n_chunks, float *__restrict__ ws) {
    const int dk = a.dk, dv = a.dv, dvp = gla_dvp(dv);
    const int per_slice = dvp * (kK / 4);
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid >= a.BH * per_slice) return;  // no barriers in this kernel
    const int bh = gid / per_slice, rem = gid % per_slice, col = rem / (kK / 4), f0 = 4 * (rem % (kK / 4));
    const size_t recf = gla_rec_floats(dvp);
    float *const base = ws + (size_t)bh * n_chunks * recf;
    const size_t kst = (size_t)kC * kK + (size_t)dvp * kC + (size_t)col * kK + f0;
    const size_t dec = (size_t)kC * kK + 2 * (size_t)dvp * kC + f0;

    float4 S = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.S_in && col < dv) {
        const float *si = a.S_in + (size_t)bh * dk * dv + col;
        S.x = f0 < dk ? si[(size_t)f0 * dv] : 0.f;
        S.y = f0 + 1 < dk ? si[(size_t)(f0 + 1) * dv] : 0.f;
        S.z = f0 + 2 < dk ? si[(size_t)(f0 + 2) * dv] : 0.f;
        S.w = f0 + 3 < dk ? si[(size_t)(f0 + 3) * dv] : 0.f;
    }
    float4 kv[kRing], dc[kRing];
    auto fetch = [&](int r, int c) {  // past the end: a harmless re-read of the last chunk
        const float *rec = base + (size_t)min(c, n_chunks - 1) * recf;
        kv[r] = *reinterpret_cast<const float4 *>(rec + kst);
        dc[r] = *reinterpret_cast<const float4 *>(rec + dec);
    };
    auto step = [&](int r, int c) {
        float4 *dst = reinterpret_cast<float4 *>(base + (size_t)c * recf + kst);
        const float4 sc = S;
        S = make_float4(fmaf(dc[r].x, S.x, kv[r].x), fmaf(dc[r].y, S.y, kv[r].y), fmaf(dc[r].z, S.z, kv[r].z),
                        fmaf(dc[r].w, S.w, kv[r].w));
        *dst = sc;
    };
#pragma unroll
    for (int r = 0; r < kRing; ++r) fetch(r, r);
    int c = 0;
    for (; c + kRing <= n_chunks; c += kRing) {
#pragma unroll
        for (int r = 0; r < kRing; ++r) {
            step(r, c + r);
            fetch(r, c + r + kRing);
        }
    }
#pragma unroll
    for (int r = 0; r < kRing; ++r)
        if (c + r < n_chunks) step(r, c + r);
    if (a.S_out && col < dv) {
        float *so = a.S_out + (size_t)bh * dk * dv + col;
        if (f0 < dk) so[(size_t)f0 * dv] = S.x;
        if (f0 + 1 < dk) so[(size_t)(f0 + 1) * dv] = S.y;
        if (f0 + 2 < dk) so[(size_t)(f0 + 2) * dv] = S.z;
        if (f0 + 3 < dk) so[(size_t)(f0 + 3) * dv] = S.w;
    }
}

// O = QD S_c + P V, one workgroup per (slice, chunk); wave w owns token rows
// 16w..16w+15.  A = QD rows (k-slot g of step ks = channel 16g + ks), B = S_c
// (lane: column c16, channels 16g..16g+15, a contiguous run of the record's
// S_c^T), C = (P V) rows; every load of the chunk is issued before the products.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_gla_out(GatedArgs a, int n_chunks, const float *__restrict__ ws) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int dv = a.dv, dvp = gla_dvp(dv), N = a.N;
    const int bh = blockIdx.x / n_chunks, ch = blockIdx.x % n_chunks;
    const int t0 = ch * kC, nt = min(kC, N - t0);
    const float *rec = ws + ((size_t)bh * n_chunks + ch) * gla_rec_floats(dvp);
    const float *QD = rec, *PVT = rec + kC * kK, *SST = PVT + (size_t)dvp * kC;
    T *O = static_cast<T *>(a.O) + (size_t)bh * N * dv;
    const auto ro = out_rsrc(O + (size_t)t0 * dv, nt * dv * (int)sizeof(T));

    float qa[16];
    row16(QD + (16 * w + c16) * kK + 16 * g, qa);
    for (int cb0 = 0; cb0 < dvp; cb0 += 64) {
        float sb[4][16];
        float4 pv[4];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = min(cb0 + 16 * cb, dvp - 16);  // past d_v: a re-read, not stored
            row16(SST + (size_t)(col + c16) * kK + 16 * g, sb[cb]);
            pv[cb] = *reinterpret_cast<const float4 *>(PVT + (size_t)(col + c16) * kC + 16 * w + 4 * g);
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            const int col = cb0 + 16 * cb;
            f32x4 o0 = f32x4{pv[cb].x, pv[cb].y, pv[cb].z, pv[cb].w}, o1 = zero4();
#pragma unroll
            for (int ks = 0; ks < 16; ks += 2) {
                o0 = mma(qa[ks], sb[cb][ks], o0);
                o1 = mma(qa[ks + 1], sb[cb][ks + 1], o1);
            }
            const f32x4 o = o0 + o1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 16 * w + 4 * g + e, j = col + c16;
                const int off = (i < nt && j < dv && col < dvp) ? (i * dv + j) * (int)sizeof(T) : nt * dv * (int)sizeof(T);
                store_elem<T>(ro, off, o[e]);
            }
        }
    }
}

}  // namespace

bool gla_chunk_supported(const GatedArgs &a) { return a.dk <= kK && a.N >= kC; }

hipError_t launch_gla_chunk(const GatedArgs &a, int dtype, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)a.BH, (unsigned)((a.dv + kNC - 1) / kNC)), block(kThreads);
    if (dtype == kF32) return launch_kernel_ev(k_gla_chunk<float>, grid, block, 0, st, ev, a);
    return launch_kernel_ev(k_gla_chunk<uint16_t>, grid, block, 0, st, ev, a);
}

size_t gla_chunk_ws_bytes(int BH, int N, int dv) {
    const size_t n_chunks = (size_t)(N + kC - 1) / kC;
    return sizeof(float) * (size_t)BH * n_chunks * gla_rec_floats(gla_dvp(dv));
}

hipError_t launch_gla_split(const GatedArgs &a, int dtype, float *ws, hipStream_t st, KEvents ev_prep,
                            KEvents ev_chain, KEvents ev_out) {
    const int n_chunks = (a.N + kC - 1) / kC;
    const dim3 gp((unsigned)((size_t)a.BH * n_chunks)), blk(kThreads);
    const size_t chain_threads = (size_t)a.BH * gla_dvp(a.dv) * (kK / 4);
    const dim3 gc((unsigned)((chain_threads + 255) / 256)), bc(256);
    hipError_t e;
    if (dtype == kF32) {
        e = launch_kernel_ev(k_gla_prep<float>, gp, blk, 0, st, ev_prep, a, n_chunks, ws);
        if (e == hipSuccess) e = launch_kernel_ev(k_gla_chain, gc, bc, 0, st, ev_chain, a, n_chunks, ws);
        if (e == hipSuccess)
            e = launch_kernel_ev(k_gla_out<float>, gp, blk, 0, st, ev_out, a, n_chunks, static_cast<const float *>(ws));
        return e;
    }
    e = launch_kernel_ev(k_gla_prep<uint16_t>, gp, blk, 0, st, ev_prep, a, n_chunks, ws);
    if (e == hipSuccess) e = launch_kernel_ev(k_gla_chain, gc, bc, 0, st, ev_chain, a, n_chunks, ws);
    if (e == hipSuccess)
        e = launch_kernel_ev(k_gla_out<uint16_t>, gp, blk, 0, st, ev_out, a, n_chunks, static_cast<const float *>(ws));
    return e;
}

}  // namespace la
