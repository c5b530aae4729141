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

// The per-chunk preparation (k_gla_prep) uses only the first fields: its own
// 53 KB layout lets two of its workgroups share a CU (the one-launch kernel's
// layout, 97 KB, allows one).
struct GlaPrepSmem {
    float Q[kC][kRS];
    float K[kC][kRS];
    float L[kC][kRS];
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
// The same chunk form in two launches (la_forward_gla_chunked).  Everything
// above that does not depend on the value columns -- the gate sums, the
// decayed keys KE[c][t] = k_tc 2^{l_last,c - l_tc}, the masked pair scores
// P[i][t] (pivot split, element-wise diagonal block for extreme decays), the
// decayed queries QD[i][c] = q_ic 2^{l_ic - l_start,c} and the chunk decay
// 2^{l_last,c - l_start,c} -- is formed once per chunk by k_gla_prep (one
// workgroup per (slice, chunk), every chunk at once) into a workspace record;
// k_gla_scan then walks the chunks of each (slice, 16 value columns) with only
// the three products that touch the values:
//   O = QD S_0 + P V,   S_C = diag(decay) S_0 + KE V.
// ---------------------------------------------------------------------------

// Per-chunk record (floats): P [64][64], QD [64][64], KE [64][64], decay [64].
__host__ __device__ inline size_t gla_rec_floats() { return 3 * kC * kK + kK; }

template <typename T>
__global__ __launch_bounds__(kThreads) void k_gla_prep(GatedArgs a, int n_chunks, float *__restrict__ ws) {
    __shared__ __align__(16) GlaPrepSmem sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int dk = a.dk, N = a.N;
    const int bh = blockIdx.x / n_chunks, ch = blockIdx.x % n_chunks;
    const int t0 = ch * kC, nt = min(kC, N - t0);
    const T *Q = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *K = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const float *Al = a.alpha + (size_t)bh * N * dk;
    float *rec = ws + ((size_t)bh * n_chunks + ch) * gla_rec_floats();
    float *P = rec, *QD = rec + kC * kK, *KE = rec + 2 * kC * kK, *DEC = rec + 3 * kC * kK;
    auto as_f32 = [](T x) {
        if constexpr (sizeof(T) == 2) return bf16_to_f32(x);
        else return static_cast<float>(x);
    };

    // stage q, k (zero past the end and in padded channels) and the log2
    // gates (1 there) summed within each 16-token quarter: thread = channel
    // tid % 64, tokens 16 (tid / 64) .. +15
    const int sc = tid & 63, sq = tid >> 6;
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
    // decayed keys k_t 2^{l_last - l_t} ([feature][token]) and the diagonal-block check
    {
        float later = 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) later += q > sq ? sm.tot[q][sc] : 0.f;
        const float own = lf[15];
#pragma unroll
        for (int j = 0; j < 16; j += 4)
            *reinterpret_cast<float4 *>(&KE[sc * kC + 16 * sq + j]) =
                make_float4(kf[j] * ex2((own - lf[j]) + later), kf[j + 1] * ex2((own - lf[j + 1]) + later),
                            kf[j + 2] * ex2((own - lf[j + 2]) + later), kf[j + 3] * ex2((own - lf[j + 3]) + later));
        const float dmax = lf[0] - lf[15];
        const bool over = __builtin_amdgcn_ballot_w64(dmax > kPivotBound) != 0;
        if (lane == 0) sm.big[sq] = over ? 1 : 0;
        if (sq == 0) DEC[sc] = ex2((sm.tot[0][sc] + sm.tot[1][sc]) + (sm.tot[2][sc] + sm.tot[3][sc]));
    }
    lds_barrier();

    // scores and decayed queries of query block I = w (as in k_gla_chunk)
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
                P[(16 * I + 4 * g + e) * kC + 16 * Tb + c16] =
                    (Tb < I || (Tb == I && 4 * g + e >= c16)) ? pv4[e] : 0.f;
        }
    }
    // QD[i][c] = q_ic 2^{l_i - l_start} = qp 2^{piv + totals of blocks 0..I-1}
#pragma unroll
    for (int ks = 0; ks < 16; ks += 4)
        *reinterpret_cast<float4 *>(&QD[(16 * I + c16) * kK + 16 * g + ks]) =
            make_float4(qp[ks] * ex2(piv[ks] + span[ks]), qp[ks + 1] * ex2(piv[ks + 1] + span[ks + 1]),
                        qp[ks + 2] * ex2(piv[ks + 2] + span[ks + 2]), qp[ks + 3] * ex2(piv[ks + 3] + span[ks + 3]));
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

// One workgroup per (slice, 16 value columns), the chunks in order; wave w
// owns token rows 16w..16w+15 of O and feature rows 16w..16w+15 of the state.
// Row operands (QD, P, KE rows) come straight from the record into registers
// one chunk ahead; k-step j of lane group q takes index 16q + j.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_gla_scan(GatedArgs a, int n_chunks, const float *__restrict__ ws) {
    __shared__ float sV[kC * 20], sS[kK * 20], sD[kK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;
    const int r = c16, q = g;
    const int dk = a.dk, dv = a.dv, N = a.N;
    const int bh = blockIdx.x, col0 = kNC * blockIdx.y;
    const int ncol = min(kNC, dv - col0);
    const T *V = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *O = static_cast<T *>(a.O) + (size_t)bh * N * dv;

    f32x4 S = zero4();
    if (a.S_in) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 16 * w + 4 * g + e;
            S[e] = (f < dk && c16 < ncol) ? a.S_in[((size_t)bh * dk + f) * dv + col0 + c16] : 0.f;
        }
    }
    // Every load is unconditional (indices clamped to valid elements; the
    // selects happen where the values are used): a load under a branch makes
    // the compiler wait for all outstanding loads right after it, which would
    // turn the prefetch into a synchronous read.
    struct Pre {
        float4 qd[4], p[4], ke[4];
        T v[4];
        float dec;
    };
    auto fetch = [&](Pre &f, int ch_) {
        const int ch = min(ch_, n_chunks - 1);  // past the end: a harmless re-read of the last chunk
        const int t0 = ch * kC, nt = min(kC, N - t0);
        const float *rec = ws + ((size_t)bh * n_chunks + ch) * gla_rec_floats();
        const float *Pr = rec + (16 * w + r) * kC + 16 * q;
        const float *Qr = rec + kC * kK + (16 * w + r) * kK + 16 * q;
        const float *Kr = rec + 2 * kC * kK + (16 * w + r) * kC + 16 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f.p[i] = *reinterpret_cast<const float4 *>(Pr + 4 * i);
            f.qd[i] = *reinterpret_cast<const float4 *>(Qr + 4 * i);
            f.ke[i] = *reinterpret_cast<const float4 *>(Kr + 4 * i);
        }
        f.dec = rec[3 * kC * kK + (tid & (kK - 1))];
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // values: token e / 16, column e % 16
            const int e = tid + j * kThreads, t = e / kNC, cc = e % kNC;
            const bool in = t < nt && cc < ncol;
            f.v[j] = V[(size_t)(t0 + (in ? t : 0)) * dv + col0 + (in ? cc : 0)];
        }
    };
    auto as_f32 = [](T x) {
        if constexpr (sizeof(T) == 2) return bf16_to_f32(x);
        else return static_cast<float>(x);
    };
    Pre pre;
    fetch(pre, 0);
    for (int ch = 0; ch < n_chunks; ++ch) {
        const int t0 = ch * kC, nt = min(kC, N - t0);
        float pa[16], qa[16], ka[16];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pa[4 * i] = pre.p[i].x; pa[4 * i + 1] = pre.p[i].y; pa[4 * i + 2] = pre.p[i].z; pa[4 * i + 3] = pre.p[i].w;
            qa[4 * i] = pre.qd[i].x; qa[4 * i + 1] = pre.qd[i].y; qa[4 * i + 2] = pre.qd[i].z; qa[4 * i + 3] = pre.qd[i].w;
            ka[4 * i] = pre.ke[i].x; ka[4 * i + 1] = pre.ke[i].y; ka[4 * i + 2] = pre.ke[i].z; ka[4 * i + 3] = pre.ke[i].w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = tid + j * kThreads, t = e / kNC, cc = e % kNC;
            sV[t * 20 + cc] = (t < nt && cc < ncol) ? as_f32(pre.v[j]) : 0.f;
        }
        if (tid < kK) sD[tid] = pre.dec;
#pragma unroll
        for (int e = 0; e < 4; ++e) sS[(16 * w + 4 * g + e) * 20 + c16] = S[e];
        lds_barrier();
        fetch(pre, ch + 1);
        // O = QD S_0 + P V for token rows 16w.. ; S = decay S_0 + KE V for feature rows 16w..
        // (the B operands read from LDS all at once, then the products)
        float sb[16], vb[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sb[j] = sS[(16 * q + j) * 20 + c16];
            vb[j] = sV[(16 * q + j) * 20 + c16];
        }
        f32x4 o0 = zero4(), o1 = zero4(), u0 = zero4(), u1 = zero4();
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & 1) {
                o1 = mma(qa[j], sb[j], o1);
                o1 = mma(pa[j], vb[j], o1);
                u1 = mma(ka[j], vb[j], u1);
            } else {
                o0 = mma(qa[j], sb[j], o0);
                o0 = mma(pa[j], vb[j], o0);
                u0 = mma(ka[j], vb[j], u0);
            }
        }
        const f32x4 o = o0 + o1, u = u0 + u1;
        const auto ro = out_rsrc(O + (size_t)t0 * dv, nt * dv * (int)sizeof(T));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 16 * w + 4 * g + e;
            S[e] = sD[f] * S[e] + u[e];
            const int i = 16 * w + 4 * g + e;
            const int off = (i < nt && c16 < ncol) ? (i * dv + col0 + c16) * (int)sizeof(T) : nt * dv * (int)sizeof(T);
            store_elem<T>(ro, off, o[e]);
        }
        lds_barrier();  // this chunk's values, decay and state image read before the next staging
    }
    if (a.S_out) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 16 * w + 4 * g + e;
            if (f < dk && c16 < ncol) a.S_out[((size_t)bh * dk + f) * dv + col0 + c16] = S[e];
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

size_t gla_chunk_ws_bytes(int BH, int N) {
    const size_t n_chunks = (size_t)(N + kC - 1) / kC;
    return sizeof(float) * (size_t)BH * n_chunks * gla_rec_floats();
}

hipError_t launch_gla_split(const GatedArgs &a, int dtype, float *ws, hipStream_t st, KEvents ev_prep,
                            KEvents ev_scan) {
    const int n_chunks = (a.N + kC - 1) / kC;
    const dim3 gp((unsigned)((size_t)a.BH * n_chunks)), gs((unsigned)a.BH, (unsigned)((a.dv + kNC - 1) / kNC));
    const dim3 blk(kThreads);
    hipError_t e;
    if (dtype == kF32) {
        e = launch_kernel_ev(k_gla_prep<float>, gp, blk, 0, st, ev_prep, a, n_chunks, ws);
        if (e != hipSuccess) return e;
        return launch_kernel_ev(k_gla_scan<float>, gs, blk, 0, st, ev_scan, a, n_chunks, static_cast<const float *>(ws));
    }
    e = launch_kernel_ev(k_gla_prep<uint16_t>, gp, blk, 0, st, ev_prep, a, n_chunks, ws);
    if (e != hipSuccess) return e;
    return launch_kernel_ev(k_gla_scan<uint16_t>, gs, blk, 0, st, ev_scan, a, n_chunks, static_cast<const float *>(ws));
}

}  // namespace la
