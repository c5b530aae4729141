// Gated and delta-rule states, token by token ("Linear Attention" (aiwiki.ai),
// GLA's gated recurrence and the delta-rule update; "Story of Attention Part
// 5", section 7 Gated DeltaNet).  Raw q, k; state S [d_k][d_v] fp32,
// feature-major; the output is read after the update, o_t = S_t^T q_t.
//   GLA (diagonal gate over the key channels):
//     S_t = diag(alpha_t) S_{t-1} + k_t v_t^T
//   gated delta rule (alpha_t = 1 when no gate is given):
//     p_t = alpha_t S_{t-1}^T k_t,   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - p_t)^T
// The recurrence is serial in t, but every value column of the state evolves
// on its own (S^T k, the update and S^T q act column by column), so a
// workgroup of 8 waves owns 64 value columns of one (b, h) slice and keeps
// them in registers for the whole sequence: wave w owns columns 8w..8w+7 of
// the group, the 8 lanes 8c..8c+7 hold column 8w + c, each a block of
// consecutive rows.  The reductions over rows (S^T k, S^T q) are a per-lane
// partial sum and three DPP steps.  Tokens are staged through LDS TC at a
// time (rows padded with zeros to 8 R features, so padded rows of S stay
// zero); the next round's inputs are loaded into registers while the current
// round runs.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kRG = 8;     // row groups per value column (lanes 8c .. 8c + 7)

// R rows per lane: lane 8c + r owns rows R r .. R r + R - 1 of column
// 64 blockIdx.y + 8w + c.
template <typename T, bool GLA, int R>
__global__ __launch_bounds__(512) void k_gated(GatedArgs a) {
    constexpr int NW = 8;
    constexpr int DP = kRG * R;   // padded key width
    constexpr int NTH = 64 * NW;
    constexpr int TC = 32;        // tokens per staging round
    constexpr int NC = 8 * NW;    // value columns of the workgroup
    constexpr int JK = (TC * DP + NTH - 1) / NTH;  // staged key-side values per thread
    constexpr int JV = (TC * NC + NTH - 1) / NTH;  // staged values per thread
    __shared__ __align__(16) float sQ[TC][DP], sK[TC][DP], sA[GLA ? TC : 1][GLA ? DP : 4];
    __shared__ float sV[TC][NC], sO[TC][NC];
    __shared__ float sAl[TC], sBe[TC];
    const int dk = a.dk, dv = a.dv, N = a.N;
    const int bh = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int r = lane & 7, c = lane >> 3;
    const int col0 = NC * blockIdx.y;  // first value column of the workgroup
    const int lc = 8 * w + c;          // this lane's column within the group
    const int col = col0 + lc;
    const bool live = col < dv;
    const int f0 = R * r;

    const T *Q = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *K = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *V = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *O = static_cast<T *>(a.O) + (size_t)bh * N * dv;
    const float *Ag = GLA ? a.alpha + (size_t)bh * N * dk : nullptr;

    float S[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
        const int f = f0 + i;
        S[i] = (a.S_in && live && f < dk) ? a.S_in[((size_t)bh * dk + f) * dv + col] : 0.f;
    }
    auto rows = [&](const float *src, float *dst) {  // this lane's R consecutive features
        if constexpr (R % 4 == 0) {
#pragma unroll
            for (int i = 0; i < R; i += 4) {
                const float4 x = *reinterpret_cast<const float4 *>(src + f0 + i);
                dst[i] = x.x; dst[i + 1] = x.y; dst[i + 2] = x.z; dst[i + 3] = x.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < R; ++i) dst[i] = src[f0 + i];
        }
    };

    // next round's inputs, held in registers while the current round runs
    float pq[JK], pk[JK], pa[GLA ? JK : 1], pv[JV], pal = 1.f, pbe = 0.f;
    auto fetch = [&](int t0) {
        const int nt = min(TC, N - t0);
#pragma unroll
        for (int j = 0; j < JK; ++j) {
            const int e = tid + j * NTH, t = e / DP, f = e % DP;
            const bool in = t < nt && f < dk;
            const size_t g = (size_t)(t0 + t) * dk + f;
            pq[j] = in ? load_as_f32(Q, g) : 0.f;
            pk[j] = in ? load_as_f32(K, g) : 0.f;
            if constexpr (GLA) pa[j] = in ? Ag[g] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < JV; ++j) {
            const int e = tid + j * NTH, t = e / NC, cc = col0 + e % NC;
            pv[j] = (t < nt && cc < dv) ? load_as_f32(V, (size_t)(t0 + t) * dv + cc) : 0.f;
        }
        if constexpr (!GLA) {
            if (tid < nt) {
                pal = a.alpha ? a.alpha[(size_t)bh * N + t0 + tid] : 1.f;
                pbe = a.beta[(size_t)bh * N + t0 + tid];
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int j = 0; j < JK; ++j) {
            const int e = tid + j * NTH;
            if (e < TC * DP) {
                sQ[e / DP][e % DP] = pq[j];
                sK[e / DP][e % DP] = pk[j];
                if constexpr (GLA) sA[e / DP][e % DP] = pa[j];
            }
        }
#pragma unroll
        for (int j = 0; j < JV; ++j) {
            const int e = tid + j * NTH;
            if (e < TC * NC) sV[e / NC][e % NC] = pv[j];
        }
        if constexpr (!GLA) {
            if (tid < TC) {
                sAl[tid] = pal;
                sBe[tid] = pbe;
            }
        }
    };

    fetch(0);
    for (int t0 = 0; t0 < N; t0 += TC) {
        const int nt = min(TC, N - t0);
        stage();
        __syncthreads();
        if (t0 + TC < N) fetch(t0 + TC);  // in flight during the token loop
#pragma unroll 4
        for (int t = 0; t < nt; ++t) {
            const float vc = sV[t][lc];
            float kr[R], qr[R];
            rows(sK[t], kr);
            rows(sQ[t], qr);
            if constexpr (GLA) {
                float ar[R];
                rows(sA[t], ar);
#pragma unroll
                for (int i = 0; i < R; ++i) S[i] = ar[i] * S[i] + kr[i] * vc;
            } else {
                float p0 = 0.f, p1 = 0.f;  // S^T k over this lane's rows (two chains)
#pragma unroll
                for (int i = 0; i < R; i += 2) {
                    p0 += kr[i] * S[i];
                    if (i + 1 < R) p1 += kr[i + 1] * S[i + 1];
                }
                const float p = group8_sum(p0 + p1);
                const float al = sAl[t], be = sBe[t];
                const float bd = be * (vc - al * p);
#pragma unroll
                for (int i = 0; i < R; ++i) S[i] = al * S[i] + kr[i] * bd;
            }
            float o0 = 0.f, o1 = 0.f;  // S^T q over this lane's rows
#pragma unroll
            for (int i = 0; i < R; i += 2) {
                o0 += qr[i] * S[i];
                if (i + 1 < R) o1 += qr[i + 1] * S[i + 1];
            }
            const float o = group8_sum(o0 + o1);
            if (r == 0) sO[t][lc] = o;
        }
        __syncthreads();  // every output of the round is in LDS, every staged input read
        const int ncol = min(NC, dv - col0);
        for (int e = tid; e < nt * ncol; e += NTH) {
            const int t = e / ncol, cc = e - t * ncol;
            store_from_f32(O, (size_t)(t0 + t) * dv + col0 + cc, sO[t][cc]);
        }
    }
    if (a.S_out) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
            const int f = f0 + i;
            if (live && f < dk) a.S_out[((size_t)bh * dk + f) * dv + col] = S[i];
        }
    }
}

template <typename T, bool GLA>
hipError_t launch_gated_t(const GatedArgs &a, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)a.BH, (unsigned)((a.dv + 63) / 64)), block(512);
    if (a.dk <= 16) return launch_kernel_ev(k_gated<T, GLA, 2>, grid, block, 0, st, ev, a);
    if (a.dk <= 32) return launch_kernel_ev(k_gated<T, GLA, 4>, grid, block, 0, st, ev, a);
    if (a.dk <= 64) return launch_kernel_ev(k_gated<T, GLA, 8>, grid, block, 0, st, ev, a);
    return launch_kernel_ev(k_gated<T, GLA, 16>, grid, block, 0, st, ev, a);
}

}  // namespace

hipError_t launch_gated(const GatedArgs &a, bool gla, int dtype, hipStream_t st, KEvents ev) {
    if (gla && gla_chunk_supported(a)) return launch_gla_chunk(a, dtype, st, ev);
    if (dtype == kF32)
        return gla ? launch_gated_t<float, true>(a, st, ev) : launch_gated_t<float, false>(a, st, ev);
    return gla ? launch_gated_t<uint16_t, true>(a, st, ev) : launch_gated_t<uint16_t, false>(a, st, ev);
}

}  // namespace la
