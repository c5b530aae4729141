// Gated and delta-rule states, token by token ("Linear Attention" (aiwiki.ai),
// GLA's gated recurrence and the delta-rule update; "Story of Attention Part
// 5", section 7 Gated DeltaNet).  Raw q, k; state S [d_k][d_v] fp32,
// feature-major; the output is read after the update, o_t = S_t^T q_t.
//   GLA (diagonal gate over the key channels):
//     S_t = diag(alpha_t) S_{t-1} + k_t v_t^T
//   gated delta rule (alpha_t = 1 when no gate is given):
//     p_t = alpha_t S_{t-1}^T k_t,   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - p_t)^T
// The recurrence is serial in t and each step is an O(d_k d_v) update, so one
// workgroup owns one (b, h) slice and keeps its state in registers for the
// whole sequence: wave w owns value columns 8w..8w+7, lane 8r + c holds
// column 8w + c of rows r, r + 8, r + 16, ...  The reductions over rows
// (S^T k, S^T q) are a per-lane partial sum and three cross-lane steps.
// Tokens are staged through LDS kTC at a time; outputs leave through LDS as
// whole rows.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kRG = 8;     // row groups (lanes) per column
constexpr int kRmax = 16;  // rows per lane: d_k <= 128
constexpr int kTC = 16;    // tokens per staging round
constexpr int kMaxD = 128;

template <typename T, bool GLA>
__global__ __launch_bounds__(1024) void k_gated(GatedArgs a) {
    __shared__ float sQ[kTC][kMaxD], sK[kTC][kMaxD], sV[kTC][kMaxD], sO[kTC][kMaxD];
    __shared__ float sA[GLA ? kTC : 1][GLA ? kMaxD : 1];
    __shared__ float sAl[kTC], sBe[kTC];
    const int dk = a.dk, dv = a.dv, N = a.N;
    const int bh = blockIdx.x;
    const int tid = threadIdx.x, nth = blockDim.x;
    const int lane = tid & 63, w = tid >> 6;
    const int c = lane & 7, r = lane >> 3;
    const int col = 8 * w + c;
    const bool live = col < dv;

    const T *Q = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *K = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *V = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *O = static_cast<T *>(a.O) + (size_t)bh * N * dv;

    float S[kRmax];
#pragma unroll
    for (int i = 0; i < kRmax; ++i) {
        const int f = r + kRG * i;
        S[i] = (a.S_in && live && f < dk) ? a.S_in[((size_t)bh * dk + f) * dv + col] : 0.f;
    }

    for (int t0 = 0; t0 < N; t0 += kTC) {
        const int nt = min(kTC, N - t0);
        __syncthreads();  // the previous round's tiles have been read and written out
        for (int e = tid; e < nt * dk; e += nth) {
            const int t = e / dk, f = e - t * dk;
            sQ[t][f] = load_as_f32(Q, (size_t)t0 * dk + e);
            sK[t][f] = load_as_f32(K, (size_t)t0 * dk + e);
            if constexpr (GLA) sA[t][f] = a.alpha[((size_t)bh * N + t0) * dk + e];
        }
        for (int e = tid; e < nt * dv; e += nth) {
            const int t = e / dv;
            sV[t][e - t * dv] = load_as_f32(V, (size_t)t0 * dv + e);
        }
        if constexpr (!GLA) {
            if (tid < nt) {
                sAl[tid] = a.alpha ? a.alpha[(size_t)bh * N + t0 + tid] : 1.f;
                sBe[tid] = a.beta[(size_t)bh * N + t0 + tid];
            }
        }
        __syncthreads();
        for (int t = 0; t < nt; ++t) {
            const float vc = live ? sV[t][col] : 0.f;
            if constexpr (GLA) {
#pragma unroll
                for (int i = 0; i < kRmax; ++i) {
                    const int f = r + kRG * i;
                    if (f < dk) S[i] = sA[t][f] * S[i] + sK[t][f] * vc;
                }
            } else {
                float p0 = 0.f, p1 = 0.f;  // S^T k over this lane's rows (two chains)
#pragma unroll
                for (int i = 0; i < kRmax; i += 2) {
                    const int f0 = r + kRG * i, f1 = f0 + kRG;
                    if (f0 < dk) p0 += sK[t][f0] * S[i];
                    if (f1 < dk) p1 += sK[t][f1] * S[i + 1];
                }
                float p = p0 + p1;
                p += __shfl_xor(p, 8, 64);
                p += __shfl_xor(p, 16, 64);
                p += __shfl_xor(p, 32, 64);
                const float al = sAl[t], be = sBe[t];
                const float delta = vc - al * p;
#pragma unroll
                for (int i = 0; i < kRmax; ++i) {
                    const int f = r + kRG * i;
                    if (f < dk) S[i] = al * S[i] + be * sK[t][f] * delta;
                }
            }
            float o0 = 0.f, o1 = 0.f;  // S^T q over this lane's rows
#pragma unroll
            for (int i = 0; i < kRmax; i += 2) {
                const int f0 = r + kRG * i, f1 = f0 + kRG;
                if (f0 < dk) o0 += sQ[t][f0] * S[i];
                if (f1 < dk) o1 += sQ[t][f1] * S[i + 1];
            }
            float o = o0 + o1;
            o += __shfl_xor(o, 8, 64);
            o += __shfl_xor(o, 16, 64);
            o += __shfl_xor(o, 32, 64);
            if (r == 0 && live) sO[t][col] = o;
        }
        __syncthreads();
        for (int e = tid; e < nt * dv; e += nth) {
            const int t = e / dv;
            store_from_f32(O, (size_t)t0 * dv + e, sO[t][e - t * dv]);
        }
    }
    if (a.S_out) {
#pragma unroll
        for (int i = 0; i < kRmax; ++i) {
            const int f = r + kRG * i;
            if (live && f < dk) a.S_out[((size_t)bh * dk + f) * dv + col] = S[i];
        }
    }
}

}  // namespace

hipError_t launch_gated(const GatedArgs &a, bool gla, int dtype, hipStream_t st, KEvents ev) {
    const dim3 grid((unsigned)a.BH), block((unsigned)(64 * ((a.dv + 7) / 8)));
    if (dtype == kF32)
        return gla ? launch_kernel_ev(k_gated<float, true>, grid, block, 0, st, ev, a)
                   : launch_kernel_ev(k_gated<float, false>, grid, block, 0, st, ev, a);
    return gla ? launch_kernel_ev(k_gated<uint16_t, true>, grid, block, 0, st, ev, a)
               : launch_kernel_ev(k_gated<uint16_t, false>, grid, block, 0, st, ev, a);
}

}  // namespace la
