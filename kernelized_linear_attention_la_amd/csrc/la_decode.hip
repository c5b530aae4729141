// One recurrent decode step for every (batch, head) slice:
//   S += phi(k) v^T,  z += phi(k),  o = phi(q)^T S / phi(q)^T z
// ("Linear Attention": constant work and memory per generated token;
// "Story of Attention Part 5", 1a recurrence, update before read).
//
// The step is a single streaming pass over the fp32 state (d' x d_v per
// slice): each element is read once, updated with the rank-1 term and written
// back, and the column sums phi(q)^T S' are formed on the fly from the updated
// value.  One 256-thread workgroup per slice; thread (row group g, column
// quad c) owns rows g, g + G, g + 2G, ... of columns 4c..4c+3, so a wavefront
// touches whole contiguous rows (coalesced 16-byte accesses).  Partial column
// sums meet in LDS; phi(q)^T z' is a block reduction.
//
// Retention variant (RET; "Story of Attention Part 5", section 4 recurrent
// form): S = gamma S + phi(k) v^T, o = phi(q)^T S, with no z and no division.
// Every feature map of the library is available; the cosFormer token sits at
// position pos0.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxDp = 256;
constexpr int kMaxD = 128;
constexpr int kBatch = 8;  // rows in flight per thread between load and store
typedef float f32x4v __attribute__((ext_vector_type(4)));

template <typename T, int VW, bool RET>
__global__ __launch_bounds__(kThreads) void k_decode(Shape sh, const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, T *__restrict__ o,
                                                     float *__restrict__ S, float *__restrict__ z) {
    __shared__ float s_pq[kMaxDp], s_pk[kMaxDp], s_v[kMaxD];
    __shared__ float s_x[2][kMaxD];
    __shared__ float s_red[kThreads * 4];  // partial column sums [row group][dv] (G * dv <= 4 * 256)
    __shared__ float s_den[kThreads / 64];
    __shared__ float s_sq[2];
    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int dk = sh.dk, dv = sh.dv, dp = sh.dp;

    const T *qs = q + (size_t)bh * dk;
    const T *ks = k + (size_t)bh * dk;
    const T *vs = v + (size_t)bh * dv;
    float *Ss = S + (size_t)bh * dp * dv;
    float *zs = RET ? nullptr : z + (size_t)bh * dp;
    const float gam = RET ? sh.gamma[bh % sh.H] : 1.f;

    // feature maps of q and k, value row
    if (tid < dv) s_v[tid] = load_as_f32(vs, tid);
    if (sh.phi == kIdentity) {
        if (tid < dk) {
            s_pq[tid] = load_as_f32(qs, tid);
            s_pk[tid] = load_as_f32(ks, tid);
        }
    } else if (sh.phi == kElu1) {
        // the normalised query takes its power-of-two scale (cancels in the
        // division); retention's unnormalised read keeps 1
        const float xq = tid < dk ? load_as_f32(qs, tid) : -__builtin_huge_valf();
        float m = xq;
        for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
        if ((tid & 63) == 0) s_den[tid >> 6] = m;
        __syncthreads();
        float e = 0.f;
        if constexpr (!RET) e = elu1_query_shift(fmaxf(fmaxf(s_den[0], s_den[1]), fmaxf(s_den[2], s_den[3])));
        __syncthreads();  // s_den is reused for the denominator below
        if (tid < dk) {
            s_pq[tid] = RET ? elu1_accurate(xq) : elu1_accurate_scaled(xq, e);
            s_pk[tid] = elu1_accurate(load_as_f32(ks, tid));
        }
    } else if (sh.phi == kCosformer) {
        // ReLU(x) cos(pi p / 2M), ReLU(x) sin(pi p / 2M) at the token's position p = pos0
        const double ang = 3.14159265358979323846 * (double)sh.pos0 / (2.0 * (double)sh.param);
        const float cw = (float)cos(ang), sw = (float)sin(ang);
        if (tid < dk) {
            const float xq = fmaxf(load_as_f32(qs, tid), 0.f), xk = fmaxf(load_as_f32(ks, tid), 0.f);
            s_pq[tid] = xq * cw;
            s_pq[dk + tid] = xq * sw;
            s_pk[tid] = xk * cw;
            s_pk[dk + tid] = xk * sw;
        }
    } else if (sh.phi == kDpfp) {
        // r = ReLU([x, -x]); block i = 1..nu holds r_j r_{(j+i) mod 2d}
        if (tid < dk) {
            s_x[0][tid] = load_as_f32(qs, tid);
            s_x[1][tid] = load_as_f32(ks, tid);
        }
        __syncthreads();
        const int n2 = 2 * dk;
        auto rpm = [&](int w, int j) {
            const float x = j < dk ? s_x[w][j] : -s_x[w][j - dk];
            return x > 0.f ? x : 0.f;
        };
        for (int f = tid; f < dp; f += kThreads) {
            const int i = f / n2 + 1, j = f - (i - 1) * n2;
            const int jj = j + i < n2 ? j + i : j + i - n2;
            s_pq[f] = rpm(0, j) * rpm(0, jj);
            s_pk[f] = rpm(1, j) * rpm(1, jj);
        }
    } else {
        if (tid < dk) {
            s_x[0][tid] = load_as_f32(qs, tid);
            s_x[1][tid] = load_as_f32(ks, tid);
        }
        __syncthreads();
        if (tid < 2) {
            float a = 0.f;
            for (int c = 0; c < dk; ++c) a += s_x[tid][c] * s_x[tid][c];
            s_sq[tid] = a;
        }
        __syncthreads();
        // FAVOR+: exp(w_f . x - |x|^2 / 2) / sqrt(m); cos/sin projections: [cos(W x); sin(W x)]
        const float inv_sqrt_m = 1.0f / sqrtf(static_cast<float>(sh.m));
        for (int f = tid; f < sh.m; f += kThreads) {
            const float *w = sh.W + (size_t)f * dk;
            float aq = 0.f, ak = 0.f;
            for (int c = 0; c < dk; ++c) {
                float wc = w[c];
                aq += wc * s_x[0][c];
                ak += wc * s_x[1][c];
            }
            if (sh.phi == kTrig) {
                s_pq[f] = cosf(aq);
                s_pq[sh.m + f] = sinf(aq);
                s_pk[f] = cosf(ak);
                s_pk[sh.m + f] = sinf(ak);
            } else {
                s_pq[f] = expf(aq - 0.5f * s_sq[0]) * inv_sqrt_m;
                s_pk[f] = expf(ak - 0.5f * s_sq[1]) * inv_sqrt_m;
            }
        }
    }
    __syncthreads();

    // streaming rank-1 update of S and column sums of phi(q)^T S'
    const int cols = dv / VW;               // column groups
    const int G = kThreads / cols;          // row groups
    const int g = tid / cols, cg = tid - g * cols;
    float acc[VW];
#pragma unroll
    for (int u = 0; u < VW; ++u) acc[u] = 0.f;
    if (g < G) {
        float vv[VW];
#pragma unroll
        for (int u = 0; u < VW; ++u) vv[u] = s_v[cg * VW + u];
        for (int f0 = g; f0 < dp; f0 += G * kBatch) {
            float buf[kBatch][VW];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int f = f0 + b * G;
                if (f < dp) {
                    const float *src = Ss + (size_t)f * dv + cg * VW;
                    if constexpr (VW == 4) {
                        // streamed once per step: non-temporal, so the state does not displace cached lines
                        const f32x4v t4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4v *>(src));
                        buf[b][0] = t4[0]; buf[b][1] = t4[1]; buf[b][2] = t4[2]; buf[b][3] = t4[3];
                    } else {
#pragma unroll
                        for (int u = 0; u < VW; ++u) buf[b][u] = src[u];
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int f = f0 + b * G;
                if (f < dp) {
                    const float pk = s_pk[f], pq = s_pq[f];
#pragma unroll
                    for (int u = 0; u < VW; ++u) {
                        if constexpr (RET) buf[b][u] = gam * buf[b][u] + pk * vv[u];
                        else buf[b][u] += pk * vv[u];
                        acc[u] += pq * buf[b][u];
                    }
                    float *dst = Ss + (size_t)f * dv + cg * VW;
                    if constexpr (VW == 4) {
                        __builtin_nontemporal_store(f32x4v{buf[b][0], buf[b][1], buf[b][2], buf[b][3]},
                                                    reinterpret_cast<f32x4v *>(dst));
                    } else {
#pragma unroll
                        for (int u = 0; u < VW; ++u) dst[u] = buf[b][u];
                    }
                }
            }
        }
    }

    // z' = z + phi(k) and its read phi(q)^T z'
    float dpart = 0.f;
    if constexpr (!RET)
        for (int f = tid; f < dp; f += kThreads) {
            float zn = zs[f] + s_pk[f];
            zs[f] = zn;
            dpart += s_pq[f] * zn;
        }
    for (int off = 32; off > 0; off >>= 1) dpart += __shfl_down(dpart, off, 64);
    if ((tid & 63) == 0) s_den[tid >> 6] = dpart;

    // column sums across row groups
    if (g < G) {
#pragma unroll
        for (int u = 0; u < VW; ++u) s_red[g * dv + cg * VW + u] = acc[u];
    }
    __syncthreads();
    if (tid < dv) {
        float num = 0.f;
        for (int gg = 0; gg < G; ++gg) num += s_red[gg * dv + tid];
        if constexpr (RET) {
            store_from_f32(o + (size_t)bh * dv, tid, num);
        } else {
            float den = 0.f;
            for (int w = 0; w < kThreads / 64; ++w) den += s_den[w];
            store_from_f32(o + (size_t)bh * dv, tid, num / den);
        }
    }
}

template <bool RET>
hipError_t launch_decode_t(const Shape &sh, const void *q, const void *k, const void *v, void *o, float *S, float *z,
                           hipStream_t stream) {
    const bool vec = (sh.dv % 4) == 0;
    dim3 grid((unsigned)sh.BH), block(kThreads);
    if (sh.dtype == kF32) {
        auto *qq = static_cast<const float *>(q); auto *kk = static_cast<const float *>(k);
        auto *vv = static_cast<const float *>(v); auto *oo = static_cast<float *>(o);
        return vec ? launch_kernel(k_decode<float, 4, RET>, grid, block, 0, stream, sh, qq, kk, vv, oo, S, z)
                   : launch_kernel(k_decode<float, 1, RET>, grid, block, 0, stream, sh, qq, kk, vv, oo, S, z);
    }
    auto *qq = static_cast<const uint16_t *>(q); auto *kk = static_cast<const uint16_t *>(k);
    auto *vv = static_cast<const uint16_t *>(v); auto *oo = static_cast<uint16_t *>(o);
    return vec ? launch_kernel(k_decode<uint16_t, 4, RET>, grid, block, 0, stream, sh, qq, kk, vv, oo, S, z)
               : launch_kernel(k_decode<uint16_t, 1, RET>, grid, block, 0, stream, sh, qq, kk, vv, oo, S, z);
}

}  // namespace

hipError_t launch_decode(const Shape &sh, const void *q, const void *k, const void *v, void *o, float *S, float *z,
                         hipStream_t stream) {
    return sh.ret ? launch_decode_t<true>(sh, q, k, v, o, S, z, stream)
                    : launch_decode_t<false>(sh, q, k, v, o, S, z, stream);
}

}  // namespace la
