// Generic chunkwise kernels: fp32 arithmetic, any d_k, d_v <= 128, any m <= 256,
// fp32 or bf16 storage.  This is the path for fp32 problems (where bf16 matrix
// cores would not meet fp32 accuracy) and for shapes without an MFMA variant.
//
// One workgroup owns one (slice, segment, 32-column value slab).  It walks its
// chunks in order ("Linear Attention", chunkwise parallel form; "Story of
// Attention Part 5", section 6 blockwise split with decay 1 plus the
// normaliser of section 1a):
//   for each chunk c:
//     for each query tile (T rows):  O = [phiQ S + (phiQ phiK^T (masked j<=i)) V]
//                                      / [phiQ z + (phiQ phiK^T (masked)) 1]
//     then S += phiK_c^T V_c, z += phiK_c^T 1
// The state S (d' x 32 slab) and z live in LDS in fp32 for the whole segment.
//
// Retention (sh.ret: decayed, unnormalised; "Story of Attention Part
// 5", section 6 blockwise form with its decay lambda): no z, no division, and
// with chunk rows i, t counted from 0 and Lc the tokens of the chunk
//     O_i = sum_{t<=i} lambda^(i-t) P[i,t] v_t + lambda^(i+1) phiQ_i S,
//     S   = lambda^Lc S + sum_t lambda^(Lc-1-t) phiK_t v_t^T.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kVS = 32;  // value columns per workgroup

struct GenLayout {
    int T;    // rows per tile
    int dpp;  // padded row stride of the phi tiles (avoids LDS bank conflicts)
    int offS, offZ, offX, offSq, offPQ, offPK, offV, offP, offW, total;
};

__host__ __device__ inline GenLayout gen_layout(int dk, int dp) {
    GenLayout L;
    L.T = dp <= 128 ? 16 : 8;
    L.dpp = dp + 1;
    int o = 0;
    L.offS = o;  o += dp * kVS;
    L.offZ = o;  o += dp;
    L.offX = o;  o += L.T * dk;
    L.offSq = o; o += L.T;
    L.offPQ = o; o += L.T * L.dpp;
    L.offPK = o; o += L.T * L.dpp;
    L.offV = o;  o += L.T * kVS;
    L.offP = o;  o += L.T * L.T;
    L.offW = o;  o += L.T;
    L.total = o;
    return L;
}

// phi of `nvalid` rows starting at row0 of X [*, dk] into out [T][dpp]; rows
// past nvalid become zero (they must not contribute to any sum).
template <typename T>
__device__ void phi_tile(const Shape &sh, const GenLayout &L, const T *X, int row0, int nvalid,
                         float *sX, float *sSq, float *out, bool query = false) {
    const int tid = threadIdx.x;
    const int dk = sh.dk;
    if (sh.phi == kIdentity) {  // raw rows (retention's q and k)
        for (int e = tid; e < L.T * dk; e += kThreads) {
            int r = e / dk, c = e - r * dk;
            out[r * L.dpp + c] = r < nvalid ? load_as_f32(X, (size_t)(row0 + r) * dk + c) : 0.f;
        }
        return;
    }
    if (sh.phi == kElu1) {
        // normalised queries: each row takes its power-of-two scale (it
        // cancels in the division; the unnormalised retention form keeps 1)
        const bool scaled = query && !sh.ret;
        if (scaled) {
            if (tid < L.T) {
                float m = 0.f;  // rows past nvalid are zero anyway
                if (tid < nvalid) {
                    m = -__builtin_huge_valf();
                    for (int c = 0; c < dk; ++c) m = fmaxf(m, load_as_f32(X, (size_t)(row0 + tid) * dk + c));
                }
                sSq[tid] = elu1_query_shift(m);
            }
            __syncthreads();
        }
        for (int e = tid; e < L.T * dk; e += kThreads) {
            int r = e / dk, c = e - r * dk;
            float v = 0.f;
            if (r < nvalid) {
                const float x = load_as_f32(X, (size_t)(row0 + r) * dk + c);
                v = scaled ? elu1_accurate_scaled(x, sSq[r]) : elu1_accurate(x);
            }
            out[r * L.dpp + c] = v;
        }
        return;
    }
    if (sh.phi == kDpfp) {
        // DPFP ("Linear Attention", feature-map table): r = ReLU([x, -x]);
        // block i = 1..nu holds r_j r_{(j+i) mod 2d}
        const int n2 = 2 * dk, dp = n2 * sh.param;
        for (int e = tid; e < L.T * dk; e += kThreads) {
            int r = e / dk;
            sX[e] = r < nvalid ? load_as_f32(X, (size_t)(row0 + r) * dk + (e - r * dk)) : 0.f;
        }
        __syncthreads();
        auto relu_pm = [&](int r, int j) {  // ReLU([x, -x])_j of row r
            const float x = j < dk ? sX[r * dk + j] : -sX[r * dk + j - dk];
            return x > 0.f ? x : 0.f;
        };
        for (int e = tid; e < L.T * dp; e += kThreads) {
            const int r = e / dp, f = e - r * dp;
            const int i = f / n2 + 1, j = f - (i - 1) * n2;
            const int jj = j + i < n2 ? j + i : j + i - n2;
            out[r * L.dpp + f] = relu_pm(r, j) * relu_pm(r, jj);
        }
        return;
    }
    if (sh.phi == kCosformer) {
        // cosFormer ("Story of Attention Part 5", section 3): ReLU(x) cos(pi p / 2M),
        // then ReLU(x) sin(pi p / 2M), p = pos0 + token index (phase in double)
        for (int e = tid; e < L.T * dk; e += kThreads) {
            const int r = e / dk, c = e - r * dk;
            float cw = 0.f, sw = 0.f, x = 0.f;
            if (r < nvalid) {
                const double ang = 3.14159265358979323846 * (double)(sh.pos0 + row0 + r) / (2.0 * (double)sh.param);
                cw = (float)cos(ang);
                sw = (float)sin(ang);
                x = load_as_f32(X, (size_t)(row0 + r) * dk + c);
                x = x > 0.f ? x : 0.f;
            }
            out[r * L.dpp + c] = x * cw;
            out[r * L.dpp + dk + c] = x * sw;
        }
        return;
    }
    // FAVOR+ ("Story of Attention Part 5", 1b): exp(w_r . x - |x|^2/2) / sqrt(m);
    // cos/sin projections ("Linear Attention", feature-map table): [cos(W x); sin(W x)]
    for (int e = tid; e < L.T * dk; e += kThreads) {
        int r = e / dk, c = e - r * dk;
        sX[e] = r < nvalid ? load_as_f32(X, (size_t)(row0 + r) * dk + c) : 0.f;
    }
    __syncthreads();
    if (tid < L.T) {
        float s = 0.f;
        for (int c = 0; c < dk; ++c) s += sX[tid * dk + c] * sX[tid * dk + c];
        sSq[tid] = s;
    }
    __syncthreads();
    const float inv_sqrt_m = 1.0f / sqrtf(static_cast<float>(sh.m));
    for (int f = tid; f < sh.m; f += kThreads) {
        const float *w = sh.W + (size_t)f * dk;
        float acc[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
        for (int c = 0; c < dk; ++c) {
            float wc = w[c];
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r < L.T) acc[r] += wc * sX[r * dk + c];
        }
        if (sh.phi == kTrig) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r < L.T) {
                    out[r * L.dpp + f] = r < nvalid ? cosf(acc[r]) : 0.f;
                    out[r * L.dpp + sh.m + f] = r < nvalid ? sinf(acc[r]) : 0.f;
                }
        } else {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r < L.T) out[r * L.dpp + f] = r < nvalid ? expf(acc[r] - 0.5f * sSq[r]) * inv_sqrt_m : 0.f;
        }
    }
}

template <typename T>
__device__ void value_tile(const Shape &sh, const GenLayout &L, const T *V, int row0, int nvalid, int j0, int vw,
                           float *sV) {
    for (int e = threadIdx.x; e < L.T * kVS; e += kThreads) {
        int r = e / kVS, j = e - r * kVS;
        float v = 0.f;
        if (r < nvalid && j < vw) v = load_as_f32(V, (size_t)(row0 + r) * sh.dv + j0 + j);
        sV[e] = v;
    }
}

// lambda^x for x >= 0 from l2 = log2(lambda): exactly 1 at x = 0 (also for
// lambda = 0), accurate exp2f otherwise.
__device__ __forceinline__ float decay_pow(float l2, float x) { return x == 0.f ? 1.f : exp2f(x * l2); }

template <typename T, int MODE>
__global__ __launch_bounds__(kThreads) void k_generic(FwdArgs a) {
    extern __shared__ float smem[];
    const Shape sh = a.sh;
    const Segments sg = a.sg;
    const int dp = sh.dp, dk = sh.dk, dv = sh.dv;
    const GenLayout L = gen_layout(dk, dp);
    float *sS = smem + L.offS, *sz = smem + L.offZ, *sX = smem + L.offX, *sSq = smem + L.offSq;
    float *sPQ = smem + L.offPQ, *sPK = smem + L.offPK, *sV = smem + L.offV, *sP = smem + L.offP;
    float *sW = smem + L.offW;
    const int tid = threadIdx.x;

    const int nslab = (dv + kVS - 1) / kVS;
    const int slab = blockIdx.x % nslab;
    const int seg = (blockIdx.x / nslab) % sg.P;
    const int bh = blockIdx.x / (nslab * sg.P);
    const int j0 = slab * kVS;
    const int vw = min(kVS, dv - j0);

    const int c_begin = seg * sg.seg_chunks;
    const int c_end = min(sg.n_chunks, c_begin + sg.seg_chunks);
    const int N = sh.N, C = sg.chunk;
    const bool ret = sh.ret != 0;  // retention
    const float l2 = ret ? log2f(sh.gamma[bh % sh.H]) : 0.f;

    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *Os = a.O ? static_cast<T *>(a.O) + (size_t)bh * N * dv : nullptr;

    // starting state
    const float *Ssrc = a.st.S_src ? a.st.S_src + bh * a.st.src_slice + seg * a.st.src_seg : nullptr;
    const float *zsrc = a.st.z_src ? a.st.z_src + bh * a.st.zsrc_slice + seg * a.st.zsrc_seg : nullptr;
    for (int e = tid; e < dp * kVS; e += kThreads) {
        int f = e / kVS, j = e - f * kVS;
        sS[e] = (Ssrc && j < vw) ? Ssrc[(size_t)f * dv + j0 + j] : 0.f;
    }
    for (int f = tid; f < dp; f += kThreads) sz[f] = zsrc ? zsrc[f] : 0.f;
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        const int Lc = min(C, N - t0);
        if constexpr (MODE != kModeState) {
            for (int qt = 0; qt < Lc; qt += L.T) {
                const int nq = min(L.T, Lc - qt);
                phi_tile(sh, L, Qs, t0 + qt, nq, sX, sSq, sPQ, true);
                __syncthreads();
                // inter-chunk read of the carried state: phiQ S, phiQ z
                float acc[2], den[2];
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    int e = tid + r * kThreads;
                    acc[r] = 0.f; den[r] = 0.f;
                    if (e < L.T * kVS) {
                        int i = e / kVS, j = e - i * kVS;
                        const float *pq = sPQ + i * L.dpp;
                        if (ret) {
                            for (int f = 0; f < dp; ++f) acc[r] += pq[f] * sS[f * kVS + j];
                            acc[r] *= decay_pow(l2, (float)(qt + i + 1));
                        } else {
                            for (int f = 0; f < dp; ++f) {
                                acc[r] += pq[f] * sS[f * kVS + j];
                                den[r] += pq[f] * sz[f];
                            }
                        }
                    }
                }
                if constexpr (MODE == kModeCausal) {
                    // intra-chunk masked pairwise part, key tiles up to the query tile
                    for (int kt = 0; kt <= qt; kt += L.T) {
                        const int nk = min(L.T, Lc - kt);
                        __syncthreads();  // previous users of sX / sPK / sV / sP are done
                        phi_tile(sh, L, Ks, t0 + kt, nk, sX, sSq, sPK);
                        value_tile(sh, L, Vs, t0 + kt, nk, j0, vw, sV);
                        __syncthreads();
                        for (int e = tid; e < L.T * L.T; e += kThreads) {
                            int i = e / L.T, t = e - i * L.T;
                            float p = 0.f;
                            if (kt + t <= qt + i) {
                                const float *pq = sPQ + i * L.dpp, *pk = sPK + t * L.dpp;
                                for (int f = 0; f < dp; ++f) p += pq[f] * pk[f];
                                if (ret) p *= decay_pow(l2, (float)(qt + i - kt - t));
                            }
                            sP[e] = p;
                        }
                        __syncthreads();
#pragma unroll
                        for (int r = 0; r < 2; ++r) {
                            int e = tid + r * kThreads;
                            if (e < L.T * kVS) {
                                int i = e / kVS, j = e - i * kVS;
                                for (int t = 0; t < L.T; ++t) {
                                    float p = sP[i * L.T + t];
                                    acc[r] += p * sV[t * kVS + j];
                                    den[r] += p;
                                }
                            }
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    int e = tid + r * kThreads;
                    if (e < L.T * kVS) {
                        int i = e / kVS, j = e - i * kVS;
                        if (i < nq && j < vw)
                            store_from_f32(Os, (size_t)(t0 + qt + i) * dv + j0 + j, ret ? acc[r] : acc[r] / den[r]);
                    }
                }
                __syncthreads();  // sPQ is reused by the next query tile
            }
        }
        if constexpr (MODE != kModeRead) {
            // carry the state past this chunk: S += phiK^T V, z += phiK^T 1
            // (retention: S = lambda^Lc S + sum_t lambda^(Lc-1-t) phiK_t v_t^T)
            for (int kt = 0; kt < Lc; kt += L.T) {
                const int nk = min(L.T, Lc - kt);
                phi_tile(sh, L, Ks, t0 + kt, nk, sX, sSq, sPK);
                value_tile(sh, L, Vs, t0 + kt, nk, j0, vw, sV);
                if (ret && tid < L.T) sW[tid] = tid < nk ? decay_pow(l2, (float)(Lc - 1 - kt - tid)) : 0.f;
                __syncthreads();
                if (ret) {
                    const float carry = kt == 0 ? decay_pow(l2, (float)Lc) : 1.f;
                    for (int e = tid; e < dp * kVS; e += kThreads) {
                        int f = e / kVS, j = e - f * kVS;
                        float s = carry * sS[e];
                        for (int t = 0; t < L.T; ++t) s += sW[t] * sPK[t * L.dpp + f] * sV[t * kVS + j];
                        sS[e] = s;
                    }
                } else {
                    for (int e = tid; e < dp * kVS; e += kThreads) {
                        int f = e / kVS, j = e - f * kVS;
                        float s = sS[e];
                        for (int t = 0; t < L.T; ++t) s += sPK[t * L.dpp + f] * sV[t * kVS + j];
                        sS[e] = s;
                    }
                    for (int f = tid; f < dp; f += kThreads) {
                        float s = sz[f];
                        for (int t = 0; t < L.T; ++t) s += sPK[t * L.dpp + f];
                        sz[f] = s;
                    }
                }
                __syncthreads();
            }
        }
    }

    if (a.st.S_dst) {
        float *Sd = a.st.S_dst + bh * a.st.dst_slice + seg * a.st.dst_seg;
        for (int e = tid; e < dp * kVS; e += kThreads) {
            int f = e / kVS, j = e - f * kVS;
            if (j < vw) Sd[(size_t)f * dv + j0 + j] = sS[e];
        }
        if (slab == 0 && a.st.z_dst) {
            float *zd = a.st.z_dst + bh * a.st.zdst_slice + seg * a.st.zdst_seg;
            for (int f = tid; f < dp; f += kThreads) zd[f] = sz[f];
        }
    }
}

// Exclusive prefix over the P segment states of each slice, in place:
//   slot s <- S_in + sum_{s' < s} slot s'   and   S_out <- S_in + sum_s slot s.
// With total_to_slot0, slot 0 <- sum_s slot s instead (non-causal total).
// Retention (gamma set): the state decays across each segment, so the
// running value is acc <- lambda^(len s) acc + slot s (Horner form), with
// len s the tokens of segment s (seg_tokens, the last one shorter).
// One thread per state element; the segment order is fixed, so repeated runs
// give identical bits.
__global__ __launch_bounds__(kThreads) void k_scan(int BH, int P, int nS, int nz, float *ws_S, float *ws_z,
                                                   const float *S_in, const float *z_in, float *S_out,
                                                   float *z_out, int total_to_slot0, const float *gamma, int H,
                                                   int seg_tokens, int N) {
    const int per = nS + nz;
    const int blocks_per_slice = (per + kThreads - 1) / kThreads;
    const int bh = blockIdx.x / blocks_per_slice;
    const int e = (blockIdx.x - bh * blocks_per_slice) * kThreads + threadIdx.x;
    if (bh >= BH || e >= per) return;
    const bool isS = e < nS;
    const int idx = isS ? e : e - nS;
    const int n = isS ? nS : nz;
    float *slots = (isS ? ws_S : ws_z) + (size_t)bh * P * n + idx;
    const float *in = isS ? S_in : z_in;
    float *out = isS ? S_out : z_out;
    float acc = in ? in[(size_t)bh * n + idx] : 0.f;
    // up to kB loads in flight at once, then the ordered running sum
    constexpr int kB = 32;
    if (total_to_slot0) acc = 0.f;
    for (int s0 = 0; s0 < P; s0 += kB) {
        float d[kB];
#pragma unroll
        for (int b = 0; b < kB; ++b) d[b] = s0 + b < P ? slots[(size_t)(s0 + b) * n] : 0.f;
        if (total_to_slot0) {
#pragma unroll
            for (int b = 0; b < kB; ++b) acc += d[b];
        } else if (gamma) {
            const float l2 = log2f(gamma[bh % H]);
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                if (s0 + b < P) {
                    slots[(size_t)(s0 + b) * n] = acc;
                    const int len = min(seg_tokens, N - (s0 + b) * seg_tokens);
                    acc = decay_pow(l2, (float)len) * acc + d[b];
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < kB; ++b) {
                if (s0 + b < P) slots[(size_t)(s0 + b) * n] = acc;
                acc += d[b];
            }
        }
    }
    if (total_to_slot0) slots[0] = acc;
    if (out) out[(size_t)bh * n + idx] = acc;
}

// Copies the hand-off error word of a workspace control block (ctl[2], set by
// a single-pass launch whose bounded wait expired) to *out, and clears it
// when asked.  One thread; agent-scope accesses like the writers'.
__global__ void k_ws_error(uint32_t *ctl, uint32_t *out, int clear) {
    out[0] = __hip_atomic_load(ctl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (clear) __hip_atomic_store(ctl + 2, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

size_t generic_lds_bytes(int dk, int dp) { return sizeof(float) * (size_t)gen_layout(dk, dp).total; }

hipError_t launch_generic(const FwdArgs &a, hipStream_t stream, KEvents ev) {
    if (f32mma_supported(a.sh)) return launch_f32mma(a, stream, ev);
    const int nslab = (a.sh.dv + kVS - 1) / kVS;
    const size_t grid = (size_t)a.sh.BH * a.sg.P * nslab;
    const size_t lds = generic_lds_bytes(a.sh.dk, a.sh.dp);
    const dim3 gr((unsigned)grid), bl(kThreads);
    const bool f32 = a.sh.dtype == kF32;
    switch (a.mode) {
        case kModeState:
            return f32 ? launch_kernel_ev(k_generic<float, kModeState>, gr, bl, lds, stream, ev, a)
                       : launch_kernel_ev(k_generic<uint16_t, kModeState>, gr, bl, lds, stream, ev, a);
        case kModeCausal:
            return f32 ? launch_kernel_ev(k_generic<float, kModeCausal>, gr, bl, lds, stream, ev, a)
                       : launch_kernel_ev(k_generic<uint16_t, kModeCausal>, gr, bl, lds, stream, ev, a);
        default:
            return f32 ? launch_kernel_ev(k_generic<float, kModeRead>, gr, bl, lds, stream, ev, a)
                       : launch_kernel_ev(k_generic<uint16_t, kModeRead>, gr, bl, lds, stream, ev, a);
    }
}

hipError_t launch_scan(const Shape &sh, int P, float *ws_S, float *ws_z, const float *S_in, const float *z_in,
                       float *S_out, float *z_out, bool total_to_slot0, hipStream_t stream, KEvents ev,
                       int seg_tokens) {
    const int nS = sh.dp * sh.dv, nz = sh.ret ? 0 : sh.dp;  // retention carries no z
    const int bps = (nS + nz + kThreads - 1) / kThreads;
    return launch_kernel_ev(k_scan, dim3((unsigned)((size_t)sh.BH * bps)), dim3(kThreads), 0, stream, ev, sh.BH, P,
                            nS, nz, ws_S, ws_z, S_in, z_in, S_out, z_out, total_to_slot0 ? 1 : 0,
                            sh.ret ? sh.gamma : nullptr, sh.H,
                            seg_tokens, sh.N);
}

// Zero fill of n 16-byte words (grid-stride).
__global__ void k_zero_fill(uint4 *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream) {
    const size_t n = bytes / 16;
    const unsigned blocks = (unsigned)((n + kThreads - 1) / kThreads < 1024 ? (n + kThreads - 1) / kThreads : 1024);
    return launch_kernel(k_zero_fill, dim3(blocks > 0 ? blocks : 1), dim3(kThreads), 0, stream,
                         static_cast<uint4 *>(p), n);
}

hipError_t launch_ws_error(uint32_t *ctl, uint32_t *out, bool clear, hipStream_t stream) {
    return launch_kernel(k_ws_error, dim3(1), dim3(1), 0, stream, ctl, out, clear ? 1 : 0);
}

}  // namespace la
