// Backward of the causal normalised form, chunkwise ("Linear Attention:
// Removing the Softmax Buys Associativity", the parallel mode used for
// training; the pages give no gradients, these follow from the recurrence by
// reverse-mode differentiation).  With psi_i = phi(q_i), kappa_j = phi(k_j),
// V_aug = [V | 1], S_aug = [S | z]:
//   G_aug_i = [dO_i / den_i | -(dO_i . o_i) / den_i]
//   dpsi_i   = S_aug_i G_aug_i                       (state up to and with token i)
//   dkappa_j = R_aug_j v_aug_j,  dv_j = R_j^T kappa_j (R_aug_j = dS_out_aug + sum_{i>=j} psi_i G_aug_i^T)
// Chunked: inside a chunk the sums over tokens are explicit masked pairwise
// products, across chunks they go through the carried states, and across
// segments through per-segment sums and fixed-order scans (forward for S_aug,
// reverse for R_aug).
//
// Kernels (one 256-thread workgroup per (slice, segment), fp32 arithmetic,
// fp32 or bf16 storage):
//   k_bwd_dq   chunks in order from the forward prefix: recomputes num, den,
//              writes G_aug to the workspace and dQ;
//   k_bwd_usum sums psi^T G_aug over each segment;
//   k_bwd_rscan exclusive suffix of those sums (+ dS_out), in place; dS_in;
//   k_bwd_dkv  chunks in reverse from the suffix: dK, dV.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int kTh = 256;
constexpr int kT = 16;  // rows per tile

struct BwdLayout {
    int ldp, dva;  // padded phi row stride, augmented value width (d_v + 1)
    int offS, offXq, offSqq, offPQ, offXk, offSqk, offPK, offV, offG, offDO, offP, offB, offDP, offDV, offH, offRD,
        total;
};

__host__ __device__ inline BwdLayout bwd_layout(int dk, int dp, int dv) {
    BwdLayout L;
    L.ldp = dp + 1;
    L.dva = dv + 1;
    int o = 0;
    L.offS = o;   o += dp * L.dva;   // S_aug (dq pass) or R_aug (dkv pass)
    L.offXq = o;  o += kT * dk;      // raw query rows
    L.offSqq = o; o += kT;
    L.offPQ = o;  o += kT * L.ldp;   // phi(q) tile
    L.offXk = o;  o += kT * dk;      // raw key rows
    L.offSqk = o; o += kT;
    L.offPK = o;  o += kT * L.ldp;   // phi(k) tile
    L.offV = o;   o += kT * L.dva;   // [v | 1] tile
    L.offG = o;   o += kT * L.dva;   // num_aug, then G_aug (dq pass); G_aug tile (dkv pass)
    L.offDO = o;  o += kT * dv;      // dO tile (dq pass)
    L.offP = o;   o += kT * kT;      // masked pairwise scores (psi . kappa)
    L.offB = o;   o += kT * kT;      // masked pairwise scores (G_aug . v_aug)
    L.offDP = o;  o += kT * L.ldp;   // dphi accumulators
    L.offDV = o;  o += kT * dv;      // dV accumulators (dkv pass)
    L.offH = o;   o += kT;           // h_i = -(dO_i . o_i) / den_i
    L.offRD = o;  o += kT;           // 1 / den_i
    L.total = o;
    return L;
}

struct BwdArgs {
    Shape sh;
    Segments sg;
    const void *Q, *K, *V, *dO;
    void *dQ, *dK, *dV;
    const float *Spre, *zpre;  // forward prefix per segment: [BH][P][dp*dv], [BH][P][dp]
    float *U;                  // [BH][P][dp*(dv+1)] segment sums psi^T G_aug, then suffixes R_aug
    float *G;                  // [BH][N][dv+1] G_aug per token
};

// raw rows [row0, row0 + nvalid) of X into sX [kT][dk] and phi into out [kT][ldp];
// rows past nvalid are zero in both (they add nothing to any sum)
template <typename T>
__device__ void load_phi(const Shape &sh, const BwdLayout &L, const T *X, int row0, int nvalid, float *sX,
                         float *sSq, float *out) {
    const int tid = threadIdx.x, dk = sh.dk;
    for (int e = tid; e < kT * dk; e += kTh) {
        const int r = e / dk, c = e - r * dk;
        sX[e] = r < nvalid ? load_as_f32(X, (size_t)(row0 + r) * dk + c) : 0.f;
    }
    __syncthreads();
    if (sh.phi == kElu1) {
        for (int e = tid; e < kT * dk; e += kTh) {
            const int r = e / dk, c = e - r * dk;
            out[r * L.ldp + c] = r < nvalid ? elu1_accurate(sX[e]) : 0.f;
        }
        return;
    }
    // FAVOR+ ("Story of Attention Part 5", 1b): exp(w_f . x - |x|^2 / 2) / sqrt(m)
    if (tid < kT) {
        float s = 0.f;
        for (int c = 0; c < dk; ++c) s += sX[tid * dk + c] * sX[tid * dk + c];
        sSq[tid] = s;
    }
    __syncthreads();
    const float inv_sqrt_m = 1.0f / sqrtf(static_cast<float>(sh.m));
    for (int e = tid; e < kT * sh.m; e += kTh) {
        const int r = e / sh.m, f = e - r * sh.m;
        const float *w = sh.W + (size_t)f * dk;
        float a = 0.f;
        for (int c = 0; c < dk; ++c) a += w[c] * sX[r * dk + c];
        out[r * L.ldp + f] = r < nvalid ? expf(a - 0.5f * sSq[r]) * inv_sqrt_m : 0.f;
    }
}

// [v | 1] rows into sV [kT][dva]; zero past nvalid
template <typename T>
__device__ void load_vaug(const Shape &sh, const BwdLayout &L, const T *V, int row0, int nvalid, float *sV) {
    for (int e = threadIdx.x; e < kT * L.dva; e += kTh) {
        const int r = e / L.dva, c = e - r * L.dva;
        float v = 0.f;
        if (r < nvalid) v = c < sh.dv ? load_as_f32(V, (size_t)(row0 + r) * sh.dv + c) : 1.f;
        sV[e] = v;
    }
}

// dx = J_phi(x)^T dphi for the nvalid rows of a tile, stored to D rows row0..
//   ELU+1: dphi * (x > 0 ? 1 : exp(x)), and exp(x) = phi(x) there;
//   FAVOR+: d phi_f / dx = phi_f (w_f - x), so dx = W^T (dphi . phi) - x (dphi . phi summed)
template <typename T>
__device__ void store_input_grad(const Shape &sh, const BwdLayout &L, const float *sX, const float *sPhi,
                                 const float *sDphi, float *sScratch, int nvalid, T *D, int row0) {
    const int tid = threadIdx.x, dk = sh.dk;
    if (sh.phi == kElu1) {
        for (int e = tid; e < kT * dk; e += kTh) {
            const int r = e / dk, c = e - r * dk;
            if (r < nvalid) {
                const float x = sX[e];
                const float j = x > 0.f ? 1.f : sPhi[r * L.ldp + c];
                store_from_f32(D, (size_t)(row0 + r) * dk + c, sDphi[r * L.ldp + c] * j);
            }
        }
        return;
    }
    if (tid < kT) {
        float s = 0.f;
        for (int f = 0; f < sh.m; ++f) s += sDphi[tid * L.ldp + f] * sPhi[tid * L.ldp + f];
        sScratch[tid] = s;
    }
    __syncthreads();
    for (int e = tid; e < kT * dk; e += kTh) {
        const int r = e / dk, c = e - r * dk;
        if (r < nvalid) {
            float a = 0.f;
            for (int f = 0; f < sh.m; ++f) a += sDphi[r * L.ldp + f] * sPhi[r * L.ldp + f] * sh.W[(size_t)f * dk + c];
            store_from_f32(D, (size_t)(row0 + r) * dk + c, a - sX[e] * sScratch[r]);
        }
    }
}

// Largest state the kernels hold: d' * (d_v + 1) <= kMaxAug elements, kMaxU per thread.
constexpr int kMaxU = 65;
constexpr int kMaxAug = kMaxU * kTh;

template <typename T>
__global__ __launch_bounds__(kTh) void k_bwd_dq(BwdArgs a) {
    extern __shared__ float smem[];
    const Shape sh = a.sh;
    const Segments sg = a.sg;
    const int dp = sh.dp, dk = sh.dk, dv = sh.dv;
    const BwdLayout L = bwd_layout(dk, dp, dv);
    const int dva = L.dva;
    float *sS = smem + L.offS, *sXq = smem + L.offXq, *sSqq = smem + L.offSqq, *sPQ = smem + L.offPQ;
    float *sXk = smem + L.offXk, *sSqk = smem + L.offSqk, *sPK = smem + L.offPK, *sV = smem + L.offV;
    float *sG = smem + L.offG, *sDO = smem + L.offDO, *sP = smem + L.offP, *sDP = smem + L.offDP;
    float *sH = smem + L.offH, *sRD = smem + L.offRD;
    const int tid = threadIdx.x;
    const int seg = blockIdx.x % sg.P, bh = blockIdx.x / sg.P;
    const int N = sh.N, C = sg.chunk;
    const int c_begin = seg * sg.seg_chunks, c_end = min(sg.n_chunks, c_begin + sg.seg_chunks);
    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    const T *dOs = static_cast<const T *>(a.dO) + (size_t)bh * N * dv;
    T *dQs = static_cast<T *>(a.dQ) + (size_t)bh * N * dk;
    float *Gs = a.G + (size_t)bh * N * dva;

    // S_aug = [S | z] entering the segment
    const float *Sp = a.Spre + ((size_t)bh * sg.P + seg) * dp * dv;
    const float *zp = a.zpre + ((size_t)bh * sg.P + seg) * dp;
    for (int e = tid; e < dp * dva; e += kTh) {
        const int f = e / dva, c = e - f * dva;
        sS[e] = c < dv ? Sp[(size_t)f * dv + c] : zp[f];
    }
    __syncthreads();

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C, Lc = min(C, N - t0);
        for (int qt = 0; qt < Lc; qt += kT) {
            const int nq = min(kT, Lc - qt);
            load_phi(sh, L, Qs, t0 + qt, nq, sXq, sSqq, sPQ);
            for (int e = tid; e < kT * dv; e += kTh) {
                const int r = e / dv, col = e - r * dv;
                sDO[e] = r < nq ? load_as_f32(dOs, (size_t)(t0 + qt + r) * dv + col) : 0.f;
            }
            __syncthreads();
            // num_aug = psi S_aug (state before the chunk) ...
            for (int e = tid; e < kT * dva; e += kTh) {
                const int i = e / dva, col = e - i * dva;
                float s = 0.f;
                for (int f = 0; f < dp; ++f) s += sPQ[i * L.ldp + f] * sS[f * dva + col];
                sG[e] = s;
            }
            // ... + sum over the chunk's keys up to the query of (psi . kappa) v_aug
            for (int kt = 0; kt <= qt; kt += kT) {
                const int nk = min(kT, Lc - kt);
                __syncthreads();
                load_phi(sh, L, Ks, t0 + kt, nk, sXk, sSqk, sPK);
                load_vaug(sh, L, Vs, t0 + kt, nk, sV);
                __syncthreads();
                {
                    const int i = tid / kT, t = tid % kT;
                    float p = 0.f;
                    if (kt + t <= qt + i)
                        for (int f = 0; f < dp; ++f) p += sPQ[i * L.ldp + f] * sPK[t * L.ldp + f];
                    sP[tid] = p;
                }
                __syncthreads();
                for (int e = tid; e < kT * dva; e += kTh) {
                    const int i = e / dva, col = e - i * dva;
                    float s = sG[e];
                    for (int t = 0; t < kT; ++t) s += sP[i * kT + t] * sV[t * dva + col];
                    sG[e] = s;
                }
            }
            __syncthreads();
            // G_aug = [dO / den | -(dO . o) / den]; rows past the end: 0
            if (tid < kT) {
                const int i = tid;
                const float den = sG[i * dva + dv];
                float dot = 0.f;
                for (int col = 0; col < dv; ++col) dot += sDO[i * dv + col] * (sG[i * dva + col] / den);
                sH[i] = i < nq ? -dot / den : 0.f;
                sRD[i] = i < nq ? 1.f / den : 0.f;
            }
            __syncthreads();
            for (int e = tid; e < kT * dva; e += kTh) {
                const int i = e / dva, col = e - i * dva;
                const float g = col < dv ? sDO[i * dv + col] * sRD[i] : sH[i];
                sG[e] = i < nq ? g : 0.f;
                if (i < nq) Gs[(size_t)(t0 + qt + i) * dva + col] = g;
            }
            __syncthreads();
            // dpsi = G_aug S_aug^T (state before the chunk) ...
            for (int e = tid; e < kT * dp; e += kTh) {
                const int i = e / dp, f = e - i * dp;
                float s = 0.f;
                for (int col = 0; col < dva; ++col) s += sG[i * dva + col] * sS[f * dva + col];
                sDP[i * L.ldp + f] = s;
            }
            // ... + sum over the chunk's keys up to the query of (G_aug . v_aug) kappa
            for (int kt = 0; kt <= qt; kt += kT) {
                const int nk = min(kT, Lc - kt);
                __syncthreads();
                load_phi(sh, L, Ks, t0 + kt, nk, sXk, sSqk, sPK);
                load_vaug(sh, L, Vs, t0 + kt, nk, sV);
                __syncthreads();
                {
                    const int i = tid / kT, t = tid % kT;
                    float p = 0.f;
                    if (kt + t <= qt + i)
                        for (int col = 0; col < dva; ++col) p += sG[i * dva + col] * sV[t * dva + col];
                    sP[tid] = p;
                }
                __syncthreads();
                for (int e = tid; e < kT * dp; e += kTh) {
                    const int i = e / dp, f = e - i * dp;
                    float s = sDP[i * L.ldp + f];
                    for (int t = 0; t < kT; ++t) s += sP[i * kT + t] * sPK[t * L.ldp + f];
                    sDP[i * L.ldp + f] = s;
                }
            }
            __syncthreads();
            store_input_grad(sh, L, sXq, sPQ, sDP, sH, nq, dQs, t0 + qt);
            __syncthreads();
        }
        // carry the state past the chunk: S_aug += kappa^T v_aug
        for (int kt = 0; kt < Lc; kt += kT) {
            const int nk = min(kT, Lc - kt);
            load_phi(sh, L, Ks, t0 + kt, nk, sXk, sSqk, sPK);
            load_vaug(sh, L, Vs, t0 + kt, nk, sV);
            __syncthreads();
            for (int e = tid; e < dp * dva; e += kTh) {
                const int f = e / dva, col = e - f * dva;
                float s = sS[e];
                for (int t = 0; t < kT; ++t) s += sPK[t * L.ldp + f] * sV[t * dva + col];
                sS[e] = s;
            }
            __syncthreads();
        }
    }
}

// U of a segment = sum over its tokens of psi_i G_aug_i^T (the reverse scan's
// input), accumulated in LDS over 16-token tiles (psi recomputed, G_aug read
// back from the workspace).
template <typename T>
__global__ __launch_bounds__(kTh) void k_bwd_usum(BwdArgs a) {
    extern __shared__ float smem[];
    const Shape sh = a.sh;
    const Segments sg = a.sg;
    const int dp = sh.dp, dk = sh.dk, dv = sh.dv;
    const BwdLayout L = bwd_layout(dk, dp, dv);
    const int dva = L.dva, naug = dp * dva;
    float *sU = smem + L.offS, *sXq = smem + L.offXq, *sSqq = smem + L.offSqq, *sPQ = smem + L.offPQ;
    float *sG = smem + L.offG;
    const int tid = threadIdx.x;
    const int seg = blockIdx.x % sg.P, bh = blockIdx.x / sg.P;
    const int N = sh.N;
    const int t_begin = seg * sg.seg_chunks * sg.chunk, t_end = min(N, t_begin + sg.seg_chunks * sg.chunk);
    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const float *Gs = a.G + (size_t)bh * N * dva;
    for (int e = tid; e < naug; e += kTh) sU[e] = 0.f;
    for (int t0 = t_begin; t0 < t_end; t0 += kT) {
        const int nq = min(kT, t_end - t0);
        __syncthreads();  // the previous tile is consumed
        load_phi(sh, L, Qs, t0, nq, sXq, sSqq, sPQ);
        for (int e = tid; e < kT * dva; e += kTh) {
            const int r = e / dva;
            sG[e] = r < nq ? Gs[(size_t)(t0 + r) * dva + (e - r * dva)] : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < naug; e += kTh) {
            const int f = e / dva, col = e - f * dva;
            float acc = sU[e];
            for (int i = 0; i < kT; ++i) acc += sPQ[i * L.ldp + f] * sG[i * dva + col];
            sU[e] = acc;
        }
    }
    __syncthreads();
    float *Us = a.U + ((size_t)bh * sg.P + seg) * naug;
    for (int e = tid; e < naug; e += kTh) Us[e] = sU[e];
}

// R_aug entering each segment: dS_out_aug + the sums of the later segments,
// added from the last segment down (fixed order); dS_in_aug = the total.
__global__ __launch_bounds__(kTh) void k_bwd_rscan(int BH, int P, int dp, int dv, float *U, const float *dS_out,
                                                   const float *dz_out, float *dS_in, float *dz_in) {
    const int dva = dv + 1, naug = dp * dva;
    const int bps = (naug + kTh - 1) / kTh;
    const int bh = blockIdx.x / bps;
    const int e = (blockIdx.x - bh * bps) * kTh + threadIdx.x;
    if (bh >= BH || e >= naug) return;
    const int f = e / dva, c = e - f * dva;
    float acc = 0.f;
    if (dS_out) acc = c < dv ? dS_out[((size_t)bh * dp + f) * dv + c] : dz_out[(size_t)bh * dp + f];
    float *slots = U + (size_t)bh * P * naug + e;
    for (int s = P - 1; s >= 0; --s) {
        const float d = slots[(size_t)s * naug];
        slots[(size_t)s * naug] = acc;
        acc += d;
    }
    if (dS_in) {
        if (c < dv) dS_in[((size_t)bh * dp + f) * dv + c] = acc;
        else dz_in[(size_t)bh * dp + f] = acc;
    }
}

template <typename T>
__global__ __launch_bounds__(kTh) void k_bwd_dkv(BwdArgs a) {
    extern __shared__ float smem[];
    const Shape sh = a.sh;
    const Segments sg = a.sg;
    const int dp = sh.dp, dk = sh.dk, dv = sh.dv;
    const BwdLayout L = bwd_layout(dk, dp, dv);
    const int dva = L.dva;
    float *sR = smem + L.offS, *sXq = smem + L.offXq, *sSqq = smem + L.offSqq, *sPQ = smem + L.offPQ;
    float *sXk = smem + L.offXk, *sSqk = smem + L.offSqk, *sPK = smem + L.offPK, *sV = smem + L.offV;
    float *sG = smem + L.offG, *sP = smem + L.offP, *sB = smem + L.offB, *sDP = smem + L.offDP;
    float *sDV = smem + L.offDV, *sH = smem + L.offH;
    const int tid = threadIdx.x;
    const int seg = blockIdx.x % sg.P, bh = blockIdx.x / sg.P;
    const int N = sh.N, C = sg.chunk;
    const int c_begin = seg * sg.seg_chunks, c_end = min(sg.n_chunks, c_begin + sg.seg_chunks);
    const T *Qs = static_cast<const T *>(a.Q) + (size_t)bh * N * dk;
    const T *Ks = static_cast<const T *>(a.K) + (size_t)bh * N * dk;
    const T *Vs = static_cast<const T *>(a.V) + (size_t)bh * N * dv;
    T *dKs = static_cast<T *>(a.dK) + (size_t)bh * N * dk;
    T *dVs = static_cast<T *>(a.dV) + (size_t)bh * N * dv;
    const float *Gs = a.G + (size_t)bh * N * dva;
    const int naug = dp * dva;

    const float *Rs = a.U + ((size_t)bh * sg.P + seg) * naug;  // suffix of the later segments
    for (int e = tid; e < naug; e += kTh) sR[e] = Rs[e];
    __syncthreads();

    auto load_g = [&](int row0, int nvalid) {
        for (int e = tid; e < kT * dva; e += kTh) {
            const int r = e / dva;
            sG[e] = r < nvalid ? Gs[(size_t)(row0 + r) * dva + (e - r * dva)] : 0.f;
        }
    };

    for (int c = c_end - 1; c >= c_begin; --c) {
        const int t0 = c * C, Lc = min(C, N - t0);
        for (int kt = 0; kt < Lc; kt += kT) {
            const int nk = min(kT, Lc - kt);
            load_phi(sh, L, Ks, t0 + kt, nk, sXk, sSqk, sPK);
            load_vaug(sh, L, Vs, t0 + kt, nk, sV);
            __syncthreads();
            // from the later chunks: dkappa = R_aug v_aug, dv = R^T kappa
            for (int e = tid; e < kT * dp; e += kTh) {
                const int j = e / dp, f = e - j * dp;
                float s = 0.f;
                for (int col = 0; col < dva; ++col) s += sR[f * dva + col] * sV[j * dva + col];
                sDP[j * L.ldp + f] = s;
            }
            for (int e = tid; e < kT * dv; e += kTh) {
                const int j = e / dv, col = e - j * dv;
                float s = 0.f;
                for (int f = 0; f < dp; ++f) s += sPK[j * L.ldp + f] * sR[f * dva + col];
                sDV[e] = s;
            }
            // from the chunk's queries at or after each key
            for (int qt = kt; qt < Lc; qt += kT) {
                const int nq = min(kT, Lc - qt);
                __syncthreads();
                load_phi(sh, L, Qs, t0 + qt, nq, sXq, sSqq, sPQ);
                load_g(t0 + qt, nq);
                __syncthreads();
                {
                    const int j = tid / kT, i = tid % kT;
                    float p = 0.f, b = 0.f;
                    if (kt + j <= qt + i) {
                        for (int f = 0; f < dp; ++f) p += sPK[j * L.ldp + f] * sPQ[i * L.ldp + f];
                        for (int col = 0; col < dva; ++col) b += sV[j * dva + col] * sG[i * dva + col];
                    }
                    sP[tid] = p;
                    sB[tid] = b;
                }
                __syncthreads();
                for (int e = tid; e < kT * dp; e += kTh) {
                    const int j = e / dp, f = e - j * dp;
                    float s = sDP[j * L.ldp + f];
                    for (int i = 0; i < kT; ++i) s += sB[j * kT + i] * sPQ[i * L.ldp + f];
                    sDP[j * L.ldp + f] = s;
                }
                for (int e = tid; e < kT * dv; e += kTh) {
                    const int j = e / dv, col = e - j * dv;
                    float s = sDV[e];
                    for (int i = 0; i < kT; ++i) s += sP[j * kT + i] * sG[i * dva + col];
                    sDV[e] = s;
                }
            }
            __syncthreads();
            store_input_grad(sh, L, sXk, sPK, sDP, sH, nk, dKs, t0 + kt);
            for (int e = tid; e < kT * dv; e += kTh) {
                const int j = e / dv;
                if (j < nk) store_from_f32(dVs, (size_t)(t0 + kt + j) * dv + (e - j * dv), sDV[e]);
            }
            __syncthreads();
        }
        // carry R past the chunk (towards its start): R_aug += psi^T G_aug
        for (int qt = 0; qt < Lc; qt += kT) {
            const int nq = min(kT, Lc - qt);
            load_phi(sh, L, Qs, t0 + qt, nq, sXq, sSqq, sPQ);
            load_g(t0 + qt, nq);
            __syncthreads();
            for (int e = tid; e < naug; e += kTh) {
                const int f = e / dva, col = e - f * dva;
                float s = sR[e];
                for (int i = 0; i < kT; ++i) s += sPQ[i * L.ldp + f] * sG[i * dva + col];
                sR[e] = s;
            }
            __syncthreads();
        }
    }
}

template <typename K>
hipError_t launch_big_lds(K kernel, dim3 grid, size_t lds, hipStream_t st, KEvents ev, const BwdArgs &a) {
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    return launch_kernel_ev(kernel, grid, dim3(kTh), lds, st, ev, a);
}

}  // namespace

bool backward_supported(const Shape &sh) {
    if (sh.phi != kElu1 && sh.phi != kFavor) return false;
    if ((size_t)sh.dp * (sh.dv + 1) > (size_t)kMaxAug) return false;
    return backward_lds_bytes(sh) <= 160 * 1024;
}

size_t backward_lds_bytes(const Shape &sh) {
    return sizeof(float) * (size_t)bwd_layout(sh.dk, sh.dp, sh.dv).total;
}

hipError_t launch_bwd_rscan(int BH, int P, int dp, int dv, float *U, const float *dS_out, const float *dz_out,
                            float *dS_in, float *dz_in, hipStream_t st, KEvents ev) {
    const int naug = dp * (dv + 1);
    const unsigned bps = (unsigned)((naug + kTh - 1) / kTh);
    return launch_kernel_ev(k_bwd_rscan, dim3((unsigned)BH * bps), dim3(kTh), 0, st, ev, BH, P, dp, dv, U, dS_out,
                            dz_out, dS_in, dz_in);
}

hipError_t launch_backward(const BwdLaunch &b, hipStream_t st, KEvents ev_dq, KEvents ev_scan, KEvents ev_dkv) {
    BwdArgs a;
    a.sh = b.sh; a.sg = b.sg;
    a.Q = b.Q; a.K = b.K; a.V = b.V; a.dO = b.dO;
    a.dQ = b.dQ; a.dK = b.dK; a.dV = b.dV;
    a.Spre = b.Spre; a.zpre = b.zpre; a.U = b.U; a.G = b.G;
    const size_t lds = backward_lds_bytes(b.sh);
    const dim3 grid((unsigned)((size_t)b.sh.BH * b.sg.P));
    const bool f32 = b.sh.dtype == kF32;
    hipError_t e = f32 ? launch_big_lds(k_bwd_dq<float>, grid, lds, st, ev_dq, a)
                       : launch_big_lds(k_bwd_dq<uint16_t>, grid, lds, st, ev_dq, a);
    if (e != hipSuccess) return e;
    e = f32 ? launch_big_lds(k_bwd_usum<float>, grid, lds, st, KEvents{}, a)
            : launch_big_lds(k_bwd_usum<uint16_t>, grid, lds, st, KEvents{}, a);
    if (e != hipSuccess) return e;
    const int naug = b.sh.dp * (b.sh.dv + 1);
    const unsigned bps = (unsigned)((naug + kTh - 1) / kTh);
    e = launch_kernel_ev(k_bwd_rscan, dim3((unsigned)b.sh.BH * bps), dim3(kTh), 0, st, ev_scan, b.sh.BH, b.sg.P,
                         b.sh.dp, b.sh.dv, b.U, b.dS_out, b.dz_out, b.dS_in, b.dz_in);
    if (e != hipSuccess) return e;
    return f32 ? launch_big_lds(k_bwd_dkv<float>, grid, lds, st, ev_dkv, a)
               : launch_big_lds(k_bwd_dkv<uint16_t>, grid, lds, st, ev_dkv, a);
}

}  // namespace la
