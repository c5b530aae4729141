/*
 * la_oracle.c -- fp64 CPU oracle for kernelized (linear) attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark can check the HIP library against the plain
 * definitions.  It shares no code, header or constant with the HIP sources.
 *
 * Everything is computed in double precision with plain loops in the order
 * the definitions are written, ascending token index.  Independent
 * (batch, head) slices are spread over OpenMP threads; no arithmetic is
 * reordered inside a slice.
 *
 * Sources (cited by page title and section):
 *  [LA]   "Linear Attention" (aiwiki.ai): the generalised kernel attention,
 *         the factorised form, the causal running sums S_i, z_i, the
 *         feature-map table and the chunkwise parallel form.
 *  [ASSOC] "Linear Attention: Removing the Softmax Buys Associativity"
 *         (anylearn.cc): the state as a running sum of outer products that
 *         starts at zero; parallel and recurrent modes compute one function.
 *  [SOA5] "Story of Attention Part 5": section 1a (kernel linear attention,
 *         its matrix form, its recurrence and the n = 4 worked example),
 *         section 1b (Performer / FAVOR+ feature map), section 4 (RetNet
 *         retention: parallel form with the causal decay matrix D, recurrent
 *         form S_n = gamma S_{n-1} + k_n^T v_n, and its n = 4 worked
 *         example), section 5 (Infini-attention memory read), section 6
 *         (Lightning Attention blockwise split: with decay lambda = 1 for the
 *         normalised kernel attention, and with its decay for retention).
 *
 * Memory layout of every array (row-major, slices independent):
 *   Q, K  [BH, N, dk]     V, O  [BH, N, dv]
 *   S     [BH, dp, dv]    z     [BH, dp]         dp = dk (ELU+1) or m (FAVOR+)
 *   W     [m, dk]         (FAVOR+ projection rows w_r, shared by all slices)
 *
 * Retention (the decayed, unnormalised variant of section 4 / 6) uses a
 * decay gamma per head: slice s of BH = B * H has head h = s % H and decay
 * gamma[h].  The identity feature map (phi(x) = x, RetNet's raw q and k) is
 * kind 2; ELU+1 and FAVOR+ may be used with retention as well.
 *
 * Parity status: every function below is pinned by tests/test_oracle_pins.py
 * (printed worked examples, brute force agreement of independent forms,
 * closed forms, invariants, a library routine).  The FAVOR+ map is pinned
 * statistically (unbiasedness, convergence to softmax attention) and by
 * closed forms for special W; the exact value of a given finite-m FAVOR+
 * estimate has no independent pin beyond those.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORA_PHI_ELU1 0
#define ORA_PHI_FAVOR 1
#define ORA_PHI_IDENTITY 2
#define ORA_PHI_DPFP 3
#define ORA_PHI_TRIG 4
#define ORA_PHI_COSFORMER 5

/* Parameters of the maps that have one: DPFP's number of shifts nu, the
 * cosFormer horizon M, and the position of the first token of a call (the
 * cosFormer reweighting depends on absolute positions).  Set by
 * ora_set_map before a call; 0 by default. */
static int g_map_param = 0;
static long long g_pos0 = 0;

void ora_set_map(int param, long long pos0) {
    g_map_param = param;
    g_pos0 = pos0;
}

int ora_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void ora_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * Feature maps.
 * ELU+1 [LA feature-map table; SOA5 1a]: elu with alpha = 1 plus one, applied
 * per coordinate.  For x > 0 that is x + 1; otherwise exp(x) - 1 + 1, which is
 * exp(x) exactly.  Output dimension dp = d.
 * FAVOR+ [SOA5 1b]: phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), r = 1..m.
 * DPFP [LA feature-map table: concatenation of products of ReLU shifts]:
 *   r = ReLU([x, -x]) (2d entries); for shift i = 1..nu, block i holds
 *   r_j * r_{(j + i) mod 2d}, j = 0..2d-1.  Output dimension 2 d nu.
 * Cosine / sine projections [LA feature-map table]: [cos(W x); sin(W x)],
 *   cos(w_r . x) for r = 1..m, then sin(w_r . x).  Output dimension 2m.
 * cosFormer [SOA5 3]: ReLU(x) times cos(pi p / 2M), then ReLU(x) times
 *   sin(pi p / 2M), for the token at position p (counted from 0, plus the
 *   call's first position); the product of two such features is
 *   ReLU(q)^T ReLU(k) cos(pi (p_q - p_k) / 2M).  Output dimension 2d.
 * ------------------------------------------------------------------------- */
static void phi_elu1_row(const double *x, int d, double *out) {
    for (int f = 0; f < d; ++f) out[f] = x[f] > 0.0 ? x[f] + 1.0 : exp(x[f]);
}

static void phi_favor_row(const double *x, int d, const double *W, int m, double *out) {
    double sq = 0.0;
    for (int c = 0; c < d; ++c) sq += x[c] * x[c];
    double inv_sqrt_m = 1.0 / sqrt((double)m);
    for (int r = 0; r < m; ++r) {
        double proj = 0.0;
        for (int c = 0; c < d; ++c) proj += W[(size_t)r * d + c] * x[c];
        out[r] = exp(proj - 0.5 * sq) * inv_sqrt_m;
    }
}

static void phi_dpfp_row(const double *x, int d, int nu, double *out) {
    const int n2 = 2 * d;
    double *r = (double *)malloc(sizeof(double) * n2);
    for (int j = 0; j < d; ++j) {
        r[j] = x[j] > 0.0 ? x[j] : 0.0;
        r[d + j] = -x[j] > 0.0 ? -x[j] : 0.0;
    }
    for (int i = 1; i <= nu; ++i)
        for (int j = 0; j < n2; ++j) out[(size_t)(i - 1) * n2 + j] = r[j] * r[(j + i) % n2];
    free(r);
}

static void phi_trig_row(const double *x, int d, const double *W, int m, double *out) {
    for (int r = 0; r < m; ++r) {
        double proj = 0.0;
        for (int c = 0; c < d; ++c) proj += W[(size_t)r * d + c] * x[c];
        out[r] = cos(proj);
        out[m + r] = sin(proj);
    }
}

static void phi_cosformer_row(const double *x, int d, long long pos, double *out) {
    const double pi = 3.14159265358979323846;
    const double ang = pi * (double)pos / (2.0 * (double)g_map_param);
    const double cw = cos(ang), sw = sin(ang);
    for (int c = 0; c < d; ++c) {
        const double r = x[c] > 0.0 ? x[c] : 0.0;
        out[c] = r * cw;
        out[d + c] = r * sw;
    }
}

/* phi of one row x [d] of the token at position `pos` within the call */
static void phi_row(int kind, const double *x, int d, const double *W, int m, long long pos, double *out) {
    if (kind == ORA_PHI_FAVOR) phi_favor_row(x, d, W, m, out);
    else if (kind == ORA_PHI_IDENTITY) memcpy(out, x, sizeof(double) * d);
    else if (kind == ORA_PHI_DPFP) phi_dpfp_row(x, d, g_map_param, out);
    else if (kind == ORA_PHI_TRIG) phi_trig_row(x, d, W, m, out);
    else if (kind == ORA_PHI_COSFORMER) phi_cosformer_row(x, d, g_pos0 + pos, out);
    else phi_elu1_row(x, d, out);
}

static int feat_dim(int kind, int dk, int m) {
    switch (kind) {
        case ORA_PHI_FAVOR: return m;
        case ORA_PHI_DPFP: return 2 * dk * g_map_param;
        case ORA_PHI_TRIG: return 2 * m;
        case ORA_PHI_COSFORMER: return 2 * dk;
        default: return dk;
    }
}

/* phi applied to n rows of X [n, d] at positions row0.. -> out [n, dp]. */
static void phi_rows_at(int kind, int n, int d, const double *X, int m, const double *W, long long row0,
                        double *out) {
    int dp = feat_dim(kind, d, m);
    for (int i = 0; i < n; ++i) phi_row(kind, X + (size_t)i * d, d, W, m, row0 + i, out + (size_t)i * dp);
}

/* phi applied to n rows of X [n, d] (positions 0..n-1) -> out [n, dp]. */
void ora_phi(int kind, int n, int d, const double *X, int m, const double *W, double *out) {
    phi_rows_at(kind, n, d, X, m, W, 0, out);
}

int ora_feature_dim(int kind, int dk, int m) { return feat_dim(kind, dk, m); }

/* ---------------------------------------------------------------------------
 * State read [SOA5 5 (memory read num = sigma(Q) M, den = sigma(Q) z);
 * SOA5 6 (the Q_i S_{i-1} inter-block term)]:
 *   num[i, j] = sum_f phiQ[i, f] S[f, j],   den[i] = sum_f phiQ[i, f] z[f].
 * ------------------------------------------------------------------------- */
void ora_state_read(int n, int dp, int dv, const double *phiQ, const double *S, const double *z,
                    double *num, double *den) {
    for (int i = 0; i < n; ++i) {
        const double *pq = phiQ + (size_t)i * dp;
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int f = 0; f < dp; ++f) acc += pq[f] * S[(size_t)f * dv + j];
            num[(size_t)i * dv + j] = acc;
        }
        double dacc = 0.0;
        for (int f = 0; f < dp; ++f) dacc += pq[f] * z[f];
        den[i] = dacc;
    }
}

/* helpers: per-slice phi of all rows */
static double *phi_all(int kind, int N, int dk, const double *X, int m, const double *W) {
    int dp = feat_dim(kind, dk, m);
    double *out = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * dp);
    ora_phi(kind, N, dk, X, m, W, out);
    return out;
}

/* ---------------------------------------------------------------------------
 * Non-causal factorised attention [LA factorised form; SOA5 1a matrix form]:
 *   S = sum_j phi(k_j) v_j^T,  z = sum_j phi(k_j),
 *   y_i = (phi(q_i)^T S) / (phi(q_i)^T z).
 * S_out, z_out (may be NULL) receive S and z.
 * ------------------------------------------------------------------------- */
void ora_noncausal(int BH, int N, int dk, int dv, int kind, int m, const double *W,
                   const double *Q, const double *K, const double *V,
                   double *O, double *S_out, double *z_out) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *pk = phi_all(kind, N, dk, k, m, W);
        double *pq = phi_all(kind, N, dk, q, m, W);
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        double *z = (double *)calloc((size_t)dp, sizeof(double));
        for (int j = 0; j < N; ++j)
            for (int f = 0; f < dp; ++f) {
                double a = pk[(size_t)j * dp + f];
                z[f] += a;
                for (int c = 0; c < dv; ++c) S[(size_t)f * dv + c] += a * v[(size_t)j * dv + c];
            }
        double *num = (double *)malloc(sizeof(double) * dv);
        double den;
        for (int i = 0; i < N; ++i) {
            ora_state_read(1, dp, dv, pq + (size_t)i * dp, S, z, num, &den);
            for (int c = 0; c < dv; ++c) O[((size_t)s * N + i) * dv + c] = num[c] / den;
        }
        if (S_out) memcpy(S_out + (size_t)s * dp * dv, S, sizeof(double) * dp * dv);
        if (z_out) memcpy(z_out + (size_t)s * dp, z, sizeof(double) * dp);
        free(num); free(S); free(z); free(pk); free(pq);
    }
}

/* ---------------------------------------------------------------------------
 * Causal recurrence [LA causal running sums; SOA5 1a recurrence;
 * ASSOC: the state starts from zero]:
 *   S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *   y_i = phi(q_i)^T S_i / phi(q_i)^T z_i      (update, then read)
 * with S_0, z_0 = S_in, z_in (zero when S_in == NULL).
 * ------------------------------------------------------------------------- */
void ora_causal_recurrent(int BH, int N, int dk, int dv, int kind, int m, const double *W,
                          const double *Q, const double *K, const double *V,
                          const double *S_in, const double *z_in,
                          double *O, double *S_out, double *z_out) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        double *z = (double *)calloc((size_t)dp, sizeof(double));
        if (S_in) {
            memcpy(S, S_in + (size_t)s * dp * dv, sizeof(double) * dp * dv);
            memcpy(z, z_in + (size_t)s * dp, sizeof(double) * dp);
        }
        double *pk = (double *)malloc(sizeof(double) * dp);
        double *pq = (double *)malloc(sizeof(double) * dp);
        double *num = (double *)malloc(sizeof(double) * dv);
        double den;
        for (int i = 0; i < N; ++i) {
            phi_row(kind, k + (size_t)i * dk, dk, W, m, i, pk);
            for (int f = 0; f < dp; ++f) {
                z[f] += pk[f];
                for (int c = 0; c < dv; ++c) S[(size_t)f * dv + c] += pk[f] * v[(size_t)i * dv + c];
            }
            phi_row(kind, q + (size_t)i * dk, dk, W, m, i, pq);
            ora_state_read(1, dp, dv, pq, S, z, num, &den);
            for (int c = 0; c < dv; ++c) O[((size_t)s * N + i) * dv + c] = num[c] / den;
        }
        if (S_out) memcpy(S_out + (size_t)s * dp * dv, S, sizeof(double) * dp * dv);
        if (z_out) memcpy(z_out + (size_t)s * dp, z, sizeof(double) * dp);
        free(S); free(z); free(pk); free(pq); free(num);
    }
}

/* ---------------------------------------------------------------------------
 * Quadratic (parallel-mode) brute force [LA generalised kernel attention with
 * sim(q, k) = phi(q)^T phi(k); ASSOC parallel mode]:
 *   y_i = [phi(q_i)^T S_in + sum_j sim(q_i, k_j) v_j]
 *         / [phi(q_i)^T z_in + sum_j sim(q_i, k_j)]
 * with j over all positions (causal == 0) or j <= i (causal != 0).
 * No state is formed: every similarity is an explicit pair.
 * ------------------------------------------------------------------------- */
void ora_quadratic(int BH, int N, int dk, int dv, int kind, int m, const double *W,
                   const double *Q, const double *K, const double *V,
                   const double *S_in, const double *z_in, int causal, double *O) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *pk = phi_all(kind, N, dk, k, m, W);
        double *pq = phi_all(kind, N, dk, q, m, W);
        double *num = (double *)malloc(sizeof(double) * dv);
        for (int i = 0; i < N; ++i) {
            double den = 0.0;
            const double *pqi = pq + (size_t)i * dp;
            if (S_in) {
                ora_state_read(1, dp, dv, pqi, S_in + (size_t)s * dp * dv, z_in + (size_t)s * dp, num, &den);
            } else {
                for (int c = 0; c < dv; ++c) num[c] = 0.0;
            }
            int jmax = causal ? i : N - 1;
            for (int j = 0; j <= jmax; ++j) {
                double sim = 0.0;
                for (int f = 0; f < dp; ++f) sim += pqi[f] * pk[(size_t)j * dp + f];
                den += sim;
                for (int c = 0; c < dv; ++c) num[c] += sim * v[(size_t)j * dv + c];
            }
            for (int c = 0; c < dv; ++c) O[((size_t)s * N + i) * dv + c] = num[c] / den;
        }
        free(num); free(pk); free(pq);
    }
}

/* ---------------------------------------------------------------------------
 * Chunkwise form [LA chunkwise parallel form; SOA5 6 blockwise split with
 * lambda = 1, plus the kernel-attention normaliser of SOA5 1a].  Tokens are
 * cut into consecutive chunks of C (the last may be shorter).  For a chunk
 * with rows i and state (S, z) carried from the previous chunks:
 *   P[i, t]  = phi(q_i)^T phi(k_t) for t <= i in the chunk, else 0,
 *   num_i    = sum_t P[i, t] v_t + phi(q_i)^T S,
 *   den_i    = sum_t P[i, t]     + phi(q_i)^T z,
 *   y_i      = num_i / den_i,
 * then S += phi(K_c)^T V_c and z += phi(K_c)^T 1.
 * ------------------------------------------------------------------------- */
void ora_causal_chunked(int BH, int N, int dk, int dv, int kind, int m, const double *W,
                        const double *Q, const double *K, const double *V,
                        const double *S_in, const double *z_in, int C,
                        double *O, double *S_out, double *z_out) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        double *z = (double *)calloc((size_t)dp, sizeof(double));
        if (S_in) {
            memcpy(S, S_in + (size_t)s * dp * dv, sizeof(double) * dp * dv);
            memcpy(z, z_in + (size_t)s * dp, sizeof(double) * dp);
        }
        double *pq = (double *)malloc(sizeof(double) * (size_t)C * dp);
        double *pk = (double *)malloc(sizeof(double) * (size_t)C * dp);
        double *P = (double *)malloc(sizeof(double) * (size_t)C * C);
        double *num = (double *)malloc(sizeof(double) * (size_t)C * dv);
        double *den = (double *)malloc(sizeof(double) * (size_t)C);
        for (int t0 = 0; t0 < N; t0 += C) {
            int L = N - t0 < C ? N - t0 : C;
            phi_rows_at(kind, L, dk, q + (size_t)t0 * dk, m, W, t0, pq);
            phi_rows_at(kind, L, dk, k + (size_t)t0 * dk, m, W, t0, pk);
            /* masked intra-chunk similarities */
            for (int i = 0; i < L; ++i)
                for (int t = 0; t < L; ++t) {
                    double a = 0.0;
                    if (t <= i)
                        for (int f = 0; f < dp; ++f) a += pq[(size_t)i * dp + f] * pk[(size_t)t * dp + f];
                    P[(size_t)i * C + t] = a;
                }
            /* inter-chunk read of the carried state */
            ora_state_read(L, dp, dv, pq, S, z, num, den);
            /* intra-chunk numerator and denominator, then normalise */
            for (int i = 0; i < L; ++i) {
                for (int t = 0; t < L; ++t) {
                    double a = P[(size_t)i * C + t];
                    den[i] += a;
                    for (int c = 0; c < dv; ++c) num[(size_t)i * dv + c] += a * v[(size_t)(t0 + t) * dv + c];
                }
                for (int c = 0; c < dv; ++c)
                    O[((size_t)s * N + t0 + i) * dv + c] = num[(size_t)i * dv + c] / den[i];
            }
            /* carry the state past this chunk */
            for (int f = 0; f < dp; ++f)
                for (int t = 0; t < L; ++t) {
                    double a = pk[(size_t)t * dp + f];
                    z[f] += a;
                    for (int c = 0; c < dv; ++c) S[(size_t)f * dv + c] += a * v[(size_t)(t0 + t) * dv + c];
                }
        }
        if (S_out) memcpy(S_out + (size_t)s * dp * dv, S, sizeof(double) * dp * dv);
        if (z_out) memcpy(z_out + (size_t)s * dp, z, sizeof(double) * dp);
        free(S); free(z); free(pq); free(pk); free(P); free(num); free(den);
    }
}

/* ---------------------------------------------------------------------------
 * One recurrent decode step [LA: constant work per generated token; SOA5 1a
 * recurrence]: S += phi(k) v^T, z += phi(k), o = phi(q)^T S / phi(q)^T z.
 * q, k [BH, dk]; v, o [BH, dv]; S [BH, dp, dv] and z [BH, dp] updated in place.
 * ------------------------------------------------------------------------- */
void ora_decode_step(int BH, int dk, int dv, int kind, int m, const double *W,
                     const double *q, const double *k, const double *v,
                     double *S, double *z, double *o) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(static)
    for (int s = 0; s < BH; ++s) {
        double *pk = (double *)malloc(sizeof(double) * dp);
        double *pq = (double *)malloc(sizeof(double) * dp);
        double *Ss = S + (size_t)s * dp * dv, *zs = z + (size_t)s * dp;
        const double *vs = v + (size_t)s * dv;
        phi_row(kind, k + (size_t)s * dk, dk, W, m, 0, pk);
        phi_row(kind, q + (size_t)s * dk, dk, W, m, 0, pq);
        for (int f = 0; f < dp; ++f) {
            zs[f] += pk[f];
            for (int c = 0; c < dv; ++c) Ss[(size_t)f * dv + c] += pk[f] * vs[c];
        }
        double den;
        ora_state_read(1, dp, dv, pq, Ss, zs, o + (size_t)s * dv, &den);
        for (int c = 0; c < dv; ++c) o[(size_t)s * dv + c] /= den;
        free(pk); free(pq);
    }
}

/* ===========================================================================
 * Retention: decayed, unnormalised linear attention [SOA5 4 RetNet; SOA5 6
 * Lightning Attention].  There is no normaliser z: the outputs are the
 * decayed numerators.  gamma[H]: decay of head h; slice s uses gamma[s % H].
 * S [BH, dp, dv] only.
 * ======================================================================== */

/* Recurrent form [SOA5 4]: S_n = gamma S_{n-1} + phi(k_n) v_n^T,
 * o_n = phi(q_n)^T S_n (update, then read), S_0 = S_in or zero. */
void ora_retention_recurrent(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                             const double *gamma, const double *Q, const double *K, const double *V,
                             const double *S_in, double *O, double *S_out) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double g = gamma[s % H];
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        if (S_in) memcpy(S, S_in + (size_t)s * dp * dv, sizeof(double) * dp * dv);
        double *pk = (double *)malloc(sizeof(double) * dp);
        double *pq = (double *)malloc(sizeof(double) * dp);
        for (int i = 0; i < N; ++i) {
            phi_row(kind, k + (size_t)i * dk, dk, W, m, i, pk);
            for (int f = 0; f < dp; ++f)
                for (int c = 0; c < dv; ++c)
                    S[(size_t)f * dv + c] = g * S[(size_t)f * dv + c] + pk[f] * v[(size_t)i * dv + c];
            phi_row(kind, q + (size_t)i * dk, dk, W, m, i, pq);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < dp; ++f) acc += pq[f] * S[(size_t)f * dv + c];
                O[((size_t)s * N + i) * dv + c] = acc;
            }
        }
        if (S_out) memcpy(S_out + (size_t)s * dp * dv, S, sizeof(double) * dp * dv);
        free(S); free(pk); free(pq);
    }
}

/* Parallel form [SOA5 4]: O = (phi(Q) phi(K)^T (.) D) V with the causal decay
 * matrix D_ij = gamma^(i-j) for i >= j, else 0.  A starting state S_in
 * enters as it does in the recurrence unrolled from it: token i (counting
 * from 0) reads gamma^(i+1) phi(q_i)^T S_in.  Every pair is explicit. */
void ora_retention_parallel(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                            const double *gamma, const double *Q, const double *K, const double *V,
                            const double *S_in, double *O) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double g = gamma[s % H];
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *pk = phi_all(kind, N, dk, k, m, W);
        double *pq = phi_all(kind, N, dk, q, m, W);
        for (int i = 0; i < N; ++i) {
            const double *pqi = pq + (size_t)i * dp;
            for (int c = 0; c < dv; ++c) O[((size_t)s * N + i) * dv + c] = 0.0;
            if (S_in) {
                const double *Si = S_in + (size_t)s * dp * dv;
                const double w = pow(g, (double)(i + 1));
                for (int c = 0; c < dv; ++c) {
                    double acc = 0.0;
                    for (int f = 0; f < dp; ++f) acc += pqi[f] * Si[(size_t)f * dv + c];
                    O[((size_t)s * N + i) * dv + c] += w * acc;
                }
            }
            for (int j = 0; j <= i; ++j) {
                double qk = 0.0;
                for (int f = 0; f < dp; ++f) qk += pqi[f] * pk[(size_t)j * dp + f];
                const double a = qk * pow(g, (double)(i - j)); /* (Q K^T (.) D)_ij */
                for (int c = 0; c < dv; ++c) O[((size_t)s * N + i) * dv + c] += a * v[(size_t)j * dv + c];
            }
        }
        free(pk); free(pq);
    }
}

/* Blockwise form [SOA5 6, Lightning Attention], blocks of C tokens (the last
 * may be shorter, of length L).  With rows s, t = 1..L of a block and
 * lambda = gamma[h]:
 *   O_i = (phi(Q_i) phi(K_i)^T (.) M) V_i + Lambda phi(Q_i) S_{i-1},
 *   S_i = lambda^L S_{i-1} + (lambda^L Lambda^{-1} phi(K_i))^T V_i,
 * M_st = lambda^(s-t) for s >= t else 0, Lambda = diag(lambda^1..lambda^L).
 * The key scale lambda^L (Lambda^{-1})_tt is evaluated as lambda^(L-t), the
 * same number without the overflow of lambda^-t on its own. */
void ora_retention_chunked(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                           const double *gamma, const double *Q, const double *K, const double *V,
                           const double *S_in, int C, double *O, double *S_out) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double lam = gamma[s % H];
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        if (S_in) memcpy(S, S_in + (size_t)s * dp * dv, sizeof(double) * dp * dv);
        double *pq = (double *)malloc(sizeof(double) * (size_t)C * dp);
        double *pk = (double *)malloc(sizeof(double) * (size_t)C * dp);
        double *A = (double *)malloc(sizeof(double) * (size_t)C * C);
        double *Sn = (double *)malloc(sizeof(double) * (size_t)dp * dv);
        for (int t0 = 0; t0 < N; t0 += C) {
            int L = N - t0 < C ? N - t0 : C;
            phi_rows_at(kind, L, dk, q + (size_t)t0 * dk, m, W, t0, pq);
            phi_rows_at(kind, L, dk, k + (size_t)t0 * dk, m, W, t0, pk);
            /* intra-block scores with the causal-decay mask M (rows i, cols t, 0-based) */
            for (int i = 0; i < L; ++i)
                for (int t = 0; t < L; ++t) {
                    double a = 0.0;
                    if (t <= i) {
                        for (int f = 0; f < dp; ++f) a += pq[(size_t)i * dp + f] * pk[(size_t)t * dp + f];
                        a *= pow(lam, (double)(i - t));
                    }
                    A[(size_t)i * C + t] = a;
                }
            for (int i = 0; i < L; ++i) {
                const double lam_row = pow(lam, (double)(i + 1)); /* Lambda_ii */
                for (int c = 0; c < dv; ++c) {
                    double intra = 0.0, inter = 0.0;
                    for (int t = 0; t < L; ++t) intra += A[(size_t)i * C + t] * v[(size_t)(t0 + t) * dv + c];
                    for (int f = 0; f < dp; ++f) inter += pq[(size_t)i * dp + f] * S[(size_t)f * dv + c];
                    O[((size_t)s * N + t0 + i) * dv + c] = intra + lam_row * inter;
                }
            }
            /* state carried past the block */
            const double lamL = pow(lam, (double)L);
            for (int f = 0; f < dp; ++f)
                for (int c = 0; c < dv; ++c) {
                    double acc = lamL * S[(size_t)f * dv + c];
                    for (int t = 0; t < L; ++t)
                        acc += pow(lam, (double)(L - (t + 1))) * pk[(size_t)t * dp + f] * v[(size_t)(t0 + t) * dv + c];
                    Sn[(size_t)f * dv + c] = acc;
                }
            memcpy(S, Sn, sizeof(double) * dp * dv);
        }
        if (S_out) memcpy(S_out + (size_t)s * dp * dv, S, sizeof(double) * dp * dv);
        free(S); free(pq); free(pk); free(A); free(Sn);
    }
}

/* One retention decode step [SOA5 4 recurrent form]: S = gamma S + phi(k) v^T,
 * o = phi(q)^T S.  q, k [BH, dk]; v, o [BH, dv]; S [BH, dp, dv] in place. */
void ora_retention_decode_step(int BH, int H, int dk, int dv, int kind, int m, const double *W,
                               const double *gamma, const double *q, const double *k, const double *v,
                               double *S, double *o) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(static)
    for (int s = 0; s < BH; ++s) {
        const double g = gamma[s % H];
        double *pk = (double *)malloc(sizeof(double) * dp);
        double *pq = (double *)malloc(sizeof(double) * dp);
        double *Ss = S + (size_t)s * dp * dv;
        const double *vs = v + (size_t)s * dv;
        phi_row(kind, k + (size_t)s * dk, dk, W, m, 0, pk);
        phi_row(kind, q + (size_t)s * dk, dk, W, m, 0, pq);
        for (int f = 0; f < dp; ++f)
            for (int c = 0; c < dv; ++c) Ss[(size_t)f * dv + c] = g * Ss[(size_t)f * dv + c] + pk[f] * vs[c];
        for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int f = 0; f < dp; ++f) acc += pq[f] * Ss[(size_t)f * dv + c];
            o[(size_t)s * dv + c] = acc;
        }
        free(pk); free(pq);
    }
}

/* ---------------------------------------------------------------------------
 * Backward of the causal form.  The pages present the parallel (quadratic)
 * mode as the training mode [ASSOC, the two computation modes] but give no
 * gradients; this is reverse-mode differentiation of the causal recurrence
 * above, written out.  With kappa_j = phi(k_j), psi_i = phi(q_i):
 *   forward:  S_i = S_{i-1} + kappa_i v_i^T, z_i = z_{i-1} + kappa_i,
 *             num_i = S_i^T psi_i, den_i = z_i^T psi_i, o_i = num_i / den_i,
 *             S_out = S_N, z_out = z_N.
 * For a loss L with dO_i = dL/do_i and dS_out, dz_out = dL/dS_N, dL/dz_N:
 *   g_i = dL/dnum_i = dO_i / den_i,   h_i = dL/dden_i = -(dO_i . o_i) / den_i,
 *   dpsi_i = S_i g_i + z_i h_i                         (forward sweep),
 *   R_j = dS_out + sum_{i >= j} psi_i g_i^T,  r_j = dz_out + sum_{i >= j} psi_i h_i,
 *   dkappa_j = R_j v_j + r_j,   dv_j = R_j^T kappa_j   (reverse sweep),
 *   dS_in = R_1, dz_in = r_1.
 * The map's Jacobian takes dpsi, dkappa back to the inputs:
 *   ELU+1: dx = dphi * (x > 0 ? 1 : exp(x));  identity: dx = dphi;
 *   FAVOR+: dphi_r/dx = phi_r (w_r - x), so dx = sum_r dphi_r phi_r (w_r - x)
 *   (W is a fixed random projection: no gradient for it).
 * dS_out / dz_out may be NULL (zero); dS_in / dz_in may be NULL (not wanted).
 * ------------------------------------------------------------------------- */
static void phi_vjp_row(int kind, const double *x, int d, const double *W, int m, const double *dphi, double *dx) {
    if (kind == ORA_PHI_FAVOR) {
        double *ph = (double *)malloc(sizeof(double) * m);
        phi_favor_row(x, d, W, m, ph);
        double s = 0.0;
        for (int r = 0; r < m; ++r) s += dphi[r] * ph[r];
        for (int c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int r = 0; r < m; ++r) acc += dphi[r] * ph[r] * W[(size_t)r * d + c];
            dx[c] = acc - s * x[c];
        }
        free(ph);
    } else if (kind == ORA_PHI_IDENTITY) {
        for (int c = 0; c < d; ++c) dx[c] = dphi[c];
    } else if (kind != ORA_PHI_ELU1) {  /* the other maps are not differentiated here */
        for (int c = 0; c < d; ++c) dx[c] = NAN;
    } else {
        for (int c = 0; c < d; ++c) dx[c] = dphi[c] * (x[c] > 0.0 ? 1.0 : exp(x[c]));
    }
}

void ora_causal_backward(int BH, int N, int dk, int dv, int kind, int m, const double *W,
                         const double *Q, const double *K, const double *V,
                         const double *S_in, const double *z_in,
                         const double *dO, const double *dS_out, const double *dz_out,
                         double *dQ, double *dK, double *dV, double *dS_in, double *dz_in) {
    int dp = feat_dim(kind, dk, m);
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        const double *dOs = dO + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dp * dv, sizeof(double));
        double *z = (double *)calloc((size_t)dp, sizeof(double));
        if (S_in) {
            memcpy(S, S_in + (size_t)s * dp * dv, sizeof(double) * dp * dv);
            memcpy(z, z_in + (size_t)s * dp, sizeof(double) * dp);
        }
        double *psi = (double *)malloc(sizeof(double) * (size_t)N * dp);  /* phi(q_i), kept for the reverse sweep */
        double *g = (double *)malloc(sizeof(double) * (size_t)N * dv);
        double *h = (double *)malloc(sizeof(double) * (size_t)N);
        double *kap = (double *)malloc(sizeof(double) * dp);
        double *num = (double *)malloc(sizeof(double) * dv);
        double *dphi = (double *)malloc(sizeof(double) * dp);
        /* forward sweep: the state after token i, the output, g_i, h_i and dpsi_i */
        for (int i = 0; i < N; ++i) {
            phi_row(kind, k + (size_t)i * dk, dk, W, m, i, kap);
            for (int f = 0; f < dp; ++f) {
                z[f] += kap[f];
                for (int c = 0; c < dv; ++c) S[(size_t)f * dv + c] += kap[f] * v[(size_t)i * dv + c];
            }
            double *ps = psi + (size_t)i * dp;
            phi_row(kind, q + (size_t)i * dk, dk, W, m, i, ps);
            double den;
            ora_state_read(1, dp, dv, ps, S, z, num, &den);
            double dot = 0.0;
            for (int c = 0; c < dv; ++c) dot += dOs[(size_t)i * dv + c] * (num[c] / den);
            for (int c = 0; c < dv; ++c) g[(size_t)i * dv + c] = dOs[(size_t)i * dv + c] / den;
            h[i] = -dot / den;
            for (int f = 0; f < dp; ++f) {
                double acc = 0.0;
                for (int c = 0; c < dv; ++c) acc += S[(size_t)f * dv + c] * g[(size_t)i * dv + c];
                dphi[f] = acc + z[f] * h[i];
            }
            phi_vjp_row(kind, q + (size_t)i * dk, dk, W, m, dphi, dQ + ((size_t)s * N + i) * dk);
        }
        /* reverse sweep: R, r accumulate psi_i g_i^T, psi_i h_i from the end */
        double *R = S, *r = z; /* reuse the buffers */
        if (dS_out) memcpy(R, dS_out + (size_t)s * dp * dv, sizeof(double) * dp * dv);
        else memset(R, 0, sizeof(double) * dp * dv);
        if (dz_out) memcpy(r, dz_out + (size_t)s * dp, sizeof(double) * dp);
        else memset(r, 0, sizeof(double) * dp);
        for (int j = N - 1; j >= 0; --j) {
            const double *ps = psi + (size_t)j * dp;
            for (int f = 0; f < dp; ++f) {
                r[f] += ps[f] * h[j];
                for (int c = 0; c < dv; ++c) R[(size_t)f * dv + c] += ps[f] * g[(size_t)j * dv + c];
            }
            phi_row(kind, k + (size_t)j * dk, dk, W, m, j, kap);
            for (int f = 0; f < dp; ++f) {
                double acc = r[f];
                for (int c = 0; c < dv; ++c) acc += R[(size_t)f * dv + c] * v[(size_t)j * dv + c];
                dphi[f] = acc;
            }
            phi_vjp_row(kind, k + (size_t)j * dk, dk, W, m, dphi, dK + ((size_t)s * N + j) * dk);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < dp; ++f) acc += R[(size_t)f * dv + c] * kap[f];
                dV[((size_t)s * N + j) * dv + c] = acc;
            }
        }
        if (dS_in) memcpy(dS_in + (size_t)s * dp * dv, R, sizeof(double) * dp * dv);
        if (dz_in) memcpy(dz_in + (size_t)s * dp, r, sizeof(double) * dp);
        free(S); free(z); free(psi); free(g); free(h); free(kap); free(num); free(dphi);
    }
}

/* ---------------------------------------------------------------------------
 * Gated and delta-rule states ("Linear Attention" (aiwiki.ai), the GLA gated
 * recurrence and the delta-rule update; "Story of Attention Part 5", section 7
 * Gated DeltaNet).  Raw q, k (no feature map), no normaliser; the state is
 * feature-major S [dk][dv] as everywhere in this file, so the page's S k
 * (what the state returns for key k) is S^T k here, and the page's outer
 * product x k^T is k x^T here.  Output after the update: o_t = S_t^T q_t.
 *
 * GLA with a diagonal gate over the key channels (the gate matrix G_t =
 * alpha_t 1^T multiplies row f of S by alpha_t[f]):
 *   S_t = diag(alpha_t) S_{t-1} + k_t v_t^T,        alpha [BH, N, dk]
 * ------------------------------------------------------------------------- */
void ora_gla_recurrent(int BH, int N, int dk, int dv, const double *Q, const double *K, const double *V,
                       const double *A, const double *S_in, double *O, double *S_out) {
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        const double *a = A + (size_t)s * N * dk;
        double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
        if (S_in) memcpy(S, S_in + (size_t)s * dk * dv, sizeof(double) * dk * dv);
        for (int t = 0; t < N; ++t) {
            for (int f = 0; f < dk; ++f)
                for (int c = 0; c < dv; ++c)
                    S[(size_t)f * dv + c] = a[(size_t)t * dk + f] * S[(size_t)f * dv + c] +
                                            k[(size_t)t * dk + f] * v[(size_t)t * dv + c];
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < dk; ++f) acc += q[(size_t)t * dk + f] * S[(size_t)f * dv + c];
                O[((size_t)s * N + t) * dv + c] = acc;
            }
        }
        if (S_out) memcpy(S_out + (size_t)s * dk * dv, S, sizeof(double) * dk * dv);
        free(S);
    }
}

/* ---------------------------------------------------------------------------
 * Gated delta rule [SOA5 7]: with a scalar forget gate alpha_t (1 when alpha
 * is NULL: the plain delta rule) and write strength beta_t,
 *   prediction  p_t = alpha_t S_{t-1}^T k_t
 *   S_t = alpha_t S_{t-1} + beta_t k_t (v_t - p_t)^T,   o_t = S_t^T q_t.
 * alpha, beta [BH, N].
 * ------------------------------------------------------------------------- */
void ora_delta_recurrent(int BH, int N, int dk, int dv, const double *Q, const double *K, const double *V,
                         const double *alpha, const double *beta, const double *S_in, double *O,
                         double *S_out) {
#pragma omp parallel for schedule(dynamic)
    for (int s = 0; s < BH; ++s) {
        const double *q = Q + (size_t)s * N * dk, *k = K + (size_t)s * N * dk, *v = V + (size_t)s * N * dv;
        double *S = (double *)calloc((size_t)dk * dv, sizeof(double));
        double *pred = (double *)malloc(sizeof(double) * dv);
        if (S_in) memcpy(S, S_in + (size_t)s * dk * dv, sizeof(double) * dk * dv);
        for (int t = 0; t < N; ++t) {
            const double a = alpha ? alpha[(size_t)s * N + t] : 1.0;
            const double b = beta[(size_t)s * N + t];
            const double *kt = k + (size_t)t * dk;
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < dk; ++f) acc += S[(size_t)f * dv + c] * kt[f];
                pred[c] = a * acc;
            }
            for (int f = 0; f < dk; ++f)
                for (int c = 0; c < dv; ++c)
                    S[(size_t)f * dv + c] = a * S[(size_t)f * dv + c] + b * kt[f] * (v[(size_t)t * dv + c] - pred[c]);
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int f = 0; f < dk; ++f) acc += q[(size_t)t * dk + f] * S[(size_t)f * dv + c];
                O[((size_t)s * N + t) * dv + c] = acc;
            }
        }
        if (S_out) memcpy(S_out + (size_t)s * dk * dv, S, sizeof(double) * dk * dv);
        free(S); free(pred);
    }
}
