/*
 * Sanitizer driver for the fp64 oracle (test infrastructure): built together
 * with oracle/la_oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer
 * by tests/test_sanitizers_cpu.py, it calls every oracle function on small
 * seeded shapes (ragged chunks, one token, every feature map, with and without
 * starting states) and checks two agreements the definitions fix, so that a
 * run both exercises every loop bound and means something.  Exit status 0:
 * no sanitizer report and every agreement holds.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void ora_set_map(int param, long long pos0);
void ora_set_num_threads(int n);
int ora_feature_dim(int kind, int dk, int m);
void ora_phi(int kind, int n, int d, const double *X, int m, const double *W, double *out);
void ora_state_read(int n, int dp, int dv, const double *phiQ, const double *S, const double *z, double *num,
                    double *den);
void ora_noncausal(int BH, int N, int dk, int dv, int kind, int m, const double *W, const double *Q, const double *K,
                   const double *V, double *O, double *S_out, double *z_out);
void ora_causal_recurrent(int BH, int N, int dk, int dv, int kind, int m, const double *W, const double *Q,
                          const double *K, const double *V, const double *S_in, const double *z_in, double *O,
                          double *S_out, double *z_out);
void ora_quadratic(int BH, int N, int dk, int dv, int kind, int m, const double *W, const double *Q, const double *K,
                   const double *V, const double *S_in, const double *z_in, int causal, double *O);
void ora_causal_chunked(int BH, int N, int dk, int dv, int kind, int m, const double *W, const double *Q,
                        const double *K, const double *V, const double *S_in, const double *z_in, int C, double *O,
                        double *S_out, double *z_out);
void ora_decode_step(int BH, int dk, int dv, int kind, int m, const double *W, const double *q, const double *k,
                     const double *v, double *S, double *z, double *o);
void ora_retention_recurrent(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                             const double *gamma, const double *Q, const double *K, const double *V,
                             const double *S_in, double *O, double *S_out);
void ora_retention_parallel(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                            const double *gamma, const double *Q, const double *K, const double *V,
                            const double *S_in, double *O);
void ora_retention_chunked(int BH, int H, int N, int dk, int dv, int kind, int m, const double *W,
                           const double *gamma, const double *Q, const double *K, const double *V,
                           const double *S_in, int C, double *O, double *S_out);
void ora_retention_decode_step(int BH, int H, int dk, int dv, int kind, int m, const double *W, const double *gamma,
                               const double *q, const double *k, const double *v, double *S, double *o);
void ora_causal_backward(int BH, int N, int dk, int dv, int kind, int m, const double *W, const double *Q,
                         const double *K, const double *V, const double *S_in, const double *z_in, const double *dO,
                         const double *dS_out, const double *dz_out, double *dQ, double *dK, double *dV,
                         double *dS_in, double *dz_in);
void ora_gla_recurrent(int BH, int N, int dk, int dv, const double *Q, const double *K, const double *V,
                       const double *A, const double *S_in, double *O, double *S_out);
void ora_delta_recurrent(int BH, int N, int dk, int dv, const double *Q, const double *K, const double *V,
                         const double *alpha, const double *beta, const double *S_in, double *O, double *S_out);

static unsigned long long rng_state = 88172645463325252ULL;
static double urand(void) { /* xorshift64, uniform in [0, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}
static double *arr(size_t n, double lo, double hi) {
    double *p = (double *)malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * urand();
    return p;
}
static double maxdiff(const double *a, const double *b, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) {
        double d = fabs(a[i] - b[i]);
        if (!(d <= m)) m = d; /* NaN propagates */
    }
    return m;
}

static int failures = 0;
static void expect(int ok, const char *what) {
    if (!ok) {
        fprintf(stderr, "mismatch: %s\n", what);
        ++failures;
    }
}

/* kinds: 0 ELU+1, 1 FAVOR+, 2 identity, 3 DPFP, 4 cos/sin, 5 cosFormer */
static void run_normalised(int kind, int N, int dk, int dv, int m, int param) {
    const int BH = 3;
    ora_set_map(param, 5);
    int dp = ora_feature_dim(kind, dk, m);
    double *W = arr((size_t)(m ? m : 1) * dk, -0.5, 0.5);
    double lo = kind == 0 ? -1.0 : 0.0; /* positive sums for the signed maps: inputs >= 0 */
    double *Q = arr((size_t)BH * N * dk, lo, 1.0), *K = arr((size_t)BH * N * dk, lo, 1.0);
    double *V = arr((size_t)BH * N * dv, -1.0, 1.0);
    double *Si = arr((size_t)BH * dp * dv, 0.0, 1.0), *zi = arr((size_t)BH * dp, 1.0, 2.0);
    double *O1 = arr((size_t)BH * N * dv, 0, 0), *O2 = arr((size_t)BH * N * dv, 0, 0), *O3 = arr((size_t)BH * N * dv, 0, 0);
    double *S1 = arr((size_t)BH * dp * dv, 0, 0), *z1 = arr((size_t)BH * dp, 0, 0);
    double *S2 = arr((size_t)BH * dp * dv, 0, 0), *z2 = arr((size_t)BH * dp, 0, 0);
    ora_noncausal(BH, N, dk, dv, kind, m, W, Q, K, V, O1, S1, z1);
    ora_quadratic(BH, N, dk, dv, kind, m, W, Q, K, V, NULL, NULL, 0, O2);
    expect(maxdiff(O1, O2, (size_t)BH * N * dv) < 1e-9, "noncausal vs pairwise");
    ora_causal_recurrent(BH, N, dk, dv, kind, m, W, Q, K, V, Si, zi, O1, S1, z1);
    ora_quadratic(BH, N, dk, dv, kind, m, W, Q, K, V, Si, zi, 1, O2);
    expect(maxdiff(O1, O2, (size_t)BH * N * dv) < 1e-9, "recurrent vs pairwise");
    for (int C = 1; C <= N + 1; C += (C < 4 ? 1 : 5)) {
        ora_causal_chunked(BH, N, dk, dv, kind, m, W, Q, K, V, Si, zi, C, O3, S2, z2);
        expect(maxdiff(O1, O3, (size_t)BH * N * dv) < 1e-9, "chunked vs recurrent");
        expect(maxdiff(S1, S2, (size_t)BH * dp * dv) < 1e-9, "chunked state");
    }
    /* decode: step from S_in over the tokens */
    double *q1 = arr((size_t)BH * dk, 0, 0), *k1 = arr((size_t)BH * dk, 0, 0), *v1 = arr((size_t)BH * dv, 0, 0);
    double *o1 = arr((size_t)BH * dv, 0, 0);
    memcpy(S2, Si, sizeof(double) * BH * dp * dv);
    memcpy(z2, zi, sizeof(double) * BH * dp);
    for (int t = 0; t < N; ++t) {
        ora_set_map(param, 5 + t);
        for (int s = 0; s < BH; ++s) {
            memcpy(q1 + s * dk, Q + ((size_t)s * N + t) * dk, sizeof(double) * dk);
            memcpy(k1 + s * dk, K + ((size_t)s * N + t) * dk, sizeof(double) * dk);
            memcpy(v1 + s * dv, V + ((size_t)s * N + t) * dv, sizeof(double) * dv);
        }
        ora_decode_step(BH, dk, dv, kind, m, W, q1, k1, v1, S2, z2, o1);
        for (int s = 0; s < BH; ++s)
            expect(maxdiff(o1 + s * dv, O1 + ((size_t)s * N + t) * dv, dv) < 1e-9, "decode vs recurrent");
    }
    ora_set_map(param, 5);
    if (kind == 0 || kind == 1) {
        double *dO = arr((size_t)BH * N * dv, -1, 1), *dS = arr((size_t)BH * dp * dv, -1, 1), *dz = arr((size_t)BH * dp, -1, 1);
        double *dQ = arr((size_t)BH * N * dk, 0, 0), *dK = arr((size_t)BH * N * dk, 0, 0), *dV = arr((size_t)BH * N * dv, 0, 0);
        double *dSi = arr((size_t)BH * dp * dv, 0, 0), *dzi = arr((size_t)BH * dp, 0, 0);
        ora_causal_backward(BH, N, dk, dv, kind, m, W, Q, K, V, Si, zi, dO, dS, dz, dQ, dK, dV, dSi, dzi);
        ora_causal_backward(BH, N, dk, dv, kind, m, W, Q, K, V, NULL, NULL, dO, NULL, NULL, dQ, dK, dV, NULL, NULL);
        free(dO); free(dS); free(dz); free(dQ); free(dK); free(dV); free(dSi); free(dzi);
    }
    double *ph = arr((size_t)N * dp, 0, 0), *num = arr((size_t)N * dv, 0, 0), *den = arr((size_t)N, 0, 0);
    ora_phi(kind, N, dk, Q, m, W, ph);
    ora_state_read(N, dp, dv, ph, Si, zi, num, den);
    free(ph); free(num); free(den);
    free(W); free(Q); free(K); free(V); free(Si); free(zi); free(O1); free(O2); free(O3);
    free(S1); free(z1); free(S2); free(z2); free(q1); free(k1); free(v1); free(o1);
}

static void run_retention(int kind, int N, int dk, int dv, int m) {
    const int H = 2, BH = 4;
    int dp = ora_feature_dim(kind, dk, m);
    double *W = arr((size_t)(m ? m : 1) * dk, -0.5, 0.5);
    double gamma[2] = {0.9, 0.5};
    double *Q = arr((size_t)BH * N * dk, -1, 1), *K = arr((size_t)BH * N * dk, -1, 1), *V = arr((size_t)BH * N * dv, -1, 1);
    double *Si = arr((size_t)BH * dp * dv, -1, 1);
    double *O1 = arr((size_t)BH * N * dv, 0, 0), *O2 = arr((size_t)BH * N * dv, 0, 0);
    double *S1 = arr((size_t)BH * dp * dv, 0, 0), *S2 = arr((size_t)BH * dp * dv, 0, 0);
    ora_retention_recurrent(BH, H, N, dk, dv, kind, m, W, gamma, Q, K, V, Si, O1, S1);
    ora_retention_parallel(BH, H, N, dk, dv, kind, m, W, gamma, Q, K, V, Si, O2);
    expect(maxdiff(O1, O2, (size_t)BH * N * dv) < 1e-9, "retention parallel vs recurrent");
    for (int C = 1; C <= N + 1; C += 3) {
        ora_retention_chunked(BH, H, N, dk, dv, kind, m, W, gamma, Q, K, V, Si, C, O2, S2);
        expect(maxdiff(O1, O2, (size_t)BH * N * dv) < 1e-9, "retention chunked");
    }
    double *q1 = arr((size_t)BH * dk, -1, 1), *k1 = arr((size_t)BH * dk, -1, 1), *v1 = arr((size_t)BH * dv, -1, 1);
    double *o1 = arr((size_t)BH * dv, 0, 0);
    ora_retention_decode_step(BH, H, dk, dv, kind, m, W, gamma, q1, k1, v1, S1, o1);
    free(W); free(Q); free(K); free(V); free(Si); free(O1); free(O2); free(S1); free(S2);
    free(q1); free(k1); free(v1); free(o1);
}

static void run_gated(int N, int dk, int dv) {
    const int BH = 2;
    double *Q = arr((size_t)BH * N * dk, -1, 1), *K = arr((size_t)BH * N * dk, -1, 1), *V = arr((size_t)BH * N * dv, -1, 1);
    double *A = arr((size_t)BH * N * dk, 0, 1), *al = arr((size_t)BH * N, 0.5, 1), *be = arr((size_t)BH * N, 0, 1);
    double *Si = arr((size_t)BH * dk * dv, -1, 1);
    double *O = arr((size_t)BH * N * dv, 0, 0), *S = arr((size_t)BH * dk * dv, 0, 0);
    ora_gla_recurrent(BH, N, dk, dv, Q, K, V, A, Si, O, S);
    ora_gla_recurrent(BH, N, dk, dv, Q, K, V, A, NULL, O, NULL);
    ora_delta_recurrent(BH, N, dk, dv, Q, K, V, al, be, Si, O, S);
    ora_delta_recurrent(BH, N, dk, dv, Q, K, V, NULL, be, NULL, O, NULL);
    free(Q); free(K); free(V); free(A); free(al); free(be); free(Si); free(O); free(S);
}

int main(void) {
    ora_set_num_threads(2);
    int Ns[] = {1, 2, 7, 13};
    for (int i = 0; i < 4; ++i) {
        run_normalised(0, Ns[i], 5, 3, 0, 0);  /* ELU+1 */
        run_normalised(1, Ns[i], 4, 3, 6, 0);  /* FAVOR+ */
        run_normalised(3, Ns[i], 3, 2, 0, 2);  /* DPFP, two shifts */
        run_normalised(4, Ns[i], 3, 2, 5, 0);  /* cos/sin */
        run_normalised(5, Ns[i], 4, 3, 0, 9);  /* cosFormer */
        run_retention(2, Ns[i], 4, 3, 0);
        run_retention(0, Ns[i], 3, 2, 0);
        run_retention(1, Ns[i], 3, 2, 4);
        run_gated(Ns[i], 4, 3);
    }
    if (failures) {
        fprintf(stderr, "%d agreement(s) failed\n", failures);
        return 1;
    }
    printf("oracle driver: all agreements hold\n");
    return 0;
}
