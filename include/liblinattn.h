/*
 * liblinattn -- causal kernelized linear attention on AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h, all slices independent):
 *
 *   phi      feature map R^{d_k} -> R^{d'} with positive outputs:
 *            ELU+1:  phi(x)_f = elu(x_f) + 1  (x_f + 1 for x_f > 0, else exp(x_f));  d' = d_k
 *            FAVOR+: phi(x)_r = exp(w_r . x - |x|^2 / 2) / sqrt(m), r = 1..m;         d' = m
 *            ("Linear Attention" (aiwiki.ai), feature-map table; "Story of Attention
 *            Part 5", sections 1a and 1b.)
 *   causal   S_i = S_{i-1} + phi(k_i) v_i^T,  z_i = z_{i-1} + phi(k_i),
 *            out_i = phi(q_i)^T S_i / (phi(q_i)^T z_i)          (update, then read)
 *            ("Linear Attention", causal running sums; "Story of Attention Part 5", 1a.)
 *   non-causal  out_i = phi(q_i)^T S / (phi(q_i)^T z) with S, z summed over all tokens
 *            ("Story of Attention Part 5", 1a, matrix form.)
 *
 * Tensors (caller-owned device memory, row-major, innermost dimension last):
 *   Q, K      [B, H, N, d_k]      dtype LA_F32 (float) or LA_BF16 (uint16 bf16 bits)
 *   V, O      [B, H, N, d_v]      same dtype as Q
 *   S         [B, H, d', d_v]     float32, feature-major: S[b][h][f][j]
 *   z         [B, H, d']          float32
 *   W         [m, d_k]            float32, FAVOR+ projection rows, shared by all (b, h)
 * Every pointer must be 16-byte aligned.  The library never allocates, frees or
 * synchronises: all work is enqueued on `stream` (a hipStream_t passed as void*,
 * NULL = the legacy default stream) and the call returns once it is enqueued.
 * Results are valid after the caller synchronises that stream.  Faults during
 * execution surface at that synchronisation, not as a return value.
 *
 * Validation happens on the host before anything is enqueued: on any non-zero
 * la_status nothing has been launched and no buffer was touched.  No C++
 * exception crosses this interface.  The library holds no mutable global state;
 * calls on different streams may run concurrently when their buffers do not
 * overlap.  Q, K, V, O must not overlap each other or the state buffers.
 */
#ifndef LIBLINATTN_H
#define LIBLINATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_ABI_VERSION 6

typedef enum {
    LA_OK = 0,
    LA_ERR_NULL = 1,        /* a required pointer is NULL, or S/z pointers not paired     */
    LA_ERR_SHAPE = 2,       /* B,H,N < 1; d_k, d_v outside [1,128]; m outside [1,256];
                               decode with N != 1; sizes overflowing 2^31 elements/slice */
    LA_ERR_DTYPE = 3,       /* dtype not LA_F32 / LA_BF16                                */
    LA_ERR_UNSUPPORTED = 4, /* phi kind unknown; chunk not in {16, 32, 64, 128}           */
    LA_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned                          */
    LA_ERR_WORKSPACE = 6,   /* ws NULL or ws_bytes below la_workspace_bytes()            */
    LA_ERR_DEVICE = 7,      /* the HIP runtime refused a launch                          */
    LA_ERR_SCRATCH = 8      /* la_forward_causal_chunked_noalloc: the problem needs more
                               scratch than LA_NOALLOC_SCRATCH_BYTES                    */
} la_status;

typedef enum { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

/*
 * Feature maps (d' = feature dimension):
 *   LA_PHI_ELU1       elu(x) + 1 per coordinate; d' = d_k
 *   LA_PHI_FAVOR      exp(w_r . x - |x|^2 / 2) / sqrt(m), W [m, d_k]; d' = m
 *   LA_PHI_IDENTITY   raw x (retention and the gated recurrences only); d' = d_k
 *   LA_PHI_DPFP       r = ReLU([x, -x]); for shift i = 1..nu the block r_j r_{(j+i) mod 2d_k},
 *                     j = 0..2d_k-1 ("Linear Attention", feature-map table); nu = map_param;
 *                     d' = 2 d_k nu
 *   LA_PHI_TRIG       [cos(W x); sin(W x)], W [m, d_k] (same table); d' = 2m
 *   LA_PHI_COSFORMER  [ReLU(x) cos(pi p / 2M); ReLU(x) sin(pi p / 2M)] for the token at
 *                     position p = pos0 + (index within the call), M = map_param ("Story of
 *                     Attention Part 5", section 3); d' = 2 d_k
 * d' <= 256 for every map.  With bf16 storage, d_k = d_v = 64 and 64-token chunks,
 * one-shift DPFP, cosFormer and TRIG with m = 64 run on the matrix cores; the
 * other shapes of these maps run on the fp32-arithmetic kernels.
 */
typedef enum {
    LA_PHI_ELU1 = 0,
    LA_PHI_FAVOR = 1,
    LA_PHI_IDENTITY = 2,
    LA_PHI_DPFP = 3,
    LA_PHI_TRIG = 4,
    LA_PHI_COSFORMER = 5
} la_phi_kind;

typedef struct {
    int B, H, N;        /* batch, heads, tokens (N = 1 for la_decode_step)                   */
    int d_k, d_v;       /* key/query and value widths, each in [1, 128]                     */
    la_dtype dtype;     /* storage type of Q, K, V and O; S and z are always float32        */
    la_phi_kind phi;    /* feature map                                                      */
    int m;              /* FAVOR+: random features in [1, 256]; TRIG: in [1, 128]; else 0    */
    const float *W;     /* FAVOR+ / TRIG: device pointer to W [m, d_k] float32; else NULL     */
    int map_param;      /* DPFP: nu >= 1 (2 d_k nu <= 256); cosFormer: M >= 1; else 0         */
    long long pos0;     /* cosFormer: position of the call's first token (>= 0); else ignored */
} la_problem;

/* ABI version of the loaded library (LA_ABI_VERSION of the build). */
int la_abi_version(void);

/* Static text for a status code (never NULL). */
const char *la_status_string(la_status s);

/* Feature dimension d' of a problem: d_k for ELU+1, m for FAVOR+ (0 if p is NULL). */
int la_feature_dim(const la_problem *p);

/*
 * Device workspace (bytes) that la_forward_causal_chunked(p, chunk, ...) and
 * la_forward_noncausal(p, ...) need; 0 means ws may be NULL.  The value depends
 * only on the problem shape and chunk.  Returns 0 for an invalid problem.
 * Fill a workspace with zeros before the first call that uses it; every call
 * leaves it ready for the next one (whatever the shape).  Its first 256 bytes
 * hold the hand-off state of the single-pass causal path (launch counter,
 * done count, error word): keep them between calls, and give calls that may
 * run at the same time (on any streams) workspaces of their own.  Every other
 * call that takes a workspace (non-causal forward, backward, chunkwise GLA
 * and delta rule) leaves those 256 bytes untouched, so one buffer of the
 * largest size asked may serve all of them in turn on one stream.
 */
size_t la_workspace_bytes(const la_problem *p, int chunk);

/*
 * Error word of a workspace (its first 256 bytes, see la_workspace_bytes):
 * enqueues on `stream` a copy of the word into *err (caller-owned device
 * memory, 4-byte aligned) and, when clear != 0, resets it to 0.  The word is
 * 0 until a single-pass causal launch on this workspace had a hand-off wait
 * expire (each wait is bounded at about 10 s); it then reads 1 and stays 1
 * until cleared, and the outputs of the launch that set it hold NaN where
 * the lost hand-off mattered.  ws_bytes must be at least 256.
 * Errors: LA_ERR_NULL (ws or err NULL), LA_ERR_ALIGN (ws not 16-byte or err
 * not 4-byte aligned), LA_ERR_WORKSPACE (ws_bytes < 256), LA_ERR_DEVICE.
 */
la_status la_workspace_error(void *ws, size_t ws_bytes, unsigned int *err, int clear, void *stream);

/*
 * Non-causal forward ("Story of Attention Part 5", 1a, matrix form):
 *   S = phi(K)^T V,  z = phi(K)^T 1,  O = (phi(Q) S) / (phi(Q) z)  row-wise.
 * S_out/z_out (both or neither; may be NULL) receive S and z.
 * ws: caller-provided device scratch of at least la_workspace_bytes(p, 64)
 * bytes (its first 256 bytes are left untouched).
 */
la_status la_forward_noncausal(const la_problem *p, const void *Q, const void *K, const void *V,
                               void *O, float *S_out, float *z_out, void *ws, size_t ws_bytes,
                               void *stream);

/*
 * Causal forward in the chunkwise hybrid ("Linear Attention", chunkwise parallel
 * form; "Story of Attention Part 5", section 6 blockwise split, with decay 1 and
 * the normaliser of 1a): tokens are cut into chunks of `chunk` tokens; inside a
 * chunk the masked pairwise form phi(Q_c) phi(K_c)^T (j <= i) is applied to V_c,
 * the state carried from earlier chunks is read as phi(Q_c) S, phi(Q_c) z, and
 * the state then absorbs phi(K_c)^T V_c, phi(K_c)^T 1.
 *   chunk        in {16, 32, 64, 128}; it changes speed, never the result
 *                beyond floating-point rounding.  N need not be a multiple.
 *                The maps that run on the matrix cores at 64-token chunks only
 *                (FAVOR+, DPFP, TRIG, cosFormer with bf16 storage and d_k = d_v
 *                = 64) run a 128-token request on that 64-token tiling.
 *   S_in, z_in   initial state (both NULL = zero state), [B,H,d',d_v] / [B,H,d'].
 *   S_out, z_out final state after token N (both NULL = not exported).  May be
 *                the same buffers as S_in, z_in (updated in place).
 *   ws           device scratch of at least la_workspace_bytes(p, chunk) bytes
 *                (NULL allowed when that is 0), zero-filled before its first
 *                use and otherwise as the previous call left it.
 * With the bf16 matrix-core kernels and more than one segment per slice the
 * call is a single launch: each workgroup sums its segment, hands the sums to
 * the later segments of its slice through ws and runs its chunks from the
 * prefix it receives.  Each hand-off wait is bounded (about 10 s); should one
 * ever expire, the outputs that depend on it are NaN instead of a hung device.
 */
la_status la_forward_causal_chunked(const la_problem *p, int chunk,
                                    const void *Q, const void *K, const void *V, void *O,
                                    const float *S_in, const float *z_in,
                                    float *S_out, float *z_out,
                                    void *ws, size_t ws_bytes, void *stream);

/*
 * la_forward_causal_chunked for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same computation and kernels, with the workspace taken
 * from a fixed device array inside the library instead of the caller's ws.
 *   Arguments and results as la_forward_causal_chunked, without ws/ws_bytes.
 *   The array is LA_NOALLOC_SCRATCH_BYTES (32 MiB) on every device the library
 *   runs on, held until the process ends; a problem whose
 *   la_workspace_bytes(p, chunk) exceeds it returns LA_ERR_SCRATCH and
 *   launches nothing.  The call never allocates or frees memory.  Its first
 *   call on a device looks up that device's array and enqueues one zero fill
 *   of it on `stream` ahead of its own kernels; every call then leaves the
 *   array ready for the next.  All calls on one device share its array:
 *   calls that may run at the same time on one device (on different streams)
 *   race on it and must be ordered by the caller.  The hand-off error word
 *   of the array is not exposed.
 */
#define LA_NOALLOC_SCRATCH_BYTES (32u << 20)

la_status la_forward_causal_chunked_noalloc(const la_problem *p, int chunk,
                                            const void *Q, const void *K, const void *V, void *O,
                                            const float *S_in, const float *z_in,
                                            float *S_out, float *z_out, void *stream);

/*
 * Per-kernel timing hook for profiling and benchmarking.  A causal call
 * enqueues up to three kernels, each in its own slot:
 *   LA_KSLOT_STATE  per-segment sums phi(K)^T V, phi(K)^T 1 (only on the
 *                   fp32 path when the sequence is split into segments),
 *   LA_KSLOT_SCAN   exclusive prefix of those sums over segments (same case),
 *   LA_KSLOT_CHUNK  the kernel that writes O (always; on the single-pass
 *                   path the one kernel of the call).
 * For every slot whose kernel is enqueued, the launch of that kernel records
 * start[slot] when it begins and stop[slot] when it ends (hipExtLaunchKernel),
 * so the pair brackets exactly that kernel.  Entries may be NULL (not
 * recorded).  The events are created, owned and queried by the caller
 * (hipEvent_t passed as void*).  launched[slot] is set to 1 for each kernel
 * enqueued, 0 otherwise.
 */
enum { LA_KSLOT_STATE = 0, LA_KSLOT_SCAN = 1, LA_KSLOT_CHUNK = 2, LA_KSLOTS = 3 };

typedef struct {
    void *start[LA_KSLOTS];
    void *stop[LA_KSLOTS];
    int launched[LA_KSLOTS];
} la_kernel_events;

/*
 * la_forward_causal_chunked with the timing hook above; identical results.
 * ev may be NULL (then this is exactly la_forward_causal_chunked).
 */
la_status la_forward_causal_chunked_timed(const la_problem *p, int chunk,
                                          const void *Q, const void *K, const void *V, void *O,
                                          const float *S_in, const float *z_in,
                                          float *S_out, float *z_out,
                                          void *ws, size_t ws_bytes, void *stream,
                                          la_kernel_events *ev);

/*
 * One recurrent decode step for every (b, h) ("Linear Attention": constant work
 * and memory per generated token; "Story of Attention Part 5", 1a recurrence):
 *   S += phi(k) v^T,  z += phi(k),  o = (phi(q)^T S) / (phi(q)^T z).
 * p->N must be 1.  q, k: [B, H, 1, d_k]; v, o: [B, H, 1, d_v] (dtype p->dtype).
 * S [B,H,d',d_v] and z [B,H,d'] (float32) are read and overwritten in place.
 */
la_status la_decode_step(const la_problem *p, const void *q, const void *k, const void *v,
                         void *o, float *S, float *z, void *stream);

/*
 * Retention: decayed, unnormalised linear attention ("Story of Attention
 * Part 5", section 4 RetNet and section 6 Lightning Attention), per head h
 * with decay lambda = gamma[h]:
 *   recurrent   S_n = lambda S_{n-1} + phi(k_n) v_n^T,  o_n = phi(q_n)^T S_n,
 *   parallel    O = (phi(Q) phi(K)^T (.) D) V,  D_ij = lambda^(i-j) for i >= j,
 *   blockwise   O_i = (phi(Q_i) phi(K_i)^T (.) M) V_i + Lambda phi(Q_i) S_{i-1},
 *               S_i = lambda^B S_{i-1} + (lambda^B Lambda^{-1} phi(K_i))^T V_i,
 * the form this call runs (blocks of `chunk` tokens).  No normaliser: there
 * is no z and no division.
 *   p->phi       LA_PHI_IDENTITY (RetNet's raw q and k: the bf16 matrix-core
 *                kernels for d_k = d_v in {64, 128}, chunk in {64, 128}), or
 *                LA_PHI_ELU1 / LA_PHI_FAVOR (fp32-arithmetic kernels).
 *   gamma        device float [H], decay of each head, in (0, 1]; 4-byte aligned.
 *   S_in, S_out  [B,H,d',d_v] fp32 initial / final state (NULL = zero / not
 *                exported); S_out may be S_in.
 *   ws           as for la_forward_causal_chunked (la_workspace_bytes covers
 *                retention; zero-filled before its first use).
 *   ev           per-kernel timing hook as in la_forward_causal_chunked_timed,
 *                or NULL.
 */
la_status la_forward_retention_chunked(const la_problem *p, const float *gamma, int chunk,
                                       const void *Q, const void *K, const void *V, void *O,
                                       const float *S_in, float *S_out,
                                       void *ws, size_t ws_bytes, void *stream,
                                       la_kernel_events *ev);

/*
 * One retention decode step for every (b, h) ("Story of Attention Part 5",
 * section 4 recurrent form): S = gamma[h] S + phi(k) v^T, o = phi(q)^T S.
 * p->N must be 1; q, k [B,H,1,d_k], v, o [B,H,1,d_v]; S [B,H,d',d_v] fp32 in
 * place.  gamma as for la_forward_retention_chunked.
 */
la_status la_retention_decode_step(const la_problem *p, const float *gamma, const void *q, const void *k,
                                   const void *v, void *o, float *S, void *stream);

/*
 * Backward of the causal form (la_forward_causal_chunked with the ELU+1 or
 * FAVOR+ map).  The pages use the parallel mode for training ("Linear
 * Attention: Removing the Softmax Buys Associativity", the two computation
 * modes) but print no gradients; these are the reverse-mode derivatives of the
 * causal recurrence.  With psi_i = phi(q_i), kappa_j = phi(k_j), den_i =
 * psi_i^T z_i and o_i the forward output:
 *   g_i = dO_i / den_i,  h_i = -(dO_i . o_i) / den_i,
 *   dpsi_i   = S_i g_i + z_i h_i,
 *   dkappa_j = R_j v_j + r_j,  dv_j = R_j^T kappa_j,
 *   R_j = dS_out + sum_{i >= j} psi_i g_i^T,  r_j = dz_out + sum_{i >= j} psi_i h_i,
 *   dS_in = R_1, dz_in = r_1,
 * and dQ, dK are dpsi, dkappa through the map's Jacobian (ELU+1: 1 for x > 0,
 * exp(x) otherwise; FAVOR+: d phi_r / dx = phi_r (w_r - x); W gets no
 * gradient).  The forward is recomputed inside the call; O is not an input.
 *   p            as for the forward; LA_PHI_IDENTITY is refused.  Supported
 *                while d' * (d_v + 1) <= 16640 (d' = 128 with d_v <= 128, or
 *                d' = 256 with d_v <= 64); larger: LA_ERR_UNSUPPORTED.
 *   chunk        16, 32, 64 or 128: tokens per chunk of the chunked form.  The
 *                gradients do not depend on it.  ELU+1 (bf16 or fp32) with
 *                d_k = d_v = 64 and 64-token chunks, or d_k = d_v = 128 and
 *                chunks of 32, 64 or 128 tokens (run on 32-token tiles), runs
 *                on matrix instructions with fp32-class products (fp32
 *                instructions for fp32 storage; for bf16 storage bf16
 *                instructions on operands split into hi and lo parts, about
 *                2^-16 relative); everything else runs on
 *                fp32-arithmetic kernels that tile at most 16 tokens whatever
 *                is asked.
 *   Q, K, V      forward inputs; dO [B,H,N,d_v] the gradient of the loss with
 *                respect to O (all of dtype p->dtype).
 *   S_in, z_in   the forward's starting state, or both NULL (zero).
 *   dS_out, dz_out  gradient with respect to the forward's final state
 *                [B,H,d',d_v], [B,H,d'] fp32, or both NULL (zero).
 *   dQ, dK, dV   outputs, [B,H,N,d_k] / [B,H,N,d_v] of dtype p->dtype
 *                (fp32 arithmetic, rounded once at the store).
 *   dS_in, dz_in gradient with respect to S_in, z_in, or both NULL (not
 *                written).
 *   ws           device workspace of at least la_backward_workspace_bytes()
 *                bytes (no initial contents required; its first 256 bytes
 *                are left untouched, so a forward's workspace may be reused).
 *   ev           per-kernel timing hook (slots below), or NULL.
 * Six kernels are enqueued: the forward's per-segment sums and their prefix
 * scan, then the forward-direction pass (recomputes the outputs, writes dQ and
 * the per-token g, h to ws), the per-segment sums of psi g^T, psi h (no
 * timing slot), their reverse scan (writes dS_in, dz_in), and the
 * reverse-direction pass (dK, dV).  On the matrix-instruction kernels three:
 * the forward's per-segment sums, the forward-direction pass (it adds the
 * earlier segments' sums to S_in, z_in itself and also forms the per-segment
 * sums of psi g^T, psi h) and the reverse-direction pass (it adds the later
 * segments' sums to dS_out, dz_out itself; its first segment writes dS_in,
 * dz_in); LA_BSLOT_FWD_SCAN and LA_BSLOT_RSCAN are then not launched.
 * Outputs must not overlap inputs or each other.
 */
enum { LA_BSLOT_FWD_SUMS = 0, LA_BSLOT_FWD_SCAN = 1, LA_BSLOT_DQ = 2, LA_BSLOT_RSCAN = 3, LA_BSLOT_DKV = 4,
       LA_BSLOTS = 5 };

typedef struct {
    void *start[LA_BSLOTS];
    void *stop[LA_BSLOTS];
    int launched[LA_BSLOTS];
} la_backward_events;

/* Workspace bytes for la_backward_causal_chunked; 0 for an invalid or unsupported problem. */
size_t la_backward_workspace_bytes(const la_problem *p, int chunk);

la_status la_backward_causal_chunked(const la_problem *p, int chunk,
                                     const void *Q, const void *K, const void *V, const void *dO,
                                     const float *S_in, const float *z_in,
                                     const float *dS_out, const float *dz_out,
                                     void *dQ, void *dK, void *dV,
                                     float *dS_in, float *dz_in,
                                     void *ws, size_t ws_bytes, void *stream,
                                     la_backward_events *ev);

/*
 * Gated and delta-rule states, run as the recurrence token by token ("Linear
 * Attention" (aiwiki.ai), GLA's gated recurrence and the delta-rule update;
 * "Story of Attention Part 5", section 7 Gated DeltaNet).  Raw q and k (p->phi
 * must be LA_PHI_IDENTITY), no normaliser, state S [B,H,d_k,d_v] fp32
 * feature-major (the pages' S k, the value the state returns for key k, is
 * S^T k here), output read after the update: o_t = S_t^T q_t.
 *   GLA:   S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, a gate per key channel,
 *          alpha [B,H,N,d_k] fp32.
 *   delta: p_t = alpha_t S_{t-1}^T k_t,  S_t = alpha_t S_{t-1} + beta_t k_t (v_t - p_t)^T,
 *          beta [B,H,N] fp32 (write strength), alpha [B,H,N] fp32 scalar
 *          forget gate or NULL (alpha = 1: the plain delta rule).
 * Q, K [B,H,N,d_k], V, O [B,H,N,d_v] of dtype p->dtype; the state stays fp32
 * and all arithmetic is fp32.  The delta rule, and GLA with d_k > 64 or
 * N < 64, run token by token; GLA with d_k <= 64 and N >= 64 runs in
 * chunkwise form (64-token chunks; the same sums up to rounding order; GLA
 * gates are expected in [0, 1], a gate of 0 is taken as 2^-115).  S_in NULL
 * = zero; S_out (may be S_in, may be NULL) receives the final state.  N = 1
 * is the decode step.  Workgroups per (b, h) own value columns: no workspace.
 */
la_status la_forward_gla_recurrent(const la_problem *p, const void *Q, const void *K, const void *V,
                                   const float *alpha, const float *S_in, float *S_out, void *O, void *stream);

la_status la_forward_delta_recurrent(const la_problem *p, const void *Q, const void *K, const void *V,
                                     const float *alpha, const float *beta, const float *S_in, float *S_out,
                                     void *O, void *stream);

/*
 * The gated delta rule above in chunkwise form (64-token chunks; the pages'
 * Gated DeltaNet, "Story of Attention Part 5", section 7, with the state
 * written as S_t = g_t S0 + sum_s (g_t / g_s) k_s u_s^T inside a chunk, g the
 * cumulative forget gates).  The write vectors of a chunk solve the unit
 * lower-triangular system (I + M) U = diag(beta) V - diag(beta g) K S0,
 * M[t][s] = beta_t (g_t / g_s) k_t . k_s for s < t, so U = Ut - W S0 with W and
 * Ut independent of the entering state.  Substituted, O = Qt S0 + P Ut with
 * Qt = diag(g) Q - P W (P the causal score matrix) and the chunk's final
 * state A S0 + B with A = g_C I - K^T diag(g_C / g) W, B = K^T diag(g_C / g) Ut:
 * the library forms Qt, A, P Ut and B of every chunk at once (first launch),
 * runs the chunks of each (b, h) slice in order per 16 value columns, one
 * product on the state per chunk (second launch), then forms the outputs of
 * every chunk at once (third launch).
 * The same sums as la_forward_delta_recurrent up to rounding order (fp32
 * arithmetic).  Arguments as there, plus:
 *   chunk  must be 64;  p->d_k must be 64 and p->d_v a multiple of 16 up to
 *          128, else LA_ERR_UNSUPPORTED (the token-by-token entry point takes
 *          every shape);
 *   ws     device workspace of at least la_delta_workspace_bytes(p, chunk)
 *          bytes (16-byte aligned; no initial contents needed; past its
 *          first 256 bytes, which are left untouched, one record per
 *          (b, h, chunk): Qt, A [64 x 64], (P Ut)^T, B^T [d_v x 64], fp32),
 *          owned by the caller; else LA_ERR_WORKSPACE;
 *   ev     optional timing hook: slot LA_KSLOT_STATE brackets the per-chunk
 *          launch, LA_KSLOT_SCAN the state chain over chunks, LA_KSLOT_CHUNK
 *          the outputs of every chunk.
 * Forget gates below 2^-80 are taken as 2^-80.  S_out may alias S_in.
 */
size_t la_delta_workspace_bytes(const la_problem *p, int chunk);

/*
 * GLA (la_forward_gla_recurrent) in chunkwise form, three launches ("Linear
 * Attention", gated linear attention; chunkwise parallel form).  With S_c
 * the state entering 64-token chunk c, O_c = QD_c S_c + P_c V_c and
 * S_{c+1} = diag(decay_c) S_c + KE_c^T V_c, where QD are the decayed
 * queries, P the masked pair scores (overflow-safe pivot split), KE the
 * decayed keys and decay the chunk's gate product per key channel.
 *   1. every chunk at once: QD, P, KE, decay, P V and KE^T V;
 *   2. the state chain, element by element over the chunks (the only serial
 *      step): S_c of every chunk, S_out;
 *   3. every chunk at once: O = QD S_c + P V.
 * Arguments as la_forward_gla_recurrent, plus: chunk must be 64 and
 * p->d_k <= 64 (else LA_ERR_UNSUPPORTED); any N >= 1; ws: device workspace
 * of at least la_gla_workspace_bytes(p, chunk) bytes (16-byte aligned, no
 * initial contents; its first 256 bytes are left untouched, then one record
 * of 64 x 64 + 2 x 64 x dvp + 64 floats per (b, h, chunk), dvp = d_v rounded
 * up to 16), else LA_ERR_WORKSPACE; ev: optional timing hook (LA_KSLOT_STATE:
 * the per-chunk products, LA_KSLOT_SCAN: the state chain, LA_KSLOT_CHUNK: the
 * outputs).  S_out may alias S_in.
 */
size_t la_gla_workspace_bytes(const la_problem *p, int chunk);

la_status la_forward_gla_chunked(const la_problem *p, int chunk, const void *Q, const void *K, const void *V,
                                 const float *alpha, const float *S_in, float *S_out, void *O, void *ws,
                                 size_t ws_bytes, void *stream, la_kernel_events *ev);

la_status la_forward_delta_chunked(const la_problem *p, int chunk, const void *Q, const void *K, const void *V,
                                   const float *alpha, const float *beta, const float *S_in, float *S_out,
                                   void *O, void *ws, size_t ws_bytes, void *stream, la_kernel_events *ev);

#ifdef __cplusplus
}
#endif

#endif /* LIBLINATTN_H */
