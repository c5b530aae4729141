// liblinattn C ABI: host-side validation and dispatch.  Everything here runs on
// the host; the arithmetic is in the kernels (la_generic.hip, la_mfma.hip,
// la_decode.hip).  No allocation, no synchronisation, no global state.
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "../../include/liblinattn.h"
#include "la_internal.h"

#define LA_API extern "C" __attribute__((visibility("default")))

namespace la {
namespace {

constexpr int kTargetWorkgroups = 1024;  // generic path: several workgroups per CU
// MFMA path: one workgroup per CU of the 256-CU part.  Every workgroup streams
// its segment chunk after chunk, so more segments only add state traffic and
// shorten the stream (measured on MI355X for d = 64 / 128 and FAVOR+).
constexpr int kMfmaWorkgroups = 256;
constexpr size_t kAlign = 256;

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

la_status check_problem(const la_problem *p) {
    if (!p) return LA_ERR_NULL;
    if (p->dtype != LA_F32 && p->dtype != LA_BF16) return LA_ERR_DTYPE;
    if (p->phi < LA_PHI_ELU1 || p->phi > LA_PHI_COSFORMER) return LA_ERR_UNSUPPORTED;
    if (p->B < 1 || p->H < 1 || p->N < 1) return LA_ERR_SHAPE;
    if (p->d_k < 1 || p->d_k > 128 || p->d_v < 1 || p->d_v > 128) return LA_ERR_SHAPE;
    if (p->phi == LA_PHI_FAVOR || p->phi == LA_PHI_TRIG) {
        if (p->m < 1 || p->m > (p->phi == LA_PHI_TRIG ? 128 : 256)) return LA_ERR_SHAPE;
        if (!p->W) return LA_ERR_NULL;
        if (!aligned16(p->W)) return LA_ERR_ALIGN;
    } else if (p->m != 0 || p->W) {
        return LA_ERR_SHAPE;
    }
    if (p->phi == LA_PHI_DPFP) {
        if (p->map_param < 1 || 2LL * p->d_k * p->map_param > 256) return LA_ERR_SHAPE;
    } else if (p->phi == LA_PHI_COSFORMER) {
        if (p->map_param < 1 || p->pos0 < 0) return LA_ERR_SHAPE;
    } else if (p->map_param != 0) {
        return LA_ERR_SHAPE;
    }
    // element counts of one slice must fit comfortably in 32-bit kernel indices
    const long long per_slice = (long long)p->N * (p->d_k > p->d_v ? p->d_k : p->d_v);
    if (per_slice > (long long)INT_MAX) return LA_ERR_SHAPE;
    if ((long long)p->B * p->H > (long long)INT_MAX / 4) return LA_ERR_SHAPE;
    return LA_OK;
}

static_assert((int)LA_PHI_ELU1 == (int)kElu1 && (int)LA_PHI_FAVOR == (int)kFavor &&
                  (int)LA_PHI_IDENTITY == (int)kIdentity && (int)LA_PHI_DPFP == (int)kDpfp &&
                  (int)LA_PHI_TRIG == (int)kTrig && (int)LA_PHI_COSFORMER == (int)kCosformer,
              "feature-map codes");

Shape make_shape(const la_problem *p) {
    Shape s;
    s.BH = p->B * p->H;
    s.N = p->N;
    s.dk = p->d_k;
    s.dv = p->d_v;
    s.phi = p->phi;  // the la_phi_kind values are the Phi values
    s.m = (p->phi == LA_PHI_FAVOR || p->phi == LA_PHI_TRIG) ? p->m : 0;
    s.W = (p->phi == LA_PHI_FAVOR || p->phi == LA_PHI_TRIG) ? p->W : nullptr;
    s.param = p->map_param;
    s.pos0 = p->phi == LA_PHI_COSFORMER ? p->pos0 : 0;
    switch (p->phi) {
        case LA_PHI_FAVOR: s.dp = p->m; break;
        case LA_PHI_DPFP: s.dp = 2 * p->d_k * p->map_param; break;
        case LA_PHI_TRIG: s.dp = 2 * p->m; break;
        case LA_PHI_COSFORMER: s.dp = 2 * p->d_k; break;
        default: s.dp = p->d_k;
    }
    s.dtype = p->dtype == LA_BF16 ? kBF16 : kF32;
    s.ret = 0;
    s.gamma = nullptr;
    s.H = p->H;
    return s;
}

bool chunk_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64 || chunk == 128; }

// Split each slice into P segments of whole chunks so that B*H*P*(columns)
// workgroups fill the device.  Depends on the shape only.
Segments plan_segments(const Shape &sh, int chunk, int columns_per_slice, int min_seg_chunks,
                       int target = kTargetWorkgroups) {
    Segments g;
    g.chunk = chunk;
    g.n_chunks = (sh.N + chunk - 1) / chunk;
    const long long units = (long long)sh.BH * columns_per_slice;
    int want = (int)((target + units - 1) / units);
    if (want < 1) want = 1;
    int max_p = (g.n_chunks + min_seg_chunks - 1) / min_seg_chunks;
    if (want > max_p) want = max_p;
    if (want < 1) want = 1;
    g.seg_chunks = (g.n_chunks + want - 1) / want;
    g.P = (g.n_chunks + g.seg_chunks - 1) / g.seg_chunks;
    return g;
}

// Workgroups per (slice, segment) on the fp32-arithmetic path: one 32-column
// value slab each on the FMA kernels; the fp32 matrix-instruction kernel
// covers every column in one workgroup.
int generic_columns(const Shape &sh) { return f32mma_supported(sh) ? 1 : (sh.dv + 31) / 32; }

// The projected and widened maps on the matrix cores (FAVOR+, DPFP, cos/sin,
// cosFormer) tile 64 tokens: at m = 256 a 128-token tile of phi(K) and
// phi(Q) alone would take 132 KiB of the 160 KiB of LDS, and the d' = 128
// maps' 128-token tiles with their raw rows about 180 KiB.  The chunkwise form
// gives the same function for every chunk length ("Linear Attention",
// chunkwise parallel form), so a 128-token request runs on the 64-token tiling
// rather than on the fp32-arithmetic kernels.
int tile_chunk(const Shape &sh, int chunk) {
    const bool tiled64 = sh.phi == kFavor || sh.phi == kDpfp || sh.phi == kTrig || sh.phi == kCosformer;
    return tiled64 && chunk == 128 && mfma_supported(sh, 64) ? 64 : chunk;
}

Segments causal_plan(const Shape &sh, int chunk_req, bool *use_mfma) {
    const int chunk = tile_chunk(sh, chunk_req);
    const bool mf = mfma_supported(sh, chunk);
    if (use_mfma) *use_mfma = mf;
    return mf ? plan_segments(sh, chunk, 1, 1, kMfmaWorkgroups) : plan_segments(sh, chunk, generic_columns(sh), 1);
}

constexpr int kNoncausalChunk = 64;

Segments noncausal_plan(const Shape &sh, bool *use_mfma) {
    const bool mf = mfma_supported(sh, kNoncausalChunk);
    if (use_mfma) *use_mfma = mf;
    return mf ? plan_segments(sh, kNoncausalChunk, 1, 1, kMfmaWorkgroups)
              : plan_segments(sh, kNoncausalChunk, generic_columns(sh), 1);
}

// Workspace: [control block][segment flags][S part][z part].
//  * control block (kCtlBytes, fixed offset for every shape): launch counter,
//    done count and error word of the single-pass mode;
//  * flags: kFlagsPerSegment words per (slice, segment);
//  * S part: P + 1 single-pass slots of d' x (d_v + 16) floats per slice (S,
//    z and padding in the matrix-core accumulator order); the separate passes
//    use P x d' x d_v of it, with the z part.
constexpr size_t kCtlBytes = 256;

struct WsLayout {
    size_t f_off, s_off, z_off, total;
};

WsLayout ws_layout(const Shape &sh, int P) {
    const size_t f_bytes = round_up(sizeof(uint32_t) * (size_t)sh.BH * P * kFlagsPerSegment, kAlign);
    const size_t s_bytes = round_up(sizeof(float) * (size_t)sh.BH * (P + 1) * sh.dp * (sh.dv + 16), kAlign);
    const size_t z_bytes = round_up(sizeof(float) * (size_t)sh.BH * P * sh.dp, kAlign);
    WsLayout w;
    w.f_off = kCtlBytes;
    w.s_off = w.f_off + f_bytes;
    w.z_off = w.s_off + s_bytes;
    w.total = w.z_off + z_bytes;
    return w;
}

// Bound of one hand-off wait of the single-pass mode: 10 s of the 100 MHz
// constant-rate clock.  A correct launch waits microseconds; the bound only
// turns a lost hand-off into NaN output instead of a hung device.
constexpr long long kSpinTicks = 1000000000LL;

// A single workgroup per slice can start from S_in and finish into S_out by
// itself (safe even when they alias).  Several segments, or several value
// slabs that would all read z_in while one of them writes z_out, go through
// the workspace: per-segment sums, a prefix scan, then the chunk loop.
bool causal_direct(const Shape &sh, const Segments &g, bool mfma) {
    return g.P == 1 && (mfma || generic_columns(sh) == 1);
}

// Single-pass mode: the LDS-resident variant when a segment's phi(K), V fit
// (d = 64, 64-token chunks, at most kResChunks chunks per segment).
int fused_mode(const Shape &sh, const Segments &g) {
    const bool res = g.seg_chunks <= kResChunks && sh.dk == 64 && sh.dv == 64 && g.chunk == 64 &&
                     (sh.phi == kElu1 || sh.phi == kIdentity);
    return res ? kModeFusedRes : kModeFused;
}

// Single pass on the matrix cores: the whole-segment kernel where a segment
// fits one 16-wave workgroup, the eight-wave FAVOR+ kernel for its shape,
// else the chunk loop.
hipError_t launch_single_pass(const FwdArgs &f, hipStream_t st, KEvents ev) {
    if (seg_supported(f.sh, f.sg)) return launch_seg(f, st, ev);
    if (f.mode == kModeFused && favor_supported(f.sh, f.sg)) return launch_favor(f, st, ev);
    return launch_mfma(f, st, ev);
}

size_t causal_ws(const Shape &sh, int chunk) {
    bool mf = false;
    Segments g = causal_plan(sh, chunk, &mf);
    return causal_direct(sh, g, mf) ? 0 : ws_layout(sh, g.P).total;
}

size_t noncausal_ws(const Shape &sh) {
    Segments g = noncausal_plan(sh, nullptr);
    return ws_layout(sh, g.P).total;
}

hipError_t launch_fwd(bool mfma, const FwdArgs &a, hipStream_t st, KEvents ev = {}) {
    return mfma ? launch_mfma(a, st, ev) : launch_generic(a, st, ev);
}

// Argument checks of a causal call (everything but the workspace).
la_status causal_validate(const la_problem *p, int chunk, const void *Q, const void *K, const void *V, const void *O,
                          const float *S_in, const float *z_in, const float *S_out, const float *z_out) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi == LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;  // the normaliser needs a positive map
    if (!chunk_ok(chunk)) return LA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O) return LA_ERR_NULL;
    if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr)) return LA_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(S_in) || !aligned16(z_in) ||
        !aligned16(S_out) || !aligned16(z_out))
        return LA_ERR_ALIGN;
    return LA_OK;
}

// Timing events of one kernel slot of a call (profiling hook); marks the slot launched.
KEvents slot_events(la_kernel_events *ev, int slot) {
    KEvents k;
    if (!ev) return k;
    ev->launched[slot] = 1;
    k.start = static_cast<hipEvent_t>(ev->start[slot]);
    k.stop = static_cast<hipEvent_t>(ev->stop[slot]);
    return k;
}

}  // namespace
}  // namespace la

using namespace la;

LA_API int la_abi_version(void) { return LA_ABI_VERSION; }

LA_API const char *la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_NULL: return "required pointer is NULL (or S/z pointers not paired)";
        case LA_ERR_SHAPE: return "shape out of range";
        case LA_ERR_DTYPE: return "unsupported dtype";
        case LA_ERR_UNSUPPORTED: return "unsupported feature map or chunk size";
        case LA_ERR_ALIGN: return "pointer not 16-byte aligned";
        case LA_ERR_WORKSPACE: return "workspace missing or too small";
        case LA_ERR_DEVICE: return "HIP launch failed";
        case LA_ERR_SCRATCH: return "problem needs more scratch than the fixed array of the allocation-free entry point";
    }
    return "unknown status";
}

LA_API int la_feature_dim(const la_problem *p) {
    if (check_problem(p) != LA_OK) return 0;
    return make_shape(p).dp;
}

LA_API size_t la_workspace_bytes(const la_problem *p, int chunk) {
    if (check_problem(p) != LA_OK || !chunk_ok(chunk)) return 0;
    Shape sh = make_shape(p);
    size_t need = 0;
    if (p->phi != LA_PHI_IDENTITY) {  // normalised causal and non-causal calls
        const size_t a = causal_ws(sh, chunk), b = noncausal_ws(sh);
        need = a > b ? a : b;
    }
    sh.ret = 1;  // retention calls plan their own segments
    const size_t r = causal_ws(sh, chunk);
    return r > need ? r : need;
}

LA_API la_status la_workspace_error(void *ws, size_t ws_bytes, unsigned int *err, int clear, void *stream) {
    if (!ws || !err) return LA_ERR_NULL;
    if (!aligned16(ws) || (reinterpret_cast<uintptr_t>(err) & 3u) != 0) return LA_ERR_ALIGN;
    if (ws_bytes < kCtlBytes) return LA_ERR_WORKSPACE;
    static_assert(sizeof(unsigned int) == sizeof(uint32_t), "error word");
    return launch_ws_error(static_cast<uint32_t *>(ws), reinterpret_cast<uint32_t *>(err), clear != 0,
                           static_cast<hipStream_t>(stream)) == hipSuccess
               ? LA_OK
               : LA_ERR_DEVICE;
}

LA_API la_status la_forward_noncausal(const la_problem *p, const void *Q, const void *K, const void *V, void *O,
                                      float *S_out, float *z_out, void *ws, size_t ws_bytes, void *stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi == LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;  // the normaliser needs a positive map
    if (!Q || !K || !V || !O) return LA_ERR_NULL;
    if ((S_out == nullptr) != (z_out == nullptr)) return LA_ERR_NULL;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(S_out) ||
        !aligned16(z_out) || !aligned16(ws))
        return LA_ERR_ALIGN;
    Shape sh = make_shape(p);
    bool mf = false;
    Segments g = noncausal_plan(sh, &mf);
    WsLayout wl = ws_layout(sh, g.P);
    if (!ws || ws_bytes < wl.total) return LA_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    float *wsS = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.s_off);
    float *wsz = reinterpret_cast<float *>(static_cast<char *>(ws) + wl.z_off);
    const size_t nS = (size_t)sh.dp * sh.dv, nz = (size_t)sh.dp;

    // 1. per-segment sums phi(K)^T V, phi(K)^T 1
    FwdArgs a{};
    a.sh = sh; a.sg = g; a.mode = kModeState;
    a.Q = Q; a.K = K; a.V = V; a.O = nullptr;
    a.st.S_dst = wsS; a.st.z_dst = wsz;
    a.st.dst_slice = g.P * nS; a.st.dst_seg = nS; a.st.zdst_slice = g.P * nz; a.st.zdst_seg = nz;
    if (launch_fwd(mf, a, hs) != hipSuccess) return LA_ERR_DEVICE;
    // 2. fixed-order total into slot 0 (and S_out)
    if (launch_scan(sh, g.P, wsS, wsz, nullptr, nullptr, S_out, z_out, true, hs) != hipSuccess) return LA_ERR_DEVICE;
    // 3. O = phi(Q) S / phi(Q) z
    FwdArgs r{};
    r.sh = sh; r.sg = g; r.mode = kModeRead;
    r.Q = Q; r.K = K; r.V = V; r.O = O;
    r.st.S_src = wsS; r.st.z_src = wsz;
    r.st.src_slice = g.P * nS; r.st.src_seg = 0; r.st.zsrc_slice = g.P * nz; r.st.zsrc_seg = 0;
    if (launch_fwd(mf, r, hs) != hipSuccess) return LA_ERR_DEVICE;
    return LA_OK;
}

LA_API la_status la_forward_causal_chunked_timed(const la_problem *p, int chunk, const void *Q, const void *K,
                                                 const void *V, void *O, const float *S_in, const float *z_in,
                                                 float *S_out, float *z_out, void *ws, size_t ws_bytes, void *stream,
                                                 la_kernel_events *ev) {
    la_status st = causal_validate(p, chunk, Q, K, V, O, S_in, z_in, S_out, z_out);
    if (st != LA_OK) return st;
    if (!aligned16(ws)) return LA_ERR_ALIGN;
    Shape sh = make_shape(p);
    bool mf = false;
    Segments g = causal_plan(sh, chunk, &mf);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)sh.dp * sh.dv, nz = (size_t)sh.dp;
    const bool direct = causal_direct(sh, g, mf);
    WsLayout wl = ws_layout(sh, g.P);
    if (!direct && (!ws || ws_bytes < wl.total)) return LA_ERR_WORKSPACE;
    if (ev)
        for (int i = 0; i < LA_KSLOTS; ++i) ev->launched[i] = 0;

    FwdArgs c{};
    c.sh = sh; c.sg = g; c.mode = kModeCausal;
    c.Q = Q; c.K = K; c.V = V; c.O = O;
    if (direct) {
        // one workgroup per slice: start from S_in, finish into S_out
        c.st.S_src = S_in; c.st.z_src = z_in;
        c.st.src_slice = nS; c.st.zsrc_slice = nz;
        c.st.S_dst = S_out; c.st.z_dst = z_out;
        c.st.dst_slice = nS; c.st.zdst_slice = nz;
        return launch_fwd(mf, c, hs, slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
    }
    char *wsb = static_cast<char *>(ws);
    float *wsS = reinterpret_cast<float *>(wsb + wl.s_off);
    float *wsz = reinterpret_cast<float *>(wsb + wl.z_off);

    if (mf) {
        // single pass on the matrix cores: every workgroup sums its segment,
        // hands the sums on through the workspace and runs its chunks
        FwdArgs f = c;
        f.mode = fused_mode(sh, g);
        f.st.S_src = S_in; f.st.z_src = z_in;
        f.st.src_slice = nS; f.st.zsrc_slice = nz;
        f.fu.ctl = reinterpret_cast<uint32_t *>(wsb);
        f.fu.flags = reinterpret_cast<uint32_t *>(wsb + wl.f_off);
        f.fu.slots = wsS;
        f.fu.spin_ticks = kSpinTicks;
        f.fu.S_out = S_out; f.fu.z_out = z_out;
        return launch_single_pass(f, hs, slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
    }

    // A. each segment's own sums phi(K)^T V, phi(K)^T 1
    FwdArgs a{};
    a.sh = sh; a.sg = g; a.mode = kModeState;
    a.Q = Q; a.K = K; a.V = V; a.O = nullptr;
    a.st.S_dst = wsS; a.st.z_dst = wsz;
    a.st.dst_slice = g.P * nS; a.st.dst_seg = nS; a.st.zdst_slice = g.P * nz; a.st.zdst_seg = nz;
    if (launch_fwd(mf, a, hs, slot_events(ev, LA_KSLOT_STATE)) != hipSuccess) return LA_ERR_DEVICE;
    // B. exclusive prefix over segments (+ S_in); final state to S_out
    if (launch_scan(sh, g.P, wsS, wsz, S_in, z_in, S_out, z_out, false, hs, slot_events(ev, LA_KSLOT_SCAN)) !=
        hipSuccess)
        return LA_ERR_DEVICE;
    // C. chunk loop of every segment from its prefix state
    c.st.S_src = wsS; c.st.z_src = wsz;
    c.st.src_slice = g.P * nS; c.st.src_seg = nS; c.st.zsrc_slice = g.P * nz; c.st.zsrc_seg = nz;
    if (launch_fwd(mf, c, hs, slot_events(ev, LA_KSLOT_CHUNK)) != hipSuccess) return LA_ERR_DEVICE;
    return LA_OK;
}

LA_API la_status la_forward_causal_chunked(const la_problem *p, int chunk, const void *Q, const void *K,
                                           const void *V, void *O, const float *S_in, const float *z_in,
                                           float *S_out, float *z_out, void *ws, size_t ws_bytes, void *stream) {
    return la_forward_causal_chunked_timed(p, chunk, Q, K, V, O, S_in, z_in, S_out, z_out, ws, ws_bytes, stream,
                                           nullptr);
}

LA_API la_status la_decode_step(const la_problem *p, const void *q, const void *k, const void *v, void *o, float *S,
                                float *z, void *stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi == LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;  // the normaliser needs a positive map
    if (p->N != 1) return LA_ERR_SHAPE;
    if (!q || !k || !v || !o || !S || !z) return LA_ERR_NULL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(S) || !aligned16(z))
        return LA_ERR_ALIGN;
    Shape sh = make_shape(p);
    return launch_decode(sh, q, k, v, o, S, z, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK
                                                                                             : LA_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Retention: decayed, unnormalised ("Story of Attention Part 5", sections 4, 6)
// ---------------------------------------------------------------------------
LA_API la_status la_forward_retention_chunked(const la_problem *p, const float *gamma, int chunk, const void *Q,
                                              const void *K, const void *V, void *O, const float *S_in,
                                              float *S_out, void *ws, size_t ws_bytes, void *stream,
                                              la_kernel_events *ev) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (!chunk_ok(chunk)) return LA_ERR_UNSUPPORTED;
    if (!gamma || !Q || !K || !V || !O) return LA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LA_ERR_ALIGN;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(S_in) ||
        !aligned16(S_out) || !aligned16(ws))
        return LA_ERR_ALIGN;
    Shape sh = make_shape(p);
    sh.ret = 1;
    sh.gamma = gamma;
    bool mf = false;
    Segments g = causal_plan(sh, chunk, &mf);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t nS = (size_t)sh.dp * sh.dv;
    const bool direct = causal_direct(sh, g, mf);
    WsLayout wl = ws_layout(sh, g.P);
    if (!direct && (!ws || ws_bytes < wl.total)) return LA_ERR_WORKSPACE;
    if (ev)
        for (int i = 0; i < LA_KSLOTS; ++i) ev->launched[i] = 0;

    FwdArgs c{};
    c.sh = sh; c.sg = g; c.mode = kModeCausal;
    c.Q = Q; c.K = K; c.V = V; c.O = O;
    if (direct) {
        c.st.S_src = S_in; c.st.src_slice = nS;
        c.st.S_dst = S_out; c.st.dst_slice = nS;
        return launch_fwd(mf, c, hs, slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
    }
    char *wsb = static_cast<char *>(ws);
    float *wsS = reinterpret_cast<float *>(wsb + wl.s_off);
    if (mf) {
        FwdArgs f = c;
        f.mode = fused_mode(sh, g);
        f.st.S_src = S_in; f.st.src_slice = nS;
        f.fu.ctl = reinterpret_cast<uint32_t *>(wsb);
        f.fu.flags = reinterpret_cast<uint32_t *>(wsb + wl.f_off);
        f.fu.slots = wsS;
        f.fu.spin_ticks = kSpinTicks;
        f.fu.S_out = S_out;
        return launch_single_pass(f, hs, slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
    }
    // fp32 path: segment sums (decayed to the segment end), Horner scan, chunk loop
    FwdArgs a{};
    a.sh = sh; a.sg = g; a.mode = kModeState;
    a.Q = Q; a.K = K; a.V = V; a.O = nullptr;
    a.st.S_dst = wsS; a.st.dst_slice = g.P * nS; a.st.dst_seg = nS;
    if (launch_fwd(false, a, hs, slot_events(ev, LA_KSLOT_STATE)) != hipSuccess) return LA_ERR_DEVICE;
    if (launch_scan(sh, g.P, wsS, nullptr, S_in, nullptr, S_out, nullptr, false, hs, slot_events(ev, LA_KSLOT_SCAN),
                    g.seg_chunks * chunk) != hipSuccess)
        return LA_ERR_DEVICE;
    c.st.S_src = wsS; c.st.src_slice = g.P * nS; c.st.src_seg = nS;
    return launch_fwd(false, c, hs, slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
}

LA_API la_status la_retention_decode_step(const la_problem *p, const float *gamma, const void *q, const void *k,
                                          const void *v, void *o, float *S, void *stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->N != 1) return LA_ERR_SHAPE;
    if (!gamma || !q || !k || !v || !o || !S) return LA_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(gamma) & 3u) != 0) return LA_ERR_ALIGN;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(S)) return LA_ERR_ALIGN;
    Shape sh = make_shape(p);
    sh.ret = 1;
    sh.gamma = gamma;
    return launch_decode(sh, q, k, v, o, S, nullptr, static_cast<hipStream_t>(stream)) == hipSuccess ? LA_OK
                                                                                                    : LA_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Backward of the causal normalised form (kernels in la_backward.hip)
// ---------------------------------------------------------------------------
namespace la {
namespace {

// [control block, untouched][forward prefix S][forward prefix z][per-segment
// sums psi^T G_aug][G_aug per token].  The first kCtlBytes are the forward's
// single-pass hand-off state: a buffer shared between forward and backward
// calls keeps it intact.
struct BwdWs {
    size_t s_off, z_off, u_off, g_off, total;
};

// The fp32-arithmetic backward walks a chunk in 16-row tiles and pays, per
// token, for the pairwise products with the chunk's earlier key tiles and for
// reloading them; the chunkwise form gives the same gradients for every chunk
// length, so it runs on chunks of at most this many tokens.
constexpr int kBwdFp32Chunk = 16;

Segments backward_plan(const Shape &sh, int chunk) {
    // matrix-core kernels: one workgroup per CU; fp32 kernels: several
    if (backward_mfma_supported(sh, chunk)) return plan_segments(sh, backward_mfma_tile(sh), 1, 1, kMfmaWorkgroups);
    return plan_segments(sh, chunk < kBwdFp32Chunk ? chunk : kBwdFp32Chunk, 1, 1, kTargetWorkgroups);
}

BwdWs bwd_ws(const Shape &sh, const Segments &g) {
    const size_t bh = (size_t)sh.BH, dp = (size_t)sh.dp, dv = (size_t)sh.dv;
    BwdWs w;
    w.s_off = kCtlBytes;
    w.z_off = w.s_off + round_up(sizeof(float) * bh * g.P * dp * dv, kAlign);
    w.u_off = w.z_off + round_up(sizeof(float) * bh * g.P * dp, kAlign);
    w.g_off = w.u_off + round_up(sizeof(float) * bh * g.P * dp * (dv + 1), kAlign);
    // G_aug per token: fp32 [d_v + 1] (fp32-FMA kernels) or fp32 [backward_mfma_g_floats()] (matrix cores)
    const size_t g_row = sizeof(float) * (backward_mfma_supported(sh, g.chunk) ? backward_mfma_g_floats(sh) : dv + 1);
    w.total = w.g_off + round_up(g_row * bh * sh.N, kAlign);
    return w;
}

}  // namespace
}  // namespace la

LA_API size_t la_backward_workspace_bytes(const la_problem *p, int chunk) {
    if (check_problem(p) != LA_OK || !chunk_ok(chunk) || p->phi == LA_PHI_IDENTITY) return 0;
    const Shape sh = make_shape(p);
    if (!backward_supported(sh)) return 0;
    return bwd_ws(sh, backward_plan(sh, chunk)).total;
}

LA_API la_status la_backward_causal_chunked(const la_problem *p, int chunk, const void *Q, const void *K,
                                            const void *V, const void *dO, const float *S_in, const float *z_in,
                                            const float *dS_out, const float *dz_out, void *dQ, void *dK, void *dV,
                                            float *dS_in, float *dz_in, void *ws, size_t ws_bytes, void *stream,
                                            la_backward_events *ev) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi == LA_PHI_IDENTITY || !chunk_ok(chunk)) return LA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return LA_ERR_NULL;
    if ((S_in == nullptr) != (z_in == nullptr) || (dS_out == nullptr) != (dz_out == nullptr) ||
        (dS_in == nullptr) != (dz_in == nullptr))
        return LA_ERR_NULL;
    const void *ptrs[] = {Q, K, V, dO, S_in, z_in, dS_out, dz_out, dQ, dK, dV, dS_in, dz_in, ws};
    for (const void *q : ptrs)
        if (!aligned16(q)) return LA_ERR_ALIGN;
    const Shape sh = make_shape(p);
    if (!backward_supported(sh)) return LA_ERR_UNSUPPORTED;
    const Segments g = backward_plan(sh, chunk);
    const BwdWs wl = bwd_ws(sh, g);
    if (!ws || ws_bytes < wl.total) return LA_ERR_WORKSPACE;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    char *wsb = static_cast<char *>(ws);
    float *wsS = reinterpret_cast<float *>(wsb + wl.s_off);
    float *wsz = reinterpret_cast<float *>(wsb + wl.z_off);
    const size_t nS = (size_t)sh.dp * sh.dv, nz = (size_t)sh.dp;
    auto slot = [&](int i) {
        KEvents k;
        if (!ev) return k;
        ev->launched[i] = 1;
        k.start = static_cast<hipEvent_t>(ev->start[i]);
        k.stop = static_cast<hipEvent_t>(ev->stop[i]);
        return k;
    };
    if (ev)
        for (int i = 0; i < LA_BSLOTS; ++i) ev->launched[i] = 0;

    // forward prefix entering each segment: per-segment sums, then S_in + exclusive scan
    // (a scan launch for the fp32-FMA passes; the matrix-core passes add the
    // sums in their prologues).  The sums run on the matrix-core state pass when the segments are whole
    // chunks of a length it takes (same boundaries, same P): the backward's own
    // tile, else 128 or 64 tokens.
    const bool mf = backward_mfma_supported(sh, chunk);
    Segments gs = g;
    bool sums_mf = mfma_supported(sh, g.chunk);
    if (!sums_mf)
        for (int c2 : {128, 64})
            if (!sums_mf && (g.seg_chunks * g.chunk) % c2 == 0 && mfma_supported(sh, c2)) {
                gs.chunk = c2;
                gs.n_chunks = (sh.N + c2 - 1) / c2;
                gs.seg_chunks = g.seg_chunks * g.chunk / c2;
                sums_mf = true;
            }
    FwdArgs a{};
    a.sh = sh; a.sg = gs; a.mode = kModeState;
    a.Q = Q; a.K = K; a.V = V; a.O = nullptr;
    a.st.S_dst = wsS; a.st.z_dst = wsz;
    a.st.dst_slice = g.P * nS; a.st.dst_seg = nS; a.st.zdst_slice = g.P * nz; a.st.zdst_seg = nz;
    if (launch_fwd(sums_mf, a, hs, slot(LA_BSLOT_FWD_SUMS)) != hipSuccess) return LA_ERR_DEVICE;
    if (mf) {
        // the matrix-core passes gather their starting states from the
        // per-segment sums themselves (no scan launches)
        BwdMfmaArgs m;
        m.D = sh.dk; m.BH = sh.BH; m.N = sh.N; m.P = g.P; m.seg_chunks = g.seg_chunks; m.n_chunks = g.n_chunks;
        m.f32 = sh.dtype == kF32;
        m.Q = Q; m.K = K; m.V = V; m.dO = dO;
        m.dQ = dQ; m.dK = dK; m.dV = dV;
        m.Ssum = wsS; m.zsum = wsz;
        m.S_in = S_in; m.z_in = z_in;
        m.dS_out = dS_out; m.dz_out = dz_out;
        m.dS_in = dS_in; m.dz_in = dz_in;
        m.U = reinterpret_cast<float *>(wsb + wl.u_off);
        m.G = reinterpret_cast<float *>(wsb + wl.g_off);
        if (launch_bwd_dq_mfma(m, hs, slot(LA_BSLOT_DQ)) != hipSuccess) return LA_ERR_DEVICE;
        return launch_bwd_dkv_mfma(m, hs, slot(LA_BSLOT_DKV)) == hipSuccess ? LA_OK : LA_ERR_DEVICE;
    }
    if (launch_scan(sh, g.P, wsS, wsz, S_in, z_in, nullptr, nullptr, false, hs, slot(LA_BSLOT_FWD_SCAN)) !=
        hipSuccess)
        return LA_ERR_DEVICE;
    BwdLaunch b;
    b.sh = sh; b.sg = g;
    b.Q = Q; b.K = K; b.V = V; b.dO = dO;
    b.dQ = dQ; b.dK = dK; b.dV = dV;
    b.Spre = wsS; b.zpre = wsz;
    b.U = reinterpret_cast<float *>(wsb + wl.u_off);
    b.G = reinterpret_cast<float *>(wsb + wl.g_off);
    b.dS_out = dS_out; b.dz_out = dz_out;
    b.dS_in = dS_in; b.dz_in = dz_in;
    return launch_backward(b, hs, slot(LA_BSLOT_DQ), slot(LA_BSLOT_RSCAN), slot(LA_BSLOT_DKV)) == hipSuccess
               ? LA_OK
               : LA_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Gated and delta-rule recurrences (kernel in la_gated.hip)
// ---------------------------------------------------------------------------
namespace la {
namespace {

la_status gated_call(const la_problem *p, bool gla, const void *Q, const void *K, const void *V, const float *alpha,
                     const float *beta, const float *S_in, float *S_out, void *O, void *stream) {
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;  // raw q, k
    if (!Q || !K || !V || !O) return LA_ERR_NULL;
    if (gla ? !alpha : !beta) return LA_ERR_NULL;
    const void *ptrs[] = {Q, K, V, O, S_in, S_out};
    for (const void *q : ptrs)
        if (!aligned16(q)) return LA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u)) return LA_ERR_ALIGN;
    GatedArgs a;
    a.BH = p->B * p->H; a.N = p->N; a.dk = p->d_k; a.dv = p->d_v;
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    a.alpha = alpha; a.beta = gla ? nullptr : beta;
    a.S_in = S_in; a.S_out = S_out;
    return launch_gated(a, gla, p->dtype == LA_BF16 ? kBF16 : kF32, static_cast<hipStream_t>(stream)) == hipSuccess
               ? LA_OK
               : LA_ERR_DEVICE;
}

}  // namespace
}  // namespace la

LA_API la_status la_forward_gla_recurrent(const la_problem *p, const void *Q, const void *K, const void *V,
                                          const float *alpha, const float *S_in, float *S_out, void *O,
                                          void *stream) {
    return gated_call(p, true, Q, K, V, alpha, nullptr, S_in, S_out, O, stream);
}

LA_API la_status la_forward_delta_recurrent(const la_problem *p, const void *Q, const void *K, const void *V,
                                            const float *alpha, const float *beta, const float *S_in, float *S_out,
                                            void *O, void *stream) {
    return gated_call(p, false, Q, K, V, alpha, beta, S_in, S_out, O, stream);
}

LA_API size_t la_gla_workspace_bytes(const la_problem *p, int chunk) {
    if (la::check_problem(p) != LA_OK || p->phi != LA_PHI_IDENTITY || p->d_k > 64 || chunk != 64) return 0;
    return la::kCtlBytes + la::gla_chunk_ws_bytes(p->B * p->H, p->N, p->d_v);
}

LA_API la_status la_forward_gla_chunked(const la_problem *p, int chunk, const void *Q, const void *K, const void *V,
                                        const float *alpha, const float *S_in, float *S_out, void *O, void *ws,
                                        size_t ws_bytes, void *stream, la_kernel_events *ev) {
    using namespace la;
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi != LA_PHI_IDENTITY || p->d_k > 64 || chunk != 64) return LA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O || !alpha) return LA_ERR_NULL;
    const void *ptrs[] = {Q, K, V, O, S_in, S_out, ws};
    for (const void *q : ptrs)
        if (!aligned16(q)) return LA_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(alpha) & 3u) return LA_ERR_ALIGN;
    if (!ws || ws_bytes < kCtlBytes + gla_chunk_ws_bytes(p->B * p->H, p->N, p->d_v)) return LA_ERR_WORKSPACE;
    if (ev)
        for (int i = 0; i < LA_KSLOTS; ++i) ev->launched[i] = 0;
    GatedArgs a;
    a.BH = p->B * p->H; a.N = p->N; a.dk = p->d_k; a.dv = p->d_v;
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    a.alpha = alpha; a.beta = nullptr;
    a.S_in = S_in; a.S_out = S_out;
    // the records start past the control block (kept for the forward's hand-off)
    return launch_gla_split(a, p->dtype == LA_BF16 ? kBF16 : kF32,
                            reinterpret_cast<float *>(static_cast<char *>(ws) + kCtlBytes),
                            static_cast<hipStream_t>(stream), slot_events(ev, LA_KSLOT_STATE),
                            slot_events(ev, LA_KSLOT_SCAN), slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess
               ? LA_OK
               : LA_ERR_DEVICE;
}

LA_API size_t la_delta_workspace_bytes(const la_problem *p, int chunk) {
    if (la::check_problem(p) != LA_OK || p->phi != LA_PHI_IDENTITY ||
        !la::delta_chunk_supported(p->d_k, p->d_v, chunk))
        return 0;
    return la::kCtlBytes + la::delta_chunk_ws_bytes(p->B * p->H, p->N, p->d_v);
}

LA_API la_status la_forward_delta_chunked(const la_problem *p, int chunk, const void *Q, const void *K, const void *V,
                                          const float *alpha, const float *beta, const float *S_in, float *S_out,
                                          void *O, void *ws, size_t ws_bytes, void *stream, la_kernel_events *ev) {
    using namespace la;
    la_status st = check_problem(p);
    if (st != LA_OK) return st;
    if (p->phi != LA_PHI_IDENTITY) return LA_ERR_UNSUPPORTED;  // raw q, k
    if (!delta_chunk_supported(p->d_k, p->d_v, chunk)) return LA_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O || !beta) return LA_ERR_NULL;
    const void *ptrs[] = {Q, K, V, O, S_in, S_out, ws};
    for (const void *q : ptrs)
        if (!aligned16(q)) return LA_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(alpha) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u)) return LA_ERR_ALIGN;
    if (!ws || ws_bytes < kCtlBytes + delta_chunk_ws_bytes(p->B * p->H, p->N, p->d_v)) return LA_ERR_WORKSPACE;
    if (ev)
        for (int i = 0; i < LA_KSLOTS; ++i) ev->launched[i] = 0;
    GatedArgs a;
    a.BH = p->B * p->H; a.N = p->N; a.dk = p->d_k; a.dv = p->d_v;
    a.Q = Q; a.K = K; a.V = V; a.O = O;
    a.alpha = alpha; a.beta = beta;
    a.S_in = S_in; a.S_out = S_out;
    // the records start past the control block (kept for the forward's hand-off)
    return launch_delta_chunk(a, p->dtype == LA_BF16 ? kBF16 : kF32,
                              reinterpret_cast<float *>(static_cast<char *>(ws) + kCtlBytes),
                              static_cast<hipStream_t>(stream), slot_events(ev, LA_KSLOT_STATE),
                              slot_events(ev, LA_KSLOT_SCAN), slot_events(ev, LA_KSLOT_CHUNK)) == hipSuccess
               ? LA_OK
               : LA_ERR_DEVICE;
}

// ---------------------------------------------------------------------------
// Causal forward for callers that cannot allocate: the workspace is a fixed
// device array of this library
// ---------------------------------------------------------------------------
namespace la {
namespace {

constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 16-byte words");

// Workspace of la_forward_causal_chunked_noalloc: each device that runs the
// library holds its own copy until the process ends.  Host code never uses
// this name as an address (on the host it is only a stand-in for the device
// symbol); it uses the per-device address looked up in device_scratch().
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // per device: address of `scratch` there (null until set up)

// Address of the current device's scratch array.  On the first call on a
// device (with that device current) the address is looked up with
// hipGetSymbolAddress and one zero fill of the whole array is enqueued on the
// caller's stream, ahead of the call's own kernels, so the hand-off control
// block and flags start at zero; afterwards every call leaves the array ready
// for the next one, as with a caller-owned workspace.
la_status device_scratch(hipStream_t st, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return LA_ERR_DEVICE;
        if (launch_zero_fill(ptr, kScratchBytes, st) != hipSuccess) return LA_ERR_DEVICE;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA_OK;
}

}  // namespace
}  // namespace la

LA_API la_status la_forward_causal_chunked_noalloc(const la_problem *p, int chunk, const void *Q, const void *K,
                                                   const void *V, void *O, const float *S_in, const float *z_in,
                                                   float *S_out, float *z_out, void *stream) {
    la_status st = causal_validate(p, chunk, Q, K, V, O, S_in, z_in, S_out, z_out);
    if (st != LA_OK) return st;
    const size_t need = causal_ws(make_shape(p), chunk);
    if (need > kScratchBytes) return LA_ERR_SCRATCH;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    void *ws = nullptr;
    if (need > 0) {
        st = device_scratch(hs, &ws);
        if (st != LA_OK) return st;
    }
    return la_forward_causal_chunked_timed(p, chunk, Q, K, V, O, S_in, z_in, S_out, z_out, ws,
                                           need > 0 ? kScratchBytes : 0, stream, nullptr);
}
