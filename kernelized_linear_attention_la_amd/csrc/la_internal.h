// Internal declarations shared by the liblinattn HIP sources (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace la {

enum Phi : int { kElu1 = 0, kFavor = 1, kIdentity = 2, kDpfp = 3, kTrig = 4, kCosformer = 5 };
enum Dtype : int { kF32 = 0, kBF16 = 1 };

// What one launch of the chunked kernels does over its token range.
enum Mode : int {
    kModeState = 0,   // accumulate phi(K)^T [V, 1] of the segment into a state slot
    kModeCausal = 1,  // chunkwise causal forward starting from a prefix state
    kModeRead = 2,    // non-causal read: O = phi(Q) S / phi(Q) z with a fixed state
    kModeFused = 3,   // causal, single pass: segment sums, hand-off between segments, chunk loop
    kModeFusedRes = 4 // single pass with the segment's phi(K), V kept in LDS between the phases
};

// Hand-off flags per (slice, segment) in the single-pass workspace (the
// whole-segment kernel flags each 16-row strip of the state on its own).
constexpr int kFlagsPerSegment = 4;

// Chunks per segment that the LDS-resident single pass can hold (d = 64, 64-token chunks).
constexpr int kResChunks = 4;

// Shape of one call, after host validation.
struct Shape {
    int BH;       // B * H slices
    int N;        // tokens per slice
    int dk, dv;   // widths
    int dp;       // feature dimension d' (dk or m)
    int phi;      // Phi
    int m;        // FAVOR+ / TRIG random features (0 otherwise)
    const float *W;  // FAVOR+ / TRIG rows [m, dk] (device)
    int param;    // DPFP nu, cosFormer M (0 otherwise)
    long long pos0;  // cosFormer: position of the call's first token
    int dtype;    // Dtype of Q/K/V/O
    // Retention (decayed, unnormalised): ret = 1 and the decay of head h is
    // gamma[h] (device, [H]; slice b*H + h uses gamma[h]).  Normalised kernel
    // attention: ret = 0, gamma = NULL.
    int ret;
    const float *gamma;
    int H;
};

// Token ranges split into segments of whole chunks; one workgroup column per segment.
struct Segments {
    int chunk;        // tokens per chunk
    int n_chunks;     // ceil(N / chunk)
    int seg_chunks;   // chunks per segment
    int P;            // number of segments = ceil(n_chunks / seg_chunks)
};

// State storage of a launch.  Slot s of slice b lives at
// S + ((size_t)b * P + s) * dp * dv (and z + ((size_t)b * P + s) * dp).
struct StateArgs {
    const float *S_src;   // prefix/total state to start from (NULL = zero)
    const float *z_src;
    size_t src_slice, src_seg;    // floats between slices / segments in S_src
    size_t zsrc_slice, zsrc_seg;  // same for z_src
    float *S_dst;         // where the final state of the range goes (NULL = nowhere)
    float *z_dst;
    size_t dst_slice, dst_seg;
    size_t zdst_slice, zdst_seg;
};

// Hand-off of the single-pass causal mode (one launch, P segments per slice).
// ctl[0] counts completed launches on this workspace, ctl[1] counts the
// workgroups of the running launch that are done, ctl[2] is set to 1 when a
// wait expired (the affected outputs are then NaN).  A launch tags its flags
// with ctl[0] + 1; the last workgroup to finish advances ctl[0] and clears
// ctl[1].  The control block and flags must be zero before the first launch
// on a workspace.  Slot 0 of a slice holds S_in, slot 1 + s the sums of
// segment s (slot P also parks the last segment's own sums).
struct FusedArgs {
    uint32_t *ctl;         // [3] launch counter, done count, error word
    uint32_t *flags;       // [B*H*P*kFlagsPerSegment] tags of the launch whose segment sums are ready
    float *slots;          // [B*H][P+1][d' * (d_v + 16)] accumulator-order states
    long long spin_ticks;  // wall-clock bound of one wait (s_memrealtime ticks)
    float *S_out, *z_out;  // final state of each slice (NULL = not exported)
};

struct FwdArgs {
    Shape sh;
    Segments sg;
    int mode;
    const void *Q, *K, *V;
    void *O;
    StateArgs st;
    FusedArgs fu;
};

// Optional timing events of one kernel launch (profiling hook).
struct KEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};

// Launch `kernel` and return the status of this launch alone, never an error
// left pending by earlier runtime calls of the caller.  With events, the
// launch itself records them (hipExtLaunchKernel), so they bracket exactly
// the kernel's execution.
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel_ev(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                                   KEvents ev, Args &&...args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel argument count");
    std::tuple<KArgs...> vals(std::forward<Args>(args)...);
    return std::apply(
        [&](auto &...v) {
            void *ptrs[] = {static_cast<void *>(&v)...};
            const void *f = reinterpret_cast<const void *>(kernel);
            if (ev.start || ev.stop) return hipExtLaunchKernel(f, grid, block, ptrs, lds, st, ev.start, ev.stop, 0);
            return hipLaunchKernel(f, grid, block, ptrs, lds, st);
        },
        vals);
}

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                                Args &&...args) {
    return launch_kernel_ev(kernel, grid, block, lds, st, KEvents{}, std::forward<Args>(args)...);
}

// Host-side launchers (return hipSuccess or the launch error).
hipError_t launch_generic(const FwdArgs &a, hipStream_t stream, KEvents ev = {});
hipError_t launch_scan(const Shape &sh, int P, float *ws_S, float *ws_z, const float *S_in,
                       const float *z_in, float *S_out, float *z_out, bool total_to_slot0,
                       hipStream_t stream, KEvents ev = {}, int seg_tokens = 0);
// Zero fill of `bytes` (a multiple of 16) at p, on the stream (a kernel, so
// it may be recorded into a graph).
hipError_t launch_zero_fill(void *p, size_t bytes, hipStream_t stream);
// Error word of a workspace control block to *out (cleared when asked).
hipError_t launch_ws_error(uint32_t *ctl, uint32_t *out, bool clear, hipStream_t stream);
hipError_t launch_decode(const Shape &sh, const void *q, const void *k, const void *v, void *o,
                         float *S, float *z, hipStream_t stream);
// fp32 storage on fp32 matrix instructions (la_f32mma.hip): ELU+1,
// normalised, d_k = d_v in {64, 128}; one workgroup per (slice, segment)
// covers every value column.  launch_generic takes it where it applies.
bool f32mma_supported(const Shape &sh);
hipError_t launch_f32mma(const FwdArgs &a, hipStream_t stream, KEvents ev = {});
// bf16 MFMA path; returns hipErrorNotSupported when the shape has no MFMA variant.
hipError_t launch_mfma(const FwdArgs &a, hipStream_t stream, KEvents ev = {});
bool mfma_supported(const Shape &sh, int chunk);
// Single pass with a whole segment (at most 256 tokens) per 16-wave
// workgroup (la_mfma_seg.hip): bf16, d = 64, ELU+1 or retention, P > 1.
bool seg_supported(const Shape &sh, const Segments &g);
hipError_t launch_seg(const FwdArgs &a, hipStream_t stream, KEvents ev = {});
// FAVOR+ single pass with eight waves per workgroup (la_favor.hip): bf16,
// d_k = d_v = 64, m = 256, 64-token chunks, P > 1.
bool favor_supported(const Shape &sh, const Segments &g);
hipError_t launch_favor(const FwdArgs &a, hipStream_t stream, KEvents ev = {});

// Backward of the causal normalised form (la_backward.hip): three launches
// per call after the forward prefix is in Spre / zpre.
struct BwdLaunch {
    Shape sh;
    Segments sg;
    const void *Q, *K, *V, *dO;
    void *dQ, *dK, *dV;
    const float *Spre, *zpre;       // forward prefix entering each segment
    float *U;                       // [BH][P][d' (d_v + 1)] workspace
    float *G;                       // [BH][N][d_v + 1] workspace
    const float *dS_out, *dz_out;   // NULL = zero
    float *dS_in, *dz_in;           // NULL = not wanted
};
bool backward_supported(const Shape &sh);
// Reverse scan of the per-segment sums (la_backward.hip): U [BH][P][d' (d_v+1)]
// becomes the exclusive suffixes (+ dS_out); dS_in / dz_in get the totals.
hipError_t launch_bwd_rscan(int BH, int P, int dp, int dv, float *U, const float *dS_out, const float *dz_out,
                            float *dS_in, float *dz_in, hipStream_t stream, KEvents ev = {});

// Matrix-core backward (la_backward_mfma.hip): bf16 storage, fp32 matrix
// instructions, ELU+1, d_k = d_v = 64, 64-token chunks.  G holds G_aug as
// fp32 [BH][N][backward_mfma_g_floats()].
struct BwdMfmaArgs {
    int D, BH, N, P, seg_chunks, n_chunks;  // d_k = d_v = D; chunks are backward_mfma_tile() tokens
    int f32;                                // storage: fp32 (1) or bf16 (0)
    const void *Q, *K, *V, *dO;
    void *dQ, *dK, *dV;
    const float *Ssum, *zsum;  // forward sums per segment, [BH][P][D][D] and [BH][P][D]
    const float *S_in, *z_in;  // forward starting state [BH][D][D], [BH][D], or both null (zero)
    const float *dS_out, *dz_out;  // gradient of the final state, or both null (zero)
    float *dS_in, *dz_in;      // gradient of the starting state (written), or both null
    float *U;                  // [BH][P][D * (D + 1)]: per-segment sums of phi(Q)^T G_aug
    float *G;                  // [BH][N][backward_mfma_g_floats()]
};
// ELU+1 (bf16 or fp32), d_k = d_v = 64 with 64-token chunks, or 128 with chunks of a multiple of 32
bool backward_mfma_supported(const Shape &sh, int chunk);
int backward_mfma_tile(const Shape &sh);            // tokens per tile: 64 (d 64), 32 (d 128)
size_t backward_mfma_g_floats(const Shape &sh);     // G_aug floats per token: d_v + 4
hipError_t launch_bwd_dq_mfma(const BwdMfmaArgs &a, hipStream_t stream, KEvents ev = {});
hipError_t launch_bwd_dkv_mfma(const BwdMfmaArgs &a, hipStream_t stream, KEvents ev = {});

// Gated / delta-rule recurrences (la_gated.hip): one workgroup per slice.
struct GatedArgs {
    int BH, N, dk, dv;
    const void *Q, *K, *V;
    void *O;
    const float *alpha;  // GLA: [BH, N, dk]; delta rule: [BH, N] or NULL (no gate)
    const float *beta;   // delta rule: [BH, N]; GLA: unused
    const float *S_in;   // [BH, dk, dv] or NULL (zero)
    float *S_out;        // [BH, dk, dv] or NULL; may be S_in
};
hipError_t launch_gated(const GatedArgs &a, bool gla, int dtype, hipStream_t stream, KEvents ev = {});
// GLA in chunkwise form (la_gla_chunk.hip): d_k <= 64, N >= 64.
bool gla_chunk_supported(const GatedArgs &a);
hipError_t launch_gla_chunk(const GatedArgs &a, int dtype, hipStream_t stream, KEvents ev = {});
// The same chunk form in three launches (every product per chunk at once, the
// element-wise state chain over chunks, the outputs per chunk at once); ws
// holds one record per chunk.  Same support.
size_t gla_chunk_ws_bytes(int BH, int N, int dv);
hipError_t launch_gla_split(const GatedArgs &a, int dtype, float *ws, hipStream_t stream, KEvents ev_prep = {},
                            KEvents ev_chain = {}, KEvents ev_out = {});
// Gated delta rule in chunkwise form (la_delta_chunk.hip): d_k = 64, d_v a
// multiple of 16 up to 128, 64-token chunks; ws holds one record per chunk.
// Three launches: the per-chunk operators, the state chain, the outputs.
bool delta_chunk_supported(int dk, int dv, int chunk);
size_t delta_chunk_ws_bytes(int BH, int N, int dv);
hipError_t launch_delta_chunk(const GatedArgs &a, int dtype, float *ws, hipStream_t stream, KEvents ev_prep = {},
                              KEvents ev_scan = {}, KEvents ev_out = {});
size_t backward_lds_bytes(const Shape &sh);
hipError_t launch_backward(const BwdLaunch &b, hipStream_t stream, KEvents ev_dq = {}, KEvents ev_scan = {},
                           KEvents ev_dkv = {});

}  // namespace la
