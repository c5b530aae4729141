// Single-pass causal forward, one whole segment (at most 256 tokens) per
// workgroup at once: bf16, d_k = d_v = 64, ELU+1 (normalised) or retention.
//
// The state is additive over tokens ("Linear Attention", recurrent form;
// "Story of Attention Part 5", section 6 blockwise split), so the output of
// a query inside a segment is the segment-local causal attention plus the
// read of the state that enters the segment:
//   num_i = sum_{t <= i, t in segment} phi(q_i).phi(k_t) [v_t | 1]  +  phi(q_i) [S | z]_prefix
//   o_i   = num_i / den_i           (retention: decay lambda^(i-t) on the pairs,
//                                    lambda^(i+1) on the prefix read, no normaliser)
// Sixteen waves share the segment: wave w owns query rows 16w..16w+15 and
// forms their local part in the parallel (masked quadratic) form over every
// key block up to its diagonal, so no wave waits for another's chunk.
// Order of work:
//   1. stage phi(K) and [V | 1] of the segment in LDS (token-major);
//   2. waves 8..11 (sum waves) each sum one 16-row feature strip of the
//      segment's phi(K)^T [V | 1] and publish it to the segment's hand-off
//      slot (device-coherent stores, then a tagged flag per strip), then form
//      the local part of their rows like waves 12..15;
//      waves 0..7 (gather waves) first form their own local rows (the
//      eight shortest), then each waits for one strip of the earlier slots
//      (S_in, then the earlier segments' sums), adds half of its value
//      blocks over those slots in ascending order and writes them to a bf16
//      LDS image of the prefix;
//   3. each wave adds phi(Q) [S | z]_prefix, divides and stores its rows.
// Slots, the launch tag, the bounded waits and the last segment writing
// S_out follow the chunk-loop single pass; the flags are per (segment, strip).
#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_ops.h"

namespace la {
namespace {

constexpr int kSD = 64;         // d_k = d_v = d'
constexpr int kSL = 256;        // tokens of a segment (at most)
constexpr int kSW = 16;         // waves
constexpr int kSThreads = 64 * kSW;
constexpr int kSRK = kSD + 8;   // phi(K) row stride (bf16): 16-row 128-bit reads conflict free
constexpr int kSRV = 144;       // V_aug row stride: 16 mod 128 keeps the transpose reads conflict free
constexpr int kSKB = kSD / 32;  // 32-feature k-blocks
constexpr int kStrips = kSD / 16;  // 16-row feature strips of the state, one state wave each
static_assert(kStrips <= kFlagsPerSegment, "one hand-off flag per strip");

template <bool RET>
struct SegSmem {
    static constexpr int NJ = RET ? 4 : 5;  // value column blocks (+ the normaliser block)
    uint16_t K[kSL * kSRK];                 // phi(K) token-major; afterwards the per-wave output staging
    uint16_t V[kSL * kSRV];                 // [V | 1 | 0] token-major
    uint4 STB[NJ][kSKB][64];                // bf16 prefix [S | z]: B operand of phi(Q) S
    f32x4 PB[kStrips][kSD / 16][64];        // prefix strips, accumulator order (value blocks)
    float PZ[kStrips][16];                  // prefix strips, normaliser column
    f32x4 OWN[kStrips][NJ][64];             // last segment: its own sums, accumulator order
    // retention: lambda^x for x < kSL, then the key weights lambda^(L-1-t)
    // of the segment's tokens (0 past its end)
    alignas(16) float DW[RET ? 2 * kSL : 4];
};

// 16x16 fp32 tile (lane l: rows 16fb + 4g + e, column 16nb + l%16) into the
// bf16 B-operand image of the state
template <int NJ>
__device__ __forceinline__ void put_tile(uint4 (*STB)[kSKB][64], int fb, int nb, int lane, f32x4 s) {
    const int g = lane >> 4, c = lane & 15;
    const uint2 v = pack4(s[0], s[1], s[2], s[3]);
    const int x = 16 * (fb & 1) + 4 * g;  // feature slot inside the 32-feature k-block
    reinterpret_cast<uint2 *>(&STB[nb][fb >> 1][c + 16 * (x >> 3)])[(x >> 2) & 1] = v;
}

template <int PHI>
__global__ __launch_bounds__(kSThreads) void k_seg(FwdArgs a) {
    constexpr bool RET = PHI == kIdentity;
    using Sm = SegSmem<RET>;
    constexpr int NJ = Sm::NJ;
    __shared__ Sm sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, c16 = lane & 15;

    const Segments sg = a.sg;
    const int N = a.sh.N;
    const int P = sg.P;
    int bh, seg;
    seg_of_block(blockIdx.x, a.sh.BH, P, bh, seg);
    const int seg_tokens = sg.seg_chunks * sg.chunk;
    const int t0 = seg * seg_tokens;
    const int L = min(seg_tokens, N - t0);  // tokens of this segment, 1..256

    const float l2 = RET ? log2f(a.sh.gamma[bh % a.sh.H]) : 0.f;
    auto dpow = [&](float x) { return x == 0.f ? 1.f : __builtin_amdgcn_exp2f(x * l2); };

    const uint16_t *Qs = static_cast<const uint16_t *>(a.Q) + ((size_t)bh * N + t0) * kSD;
    const uint16_t *Ks = static_cast<const uint16_t *>(a.K) + ((size_t)bh * N + t0) * kSD;
    const uint16_t *Vs = static_cast<const uint16_t *>(a.V) + ((size_t)bh * N + t0) * kSD;
    uint16_t *Os = static_cast<uint16_t *>(a.O) + ((size_t)bh * N + t0) * kSD;

    // ---- loads of the whole segment go out first (rows past the end read zero)
    const auto rk = make_rsrc(Ks, L * kSD * 2), rv = make_rsrc(Vs, L * kSD * 2), rq = make_rsrc(Qs, L * kSD * 2);
    constexpr int PT = kSL * kSD / 8 / kSThreads;  // 16-byte pieces of K (and of V) per thread
    uint4 kraw[PT], vraw[PT], qraw[kSKB];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        kraw[i] = bload16_nt(rk, 16 * (tid + i * kSThreads));
        vraw[i] = bload16_nt(rv, 16 * (tid + i * kSThreads));
    }
    const int qb = w;              // this wave's 16-row query block inside the segment
    const int row = 16 * qb + c16;  // this lane's query row (A operand of phi(Q) S)

    // hand-off slots: strip fb (feature rows 16fb..16fb+15, all value blocks)
    // of a state is 64 lanes x NJ x 16 bytes in accumulator order
    constexpr int SLOT = kSD * (kSD + 16);  // floats per hand-off slot
    float *const slots = a.fu.slots + (size_t)bh * (P + 1) * SLOT;
    auto slot_rsrc = [&](int i, bool live) { return make_rsrc(slots + (size_t)i * SLOT, live ? SLOT * 4 : 0); };
    // In the normaliser block only column d_v is data: lane (g, 0) stores
    // rows 4g..4g+3 of the strip's 16 contiguous floats; the other lanes
    // address past the slot (their stores drop).
    auto piece_off = [&](int fb, int nb) {
        return nb == 4 ? (c16 != 0 ? SLOT * 4 : ((fb * 5 + 4) * 64 + g) * 16) : ((fb * 5 + nb) * 64 + lane) * 16;
    };
    const bool has_in = a.st.S_src != nullptr;

    // ---- 1. stage phi(K) (zero past the end: phi(0) would be 1) and [V | 1 | 0]
#pragma unroll
    for (int i = 0; i < PT; ++i) {
        const int u = tid + i * kSThreads, t = u / (kSD / 8), c8 = u % (kSD / 8);
        uint4 ph = RET ? kraw[i] : elu1_bf16x8(kraw[i]);
        if (t >= L) ph = make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4 *>(&sm.K[t * kSRK + 8 * c8]) = ph;
        *reinterpret_cast<uint4 *>(&sm.V[t * kSRV + 8 * c8]) = vraw[i];
    }
    if constexpr (!RET) {
        for (int u = tid; u < kSL * 2; u += kSThreads) {
            const int t = u >> 1, half = u & 1;
            *reinterpret_cast<uint4 *>(&sm.V[t * kSRV + kSD + 8 * half]) = make_uint4(half == 0 ? 0x3f80u : 0u, 0, 0, 0);
        }
    }
    if constexpr (RET) {  // the decay tables: one exponential per thread instead of one per use
        if (tid < kSL) {
            sm.DW[tid] = dpow((float)tid);
        } else if (tid < 2 * kSL) {
            const int t = tid - kSL;
            sm.DW[tid] = t < L ? dpow((float)(L - 1 - t)) : 0.f;
        }
    }
    static_assert(kSThreads >= 2 * kSL, "one table entry per thread");
    // the query rows go out once the keys and values (which the hand-off
    // waits for) have arrived
#pragma unroll
    for (int kb = 0; kb < kSKB; ++kb) qraw[kb] = bload16_nt(rq, 2 * (row * kSD + 8 * g + 32 * kb));
    block_sync_lds();

    Op8 phq[kSKB];
    f32x4 acc[NJ];
    // local part of this wave's rows: (P (.) M) V_aug over the key blocks up
    // to the diagonal (every wave calls it once, before the prefix read)
    auto local_rows = [&]() {
        if constexpr (RET) {
#pragma unroll
            for (int kb = 0; kb < kSKB; ++kb) phq[kb].u = qraw[kb];
        } else {  // ELU+1 with the row's power-of-two scale (cancels in the division)
            uint4 ph[kSKB];
            elu1_query_pieces<kSKB>(qraw, ph);
#pragma unroll
            for (int kb = 0; kb < kSKB; ++kb) phq[kb].u = ph[kb];
        }
#pragma unroll
        for (int nb = 0; nb < NJ; ++nb) acc[nb] = zero4();
        for (int kt = 0; 2 * kt <= qb; ++kt) {
            f32x4 p[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int jb = 2 * kt + h;
                p[h] = zero4();
                if (jb <= qb) {
                    const uint16_t *krow = &sm.K[(16 * jb + c16) * kSRK];
#pragma unroll
                    for (int kf = 0; kf < kSKB; ++kf) {
                        Op8 ka;
                        ka.u = *reinterpret_cast<const uint4 *>(krow + 32 * kf + 8 * g);
                        p[h] = mfma(ka, phq[kf], p[h]);
                    }
                    if (jb == qb) {  // diagonal block: key 4g+e <= query c16
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * g + e > c16) p[h][e] = 0.f;
                    }
                    if constexpr (RET) {  // decay lambda^(query - key)
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            const int d = 16 * (qb - jb) + c16 - 4 * g - e;
                            p[h][e] *= d >= 0 ? sm.DW[max(d, 0)] : 0.f;  // d <= 255
                        }
                    }
                }
            }
            Op8 pa;
            pa.q[0] = pack4(p[0][0], p[0][1], p[0][2], p[0][3]);
            pa.q[1] = pack4(p[1][0], p[1][1], p[1][2], p[1][3]);
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) acc[nb] = mfma(pa, token_operand<kSRV>(sm.V, kt, 16 * nb, lane), acc[nb]);
        }
    };

    const uint32_t tag = __hip_atomic_load(a.fu.ctl, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    uint32_t *fl = a.fu.flags + (size_t)bh * P * kStrips;
    // retention: the state decays across each segment, so slot j enters the
    // prefix as S = lambda^(tokens of segment j-1) S + slot j (Horner form);
    // every segment before this one is full
    // ---- 2a. sum waves 8..11: strip fb = w - 8 of the segment sum phi(K)^T V_aug
    // (retention: sum_t lambda^(L-1-t) k_t v_t^T, the key weights on the operand
    // slots).  The other waves wait meanwhile: the strips are what the later
    // segments wait for, and alone the sum waves have the LDS to themselves.
    const bool sum_wave = w >= 8 && w < 8 + kStrips;
    f32x4 own[NJ];
    if (sum_wave) {
        const int fb = w - 8;
#pragma unroll
        for (int nb = 0; nb < NJ; ++nb) own[nb] = zero4();
        // every 32-token block of the segment, a fixed count so the operand
        // loads can run ahead: rows past the end hold phi(k) = 0 and add nothing
#pragma unroll
        for (int kt = 0; kt < kSL / 32; ++kt) {
            Op8 ka = token_operand<kSRK>(sm.K, kt, 16 * fb, lane);
            if constexpr (RET) {  // key weight of slot sl: token 32kt + 16(sl/4) + 4g + sl%4
                const float4 w0 = *reinterpret_cast<const float4 *>(&sm.DW[kSL + 32 * kt + 4 * g]);
                const float4 w1 = *reinterpret_cast<const float4 *>(&sm.DW[kSL + 32 * kt + 16 + 4 * g]);
                const float kw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    ka.u32[j] = cvt2(lo_bf16(ka.u32[j]) * kw[2 * j], hi_bf16(ka.u32[j]) * kw[2 * j + 1]);
            }
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) own[nb] = mfma(ka, token_operand<kSRV>(sm.V, kt, 16 * nb, lane), own[nb]);
        }
    }
    block_sync_lds();
    if (sum_wave) {
        // published to slot 1 + seg with flag (seg, fb); segment 0 also copies
        // strip fb of S_in into slot 0 (only segment 0 reads S_in, so S_out may alias it)
        const int fb = w - 8;
        if (seg < P - 1) {
            auto store_strip = [&](int i, const f32x4 *t) {
                const auto r = slot_rsrc(i, true);
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, t[nb]), r, piece_off(fb, nb), 0,
                                                           kCoherent);
            };
            if (seg == 0 && has_in) {
                const float *Sin = a.st.S_src + bh * a.st.src_slice;
                const float *zin = a.st.z_src + bh * a.st.zsrc_slice;
                f32x4 t[NJ];
#pragma unroll
                for (int nb = 0; nb < NJ; ++nb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int f = 16 * fb + 4 * g + e, j = 16 * nb + c16;
                        t[nb][e] = j < kSD ? Sin[(size_t)f * kSD + j] : (j == kSD ? zin[f] : 0.f);
                    }
                store_strip(0, t);
            }
            store_strip(1 + seg, own);
            wait_stores();  // this wave's stores have completed ...
            if (lane == 0)  // ... before its flag is tagged
                __hip_atomic_store(fl + seg * kStrips + fb, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (seg == P - 1)  // kept for S_out
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) sm.OWN[fb][nb][lane] = own[nb];
    }
    // ---- 2b. gather waves 0..7: wave w adds value blocks 2ch, 2ch+1
    // (ch = w / 4; ch 0 also the normaliser column) of strip fb = w % 4 over
    // the prefix's slots in ascending order (S_in in slot 0, then the earlier
    // segments' sums) and writes them to the bf16 image and, for S_out, to
    // LDS.  The normaliser column travels as one float per lane (lane l:
    // row l % 16).  The gather waves' own rows are the eight shortest; they
    // are formed first, while the earlier strips are on their way.
    if (w < 2 * kStrips) {
        const int fb = w % kStrips, ch = w / kStrips;
        local_rows();
        f32x4 pre[2] = {zero4(), zero4()};
        float zpre = 0.f;
        bool late = false;
        if (seg == 0) {
            if (has_in) {  // segment 0 reads S_in itself
                const float *Sin = a.st.S_src + bh * a.st.src_slice;
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) pre[q][e] = Sin[(size_t)(16 * fb + 4 * g + e) * kSD + 16 * (2 * ch + q) + c16];
                if constexpr (!RET)
                    if (ch == 0) zpre = a.st.z_src[bh * a.st.zsrc_slice + 16 * fb + c16];
            }
        } else {
            // slot j >= 1 comes with flag (j - 1, fb), slot 0 with flag (0, fb):
            // lane i polls flag (i, fb), one access per poll
            const long long t_begin = wall_clock64();
            for (int base = 0; base < seg && !late; base += 64) {
                const int i = base + lane;
                while (true) {
                    const bool ok =
                        i >= seg || __hip_atomic_load(fl + i * kStrips + fb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
                    if (__builtin_amdgcn_ballot_w64(!ok) == 0) break;
                    if (wall_clock64() - t_begin > a.fu.spin_ticks) {
                        late = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(2);
                }
            }
            asm volatile("" ::: "memory");  // the slot loads stay behind the flag reads
            auto load4 = [&](int j, bool live, int off) {
                return __builtin_amdgcn_raw_buffer_load_b128(slot_rsrc(j, live), off, 0, kCoherent);
            };
            auto load1 = [&](int j, bool live, int off) {
                return __builtin_amdgcn_raw_buffer_load_b32(slot_rsrc(j, live), off, 0, kCoherent);
            };
            constexpr int GD = 8;            // slots in flight
            const int first = has_in ? 0 : 1;
            for (int j0 = first; j0 <= seg; j0 += GD) {
                f32x4 buf[GD][2];
                float zb[GD];
#pragma unroll
                for (int d = 0; d < GD; ++d) {
                    const int j = j0 + d;
                    const bool live = j <= seg;  // past the range: zeros
#pragma unroll
                    for (int q = 0; q < 2; ++q) buf[d][q] = __builtin_bit_cast(f32x4, load4(j, live, piece_off(fb, 2 * ch + q)));
                    zb[d] = 0.f;
                    if (!RET && ch == 0) zb[d] = __builtin_bit_cast(float, load1(j, live, ((fb * 5 + 4) * 64) * 16 + 4 * c16));
                }
#pragma unroll
                for (int d = 0; d < GD; ++d) {
                    const int j = j0 + d;
                    // retention: slot j enters as S = lambda^(tokens of segment j-1) S + slot j
                    // (Horner form); every segment before this one is full
                    const float mul = RET && j >= 1 && j <= seg ? dpow((float)seg_tokens) : 1.f;
#pragma unroll
                    for (int q = 0; q < 2; ++q) pre[q] = RET ? pre[q] * mul + buf[d][q] : pre[q] + buf[d][q];
                    zpre += zb[d];
                }
            }
        }
        if (late) {
            const float qn = __builtin_nanf("");
            pre[0] = pre[1] = f32x4{qn, qn, qn, qn};
            zpre = qn;
            if (lane == 0) __hip_atomic_store(a.fu.ctl + 2, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            sm.PB[fb][2 * ch + q][lane] = pre[q];  // kept for S_out
            put_tile<NJ>(sm.STB, fb, 2 * ch + q, lane, pre[q]);
        }
        if constexpr (!RET) {
            if (ch == 0) {
                if (lane < 16) sm.PZ[fb][lane] = zpre;
                // accumulator layout of the normaliser block: lane (g, 0) holds rows 4g..4g+3
                f32x4 zt;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float zr = __shfl(zpre, 4 * g + e, 64);
                    zt[e] = c16 == 0 ? zr : 0.f;
                }
                put_tile<NJ>(sm.STB, fb, NJ - 1, lane, zt);
            }
        }
    } else {
        // ---- 2c. local part of the other waves' rows
        local_rows();
    }
    block_sync_lds();  // the prefix image is complete; every wave is done with phi(K)
    if (seg == P - 1 && a.fu.S_out && w >= 8 && w < 8 + kStrips) {
        // final state of the slice = prefix + own sums (retention: the prefix decays across the own segment)
        const int fb = w - 8;
        float *So = a.fu.S_out + (size_t)bh * kSD * kSD;
        const float tail = RET ? dpow((float)L) : 1.f;
#pragma unroll
        for (int nb = 0; nb < kSD / 16; ++nb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                So[(size_t)(16 * fb + 4 * g + e) * kSD + 16 * nb + c16] =
                    tail * sm.PB[fb][nb][lane][e] + sm.OWN[fb][nb][lane][e];
        if constexpr (!RET)
            if (c16 == 0)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    a.fu.z_out[(size_t)bh * kSD + 16 * fb + 4 * g + e] = sm.PZ[fb][4 * g + e] + sm.OWN[fb][NJ - 1][lane][e];
    }

    // ---- 3. phi(Q) [S | z]_prefix (retention: scaled by lambda^(i+1)), divide, store
    {
        f32x4 sq[NJ];
#pragma unroll
        for (int nb = 0; nb < NJ; ++nb) sq[nb] = zero4();
#pragma unroll
        for (int kf = 0; kf < kSKB; ++kf)
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) {
                Op8 sb;
                sb.u = sm.STB[nb][kf][lane];
                sq[nb] = mfma(phq[kf], sb, sq[nb]);
            }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float r = RET ? dpow((float)(16 * qb + 4 * g + e + 1)) : 1.f;
#pragma unroll
            for (int nb = 0; nb < NJ; ++nb) acc[nb][e] += RET ? r * sq[nb][e] : sq[nb][e];
        }
    }
    float rden[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rden[e] = RET ? 1.f : __builtin_amdgcn_rcpf(__shfl(acc[NJ - 1][e], lane & 48, 64));
    uint16_t *so = &sm.K[16 * w * kSRK];  // this wave's 16 rows of the phi(K) area
#pragma unroll
    for (int nb = 0; nb < kSD / 16; ++nb)
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
            const uint32_t two_ = cvt2(acc[nb][e] * rden[e], acc[nb][e + 1] * rden[e + 1]);
            so[(4 * g + e) * kSRK + 16 * nb + c16] = static_cast<uint16_t>(two_);
            so[(4 * g + e + 1) * kSRK + 16 * nb + c16] = static_cast<uint16_t>(two_ >> 16);
        }
    wave_lds_sync();
    const auto ro = make_rsrc(Os, L * kSD * 2);  // rows past the end are dropped
#pragma unroll
    for (int it = 0; it < 16 * kSD / 8 / 64; ++it) {
        const int idx = it * 64 + lane, r = idx / (kSD / 8), c8 = idx % (kSD / 8);
        bstore16_nt(ro, 2 * ((16 * qb + r) * kSD + 8 * c8), *reinterpret_cast<const uint4 *>(&so[r * kSRK + 8 * c8]));
    }

    // the last workgroup of the launch to finish (all flag reads done)
    // advances the launch counter and clears the done count
    if (tid == 0) {
        const uint32_t done = __hip_atomic_fetch_add(a.fu.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (done == gridDim.x - 1) {
            __hip_atomic_store(a.fu.ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(a.fu.ctl, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

bool seg_supported(const Shape &sh, const Segments &g) {
    return sh.dtype == kBF16 && sh.dk == kSD && sh.dv == kSD && (sh.phi == kElu1 || sh.phi == kIdentity) &&
           (sh.phi == kIdentity) == (sh.ret != 0) && g.chunk * g.seg_chunks <= kSL && g.P > 1;
}

hipError_t launch_seg(const FwdArgs &a, hipStream_t st, KEvents ev) {
    if (!seg_supported(a.sh, a.sg)) return hipErrorNotSupported;
    const dim3 grid((unsigned)((size_t)a.sh.BH * a.sg.P)), block(kSThreads);
    if (a.sh.phi == kIdentity) return launch_kernel_ev(k_seg<kIdentity>, grid, block, 0, st, ev, a);
    return launch_kernel_ev(k_seg<kElu1>, grid, block, 0, st, ev, a);
}

}  // namespace la
