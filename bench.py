#!/usr/bin/env python3
"""Benchmark of the causal kernelized linear attention hot path on one MI355X.

A step is one full pass of the hot path over one batch of seeded synthetic
input: la_forward_causal_chunked (feature map, intra-chunk masked products,
inter-chunk state read, fused normalisation, state scan, final state export)
for a forward workload, or one la_decode_step over every sequence and head for
the decode workload.  Inputs are resident in HBM before timing starts; the
forward workloads rotate through enough copies of the batch to overflow the
256 MB Infinity Cache, so every step streams from HBM.

Prints ONE JSON line (rank 0, N=1):
  value         whole-job throughput (tokens/s; decode: generated tokens/s,
                one token per sequence per step)
  roofline      the dominant kernel's achieved algorithmic bytes (or flops)
                per launch / its average duration, from HIP events recorded
                around that kernel on its own stream, against the MI355X peak
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

DEFAULT_WORKLOAD = "elu1_bf16_b2h16n16384d128_c128"
# measured in the same run as the default workload and reported under "extra":
# the decode half of the metric and the FAVOR+ chunked forward (the one
# workload whose flops outweigh its bytes)
EXTRA_DECODE = "decode_elu1_f32_s256h32d128_prefix1024_steps64"
EXTRA_FAVOR = "favor_bf16_b2h8n8192d64_m256_c64"
PREFIX_BLOCK = 64  # sequences of the decode prefix drawn and run at a time
EVENT_BATCH = 64  # back-to-back launches timed per HIP event pair
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 matrix cores, TFLOP/s
FP32_VECTOR_PEAK_TFS = 157.3  # MI355X fp32 vector ALUs (256 CUs x 256 flop/clk x 2.4 GHz), TFLOP/s
MFMA_F32_PEAK_TFS = 157.3    # MI355X dense fp32 matrix cores, TFLOP/s
ROTATE_BYTES = 768 << 20     # > 256 MB Infinity Cache


def elem_bytes(dtype):
    return 2 if dtype == "bf16" else 4


def forward_alg_bytes(wl):
    """Algorithmic HBM bytes of one causal forward: Q, K, V read once, O written once, final state written
    (retention carries no normaliser z)."""
    e = elem_bytes(wl.dtype)
    tok = wl.B * wl.H * wl.N
    state = wl.B * wl.H * (wl.dprime * wl.dv + (0 if wl.retention else wl.dprime)) * 4
    return tok * (2 * wl.dk + 2 * wl.dv) * e + state


def tile_chunk(wl):
    """Chunk length the library tiles a forward with: the maps that run on the
    matrix cores at 64-token chunks only (FAVOR+ with m 256, one-shift DPFP,
    cos/sin with m 64, cosFormer; bf16, d 64) run a 128-token request on that
    64-token tiling."""
    if wl.dtype != "bf16" or wl.retention or wl.dk != 64 or wl.dv != 64 or wl.chunk != 128:
        return wl.chunk
    if ((wl.phi == "favor" and wl.m == 256) or (wl.phi == "dpfp" and wl.map_param == 1) or
            (wl.phi == "trig" and wl.m == 64) or wl.phi == "cosformer"):
        return 64
    return wl.chunk


def forward_alg_flops(wl):
    """Algorithmic flops of one causal forward (causal half of the intra-chunk products).

    per token: state update 2 d' d_v, inter-chunk read 2 d' d_v (+2 d' for z),
    intra-chunk scores and values (C+1)(d' + d_v) on average, normalisation d_v,
    FAVOR+ projection 2 d_k m for q and for k.  C is the chunk length tiled.
    """
    C, dp, dv, dk = tile_chunk(wl), wl.dprime, wl.dv, wl.dk
    if wl.retention:  # no normaliser: no z read, no division
        per = 4 * dp * dv + (C + 1) * (dp + dv)
    else:
        per = 4 * dp * dv + 2 * dp + (C + 1) * (dp + dv) + dv
    if wl.phi in ("favor", "trig"):
        per += 4 * dk * wl.m
    return wl.B * wl.H * wl.N * per


def backward_alg_flops(wl, kernel):
    """Algorithmic flops of one backward kernel (causal half of the intra-chunk products).

    Per token, with a = d_v + 1 (the value block plus the normaliser column):
      forward-direction pass (dQ): state carry 2 d' a, output recompute 2 d' a +
        (C+1)(d' + a), dphi(q) 2 d' a + (C+1)(a + d'), segment sums 2 d' a;
      reverse-direction pass (dK, dV): dphi(k) from later chunks 2 d' a, dV from
        later chunks 2 d' d_v, in-chunk scores and sums (C+1)(2 d' + d_v + a),
        carry 2 d' a;
    FAVOR+ adds the projection 2 d_k m per recomputed row (q in the first pass,
    k in both) and its Jacobian 2 d_k m + 2 m per row.  C is the chunk length
    the kernels tile: 64 (d 64) or 32 (d 128) tokens on the matrix cores, at
    most 16 tokens on the fp32-arithmetic kernels.
    """
    C, dp, dv, dk = backward_tile(wl), wl.dprime, wl.dv, wl.dk
    a = dv + 1
    if kernel == "dq":
        per = 8 * dp * a + 2 * (C + 1) * (dp + a)
        if wl.phi == "favor":
            per += 2 * 2 * dk * wl.m + 2 * dk * wl.m + 2 * wl.m
    else:
        per = 4 * dp * a + 2 * dp * dv + (C + 1) * (2 * dp + dv + a)
        if wl.phi == "favor":
            per += 2 * 2 * dk * wl.m + 2 * dk * wl.m + 2 * wl.m
    return wl.B * wl.H * wl.N * per


def decode_alg_bytes(wl):
    """Algorithmic bytes of one decode step: S and z read and written once, q, k, v read, o written."""
    e = elem_bytes(wl.dtype)
    slices = wl.B * wl.H
    return slices * (2 * (wl.dprime * wl.dv + wl.dprime) * 4 + (2 * wl.dk + 2 * wl.dv) * e)


class HipEvents:
    """Raw HIP events through the runtime liblinattn is linked against."""

    def __init__(self, lib):
        self.lib = lib
        lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self):
        ev = ctypes.c_void_p()
        rc = self.lib.hipEventCreate(ctypes.byref(ev))
        if rc != 0:
            raise RuntimeError(f"hipEventCreate failed ({rc})")
        return ev

    def record(self, ev, stream):
        if self.lib.hipEventRecord(ev, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, a, b):
        self.lib.hipEventSynchronize(b)
        t = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(t.value)

    def destroy(self, ev):
        self.lib.hipEventDestroy(ev)


def batch_event_ms(hev, stream, launch, steps, batch):
    """Average GPU time per launch over `steps` launches of `launch(i)`, timed by
    one HIP event pair around each batch of `batch` launches queued back to
    back behind a short GPU sleep (all on `stream`)."""
    import torch
    raw = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = hev.create(), hev.create()
    total, done = 0.0, 0
    while done < steps:
        n = min(batch, steps - done)
        with torch.cuda.stream(stream):
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(20_000_000)
            hev.record(e0, raw)
            for i in range(n):
                launch(done + i)
            hev.record(e1, raw)
        torch.cuda.synchronize()
        total += hev.elapsed_ms(e0, e1)
        done += n
    hev.destroy(e0)
    hev.destroy(e1)
    return total / steps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def run_cpu_baseline(wl, fi, seconds):
    """Time the fp64 oracle (causal recurrence) on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    nthreads = oracle.num_threads()
    oracle.set_map(wl.map_param, 0)  # DPFP nu / cosFormer M (0 for the other maps)
    BH = wl.B * wl.H
    if wl.retention:
        # the sample runs over the first heads' slices; their decays, in slice order
        gam_all = np.tile(wl.gammas().astype(np.float64), wl.B)

        def run(Qs, Ks, Vs):  # Qs [1, n, N, d]: n slices as the "heads" of one batch row
            return oracle.retention_recurrent(wl.phi, Qs, Ks, Vs, gam_all[:Qs.shape[1]], W=fi.W)
        form = "retention recurrence"
    else:
        def run(Qs, Ks, Vs):
            return oracle.causal_recurrent(wl.phi, Qs, Ks, Vs, fi.W)
        form = "causal recurrence"
    # per-slice cost estimate from a 1-slice probe, then enough slices for `seconds`
    t0 = time.perf_counter()
    run(fi.Q.f32[:1, :1], fi.K.f32[:1, :1], fi.V.f32[:1, :1])
    t1 = time.perf_counter() - t0
    n_slices = int(max(1, min(BH, round(seconds * nthreads / max(t1, 1e-6)))))
    Qf = fi.Q.f32.reshape(1, BH, wl.N, wl.dk)[:, :n_slices]
    Kf = fi.K.f32.reshape(1, BH, wl.N, wl.dk)[:, :n_slices]
    Vf = fi.V.f32.reshape(1, BH, wl.N, wl.dv)[:, :n_slices]
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(Qf, Kf, Vf)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100000:
            break
    tokens = reps * n_slices * wl.N
    return {"value": tokens / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"fp64 {form} on {n_slices} of {BH} (b,h) slices x {wl.N} tokens, "
                      f"{reps} pass(es), {el:.1f} s on {nthreads} threads of '{cpu_model()}'"}


def run_cpu_baseline_decode(wl, seconds):
    """Time the fp64 oracle's decode step on a bounded sample of sequences (all heads)."""
    import oracle
    from kernelized_linear_attention_la_amd import inputs
    nthreads = oracle.num_threads()
    n_seq = min(wl.B, 8)
    sl = (slice(0, n_seq), slice(None))
    # starting states from the same 1024-token prefix of those sequences (not timed)
    fi = inputs.forward_inputs(wl, batch=(0, n_seq))
    _, S, z = oracle.causal_recurrent(wl.phi, fi.Q.f32, fi.K.f32, fi.V.f32, fi.W)
    steps = []
    for s in range(wl.decode_steps):
        q, k, v = inputs.decode_step_inputs(wl, s)
        steps.append((q.f32[sl][:, :, 0], k.f32[sl][:, :, 0], v.f32[sl][:, :, 0]))
    n = 0
    t0 = time.perf_counter()
    while True:
        q, k, v = steps[n % len(steps)]
        _, S, z = oracle.decode_step(wl.phi, q, k, v, S, z, fi.W)
        n += 1
        el = time.perf_counter() - t0
        if (el >= seconds and n >= len(steps)) or n >= 1000000:
            break
    return {"value": n_seq * n / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"fp64 decode steps for {n_seq} of {wl.B} sequences x {wl.H} heads, {n} steps "
                      f"(64 seeded step inputs cycled, states from the same 1024-token prefix), {el:.1f} s on "
                      f"{nthreads} threads of '{cpu_model()}'"}


def backward_on_mfma(wl):
    """The library runs the backward's two passes on matrix instructions for
    ELU+1 (bf16 or fp32 storage) with d_k = d_v = 64 and 64-token chunks, or
    d_k = d_v = 128 and chunks of a multiple of 32 tokens (run on 32-token
    tiles): fp32 products for fp32 storage, fp32 operands split into bf16 hi
    and lo parts (one to three bf16 passes per k step: the lo pass of an
    operand exact in bf16 is skipped) for bf16 storage."""
    if wl.dtype not in ("bf16", "f32") or wl.phi != "elu1" or wl.dk != wl.dv:
        return False
    return (wl.dk == 64 and wl.chunk == 64) or (wl.dk == 128 and wl.chunk % 32 == 0)


def backward_tile(wl):
    """Tokens per tile of the backward kernels that run this workload."""
    if backward_on_mfma(wl):
        return 64 if wl.dk == 64 else 32
    return min(wl.chunk, 16)


def gla_on_chunks(wl):
    """GLA in chunkwise form on fp32 matrix instructions (d_k <= 64): the three-launch entry point."""
    return wl.gated == "gla" and wl.dk <= 64


def delta_on_chunks(wl):
    """The library runs the gated delta rule in chunkwise form for d_k = 64, d_v a multiple of 16 up to 128."""
    return wl.gated == "delta" and wl.dk == 64 and wl.dv % 16 == 0 and 16 <= wl.dv <= 128


def kernel_symbol(wl, slot):
    """rocprofv3 name of the kernel a slot runs for this workload (labels only)."""
    if wl.backward:
        if backward_on_mfma(wl) and slot in ("dq", "dkv"):
            return f"k_bwd_{slot}_mfma<{wl.dk}, {backward_tile(wl)}, {'float' if wl.dtype == 'f32' else 'unsigned short'}>"
        return f"k_bwd_{slot}<{'float' if wl.dtype == 'f32' else 'unsigned short'}>"
    if wl.gated:
        t = "float" if wl.dtype == "f32" else "unsigned short"
        if delta_on_chunks(wl):
            return f"k_delta_prep<{t}, {64 if wl.dv <= 64 else 128}>"  # the longest of the chunkwise form's launches
        if gla_on_chunks(wl):
            return f"k_gla_prep<{t}>"  # the longest of the chunkwise form's three launches
        return f"k_gated<{t}, {'true' if wl.gated == 'gla' else 'false'}>"
    if wl.decode_steps and slot == "decode":
        t = "float" if wl.dtype == "f32" else "unsigned short"
        return f"k_decode<{t}, {4 if wl.dv % 4 == 0 else 1}, {'true' if wl.retention else 'false'}>"
    mode = {"state": 0, "chunk": 1}[slot]
    square = wl.dk == wl.dv and wl.dk in (64, 128) and wl.chunk in (64, 128)
    mfma = wl.dtype == "bf16" and (
        (wl.phi == "elu1" and not wl.retention and square) or
        (wl.phi == "identity" and wl.retention and square) or
        (wl.phi == "favor" and not wl.retention and wl.dk == 64 and wl.dv == 64 and wl.m == 256 and
         tile_chunk(wl) == 64) or
        (wl.phi == "cosformer" and not wl.retention and wl.dk == 64 and wl.dv == 64 and tile_chunk(wl) == 64) or
        (wl.phi == "dpfp" and not wl.retention and wl.dk == 64 and wl.dv == 64 and tile_chunk(wl) == 64 and
         wl.map_param == 1) or
        (wl.phi == "trig" and not wl.retention and wl.dk == 64 and wl.dv == 64 and wl.m == 64 and tile_chunk(wl) == 64))
    if mfma:
        # the forward workloads all split into several segments per slice: the
        # matrix-core path runs them in one single-pass launch (the library's
        # plan: about 256 workgroups, whole chunks per segment): the
        # whole-segment kernel at d 64 with segments of at most 256 tokens,
        # else the chunk loop, mode 4 when a segment's keys and values stay in
        # LDS (d 64, 64-token chunks, at most 4 chunks per segment), else mode 3
        phi_id = {"elu1": 0, "favor": 1, "identity": 2, "dpfp": 3, "trig": 4, "cosformer": 5}[wl.phi]
        n_chunks = -(-wl.N // tile_chunk(wl))
        P = min(-(-256 // (wl.B * wl.H)), n_chunks)
        seg = -(-n_chunks // P)
        if P > 1 and seg * wl.chunk <= 256 and wl.dk == 64 and wl.dv == 64 and wl.phi in ("elu1", "identity"):
            return f"k_seg<{phi_id}>"  # a whole segment (at most 256 tokens) per 16-wave workgroup
        if P > 1 and wl.phi == "favor":
            return "k_favor"  # eight waves per workgroup, two per SIMD
        res = seg <= 4 and wl.dk == 64 and wl.dv == 64 and wl.chunk == 64 and wl.phi in ("elu1", "identity")
        return f"k_mfma<{wl.dk}, {wl.dv}, {tile_chunk(wl)}, {phi_id}, {4 if res else 3}>"
    if (wl.dtype == "f32" and ((wl.phi == "elu1" and not wl.retention) or (wl.phi == "identity" and wl.retention))
            and wl.dk == wl.dv and wl.dk in (64, 128)):
        # fp32 storage on fp32 matrix instructions (ELU+1, or retention's identity map)
        return f"k_f32mma<{wl.dk}, {mode}, {'true' if wl.retention else 'false'}>"
    return f"k_generic<{'float' if wl.dtype == 'f32' else 'unsigned short'}, {mode}>"


def stored_traffic(wl, kernel):
    """HBM bytes per launch from a committed counter summary, if the kernels are unchanged since."""
    import glob
    from kernelized_linear_attention_la_amd import build as hip_build
    want = hip_build.source_hash(kernel)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))):
        try:
            with open(path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            continue
        if rec.get("workload") == wl.name and rec.get("kernel") == kernel and rec.get("source_hash") == want:
            return rec.get("bytes_per_launch")
    return None


def bench_forward(args, wl):
    import torch
    from kernelized_linear_attention_la_amd import inputs
    from kernelized_linear_attention_la_amd import linattn as la

    fi = inputs.forward_inputs(wl)
    dev = torch.device("cuda:0")

    def to_dev(ht):
        t = torch.from_numpy(ht.store)
        return (t.view(torch.bfloat16) if ht.dtype == "bf16" else t).to(dev)

    q0, k0, v0 = to_dev(fi.Q), to_dev(fi.K), to_dev(fi.V)
    W = torch.from_numpy(fi.W).to(dev) if fi.W is not None else None
    gam = torch.from_numpy(wl.gammas()).to(dev) if wl.retention else None
    set_bytes = 2 * q0.nbytes + k0.nbytes + 2 * v0.nbytes
    R = max(1, min(64, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = [(q0.clone(), k0.clone(), v0.clone(), torch.empty_like(v0)) for _ in range(R)]
    S = torch.zeros(wl.B, wl.H, wl.dprime, wl.dv, device=dev)
    z = torch.zeros(wl.B, wl.H, wl.dprime, device=dev)
    p = la._problem_of(q0, v0, wl.phi, W, wl.map_param)
    ws = torch.zeros(max(1, la.la_workspace_bytes(p, wl.chunk)), dtype=torch.uint8, device=dev)

    def step(i, stream=None, events=None):
        q, k, v, o = sets[i % R]
        if wl.retention:
            la.la_forward_retention_chunked(q, k, v, gam, wl.chunk, phi=wl.phi, W=W, S_out=S, out=o, workspace=ws,
                                            stream=stream, events=events)
        else:
            la.la_forward_causal_chunked(q, k, v, wl.chunk, phi=wl.phi, W=W, S_out=S, z_out=z, out=o,
                                         workspace=ws, stream=stream, events=events, map_param=wl.map_param)

    # the step sequence is launch-bound at small sizes: capture it in HIP graphs
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(R):  # eager warm-up on the capture stream
            step(i)
    torch.cuda.synchronize()
    # one graph replays all R rotated input sets back to back (launch cost is
    # paid once per R steps); a second graph covers the K mod R remainder
    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                step(i)
        return g

    g_all = capture(R)
    rem = args.steps % R
    g_rem = capture(rem) if rem else None
    torch.cuda.synchronize()

    for _ in range(max(1, args.warmup // R)):
        g_all.replay()
    torch.cuda.synchronize()
    # the timed loop, bracketed by one HIP event pair on the stream the graphs
    # are launched on (the current stream)
    hev = HipEvents(la.lib())
    loop_raw = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    loop_e0, loop_e1 = hev.create(), hev.create()
    t0 = time.perf_counter()
    hev.record(loop_e0, loop_raw)
    for _ in range(args.steps // R):
        g_all.replay()
    if g_rem is not None:
        g_rem.replay()
    hev.record(loop_e1, loop_raw)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    loop_gpu_ms = hev.elapsed_ms(loop_e0, loop_e1) / args.steps
    hev.destroy(loop_e0)
    hev.destroy(loop_e1)

    # live per-kernel timing over K steps: HIP events recorded around each
    # kernel of the step (timing hook), inside HIP graphs like the timed loop
    slots = (la.LA_KSLOT_STATE, la.LA_KSLOT_SCAN, la.LA_KSLOT_CHUNK)
    ev = [{sl: (hev.create(), hev.create()) for sl in slots} for _ in range(R)]
    kevs = []
    for i in range(R):
        kev = la.LaKernelEvents()
        for sl in slots:
            kev.start[sl], kev.stop[sl] = ev[i][sl][0], ev[i][sl][1]
        kevs.append(kev)
    durs = {sl: [] for sl in slots}
    torch.cuda.synchronize()
    # Launches are queued behind a short GPU sleep so the device runs them
    # back to back, as in the graph-timed loop; each event pair then brackets
    # exactly one kernel on the GPU timeline.
    done = 0
    while done < args.steps:
        n = min(R, args.steps - done)
        with torch.cuda.stream(stream):
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(20_000_000)
            for i in range(n):
                step(done + i, stream=stream, events=kevs[i])
        torch.cuda.synchronize()
        for i in range(n):
            for sl in slots:
                if kevs[i].launched[sl]:
                    durs[sl].append(hev.elapsed_ms(*ev[i][sl]))
        done += n
    timing_mode = "hip events around each kernel, launches queued back to back"
    for e in ev:
        for a_, b_ in e.values():
            hev.destroy(a_)
            hev.destroy(b_)
    avg_us = {sl: 1e3 * sum(v) / len(v) for sl, v in durs.items() if v}
    if list(avg_us) == [la.LA_KSLOT_CHUNK]:
        # a step of one kernel (the single pass): its time is the timed loop's
        # GPU time per step, so the markers of a per-launch event pair (several
        # µs per launch) do not count as kernel time
        avg_us[la.LA_KSLOT_CHUNK] = 1e3 * loop_gpu_ms
        timing_mode = "hip events around the graph-replayed timed loop (one kernel per step)"
    kern_ms = avg_us[la.LA_KSLOT_CHUNK] * 1e-3

    tokens = wl.B * wl.H * wl.N
    value = tokens / (ms_per_step * 1e-3)
    alg_bytes = forward_alg_bytes(wl)
    alg_flops = forward_alg_flops(wl)
    # chunk kernel's algorithmic bytes: Q, K, V read, O written (state traffic excluded)
    chunk_bytes = tokens * (2 * wl.dk + 2 * wl.dv) * elem_bytes(wl.dtype)
    flop_per_byte = alg_flops / alg_bytes
    ridge = MFMA_BF16_PEAK_TFS * 1e12 / (HBM_PEAK_GBS * 1e9)
    kname = kernel_symbol(wl, "chunk")
    if kname.startswith("k_f32mma"):
        # fp32 storage: fp32 arithmetic on the matrix cores, against the dense fp32 MFMA peak
        ach = alg_flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_F32_PEAK_TFS, "unit": "TFLOP/s",
                "frac": ach / MFMA_F32_PEAK_TFS, "traffic": None}
    elif kname.startswith("k_generic"):
        # fp32-arithmetic kernels: against the fp32 vector ALUs
        ach = alg_flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "alu", "achieved": ach, "peak": FP32_VECTOR_PEAK_TFS, "unit": "TFLOP/s",
                "frac": ach / FP32_VECTOR_PEAK_TFS, "traffic": None}
    elif flop_per_byte < ridge:
        ach = chunk_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": None}
    else:
        ach = alg_flops / (kern_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": ach / MFMA_BF16_PEAK_TFS, "traffic": None}
    tb = stored_traffic(wl, kname)
    roof["traffic"] = tb
    roof["kernel"] = kname
    roof["kernel_avg_us"] = kern_ms * 1e3
    roof["alg_bytes_per_launch"] = chunk_bytes
    roof["timing"] = timing_mode
    extra = {
        # three-pass path: state sums, scan, chunk loop; single-pass path:
        # flag reset, then the one forward kernel
        "kernel_avg_us": {name: round(avg_us[sl], 2) for name, sl in
                          ((("state", la.LA_KSLOT_STATE), ("scan", la.LA_KSLOT_SCAN), ("chunk", la.LA_KSLOT_CHUNK))
                           if la.LA_KSLOT_STATE in avg_us else
                           (("flag_reset", la.LA_KSLOT_SCAN), ("single_pass", la.LA_KSLOT_CHUNK)))
                          if sl in avg_us},
        "step_hbm_frac": alg_bytes / (ms_per_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "step_mfma_frac": alg_flops / (ms_per_step * 1e-3) / (MFMA_BF16_PEAK_TFS * 1e12),
        "rotated_input_sets": R,
    }
    return value, ms_per_step, roof, extra, fi


def bench_backward(args, wl):
    """One step = la_backward_causal_chunked over the whole batch (forward prefix
    sums and scan, dQ pass, reverse scan, dK/dV pass)."""
    import torch
    from kernelized_linear_attention_la_amd import inputs
    from kernelized_linear_attention_la_amd import linattn as la

    fi = inputs.forward_inputs(wl)
    dO_h = inputs.grad_output(wl.wid, wl.B, wl.H, wl.N, wl.dv, wl.dtype)
    dev = torch.device("cuda:0")

    def to_dev(ht):
        t = torch.from_numpy(ht.store)
        return (t.view(torch.bfloat16) if ht.dtype == "bf16" else t).to(dev)

    q0, k0, v0, g0 = to_dev(fi.Q), to_dev(fi.K), to_dev(fi.V), to_dev(dO_h)
    W = torch.from_numpy(fi.W).to(dev) if fi.W is not None else None
    set_bytes = 2 * q0.nbytes + 2 * k0.nbytes + 2 * v0.nbytes + g0.nbytes
    R = max(1, min(32, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = [(q0.clone(), k0.clone(), v0.clone(), g0.clone(), torch.empty_like(q0), torch.empty_like(k0),
             torch.empty_like(v0)) for _ in range(R)]
    p = la._problem_of(q0, v0, wl.phi, W)
    ws = torch.empty(la.la_backward_workspace_bytes(p, wl.chunk), dtype=torch.uint8, device=dev)

    def step(i, stream=None, events=None):
        q, k, v, g, dq, dk, dv = sets[i % R]
        la.la_backward_causal_chunked(q, k, v, g, wl.chunk, phi=wl.phi, W=W, dQ=dq, dK=dk, dV=dv, workspace=ws,
                                      stream=stream, events=events)

    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for i in range(R):
            step(i)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        with torch.cuda.stream(stream):
            step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps

    hev = HipEvents(la.lib())
    slots = (la.LA_BSLOT_FWD_SUMS, la.LA_BSLOT_FWD_SCAN, la.LA_BSLOT_DQ, la.LA_BSLOT_RSCAN, la.LA_BSLOT_DKV)
    durs = {sl: [] for sl in slots}
    ev = [{sl: (hev.create(), hev.create()) for sl in slots} for _ in range(R)]
    kevs = []
    for i in range(R):
        kev = la.LaBackwardEvents()
        for sl in slots:
            kev.start[sl], kev.stop[sl] = ev[i][sl][0], ev[i][sl][1]
        kevs.append(kev)
    done = 0
    while done < args.steps:
        n = min(R, args.steps - done)
        with torch.cuda.stream(stream):
            if hasattr(torch.cuda, "_sleep"):
                torch.cuda._sleep(20_000_000)
            for i in range(n):
                step(done + i, stream=stream, events=kevs[i])
        torch.cuda.synchronize()
        for i in range(n):
            for sl in slots:
                if kevs[i].launched[sl]:
                    durs[sl].append(hev.elapsed_ms(*ev[i][sl]))
        done += n
    for e in ev:
        for a_, b_ in e.values():
            hev.destroy(a_)
            hev.destroy(b_)
    avg_us = {sl: 1e3 * sum(v) / len(v) for sl, v in durs.items() if v}
    which = "dq" if avg_us[la.LA_BSLOT_DQ] >= avg_us[la.LA_BSLOT_DKV] else "dkv"
    kern_ms = avg_us[la.LA_BSLOT_DQ if which == "dq" else la.LA_BSLOT_DKV] * 1e-3
    flops = backward_alg_flops(wl, which)
    ach = flops / (kern_ms * 1e-3) / 1e12
    kname = kernel_symbol(wl, which)
    # fp32-class products either way: on the matrix cores (fp32 instructions, or bf16 hi/lo passes
    # that keep about 2^-16 of an fp32 product; priced at the dense fp32 MFMA peak) or in fp32 FMAs
    bound = "mfma" if backward_on_mfma(wl) else "alu"
    peak = MFMA_F32_PEAK_TFS if bound == "mfma" else FP32_VECTOR_PEAK_TFS
    roof = {"bound": bound, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
            "frac": ach / peak, "traffic": stored_traffic(wl, kname), "kernel": kname,
            "kernel_avg_us": kern_ms * 1e3, "alg_flops_per_launch": flops,
            "timing": "hip events around each kernel, launches queued back to back"}
    names = {la.LA_BSLOT_FWD_SUMS: "fwd_sums", la.LA_BSLOT_FWD_SCAN: "fwd_scan", la.LA_BSLOT_DQ: "dq",
             la.LA_BSLOT_RSCAN: "rscan", la.LA_BSLOT_DKV: "dkv"}
    tokens = wl.B * wl.H * wl.N
    extra = {"kernel_avg_us": {names[sl]: round(v, 2) for sl, v in avg_us.items()},
             "rotated_input_sets": R,
             "step_hbm_frac": tokens * (3 * wl.dk + 4 * wl.dv) * elem_bytes(wl.dtype) / (ms_per_step * 1e-3) /
             (HBM_PEAK_GBS * 1e9)}
    return tokens / (ms_per_step * 1e-3), ms_per_step, roof, extra, (fi, dO_h)


def gated_alg_flops(wl):
    """Flops of one token-by-token pass: per token GLA updates S (2 d_k d_v) and
    reads S^T q (2 d_k d_v); the gated delta rule adds S^T k (2 d_k d_v) and its
    update costs 3 d_k d_v (scale, scale, add)."""
    per = 4 * wl.dk * wl.dv if wl.gated == "gla" else 7 * wl.dk * wl.dv
    return wl.B * wl.H * wl.N * per


def bench_gated(args, wl):
    """One step = one gated recurrence over the whole batch (every (b, h) slice, all N tokens)."""
    import numpy as np
    import torch
    from kernelized_linear_attention_la_amd import inputs
    from kernelized_linear_attention_la_amd import linattn as la

    gi = inputs.gated_inputs(wl.wid, wl.B, wl.H, wl.N, wl.dk, wl.dv, wl.dtype)
    dev = torch.device("cuda:0")

    def to_dev(ht):
        t = torch.from_numpy(ht.store)
        return (t.view(torch.bfloat16) if ht.dtype == "bf16" else t).to(dev)

    q, k, v = to_dev(gi.Q), to_dev(gi.K), to_dev(gi.V)
    a_ch = torch.from_numpy(np.ascontiguousarray(gi.alpha_ch)).to(dev)
    al, be = torch.from_numpy(gi.alpha).to(dev), torch.from_numpy(gi.beta).to(dev)
    S = torch.zeros(wl.B, wl.H, wl.dk, wl.dv, device=dev)
    o = torch.empty_like(v)
    raw = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    chunked = delta_on_chunks(wl) or gla_on_chunks(wl)
    ws = None
    if chunked:
        nbytes = la.la_gla_workspace_bytes(q, v) if wl.gated == "gla" else la.la_delta_workspace_bytes(q, v)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)

    def step(events=None):
        if wl.gated == "gla" and chunked:
            la.la_forward_gla_chunked(q, k, v, a_ch, S_out=S, out=o, workspace=ws, events=events)
        elif wl.gated == "gla":
            la.la_forward_gla_recurrent(q, k, v, a_ch, S_out=S, out=o)
        elif chunked:
            la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_out=S, out=o, workspace=ws, events=events)
        else:
            la.la_forward_delta_recurrent(q, k, v, be, alpha=al, S_out=S, out=o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hev = HipEvents(la.lib())
    # the K timed steps: launches only, back to back on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # per-call time: HIP events around each call in batches of EVENT_BATCH,
    # queued behind a short GPU sleep (as for decode)
    pairs = [(hev.create(), hev.create()) for _ in range(EVENT_BATCH)]
    durs = []
    done = 0
    while done < args.steps:
        n = min(EVENT_BATCH, args.steps - done)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)
        for i in range(n):
            hev.record(pairs[i][0], raw)
            step()
            hev.record(pairs[i][1], raw)
        torch.cuda.synchronize()
        durs += [hev.elapsed_ms(*pairs[i]) for i in range(n)]
        done += n
    for a_, b_ in pairs:
        hev.destroy(a_)
        hev.destroy(b_)
    kern_ms = sum(durs) / len(durs)
    extra = {"per_token_latency_ns": kern_ms * 1e6 / wl.N}
    if chunked:
        # the launches of the chunkwise form timed one by one through the
        # library's hook: the per-chunk products (GLA) or operators (delta
        # rule), the state chain over chunks, the outputs of every chunk
        names = ({la.LA_KSLOT_STATE: "k_gla_prep", la.LA_KSLOT_SCAN: "k_gla_chain", la.LA_KSLOT_CHUNK: "k_gla_out"}
                 if wl.gated == "gla" else
                 {la.LA_KSLOT_STATE: "k_delta_prep", la.LA_KSLOT_SCAN: "k_delta_scan", la.LA_KSLOT_CHUNK: "k_delta_out"})
        slots = tuple(names)
        kd = {sl: [] for sl in slots}
        for _ in range(args.steps):
            kev = la.LaKernelEvents()
            ev = {sl: (hev.create(), hev.create()) for sl in slots}
            for sl in slots:
                kev.start[sl], kev.stop[sl] = ev[sl]
            step(events=kev)
            torch.cuda.synchronize()
            for sl in slots:
                if kev.launched[sl]:  # only the slots whose kernel the call enqueued
                    kd[sl].append(hev.elapsed_ms(*ev[sl]))
                hev.destroy(ev[sl][0])
                hev.destroy(ev[sl][1])
        extra = {"kernel_avg_us": {names[sl]: round(1e3 * sum(kd[sl]) / len(kd[sl]), 2) for sl in slots if kd[sl]},
                 "step_kernels_us": round(kern_ms * 1e3, 2)}
    flops = gated_alg_flops(wl)
    ach = flops / (kern_ms * 1e-3) / 1e12
    kname = ("k_gla_prep + k_gla_chain + k_gla_out" if wl.gated == "gla" else "k_delta_prep + k_delta_scan + k_delta_out") \
        if chunked else kernel_symbol(wl, "chunk")
    # fp32 arithmetic: the chunkwise forms on the matrix cores (dense fp32 MFMA peak),
    # the token-by-token recurrences in fp32 FMAs; the flops are the recurrence's own,
    # over the step's kernels (every launch of the chunkwise forms)
    bound = "mfma" if chunked else "alu"
    peak = MFMA_F32_PEAK_TFS if bound == "mfma" else FP32_VECTOR_PEAK_TFS
    roof = {"bound": bound, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
            "frac": ach / peak, "traffic": None if chunked else stored_traffic(wl, kname), "kernel": kname,
            "kernel_avg_us": kern_ms * 1e3, "alg_flops_per_launch": flops,
            "timing": "hip events around each call (every launch of the chunkwise form)"}
    tokens = wl.B * wl.H * wl.N
    return tokens / (ms_per_step * 1e-3), ms_per_step, roof, extra, gi


def run_cpu_baseline_gated(wl, gi, seconds):
    """Time the fp64 oracle's recurrence on a sample of slices."""
    import oracle
    nthreads = oracle.num_threads()
    BH = wl.B * wl.H
    r4 = lambda x, d: x.reshape(1, BH, wl.N, d)  # noqa: E731
    Q, K, V = r4(gi.Q.f32, wl.dk), r4(gi.K.f32, wl.dk), r4(gi.V.f32, wl.dv)
    ach, al, be = r4(gi.alpha_ch, wl.dk), gi.alpha.reshape(1, BH, wl.N), gi.beta.reshape(1, BH, wl.N)

    def run(n):
        if wl.gated == "gla":
            oracle.gla_recurrent(Q[:, :n], K[:, :n], V[:, :n], ach[:, :n])
        else:
            oracle.delta_recurrent(Q[:, :n], K[:, :n], V[:, :n], be[:, :n], alpha=al[:, :n])
    t0 = time.perf_counter()
    run(1)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(BH, round(seconds * nthreads / max(t1, 1e-6)))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(n)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100000:
            break
    return {"value": reps * n * wl.N / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"fp64 {wl.gated} recurrence on {n} of {BH} (b,h) slices x {wl.N} tokens, {reps} pass(es), "
                      f"{el:.1f} s on {nthreads} threads of '{cpu_model()}'"}


def run_cpu_baseline_backward(wl, fi, dO_h, seconds):
    """Time the fp64 oracle's backward (reverse-mode through the recurrence) on a sample of slices."""
    import oracle
    nthreads = oracle.num_threads()
    BH = wl.B * wl.H
    shp = lambda x, d: x.reshape(1, BH, wl.N, d)  # noqa: E731
    Q, K, V, G = shp(fi.Q.f32, wl.dk), shp(fi.K.f32, wl.dk), shp(fi.V.f32, wl.dv), shp(dO_h.f32, wl.dv)
    t0 = time.perf_counter()
    oracle.causal_backward(wl.phi, Q[:, :1], K[:, :1], V[:, :1], G[:, :1], W=fi.W)
    t1 = time.perf_counter() - t0
    n = int(max(1, min(BH, round(seconds * nthreads / max(t1, 1e-6)))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.causal_backward(wl.phi, Q[:, :n], K[:, :n], V[:, :n], G[:, :n], W=fi.W)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 100000:
            break
    return {"value": reps * n * wl.N / el, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "sample": f"fp64 backward through the recurrence on {n} of {BH} (b,h) slices x {wl.N} tokens, "
                      f"{reps} pass(es), {el:.1f} s on {nthreads} threads of '{cpu_model()}'"}


def bench_decode(args, wl):
    import torch
    from kernelized_linear_attention_la_amd import inputs
    from kernelized_linear_attention_la_amd import linattn as la

    dev = torch.device("cuda:0")

    def to_dev(ht):
        t = torch.from_numpy(ht.store)
        return (t.view(torch.bfloat16) if ht.dtype == "bf16" else t).to(dev)

    S = torch.zeros(wl.B, wl.H, wl.dprime, wl.dv, device=dev)
    z = torch.zeros(wl.B, wl.H, wl.dprime, device=dev)
    # the prefix (not timed), drawn and run a block of sequences at a time:
    # every (sequence, head) slice is independent and its values do not
    # depend on the block
    hev = HipEvents(la.lib())
    prefix_ms = 0.0
    raw = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for b0 in range(0, wl.B, PREFIX_BLOCK):
        b1 = min(wl.B, b0 + PREFIX_BLOCK)
        fb = inputs.forward_inputs(wl, batch=(b0, b1))
        q, k, v = to_dev(fb.Q), to_dev(fb.K), to_dev(fb.V)
        e0, e1 = hev.create(), hev.create()
        hev.record(e0, raw)
        la.la_forward_causal_chunked(q, k, v, wl.chunk, S_out=S[b0:b1], z_out=z[b0:b1])
        hev.record(e1, raw)
        prefix_ms += hev.elapsed_ms(e0, e1)  # synchronises on e1
        hev.destroy(e0)
        hev.destroy(e1)
        del q, k, v, fb
    steps_in = []
    for s in range(wl.decode_steps):
        qs, ks, vs = inputs.decode_step_inputs(wl, s)
        steps_in.append((to_dev(qs), to_dev(ks), to_dev(vs)))
    o = torch.empty(wl.B, wl.H, 1, wl.dv, device=dev, dtype=steps_in[0][0].dtype)
    stream = torch.cuda.current_stream()

    def step(i):
        qs, ks, vs = steps_in[i % len(steps_in)]
        la.la_decode_step(qs, ks, vs, S, z, phi=wl.phi, out=o)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the K timed steps: launches only, back to back on the stream
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    # kernel time over K more steps: one HIP event pair around each batch of
    # EVENT_BATCH back-to-back launches (a step is one kernel).  Hundreds of
    # outstanding per-launch events at once have stretched both the events and
    # the host's enqueue rate on this runtime while the kernel trace showed
    # unchanged kernels, and a per-launch pair adds its markers' time.
    kern_ms = batch_event_ms(hev, stream, lambda i: step(args.warmup + args.steps + i), args.steps, EVENT_BATCH)
    value = wl.B / (ms_per_step * 1e-3)  # one generated token per sequence per step
    nbytes = decode_alg_bytes(wl)
    ach = nbytes / (kern_ms * 1e-3) / 1e9
    kname = kernel_symbol(wl, "decode")
    roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
            "traffic": stored_traffic(wl, kname), "kernel": kname, "kernel_avg_us": kern_ms * 1e3,
            "alg_bytes_per_launch": nbytes, "timing": "hip events around batches of 64 back-to-back launches"}
    extra = {"head_steps_per_s": wl.B * wl.H / (ms_per_step * 1e-3),
             # the state-building prefix (not part of the step): fp32 causal forward over every
             # sequence, summed over the blocks it is run in, timed by HIP events around each call
             "prefix_forward_ms": prefix_ms,
             "prefix_forward_kernel": kernel_symbol(wl, "chunk")}
    return value, ms_per_step, roof, extra, None


def measure_extras(args):
    """The metric's other halves, measured in the same run as the headline:
    decode tokens/s with its HBM fraction (c4), and the FAVOR+ chunked forward
    with its bf16 matrix-core fraction (c5), each kernel timed by HIP events."""
    import torch
    from kernelized_linear_attention_la_amd import inputs
    # at least 100 ms of timed work each (decode ~0.2 ms, FAVOR+ ~0.07 ms per
    # step) after 10 warm-up steps; the first graph launch's latency inside a
    # timed loop is then well under 1% of it
    dec_args = argparse.Namespace(steps=max(1, args.steps), warmup=max(1, min(args.warmup, 10)))
    fav_args = argparse.Namespace(steps=max(1, 3 * args.steps), warmup=max(1, min(args.warmup, 10)))
    out = {}
    wl = inputs.WORKLOADS[EXTRA_DECODE]
    value, ms, roof, dex, _ = bench_decode(dec_args, wl)
    out["decode"] = {"workload": wl.name, "tokens_per_s": value, "ms_per_step": ms, "steps": dec_args.steps,
                     "prefix_forward_ms": dex["prefix_forward_ms"], "prefix_forward_kernel": dex["prefix_forward_kernel"],
                     "kernel": roof["kernel"], "kernel_avg_us": roof["kernel_avg_us"],
                     "hbm_achieved_GBps": roof["achieved"], "hbm_frac": roof["frac"], "traffic": roof["traffic"],
                     "alg_bytes_per_launch": roof["alg_bytes_per_launch"]}
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    wl = inputs.WORKLOADS[EXTRA_FAVOR]
    value, ms, roof, ex, _ = bench_forward(fav_args, wl)
    kern_s = roof["kernel_avg_us"] * 1e-6
    flops = forward_alg_flops(wl)
    out["favor"] = {"workload": wl.name, "tokens_per_s": value, "ms_per_step": ms, "steps": fav_args.steps,
                    "kernel": roof["kernel"], "kernel_avg_us": roof["kernel_avg_us"],
                    "alg_flops_per_launch": flops,
                    "mfma_achieved_TFs": flops / kern_s / 1e12,
                    "mfma_frac": flops / kern_s / (MFMA_BF16_PEAK_TFS * 1e12),
                    "hbm_frac": roof["alg_bytes_per_launch"] / kern_s / (HBM_PEAK_GBS * 1e9),
                    "traffic": roof["traffic"]}
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=600)  # >= 100 ms of timed work on the long-context workload
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing budget; 0 skips it")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the decode and FAVOR+ figures measured after the default workload")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path would shard over "
              f"(batch, head) slices, or over sequence segments with one exchange of segment states)",
              file=sys.stderr)
        sys.exit(2)
    from kernelized_linear_attention_la_amd import inputs
    if args.workload not in inputs.WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(inputs.WORKLOADS)}")
    wl = inputs.WORKLOADS[args.workload]
    import torch
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if wl.decode_steps:
        value, ms, roof, extra, fi = bench_decode(args, wl)
        metric = "decode tokens/s"
    elif wl.backward:
        value, ms, roof, extra, fi = bench_backward(args, wl)
        metric = "causal linear-attn bwd tokens/s (B*H*N/s)"
    elif wl.gated:
        value, ms, roof, extra, fi = bench_gated(args, wl)
        metric = ("GLA recurrence tokens/s (B*H*N/s)" if wl.gated == "gla"
                  else "gated delta-rule tokens/s (B*H*N/s)")
    else:
        value, ms, roof, extra, fi = bench_forward(args, wl)
        metric = ("causal retention fwd tokens/s (B*H*N/s)" if wl.retention
                  else "causal linear-attn fwd tokens/s (B*H*N/s)")
    cpu = None
    if args.cpu_seconds > 0:
        if wl.decode_steps:
            cpu = run_cpu_baseline_decode(wl, args.cpu_seconds)
        elif wl.backward:
            cpu = run_cpu_baseline_backward(wl, fi[0], fi[1], args.cpu_seconds)
        elif wl.gated:
            cpu = run_cpu_baseline_gated(wl, fi, args.cpu_seconds)
        else:
            cpu = run_cpu_baseline(wl, fi, args.cpu_seconds)
    config = {"workload": wl.name, "phi": wl.phi, "B": wl.B, "H": wl.H, "N": wl.N, "d_k": wl.dk, "d_v": wl.dv,
              "chunk": wl.chunk}
    if tile_chunk(wl) != wl.chunk:
        config["tile_chunk"] = tile_chunk(wl)
    if wl.m:
        config["m"] = wl.m
    if wl.retention:
        config["decay_per_head"] = [float(x) for x in wl.gammas()]
    if wl.decode_steps:
        config.update({"prefix": wl.N, "decode_steps_cycled": wl.decode_steps})
    if args.workload == DEFAULT_WORKLOAD and not args.no_extras:
        # the headline metric: causal forward tokens/s with its matrix-core
        # fraction, decode tokens/s with its HBM fraction (under extra)
        extra.update(measure_extras(args))
        metric = "causal linear-attn fwd tokens/s (B\u00b7H\u00b7N/s) + % MFMA peak; decode tokens/s + % HBM BW"
    line = {"metric": metric, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
            "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded i.i.d. Gaussian)",
            "config": config, "roofline": roof, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
