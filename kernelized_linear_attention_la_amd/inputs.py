"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws random numbers and rounds them to the storage precision of
each workload. It holds none of the attention arithmetic: the HIP library and
the fp64 oracle both receive exactly the values produced here.

Recipe (every workload):
  * one numpy ``Generator(PCG64)`` per (workload, tensor, b, h[, step]) slice,
    seeded with ``SeedSequence([workload_id, tensor_id, b, h(, step)])``;
  * draw fp64 standard normals, multiply by the workload's scale in fp64,
    round to fp32 (round-to-nearest-even), and for bf16 workloads round the
    fp32 value once more to bf16 (round-to-nearest-even);
  * tensor ids: Q=0, K=1, V=2, W=3, decode q=4, k=5, v=6, and for the
    backward dO=7, dS_out=8, dz_out=9, S_in=10, z_in=11; gated states: GLA gate
    12, scalar gate 13, write strength 14.

The FAVOR+ projection W (m rows of dimension d) is an *input*: the random
features of the Performer map are drawn here once and handed to both sides.
Rows come in blocks of d mutually orthogonal directions (QR of a Gaussian
d x d matrix with the sign of R's diagonal folded in), each row rescaled to
the length of an independent N(0, I_d) draw, so every row keeps the N(0, I_d)
marginal the Performer map assumes while rows within a block are orthogonal
(Story of Attention Part 5, section 1b).
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field

import numpy as np

TENSOR_Q, TENSOR_K, TENSOR_V, TENSOR_W = 0, 1, 2, 3
TENSOR_QSTEP, TENSOR_KSTEP, TENSOR_VSTEP = 4, 5, 6
TENSOR_DO, TENSOR_DS, TENSOR_DZ, TENSOR_SIN, TENSOR_ZIN = 7, 8, 9, 10, 11
TENSOR_GATE_CH, TENSOR_GATE, TENSOR_BETA = 12, 13, 14


# ---------------------------------------------------------------------------
# rounding helpers (storage formats, not attention arithmetic)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounding = ((u >> 16) & 1) + 0x7FFF
    out = ((u + rounding) >> 16).astype(np.uint16)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they encode (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class HostTensor:
    """A seeded tensor in its storage format plus its exact fp32 value.

    ``store`` is what the device receives (fp32 values, or uint16 bf16 bits);
    ``f32`` is the same set of numbers as fp32, which the oracle widens to
    fp64 without any rounding.
    """
    store: np.ndarray
    f32: np.ndarray
    dtype: str  # "f32" or "bf16"

    @property
    def shape(self):
        return self.f32.shape


def _round_to(x64: np.ndarray, dtype: str) -> HostTensor:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return HostTensor(store=x32, f32=x32, dtype="f32")
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return HostTensor(store=bits, f32=bf16_bits_to_f32(bits), dtype="bf16")
    raise ValueError(f"unknown dtype {dtype!r}")


def _slice_draw(key, n):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))
    return rng.standard_normal(n)


def _fill_slices(shm_name, shape, key_prefix, scale, lo, hi, b0=0):
    """Worker body: draw slices [lo, hi) into a shared fp32 buffer."""
    from multiprocessing import resource_tracker, shared_memory
    shm = shared_memory.SharedMemory(name=shm_name)
    # the creating process owns the segment; this worker must not unlink it at exit
    resource_tracker.unregister(shm._name, "shared_memory")
    try:
        per = int(np.prod(shape[2:]))
        flat = np.ndarray((shape[0] * shape[1], per), dtype=np.float32, buffer=shm.buf)
        H = shape[1]
        for s in range(lo, hi):
            b, h = divmod(s, H)
            flat[s] = (_slice_draw(tuple(key_prefix) + (b0 + b, h), per) * scale).astype(np.float32)
    finally:
        shm.close()


def normal_bhnd(workload_id: int, tensor_id: int, shape, scale: float, dtype: str,
                extra=(), workers: int | None = None, offset=0.0, b0: int = 0) -> HostTensor:
    """Seeded N(offset, scale^2) tensor of shape [B, H, n, d] (n may be 1).

    Slice (b, h) depends only on (workload_id, tensor_id, *extra, b, h), so any
    slice can be regenerated on its own.  Large tensors are drawn in a small
    pool of spawned worker processes; the values do not depend on the pool.
    offset (a number, or an array broadcast against [B, H, n, d]) is added in
    fp64 before the rounding (serial draws only).  b0: the first batch index
    of the block drawn (rows b0 .. b0 + B - 1 of a larger batch, same values).
    """
    B, H = shape[0], shape[1]
    per = int(np.prod(shape[2:]))
    key_prefix = (workload_id, tensor_id) + tuple(extra)
    total = B * H * per
    has_offset = not (np.isscalar(offset) and offset == 0.0)
    if workers is None:
        workers = 1 if (total < (1 << 26) or has_offset) else min(16, os.cpu_count() or 1)
    if has_offset and workers > 1:
        raise ValueError("offset draws are serial")
    if workers <= 1:
        out = np.empty((B * H, per), dtype=np.float64)
        for s in range(B * H):
            b, h = divmod(s, H)
            out[s] = _slice_draw(key_prefix + (b0 + b, h), per)
        out *= scale
        out = out.reshape(shape)
        if has_offset:
            out = out + np.asarray(offset, dtype=np.float64)
        return _round_to(out, dtype)

    # worker processes run this module directly (python -m ...), so they never
    # re-import the caller's main script
    import json
    import subprocess
    import sys
    from multiprocessing import shared_memory
    shm = shared_memory.SharedMemory(create=True, size=total * 4)
    try:
        nsl = B * H
        step = (nsl + workers - 1) // workers
        procs = []
        root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
        env = dict(os.environ, PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""),
                   OMP_NUM_THREADS="1")
        for lo in range(0, nsl, step):
            job = json.dumps([shm.name, list(shape), list(key_prefix), scale, lo, min(nsl, lo + step), b0])
            procs.append(subprocess.Popen([sys.executable, "-m", "kernelized_linear_attention_la_amd.inputs", job],
                                          env=env))
        codes = [p.wait() for p in procs]
        if any(codes):
            raise RuntimeError(f"input generator workers failed: {codes}")
        x32 = np.ndarray(tuple(shape), dtype=np.float32, buffer=shm.buf).copy()
    finally:
        shm.close()
        shm.unlink()
    if dtype == "f32":
        return HostTensor(store=x32, f32=x32, dtype="f32")
    bits = f32_to_bf16_bits(x32)
    return HostTensor(store=bits, f32=bf16_bits_to_f32(bits), dtype="bf16")


def orthogonal_gaussian_rows(workload_id: int, m: int, d: int) -> np.ndarray:
    """FAVOR+ projection rows w_1..w_m (fp32 [m, d]), orthogonal within blocks of d."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([workload_id, TENSOR_W])))
    rows = []
    while len(rows) * d < m:
        g = rng.standard_normal((d, d))
        qm, rm = np.linalg.qr(g)
        qm = qm * np.sign(np.diag(rm))[None, :]
        rows.append(qm.T)  # rows of an orthogonal matrix
    w = np.concatenate(rows, axis=0)[:m]
    lengths = np.linalg.norm(rng.standard_normal((m, d)), axis=1)
    return np.ascontiguousarray((w * lengths[:, None]).astype(np.float32))


def iid_gaussian_rows(seed: int, m: int, d: int) -> np.ndarray:
    """Plain i.i.d. N(0, I_d) projection rows (fp64), used by statistical checks."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TENSOR_W, 1])))
    return rng.standard_normal((m, d))


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    phi: str            # "elu1" or "favor"
    dtype: str          # "f32" or "bf16"
    B: int
    H: int
    N: int
    dk: int
    dv: int
    scale: float
    chunk: int
    m: int = 0          # FAVOR+ feature count
    modes: tuple = ("causal",)
    decode_steps: int = 0  # > 0: N is the prefix length, then this many decode steps
    retention: bool = False  # decayed, unnormalised variant (per-head decays, no normaliser)
    backward: bool = False   # gradients of the causal form for a seeded dL/dO
    gated: str = ""          # "gla" or "delta" (gated delta rule): token-by-token recurrences
    map_param: int = 0       # DPFP nu / cosFormer M

    @property
    def dprime(self) -> int:
        return {"favor": self.m, "trig": 2 * self.m, "dpfp": 2 * self.dk * self.map_param,
                "cosformer": 2 * self.dk}.get(self.phi, self.dk)

    def gammas(self) -> np.ndarray:
        """Per-head decays of a retention workload (float32 [H])."""
        return retention_decays(self.H)

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.N


WORKLOADS = {
    w.name: w for w in [
        Workload("elu1_f32_b1h2n256d64", 1, "elu1", "f32", 1, 2, 256, 64, 64, 1.0, 64,
                 modes=("noncausal", "causal")),
        Workload("elu1_bf16_b4h8n2048d64_c64", 2, "elu1", "bf16", 4, 8, 2048, 64, 64,
                 1.0 / math.sqrt(64), 64),
        Workload("elu1_bf16_b2h16n16384d128_c128", 3, "elu1", "bf16", 2, 16, 16384, 128, 128,
                 1.0 / math.sqrt(128), 128),
        Workload("decode_elu1_f32_s256h32d128_prefix1024_steps64", 4, "elu1", "f32", 256, 32,
                 1024, 128, 128, 1.0 / math.sqrt(128), 64, decode_steps=64),
        Workload("favor_bf16_b2h8n8192d64_m256_c64", 5, "favor", "bf16", 2, 8, 8192, 64, 64,
                 64 ** -0.25, 64, m=256),
        # the same at a 128-token chunk request (run on the 64-token tiling)
        Workload("favor_bf16_b2h8n8192d64_m256_c128", 5, "favor", "bf16", 2, 8, 8192, 64, 64,
                 64 ** -0.25, 128, m=256),
        # retention (decayed, unnormalised; raw q and k): the shapes of the
        # normalised workloads above, one decay per head
        Workload("ret_f32_b1h2n256d64_c64", 6, "identity", "f32", 1, 2, 256, 64, 64, 1.0 / math.sqrt(64), 64,
                 retention=True),
        Workload("ret_bf16_b4h8n2048d64_c64", 7, "identity", "bf16", 4, 8, 2048, 64, 64, 1.0 / math.sqrt(64), 64,
                 retention=True),
        Workload("ret_bf16_b2h16n16384d128_c128", 8, "identity", "bf16", 2, 16, 16384, 128, 128,
                 1.0 / math.sqrt(128), 128, retention=True),
        # backward of the causal form at the bf16 forward workloads' shapes
        Workload("bwd_elu1_bf16_b4h8n2048d64_c64", 9, "elu1", "bf16", 4, 8, 2048, 64, 64,
                 1.0 / math.sqrt(64), 64, backward=True),
        Workload("bwd_elu1_bf16_b2h16n16384d128_c128", 10, "elu1", "bf16", 2, 16, 16384, 128, 128,
                 1.0 / math.sqrt(128), 128, backward=True),
        # further feature maps at the bf16 d = 64 shape (fp32-arithmetic kernels)
        Workload("dpfp_bf16_b4h8n2048d64_c64", 13, "dpfp", "bf16", 4, 8, 2048, 64, 64, 1.0 / math.sqrt(64), 64,
                 map_param=1),
        Workload("trig_bf16_b4h8n2048d64_m64_c64", 14, "trig", "bf16", 4, 8, 2048, 64, 64, 0.5 / math.sqrt(64),
                 64, m=64),
        Workload("cosformer_bf16_b4h8n2048d64_c64", 15, "cosformer", "bf16", 4, 8, 2048, 64, 64,
                 1.0 / math.sqrt(64), 64, map_param=2048),
        # gated / delta-rule states at the bf16 d = 64 shape (raw q, k; unit-norm keys)
        Workload("gla_bf16_b4h8n2048d64", 11, "identity", "bf16", 4, 8, 2048, 64, 64, 1.0 / math.sqrt(64), 1,
                 gated="gla"),
        Workload("gdelta_bf16_b4h8n2048d64", 12, "identity", "bf16", 4, 8, 2048, 64, 64, 1.0 / math.sqrt(64), 1,
                 gated="delta"),
    ]
}


def retention_decays(H: int) -> np.ndarray:
    """Per-head decays for the retention workloads: log-spaced forgetting rates,
    gamma_h = 1 - 2^-(3 + 7 h / (H - 1)), from 1 - 1/8 (head 0) to 1 - 1/1024
    (last head); a single head gets 1 - 1/32.  Rounded to float32 (the storage
    type of the decays), so both sides see identical values."""
    if H == 1:
        e = np.array([5.0])
    else:
        e = 3.0 + 7.0 * np.arange(H) / (H - 1)
    return (1.0 - 2.0 ** (-e)).astype(np.float32)


@dataclass
class ForwardInputs:
    wl: Workload
    Q: HostTensor
    K: HostTensor
    V: HostTensor
    W: np.ndarray | None = None  # fp32 [m, dk] for FAVOR+


def forward_inputs(wl: Workload, N: int | None = None, workers=None, batch=None) -> ForwardInputs:
    """Q, K, V of a forward workload (optionally a shorter prefix length N;
    optionally only the batch rows range(*batch), the same values as those
    rows of the whole draw)."""
    n = wl.N if N is None else N
    b0, b1 = (0, wl.B) if batch is None else batch
    shp_k = (b1 - b0, wl.H, n, wl.dk)
    shp_v = (b1 - b0, wl.H, n, wl.dv)
    Q = normal_bhnd(wl.wid, TENSOR_Q, shp_k, wl.scale, wl.dtype, workers=workers, b0=b0)
    K = normal_bhnd(wl.wid, TENSOR_K, shp_k, wl.scale, wl.dtype, workers=workers, b0=b0)
    V = normal_bhnd(wl.wid, TENSOR_V, shp_v, wl.scale, wl.dtype, workers=workers, b0=b0)
    W = None
    if wl.phi == "favor":
        W = orthogonal_gaussian_rows(wl.wid, wl.m, wl.dk)
    elif wl.phi == "trig":  # cos/sin projections: i.i.d. N(0, I) rows, fp32
        W = iid_gaussian_rows(wl.wid, wl.m, wl.dk).astype(np.float32)
    return ForwardInputs(wl, Q, K, V, W)


def decode_step_inputs(wl: Workload, step: int):
    """Single-token q, k, v ([B, H, 1, d]) of one decode step."""
    q = normal_bhnd(wl.wid, TENSOR_QSTEP, (wl.B, wl.H, 1, wl.dk), wl.scale, wl.dtype, extra=(step,))
    k = normal_bhnd(wl.wid, TENSOR_KSTEP, (wl.B, wl.H, 1, wl.dk), wl.scale, wl.dtype, extra=(step,))
    v = normal_bhnd(wl.wid, TENSOR_VSTEP, (wl.B, wl.H, 1, wl.dv), wl.scale, wl.dtype, extra=(step,))
    return q, k, v


def custom_inputs(seed: int, B, H, N, dk, dv, scale=1.0, dtype="f32", phi="elu1", m=0):
    """Small seeded inputs for edge-case tests (any shape)."""
    Q = normal_bhnd(1000 + seed, TENSOR_Q, (B, H, N, dk), scale, dtype)
    K = normal_bhnd(1000 + seed, TENSOR_K, (B, H, N, dk), scale, dtype)
    V = normal_bhnd(1000 + seed, TENSOR_V, (B, H, N, dv), scale, dtype)
    W = orthogonal_gaussian_rows(1000 + seed, m, dk) if phi == "favor" else None
    wl = Workload(f"custom{seed}", 1000 + seed, phi, dtype, B, H, N, dk, dv, scale, 64, m=m)
    return ForwardInputs(wl, Q, K, V, W)


def offset_inputs(seed: int, B, H, N, dk, dv, q_offset, k_offset, spread=0.5, v_scale=None, dtype="f32"):
    """Inputs far on the negative side of the ELU+1 map: Q ~ N(q_offset,
    spread^2), K ~ N(k_offset, spread^2) per coordinate (offsets are numbers or
    arrays broadcast against [B, H, N, 1], e.g. per-row offsets), V ~ N(0,
    v_scale^2) (default 1/sqrt(d_v)).  The same recipe as every other draw
    (seeded per slice, fp64 -> fp32 -> storage)."""
    vs = dv ** -0.5 if v_scale is None else v_scale
    Q = normal_bhnd(3000 + seed, TENSOR_Q, (B, H, N, dk), spread, dtype, offset=q_offset)
    K = normal_bhnd(3000 + seed, TENSOR_K, (B, H, N, dk), spread, dtype, offset=k_offset)
    V = normal_bhnd(3000 + seed, TENSOR_V, (B, H, N, dv), vs, dtype)
    wl = Workload(f"offset{seed}", 3000 + seed, "elu1", dtype, B, H, N, dk, dv, spread, 64)
    return ForwardInputs(wl, Q, K, V, None)


def grad_output(wid: int, B, H, N, dv, dtype, scale=1.0, workers=None) -> HostTensor:
    """Seeded dL/dO [B, H, N, d_v] for the backward (N(0, scale^2), storage dtype)."""
    return normal_bhnd(wid, TENSOR_DO, (B, H, N, dv), scale, dtype, workers=workers)


def state_grads(wid: int, B, H, dp, dv):
    """Seeded dL/dS_out [B, H, d', d_v] and dL/dz_out [B, H, d'] (fp32, N(0, 1))."""
    dS = normal_bhnd(wid, TENSOR_DS, (B, H, dp, dv), 1.0, "f32").f32
    dz = normal_bhnd(wid, TENSOR_DZ, (B, H, 1, dp), 1.0, "f32").f32.reshape(B, H, dp)
    return np.ascontiguousarray(dS), np.ascontiguousarray(dz)


def positive_state(wid: int, B, H, dp, dv, tokens=64):
    """A starting state (S_in, z_in) shaped like the sums of `tokens` earlier
    tokens with positive features: S_in ~ N(0, tokens), z_in ~ tokens * U(0.5, 1.5)."""
    S = normal_bhnd(wid, TENSOR_SIN, (B, H, dp, dv), math.sqrt(tokens), "f32").f32
    u = normal_bhnd(wid, TENSOR_ZIN, (B, H, 1, dp), 1.0, "f32").f32.reshape(B, H, dp)
    z = (tokens * (1.0 + 0.5 * np.tanh(u))).astype(np.float32)
    return np.ascontiguousarray(S), np.ascontiguousarray(z)


@dataclass
class GatedInputs:
    Q: HostTensor
    K: HostTensor
    V: HostTensor
    alpha_ch: np.ndarray   # GLA gate per key channel, fp32 [B, H, N, d_k] in (0.9, 1)
    alpha: np.ndarray      # scalar forget gate, fp32 [B, H, N] in (0.95, 1)
    beta: np.ndarray       # write strength, fp32 [B, H, N] in (0, 1)


def gated_inputs(wid: int, B, H, N, dk, dv, dtype="f32", workers=None) -> GatedInputs:
    """Seeded inputs of the gated / delta-rule recurrences.

    q, v ~ N(0, 1/d); keys are N(0, I) rows scaled to unit length in fp64 before
    rounding (the delta rule's erase step I - beta k k^T then stays a
    contraction for beta in [0, 1]).  Gates and strengths are logistic
    transforms of seeded normals: alpha_ch = 1 - 0.1 s, alpha = 1 - 0.05 s,
    beta = s, s = 1 / (1 + exp(-x)).
    """
    sc = 1.0 / math.sqrt(dk)
    Q = normal_bhnd(wid, TENSOR_Q, (B, H, N, dk), sc, dtype, workers=workers)
    Kraw = normal_bhnd(wid, TENSOR_K, (B, H, N, dk), 1.0, "f32", workers=workers).f32.astype(np.float64)
    Kraw /= np.maximum(np.linalg.norm(Kraw, axis=-1, keepdims=True), 1e-30)
    K = _round_to(Kraw, dtype)
    V = normal_bhnd(wid, TENSOR_V, (B, H, N, dv), 1.0 / math.sqrt(dv), dtype, workers=workers)
    sig = lambda x: 1.0 / (1.0 + np.exp(-x.astype(np.float64)))  # noqa: E731
    ach = normal_bhnd(wid, TENSOR_GATE_CH, (B, H, N, dk), 1.0, "f32", workers=workers).f32
    al = normal_bhnd(wid, TENSOR_GATE, (B, H, N, 1), 1.0, "f32").f32.reshape(B, H, N)
    be = normal_bhnd(wid, TENSOR_BETA, (B, H, N, 1), 1.0, "f32").f32.reshape(B, H, N)
    return GatedInputs(Q, K, V, (1.0 - 0.1 * sig(ach)).astype(np.float32), (1.0 - 0.05 * sig(al)).astype(np.float32),
                       sig(be).astype(np.float32))


if __name__ == "__main__":
    # worker entry of normal_bhnd's process pool
    import json
    import sys
    _a = json.loads(sys.argv[1])
    _fill_slices(_a[0], tuple(_a[1]), tuple(_a[2]), _a[3], _a[4], _a[5], _a[6] if len(_a) > 6 else 0)
