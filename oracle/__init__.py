"""fp64 CPU oracle for kernelized linear attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library
(``kernelized_linear_attention_la_amd``) never imports, links or runs it, and
the two share no code.

The arithmetic lives in ``la_oracle.c`` (plain C, double precision, OpenMP
over independent (batch, head) slices); this module only builds it with gcc,
loads it with ctypes and widens numpy inputs to float64.  Each wrapper below
names the definition it evaluates; the C source cites the pages.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_LIB = os.path.join(_HERE, "liblaoracle.so")

PHI_ELU1 = 0
PHI_FAVOR = 1
PHI_IDENTITY = 2
PHI_DPFP = 3
PHI_TRIG = 4
PHI_COSFORMER = 5
_PHI = {"elu1": PHI_ELU1, "favor": PHI_FAVOR, "identity": PHI_IDENTITY, "dpfp": PHI_DPFP, "trig": PHI_TRIG,
        "cosformer": PHI_COSFORMER}


def build(force: bool = False) -> str:
    """Compile la_oracle.c into liblaoracle.so with gcc (fp64, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
               "-std=c11", "-Wall", "-Wextra", "-Wno-unused-parameter", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        D = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        L.ora_phi.argtypes = [i, i, i, D, i, D, D]
        L.ora_state_read.argtypes = [i, i, i, D, D, D, D, D]
        L.ora_noncausal.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, D]
        L.ora_causal_recurrent.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, D, D, D]
        L.ora_quadratic.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, i, D]
        L.ora_causal_chunked.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, i, D, D, D]
        L.ora_decode_step.argtypes = [i, i, i, i, i, D, D, D, D, D, D, D]
        L.ora_retention_recurrent.argtypes = [i, i, i, i, i, i, i, D, D, D, D, D, D, D, D]
        L.ora_retention_parallel.argtypes = [i, i, i, i, i, i, i, D, D, D, D, D, D, D]
        L.ora_retention_chunked.argtypes = [i, i, i, i, i, i, i, D, D, D, D, D, D, i, D, D]
        L.ora_retention_decode_step.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, D]
        L.ora_causal_backward.argtypes = [i, i, i, i, i, i, D, D, D, D, D, D, D, D, D, D, D, D, D, D]
        L.ora_gla_recurrent.argtypes = [i, i, i, i, D, D, D, D, D, D, D]
        L.ora_delta_recurrent.argtypes = [i, i, i, i, D, D, D, D, D, D, D, D]
        L.ora_set_map.argtypes = [i, ctypes.c_longlong]
        L.ora_feature_dim.argtypes = [i, i, i]
        L.ora_feature_dim.restype = i
        L.ora_num_threads.restype = ctypes.c_int
        L.ora_set_num_threads.argtypes = [i]
        _lib = L
    return _lib


def num_threads() -> int:
    return lib().ora_num_threads()


def set_num_threads(n: int) -> None:
    lib().ora_set_num_threads(int(n))


def _d(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(x):
    if x is None:
        return None
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _kind(phi):
    return _PHI[phi] if isinstance(phi, str) else int(phi)


def set_map(param=0, pos0=0):
    """Parameters of the maps that take one (DPFP: nu; cosFormer: the horizon M)
    and the position of the first token (cosFormer).  They stay in effect for
    every later call until set again."""
    lib().ora_set_map(int(param), int(pos0))


def feature_dim(phi, dk, m=0):
    return lib().ora_feature_dim(_kind(phi), int(dk), int(m))


def _dp(phi, dk, W):
    return feature_dim(phi, dk, 0 if W is None else W.shape[0])


def _flat4(x):
    x = _d(x)
    B, H = x.shape[0], x.shape[1]
    return x.reshape(B * H, *x.shape[2:]), (B, H)


def phi(kind, X, W=None):
    """Feature map applied to each row of X [n, d] -> [n, dp]."""
    X = _d(X)
    n, d = X.shape
    Wd = _d(W) if W is not None else None
    m = Wd.shape[0] if Wd is not None else 0
    dp = feature_dim(kind, d, m)
    out = np.empty((n, dp))
    lib().ora_phi(_kind(kind), n, d, _p(X), m, _p(Wd), _p(out))
    return out


def state_read(phiQ, S, z):
    """num = phiQ S and den = phiQ z for phiQ [n, dp], S [dp, dv], z [dp]."""
    phiQ, S, z = _d(phiQ), _d(S), _d(z)
    n, dp = phiQ.shape
    dv = S.shape[1]
    num = np.empty((n, dv))
    den = np.empty((n,))
    lib().ora_state_read(n, dp, dv, _p(phiQ), _p(S), _p(z), _p(num), _p(den))
    return num, den


def _prep(phi_kind, Q, K, V, W):
    (Qf, (B, H)), (Kf, _), (Vf, _) = _flat4(Q), _flat4(K), _flat4(V)
    BH, N, dk = Qf.shape
    dv = Vf.shape[2]
    Wd = _d(W) if W is not None else None
    m = Wd.shape[0] if Wd is not None else 0
    dp = feature_dim(phi_kind, dk, m)
    return Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp


def noncausal(phi_kind, Q, K, V, W=None):
    """Non-causal factorised attention. Returns O [B,H,N,dv], S [B,H,dp,dv], z [B,H,dp]."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dp, dv)); z = np.empty((BH, dp))
    lib().ora_noncausal(BH, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(Qf), _p(Kf), _p(Vf),
                        _p(O), _p(S), _p(z))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dp, dv), z.reshape(B, H, dp)


def _state_in(S_in, z_in, BH, dp, dv):
    if S_in is None:
        return None, None
    return _d(S_in).reshape(BH, dp, dv), _d(z_in).reshape(BH, dp)


def causal_recurrent(phi_kind, Q, K, V, W=None, S_in=None, z_in=None):
    """Causal token-by-token recurrence. Returns O, S_final, z_final."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    Si, zi = _state_in(S_in, z_in, BH, dp, dv)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dp, dv)); z = np.empty((BH, dp))
    lib().ora_causal_recurrent(BH, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(Qf), _p(Kf), _p(Vf),
                               _p(Si), _p(zi), _p(O), _p(S), _p(z))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dp, dv), z.reshape(B, H, dp)


def quadratic(phi_kind, Q, K, V, W=None, S_in=None, z_in=None, causal=True):
    """Explicit pairwise (parallel-mode) form; O only."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    Si, zi = _state_in(S_in, z_in, BH, dp, dv)
    O = np.empty((BH, N, dv))
    lib().ora_quadratic(BH, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(Qf), _p(Kf), _p(Vf),
                        _p(Si), _p(zi), int(bool(causal)), _p(O))
    return O.reshape(B, H, N, dv)


def causal_chunked(phi_kind, Q, K, V, chunk, W=None, S_in=None, z_in=None):
    """Chunkwise hybrid (quadratic inside chunks, state between). Returns O, S, z."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    Si, zi = _state_in(S_in, z_in, BH, dp, dv)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dp, dv)); z = np.empty((BH, dp))
    lib().ora_causal_chunked(BH, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(Qf), _p(Kf), _p(Vf),
                             _p(Si), _p(zi), int(chunk), _p(O), _p(S), _p(z))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dp, dv), z.reshape(B, H, dp)


def causal_backward(phi_kind, Q, K, V, dO, W=None, S_in=None, z_in=None, dS_out=None, dz_out=None):
    """Gradients of the causal form (reverse-mode through the recurrence).

    For a loss with dL/dO = dO and, optionally, dL/dS_out, dL/dz_out, returns
    (dQ, dK, dV, dS_in, dz_in); dS_in, dz_in are the gradients with respect to
    the starting state (returned whether or not S_in was given).
    """
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    Si, zi = _state_in(S_in, z_in, BH, dp, dv)
    dOf = _d(dO).reshape(BH, N, dv)
    dSo = None if dS_out is None else _d(dS_out).reshape(BH, dp, dv)
    dzo = None if dz_out is None else _d(dz_out).reshape(BH, dp)
    dQ = np.empty((BH, N, dk)); dK = np.empty((BH, N, dk)); dV = np.empty((BH, N, dv))
    dSi = np.empty((BH, dp, dv)); dzi = np.empty((BH, dp))
    lib().ora_causal_backward(BH, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(Qf), _p(Kf), _p(Vf), _p(Si), _p(zi),
                              _p(dOf), _p(dSo), _p(dzo), _p(dQ), _p(dK), _p(dV), _p(dSi), _p(dzi))
    return (dQ.reshape(B, H, N, dk), dK.reshape(B, H, N, dk), dV.reshape(B, H, N, dv),
            dSi.reshape(B, H, dp, dv), dzi.reshape(B, H, dp))


def decode_step(phi_kind, q, k, v, S, z, W=None):
    """One decode step; q,k [B,H,dk] (or [B,H,1,dk]), v [B,H,dv].

    Returns (o [B,H,dv], S_new, z_new); the inputs are not modified.
    """
    q = _d(q); k = _d(k); v = _d(v)
    B, H = q.shape[0], q.shape[1]
    dk = q.shape[-1]; dv = v.shape[-1]
    BH = B * H
    Wd = _d(W) if W is not None else None
    m = Wd.shape[0] if Wd is not None else 0
    dp = feature_dim(phi_kind, dk, m)
    Sn = _d(S).reshape(BH, dp, dv).copy()
    zn = _d(z).reshape(BH, dp).copy()
    qf = q.reshape(BH, dk); kf = k.reshape(BH, dk); vf = v.reshape(BH, dv)
    o = np.empty((BH, dv))
    lib().ora_decode_step(BH, dk, dv, _kind(phi_kind), m, _p(Wd), _p(qf), _p(kf), _p(vf),
                          _p(Sn), _p(zn), _p(o))
    return o.reshape(B, H, dv), Sn.reshape(B, H, dp, dv), zn.reshape(B, H, dp)


# ---------------------------------------------------------------------------
# Retention: decayed, unnormalised ("Story of Attention Part 5", sections 4 and 6)
# ---------------------------------------------------------------------------
def _gamma(gamma, H):
    """Per-head decays as float64 [H]; a scalar applies to every head."""
    g = np.asarray(gamma, dtype=np.float64)
    if g.ndim == 0:
        g = np.full(H, float(g))
    if g.shape != (H,):
        raise ValueError(f"gamma must be a scalar or have {H} entries")
    return np.ascontiguousarray(g)


def _rstate_in(S_in, BH, dp, dv):
    return None if S_in is None else _d(S_in).reshape(BH, dp, dv)


def retention_recurrent(phi_kind, Q, K, V, gamma, W=None, S_in=None):
    """S_n = gamma S_{n-1} + phi(k_n) v_n^T, o_n = phi(q_n)^T S_n. Returns O, S_final."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    g = _gamma(gamma, H)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dp, dv))
    lib().ora_retention_recurrent(BH, H, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(g), _p(Qf), _p(Kf), _p(Vf),
                                  _p(_rstate_in(S_in, BH, dp, dv)), _p(O), _p(S))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dp, dv)


def retention_parallel(phi_kind, Q, K, V, gamma, W=None, S_in=None):
    """O = (phi(Q) phi(K)^T (.) D) V (+ gamma^(i+1) phi(q_i)^T S_in), every pair explicit."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    g = _gamma(gamma, H)
    O = np.empty((BH, N, dv))
    lib().ora_retention_parallel(BH, H, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(g), _p(Qf), _p(Kf), _p(Vf),
                                 _p(_rstate_in(S_in, BH, dp, dv)), _p(O))
    return O.reshape(B, H, N, dv)


def retention_chunked(phi_kind, Q, K, V, gamma, chunk, W=None, S_in=None):
    """Lightning blockwise form with blocks of `chunk` tokens. Returns O, S_final."""
    Qf, Kf, Vf, Wd, B, H, BH, N, dk, dv, m, dp = _prep(phi_kind, Q, K, V, W)
    g = _gamma(gamma, H)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dp, dv))
    lib().ora_retention_chunked(BH, H, N, dk, dv, _kind(phi_kind), m, _p(Wd), _p(g), _p(Qf), _p(Kf), _p(Vf),
                                _p(_rstate_in(S_in, BH, dp, dv)), int(chunk), _p(O), _p(S))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dp, dv)


def retention_decode_step(phi_kind, q, k, v, S, gamma, W=None):
    """One retention step for every (b, h); q,k [B,H,dk], v [B,H,dv]. Returns (o, S_new)."""
    q = _d(q); k = _d(k); v = _d(v)
    B, H = q.shape[0], q.shape[1]
    dk = q.shape[-1]; dv = v.shape[-1]
    BH = B * H
    Wd = _d(W) if W is not None else None
    m = Wd.shape[0] if Wd is not None else 0
    dp = feature_dim(phi_kind, dk, m)
    g = _gamma(gamma, H)
    Sn = _d(S).reshape(BH, dp, dv).copy()
    o = np.empty((BH, dv))
    lib().ora_retention_decode_step(BH, H, dk, dv, _kind(phi_kind), m, _p(Wd), _p(g), _p(q.reshape(BH, dk)),
                                    _p(k.reshape(BH, dk)), _p(v.reshape(BH, dv)), _p(Sn), _p(o))
    return o.reshape(B, H, dv), Sn.reshape(B, H, dp, dv)


# ---------------------------------------------------------------------------
# Gated and delta-rule states ("Linear Attention", GLA and the delta rule;
# "Story of Attention Part 5", section 7).  Raw q, k; S feature-major [dk, dv].
# ---------------------------------------------------------------------------
def gla_recurrent(Q, K, V, alpha, S_in=None):
    """S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t; alpha [B,H,N,dk]. Returns O, S_final."""
    Qf, Kf, Vf, _, B, H, BH, N, dk, dv, _, _ = _prep("identity", Q, K, V, None)
    A = _d(alpha).reshape(BH, N, dk)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dk, dv))
    lib().ora_gla_recurrent(BH, N, dk, dv, _p(Qf), _p(Kf), _p(Vf), _p(A), _p(_rstate_in(S_in, BH, dk, dv)),
                            _p(O), _p(S))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dk, dv)


def delta_recurrent(Q, K, V, beta, alpha=None, S_in=None):
    """Gated delta rule: S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T, o_t = S_t^T q_t.

    beta, alpha [B,H,N] (alpha None: the plain delta rule). Returns O, S_final.
    """
    Qf, Kf, Vf, _, B, H, BH, N, dk, dv, _, _ = _prep("identity", Q, K, V, None)
    b = _d(beta).reshape(BH, N)
    a = None if alpha is None else _d(alpha).reshape(BH, N)
    O = np.empty((BH, N, dv)); S = np.empty((BH, dk, dv))
    lib().ora_delta_recurrent(BH, N, dk, dv, _p(Qf), _p(Kf), _p(Vf), _p(a), _p(b),
                              _p(_rstate_in(S_in, BH, dk, dv)), _p(O), _p(S))
    return O.reshape(B, H, N, dv), S.reshape(B, H, dk, dv)
