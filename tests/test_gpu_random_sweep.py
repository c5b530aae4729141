"""GPU parity over a seeded random sweep of problem shapes (C ABI against the oracle).

The hand-written cases elsewhere pin the kernels' edges one by one; this file
draws 120 problems from a fixed seed over everything the boundary accepts:
every feature map (ELU+1, FAVOR+, identity under retention, DPFP, cos/sin
projections, cosFormer), fp32 and bf16 storage, d_k and d_v from 16 to 128
(d_k != d_v on the plain maps), every chunk length, token counts from 1 to a
few thousand, a carried starting state or none.  Each problem runs the
causal chunked forward (normalised maps), the non-causal forward (normalised
maps, no state) and the retention forward (identity, ELU+1, FAVOR+), and is
compared with the oracle on the same inputs with the suite's metric and
tolerances (1e-4 fp32 storage, 2e-2 bf16 storage).  The draws are printed
before each call, so a failure names its problem.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import row_rel_err, state_rel_err, to_device, to_f64, tol_for, z_rel_err

pytestmark = pytest.mark.gpu

N_CASES = 120
MAX_ORACLE_WORK = 2e9  # B*H*N*d'*d_v per case: keeps the fp64 recurrence to about a second


def _say(*a):
    print("[sweep]", *a, file=sys.stderr, flush=True)


def _draw(i):
    r = np.random.default_rng([20260, i])
    phi = r.choice(["elu1", "elu1", "favor", "identity", "dpfp", "trig", "cosformer"])
    dtype = str(r.choice(["f32", "bf16"]))
    d = int(r.choice([16, 32, 48, 64, 64, 96, 128, 128]))
    dv = d
    if phi in ("elu1", "identity") and r.random() < 0.25:
        dv = int(r.choice([8, 24, 64, 80, 128]))
    m, param, pos0 = 0, 0, 0
    if phi == "favor":
        m = int(r.choice([16, 64, 256, 256]))
        if r.random() < 0.5:
            d, dv = 64, 64  # the matrix-core FAVOR+ shape (d = 64, m = 256) with bf16
            m = 256
    elif phi == "trig":
        m = int(r.choice([8, 32, 64, 128]))
    elif phi == "dpfp":
        param = int(r.integers(1, 256 // (2 * d) + 1))
    elif phi == "cosformer":
        pos0 = int(r.integers(0, 100))
    B = int(r.choice([1, 2, 3]))
    H = int(r.choice([1, 2, 4, 8]))
    N = int(np.exp(r.uniform(0.0, np.log(6000.0))))
    N = max(1, N)
    if phi == "cosformer":
        param = pos0 + N + int(r.integers(0, 500))
    chunk = int(r.choice([16, 32, 64, 128]))
    # cos/sin features take both signs: a random starting state could put a
    # denominator near zero, so those problems start from zero
    state = bool(r.random() < 0.5) and phi != "trig"
    dp = {"favor": m, "trig": 2 * m, "dpfp": 2 * d * param, "cosformer": 2 * d}.get(phi, d)
    while B * H * N * dp * dv > MAX_ORACLE_WORK and N > 1:
        N = max(1, N // 2)
    if phi == "cosformer":
        param = max(param, pos0 + N)
    return dict(phi=str(phi), dtype=dtype, B=B, H=H, N=N, dk=d, dv=dv, m=m, param=param, pos0=pos0, chunk=chunk,
                state=state, dp=dp)


CASES = [_draw(i) for i in range(N_CASES)]


def _z_err(z, zref):
    """Per-element relative error of z; entries that are exactly zero in the
    oracle (DPFP features that no token of a short sequence turns on: products
    of ReLUs, zero in exact arithmetic) must be exactly zero on the GPU too."""
    zero = zref == 0
    assert np.all(z[zero] == 0), "a feature sum that is exactly zero came out nonzero"
    return z_rel_err(z[~zero], zref[~zero]) if (~zero).any() else 0.0


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()
    oracle.set_map(0, 0)


def _inputs(i, c):
    d = c["dk"]
    scale = {"favor": d ** -0.25, "trig": 0.5 / np.sqrt(d)}.get(c["phi"], d ** -0.5)
    fi = inputs.custom_inputs(7000 + i, c["B"], c["H"], c["N"], d, c["dv"], scale=scale, dtype=c["dtype"],
                              phi=c["phi"], m=c["m"])
    W = fi.W
    if c["phi"] == "trig":
        W = inputs.iid_gaussian_rows(7000 + i, c["m"], d).astype(np.float32)
    return fi, W


@pytest.mark.parametrize("i", range(N_CASES),
                         ids=[f"{c['phi']}-{c['dtype']}-B{c['B']}H{c['H']}N{c['N']}dk{c['dk']}dv{c['dv']}"
                              f"m{c['m']}p{c['param']}C{c['chunk']}{'S' if c['state'] else ''}" for c in CASES])
def test_random_problem_against_oracle(i):
    c = CASES[i]
    _say("case", i, c)
    phi, B, H, N, dk, dv, dp = c["phi"], c["B"], c["H"], c["N"], c["dk"], c["dv"], c["dp"]
    fi, W = _inputs(i, c)
    q, k, v = to_device(fi.Q), to_device(fi.K), to_device(fi.V)
    Wt = torch.from_numpy(np.ascontiguousarray(W)).cuda() if W is not None else None
    oracle.set_map(c["param"], c["pos0"])
    tol = tol_for(c["dtype"])
    rng = np.random.default_rng([20261, i])
    S0 = (rng.standard_normal((B, H, dp, dv)) * 0.1).astype(np.float32) if c["state"] else None
    # z_in positive, as a sum of the positive maps' features is
    z0 = (np.abs(rng.standard_normal((B, H, dp))) + 0.5).astype(np.float32) if c["state"] else None
    kw = dict(phi=phi, W=Wt, map_param=c["param"], pos0=c["pos0"])

    if phi != "identity":
        S = torch.zeros(B, H, dp, dv, device="cuda")
        z = torch.zeros(B, H, dp, device="cuda")
        S_in = torch.from_numpy(S0).cuda() if c["state"] else None
        z_in = torch.from_numpy(z0).cuda() if c["state"] else None
        O = la.la_forward_causal_chunked(q, k, v, c["chunk"], S_in=S_in, z_in=z_in, S_out=S, z_out=z, **kw)
        ref, Sref, zref = oracle.causal_recurrent(phi, fi.Q.f32, fi.K.f32, fi.V.f32, W, S_in=S0, z_in=z0)
        torch.cuda.synchronize()
        e, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S), Sref)
        ez = (state_rel_err(to_f64(z)[..., None], zref[..., None]) if phi == "trig" else
              _z_err(to_f64(z), zref))
        _say(f"causal O {e:.2e} S {es:.2e} z {ez:.2e}")
        assert e < tol and es < tol and ez < tol, (e, es, ez)
        if not c["state"]:
            On = la.la_forward_noncausal(q, k, v, **kw)
            refn, _, _ = oracle.noncausal(phi, fi.Q.f32, fi.K.f32, fi.V.f32, W)
            torch.cuda.synchronize()
            en = row_rel_err(to_f64(On), refn)
            _say(f"noncausal O {en:.2e}")
            assert en < tol, en

    if phi in ("identity", "elu1", "favor"):
        gam = inputs.retention_decays(H)
        S = torch.zeros(B, H, dp, dv, device="cuda")
        S_in = torch.from_numpy(S0).cuda() if c["state"] else None
        O = la.la_forward_retention_chunked(q, k, v, torch.from_numpy(gam.astype(np.float32)).cuda(), c["chunk"],
                                            phi=phi, W=Wt, S_in=S_in, S_out=S)
        ref, Sref = oracle.retention_recurrent(phi, fi.Q.f32, fi.K.f32, fi.V.f32, gam.astype(np.float64), W=W,
                                               S_in=S0)
        torch.cuda.synchronize()
        e, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S), Sref)
        _say(f"retention O {e:.2e} S {es:.2e}")
        assert e < tol and es < tol, (e, es)
