"""GPU parity over seeded random problems for the backward, decode and gated
entry points (C ABI against the oracle).

Like tests/test_gpu_random_sweep.py for the forwards: each problem is drawn
from a fixed seed over the shapes the entry point accepts, printed, run, and
compared with the oracle on the same stored values, with the metric and
tolerance of the suite that pins that entry point by hand:
  * backward (la_backward_causal_chunked): slice_rel_err of dQ, dK, dV, dS_in,
    dz_in (one token: dQ = dK = 0, held to tol x max |dV| as in
    tests/test_gpu_backward.py);
  * decode (la_decode_step, la_retention_decode_step): a few steps from a
    positive starting state, per-row output error and the state after them;
  * gated (GLA and gated delta rule, token by token and chunkwise): per-row
    outputs and the final state.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import row_rel_err, slice_rel_err, state_rel_err, to_device, to_f64, tol_for, z_rel_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[sweep+]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()
    oracle.set_map(0, 0)


def _dev(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()


# ---------------------------------------------------------------------------
# backward
# ---------------------------------------------------------------------------
def _draw_bwd(i):
    r = np.random.default_rng([20270, i])
    phi = str(r.choice(["elu1", "elu1", "favor"]))
    dtype = str(r.choice(["f32", "bf16"]))
    dk = int(r.choice([8, 16, 32, 64, 64, 96, 128, 128]))
    dv = dk if r.random() < 0.7 else int(r.choice([8, 24, 64, 128]))
    m = 0
    if phi == "favor":
        m = int(r.choice([16, 64, 128, 256]))
        while m * (dv + 1) > 16640:
            m //= 2
    B, H = int(r.choice([1, 2])), int(r.choice([1, 2, 3]))
    N = max(1, int(np.exp(r.uniform(0.0, np.log(1500.0)))))
    chunk = int(r.choice([16, 32, 64, 128]))
    return dict(phi=phi, dtype=dtype, B=B, H=H, N=N, dk=dk, dv=dv, m=m, chunk=chunk, state=bool(r.random() < 0.5))


BWD = [_draw_bwd(i) for i in range(30)]


@pytest.mark.parametrize("i", range(len(BWD)),
                         ids=[f"{c['phi']}-{c['dtype']}-B{c['B']}H{c['H']}N{c['N']}dk{c['dk']}dv{c['dv']}m{c['m']}"
                              f"C{c['chunk']}{'S' if c['state'] else ''}" for c in BWD])
def test_random_backward_against_oracle(i):
    c = BWD[i]
    _say("backward", i, c)
    B, H, N, dk, dv, phi, m = c["B"], c["H"], c["N"], c["dk"], c["dv"], c["phi"], c["m"]
    fi = inputs.custom_inputs(8000 + i, B, H, N, dk, dv, scale=(dk ** -0.25 if phi == "favor" else dk ** -0.5),
                              dtype=c["dtype"], phi=phi, m=m)
    dO = inputs.grad_output(9000 + i, B, H, N, dv, c["dtype"])
    dp = m if phi == "favor" else dk
    S_in = z_in = dS = dz = None
    if c["state"]:
        S_in, z_in = inputs.positive_state(9000 + i, B, H, dp, dv)
        dS, dz = inputs.state_grads(9000 + i, B, H, dp, dv)
    W = torch.from_numpy(fi.W).cuda() if fi.W is not None else None
    got = la.la_backward_causal_chunked(to_device(fi.Q), to_device(fi.K), to_device(fi.V), to_device(dO), c["chunk"],
                                        phi=phi, W=W, S_in=_dev(S_in), z_in=_dev(z_in), dS_out=_dev(dS),
                                        dz_out=_dev(dz), state_grad=True)
    torch.cuda.synchronize()
    got = [to_f64(t) for t in got]
    ref = oracle.causal_backward(phi, fi.Q.f32, fi.K.f32, fi.V.f32, dO.f32, W=fi.W, S_in=S_in, z_in=z_in,
                                 dS_out=dS, dz_out=dz)
    tol = tol_for(c["dtype"])
    names = ("dQ", "dK", "dV", "dS_in", "dz_in")
    vanish = ("dQ", "dK") if N == 1 and not c["state"] else ()
    # One token and no starting state: dz_in = -phi(q) (dO . o) / den carries a
    # single dot product, whose rounding is large against it where it cancels;
    # it is held to the forward-error bound tol * sum|dO_j o_j| / |sum dO_j o_j|
    # per slice instead.
    cond = None
    if N == 1 and not c["state"]:
        o, _, _ = oracle.causal_recurrent(phi, fi.Q.f32, fi.K.f32, fi.V.f32, fi.W)
        prod = dO.f32.astype(np.float64)[:, :, 0] * o[:, :, 0]
        cond = np.abs(prod).sum(-1) / np.maximum(np.abs(prod.sum(-1)), 1e-300)
    errs = {}
    for n, g, rf in zip(names, got, ref):
        assert np.isfinite(g).all(), n
        if n in vanish:  # zero in exact arithmetic: the oracle's value is rounding noise
            assert np.abs(g).max() <= tol * np.abs(ref[2]).max(), n
            continue
        if n == "dz_in" and cond is not None:
            per = np.abs(g - rf).max(-1) / np.maximum(np.abs(rf).max(-1), 1e-300)
            assert np.all(per <= tol * np.maximum(cond, 1.0)), (per, cond)
            continue
        errs[n] = slice_rel_err(g, rf)
    _say("backward", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e < tol, (n, e)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
def _draw_dec(i):
    r = np.random.default_rng([20280, i])
    phi = str(r.choice(["elu1", "elu1", "favor", "dpfp", "trig", "cosformer", "retention"]))
    d = int(r.choice([16, 32, 64, 96, 128]))
    dv = d if r.random() < 0.7 else int(r.choice([8, 40, 128]))
    m, param, pos0 = 0, 0, 0
    if phi == "favor":
        m = int(r.choice([16, 64, 256]))
    elif phi == "trig":
        m = int(r.choice([8, 32, 64]))
    elif phi == "dpfp":
        param = int(r.integers(1, 256 // (2 * d) + 1))
    elif phi == "cosformer":
        pos0 = int(r.integers(0, 3000))
        param = pos0 + int(r.integers(8, 4000))
    B, H = int(r.choice([1, 2, 5])), int(r.choice([1, 3, 8]))
    return dict(phi=phi, B=B, H=H, dk=d, dv=dv, m=m, param=param, pos0=pos0, steps=int(r.integers(1, 6)))


DEC = [_draw_dec(i) for i in range(30)]


@pytest.mark.parametrize("i", range(len(DEC)),
                         ids=[f"{c['phi']}-B{c['B']}H{c['H']}dk{c['dk']}dv{c['dv']}m{c['m']}p{c['param']}"
                              f"x{c['steps']}" for c in DEC])
def test_random_decode_against_oracle(i):
    c = DEC[i]
    _say("decode", i, c)
    B, H, dk, dv, steps = c["B"], c["H"], c["dk"], c["dv"], c["steps"]
    ret = c["phi"] == "retention"
    phi = "identity" if ret else c["phi"]
    fi = inputs.custom_inputs(8500 + i, B, H, steps, dk, dv,
                              scale={"favor": dk ** -0.25, "trig": 0.5 / np.sqrt(dk)}.get(phi, dk ** -0.5),
                              dtype="f32", phi=phi, m=c["m"])
    W = fi.W
    if phi == "trig":
        W = inputs.iid_gaussian_rows(8500 + i, c["m"], dk).astype(np.float32)
    Wt = torch.from_numpy(np.ascontiguousarray(W)).cuda() if W is not None else None
    dp = {"favor": c["m"], "trig": 2 * c["m"], "dpfp": 2 * dk * c["param"], "cosformer": 2 * dk}.get(phi, dk)
    S0, z0 = inputs.positive_state(8600 + i, B, H, dp, dv, tokens=16)
    S, z = _dev(S0), _dev(z0)
    Sr, zr = S0.astype(np.float64), z0.astype(np.float64)
    gam = inputs.retention_decays(H)
    for t in range(steps):
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x.f32[:, :, t])).cuda() for x in (fi.Q, fi.K, fi.V))
        if ret:
            o = la.la_retention_decode_step(q, k, v, S, _dev(gam.astype(np.float32)))
            ro, Sr = oracle.retention_decode_step("identity", fi.Q.f32[:, :, t], fi.K.f32[:, :, t], fi.V.f32[:, :, t],
                                                 Sr, gam.astype(np.float64))
        else:
            oracle.set_map(c["param"], c["pos0"] + t)
            o = la.la_decode_step(q, k, v, S, z, phi=phi, W=Wt, map_param=c["param"], pos0=c["pos0"] + t)
            ro, Sr, zr = oracle.decode_step(phi, fi.Q.f32[:, :, t], fi.K.f32[:, :, t], fi.V.f32[:, :, t], Sr, zr, W)
        torch.cuda.synchronize()
        e = row_rel_err(to_f64(o).reshape(B, H, dv), ro)
        assert e < tol_for("f32"), (t, e)
    es = state_rel_err(to_f64(S), Sr)
    _say("decode", f"last O {e:.2e} S {es:.2e}")
    assert es < tol_for("f32")
    if not ret:
        ez = state_rel_err(to_f64(z)[..., None], zr[..., None]) if phi == "trig" else z_rel_err(to_f64(z), zr)
        assert ez < tol_for("f32"), ez


# ---------------------------------------------------------------------------
# gated recurrences
# ---------------------------------------------------------------------------
def _draw_gated(i):
    r = np.random.default_rng([20290, i])
    kind = str(r.choice(["gla", "gla_chunked", "delta", "gated_delta", "delta_chunked", "gated_delta_chunked"]))
    dtype = str(r.choice(["f32", "bf16"]))
    if kind.endswith("_chunked") and "delta" in kind:
        dk, dv = 64, int(r.choice([16, 32, 64, 128]))
    elif kind == "gla_chunked":
        dk, dv = int(r.choice([8, 16, 32, 64])), int(r.choice([8, 16, 40, 64, 128]))
    else:
        dk, dv = int(r.choice([4, 16, 32, 64, 128])), int(r.choice([3, 16, 64, 128]))
    B, H = int(r.choice([1, 2, 4])), int(r.choice([1, 2, 8]))
    N = max(1, int(np.exp(r.uniform(0.0, np.log(2500.0)))))
    return dict(kind=kind, dtype=dtype, B=B, H=H, N=N, dk=dk, dv=dv, state=bool(r.random() < 0.5))


GATED = [_draw_gated(i) for i in range(30)]


@pytest.mark.parametrize("i", range(len(GATED)),
                         ids=[f"{c['kind']}-{c['dtype']}-B{c['B']}H{c['H']}N{c['N']}dk{c['dk']}dv{c['dv']}"
                              f"{'S' if c['state'] else ''}" for c in GATED])
def test_random_gated_against_oracle(i):
    c = GATED[i]
    _say("gated", i, c)
    B, H, N, dk, dv, kind = c["B"], c["H"], c["N"], c["dk"], c["dv"], c["kind"]
    gi = inputs.gated_inputs(8800 + i, B, H, N, dk, dv, c["dtype"])
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    S_in = inputs.positive_state(8900 + i, B, H, dk, dv, tokens=4)[0] if c["state"] else None
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    if kind.startswith("gla"):
        fwd = la.la_forward_gla_chunked if kind == "gla_chunked" else la.la_forward_gla_recurrent
        O = fwd(q, k, v, _dev(gi.alpha_ch), S_in=_dev(S_in), S_out=S_out)
        ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.alpha_ch, S_in=S_in)
    else:
        alpha = gi.alpha if kind.startswith("gated") else None
        fwd = la.la_forward_delta_chunked if kind.endswith("_chunked") else la.la_forward_delta_recurrent
        O = fwd(q, k, v, _dev(gi.beta), alpha=_dev(alpha), S_in=_dev(S_in), S_out=S_out)
        ref, Sref = oracle.delta_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.beta, alpha=alpha, S_in=S_in)
    torch.cuda.synchronize()
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say("gated", f"O {eo:.2e} S {es:.2e}")
    tol = tol_for(c["dtype"])
    assert eo < tol and es < tol, (eo, es)
