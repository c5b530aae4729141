"""GPU parity of the gated and delta-rule recurrences (la_forward_gla_recurrent,
la_forward_delta_recurrent, through the C ABI) against the oracle.

Outputs: per row (b, h, t) max |gpu - oracle| / max |oracle| over the row
(row_rel_err, the metric of every forward in the suite: a row that a zero
gate left far below the slice's largest row is still held to its own scale;
a row that is exactly zero in exact arithmetic is held to the tolerance in
absolute terms); final states: state_rel_err.  1e-4 for fp32 storage, 2e-2 for bf16 (fp32
state and arithmetic, outputs rounded once).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import row_rel_err, state_rel_err, to_device, to_f64, tol_for

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[gated]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


CASES = [
    # (B, H, N, dk, dv, dtype, with S_in)
    (1, 2, 256, 64, 64, "f32", False),
    (2, 3, 100, 16, 8, "f32", True),
    (1, 1, 1, 32, 32, "f32", True),       # one token: the decode step
    (1, 2, 77, 5, 3, "f32", True),        # odd widths, columns not a multiple of 8
    (1, 1, 50, 128, 128, "f32", True),    # largest widths
    (2, 4, 1000, 128, 128, "bf16", False),
    (4, 8, 2048, 64, 64, "bf16", True),   # the bf16 d = 64 forward workload's shape
]


def _run(ci, case, kind):
    B, H, N, dk, dv, dtype, state = case
    gi = inputs.gated_inputs(2000 + ci, B, H, N, dk, dv, dtype)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    S_in = inputs.positive_state(2000 + ci, B, H, dk, dv, tokens=4)[0] if state else None
    dev = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    if kind == "gla":
        O = la.la_forward_gla_recurrent(q, k, v, dev(gi.alpha_ch), S_in=dev(S_in), S_out=S_out)
        ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.alpha_ch, S_in=S_in)
    else:
        alpha = gi.alpha if kind == "gated_delta" else None
        O = la.la_forward_delta_recurrent(q, k, v, dev(gi.beta), alpha=dev(alpha), S_in=dev(S_in), S_out=S_out)
        ref, Sref = oracle.delta_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.beta, alpha=alpha, S_in=S_in)
    torch.cuda.synchronize()
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say(kind, case, f"O {eo:.2e} S {es:.2e}")
    tol = tol_for(dtype)
    assert eo < tol and es < tol, (eo, es)


@pytest.mark.parametrize("kind", ["gla", "delta", "gated_delta"])
@pytest.mark.parametrize("ci", range(len(CASES)),
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}dk{c[3]}dv{c[4]}{c[5]}{'S' if c[6] else ''}" for c in CASES])
def test_gated_against_oracle(ci, kind):
    _run(ci, CASES[ci], kind)


def test_state_handoff_in_place():
    """Two calls (0..M, then M..N from the first call's state, S_out aliasing S_in) == one call."""
    B, H, N, d = 2, 2, 300, 32
    gi = inputs.gated_inputs(2100, B, H, N, d, d, "f32")
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    be, al = torch.from_numpy(gi.beta).cuda(), torch.from_numpy(gi.alpha).cuda()
    ref, Sref = oracle.delta_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.beta, alpha=gi.alpha)
    for M in (1, 100, 299):
        _say("handoff M", M)
        S = torch.zeros(B, H, d, d, device="cuda")
        c = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
        O1 = la.la_forward_delta_recurrent(c(q, 0, M), c(k, 0, M), c(v, 0, M), c(be, 0, M), alpha=c(al, 0, M),
                                           S_out=S)
        O2 = la.la_forward_delta_recurrent(c(q, M, N), c(k, M, N), c(v, M, N), c(be, M, N), alpha=c(al, M, N),
                                           S_in=S, S_out=S)
        torch.cuda.synchronize()
        assert row_rel_err(to_f64(torch.cat([O1, O2], 2)), ref) < 1e-4
        assert state_rel_err(to_f64(S), Sref) < 1e-4


def _extreme_gates(seed, B, H, N, dk):
    """GLA gates that stress the chunkwise form: exact zeros (the state is
    cleared), tiny gates (a 16-token block decays past 2^-86, so its diagonal
    block is summed element by element), mid-range and near-one gates."""
    rng = np.random.default_rng(seed)
    u = rng.random((B, H, N, dk))
    a = np.where(u < 0.1, 0.0,
                 np.where(u < 0.3, rng.uniform(1e-4, 0.05, u.shape),
                          np.where(u < 0.5, rng.uniform(0.5, 0.9, u.shape), rng.uniform(0.9, 1.0, u.shape))))
    # one slice keeps near-one gates only (the pivoted path everywhere)
    a[0, 0] = rng.uniform(0.9, 1.0, a[0, 0].shape)
    return a.astype(np.float32)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gla_extreme_gates_against_oracle(dtype):
    B, H, N, dk, dv = 1, 2, 300, 64, 40
    gi = inputs.gated_inputs(2200, B, H, N, dk, dv, dtype)
    al = _extreme_gates(2200, B, H, N, dk)
    S_in = inputs.positive_state(2200, B, H, dk, dv, tokens=4)[0]
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    O = la.la_forward_gla_recurrent(q, k, v, torch.from_numpy(al).cuda(), S_in=torch.from_numpy(S_in).cuda(),
                                    S_out=S_out)
    ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, al, S_in=S_in)
    torch.cuda.synchronize()
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say("gla extreme gates", dtype, f"O {eo:.2e} S {es:.2e}")
    tol = tol_for(dtype)
    assert np.isfinite(to_f64(O)).all()
    assert eo < tol and es < tol, (eo, es)


def test_gla_state_handoff_across_forms():
    """GLA in two calls == one call, S_out aliasing S_in: the first part runs token by
    token (fewer than 64 tokens) or chunkwise, the second part chunkwise."""
    B, H, N, d = 2, 2, 300, 32
    gi = inputs.gated_inputs(2300, B, H, N, d, d, "f32")
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    al = torch.from_numpy(gi.alpha_ch).cuda()
    ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.alpha_ch)
    for M in (30, 100):
        _say("gla handoff M", M)
        S = torch.zeros(B, H, d, d, device="cuda")
        c = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
        O1 = la.la_forward_gla_recurrent(c(q, 0, M), c(k, 0, M), c(v, 0, M), c(al, 0, M), S_out=S)
        O2 = la.la_forward_gla_recurrent(c(q, M, N), c(k, M, N), c(v, M, N), c(al, M, N), S_in=S, S_out=S)
        torch.cuda.synchronize()
        assert row_rel_err(to_f64(torch.cat([O1, O2], 2)), ref) < 1e-4
        assert state_rel_err(to_f64(S), Sref) < 1e-4


# ---------------------------------------------------------------------------
# Gated delta rule in chunkwise form (la_forward_delta_chunked): the same
# recurrence as the oracle, evaluated through per-chunk triangular solves.
# ---------------------------------------------------------------------------
CHUNKED_CASES = [
    # (B, H, N, dk, dv, dtype, with S_in)
    (1, 2, 256, 64, 64, "f32", False),
    (2, 3, 100, 64, 16, "f32", True),      # ragged last chunk, one 16-column block
    (1, 1, 1, 64, 32, "f32", True),        # one token
    (1, 2, 50, 64, 128, "f32", True),      # shorter than a chunk, widest values
    (1, 1, 65, 64, 48, "bf16", True),      # one token past a chunk
    (2, 4, 1000, 64, 128, "bf16", False),
    (4, 8, 2048, 64, 64, "bf16", True),    # the gated delta-rule workload's shape
    (1, 2, 420, 64, 32, "f32", True),      # seven chunks: one full round of the scan's ring and a ragged tail
    (2, 1, 300, 64, 80, "bf16", True),     # five chunks, d_v past one 64-column group
]


@pytest.mark.parametrize("kind", ["delta", "gated_delta"])
@pytest.mark.parametrize("ci", range(len(CHUNKED_CASES)),
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}dv{c[4]}{c[5]}{'S' if c[6] else ''}" for c in CHUNKED_CASES])
def test_delta_chunked_against_oracle(ci, kind):
    B, H, N, dk, dv, dtype, state = CHUNKED_CASES[ci]
    gi = inputs.gated_inputs(2300 + ci, B, H, N, dk, dv, dtype)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    S_in = inputs.positive_state(2300 + ci, B, H, dk, dv, tokens=4)[0] if state else None
    dev = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    alpha = gi.alpha if kind == "gated_delta" else None
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    _say("chunked", kind, CHUNKED_CASES[ci])
    O = la.la_forward_delta_chunked(q, k, v, dev(gi.beta), alpha=dev(alpha), S_in=dev(S_in), S_out=S_out)
    torch.cuda.synchronize()
    ref, Sref = oracle.delta_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.beta, alpha=alpha, S_in=S_in)
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say("chunked", kind, f"O {eo:.2e} S {es:.2e}")
    tol = tol_for(dtype)
    assert eo < tol and es < tol, (eo, es)


def test_delta_chunked_handoff_and_small_gates():
    """Two chunked calls (0..M, then M..N from the first call's state, S_out
    aliasing S_in) equal the oracle over 0..N; forget gates down to 1e-3 and
    exact zeros (the state is cleared) included."""
    B, H, N, dk, dv = 2, 2, 300, 64, 32
    gi = inputs.gated_inputs(2400, B, H, N, dk, dv, "f32")
    rng = np.random.default_rng(2400)
    al = gi.alpha.copy()
    u = rng.random(al.shape)
    al[u < 0.05] = 0.0
    al[(u >= 0.05) & (u < 0.15)] = rng.uniform(1e-3, 0.5, al[(u >= 0.05) & (u < 0.15)].shape).astype(np.float32)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    be, alt = torch.from_numpy(gi.beta).cuda(), torch.from_numpy(al).cuda()
    ref, Sref = oracle.delta_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.beta, alpha=al)
    for M in (1, 64, 130):
        _say("chunked handoff M", M)
        S = torch.zeros(B, H, dk, dv, device="cuda")
        c = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
        O1 = la.la_forward_delta_chunked(c(q, 0, M), c(k, 0, M), c(v, 0, M), c(be, 0, M), alpha=c(alt, 0, M),
                                         S_out=S)
        O2 = la.la_forward_delta_chunked(c(q, M, N), c(k, M, N), c(v, M, N), c(be, M, N), alpha=c(alt, M, N),
                                         S_in=S, S_out=S)
        torch.cuda.synchronize()
        eo = row_rel_err(to_f64(torch.cat([O1, O2], 2)), ref)
        es = state_rel_err(to_f64(S), Sref)
        _say("chunked handoff", M, f"O {eo:.2e} S {es:.2e}")
        assert eo < 1e-4 and es < 1e-4, (eo, es)


def test_delta_chunked_rejects_unsupported_shapes():
    gi = inputs.gated_inputs(2500, 1, 1, 64, 32, 32, "f32")
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    be = torch.from_numpy(gi.beta).cuda()
    with pytest.raises(RuntimeError):
        la.la_forward_delta_chunked(q, k, v, be)  # d_k = 32: the token-by-token entry point takes it
    assert la.la_delta_workspace_bytes(q, v) == 0


# ---------------------------------------------------------------------------
# GLA in chunkwise form (la_forward_gla_chunked): every chunk's products at
# once, the element-wise state chain over chunks, the outputs of every chunk.
# ---------------------------------------------------------------------------
GLA_SPLIT_CASES = [
    # (B, H, N, dk, dv, dtype, with S_in)
    (1, 2, 256, 64, 64, "f32", False),
    (2, 3, 100, 16, 8, "f32", True),       # narrow keys (padded channels), one partial column block
    (1, 1, 1, 32, 32, "f32", True),        # one token
    (1, 2, 77, 5, 3, "f32", True),         # odd widths
    (2, 2, 130, 64, 40, "bf16", True),     # ragged chunk and column block
    (1, 2, 200, 64, 80, "f32", True),      # two column groups of the per-chunk value products
    (2, 2, 190, 48, 128, "bf16", True),    # two full column groups, padded channels
    (1, 1, 600, 64, 24, "f32", True),      # ten chunks: more than one round of the chain's prefetch ring
    (4, 8, 2048, 64, 64, "bf16", True),    # the GLA workload's shape
]


@pytest.mark.parametrize("ci", range(len(GLA_SPLIT_CASES)),
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}dk{c[3]}dv{c[4]}{c[5]}{'S' if c[6] else ''}" for c in GLA_SPLIT_CASES])
def test_gla_chunked_against_oracle(ci):
    B, H, N, dk, dv, dtype, state = GLA_SPLIT_CASES[ci]
    gi = inputs.gated_inputs(2600 + ci, B, H, N, dk, dv, dtype)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    S_in = inputs.positive_state(2600 + ci, B, H, dk, dv, tokens=4)[0] if state else None
    dev = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).cuda()  # noqa: E731
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    _say("gla split", GLA_SPLIT_CASES[ci])
    O = la.la_forward_gla_chunked(q, k, v, dev(gi.alpha_ch), S_in=dev(S_in), S_out=S_out)
    torch.cuda.synchronize()
    ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.alpha_ch, S_in=S_in)
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say("gla split", f"O {eo:.2e} S {es:.2e}")
    tol = tol_for(dtype)
    assert eo < tol and es < tol, (eo, es)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gla_chunked_extreme_gates_and_handoff(dtype):
    """Zero, tiny, mid and near-one gates (the element-wise diagonal blocks)
    through the chunkwise form, also as two calls with S_out aliasing S_in."""
    B, H, N, dk, dv = 1, 2, 300, 64, 40
    gi = inputs.gated_inputs(2700, B, H, N, dk, dv, dtype)
    al = _extreme_gates(2700, B, H, N, dk)
    S_in = inputs.positive_state(2700, B, H, dk, dv, tokens=4)[0]
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    alt = torch.from_numpy(al).cuda()
    ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, al, S_in=S_in)
    tol = tol_for(dtype)
    S_out = torch.empty(B, H, dk, dv, device="cuda")
    O = la.la_forward_gla_chunked(q, k, v, alt, S_in=torch.from_numpy(S_in).cuda(), S_out=S_out)
    torch.cuda.synchronize()
    eo, es = row_rel_err(to_f64(O), ref), state_rel_err(to_f64(S_out), Sref)
    _say("gla split extreme", dtype, f"O {eo:.2e} S {es:.2e}")
    assert np.isfinite(to_f64(O)).all()
    assert eo < tol and es < tol, (eo, es)
    M = 130
    S = torch.from_numpy(S_in).cuda()
    c = lambda x, a, b: x[:, :, a:b].contiguous()  # noqa: E731
    O1 = la.la_forward_gla_chunked(c(q, 0, M), c(k, 0, M), c(v, 0, M), c(alt, 0, M), S_in=S, S_out=S)
    O2 = la.la_forward_gla_chunked(c(q, M, N), c(k, M, N), c(v, M, N), c(alt, M, N), S_in=S, S_out=S)
    torch.cuda.synchronize()
    eo, es = row_rel_err(to_f64(torch.cat([O1, O2], 2)), ref), state_rel_err(to_f64(S), Sref)
    _say("gla split handoff", dtype, f"O {eo:.2e} S {es:.2e}")
    assert eo < tol and es < tol, (eo, es)


def test_two_launch_forms_graph_replay():
    """The chunkwise GLA (three launches) and delta-rule (two) calls captured in a HIP graph: every
    replay (with eager calls on the same workspaces in between) reproduces the
    eager results bit for bit (the workspace records are rewritten each call)."""
    B, H, N, dk, dv = 2, 3, 200, 64, 48
    gi = inputs.gated_inputs(2800, B, H, N, dk, dv, "bf16")
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    a_ch = torch.from_numpy(np.ascontiguousarray(gi.alpha_ch)).cuda()
    al, be = torch.from_numpy(gi.alpha).cuda(), torch.from_numpy(gi.beta).cuda()
    S_in = torch.from_numpy(inputs.positive_state(2800, B, H, dk, dv, tokens=4)[0]).cuda()
    ws_g = torch.empty(la.la_gla_workspace_bytes(q, v), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(la.la_delta_workspace_bytes(q, v), dtype=torch.uint8, device="cuda")
    Sg, Sd = torch.empty_like(S_in), torch.empty_like(S_in)
    Og = la.la_forward_gla_chunked(q, k, v, a_ch, S_in=S_in, S_out=Sg, workspace=ws_g)
    Od = la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_in=S_in, S_out=Sd, workspace=ws_d)
    torch.cuda.synchronize()
    Og0, Od0, Sg0, Sd0 = Og.clone(), Od.clone(), Sg.clone(), Sd.clone()
    ref, Sref = oracle.gla_recurrent(gi.Q.f32, gi.K.f32, gi.V.f32, gi.alpha_ch, S_in=S_in.cpu().numpy())
    assert row_rel_err(to_f64(Og0), ref) < tol_for("bf16")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):  # warm up on the capture stream
        la.la_forward_gla_chunked(q, k, v, a_ch, S_in=S_in, S_out=Sg, out=Og, workspace=ws_g)
        la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_in=S_in, S_out=Sd, out=Od, workspace=ws_d)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        la.la_forward_gla_chunked(q, k, v, a_ch, S_in=S_in, S_out=Sg, out=Og, workspace=ws_g)
        la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_in=S_in, S_out=Sd, out=Od, workspace=ws_d)
    torch.cuda.synchronize()
    for rep in range(4):
        _say("chunkwise gated graph replay", rep)
        Og.zero_(), Od.zero_(), Sg.zero_(), Sd.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Og, Og0) and torch.equal(Sg, Sg0), rep
        assert torch.equal(Od, Od0) and torch.equal(Sd, Sd0), rep
        # eager calls on the same workspaces between replays
        la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_in=S_in, workspace=ws_d)
        la.la_forward_gla_chunked(q, k, v, a_ch, workspace=ws_g)
        torch.cuda.synchronize()
