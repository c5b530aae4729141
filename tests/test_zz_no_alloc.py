"""GPU check of la_forward_causal_chunked_noalloc (the causal forward whose
workspace is the library's fixed device array) through the C ABI.

Two calls in a row, the second with a smaller input (a different segment
plan on the same array), each against la_forward_causal_chunked on a fresh
caller workspace (same kernels: bit for bit) and against the oracle at the
suite's tolerance; then the fp32 path with a starting state, and a HIP graph
of the call replayed with eager calls in between.
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


def _say(*a):
    print("[noalloc]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def _case(seed, B, H, N, d, dtype, chunk, with_state):
    fi = inputs.custom_inputs(seed, B, H, N, d, d, scale=d ** -0.5, dtype=dtype)
    q, k, v = to_device(fi.Q), to_device(fi.K), to_device(fi.V)
    S_in = z_in = None
    if with_state:
        Sh, zh = inputs.positive_state(seed, B, H, d, d)
        S_in, z_in = torch.from_numpy(Sh).cuda(), torch.from_numpy(zh).cuda()
    return fi, q, k, v, S_in, z_in, (Sh, zh) if with_state else (None, None)


def _both(fi, q, k, v, S_in, z_in, chunk):
    B, H, N, d = q.shape
    outs = []
    for noalloc in (True, False):
        S = torch.full((B, H, d, d), float("nan"), device="cuda")
        z = torch.full((B, H, d), float("nan"), device="cuda")
        O = torch.full_like(v, float("nan"))
        if noalloc:
            la.la_forward_causal_chunked_noalloc(q, k, v, chunk, S_in=S_in, z_in=z_in, S_out=S, z_out=z, out=O)
        else:
            ws = torch.zeros(max(1, la.la_workspace_bytes(la._problem_of(q, v, "elu1", None), chunk)),
                             dtype=torch.uint8, device="cuda")
            la.la_forward_causal_chunked(q, k, v, chunk, S_in=S_in, z_in=z_in, S_out=S, z_out=z, out=O, workspace=ws)
        torch.cuda.synchronize()
        outs.append((O, S, z))
    return outs


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_two_calls_match_the_workspace_entry_point(order):
    cases = [(1, 4, 8, 2048, 64, "bf16", 64, False),   # single pass, eight segments per slice
             (2, 2, 4, 700, 64, "bf16", 64, False)]    # smaller input: another plan on the same array
    for seed, B, H, N, d, dtype, chunk, st in cases:
        _say("noalloc call", (B, H, N, d, dtype, chunk))
        fi, q, k, v, S_in, z_in, _ = _case(seed, B, H, N, d, dtype, chunk, st)
        (O, S, z), (O0, S0, z0) = _both(fi, q, k, v, S_in, z_in, chunk)
        assert torch.equal(O.view(torch.int16), O0.view(torch.int16))
        assert torch.equal(S, S0) and torch.equal(z, z0)
        ref, Sref, zref = oracle.causal_recurrent("elu1", fi.Q.f32, fi.K.f32, fi.V.f32)
        tol = tol_for(dtype)
        assert row_rel_err(to_f64(O), ref) < tol
        assert state_rel_err(to_f64(S), Sref) < tol and z_rel_err(to_f64(z), zref) < tol


def test_noalloc_fp32_path_with_state():
    # fp32 storage: the state pass, scan and chunk pass use the array's S and z parts
    seed, B, H, N, d = 3, 1, 2, 256, 64
    _say("noalloc fp32 with S_in", (B, H, N, d))
    fi, q, k, v, S_in, z_in, (Sh, zh) = _case(seed, B, H, N, d, "f32", 64, True)
    assert la.la_workspace_bytes(la._problem_of(q, v, "elu1", None), 64) > 0
    (O, S, z), (O0, S0, z0) = _both(fi, q, k, v, S_in, z_in, 64)
    assert torch.equal(O, O0) and torch.equal(S, S0) and torch.equal(z, z0)
    ref, Sref, zref = oracle.causal_recurrent("elu1", fi.Q.f32, fi.K.f32, fi.V.f32, S_in=Sh, z_in=zh)
    assert row_rel_err(to_f64(O), ref) < 1e-4
    assert state_rel_err(to_f64(S), Sref) < 1e-4 and z_rel_err(to_f64(z), zref) < 1e-4


def test_noalloc_graph_replay():
    seed, B, H, N, d = 4, 2, 4, 1500, 64
    fi, q, k, v, _, _, _ = _case(seed, B, H, N, d, "bf16", 64, False)
    (O0, S0, z0), _ = _both(fi, q, k, v, None, None, 64)
    O, S, z = torch.empty_like(O0), torch.empty_like(S0), torch.empty_like(z0)
    q2, k2, v2 = q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous()
    O2 = la.la_forward_causal_chunked_noalloc(q2, k2, v2, 64)
    torch.cuda.synchronize()
    O2_0 = O2.clone()
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        la.la_forward_causal_chunked_noalloc(q, k, v, 64, S_out=S, z_out=z, out=O)
    torch.cuda.synchronize()
    for rep in range(3):
        _say("noalloc graph replay", rep)
        O.zero_(), S.zero_(), z.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(O.view(torch.int16), O0.view(torch.int16)) and torch.equal(S, S0) and torch.equal(z, z0)
        la.la_forward_causal_chunked_noalloc(q2, k2, v2, 64, out=O2)  # an eager call between replays
        torch.cuda.synchronize()
        assert torch.equal(O2.view(torch.int16), O2_0.view(torch.int16))
