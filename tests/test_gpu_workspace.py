"""GPU checks of the workspace contract at the C ABI.

* One buffer shared in turn by the single-pass causal forward, the backward,
  the chunkwise GLA and the chunkwise delta rule (one stream): the calls other
  than the forward leave the first 256 bytes (the forward's hand-off control
  block: launch counter, done count, error word) untouched, so every later
  forward on the buffer equals a forward on a fresh zero-filled workspace bit
  for bit, and the other calls' results equal their own fresh-workspace runs.
* The error word: la_workspace_error reads 0 after good launches, reads what
  the control block holds, and clears it when asked.
"""
import sys

import numpy as np
import pytest
import torch

from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import to_device

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[workspace]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def _bits(t):
    return t.contiguous().view(torch.uint8).clone()


def test_one_workspace_shared_by_forward_backward_and_gated_calls():
    B, H, N, d = 4, 8, 2048, 64   # the bf16 d = 64 forward workload's shape: a single-pass launch
    fi = inputs.custom_inputs(910, B, H, N, d, d, scale=d ** -0.5, dtype="bf16")
    q, k, v = to_device(fi.Q), to_device(fi.K), to_device(fi.V)
    dO = to_device(inputs.grad_output(911, B, H, N, d, "bf16"))
    gi = inputs.gated_inputs(912, B, H, N, d, d, "bf16")
    gq, gk, gv = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    a_ch = torch.from_numpy(np.ascontiguousarray(gi.alpha_ch)).cuda()
    al, be = torch.from_numpy(gi.alpha).cuda(), torch.from_numpy(gi.beta).cuda()

    p = la._problem_of(q, v, "elu1", None)
    n_fwd = la.la_workspace_bytes(p, 64)
    n_bwd = la.la_backward_workspace_bytes(p, 64)
    n_gla, n_delta = la.la_gla_workspace_bytes(gq, gv), la.la_delta_workspace_bytes(gq, gv)
    assert min(n_fwd, n_bwd, n_gla, n_delta) > 256

    def forward(ws):
        S = torch.empty(B, H, d, d, device="cuda")
        z = torch.empty(B, H, d, device="cuda")
        O = la.la_forward_causal_chunked(q, k, v, 64, S_out=S, z_out=z, workspace=ws)
        return [_bits(O), _bits(S), _bits(z)]

    def backward(ws):
        return [_bits(t) for t in la.la_backward_causal_chunked(q, k, v, dO, 64, workspace=ws)[:3]]

    def gla(ws):
        S = torch.empty(B, H, d, d, device="cuda")
        return [_bits(la.la_forward_gla_chunked(gq, gk, gv, a_ch, S_out=S, workspace=ws)), _bits(S)]

    def delta(ws):
        S = torch.empty(B, H, d, d, device="cuda")
        return [_bits(la.la_forward_delta_chunked(gq, gk, gv, be, alpha=al, S_out=S, workspace=ws)), _bits(S)]

    # each call on a fresh workspace of its own
    fresh = {"fwd": forward(torch.zeros(n_fwd, dtype=torch.uint8, device="cuda")),
             "bwd": backward(torch.zeros(n_bwd, dtype=torch.uint8, device="cuda")),
             "gla": gla(torch.zeros(n_gla, dtype=torch.uint8, device="cuda")),
             "delta": delta(torch.zeros(n_delta, dtype=torch.uint8, device="cuda"))}
    torch.cuda.synchronize()

    shared = torch.zeros(max(n_fwd, n_bwd, n_gla, n_delta), dtype=torch.uint8, device="cuda")
    order = ["fwd", "bwd", "fwd", "gla", "fwd", "delta", "fwd", "fwd", "bwd", "gla", "delta", "fwd"]
    run = {"fwd": forward, "bwd": backward, "gla": gla, "delta": delta}
    for i, name in enumerate(order):
        _say("shared workspace call", i, name)
        got = run[name](shared)
        torch.cuda.synchronize()
        for a, b in zip(got, fresh[name]):
            assert torch.equal(a, b), (i, name)
    err = la.la_workspace_error(shared)
    torch.cuda.synchronize()
    assert int(err.item()) == 0


def test_workspace_error_word_read_and_clear():
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    la.la_workspace_error(ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    # the word is the third 32-bit word of the control block; set it from the host
    ws.view(torch.int32)[2] = 1
    la.la_workspace_error(ws, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    la.la_workspace_error(ws, err, clear=True)   # read, then clear
    torch.cuda.synchronize()
    assert int(err.item()) == 1
    assert int(ws.view(torch.int32)[2].item()) == 0
    # the rest of the control block is left alone
    ws.view(torch.int32)[0] = 7
    la.la_workspace_error(ws, err, clear=True)
    torch.cuda.synchronize()
    assert int(err.item()) == 0 and int(ws.view(torch.int32)[0].item()) == 7
