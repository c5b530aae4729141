"""GPU test of the per-kernel timing hook (la_kernel_events) through the C ABI.

Every call that takes the hook must report, in `launched`, the kernels it
enqueued, record a positive duration for each of them, and give results bit
for bit equal to the same call without the hook (the events only bracket the
launches).  Covered: the causal single pass (bf16, d = 64), the causal fp32
path in three launches (segment sums, their scan, the chunk pass), the
chunkwise GLA and gated delta-rule calls (per-chunk launch, state chain,
outputs), and the backward: three launches on the matrix cores (forward sums,
dQ pass, dK/dV pass; no scan launches) and five on the fp32-arithmetic kernels.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import to_device

pytestmark = pytest.mark.gpu

SLOTS = (la.LA_KSLOT_STATE, la.LA_KSLOT_SCAN, la.LA_KSLOT_CHUNK)


def _say(*a):
    print("[timing hook]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


class _Events:
    """hipEvent pairs for the slots, through the runtime the library links."""

    def __init__(self, slots=SLOTS, kind=None):
        self.lib = la.lib()
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.kev = (kind or la.LaKernelEvents)()
        self.pairs = {}
        for sl in slots:
            pair = []
            for _ in range(2):
                ev = ctypes.c_void_p()
                assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
                pair.append(ev)
            self.kev.start[sl], self.kev.stop[sl] = pair[0], pair[1]
            self.pairs[sl] = pair

    def elapsed_ms(self, sl):
        a, b = self.pairs[sl]
        assert self.lib.hipEventSynchronize(b) == 0
        t = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        return t.value

    def close(self):
        for a, b in self.pairs.values():
            self.lib.hipEventDestroy(a)
            self.lib.hipEventDestroy(b)


def _check(name, run, expect, slots=SLOTS, kind=None, exact=False):
    """run(events) -> tuple of result tensors; expect: the slots that must be
    launched (exact: and no others)."""
    ref = [t.clone() for t in run(None)]
    torch.cuda.synchronize()
    ev = _Events(slots, kind)
    try:
        got = run(ev.kev)
        torch.cuda.synchronize()
        launched = [sl for sl in slots if ev.kev.launched[sl]]
        times = {sl: ev.elapsed_ms(sl) for sl in launched}
        _say(name, "launched", launched, "ms", {k: round(v, 4) for k, v in times.items()})
        assert set(expect) <= set(launched), (launched, expect)
        if exact:
            assert set(launched) == set(expect), (launched, expect)
        assert all(t > 0 for t in times.values()), times
        for a, b in zip(ref, got):
            assert torch.equal(a, b), name
    finally:
        ev.close()


def test_causal_single_pass_reports_its_kernel():
    fi = inputs.custom_inputs(9100, 2, 4, 1000, 64, 64, scale=64 ** -0.5, dtype="bf16", phi="elu1", m=0)
    q, k, v = to_device(fi.Q), to_device(fi.K), to_device(fi.V)
    ws = torch.zeros(la.la_workspace_bytes(la._problem_of(q, v, "elu1", None, 0, 0), 64), dtype=torch.uint8,
                     device="cuda")
    S = torch.zeros(2, 4, 64, 64, device="cuda")
    z = torch.zeros(2, 4, 64, device="cuda")

    def run(events):
        O = la.la_forward_causal_chunked(q, k, v, 64, S_out=S, z_out=z, workspace=ws, events=events)
        return O, S.clone(), z.clone()
    _check("causal bf16 single pass", run, [la.LA_KSLOT_CHUNK])


def test_causal_fp32_three_launches():
    fi = inputs.custom_inputs(9101, 1, 2, 700, 64, 64, scale=64 ** -0.5, dtype="f32", phi="elu1", m=0)
    q, k, v = to_device(fi.Q), to_device(fi.K), to_device(fi.V)
    S = torch.zeros(1, 2, 64, 64, device="cuda")
    z = torch.zeros(1, 2, 64, device="cuda")

    def run(events):
        O = la.la_forward_causal_chunked(q, k, v, 64, S_out=S, z_out=z, events=events)
        return O, S.clone(), z.clone()
    _check("causal fp32", run, [la.LA_KSLOT_CHUNK])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gla_chunked_reports_three_launches(dtype):
    gi = inputs.gated_inputs(9102, 2, 3, 333, 64, 48, dtype)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    al = torch.from_numpy(np.ascontiguousarray(gi.alpha_ch)).cuda()
    ws = torch.empty(la.la_gla_workspace_bytes(q, v), dtype=torch.uint8, device="cuda")
    S = torch.empty(2, 3, 64, 48, device="cuda")

    def run(events):
        O = la.la_forward_gla_chunked(q, k, v, al, S_out=S, workspace=ws, events=events)
        return O, S.clone()
    _check(f"gla chunked {dtype}", run, SLOTS)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_delta_chunked_reports_three_launches(dtype):
    gi = inputs.gated_inputs(9103, 2, 3, 333, 64, 48, dtype)
    q, k, v = to_device(gi.Q), to_device(gi.K), to_device(gi.V)
    al, be = torch.from_numpy(gi.alpha).cuda(), torch.from_numpy(gi.beta).cuda()
    ws = torch.empty(la.la_delta_workspace_bytes(q, v), dtype=torch.uint8, device="cuda")
    S = torch.empty(2, 3, 64, 48, device="cuda")

    def run(events):
        O = la.la_forward_delta_chunked(q, k, v, be, alpha=al, S_out=S, workspace=ws, events=events)
        return O, S.clone()
    _check(f"delta chunked {dtype}", run, SLOTS)


BSLOTS = (la.LA_BSLOT_FWD_SUMS, la.LA_BSLOT_FWD_SCAN, la.LA_BSLOT_DQ, la.LA_BSLOT_RSCAN, la.LA_BSLOT_DKV)


@pytest.mark.parametrize("path", ["matrix cores", "fp32 arithmetic"])
def test_backward_reports_its_launches(path):
    # bf16 ELU+1 d64 with 64-token chunks runs on the matrix cores (the passes
    # gather their starting states: no scan launches); FAVOR+ runs on the
    # fp32-arithmetic kernels with both scans
    if path == "matrix cores":
        fi = inputs.custom_inputs(9104, 1, 2, 1000, 64, 64, scale=64 ** -0.5, dtype="bf16", phi="elu1", m=0)
        phi, W, expect = "elu1", None, (la.LA_BSLOT_FWD_SUMS, la.LA_BSLOT_DQ, la.LA_BSLOT_DKV)
    else:
        fi = inputs.custom_inputs(9105, 1, 2, 300, 32, 32, scale=32 ** -0.25, dtype="bf16", phi="favor", m=32)
        phi, W, expect = "favor", torch.from_numpy(fi.W).cuda(), BSLOTS
    dp = 32 if phi == "favor" else 64
    dO = inputs.grad_output(9106, 1, 2, fi.Q.f32.shape[2], fi.V.f32.shape[3], "bf16")
    q, k, v, g = to_device(fi.Q), to_device(fi.K), to_device(fi.V), to_device(dO)
    S_in, z_in = (torch.from_numpy(x).cuda() for x in inputs.positive_state(9107, 1, 2, dp, v.shape[3]))
    dS, dz = (torch.from_numpy(x).cuda() for x in inputs.state_grads(9107, 1, 2, dp, v.shape[3]))

    def run(events):
        return la.la_backward_causal_chunked(q, k, v, g, 64, phi=phi, W=W, S_in=S_in, z_in=z_in, dS_out=dS,
                                             dz_out=dz, state_grad=True, events=events)
    _check(f"backward, {path}", run, expect, slots=BSLOTS, kind=la.LaBackwardEvents, exact=True)
