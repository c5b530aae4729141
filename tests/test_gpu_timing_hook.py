"""GPU test of the per-kernel timing hook (la_kernel_events) through the C ABI.

Every call that takes the hook must report, in `launched`, the kernels it
enqueued, record a positive duration for each of them, and give results bit
for bit equal to the same call without the hook (the events only bracket the
launches).  Covered: the causal single pass (bf16, d = 64), the causal fp32
path in three launches (segment sums, their scan, the chunk pass), and the
chunkwise GLA and gated delta-rule calls (per-chunk launch, state chain,
outputs).
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
    """hipEvent pairs for the three slots, through the runtime the library links."""

    def __init__(self):
        self.lib = la.lib()
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.kev = la.LaKernelEvents()
        self.pairs = {}
        for sl in SLOTS:
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


def _check(name, run, expect):
    """run(events) -> tuple of result tensors; expect: the slots that must be launched."""
    ref = [t.clone() for t in run(None)]
    torch.cuda.synchronize()
    ev = _Events()
    try:
        got = run(ev.kev)
        torch.cuda.synchronize()
        launched = [sl for sl in SLOTS if ev.kev.launched[sl]]
        times = {sl: ev.elapsed_ms(sl) for sl in launched}
        _say(name, "launched", launched, "ms", {k: round(v, 4) for k, v in times.items()})
        assert set(expect) <= set(launched), (launched, expect)
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
