"""GPU parity of the backward of the causal form (la_backward_causal_chunked,
through the C ABI) against the oracle's reverse-mode gradients.

Metric: per (b, h) slice, max |gpu - oracle| / max |oracle| over the slice
(tests/parity.py slice_rel_err), for dQ, dK, dV and the starting-state
gradients; 1e-4 for fp32 storage, 2e-2 for bf16 storage (fp32 arithmetic,
outputs rounded once).  The oracle gets exactly the stored input values.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from kernelized_linear_attention_la_amd import inputs
from kernelized_linear_attention_la_amd import linattn as la
from tests.parity import slice_rel_err, to_device, to_f64, tol_for

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[backward]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    la.lib()
    yield
    torch.cuda.synchronize()


def _scale(phi, dk):
    return dk ** -0.25 if phi == "favor" else dk ** -0.5


def _run(seed, B, H, N, dk, dv, dtype, phi, m, chunk, state, slices=None, workspace_fill=None):
    fi = inputs.custom_inputs(seed, B, H, N, dk, dv, scale=_scale(phi, dk), dtype=dtype, phi=phi, m=m)
    dO = inputs.grad_output(1000 + seed, B, H, N, dv, dtype)
    dp = m if phi == "favor" else dk
    S_in = z_in = dS = dz = None
    if state:
        S_in, z_in = inputs.positive_state(1000 + seed, B, H, dp, dv)
        dS, dz = inputs.state_grads(1000 + seed, B, H, dp, dv)
    q, k, v, dOt = to_device(fi.Q), to_device(fi.K), to_device(fi.V), to_device(dO)
    W = torch.from_numpy(fi.W).cuda() if fi.W is not None else None
    dev = lambda x: None if x is None else torch.from_numpy(x).cuda()  # noqa: E731
    ws = None
    if workspace_fill is not None:
        p = la._problem_of(q, v, phi, W)
        ws = torch.full((la.la_backward_workspace_bytes(p, chunk),), workspace_fill, dtype=torch.uint8, device="cuda")
    got = la.la_backward_causal_chunked(q, k, v, dOt, chunk, phi=phi, W=W, S_in=dev(S_in), z_in=dev(z_in),
                                        dS_out=dev(dS), dz_out=dev(dz), state_grad=True, workspace=ws)
    torch.cuda.synchronize()
    got = [to_f64(t) for t in got]
    sel = (slice(None), slice(None)) if slices is None else slices
    pick = lambda x: None if x is None else x[sel]  # noqa: E731
    ref = oracle.causal_backward(phi, pick(fi.Q.f32), pick(fi.K.f32), pick(fi.V.f32), pick(dO.f32), W=fi.W,
                                 S_in=pick(S_in), z_in=pick(z_in), dS_out=pick(dS), dz_out=pick(dz))
    return [g[sel] for g in got], ref


def _check(got, ref, dtype, what, vanish=()):
    """vanish: gradients that are exactly zero in exact arithmetic (the oracle's
    are rounding noise); they are held to tol * the slice's largest dV instead."""
    tol = tol_for(dtype)
    names = ("dQ", "dK", "dV", "dS_in", "dz_in")
    for n in vanish:
        g = got[names.index(n)]
        bound = tol * np.abs(ref[2]).max()
        _say(what, n, "max |.|", float(np.abs(g).max()), "bound", bound)
        assert np.abs(g).max() <= bound, (n, what)
    errs = {n: slice_rel_err(g, r) for n, g, r in zip(names, got, ref) if n not in vanish}
    _say(what, {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e < tol, (n, e, what)
        assert np.isfinite(got[names.index(n)]).all(), n


CASES = [
    # (B, H, N, dk, dv, dtype, phi, m, chunk, state)
    (1, 2, 256, 64, 64, "f32", "elu1", 0, 64, False),   # the fp32 workload's shape
    (1, 2, 256, 64, 64, "f32", "elu1", 0, 64, True),
    (2, 3, 100, 16, 8, "f32", "elu1", 0, 16, True),     # several tiles and chunks, ragged tail
    (1, 1, 1, 32, 32, "f32", "elu1", 0, 64, False),     # one token: dV = dO, dQ = dK = 0
    (1, 1, 40, 5, 3, "f32", "elu1", 0, 32, True),       # odd widths
    (2, 1, 77, 16, 8, "f32", "favor", 24, 32, True),
    (2, 2, 333, 64, 64, "bf16", "elu1", 0, 64, False),
    (1, 2, 2048, 64, 64, "bf16", "elu1", 0, 64, True),   # d64 matrix cores, 32 one-chunk segments a slice:
                                                         # the passes' starting-state gathers span four rounds
    (1, 2, 190, 64, 64, "bf16", "favor", 256, 64, True),  # largest FAVOR+ feature count
    (1, 2, 300, 128, 128, "bf16", "elu1", 0, 128, True),  # largest widths (matrix cores, 32-token tiles)
    (1, 1, 517, 128, 96, "f32", "elu1", 0, 16, True),
    (2, 2, 333, 128, 128, "bf16", "elu1", 0, 32, True),   # d128 matrix cores, ragged tail
    (1, 3, 1000, 128, 128, "bf16", "elu1", 0, 64, False),
    (1, 2, 150, 128, 128, "bf16", "elu1", 0, 16, True),   # d128 bf16 on the fp32-arithmetic kernels
    (1, 1, 17, 128, 128, "bf16", "elu1", 0, 128, True),   # one partial tile
    # fp32 storage on the matrix-core kernels (fp32 arithmetic, 1e-4)
    (2, 2, 700, 64, 64, "f32", "elu1", 0, 64, True),
    (1, 2, 333, 128, 128, "f32", "elu1", 0, 32, True),
    (1, 1, 1000, 128, 128, "f32", "elu1", 0, 128, False),
]


@pytest.mark.parametrize("ci", range(len(CASES)),
                         ids=[f"B{c[0]}H{c[1]}N{c[2]}dk{c[3]}dv{c[4]}{c[5]}{c[6]}C{c[8]}{'S' if c[9] else ''}"
                              for c in CASES])
def test_backward_shapes_against_oracle(ci):
    case = CASES[ci]
    _say("case", case)
    got, ref = _run(ci, *case)
    # one token without a starting state: o_1 = v_1 whatever q_1 and k_1 are
    vanish = ("dQ", "dK") if case[2] == 1 and not case[9] else ()
    _check(got, ref, case[5], case, vanish)


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_backward_chunk_size_does_not_change_the_gradients(chunk):
    _say("chunk", chunk)
    got, ref = _run(77, 1, 2, 300, 32, 32, "f32", "elu1", 0, chunk, True)
    _check(got, ref, "f32", ("chunk", chunk))


def test_backward_ignores_workspace_contents():
    # the backward needs no zero-filled workspace: NaN bytes left in it change nothing
    _say("workspace filled with 0xFF")
    got, ref = _run(5, 2, 2, 200, 64, 64, "f32", "elu1", 0, 64, True, workspace_fill=255)
    _check(got, ref, "f32", "dirty workspace")


def test_backward_d128_matrix_cores_many_segments_and_dirty_workspace():
    # bf16 ELU+1 d128 on the matrix-core kernels: 2 x 4 slices of 4096 tokens
    # give several segments of 32-token tiles per slice, so the forward sums
    # and both passes' gathers of the other segments' sums (the starting
    # state of the dQ pass, the suffix and dS_in of the dK/dV pass) all take
    # part; the workspace starts as 0xFF bytes (no initial contents are needed)
    _say("B2 H4 N4096 d128 bf16 chunk 128, state, dirty workspace (slices (0,1), (1,3))")
    got, ref = _run(9, 2, 4, 4096, 128, 128, "bf16", "elu1", 0, 128, True,
                    slices=(np.array([[0], [1]]), np.array([[1], [3]])), workspace_fill=255)
    _check(got, ref, "bf16", "ELU+1 d128 B2H4N4096")


def test_backward_mid_size_bf16_workload():
    # the bf16 d = 64 workload shape (B4 H8 N2048, chunk 64), every slice
    _say("B4 H8 N2048 d64 bf16")
    got, ref = _run(2, 4, 8, 2048, 64, 64, "bf16", "elu1", 0, 64, False)
    _check(got, ref, "bf16", "B4H8N2048")


def test_backward_long_context_sampled_slices():
    # the long-context shape (B2 H16 N16384 d128, chunk 128): all slices on the
    # GPU, two of them recomputed by the oracle
    _say("B2 H16 N16384 d128 bf16 (slices (0,3), (1,14))")
    got, ref = _run(3, 2, 16, 16384, 128, 128, "bf16", "elu1", 0, 128, False,
                    slices=(np.array([[0], [1]]), np.array([[3], [14]])))
    _check(got, ref, "bf16", "B2H16N16384 sampled")


def test_backward_fp32_kernels_behind_matrix_core_sums():
    # bf16 problems on the fp32-arithmetic backward whose segments are whole
    # 64-token chunks, so the forward sums in front of it run on the matrix
    # cores: ELU+1 d64 asking for 128-token chunks, with a carried state, and
    # FAVOR+ at the B2 H8 N8192 shape (two slices recomputed by the oracle)
    _say("B4 H8 N2048 d64 bf16 chunk 128, state")
    got, ref = _run(6, 4, 8, 2048, 64, 64, "bf16", "elu1", 0, 128, True)
    _check(got, ref, "bf16", "ELU+1 d64 chunk 128")
    _say("B2 H8 N8192 d64 bf16 FAVOR+ m256 (slices (0,2), (1,7))")
    got, ref = _run(7, 2, 8, 8192, 64, 64, "bf16", "favor", 256, 64, False,
                    slices=(np.array([[0], [1]]), np.array([[2], [7]])))
    _check(got, ref, "bf16", "FAVOR+ B2H8N8192 sampled")


def test_backward_sums_on_the_128_token_state_pass():
    # bf16 ELU+1 d64 asking for 128-token chunks at B2 H8 N8192.  The
    # fp32-arithmetic backward tiles 16 tokens and aims at 1024 workgroups:
    # 16 slices x 64 segments of 8 tiles, i.e. segments of exactly 128 tokens,
    # whole chunks of the 128-token matrix-core state pass, which therefore
    # forms the forward sums in front of it (the 64-token pass is taken only
    # when the segments are not whole 128-token chunks).  Two slices are
    # recomputed by the oracle, each with a carried state.
    B, H, N = 2, 8, 8192
    n_tiles = N // 16
    want = -(-1024 // (B * H))
    seg_tiles = -(-n_tiles // want)
    assert seg_tiles * 16 == 128 and N % 128 == 0
    _say("B2 H8 N8192 d64 bf16 chunk 128, state (slices (0,1), (1,6))")
    got, ref = _run(8, B, H, N, 64, 64, "bf16", "elu1", 0, 128, True,
                    slices=(np.array([[0], [1]]), np.array([[1], [6]])))
    _check(got, ref, "bf16", "ELU+1 d64 chunk 128 on 128-token sums")
