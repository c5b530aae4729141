"""CPU-side checks of the C-ABI library: it loads, exports every declared entry
point, and its host validation rejects bad arguments before any launch.

None of these calls reaches the GPU: every argument set used here fails
validation (or is a pure host query), so they run on a machine without one.
"""
import ctypes
import os
import re
import subprocess

import pytest

from kernelized_linear_attention_la_amd import linattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "liblinattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(linattn.LIB_PATH), reason="liblinattn.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("la_forward_noncausal", "la_forward_causal_chunked", "la_decode_step", "la_workspace_bytes"):
        assert n in names
    assert set(names) == set(linattn.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = linattn.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", linattn.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (la_\w+)", out))
    for n in declared_functions():
        assert hasattr(lib, n), n
        assert n in exported, n
    # nothing else leaks out of the library under the la_ prefix
    assert exported == set(declared_functions())


def test_abi_version_and_status_strings():
    assert linattn.la_abi_version() == 6
    for s in range(9):
        assert linattn.status_string(s)
    assert "unknown" in linattn.status_string(99)


def _p(**kw):
    d = dict(B=2, H=3, N=100, d_k=64, d_v=64, dtype=linattn.LA_BF16, phi=linattn.LA_PHI_ELU1, m=0, W_ptr=0)
    d.update(kw)
    return linattn.problem(**d)


def test_feature_dim_and_workspace_queries():
    p = _p()
    assert linattn.la_feature_dim(p) == 64
    pf = _p(phi=linattn.LA_PHI_FAVOR, m=256, W_ptr=0x1000)
    assert linattn.la_feature_dim(pf) == 256
    for c in (16, 32, 64, 128):
        ws = linattn.la_workspace_bytes(p, c)
        assert ws >= 0 and ws % 256 == 0
    # invalid inputs give 0
    assert linattn.la_workspace_bytes(p, 48) == 0
    assert linattn.la_workspace_bytes(_p(d_k=129), 64) == 0
    # large problems need segment workspace: B*H*P*(d'*d_v + d') floats
    big = _p(B=2, H=16, N=16384, d_k=128, d_v=128)
    assert linattn.la_workspace_bytes(big, 128) >= 2 * 16 * 2 * (128 * 128 + 128) * 4


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first
MIS = ctypes.c_void_p(0x100004)


def _causal(p, chunk=64, Q=FAKE, K=FAKE, V=FAKE, O=FAKE, Si=None, zi=None, So=None, zo=None, ws=None, wsb=0):
    return linattn.lib().la_forward_causal_chunked(ctypes.byref(p), chunk, Q, K, V, O, Si, zi, So, zo, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), 2), (dict(H=0), 2), (dict(N=0), 2), (dict(d_k=0), 2), (dict(d_k=129), 2), (dict(d_v=200), 2),
    (dict(dtype=7), 3), (dict(phi=9), 4), (dict(m=3), 2),
    (dict(phi=linattn.LA_PHI_FAVOR, m=0, W_ptr=0x1000), 2), (dict(phi=linattn.LA_PHI_FAVOR, m=257, W_ptr=0x1000), 2),
    (dict(phi=linattn.LA_PHI_FAVOR, m=16, W_ptr=0), 1), (dict(phi=linattn.LA_PHI_FAVOR, m=16, W_ptr=0x1004), 5),
])
def test_causal_rejects_bad_problem(kw, status):
    assert _causal(_p(**kw)) == status


def test_causal_rejects_bad_arguments():
    p = _p()
    assert linattn.lib().la_forward_causal_chunked(None, 64, FAKE, FAKE, FAKE, FAKE, None, None, None, None,
                                                   None, 0, None) == 1
    for c in (0, 8, 48, 256, -64):
        assert _causal(p, chunk=c) == 4
    assert _causal(p, Q=None) == 1
    assert _causal(p, O=None) == 1
    assert _causal(p, Si=FAKE) == 1          # S_in without z_in
    assert _causal(p, So=FAKE) == 1          # S_out without z_out
    assert _causal(p, K=MIS) == 5
    assert _causal(p, Si=MIS, zi=FAKE) == 5
    # a problem that needs workspace, called without it
    big = _p(B=1, H=1, N=8192)
    assert linattn.la_workspace_bytes(big, 64) > 0
    assert _causal(big, ws=None, wsb=0) == 6
    need = linattn.la_workspace_bytes(big, 64)
    assert _causal(big, ws=FAKE, wsb=need - 1) == 6


def test_noncausal_and_decode_validation():
    L = linattn.lib()
    p = _p()
    assert L.la_forward_noncausal(ctypes.byref(p), FAKE, FAKE, FAKE, None, None, None, FAKE, 1 << 30, None) == 1
    assert L.la_forward_noncausal(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == 1
    assert L.la_forward_noncausal(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, 0, None) == 6
    assert L.la_forward_noncausal(ctypes.byref(p), FAKE, FAKE, MIS, FAKE, None, None, FAKE, 1 << 30, None) == 5
    # decode: N must be 1, state required
    assert L.la_decode_step(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    p1 = _p(N=1)
    assert L.la_decode_step(ctypes.byref(p1), FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == 1
    assert L.la_decode_step(ctypes.byref(p1), FAKE, FAKE, FAKE, FAKE, FAKE, MIS, None) == 5


def test_python_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 4)
    with pytest.raises(TypeError):
        linattn.la_forward_causal_chunked(q, q, q, 16)


def test_retention_validation():
    L = linattn.lib()
    pid = _p(phi=linattn.LA_PHI_IDENTITY)
    g = FAKE

    def ret(p, gamma=g, chunk=64, Q=FAKE, O=FAKE, Si=None, So=None, ws=None, wsb=0):
        return L.la_forward_retention_chunked(ctypes.byref(p), gamma, chunk, Q, FAKE, FAKE, O, Si, So, ws, wsb,
                                              None, None)

    # the identity map has no normaliser: the normalised entry points refuse it
    assert _causal(pid) == 4
    assert L.la_forward_noncausal(ctypes.byref(pid), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == 4
    assert L.la_decode_step(ctypes.byref(_p(N=1, phi=linattn.LA_PHI_IDENTITY)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            None) == 4
    # retention: decays required and 4-byte aligned, chunk checked, workspace checked
    assert ret(pid, gamma=None) == 1
    assert ret(pid, gamma=ctypes.c_void_p(0x100002)) == 5
    assert ret(pid, chunk=48) == 4
    assert ret(pid, Q=None) == 1
    assert ret(pid, Si=MIS) == 5
    big = _p(B=1, H=1, N=8192, phi=linattn.LA_PHI_IDENTITY)
    need = linattn.la_workspace_bytes(big, 64)
    assert need > 0
    assert ret(big, ws=None, wsb=0) == 6
    assert ret(big, ws=FAKE, wsb=need - 1) == 6
    # decode
    p1 = _p(N=1, phi=linattn.LA_PHI_IDENTITY)
    assert L.la_retention_decode_step(ctypes.byref(p1), None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 1
    assert L.la_retention_decode_step(ctypes.byref(p1), FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == 1
    assert L.la_retention_decode_step(ctypes.byref(pid), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == 2
    # the workspace query covers retention plans of every feature map
    for phi, m, W in ((linattn.LA_PHI_ELU1, 0, 0), (linattn.LA_PHI_FAVOR, 256, 0x1000)):
        pp = _p(B=1, H=2, N=4096, phi=phi, m=m, W_ptr=W)
        assert linattn.la_workspace_bytes(pp, 64) > 0


def test_backward_validation():
    L = linattn.lib()
    p = _p()

    def bwd(p=p, chunk=64, Q=FAKE, dO=FAKE, dQ=FAKE, Si=None, zi=None, dSo=None, dzo=None, dSi=None, dzi=None,
            ws=FAKE, wsb=1 << 40):
        return L.la_backward_causal_chunked(ctypes.byref(p), chunk, Q, FAKE, FAKE, dO, Si, zi, dSo, dzo, dQ, FAKE,
                                            FAKE, dSi, dzi, ws, wsb, None, None)

    need = linattn.la_backward_workspace_bytes(p, 64)
    assert need > 0 and need % 256 == 0
    # G_aug per token alone is B*H*N*(d_v + 1) floats
    assert need >= 2 * 3 * 100 * 65 * 4
    assert linattn.la_backward_workspace_bytes(p, 48) == 0
    assert linattn.la_backward_workspace_bytes(_p(phi=linattn.LA_PHI_IDENTITY), 64) == 0
    # largest supported states: d' (d_v + 1) <= 16640
    assert linattn.la_backward_workspace_bytes(_p(d_k=128, d_v=128), 64) > 0
    assert linattn.la_backward_workspace_bytes(_p(phi=linattn.LA_PHI_FAVOR, m=256, W_ptr=0x1000, d_v=64), 64) > 0
    assert linattn.la_backward_workspace_bytes(_p(phi=linattn.LA_PHI_FAVOR, m=256, W_ptr=0x1000, d_v=65), 64) == 0
    assert bwd(p=_p(phi=linattn.LA_PHI_FAVOR, m=256, W_ptr=0x1000, d_v=65)) == 4
    assert bwd(p=_p(phi=linattn.LA_PHI_IDENTITY)) == 4
    assert bwd(chunk=48) == 4
    assert bwd(Q=None) == 1
    assert bwd(dO=None) == 1
    assert bwd(dQ=None) == 1
    assert bwd(Si=FAKE) == 1                 # S_in without z_in
    assert bwd(dSo=FAKE) == 1                # dS_out without dz_out
    assert bwd(dzi=FAKE) == 1                # dz_in without dS_in
    assert bwd(dO=MIS) == 5
    assert bwd(dSi=FAKE, dzi=MIS) == 5
    assert bwd(ws=None) == 6
    assert bwd(wsb=need - 1) == 6
    assert bwd(p=_p(B=0)) == 2


def test_gated_validation():
    L = linattn.lib()
    pid = _p(phi=linattn.LA_PHI_IDENTITY)
    assert L.la_forward_gla_recurrent(ctypes.byref(_p()), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None) == 4
    assert L.la_forward_gla_recurrent(ctypes.byref(pid), FAKE, FAKE, FAKE, None, None, None, FAKE, None) == 1
    assert L.la_forward_gla_recurrent(ctypes.byref(pid), FAKE, FAKE, FAKE, FAKE, None, None, None, None) == 1
    assert L.la_forward_gla_recurrent(ctypes.byref(pid), MIS, FAKE, FAKE, FAKE, None, None, FAKE, None) == 5
    assert L.la_forward_gla_recurrent(ctypes.byref(pid), FAKE, FAKE, FAKE, ctypes.c_void_p(0x100002), None, None,
                                      FAKE, None) == 5
    # delta: beta required, alpha optional
    assert L.la_forward_delta_recurrent(ctypes.byref(pid), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, None) == 1
    assert L.la_forward_delta_recurrent(ctypes.byref(pid), FAKE, FAKE, FAKE, None, FAKE, MIS, None, FAKE, None) == 5
    assert L.la_forward_delta_recurrent(ctypes.byref(_p(phi=linattn.LA_PHI_IDENTITY, d_k=129)), FAKE, FAKE, FAKE,
                                        None, FAKE, None, None, FAKE, None) == 2


def test_gla_chunked_validation():
    L = linattn.lib()
    pid = _p(phi=linattn.LA_PHI_IDENTITY)
    need = L.la_gla_workspace_bytes(ctypes.byref(pid), 64)
    # the records start past the 256-byte control block that the forward's hand-off keeps;
    # one per (b, h, chunk): QD 64 x 64, (P V)^T and (KE^T V)^T dvp x 64 (d_v rounded up to 16), decay 64
    dvp = -(-pid.d_v // 16) * 16
    assert need == 256 + 4 * pid.B * pid.H * (-(-pid.N // 64)) * (64 * 64 + 2 * dvp * 64 + 64)
    p40 = _p(phi=linattn.LA_PHI_IDENTITY, d_v=40)
    assert L.la_gla_workspace_bytes(ctypes.byref(p40), 64) == \
        256 + 4 * p40.B * p40.H * (-(-p40.N // 64)) * (64 * 64 + 2 * 48 * 64 + 64)
    assert L.la_gla_workspace_bytes(ctypes.byref(pid), 32) == 0
    assert L.la_gla_workspace_bytes(ctypes.byref(_p(phi=linattn.LA_PHI_IDENTITY, d_k=65)), 64) == 0

    def call(p=pid, chunk=64, Q=FAKE, al=FAKE, ws=FAKE, wsb=need):
        return L.la_forward_gla_chunked(ctypes.byref(p), chunk, Q, FAKE, FAKE, al, None, None, FAKE, ws, wsb, None,
                                        None)
    assert call(chunk=128) == 4
    assert call(p=_p(phi=linattn.LA_PHI_IDENTITY, d_k=65)) == 4
    assert call(p=_p()) == 4
    assert call(al=None) == 1
    assert call(Q=MIS) == 5
    assert call(al=ctypes.c_void_p(0x100002)) == 5
    assert call(ws=None) == 6
    assert call(wsb=need - 1) == 6


def test_delta_chunked_validation():
    """la_forward_delta_chunked validates before any launch: shape support,
    pointers, alignment and workspace size (no compute without a GPU)."""
    L = linattn.lib()
    pid = _p(phi=linattn.LA_PHI_IDENTITY)  # d_k = d_v = 64
    need = L.la_delta_workspace_bytes(ctypes.byref(pid), 64)
    # one record per (b, h, chunk): Qt and A (64 x 64), (P Ut)^T and B^T (d_v x 64), fp32
    n_chunks = -(-pid.N // 64)
    assert need == 256 + 4 * pid.B * pid.H * n_chunks * (2 * 64 * 64 + 2 * 64 * pid.d_v)
    assert L.la_delta_workspace_bytes(ctypes.byref(pid), 32) == 0
    assert L.la_delta_workspace_bytes(ctypes.byref(_p(phi=linattn.LA_PHI_IDENTITY, d_k=32)), 64) == 0
    assert L.la_delta_workspace_bytes(ctypes.byref(_p(phi=linattn.LA_PHI_IDENTITY, d_v=40)), 64) == 0
    assert L.la_delta_workspace_bytes(ctypes.byref(_p()), 64) == 0  # ELU+1: raw q, k only

    def call(p=pid, chunk=64, Q=FAKE, al=None, be=FAKE, ws=FAKE, wsb=need):
        return L.la_forward_delta_chunked(ctypes.byref(p), chunk, Q, FAKE, FAKE, al, be, None, None, FAKE, ws, wsb,
                                          None, None)
    assert call(chunk=32) == 4
    assert call(p=_p(phi=linattn.LA_PHI_IDENTITY, d_k=32)) == 4
    assert call(p=_p()) == 4
    assert call(be=None) == 1
    assert call(Q=None) == 1
    assert call(Q=MIS) == 5
    assert call(al=ctypes.c_void_p(0x100002)) == 5
    assert call(ws=None) == 6
    assert call(wsb=need - 1) == 6
    assert call(p=_p(phi=linattn.LA_PHI_IDENTITY, B=0)) == 2


def test_feature_map_parameters_validation():
    pd = lambda **kw: _p(phi=linattn.LA_PHI_DPFP, **kw)  # noqa: E731
    assert linattn.la_feature_dim(pd(map_param=1)) == 128      # 2 d_k nu
    assert linattn.la_feature_dim(pd(d_k=32, map_param=4)) == 256
    assert _causal(pd(map_param=0)) == 2
    assert _causal(pd(map_param=3)) == 2                       # 2 * 64 * 3 > 256
    pt = lambda **kw: _p(phi=linattn.LA_PHI_TRIG, **kw)  # noqa: E731
    assert linattn.la_feature_dim(pt(m=100, W_ptr=0x1000)) == 200
    assert _causal(pt(m=129, W_ptr=0x1000)) == 2
    assert _causal(pt(m=16, W_ptr=0)) == 1
    pc = lambda **kw: _p(phi=linattn.LA_PHI_COSFORMER, **kw)  # noqa: E731
    assert linattn.la_feature_dim(pc(map_param=512)) == 128    # 2 d_k
    assert _causal(pc(map_param=0)) == 2
    assert _causal(pc(map_param=8, pos0=-1)) == 2
    assert _causal(_p(map_param=1)) == 2                       # ELU+1 takes no parameter
    assert linattn.la_feature_dim(_p(map_param=1)) == 0        # invalid problem
    for p in (pd(map_param=1), pt(m=16, W_ptr=0x1000), pc(map_param=100, pos0=7)):
        assert linattn.la_workspace_bytes(p, 64) > 0
        assert linattn.la_backward_workspace_bytes(p, 64) == 0  # no backward for these maps


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus N > 1 exits non-zero with a message, before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr


def test_workspace_error_validation():
    """la_workspace_error checks its pointers, alignment and the control block's size on the host."""
    L = linattn.lib()
    assert L.la_workspace_error(None, 256, FAKE, 0, None) == 1
    assert L.la_workspace_error(FAKE, 256, None, 0, None) == 1
    assert L.la_workspace_error(MIS, 256, FAKE, 0, None) == 5
    assert L.la_workspace_error(FAKE, 256, ctypes.c_void_p(0x100002), 0, None) == 5
    assert L.la_workspace_error(FAKE, 255, FAKE, 1, None) == 6



def test_noalloc_validation_and_scratch_limit():
    """la_forward_causal_chunked_noalloc validates like la_forward_causal_chunked and
    refuses, before touching a device, a problem whose workspace exceeds its fixed array."""
    L = linattn.lib()

    def call(p, chunk=64, Q=FAKE, Si=None, zi=None):
        return L.la_forward_causal_chunked_noalloc(ctypes.byref(p), chunk, Q, FAKE, FAKE, FAKE, Si, zi, None, None,
                                                   None)
    assert call(_p(), Q=None) == 1
    assert call(_p(), Q=MIS) == 5
    assert call(_p(), Si=FAKE) == 1
    assert call(_p(), chunk=48) == 4
    assert call(_p(B=0)) == 2
    big = _p(B=255, H=1, N=256, d_k=128, d_v=128)
    need = linattn.la_workspace_bytes(big, 128)
    assert need > linattn.LA_NOALLOC_SCRATCH_BYTES
    assert call(big, chunk=128) == 8
    assert "scratch" in linattn.status_string(8)
