"""Thin ctypes binding of liblinattn (the C ABI in include/liblinattn.h).

The Python functions carry the names of the C entry points and do argument
marshalling only: they check torch dtypes, shapes, devices and contiguity,
allocate outputs and workspace with torch (device memory is torch's job),
pass raw device pointers and the current HIP stream, and raise on a non-zero
status.  Every arithmetic step runs in the HIP kernels of liblinattn.so.
There is no fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblinattn.so")

LA_OK = 0
LA_F32, LA_BF16 = 0, 1
LA_PHI_ELU1, LA_PHI_FAVOR, LA_PHI_IDENTITY, LA_PHI_DPFP, LA_PHI_TRIG, LA_PHI_COSFORMER = 0, 1, 2, 3, 4, 5
_PHI_CODES = {"elu1": LA_PHI_ELU1, "favor": LA_PHI_FAVOR, "identity": LA_PHI_IDENTITY, "dpfp": LA_PHI_DPFP,
              "trig": LA_PHI_TRIG, "cosformer": LA_PHI_COSFORMER}
STATUS_NAMES = {0: "LA_OK", 1: "LA_ERR_NULL", 2: "LA_ERR_SHAPE", 3: "LA_ERR_DTYPE", 4: "LA_ERR_UNSUPPORTED",
                5: "LA_ERR_ALIGN", 6: "LA_ERR_WORKSPACE", 7: "LA_ERR_DEVICE", 8: "LA_ERR_SCRATCH"}
LA_NOALLOC_SCRATCH_BYTES = 32 << 20
EXPORTED = ("la_abi_version", "la_status_string", "la_feature_dim", "la_workspace_bytes",
            "la_forward_noncausal", "la_forward_causal_chunked", "la_forward_causal_chunked_timed",
            "la_decode_step", "la_forward_retention_chunked", "la_retention_decode_step",
            "la_backward_workspace_bytes", "la_backward_causal_chunked", "la_forward_gla_recurrent",
            "la_forward_delta_recurrent", "la_delta_workspace_bytes", "la_forward_delta_chunked",
            "la_gla_workspace_bytes", "la_forward_gla_chunked", "la_workspace_error",
            "la_forward_causal_chunked_noalloc")
LA_KSLOT_STATE, LA_KSLOT_SCAN, LA_KSLOT_CHUNK, LA_KSLOTS = 0, 1, 2, 3
LA_BSLOT_FWD_SUMS, LA_BSLOT_FWD_SCAN, LA_BSLOT_DQ, LA_BSLOT_RSCAN, LA_BSLOT_DKV, LA_BSLOTS = 0, 1, 2, 3, 4, 5


class LaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("N", ctypes.c_int),
                ("d_k", ctypes.c_int), ("d_v", ctypes.c_int),
                ("dtype", ctypes.c_int), ("phi", ctypes.c_int),
                ("m", ctypes.c_int), ("W", ctypes.c_void_p), ("map_param", ctypes.c_int),
                ("pos0", ctypes.c_longlong)]


class LaKernelEvents(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * LA_KSLOTS), ("stop", ctypes.c_void_p * LA_KSLOTS),
                ("launched", ctypes.c_int * LA_KSLOTS)]


class LaBackwardEvents(ctypes.Structure):
    _fields_ = [("start", ctypes.c_void_p * LA_BSLOTS), ("stop", ctypes.c_void_p * LA_BSLOTS),
                ("launched", ctypes.c_int * LA_BSLOTS)]


class LaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load liblinattn.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblinattn is not built ({LIB_PATH} missing); run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(LaProblem)
        vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.la_abi_version.restype = i
        L.la_status_string.restype = ctypes.c_char_p
        L.la_status_string.argtypes = [i]
        L.la_feature_dim.restype = i
        L.la_feature_dim.argtypes = [P]
        L.la_workspace_bytes.restype = sz
        L.la_workspace_bytes.argtypes = [P, i]
        L.la_forward_noncausal.restype = i
        L.la_forward_noncausal.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.la_forward_causal_chunked.restype = i
        L.la_forward_causal_chunked.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.la_forward_causal_chunked_timed.restype = i
        L.la_forward_causal_chunked_timed.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                      ctypes.POINTER(LaKernelEvents)]
        L.la_decode_step.restype = i
        L.la_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.la_forward_retention_chunked.restype = i
        L.la_forward_retention_chunked.argtypes = [P, vp, i, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                   ctypes.POINTER(LaKernelEvents)]
        L.la_retention_decode_step.restype = i
        L.la_retention_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp]
        L.la_backward_workspace_bytes.argtypes = [P, i]
        L.la_backward_workspace_bytes.restype = sz
        L.la_backward_causal_chunked.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                 ctypes.POINTER(LaBackwardEvents)]
        L.la_backward_causal_chunked.restype = i
        L.la_forward_gla_recurrent.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp]
        L.la_forward_gla_recurrent.restype = i
        L.la_forward_delta_recurrent.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.la_forward_delta_recurrent.restype = i
        L.la_delta_workspace_bytes.argtypes = [P, i]
        L.la_delta_workspace_bytes.restype = sz
        L.la_forward_delta_chunked.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                               ctypes.POINTER(LaKernelEvents)]
        L.la_forward_delta_chunked.restype = i
        L.la_gla_workspace_bytes.argtypes = [P, i]
        L.la_gla_workspace_bytes.restype = sz
        L.la_forward_gla_chunked.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                             ctypes.POINTER(LaKernelEvents)]
        L.la_forward_gla_chunked.restype = i
        L.la_workspace_error.argtypes = [vp, sz, vp, i, vp]
        L.la_workspace_error.restype = i
        L.la_forward_causal_chunked_noalloc.argtypes = [P, i, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.la_forward_causal_chunked_noalloc.restype = i
        _lib = L
    return _lib


def la_abi_version() -> int:
    return lib().la_abi_version()


def status_string(status: int) -> str:
    return lib().la_status_string(int(status)).decode()


def problem(B, H, N, d_k, d_v, dtype=LA_F32, phi=LA_PHI_ELU1, m=0, W_ptr=0, map_param=0, pos0=0) -> LaProblem:
    return LaProblem(int(B), int(H), int(N), int(d_k), int(d_v), int(dtype), int(phi), int(m),
                     ctypes.c_void_p(int(W_ptr)) if W_ptr else None, int(map_param), int(pos0))


def la_feature_dim(p: LaProblem) -> int:
    return lib().la_feature_dim(ctypes.byref(p))


def la_workspace_bytes(p: LaProblem, chunk: int) -> int:
    return int(lib().la_workspace_bytes(ctypes.byref(p), int(chunk)))


# ---------------------------------------------------------------------------
# torch marshalling
# ---------------------------------------------------------------------------
_DT = {torch.float32: LA_F32, torch.bfloat16: LA_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check_qkv(q, k, v):
    for name, t in (("Q", q), ("K", k), ("V", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA/HIP tensor")
        if t.dim() != 4:
            raise ValueError(f"{name} must be [B, H, N, d]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype not in _DT:
            raise TypeError(f"{name} must be float32 or bfloat16")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("Q, K, V must share a dtype")
    if q.shape != k.shape or q.shape[:3] != v.shape[:3]:
        raise ValueError(f"shape mismatch Q{tuple(q.shape)} K{tuple(k.shape)} V{tuple(v.shape)}")


def _problem_of(q, v, phi, W, map_param=0, pos0=0):
    """la_problem of a call: phi is a name ("elu1", "favor", "identity", "dpfp",
    "trig", "cosformer") or code; W [m, d_k] float32 for FAVOR+ and the cos/sin
    projections; map_param is DPFP's nu or cosFormer's M; pos0 the position of
    the first token (cosFormer)."""
    B, H, N, dk = q.shape
    dv = v.shape[3]
    code = _PHI_CODES[phi] if isinstance(phi, str) else int(phi)
    if code in (LA_PHI_FAVOR, LA_PHI_TRIG):
        if W is None:
            raise ValueError("this feature map needs the projection W [m, d_k]")
        if W.dtype != torch.float32 or not W.is_contiguous() or not W.is_cuda or W.dim() != 2 or W.shape[1] != dk:
            raise ValueError("W must be a contiguous float32 device tensor [m, d_k]")
        return problem(B, H, N, dk, dv, _DT[q.dtype], code, W.shape[0], W.data_ptr(), map_param, pos0)
    return problem(B, H, N, dk, dv, _DT[q.dtype], code, 0, 0, map_param, pos0)


def _state_pair(S, z, B, H, dp, dv, device, what):
    if S is None and z is None:
        return None, None
    if S is None or z is None:
        raise ValueError(f"{what}: S and z go together")
    if S.dtype != torch.float32 or z.dtype != torch.float32 or not S.is_contiguous() or not z.is_contiguous():
        raise ValueError(f"{what}: S and z must be contiguous float32")
    if tuple(S.shape) != (B, H, dp, dv) or tuple(z.shape) != (B, H, dp):
        raise ValueError(f"{what}: expected S [{B},{H},{dp},{dv}] and z [{B},{H},{dp}]")
    if S.device != device or z.device != device:
        raise ValueError(f"{what}: state must live on the inputs' device")
    return S, z


def _default_workspace(nbytes, device, zeroed, where):
    """A workspace for a call that was given none.  Not while the current
    stream is capturing a graph: the allocation (and, for the forward's
    hand-off, the zero fill) would be recorded into the graph and replayed;
    such callers pass their own workspace, zero-filled once beforehand."""
    if torch.cuda.is_current_stream_capturing():
        raise ValueError(f"{where}: pass workspace= (a device tensor of at least {nbytes} bytes"
                         f"{', zero-filled before its first use' if zeroed else ''}) while the stream is capturing")
    if zeroed:
        return torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def la_workspace_error(workspace, err=None, clear=False, stream=None):
    """Enqueue a copy of the workspace's hand-off error word (0: no wait ever
    expired) into err (int32 device tensor [1], allocated when None) and clear
    the word if asked; returns err (read it after synchronising the stream)."""
    if not isinstance(workspace, torch.Tensor) or not workspace.is_cuda:
        raise TypeError("workspace must be a device tensor")
    if err is None:
        err = torch.empty(1, dtype=torch.int32, device=workspace.device)
    st = lib().la_workspace_error(_ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(err),
                                  1 if clear else 0, _stream(stream))
    _raise(st, "la_workspace_error")
    return err


def _raise(status, where):
    if status != LA_OK:
        raise LaError(status, where)


def la_forward_causal_chunked(q, k, v, chunk=64, phi="elu1", W=None, S_in=None, z_in=None,
                              S_out=None, z_out=None, out=None, workspace=None, stream=None, events=None, map_param=0, pos0=0):
    """Causal chunkwise forward; returns O (same dtype as q).

    S_out/z_out, when given, receive the final state (they may be S_in/z_in).
    workspace: optional uint8 device tensor of la_workspace_bytes(p, chunk)
    bytes, zero-filled before its first use and reused as the last call left it.
    events: optional LaKernelEvents (per-kernel hipEvent records; see
    la_forward_causal_chunked_timed in the C header).
    """
    _check_qkv(q, k, v)
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    S_in, z_in = _state_pair(S_in, z_in, B, H, dp, dv, q.device, "initial state")
    S_out, z_out = _state_pair(S_out, z_out, B, H, dp, dv, q.device, "final state")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    nbytes = la_workspace_bytes(p, chunk)
    if workspace is None and nbytes > 0:
        # a fresh workspace starts zero-filled (the C contract); a caller that
        # passes its own keeps it between calls
        workspace = _default_workspace(nbytes, q.device, True, "la_forward_causal_chunked")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if events is None:
        st = lib().la_forward_causal_chunked(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                             _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                             _ptr(workspace), wsb, _stream(stream))
        _raise(st, "la_forward_causal_chunked")
    else:
        st = lib().la_forward_causal_chunked_timed(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                                   _ptr(out), _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out),
                                                   _ptr(workspace), wsb, _stream(stream), ctypes.byref(events))
        _raise(st, "la_forward_causal_chunked_timed")
    return out


def la_forward_causal_chunked_noalloc(q, k, v, chunk=64, phi="elu1", W=None, S_in=None, z_in=None, S_out=None,
                                      z_out=None, out=None, stream=None, map_param=0, pos0=0):
    """la_forward_causal_chunked with the library's fixed scratch array as the
    workspace (the C call allocates nothing; pass `out` to allocate nothing here
    either).  Returns O."""
    _check_qkv(q, k, v)
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    S_in, z_in = _state_pair(S_in, z_in, B, H, dp, dv, q.device, "initial state")
    S_out, z_out = _state_pair(S_out, z_out, B, H, dp, dv, q.device, "final state")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    st = lib().la_forward_causal_chunked_noalloc(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                                 _ptr(S_in), _ptr(z_in), _ptr(S_out), _ptr(z_out), _stream(stream))
    _raise(st, "la_forward_causal_chunked_noalloc")
    return out


def la_forward_noncausal(q, k, v, phi="elu1", W=None, S_out=None, z_out=None, out=None, workspace=None,
                         stream=None, map_param=0, pos0=0):
    """Non-causal forward; returns O. S_out/z_out, when given, receive phi(K)^T V and phi(K)^T 1."""
    _check_qkv(q, k, v)
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    S_out, z_out = _state_pair(S_out, z_out, B, H, dp, dv, q.device, "state")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    nbytes = la_workspace_bytes(p, 64)
    if workspace is None:
        workspace = _default_workspace(max(nbytes, 1), q.device, False, "la_forward_noncausal")
    wsb = workspace.numel() * workspace.element_size()
    st = lib().la_forward_noncausal(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S_out), _ptr(z_out),
                                    _ptr(workspace), wsb, _stream(stream))
    _raise(st, "la_forward_noncausal")
    return out


def la_decode_step(q, k, v, S, z, phi="elu1", W=None, out=None, stream=None, map_param=0, pos0=0):
    """One decode step; q, k [B,H,1,d_k] (or [B,H,d_k]); v [B,H,1,d_v]. Updates S, z in place; returns o."""
    if q.dim() == 3:
        q, k, v = q.unsqueeze(2), k.unsqueeze(2), v.unsqueeze(2)
    _check_qkv(q, k, v)
    if q.shape[2] != 1:
        raise ValueError("decode takes one token per slice")
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, _, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    S, z = _state_pair(S, z, B, H, dp, dv, q.device, "state")
    if S is None:
        raise ValueError("decode needs the state S, z")
    if out is None:
        out = torch.empty((B, H, 1, dv), dtype=q.dtype, device=q.device)
    st = lib().la_decode_step(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S), _ptr(z),
                              _stream(stream))
    _raise(st, "la_decode_step")
    return out


# ---------------------------------------------------------------------------
# retention (decayed, unnormalised)
# ---------------------------------------------------------------------------
def _check_gamma(gamma, H, device):
    if not isinstance(gamma, torch.Tensor) or gamma.dtype != torch.float32 or not gamma.is_contiguous():
        raise ValueError("gamma must be a contiguous float32 device tensor [H]")
    if tuple(gamma.shape) != (H,) or gamma.device != device:
        raise ValueError(f"gamma must have shape [{H}] on the inputs' device")


def _state_only(S, B, H, dp, dv, device, what):
    if S is None:
        return None
    if S.dtype != torch.float32 or not S.is_contiguous() or tuple(S.shape) != (B, H, dp, dv) or S.device != device:
        raise ValueError(f"{what}: expected a contiguous float32 [{B},{H},{dp},{dv}] tensor on the inputs' device")
    return S


def la_forward_retention_chunked(q, k, v, gamma, chunk=64, phi="identity", W=None, S_in=None, S_out=None, out=None,
                                 workspace=None, stream=None, events=None, map_param=0, pos0=0):
    """Retention (decayed, unnormalised) forward in the blockwise form; returns O.

    gamma: float32 device tensor [H] of per-head decays in (0, 1].
    S_out, when given, receives the final state (it may be S_in).
    """
    _check_qkv(q, k, v)
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    _check_gamma(gamma, H, q.device)
    S_in = _state_only(S_in, B, H, dp, dv, q.device, "initial state")
    S_out = _state_only(S_out, B, H, dp, dv, q.device, "final state")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    nbytes = la_workspace_bytes(p, chunk)
    if workspace is None and nbytes > 0:
        workspace = _default_workspace(nbytes, q.device, True, "la_forward_retention_chunked")
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().la_forward_retention_chunked(ctypes.byref(p), _ptr(gamma), int(chunk), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(out), _ptr(S_in), _ptr(S_out), _ptr(workspace), wsb,
                                            _stream(stream), None if events is None else ctypes.byref(events))
    _raise(st, "la_forward_retention_chunked")
    return out


def la_retention_decode_step(q, k, v, S, gamma, phi="identity", W=None, out=None, stream=None, map_param=0, pos0=0):
    """One retention step; q, k [B,H,1,d_k] (or [B,H,d_k]); v [B,H,1,d_v]. Updates S in place; returns o."""
    if q.dim() == 3:
        q, k, v = q.unsqueeze(2), k.unsqueeze(2), v.unsqueeze(2)
    _check_qkv(q, k, v)
    if q.shape[2] != 1:
        raise ValueError("decode takes one token per slice")
    p = _problem_of(q, v, phi, W, map_param, pos0)
    B, H, _, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    _check_gamma(gamma, H, q.device)
    S = _state_only(S, B, H, dp, dv, q.device, "state")
    if S is None:
        raise ValueError("decode needs the state S")
    if out is None:
        out = torch.empty((B, H, 1, dv), dtype=q.dtype, device=q.device)
    st = lib().la_retention_decode_step(ctypes.byref(p), _ptr(gamma), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(S),
                                        _stream(stream))
    _raise(st, "la_retention_decode_step")
    return out


# ---------------------------------------------------------------------------
# Backward of the causal form
# ---------------------------------------------------------------------------
def la_backward_workspace_bytes(p: LaProblem, chunk: int) -> int:
    return int(lib().la_backward_workspace_bytes(ctypes.byref(p), int(chunk)))


def la_backward_causal_chunked(q, k, v, dO, chunk=64, phi="elu1", W=None, S_in=None, z_in=None, dS_out=None,
                               dz_out=None, state_grad=False, dQ=None, dK=None, dV=None, workspace=None, stream=None,
                               events=None):
    """Gradients of the causal chunkwise forward for dL/dO = dO (and dL/dS_out,
    dL/dz_out when given).  Returns (dQ, dK, dV, dS_in, dz_in); the last two
    are None unless S_in is given or state_grad is True."""
    _check_qkv(q, k, v)
    if not isinstance(dO, torch.Tensor) or dO.shape != v.shape or dO.dtype != v.dtype or not dO.is_contiguous() \
            or dO.device != v.device:
        raise ValueError("dO must be a contiguous device tensor shaped and typed like V")
    p = _problem_of(q, v, phi, W)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    dp = la_feature_dim(p)
    S_in, z_in = _state_pair(S_in, z_in, B, H, dp, dv, q.device, "initial state")
    dS_out, dz_out = _state_pair(dS_out, dz_out, B, H, dp, dv, q.device, "final-state gradient")
    dQ = torch.empty_like(q) if dQ is None else dQ
    dK = torch.empty_like(k) if dK is None else dK
    dV = torch.empty_like(v) if dV is None else dV
    dS_in = dz_in = None
    if state_grad or S_in is not None:
        dS_in = torch.empty((B, H, dp, dv), dtype=torch.float32, device=q.device)
        dz_in = torch.empty((B, H, dp), dtype=torch.float32, device=q.device)
    nbytes = la_backward_workspace_bytes(p, chunk)
    if nbytes == 0:
        raise LaError(4, "la_backward_workspace_bytes")
    if workspace is None:
        workspace = _default_workspace(nbytes, q.device, False, "la_backward_causal_chunked")
    wsb = workspace.numel() * workspace.element_size()
    st = lib().la_backward_causal_chunked(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(dO),
                                          _ptr(S_in), _ptr(z_in), _ptr(dS_out), _ptr(dz_out), _ptr(dQ), _ptr(dK),
                                          _ptr(dV), _ptr(dS_in), _ptr(dz_in), _ptr(workspace), wsb, _stream(stream),
                                          None if events is None else ctypes.byref(events))
    _raise(st, "la_backward_causal_chunked")
    return dQ, dK, dV, dS_in, dz_in


# ---------------------------------------------------------------------------
# Gated and delta-rule states (token-by-token recurrence)
# ---------------------------------------------------------------------------
def _gate(x, shape, device, what):
    if x is None:
        return None
    if not isinstance(x, torch.Tensor) or x.dtype != torch.float32 or not x.is_contiguous() or x.device != device \
            or tuple(x.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous float32 device tensor of shape {tuple(shape)}")
    return x


def _gated_common(q, k, v, S_in, S_out, out):
    _check_qkv(q, k, v)
    B, H, N, dk = q.shape
    dv = v.shape[3]
    p = problem(B, H, N, dk, dv, _DT[q.dtype], LA_PHI_IDENTITY, 0, 0)
    S_in = _state_only(S_in, B, H, dk, dv, q.device, "initial state")
    S_out = _state_only(S_out, B, H, dk, dv, q.device, "final state")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device)
    return p, S_in, S_out, out


def la_forward_gla_recurrent(q, k, v, alpha, S_in=None, S_out=None, out=None, stream=None):
    """GLA with a per-key-channel gate: S_t = diag(alpha_t) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.

    alpha: float32 [B, H, N, d_k].  Returns O."""
    p, S_in, S_out, out = _gated_common(q, k, v, S_in, S_out, out)
    alpha = _gate(alpha, q.shape, q.device, "alpha")
    st = lib().la_forward_gla_recurrent(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(S_in),
                                        _ptr(S_out), _ptr(out), _stream(stream))
    _raise(st, "la_forward_gla_recurrent")
    return out


def la_forward_delta_recurrent(q, k, v, beta, alpha=None, S_in=None, S_out=None, out=None, stream=None):
    """Gated delta rule: S_t = a_t S_{t-1} + b_t k_t (v_t - a_t S_{t-1}^T k_t)^T, o_t = S_t^T q_t.

    beta, alpha: float32 [B, H, N] (alpha None: the plain delta rule).  Returns O."""
    p, S_in, S_out, out = _gated_common(q, k, v, S_in, S_out, out)
    beta = _gate(beta, q.shape[:3], q.device, "beta")
    alpha = _gate(alpha, q.shape[:3], q.device, "alpha")
    st = lib().la_forward_delta_recurrent(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                          _ptr(S_in), _ptr(S_out), _ptr(out), _stream(stream))
    _raise(st, "la_forward_delta_recurrent")
    return out


def la_delta_workspace_bytes(q, v, chunk=64):
    """Workspace bytes of la_forward_delta_chunked for q [B,H,N,d_k], v [B,H,N,d_v] (0: unsupported)."""
    B, H, N, dk = q.shape
    p = problem(B, H, N, dk, v.shape[3], _DT[q.dtype], LA_PHI_IDENTITY, 0, 0)
    return lib().la_delta_workspace_bytes(ctypes.byref(p), int(chunk))


def la_forward_delta_chunked(q, k, v, beta, alpha=None, S_in=None, S_out=None, out=None, chunk=64, workspace=None,
                             stream=None, events=None):
    """The gated delta rule of la_forward_delta_recurrent in chunkwise form (64-token chunks, d_k = 64,
    d_v a multiple of 16 up to 128).  workspace: a device tensor of at least la_delta_workspace_bytes
    bytes (allocated here when None).  Returns O."""
    p, S_in, S_out, out = _gated_common(q, k, v, S_in, S_out, out)
    beta = _gate(beta, q.shape[:3], q.device, "beta")
    alpha = _gate(alpha, q.shape[:3], q.device, "alpha")
    if workspace is None:
        workspace = _default_workspace(max(la_delta_workspace_bytes(q, v, chunk), 16), q.device, False,
                                       "la_forward_delta_chunked")
    wsb = workspace.numel() * workspace.element_size()
    st = lib().la_forward_delta_chunked(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(beta), _ptr(S_in), _ptr(S_out), _ptr(out), _ptr(workspace), wsb,
                                        _stream(stream), None if events is None else ctypes.byref(events))
    _raise(st, "la_forward_delta_chunked")
    return out


def la_gla_workspace_bytes(q, v, chunk=64):
    """Workspace bytes of la_forward_gla_chunked for q [B,H,N,d_k], v [B,H,N,d_v] (0: unsupported)."""
    B, H, N, dk = q.shape
    p = problem(B, H, N, dk, v.shape[3], _DT[q.dtype], LA_PHI_IDENTITY, 0, 0)
    return lib().la_gla_workspace_bytes(ctypes.byref(p), int(chunk))


def la_forward_gla_chunked(q, k, v, alpha, S_in=None, S_out=None, out=None, chunk=64, workspace=None, stream=None,
                           events=None):
    """GLA of la_forward_gla_recurrent in two launches (per-chunk products once, then the scan over chunks per
    16 value columns; d_k <= 64).  workspace: a device tensor of at least la_gla_workspace_bytes bytes
    (allocated here when None).  Returns O."""
    p, S_in, S_out, out = _gated_common(q, k, v, S_in, S_out, out)
    alpha = _gate(alpha, q.shape, q.device, "alpha")
    if workspace is None:
        workspace = _default_workspace(max(la_gla_workspace_bytes(q, v, chunk), 16), q.device, False,
                                       "la_forward_gla_chunked")
    wsb = workspace.numel() * workspace.element_size()
    st = lib().la_forward_gla_chunked(ctypes.byref(p), int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(S_in), _ptr(S_out), _ptr(out), _ptr(workspace), wsb, _stream(stream),
                                      None if events is None else ctypes.byref(events))
    _raise(st, "la_forward_gla_chunked")
    return out
