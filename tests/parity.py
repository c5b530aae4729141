"""Helpers for GPU-vs-oracle parity tests: error metrics and device transfer.

Error metric for outputs (one number per call): the largest, over rows
r = (b, h, i), of max_c |y_rc - yref_rc| / max_c |yref_rc|.  Outputs are
weighted means of zero-mean values, so many single entries sit near zero and
an entry-wise relative error would be meaningless; a row's own scale is the
natural yardstick.  States: per (b, h) slice max|dS| / max|S|; z is positive,
so it is compared entry-wise.
"""
from __future__ import annotations

import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to_device(ht, device="cuda"):
    """HostTensor (inputs module) -> torch device tensor in its storage dtype."""
    if ht.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(ht.store)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(ht.store)).to(device)


def to_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def row_rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.abs(ref).max(axis=-1)
    diff = np.abs(y - ref).max(axis=-1)
    scale = np.where(scale > 0, scale, 1.0)
    return float((diff / scale).max()) if diff.size else 0.0


def state_rel_err(S, Sref):
    S = np.asarray(S, np.float64)
    Sref = np.asarray(Sref, np.float64)
    lead = S.shape[:-2]
    d = np.abs(S - Sref).reshape(*lead, -1).max(-1)
    s = np.abs(Sref).reshape(*lead, -1).max(-1)
    s = np.where(s > 0, s, 1.0)
    return float((d / s).max()) if d.size else 0.0


def z_rel_err(z, zref):
    z = np.asarray(z, np.float64)
    zref = np.asarray(zref, np.float64)
    return float((np.abs(z - zref) / np.abs(zref)).max()) if z.size else 0.0


def slice_rel_err(y, ref):
    """Gradients: per (b, h) slice, max |y - ref| over the slice / max |ref| over
    the slice.  Gradient rows can vanish exactly (the first token's dq is 0
    without a starting state), so a row's own scale is no yardstick here; the
    slice's largest gradient is."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    B, H = ref.shape[0], ref.shape[1]
    d = np.abs(y - ref).reshape(B, H, -1).max(-1) if ref.size else np.zeros((B, H))
    s = np.abs(ref).reshape(B, H, -1).max(-1) if ref.size else np.ones((B, H))
    s = np.where(s > 0, s, 1.0)
    return float((d / s).max()) if d.size else 0.0


def tol_for(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


GUARD_BYTES = 256
CANARY = 0xA5


class Guarded:
    """A device tensor with guard bands: `t` is a contiguous view into a larger
    uint8 buffer whose GUARD_BYTES before and after `t` hold CANARY bytes.
    `intact()` is True while no kernel has written outside `t`'s own bytes."""

    def __init__(self, shape, dtype, device="cuda", fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD_BYTES + n + GUARD_BYTES,), CANARY, dtype=torch.uint8, device=device)
        self.n = n
        self.t = self.buf[GUARD_BYTES:GUARD_BYTES + n].view(dtype).view(*shape)
        if fill is not None:
            self.t.fill_(fill)

    def intact(self):
        head, tail = self.buf[:GUARD_BYTES], self.buf[GUARD_BYTES + self.n:]
        return bool((head == CANARY).all()) and bool((tail == CANARY).all())
