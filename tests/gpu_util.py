"""Helpers shared by the GPU parity tests (comparison rules and printing)."""
import sys

import numpy as np
import torch

# Tolerances, elementwise, in the form |gpu - ref| <= tol * (1 + |ref|):
# fp32 storage 1e-5; bf16 storage with fp32 accumulation 2e-2.
TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def say(*a):
    """Name the case before each GPU step, flushed, so a failing run shows where it was."""
    print(*a, flush=True)
    sys.stdout.flush()


def host64(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def assert_parity(gpu, ref, tol, what=""):
    g = host64(gpu)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    if g.size == 0:
        return 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    e = np.abs(g - r) / (1.0 + np.abs(r))
    worst = float(e.max())
    if worst > tol:
        idx = np.unravel_index(int(e.argmax()), e.shape)
        raise AssertionError(f"{what}: max err {worst:.3e} > {tol:.1e} at {idx}: gpu {g[idx]!r} ref {r[idx]!r}")
    return worst


def assert_exact_zero(gpu, mask, what=""):
    g = host64(gpu)
    m = np.broadcast_to(np.asarray(mask, dtype=bool), g.shape)
    bad = np.count_nonzero(g[m] != 0.0)
    assert bad == 0, f"{what}: {bad} masked outputs are not exactly zero"


def time_mask(lengths, B, T, clamp=True):
    """[B, T] boolean: True where the frame index is at or beyond the item's length."""
    L = np.asarray(lengths.cpu() if isinstance(lengths, torch.Tensor) else lengths, dtype=np.int64)
    L = np.clip(L, 0, T) if clamp else L
    return np.arange(T)[None, :] >= L[:, None]


# Canary bit patterns: quiet NaNs with a payload no kernel produces.
_CANARY = {torch.float32: (torch.int32, 0x7FC0BEEF), torch.bfloat16: (torch.int16, 0x7FDE),
           torch.uint8: (torch.uint8, 0xA5)}


class Guarded:
    """An output (or workspace) tensor with G canary elements on each side.

    The canaries and the tensor itself start as the canary pattern (a NaN for
    float storage), so after a call `check()` proves that nothing was written
    outside the tensor, and a finite-output check proves that every element
    inside was written.  G keeps the tensor 16-byte aligned, so the kernels'
    widest lanes still run."""

    def __init__(self, shape, dtype, device, G=1024):
        self.shape, self.dtype, self.G = tuple(shape), dtype, G
        n = 1
        for s in self.shape:
            n *= s
        self.n = n
        idt, pat = _CANARY[dtype]
        self.buf = torch.empty(n + 2 * G, dtype=dtype, device=device)
        self.buf.view(idt).fill_(pat)
        self.t = self.buf[G:G + n].view(self.shape)
        self._pat = pat
        self._idt = idt

    def check(self, what=""):
        raw = self.buf.view(self._idt)
        lo, hi = raw[:self.G], raw[self.G + self.n:]
        bad = int((lo != self._pat).sum()) + int((hi != self._pat).sum())
        assert bad == 0, f"{what}: {bad} guard elements overwritten"

    def untouched_inside(self):
        """Number of elements inside the tensor still holding the canary."""
        return int((self.t.reshape(-1).view(self._idt) == self._pat).sum())
