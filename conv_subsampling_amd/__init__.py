"""Depthwise-convolution path for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libdwconv.so``, whose C ABI is declared in
``include/dwconv.h``.  Every step of every operation runs in the library's
HIP kernels; this module only checks tensor dtypes, devices and layouts,
allocates outputs with torch when the caller gives none, and passes raw
device pointers plus torch's current HIP stream.  It fails loudly when the
library has not been built: there is no other implementation to fall back on.

Layouts are channel-last and contiguous: x [B,T,C] (1-D), [B,T,F,C] (2-D),
[B,T,F] (mel); weights tap-major w [K,C] / [3,3,C]; lengths int32 [B] on the
same device (or None for full length).
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "LIB_PATH", "DwconvError", "abi_version",
    "dwconv1d_fwd", "dwconv1d_stream_fwd", "dwconv1d_bwd", "dwconv1d_bwd_workspace_bytes", "dwsub_fused_fwd", "dwsub_fused_bwd", "dwsub_fused_bwd_workspace_bytes",
    "dwconv2d_fwd", "dwconv2d_bwd", "dwconv2d_bwd_workspace_bytes", "dwconv2d_bwd_noalloc",
    "conv2d_out_shape", "CAUSAL_PADS_2D", "front_out_shape", "out_len",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdwconv.so")

DW_OK, DW_ERR_INVALID_ARG, DW_ERR_UNSUPPORTED, DW_ERR_WORKSPACE, DW_ERR_HIP = 0, -1, -2, -3, -4
DW_F32, DW_BF16 = 0, 1
DW_PAD_SYMMETRIC, DW_PAD_CAUSAL = 0, 1


class DwconvError(RuntimeError):
    """A call into libdwconv.so returned a non-OK status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python conv_subsampling_amd/build.py, or __graft_entry__.build())")

_vp, _i64, _sz, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int


def _bind(path: str) -> ctypes.CDLL:
    """Load a build of the library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.dw_abi_version.restype = _int
    lib.dw_abi_version.argtypes = []
    lib.dw_last_error.restype = ctypes.c_char_p
    lib.dw_last_error.argtypes = []
    lib.dwconv1d_fwd.restype = _int
    lib.dwconv1d_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _int, _vp]
    lib.dwconv1d_stream_fwd.restype = _int
    lib.dwconv1d_stream_fwd.argtypes = [_vp] * 7 + [_i64] * 4 + [_int, _vp]
    lib.dwconv1d_bwd_workspace_bytes.restype = _sz
    lib.dwconv1d_bwd_workspace_bytes.argtypes = [_i64] * 4
    lib.dwconv1d_bwd.restype = _int
    lib.dwconv1d_bwd.argtypes = [_vp] * 8 + [_sz] + [_i64] * 4 + [_int, _int, _vp]
    lib.dwsub_fused_fwd_ex.restype = _int
    lib.dwsub_fused_fwd_ex.argtypes = [_vp] * 7 + [_i64] * 4 + [_int, _int, _vp]
    lib.dwsub_fused_bwd_workspace_bytes_ex.restype = _sz
    lib.dwsub_fused_bwd_workspace_bytes_ex.argtypes = [_i64] * 4 + [_int]
    lib.dwsub_fused_bwd_ex.restype = _int
    lib.dwsub_fused_bwd_ex.argtypes = [_vp] * 11 + [_sz] + [_i64] * 4 + [_int, _int, _vp]
    lib.dwsub_fused_fwd.restype = _int
    lib.dwsub_fused_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _vp]
    lib.dwsub_fused_bwd_workspace_bytes.restype = _sz
    lib.dwsub_fused_bwd_workspace_bytes.argtypes = [_i64] * 4
    lib.dwsub_fused_bwd.restype = _int
    lib.dwsub_fused_bwd.argtypes = [_vp] * 11 + [_sz] + [_i64] * 4 + [_vp]
    lib.dwconv2d_fwd.restype = _int
    lib.dwconv2d_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp] + [_i64] * 8 + [_vp]
    lib.dwconv2d_bwd_workspace_bytes.restype = _sz
    lib.dwconv2d_bwd_workspace_bytes.argtypes = [_i64] * 8
    lib.dwconv2d_bwd.restype = _int
    lib.dwconv2d_bwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz] + [_i64] * 8 + [_vp]
    lib.dwconv2d_fwd_ex.restype = _int
    lib.dwconv2d_fwd_ex.argtypes = [_vp] * 5 + [_i64] * 11 + [_int, _vp]
    lib.dwconv2d_bwd_workspace_bytes_ex.restype = _sz
    lib.dwconv2d_bwd_workspace_bytes_ex.argtypes = [_i64] * 11
    lib.dwconv2d_bwd_ex.restype = _int
    lib.dwconv2d_bwd_ex.argtypes = [_vp] * 8 + [_sz] + [_i64] * 11 + [_int, _vp]
    lib.dwconv2d_bwd_noalloc.restype = _int
    lib.dwconv2d_bwd_noalloc.argtypes = [_vp] * 7 + [_i64] * 11 + [_int, _vp]
    return lib


_lib = _bind(LIB_PATH)


def abi_version() -> int:
    return _lib.dw_abi_version()


def _check(status: int) -> None:
    if status != DW_OK:
        raise DwconvError(status, _lib.dw_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(name, t, dtype, device, shape=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def out_len(n: int) -> int:
    """Output length of a 3x3 / stride 2 / pad 1 convolution along one axis."""
    return (n + 1) // 2


def dwconv1d_fwd(x, w, bias=None, lengths=None, y=None, causal: bool = False):
    """Depthwise Conv1d in SSM_CONV form; x [B,T,C], w [K,C] (float32 or bfloat16)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    dev, dt = x.device, x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("dwconv1d_fwd takes float32 or bfloat16 tensors")
    B, T, C = x.shape
    _dev_tensor("x", x, dt, dev)
    if w.dim() != 2 or w.shape[1] != C:
        raise ValueError("w must be [K, C]")
    _dev_tensor("w", w, dt, dev)
    K = w.shape[0]
    _dev_tensor("bias", bias, dt, dev, (C,), allow_none=True)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    if y is None:
        y = torch.empty_like(x)
    _dev_tensor("y", y, dt, dev, (B, T, C))
    _check(_lib.dwconv1d_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(lengths), _ptr(y), B, T, C, K,
                             DW_PAD_CAUSAL if causal else DW_PAD_SYMMETRIC,
                             DW_BF16 if dt == torch.bfloat16 else DW_F32, _stream(dev)))
    return y


def dwconv1d_stream_fwd(x, w, bias, lengths, cache_in, cache_out=None, y=None):
    """One chunk x [B,Tc,C] of a causal 1-D depthwise conv after the cached
    K-1 frames cache_in [B,K-1,C]; returns (y, cache_out).  cache_out must be
    a different tensor from cache_in (it is allocated when not given)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, Tc, C]")
    dev, dt = x.device, x.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError(f"x must be float32 or bfloat16, not {dt}")
    B, Tc, C = x.shape
    _dev_tensor("x", x, dt, dev)
    if w.dim() != 2 or w.shape[1] != C:
        raise ValueError("w must be [K, C]")
    _dev_tensor("w", w, dt, dev)
    K = w.shape[0]
    _dev_tensor("bias", bias, dt, dev, (C,), allow_none=True)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    _dev_tensor("cache_in", cache_in, dt, dev, (B, K - 1, C))
    if cache_out is None:
        cache_out = torch.empty_like(cache_in)
    _dev_tensor("cache_out", cache_out, dt, dev, (B, K - 1, C))
    if y is None:
        y = torch.empty_like(x)
    _dev_tensor("y", y, dt, dev, (B, Tc, C))
    _check(_lib.dwconv1d_stream_fwd(_ptr(x), _ptr(w), _ptr(bias), _ptr(lengths), _ptr(cache_in), _ptr(y),
                                    _ptr(cache_out), B, Tc, C, K, DW_BF16 if dt == torch.bfloat16 else DW_F32,
                                    _stream(dev)))
    return y, cache_out


def dwconv1d_bwd_workspace_bytes(B, T, C, K) -> int:
    return int(_lib.dwconv1d_bwd_workspace_bytes(B, T, C, K))


def dwconv1d_bwd(x, w, lengths, dy, dx=None, dw=None, db=None, workspace=None, causal: bool = False,
                 need=("dx", "dw", "db")):
    """Gradients (dx, dw, db) of dwconv1d_fwd given dy [B,T,C].  x, w, dy and
    dx share one storage type (float32 or bfloat16); dw and db are float32."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    dev, f32 = x.device, torch.float32
    st, code = _storage(x)
    B, T, C = x.shape
    _dev_tensor("x", x, st, dev)
    if w.dim() != 2 or w.shape[1] != C:
        raise ValueError("w must be [K, C]")
    _dev_tensor("w", w, st, dev)
    K = w.shape[0]
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    _dev_tensor("dy", dy, st, dev, (B, T, C))
    if dx is None and "dx" in need:
        dx = torch.empty_like(x)
    if dw is None and "dw" in need:
        dw = torch.empty((K, C), dtype=f32, device=dev)
    if db is None and "db" in need:
        db = torch.empty((C,), dtype=f32, device=dev)
    _dev_tensor("dx", dx, st, dev, (B, T, C), allow_none=True)
    _dev_tensor("dw", dw, f32, dev, (K, C), allow_none=True)
    _dev_tensor("db", db, f32, dev, (C,), allow_none=True)
    ws_bytes = 0
    if dw is not None or db is not None:
        need_ws = dwconv1d_bwd_workspace_bytes(B, T, C, K)
        if workspace is None:
            workspace = torch.empty((max(need_ws, 1),), dtype=torch.uint8, device=dev)
        _dev_tensor("workspace", workspace, torch.uint8, dev)
        ws_bytes = workspace.numel()
    _check(_lib.dwconv1d_bwd(_ptr(x), _ptr(w), _ptr(lengths), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db),
                             _ptr(workspace), ws_bytes, B, T, C, K,
                             DW_PAD_CAUSAL if causal else DW_PAD_SYMMETRIC, code, _stream(dev)))
    return dx, dw, db


def front_out_shape(T, F, causal: bool = False):
    """(T2, F2) of the fused front: two stride-2 stages, each padding 1 before
    and after (symmetric) or 2 before and 1 after (causal)."""
    d = 1 if causal else 0
    half = lambda n: (n - 1 + d) // 2 + 1 if n > 0 else d
    return half(half(T)), half(half(F))


def dwsub_fused_fwd(x, w0, b0, w1, b1, lengths=None, y=None, causal: bool = False):
    """Fused subsampler front; x [B,T,F] mel -> y [B,T2,F2,C].  x, the
    parameters and y share one storage type (float32 or bfloat16)."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, F]")
    dev = x.device
    st, code = _storage(x)
    B, T, F = x.shape
    _dev_tensor("x", x, st, dev)
    if w0.dim() != 3 or w0.shape[:2] != (3, 3):
        raise ValueError("w0 must be [3, 3, C]")
    C = w0.shape[2]
    _dev_tensor("w0", w0, st, dev)
    _dev_tensor("b0", b0, st, dev, (C,), allow_none=True)
    _dev_tensor("w1", w1, st, dev, (3, 3, C))
    _dev_tensor("b1", b1, st, dev, (C,), allow_none=True)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    T2, F2 = front_out_shape(T, F, causal)
    if y is None:
        y = torch.empty((B, T2, F2, C), dtype=st, device=dev)
    _dev_tensor("y", y, st, dev, (B, T2, F2, C))
    _check(_lib.dwsub_fused_fwd_ex(_ptr(x), _ptr(w0), _ptr(b0), _ptr(w1), _ptr(b1), _ptr(lengths), _ptr(y),
                                   B, T, F, C, DW_PAD_CAUSAL if causal else DW_PAD_SYMMETRIC, code, _stream(dev)))
    return y


def dwsub_fused_bwd_workspace_bytes(B, T, F, C, causal: bool = False) -> int:
    return int(_lib.dwsub_fused_bwd_workspace_bytes_ex(B, T, F, C, DW_PAD_CAUSAL if causal else DW_PAD_SYMMETRIC))


def dwsub_fused_bwd(x, w0, b0, w1, lengths, dy, dw0=None, db0=None, dw1=None, db1=None, workspace=None,
                    need=("dw0", "db0", "dw1", "db1"), causal: bool = False):
    """Parameter gradients (dw0, db0, dw1, db1) of dwsub_fused_fwd given dy
    [B,T2,F2,C].  x, w0, b0, w1 and dy share one storage type; the gradients
    are float32."""
    if x.dim() != 3:
        raise ValueError("x must be [B, T, F]")
    dev, f32 = x.device, torch.float32
    st, code = _storage(x)
    B, T, F = x.shape
    _dev_tensor("x", x, st, dev)
    if w0.dim() != 3 or w0.shape[:2] != (3, 3):
        raise ValueError("w0 must be [3, 3, C]")
    C = w0.shape[2]
    _dev_tensor("w0", w0, st, dev)
    _dev_tensor("b0", b0, st, dev, (C,), allow_none=True)
    _dev_tensor("w1", w1, st, dev, (3, 3, C))
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    T2, F2 = front_out_shape(T, F, causal)
    _dev_tensor("dy", dy, st, dev, (B, T2, F2, C))
    outs = {}
    for name, t, shape in (("dw0", dw0, (3, 3, C)), ("db0", db0, (C,)), ("dw1", dw1, (3, 3, C)), ("db1", db1, (C,))):
        if t is None and name in need:
            t = torch.empty(shape, dtype=f32, device=dev)
        outs[name] = _dev_tensor(name, t, f32, dev, shape, allow_none=True)
    need_ws = dwsub_fused_bwd_workspace_bytes(B, T, F, C, causal)
    if workspace is None:
        workspace = torch.empty((max(need_ws, 1),), dtype=torch.uint8, device=dev)
    _dev_tensor("workspace", workspace, torch.uint8, dev)
    _check(_lib.dwsub_fused_bwd_ex(_ptr(x), _ptr(w0), _ptr(b0), _ptr(w1), _ptr(lengths), _ptr(dy),
                                   _ptr(outs["dw0"]), _ptr(outs["db0"]), _ptr(outs["dw1"]), _ptr(outs["db1"]),
                                   _ptr(workspace), workspace.numel(), B, T, F, C,
                                   DW_PAD_CAUSAL if causal else DW_PAD_SYMMETRIC, code, _stream(dev)))
    return outs["dw0"], outs["db0"], outs["dw1"], outs["db1"]


def _conv2d_dims(x, w):
    if x.dim() != 4:
        raise ValueError("x must be [B, T, F, C]")
    B, T, F, C = x.shape
    if w.dim() != 3 or w.shape[2] != C:
        raise ValueError("w must be [KH, KW, C]")
    return B, T, F, C, w.shape[0], w.shape[1]


CAUSAL_PADS_2D = (2, 1, 2, 1)   # kernel - 1 before, stride - 1 after, on each axis (3x3, stride 2)


def _pads(pad, pads):
    if pads is None:
        return (pad, pad, pad, pad)
    pads = tuple(int(v) for v in pads)
    if len(pads) != 4:
        raise ValueError("pads must be (time before, time after, freq before, freq after)")
    return pads


def conv2d_out_shape(T, F, KH=3, KW=3, stride=2, pad=1, pads=None):
    """(T', F') of the conv2d for these sizes and pads."""
    pt0, pt1, pf0, pf1 = _pads(pad, pads)
    return max(0, (T + pt0 + pt1 - KH) // stride + 1), max(0, (F + pf0 + pf1 - KW) // stride + 1)


def _storage(x):
    if x.dtype == torch.float32:
        return torch.float32, DW_F32
    if x.dtype == torch.bfloat16:
        return torch.bfloat16, DW_BF16
    raise TypeError(f"x must be float32 or bfloat16, not {x.dtype}")


def dwconv2d_fwd(x, w, bias=None, lengths=None, y=None, stride: int = 2, pad: int = 1, pads=None):
    """Masked depthwise conv2d; x [B,T,F,C], w [3,3,C] -> y [B,T',F',C].
    x, w, bias and y share one storage type (float32 or bfloat16); pads =
    (time before, time after, freq before, freq after) overrides pad
    (CAUSAL_PADS_2D is the causal padding)."""
    dev = x.device
    st, code = _storage(x)
    B, T, F, C, KH, KW = _conv2d_dims(x, w)
    _dev_tensor("x", x, st, dev)
    _dev_tensor("w", w, st, dev)
    _dev_tensor("bias", bias, st, dev, (C,), allow_none=True)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    pt0, pt1, pf0, pf1 = _pads(pad, pads)
    To, Fo = conv2d_out_shape(T, F, KH, KW, stride, pads=(pt0, pt1, pf0, pf1))
    if y is None:
        y = torch.empty((B, To, Fo, C), dtype=st, device=dev)
    _dev_tensor("y", y, st, dev, (B, To, Fo, C))
    _check(_lib.dwconv2d_fwd_ex(_ptr(x), _ptr(w), _ptr(bias), _ptr(lengths), _ptr(y),
                                B, T, F, C, KH, KW, stride, pt0, pt1, pf0, pf1, code, _stream(dev)))
    return y


def dwconv2d_bwd_workspace_bytes(B, T, F, C, KH=3, KW=3, stride=2, pad=1, pads=None) -> int:
    pt0, pt1, pf0, pf1 = _pads(pad, pads)
    return int(_lib.dwconv2d_bwd_workspace_bytes_ex(B, T, F, C, KH, KW, stride, pt0, pt1, pf0, pf1))


def dwconv2d_bwd(x, w, lengths, dy, dx=None, dw=None, db=None, workspace=None,
                 need=("dx", "dw", "db"), stride: int = 2, pad: int = 1, pads=None):
    """Gradients (dx, dw, db) of dwconv2d_fwd given dy; outputs not in `need`
    are skipped (None).  x, w, dy and dx share one storage type; dw and db
    are float32."""
    dev, f32 = x.device, torch.float32
    st, code = _storage(x)
    B, T, F, C, KH, KW = _conv2d_dims(x, w)
    _dev_tensor("x", x, st, dev)
    _dev_tensor("w", w, st, dev)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    pt0, pt1, pf0, pf1 = _pads(pad, pads)
    To, Fo = conv2d_out_shape(T, F, KH, KW, stride, pads=(pt0, pt1, pf0, pf1))
    _dev_tensor("dy", dy, st, dev, (B, To, Fo, C))
    if dx is None and "dx" in need:
        dx = torch.empty_like(x)
    if dw is None and "dw" in need:
        dw = torch.empty((KH, KW, C), dtype=f32, device=dev)
    if db is None and "db" in need:
        db = torch.empty((C,), dtype=f32, device=dev)
    _dev_tensor("dx", dx, st, dev, (B, T, F, C), allow_none=True)
    _dev_tensor("dw", dw, f32, dev, (KH, KW, C), allow_none=True)
    _dev_tensor("db", db, f32, dev, (C,), allow_none=True)
    ws_bytes = 0
    if dw is not None or db is not None:
        need_ws = dwconv2d_bwd_workspace_bytes(B, T, F, C, KH, KW, stride, pads=(pt0, pt1, pf0, pf1))
        if workspace is None:
            workspace = torch.empty((max(need_ws, 1),), dtype=torch.uint8, device=dev)
        _dev_tensor("workspace", workspace, torch.uint8, dev)
        ws_bytes = workspace.numel()
    _check(_lib.dwconv2d_bwd_ex(_ptr(x), _ptr(w), _ptr(lengths), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db),
                                _ptr(workspace), ws_bytes, B, T, F, C, KH, KW, stride, pt0, pt1, pf0, pf1, code,
                                _stream(dev)))
    return dx, dw, db


def dwconv2d_bwd_noalloc(x, w, lengths, dy, dx=None, dw=None, db=None, stride: int = 2, pad: int = 1, pads=None):
    """dwconv2d_bwd through the allocation-free entry point: the caller gives
    every output it wants (None skips it) and no workspace; the library keeps
    the partial sums in its own per-device scratch array.  Nothing here
    allocates device memory.  Calls that overlap in time on one GPU race."""
    dev, f32 = x.device, torch.float32
    st, code = _storage(x)
    B, T, F, C, KH, KW = _conv2d_dims(x, w)
    _dev_tensor("x", x, st, dev)
    _dev_tensor("w", w, st, dev)
    _dev_tensor("lengths", lengths, torch.int32, dev, (B,), allow_none=True)
    pt0, pt1, pf0, pf1 = _pads(pad, pads)
    To, Fo = conv2d_out_shape(T, F, KH, KW, stride, pads=(pt0, pt1, pf0, pf1))
    _dev_tensor("dy", dy, st, dev, (B, To, Fo, C))
    _dev_tensor("dx", dx, st, dev, (B, T, F, C), allow_none=True)
    _dev_tensor("dw", dw, f32, dev, (KH, KW, C), allow_none=True)
    _dev_tensor("db", db, f32, dev, (C,), allow_none=True)
    _check(_lib.dwconv2d_bwd_noalloc(_ptr(x), _ptr(w), _ptr(lengths), _ptr(dy), _ptr(dx), _ptr(dw), _ptr(db),
                                     B, T, F, C, KH, KW, stride, pt0, pt1, pf0, pf1, code, _stream(dev)))
    return dx, dw, db
