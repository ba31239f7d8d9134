"""CPU oracle for the depthwise-convolution path (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark use
this package; the library and its Python binding never import it.  It shares
no code with the HIP path: the arithmetic lives in ``oracle.c`` (plain
single-threaded C, fp64 accumulation), loaded here through ctypes.  Inputs
are float32 numpy arrays (or anything ``numpy.asarray`` accepts), outputs
are float64 numpy arrays.

Parity pins for every function here live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_F = ctypes.POINTER(ctypes.c_float)
_D = ctypes.POINTER(ctypes.c_double)
_I = ctypes.POINTER(ctypes.c_int32)
_L = ctypes.c_long


def compile_c(src: str, out: str) -> str:
    """gcc, plain IEEE arithmetic: no fast-math, no FMA contraction."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.check_call([
        "gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c99",
        "-shared", "-fPIC", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_c(_SRC, _LIB)
    return _LIB


def _bind(path: str):
    """Load a build of oracle.c and declare its C signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_dwconv1d_fwd.argtypes = [_F, _F, _F, _I, _D, _L, _L, _L, _L, ctypes.c_int]
    lib.oracle_dwconv2d_fwd.argtypes = [_F, _F, _F, _I, _D] + [_L] * 11
    lib.oracle_dwconv2d_bwd.argtypes = [_F, _F, _I, _F, _D, _D, _D] + [_L] * 11
    lib.oracle_dwsub_front_fwd.argtypes = [_F, _F, _F, _F, _F, _I, _D, _L, _L, _L, _L, ctypes.c_int]
    lib.oracle_dwsub_front_bwd.argtypes = [_F, _F, _F, _F, _I, _F, _D, _D, _D, _D, _L, _L, _L, _L, ctypes.c_int]
    lib.oracle_dwconv1d_bwd.argtypes = [_F, _F, _I, _F, _D, _D, _D, _L, _L, _L, _L, ctypes.c_int]
    lib.oracle_dwconv1d_stream_fwd.argtypes = [_F, _F, _F, _I, _F, _D, _D, _L, _L, _L, _L]
    for f in (lib.oracle_dwconv1d_fwd, lib.oracle_dwconv2d_fwd, lib.oracle_dwconv2d_bwd,
              lib.oracle_dwsub_front_fwd, lib.oracle_dwsub_front_bwd, lib.oracle_dwconv1d_bwd):
        f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _bind(_LIB)
    return _lib


def _f32(a, shape=None):
    if a is None:
        return None, None
    if hasattr(a, "detach"):  # a torch tensor: take its float32 values on the host
        a = a.detach().float().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    if shape is not None and a.shape != tuple(shape):
        raise ValueError(f"expected shape {tuple(shape)}, got {a.shape}")
    return a, a.ctypes.data_as(_F)


def _lens(lengths, B):
    if lengths is None:
        return None, None
    if hasattr(lengths, "detach"):
        lengths = lengths.detach().cpu().numpy()
    a = np.ascontiguousarray(np.asarray(lengths, dtype=np.int32))
    if a.shape != (B,):
        raise ValueError(f"lengths must have shape ({B},), got {a.shape}")
    return a, a.ctypes.data_as(_I)


def _ptr_d(a):
    return a.ctypes.data_as(_D) if a is not None else None


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid arguments")


def conv_out_len(n: int, k: int, s: int, p: int, p_hi=None) -> int:
    """floor((n + p + p_hi - k) / s) + 1, never below zero: the convolution
    output length with p zeros before the input and p_hi (default p) after."""
    p_hi = p if p_hi is None else p_hi
    return max(0, (n + p + p_hi - k) // s + 1)


def pads_of(pad, pads):
    """(pt0, pt1, pf0, pf1): `pads` if given, else the symmetric `pad`."""
    if pads is None:
        return (pad, pad, pad, pad)
    pads = tuple(int(v) for v in pads)
    if len(pads) != 4:
        raise ValueError("pads must be (time before, time after, freq before, freq after)")
    return pads


def front_pads(causal: bool):
    """The front's padding per axis: (before, after)."""
    return (2, 1) if causal else (1, 1)


def dwconv1d_fwd(x, w, b, lengths, causal: bool):
    """y [B,T,C] of the masked, padded 1-D depthwise conv; x [B,T,C], w [K,C]."""
    xa, xp = _f32(x)
    B, T, C = xa.shape
    wa, wp = _f32(w)
    K = wa.shape[0]
    if wa.shape != (K, C):
        raise ValueError("w must be [K, C]")
    ba, bp = _f32(b, (C,))
    la, lp = _lens(lengths, B)
    y = np.empty((B, T, C), dtype=np.float64)
    _check(_load().oracle_dwconv1d_fwd(xp, wp, bp, lp, _ptr_d(y), B, T, C, K, int(bool(causal))),
           "oracle_dwconv1d_fwd")
    return y


def dwconv1d_stream_fwd(x, w, b, lengths, cache):
    """(y [B,Tc,C], new cache [B,K-1,C]) of the causal 1-D depthwise conv run on
    one chunk x [B,Tc,C] after the cached K-1 frames cache [B,K-1,C]."""
    xa, xp = _f32(x)
    B, Tc, C = xa.shape
    wa, wp = _f32(w)
    K = wa.shape[0]
    if wa.shape != (K, C):
        raise ValueError("w must be [K, C]")
    ba, bp = _f32(b, (C,))
    la, lp = _lens(lengths, B)
    ca, cp = _f32(cache, (B, K - 1, C))
    y = np.empty((B, Tc, C), dtype=np.float64)
    cache_out = np.empty((B, K - 1, C), dtype=np.float64)
    _check(_load().oracle_dwconv1d_stream_fwd(xp, wp, bp, lp, cp, _ptr_d(y), _ptr_d(cache_out), B, Tc, C, K),
           "oracle_dwconv1d_stream_fwd")
    return y, cache_out


def dwconv1d_bwd(x, w, lengths, dy, causal: bool, want=("dx", "dw", "db")):
    """(dx, dw, db) of the masked, padded 1-D depthwise conv given dy [B,T,C]."""
    xa, xp = _f32(x)
    B, T, C = xa.shape
    wa, wp = _f32(w)
    K = wa.shape[0]
    if wa.shape != (K, C):
        raise ValueError("w must be [K, C]")
    la, lp = _lens(lengths, B)
    da, dp = _f32(dy, (B, T, C))
    dx = np.empty((B, T, C), dtype=np.float64) if "dx" in want else None
    dw = np.empty((K, C), dtype=np.float64) if "dw" in want else None
    db = np.empty((C,), dtype=np.float64) if "db" in want else None
    _check(_load().oracle_dwconv1d_bwd(xp, wp, lp, dp, _ptr_d(dx), _ptr_d(dw), _ptr_d(db), B, T, C, K,
                                       int(bool(causal))), "oracle_dwconv1d_bwd")
    return dx, dw, db


def dwconv2d_fwd(x, w, b, lengths, stride: int = 2, pad: int = 1, pads=None):
    """y [B,T',F',C] of the masked depthwise conv2d; x [B,T,F,C], w [KH,KW,C].
    pads = (time before, time after, freq before, freq after) overrides pad."""
    xa, xp = _f32(x)
    B, T, F, C = xa.shape
    wa, wp = _f32(w)
    KH, KW = wa.shape[0], wa.shape[1]
    if wa.shape != (KH, KW, C):
        raise ValueError("w must be [KH, KW, C]")
    ba, bp = _f32(b, (C,))
    la, lp = _lens(lengths, B)
    pt0, pt1, pf0, pf1 = pads_of(pad, pads)
    To, Fo = conv_out_len(T, KH, stride, pt0, pt1), conv_out_len(F, KW, stride, pf0, pf1)
    y = np.empty((B, To, Fo, C), dtype=np.float64)
    _check(_load().oracle_dwconv2d_fwd(xp, wp, bp, lp, _ptr_d(y), B, T, F, C, KH, KW, stride,
                                       pt0, pt1, pf0, pf1), "oracle_dwconv2d_fwd")
    return y


def dwconv2d_bwd(x, w, lengths, dy, stride: int = 2, pad: int = 1, want=("dx", "dw", "db"), pads=None):
    """(dx, dw, db) of the masked depthwise conv2d given dy; entries not in `want` are None."""
    xa, xp = _f32(x)
    B, T, F, C = xa.shape
    wa, wp = _f32(w)
    KH, KW = wa.shape[0], wa.shape[1]
    la, lp = _lens(lengths, B)
    pt0, pt1, pf0, pf1 = pads_of(pad, pads)
    To, Fo = conv_out_len(T, KH, stride, pt0, pt1), conv_out_len(F, KW, stride, pf0, pf1)
    da, dp = _f32(dy, (B, To, Fo, C))
    dx = np.empty((B, T, F, C), dtype=np.float64) if "dx" in want else None
    dw = np.empty((KH, KW, C), dtype=np.float64) if "dw" in want else None
    db = np.empty((C,), dtype=np.float64) if "db" in want else None
    _check(_load().oracle_dwconv2d_bwd(xp, wp, lp, dp, _ptr_d(dx), _ptr_d(dw), _ptr_d(db),
                                       B, T, F, C, KH, KW, stride, pt0, pt1, pf0, pf1), "oracle_dwconv2d_bwd")
    return dx, dw, db


def dwsub_front_fwd(x, w0, b0, w1, b1, lengths, causal: bool = False):
    """y [B,T2,F2,C] of the subsampler front; x [B,T,F] (one mel channel)."""
    xa, xp = _f32(x)
    B, T, F = xa.shape
    w0a, w0p = _f32(w0)
    C = w0a.shape[2]
    if w0a.shape != (3, 3, C):
        raise ValueError("w0 must be [3, 3, C]")
    b0a, b0p = _f32(b0, (C,))
    w1a, w1p = _f32(w1, (3, 3, C))
    b1a, b1p = _f32(b1, (C,))
    la, lp = _lens(lengths, B)
    pl, ph = front_pads(causal)
    T1, F1 = conv_out_len(T, 3, 2, pl, ph), conv_out_len(F, 3, 2, pl, ph)
    T2, F2 = conv_out_len(T1, 3, 2, pl, ph), conv_out_len(F1, 3, 2, pl, ph)
    y = np.empty((B, T2, F2, C), dtype=np.float64)
    _check(_load().oracle_dwsub_front_fwd(xp, w0p, b0p, w1p, b1p, lp, _ptr_d(y), B, T, F, C, int(bool(causal))),
           "oracle_dwsub_front_fwd")
    return y


def dwsub_front_bwd(x, w0, b0, w1, lengths, dy, causal: bool = False):
    """(dw0, db0, dw1, db1) of the subsampler front given dy [B,T2,F2,C]."""
    xa, xp = _f32(x)
    B, T, F = xa.shape
    w0a, w0p = _f32(w0)
    C = w0a.shape[2]
    if w0a.shape != (3, 3, C):
        raise ValueError("w0 must be [3, 3, C]")
    b0a, b0p = _f32(b0, (C,))
    w1a, w1p = _f32(w1, (3, 3, C))
    la, lp = _lens(lengths, B)
    pl, ph = front_pads(causal)
    T1, F1 = conv_out_len(T, 3, 2, pl, ph), conv_out_len(F, 3, 2, pl, ph)
    T2, F2 = conv_out_len(T1, 3, 2, pl, ph), conv_out_len(F1, 3, 2, pl, ph)
    da, dp = _f32(dy, (B, T2, F2, C))
    dw0, db0 = np.empty((3, 3, C)), np.empty((C,))
    dw1, db1 = np.empty((3, 3, C)), np.empty((C,))
    _check(_load().oracle_dwsub_front_bwd(xp, w0p, b0p, w1p, lp, dp, _ptr_d(dw0), _ptr_d(db0), _ptr_d(dw1),
                                          _ptr_d(db1), B, T, F, C, int(bool(causal))), "oracle_dwsub_front_bwd")
    return dw0, db0, dw1, db1
