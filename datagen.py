"""Seeded synthetic inputs for the depthwise-convolution path.

This module draws random tensors and nothing else: it holds none of the
convolution arithmetic, so both the HIP path and the CPU oracle can be fed from
it without sharing any of the method's code.

Every tensor is drawn from its own torch.Generator, seeded from a stable hash
of (seed, stream name).  A draw is reproducible on the same kind of device;
the CPU and the GPU generators are different algorithms, so the same
(seed, stream) gives different values on the two.  Callers that compare a GPU
result with the oracle therefore copy the GPU's inputs to the host rather
than redraw them.

Variance convention: ``normal(shape, var)`` takes the *variance*, so the
workloads' "w ~ N(0, 1/9)" has standard deviation 1/3 and "b ~ N(0, 0.1)" has
standard deviation sqrt(0.1).

The workload recipes below give the shapes, value distributions and length
mixes of the five workloads of the encoder depthwise path (log-mel frames
every 10 ms, 80 mel bins, 256 subsampler channels, kernel width 9, padded
batches whose valid lengths are spread between half and all of the padded
length).  They stand in for real audio, which the throughput figures do not
depend on.
"""
from __future__ import annotations

import hashlib
import math

import torch

DEFAULT_SEED = 0


def _stream_seed(seed: int, stream: str) -> int:
    h = hashlib.sha256(f"{seed}/{stream}".encode()).digest()
    return int.from_bytes(h[:8], "little") & 0x7FFF_FFFF_FFFF_FFFF


def _generator(seed: int, stream: str, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_stream_seed(seed, stream))
    return g


def normal(shape, var: float, stream: str, seed: int = DEFAULT_SEED, device="cpu") -> torch.Tensor:
    """float32 N(0, var) of the given shape."""
    g = _generator(seed, stream, device)
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if var != 1.0:
        t.mul_(math.sqrt(var))
    return t


def uniform(shape, lo: float, hi: float, stream: str, seed: int = DEFAULT_SEED, device="cpu") -> torch.Tensor:
    """float32 U(lo, hi) of the given shape."""
    g = _generator(seed, stream, device)
    t = torch.rand(tuple(shape), generator=g, device=device, dtype=torch.float32)
    return t.mul_(hi - lo).add_(lo)


def int_uniform(n: int, lo: int, hi: int, stream: str, seed: int = DEFAULT_SEED) -> torch.Tensor:
    """int32 [n] drawn uniformly from the inclusive range [lo, hi], on the host."""
    g = _generator(seed, stream, "cpu")
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int32)


# ---------------------------------------------------------------------------
# Workload recipes.  Each returns a dict of tensors on `device` plus the scalar
# arguments of the call.  Shapes can be overridden to make smaller cases with
# the same distributions.
# ---------------------------------------------------------------------------

def conv1d_small(device="cpu", seed=DEFAULT_SEED):
    """1-D depthwise conv, fp32, B=2 T=64 C=8 K=9 symmetric; lengths {64, 41}."""
    B, T, C, K = 2, 64, 8, 9
    return dict(
        x=normal((B, T, C), 1.0, "c1/x", seed, device),
        w=uniform((K, C), -1.0 / 3, 1.0 / 3, "c1/w", seed, device),
        b=normal((C,), 0.1, "c1/b", seed, device),
        lengths=torch.tensor([64, 41], dtype=torch.int32),
        B=B, T=T, C=C, K=K, causal=False, dtype="f32",
    )


def fused_front(device="cpu", seed=DEFAULT_SEED, B=4, T=1000, F=80, C=256, len_lo=None, len_hi=None):
    """Fused subsampler front: mel [B,T,F] -> [B,T/4,F/4,C]; lengths ~U[T/2, T]."""
    len_lo = T // 2 if len_lo is None else len_lo
    len_hi = T if len_hi is None else len_hi
    return dict(
        x=normal((B, T, F), 1.0, "c2/x", seed, device),
        w0=normal((3, 3, C), 1.0 / 9, "c2/w0", seed, device),
        b0=normal((C,), 0.1, "c2/b0", seed, device),
        w1=normal((3, 3, C), 1.0 / 9, "c2/w1", seed, device),
        b1=normal((C,), 0.1, "c2/b1", seed, device),
        lengths=int_uniform(B, len_lo, len_hi, "c2/len", seed),
        B=B, T=T, F=F, C=C,
    )


def conv1d_encoder_bf16(device="cpu", seed=DEFAULT_SEED, B=16, T=750, C=1024, K=9):
    """Conformer conv-module depthwise Conv1d, bf16 storage, symmetric pad; lengths ~U[T/2, T]."""
    return dict(
        x=normal((B, T, C), 1.0, "c3/x", seed, device).to(torch.bfloat16),
        w=normal((K, C), 1.0 / 9, "c3/w", seed, device).to(torch.bfloat16),
        b=normal((C,), 0.1, "c3/b", seed, device).to(torch.bfloat16),
        lengths=int_uniform(B, T // 2, T, "c3/len", seed),
        B=B, T=T, C=C, K=K, causal=False, dtype="bf16",
    )


def conv1d_causal_sweep(K, device="cpu", seed=DEFAULT_SEED, B=32, T=1500, C=512):
    """Causal 1-D depthwise conv, fp32, w ~ N(0, 1/K), zero bias; lengths ~U[T/2, T].
    Each width gets its own input draw, so that back-to-back runs of the sweep
    never find another width's input in a cache."""
    return dict(
        x=normal((B, T, C), 1.0, f"c4/x/K{K}/C{C}", seed, device),
        w=normal((K, C), 1.0 / K, f"c4/w/K{K}/C{C}", seed, device),
        b=torch.zeros((C,), dtype=torch.float32, device=device),
        lengths=int_uniform(B, T // 2, T, f"c4/len/C{C}", seed),
        B=B, T=T, C=C, K=K, causal=True, dtype="f32",
    )


def conv1d_stream(device="cpu", seed=DEFAULT_SEED, B=1024, Tc=8, C=1024, K=9, bf16=True):
    """Streaming conv module: B concurrent streams, one chunk of Tc frames
    each per call, w ~ N(0, 1/K), b ~ N(0, 0.1), a cache of K-1 frames
    ~ N(0,1) per stream (a stream mid-utterance), chunk lengths ~U[Tc/2, Tc];
    all bf16 by default."""
    d = dict(
        x=normal((B, Tc, C), 1.0, "c6/x", seed, device),
        w=normal((K, C), 1.0 / K, "c6/w", seed, device),
        b=normal((C,), 0.1, "c6/b", seed, device),
        cache=normal((B, K - 1, C), 1.0, "c6/cache", seed, device),
        lengths=int_uniform(B, Tc // 2, Tc, "c6/len", seed),
        B=B, Tc=Tc, C=C, K=K,
    )
    if bf16:
        for k in ("x", "w", "b", "cache"):
            d[k] = d[k].to(torch.bfloat16)
    return d


def conv2d_stage(device="cpu", seed=DEFAULT_SEED, B=32, T=1500, F=64, C=256, dy_rows_cols=None, bf16=False):
    """Depthwise 3x3 stride-2 conv2d fwd+bwd: x = max(N(0,1), 0) [B,T,F,C],
    dy ~ N(0,1) [B,T',F',C] with (T', F') = dy_rows_cols, by default
    (ceil(T/2), ceil(F/2)); lengths ~U[T/2, T] in input frames.  With bf16,
    x, w, b and dy are the same draws rounded to bfloat16 (nearest even)."""
    T2, F2 = dy_rows_cols if dy_rows_cols is not None else ((T + 1) // 2, (F + 1) // 2)
    x = normal((B, T, F, C), 1.0, "c5/x", seed, device).clamp_(min=0.0)
    d = dict(
        x=x,
        w=normal((3, 3, C), 1.0 / 9, "c5/w", seed, device),
        b=normal((C,), 0.1, "c5/b", seed, device),
        dy=normal((B, T2, F2, C), 1.0, "c5/dy", seed, device),
        lengths=int_uniform(B, T // 2, T, "c5/len", seed),
        B=B, T=T, F=F, C=C,
    )
    if bf16:
        for k in ("x", "w", "b", "dy"):
            d[k] = d[k].to(torch.bfloat16)
    return d
