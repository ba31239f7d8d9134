"""Seeded random shapes, lengths, paddings and storage types for every
operation, each checked against the CPU oracle.

The hand-picked grids in the other files cover the edges one at a time; this
sweep draws them together (ragged tiles, column chunks with a short last
chunk, channel counts that do or do not fill whole lanes and slabs, lengths
from 0 past T).  Sizes stay small so that the oracle finishes in well under
a second per case.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_exact_zero, assert_parity, say, time_mask

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
# Cases per family; DW_RANDOM_CASES raises it for a longer sweep.
N_CASES = int(os.environ.get("DW_RANDOM_CASES", "64"))


def lib():
    import conv_subsampling_amd as dw
    return dw


def rng(tag, i):
    """A generator seeded by the test family and the case number."""
    return np.random.default_rng([ord(c) for c in tag] + [i])


def tensor(r, shape, scale, dtype):
    return torch.as_tensor(r.standard_normal(shape) * scale, dtype=torch.float32).to(DEV).to(dtype)


def lengths(r, B, T):
    return torch.as_tensor(r.integers(-1, T + 2, size=B), dtype=torch.int32).to(DEV)


def tol(dtype):
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


@pytest.mark.parametrize("i", range(N_CASES))
def test_dwconv1d_fwd_bwd(i):
    r = rng("1d", i)
    B, T = int(r.integers(1, 4)), int(r.integers(1, 90))
    C = int(r.choice([1, 3, 8, 20, 64, 100, 256, 260, 512]))
    K = int(r.choice([3, 4, 5, 7, 9, 15]))
    causal = bool(r.integers(0, 2))
    dtype = torch.bfloat16 if r.integers(0, 2) else torch.float32
    say(f"random 1d #{i}: B={B} T={T} C={C} K={K} causal={causal} {dtype}")
    x, w = tensor(r, (B, T, C), 1.0, dtype), tensor(r, (K, C), 1.0 / K, dtype)
    b = tensor(r, (C,), 0.1, dtype) if r.integers(0, 2) else None
    dy = tensor(r, (B, T, C), 1.0, dtype)
    L = lengths(r, B, T)
    y = lib().dwconv1d_fwd(x, w, b, L, causal=causal)
    g = lib().dwconv1d_bwd(x, w, L, dy, causal=causal)
    torch.cuda.synchronize()
    assert_parity(y, oracle.dwconv1d_fwd(x, w, b, L, causal), tol(dtype), "y")
    Lh = L.cpu().clamp(0, T)
    assert_exact_zero(y, time_mask(Lh, B, T)[:, :, None], "y")
    rdx, rdw, rdb = oracle.dwconv1d_bwd(x, w, L, dy, causal)
    assert_parity(g[0], rdx, tol(dtype), "dx")
    assert_parity(g[1], rdw, TOL_F32, "dw")
    assert_parity(g[2], rdb, TOL_F32, "db")


@pytest.mark.parametrize("i", range(N_CASES))
def test_dwconv2d_fwd_bwd(i):
    r = rng("2d", i)
    B, T, F = int(r.integers(1, 4)), int(r.integers(1, 40)), int(r.integers(1, 70))
    C = int(r.choice([1, 4, 12, 64, 100, 256]))
    pads = (int(r.integers(1, 3)), int(r.integers(0, 3)), int(r.integers(1, 3)), int(r.integers(0, 3)))
    dtype = torch.bfloat16 if r.integers(0, 2) else torch.float32
    To, Fo = oracle.conv_out_len(T, 3, 2, pads[0], pads[1]), oracle.conv_out_len(F, 3, 2, pads[2], pads[3])
    say(f"random 2d #{i}: B={B} T={T} F={F} C={C} pads={pads} {dtype}")
    x = tensor(r, (B, T, F, C), 1.0, dtype)
    w, b = tensor(r, (3, 3, C), 1.0 / 3, dtype), tensor(r, (C,), 0.1, dtype)
    dy = tensor(r, (B, max(To, 0), max(Fo, 0), C), 1.0, dtype)
    L = lengths(r, B, T)
    y = lib().dwconv2d_fwd(x, w, b, L, pads=pads)
    g = lib().dwconv2d_bwd(x, w, L, dy, pads=pads)
    torch.cuda.synchronize()
    assert_parity(y, oracle.dwconv2d_fwd(x, w, b, L, pads=pads), tol(dtype), "y")
    rdx, rdw, rdb = oracle.dwconv2d_bwd(x, w, L, dy, pads=pads)
    assert_parity(g[0], rdx, tol(dtype), "dx")
    assert_parity(g[1], rdw, TOL_F32, "dw")
    assert_parity(g[2], rdb, TOL_F32, "db")


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_front_fwd_bwd(i):
    r = rng("front", i)
    B, T, F = int(r.integers(1, 3)), int(r.integers(1, 60)), int(r.integers(1, 40))
    C = int(r.choice([1, 16, 64, 100, 256, 300]))
    causal = bool(r.integers(0, 2))
    dtype = torch.bfloat16 if r.integers(0, 2) else torch.float32
    say(f"random front #{i}: B={B} T={T} F={F} C={C} causal={causal} {dtype}")
    x = tensor(r, (B, T, F), 1.0, dtype)
    w0, w1 = tensor(r, (3, 3, C), 1.0 / 3, dtype), tensor(r, (3, 3, C), 1.0 / 3, dtype)
    b0, b1 = tensor(r, (C,), 0.1, dtype), tensor(r, (C,), 0.1, dtype)
    L = lengths(r, B, T)
    y = lib().dwsub_fused_fwd(x, w0, b0, w1, b1, L, causal=causal)
    dy = tensor(r, tuple(y.shape), 1.0, dtype)
    g = lib().dwsub_fused_bwd(x, w0, b0, w1, L, dy, causal=causal)
    torch.cuda.synchronize()
    assert_parity(y, oracle.dwsub_front_fwd(x, w0, b0, w1, b1, L, causal=causal), tol(dtype), "y")
    ref = oracle.dwsub_front_bwd(x, w0, b0, w1, L, dy, causal=causal)
    for name, a, e in zip(("dw0", "db0", "dw1", "db1"), g, ref):
        assert_parity(a, e, TOL_F32, name)


@pytest.mark.parametrize("i", range(N_CASES // 2))
def test_stream_chunk(i):
    r = rng("stream", i)
    B, Tc = int(r.integers(1, 5)), int(r.integers(1, 20))
    C = int(r.choice([1, 8, 64, 200, 1024]))
    K = int(r.choice([1, 2, 3, 4, 5, 9, 15, 31]))
    dtype = torch.bfloat16 if r.integers(0, 2) else torch.float32
    say(f"random stream #{i}: B={B} Tc={Tc} C={C} K={K} {dtype}")
    x, w = tensor(r, (B, Tc, C), 1.0, dtype), tensor(r, (K, C), 1.0 / K, dtype)
    b = tensor(r, (C,), 0.1, dtype)
    cache = tensor(r, (B, K - 1, C), 1.0, dtype)
    L = lengths(r, B, Tc)
    y, c2 = lib().dwconv1d_stream_fwd(x, w, b, L, cache)
    torch.cuda.synchronize()
    ry, rc = oracle.dwconv1d_stream_fwd(x, w, b, L, cache)
    assert_parity(y, ry, tol(dtype), "y")
    assert np.array_equal(c2.float().cpu().numpy().astype(np.float64), rc), "cache"
