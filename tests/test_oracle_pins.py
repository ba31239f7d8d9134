"""Pins for the CPU oracle, on the host.

The oracle is checked against things other than itself:
  * the library convolutions of torch on the CPU in float64 (Conv1d / Conv2d
    with groups = C, which is the depthwise convolution the pages say the
    method equals), with the masks and padding applied around them;
  * the pages' own alternative formulation of the 1-D conv (im2col followed by
    a matrix product, per item);
  * numpy.correlate for a single channel;
  * closed forms for delta kernels;
  * identities: linearity, causality, batch independence, adjoint and
    finite-difference identities for the backward, exact zeros and no NaN
    leak from masked frames.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle

RTOL = 1e-11


def close(a, b, rtol=RTOL):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= rtol, f"max rel err {err}"


def rng(seed):
    return np.random.default_rng(seed)


def f32(a):
    return np.asarray(a, dtype=np.float32)


def eff_len(lengths, B, T):
    if lengths is None:
        return np.full(B, T)
    return np.clip(np.asarray(lengths), 0, T)


# ---------------------------------------------------------------- 1-D -----

def torch_dwconv1d(x, w, b, lengths, causal):
    """Masked, padded depthwise Conv1d via torch's grouped conv1d in float64."""
    B, T, C = x.shape
    K = w.shape[0]
    L = eff_len(lengths, B, T)
    tmask = torch.arange(T)[None, :] < torch.as_tensor(L)[:, None]          # [B,T]
    xt = torch.from_numpy(x.astype(np.float64))
    xt = torch.where(tmask[:, :, None], xt, torch.zeros(()))                # pre-mask
    xt = xt.permute(0, 2, 1)                                                 # [B,C,T]
    pL = K - 1 if causal else (K - 1) // 2
    xt = Fn.pad(xt, (pL, K - 1 - pL))
    wt = torch.from_numpy(w.astype(np.float64)).t().contiguous()[:, None, :]  # [C,1,K]
    bt = None if b is None else torch.from_numpy(b.astype(np.float64))
    y = Fn.conv1d(xt, wt, bt, groups=C).permute(0, 2, 1)
    y = torch.where(tmask[:, :, None], y, torch.zeros(()))                  # post-mask
    return y.numpy()


def im2col_dwconv1d(x, w, b, lengths, causal):
    """The im2col + matrix-product formulation, run once per item."""
    B, T, C = x.shape
    K = w.shape[0]
    pL = K - 1 if causal else (K - 1) // 2
    L = eff_len(lengths, B, T)
    out = np.zeros((B, T, C))
    for bi in range(B):
        xm = x[bi].astype(np.float64).copy()
        xm[L[bi]:] = 0.0
        xp = np.zeros((T + K - 1, C))
        xp[pL:pL + T] = xm
        for c in range(C):
            cols = np.stack([xp[t:t + K, c] for t in range(T)]) if T else np.zeros((0, K))
            out[bi, :, c] = cols @ w[:, c].astype(np.float64)
        if b is not None:
            out[bi] += b.astype(np.float64)
        out[bi, L[bi]:] = 0.0
    return out


GRID_1D = [
    # (B, T, C, K, causal)
    (1, 1, 3, 3, False), (3, 1, 3, 9, True), (1, 2, 1, 5, False), (3, 7, 8, 4, False),
    (3, 7, 8, 4, True), (2, 50, 3, 15, False), (2, 50, 3, 15, True), (3, 20, 5, 1, False),
    (2, 13, 4, 2, False), (2, 13, 4, 2, True), (1, 33, 6, 9, False), (3, 9, 2, 9, True),
]


@pytest.mark.parametrize("B,T,C,K,causal", GRID_1D)
def test_1d_matches_torch_grouped_conv(B, T, C, K, causal):
    r = rng(B * 1000 + T * 10 + K)
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    b = f32(r.standard_normal(C))
    for lengths in (None, r.integers(-2, T + 3, B).astype(np.int32)):
        for bias in (None, b):
            close(oracle.dwconv1d_fwd(x, w, bias, lengths, causal),
                  torch_dwconv1d(x, w, bias, lengths, causal))


@pytest.mark.parametrize("B,T,C,K,causal", GRID_1D)
def test_1d_matches_im2col_matmul(B, T, C, K, causal):
    r = rng(7 + B * 1000 + T * 10 + K)
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    b = f32(r.standard_normal(C))
    lengths = r.integers(0, T + 1, B).astype(np.int32)
    close(oracle.dwconv1d_fwd(x, w, b, lengths, causal), im2col_dwconv1d(x, w, b, lengths, causal))


@pytest.mark.parametrize("K,causal", [(3, False), (9, False), (4, False), (4, True), (9, True)])
def test_1d_single_channel_is_numpy_correlate(K, causal):
    r = rng(K)
    T = 40
    x = f32(r.standard_normal((1, T, 1)))
    w = f32(r.standard_normal((K, 1)))
    pL = K - 1 if causal else (K - 1) // 2
    xp = np.concatenate([np.zeros(pL), x[0, :, 0].astype(np.float64), np.zeros(K - 1 - pL)])
    ref = np.correlate(xp, w[:, 0].astype(np.float64), mode="valid")
    close(oracle.dwconv1d_fwd(x, w, None, None, causal)[0, :, 0], ref)


@pytest.mark.parametrize("K,causal", [(3, False), (9, False), (4, False), (15, True), (5, True)])
def test_1d_delta_kernels(K, causal):
    """w = e_pL copies the masked input; w = e_0 shifts it right by pL."""
    r = rng(100 + K)
    B, T, C = 2, 30, 4
    x = f32(r.standard_normal((B, T, C)))
    lengths = np.array([30, 17], dtype=np.int32)
    pL = K - 1 if causal else (K - 1) // 2
    xm = x.astype(np.float64).copy()
    xm[1, 17:] = 0
    w = np.zeros((K, C), np.float32)
    w[pL] = 1
    y = oracle.dwconv1d_fwd(x, w, None, lengths, causal)
    assert np.array_equal(y, xm)
    w = np.zeros((K, C), np.float32)
    w[0] = 1
    y = oracle.dwconv1d_fwd(x, w, None, lengths, causal)
    shifted = np.zeros_like(xm)
    shifted[:, pL:] = xm[:, :T - pL]
    shifted[1, 17:] = 0
    assert np.array_equal(y, shifted)


def test_1d_linearity_and_bias_superposition():
    r = rng(5)
    B, T, C, K = 2, 25, 3, 5
    # small integers, so that a*x1 + c*x2 is exact in float32
    x1, x2 = f32(r.integers(-8, 9, (B, T, C))), f32(r.integers(-8, 9, (B, T, C)))
    w = f32(r.standard_normal((K, C)))
    b = f32(r.standard_normal(C))
    lengths = np.array([25, 11], np.int32)
    a, c = 2.0, -0.5
    y = oracle.dwconv1d_fwd(f32(a * x1 + c * x2), w, None, lengths, False)
    close(y, a * oracle.dwconv1d_fwd(x1, w, None, lengths, False) + c * oracle.dwconv1d_fwd(x2, w, None, lengths, False))
    yb = oracle.dwconv1d_fwd(x1, w, b, lengths, False)
    mask = (np.arange(T)[None, :] < lengths[:, None])[:, :, None]
    close(yb, oracle.dwconv1d_fwd(x1, w, None, lengths, False) + mask * b.astype(np.float64))


def test_1d_causality_and_batch_independence():
    r = rng(6)
    B, T, C, K = 3, 40, 4, 9
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    y = oracle.dwconv1d_fwd(x, w, None, None, True)
    x2 = x.copy()
    x2[:, 20] += 5.0
    y2 = oracle.dwconv1d_fwd(x2, w, None, None, True)
    assert np.array_equal(y[:, :20], y2[:, :20])
    assert not np.array_equal(y[:, 20], y2[:, 20])
    lengths = np.array([40, 3, 22], np.int32)
    yb = oracle.dwconv1d_fwd(x, w, None, lengths, False)
    for bi in range(B):
        assert np.array_equal(yb[bi:bi + 1], oracle.dwconv1d_fwd(x[bi:bi + 1], w, None, lengths[bi:bi + 1], False))


def test_1d_masked_frames_exact_zero_and_no_nan_leak():
    r = rng(8)
    B, T, C, K = 2, 30, 5, 9
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    b = f32(r.standard_normal(C))
    lengths = np.array([12, 0], np.int32)
    y = oracle.dwconv1d_fwd(x, w, b, lengths, False)
    xn = x.copy()
    xn[0, 12:] = np.nan
    xn[1] = np.inf
    yn = oracle.dwconv1d_fwd(xn, w, b, lengths, False)
    assert np.array_equal(y, yn)
    assert np.all(y[0, 12:] == 0) and np.all(y[1] == 0)


# ---------------------------------------------------------------- 2-D -----

def torch_dwconv2d(x, w, b, lengths, stride, pad):
    B, T, F, C = x.shape
    KH, KW = w.shape[:2]
    L = eff_len(lengths, B, T)
    xt = torch.from_numpy(x.astype(np.float64))
    m = (torch.arange(T)[None, :] < torch.as_tensor(L)[:, None])[:, :, None, None]
    xt = torch.where(m, xt, torch.zeros(())).permute(0, 3, 1, 2)
    wt = torch.from_numpy(w.astype(np.float64)).permute(2, 0, 1).contiguous()[:, None]
    bt = None if b is None else torch.from_numpy(b.astype(np.float64))
    y = Fn.conv2d(xt, wt, bt, stride=stride, padding=pad, groups=C).permute(0, 2, 3, 1)
    To = y.shape[1]
    Lo = np.array([min(oracle.conv_out_len(l, KH, stride, pad), To) if l > 0 else 0 for l in L])
    mo = (torch.arange(To)[None, :] < torch.as_tensor(Lo)[:, None])[:, :, None, None]
    return torch.where(mo, y, torch.zeros(())).numpy()


GRID_2D = [
    # (B, T, F, C, KH, KW, stride, pad)
    (2, 9, 8, 3, 3, 3, 2, 1), (2, 10, 7, 2, 3, 3, 2, 1), (1, 1, 1, 2, 3, 3, 2, 1),
    (3, 6, 5, 4, 3, 3, 1, 1), (2, 8, 6, 3, 1, 1, 1, 0), (2, 7, 9, 2, 3, 1, 2, 1),
    (2, 8, 8, 2, 2, 2, 2, 0), (1, 12, 4, 5, 5, 3, 3, 2),
]


@pytest.mark.parametrize("B,T,F,C,KH,KW,s,p", GRID_2D)
def test_2d_matches_torch_grouped_conv(B, T, F, C, KH, KW, s, p):
    r = rng(B + T * 7 + F * 31 + KH)
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((KH, KW, C)))
    b = f32(r.standard_normal(C))
    for lengths in (None, r.integers(-1, T + 2, B).astype(np.int32)):
        for bias in (None, b):
            close(oracle.dwconv2d_fwd(x, w, bias, lengths, s, p), torch_dwconv2d(x, w, bias, lengths, s, p))


def test_2d_center_delta_closed_form():
    r = rng(11)
    B, T, F, C = 2, 11, 9, 3
    x = f32(r.standard_normal((B, T, F, C)))
    w = np.zeros((3, 3, C), np.float32)
    w[1, 1] = 1.0
    lengths = np.array([11, 6], np.int32)
    y = oracle.dwconv2d_fwd(x, w, None, lengths)
    ref = x[:, 0::2, 0::2].astype(np.float64).copy()
    ref[1, 3:] = 0.0  # ceil(6/2) = 3 valid output rows
    assert np.array_equal(y, ref)


def test_2d_masked_rows_exact_zero_and_no_nan_leak():
    r = rng(12)
    B, T, F, C = 2, 12, 6, 3
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((3, 3, C)))
    b = f32(r.standard_normal(C))
    lengths = np.array([7, 0], np.int32)
    y = oracle.dwconv2d_fwd(x, w, b, lengths)
    xn = x.copy()
    xn[0, 7:] = np.nan
    xn[1] = np.nan
    assert np.array_equal(y, oracle.dwconv2d_fwd(xn, w, b, lengths))
    assert np.all(y[0, 4:] == 0) and np.all(y[1] == 0)


# ----------------------------------------------- asymmetric (causal) pads -----
# The causal padding the pages name for the conv2d and the front (NeMo PR
# #16114, "What does this PR do") is read as kernel - 1 zeros before and
# stride - 1 after, on each axis.  The reference here pads explicitly with
# F.pad and convolves without padding, a different route from the oracle's
# index arithmetic.

def torch_dwconv2d_pads(x, w, b, lengths, stride, pads, dy=None):
    B, T, F, C = x.shape
    KH, KW = w.shape[:2]
    pt0, pt1, pf0, pf1 = pads
    L = eff_len(lengths, B, T)
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(dy is not None)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(dy is not None)
    bt = torch.from_numpy((b if b is not None else np.zeros(C, np.float32)).astype(np.float64))
    bt.requires_grad_(dy is not None)
    m = (torch.arange(T)[None, :] < torch.as_tensor(L)[:, None])[:, :, None, None]
    xm = torch.where(m, xt, torch.zeros(())).permute(0, 3, 1, 2)
    xm = Fn.pad(xm, (pf0, pf1, pt0, pt1))
    y = Fn.conv2d(xm, wt.permute(2, 0, 1)[:, None], bt, stride=stride, groups=C).permute(0, 2, 3, 1)
    To = y.shape[1]
    Lo = np.array([min(max(0, (l + pt0 + pt1 - KH) // stride + 1), To) if l > 0 else 0 for l in L])
    mo = (torch.arange(To)[None, :] < torch.as_tensor(Lo)[:, None])[:, :, None, None]
    y = torch.where(mo, y, torch.zeros(()))
    if dy is None:
        return y.detach().numpy()
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return xt.grad.numpy(), wt.grad.numpy(), bt.grad.numpy()


PADS_2D = [
    # (B, T, F, C, KH, KW, stride, (pt0, pt1, pf0, pf1))
    (2, 9, 8, 3, 3, 3, 2, (2, 1, 2, 1)), (3, 10, 7, 2, 3, 3, 2, (2, 1, 2, 1)), (1, 1, 1, 2, 3, 3, 2, (2, 1, 2, 1)),
    (2, 11, 6, 2, 3, 3, 2, (2, 1, 1, 1)), (2, 8, 9, 3, 3, 3, 2, (1, 1, 2, 1)), (2, 12, 10, 2, 3, 3, 2, (1, 0, 0, 2)),
    (2, 7, 5, 2, 3, 3, 2, (2, 2, 1, 0)), (2, 9, 8, 2, 3, 2, 1, (2, 0, 1, 0)), (1, 13, 7, 3, 5, 3, 3, (4, 2, 2, 0)),
]


@pytest.mark.parametrize("B,T,F,C,KH,KW,s,pads", PADS_2D)
def test_2d_asymmetric_pads_match_torch(B, T, F, C, KH, KW, s, pads):
    r = rng(B + T * 5 + F * 17 + sum(pads) * 3)
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((KH, KW, C)))
    b = f32(r.standard_normal(C))
    lengths = r.integers(-1, T + 2, B).astype(np.int32)
    lengths[0] = 0  # an empty item: no output row is valid, whatever the padding
    for L in (None, lengths):
        for bias in (None, b):
            close(oracle.dwconv2d_fwd(x, w, bias, L, s, pads=pads), torch_dwconv2d_pads(x, w, bias, L, s, pads))


@pytest.mark.parametrize("B,T,F,C,KH,KW,s,pads", PADS_2D)
def test_bwd_asymmetric_pads_match_torch_autograd(B, T, F, C, KH, KW, s, pads):
    r = rng(7 * B + T + F * 11 + sum(pads))
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((KH, KW, C)))
    b = f32(r.standard_normal(C))
    To = oracle.conv_out_len(T, KH, s, pads[0], pads[1])
    Fo = oracle.conv_out_len(F, KW, s, pads[2], pads[3])
    dy = f32(r.standard_normal((B, To, Fo, C)))
    lengths = r.integers(0, T + 2, B).astype(np.int32)
    got = oracle.dwconv2d_bwd(x, w, lengths, dy, s, pads=pads)
    for g, rf in zip(got, torch_dwconv2d_pads(x, w, b, lengths, s, pads, dy=dy)):
        close(g, rf)


def test_2d_causal_pads_never_look_ahead():
    """With kernel - 1 rows of padding before and stride - 1 after, output row
    t' reads input rows up to s t' only; symmetric padding reads s t' + 1."""
    r = rng(13)
    B, T, F, C = 2, 14, 6, 3
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((3, 3, C)))
    b = f32(r.standard_normal(C))
    causal = (2, 1, 2, 1)
    y = oracle.dwconv2d_fwd(x, w, b, None, 2, pads=causal)
    for t0 in (1, 5, 8):
        x2 = x.copy()
        x2[:, t0:] += 1.0 + r.standard_normal((B, T - t0, F, C)).astype(np.float32) ** 2
        y2 = oracle.dwconv2d_fwd(x2, w, b, None, 2, pads=causal)
        keep = (t0 + 1) // 2                            # rows t' with 2 t' < t0
        assert np.array_equal(y[:, :keep], y2[:, :keep])
        assert not np.array_equal(y[:, keep], y2[:, keep])
        ys, ys2 = oracle.dwconv2d_fwd(x, w, b, None), oracle.dwconv2d_fwd(x2, w, b, None)
        assert not np.array_equal(ys[:, :keep], ys2[:, :keep]) or t0 % 2 == 0


def test_2d_causal_present_tap_closed_form():
    """Causal pads and w = e_{2,2} (the tap on the present row and column):
    y[t', f'] = x[2t', 2f'], masked at t' >= floor(len/2) + 1."""
    r = rng(14)
    B, T, F, C = 3, 11, 9, 2
    x = f32(r.standard_normal((B, T, F, C)))
    w = np.zeros((3, 3, C), np.float32)
    w[2, 2] = 1.0
    lengths = np.array([11, 6, 0], np.int32)
    y = oracle.dwconv2d_fwd(x, w, None, lengths, 2, pads=(2, 1, 2, 1))
    assert y.shape == (B, T // 2 + 1, F // 2 + 1, C)
    xm = x.astype(np.float64).copy()
    for bi, l in enumerate(lengths):
        xm[bi, l:] = 0.0
    ref = np.zeros_like(y)
    ref[:, : (T + 1) // 2, : (F + 1) // 2] = xm[:, 0::2, 0::2]
    for bi, l in enumerate(lengths):
        ref[bi, (l // 2 + 1 if l > 0 else 0):] = 0.0
    assert np.array_equal(y, ref)


# ---------------------------------------------------------- backward -----

def torch_dwconv2d_grads(x, w, b, lengths, dy, stride, pad):
    B, T, F, C = x.shape
    KH, KW = w.shape[:2]
    L = eff_len(lengths, B, T)
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    bt = torch.from_numpy(b.astype(np.float64)).requires_grad_(True)
    m = (torch.arange(T)[None, :] < torch.as_tensor(L)[:, None])[:, :, None, None]
    xm = torch.where(m, xt, torch.zeros(())).permute(0, 3, 1, 2)
    y = Fn.conv2d(xm, wt.permute(2, 0, 1)[:, None], bt, stride=stride, padding=pad, groups=C).permute(0, 2, 3, 1)
    To = y.shape[1]
    Lo = np.array([min(oracle.conv_out_len(l, KH, stride, pad), To) if l > 0 else 0 for l in L])
    mo = (torch.arange(To)[None, :] < torch.as_tensor(Lo)[:, None])[:, :, None, None]
    y = torch.where(mo, y, torch.zeros(()))
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return xt.grad.numpy(), wt.grad.numpy(), bt.grad.numpy()


@pytest.mark.parametrize("B,T,F,C,KH,KW,s,p", GRID_2D)
def test_bwd_matches_torch_autograd(B, T, F, C, KH, KW, s, p):
    r = rng(3 * B + T + F * 13 + KW)
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((KH, KW, C)))
    b = f32(r.standard_normal(C))
    To, Fo = oracle.conv_out_len(T, KH, s, p), oracle.conv_out_len(F, KW, s, p)
    dy = f32(r.standard_normal((B, To, Fo, C)))
    lengths = r.integers(0, T + 2, B).astype(np.int32)
    dx, dw, db = oracle.dwconv2d_bwd(x, w, lengths, dy, s, p)
    tdx, tdw, tdb = torch_dwconv2d_grads(x, w, b, lengths, dy, s, p)
    close(dx, tdx)
    close(dw, tdw)
    close(db, tdb)


def test_bwd_adjoint_and_bilinear_identities():
    r = rng(21)
    B, T, F, C = 3, 13, 10, 4
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((3, 3, C)))
    b = f32(r.standard_normal(C))
    dy = f32(r.standard_normal((B, 7, 5, C)))
    lengths = np.array([13, 8, 3], np.int32)
    dx, dw, db = oracle.dwconv2d_bwd(x, w, lengths, dy)
    y_nb = oracle.dwconv2d_fwd(x, w, None, lengths)
    Lo = (lengths + 1) // 2
    g = dy.astype(np.float64) * (np.arange(7)[None, :] < Lo[:, None])[:, :, None, None]
    inner = np.sum(g * y_nb)
    close(np.sum(dx * x.astype(np.float64)), inner, 1e-10)        # <g, A x> = <A^T g, x>
    close(np.sum(dw * w.astype(np.float64)), inner, 1e-10)        # bilinear in (x, w)
    close(db, g.sum(axis=(0, 1, 2)))                              # db is the masked dy sum
    y_b = oracle.dwconv2d_fwd(x, w, b, lengths)
    close(np.sum(g * (y_b - y_nb)), np.sum(db * b.astype(np.float64)), 1e-10)


def test_bwd_finite_differences():
    """The op is linear in x and in w, so a central difference is exact up to rounding."""
    r = rng(22)
    B, T, F, C = 2, 7, 6, 2
    # integer-valued data, so that x +- e and w +- e are exact in float32
    x = f32(r.integers(-9, 10, (B, T, F, C)))
    w = f32(r.integers(-9, 10, (3, 3, C)))
    dy = f32(r.standard_normal((B, 4, 3, C)))
    lengths = np.array([7, 4], np.int32)
    dx, dw, _ = oracle.dwconv2d_bwd(x, w, lengths, dy)
    loss = lambda xx, ww: float(np.sum(oracle.dwconv2d_fwd(xx, ww, None, lengths) * dy.astype(np.float64)))
    for idx in itertools.islice(itertools.product(range(B), range(T), range(F), range(C)), 0, None, 5):
        e = np.zeros_like(x)
        e[idx] = 1.0
        fd = (loss(x + e, w) - loss(x - e, w)) / 2.0
        assert abs(fd - dx[idx]) <= 1e-9 * (1 + abs(dx[idx]))
    for idx in itertools.product(range(3), range(3), range(C)):
        e = np.zeros_like(w)
        e[idx] = 1.0
        fd = (loss(x, w + e) - loss(x, w - e)) / 2.0
        assert abs(fd - dw[idx]) <= 1e-9 * (1 + abs(dw[idx]))


def test_bwd_masks_and_no_nan_leak():
    r = rng(23)
    B, T, F, C = 2, 10, 6, 3
    x = f32(r.standard_normal((B, T, F, C)))
    w = f32(r.standard_normal((3, 3, C)))
    dy = f32(r.standard_normal((B, 5, 3, C)))
    lengths = np.array([5, 10], np.int32)
    dx, dw, db = oracle.dwconv2d_bwd(x, w, lengths, dy)
    assert np.all(dx[0, 5:] == 0)
    xn, dyn = x.copy(), dy.copy()
    xn[0, 5:] = np.nan
    dyn[0, 3:] = np.nan  # ceil(5/2) = 3 valid output rows
    dx2, dw2, db2 = oracle.dwconv2d_bwd(xn, w, lengths, dyn)
    assert np.array_equal(dx, dx2) and np.array_equal(dw, dw2) and np.array_equal(db, db2)


def test_bwd_center_tap_equals_db_for_unit_input():
    """With x = 1 on every valid frame, the centre tap's gradient is the bias gradient."""
    r = rng(24)
    B, T, F, C = 2, 9, 8, 3
    x = np.ones((B, T, F, C), np.float32)
    w = f32(r.standard_normal((3, 3, C)))
    dy = f32(r.standard_normal((B, 5, 4, C)))
    lengths = np.array([9, 4], np.int32)
    _, dw, db = oracle.dwconv2d_bwd(x, w, lengths, dy)
    close(dw[1, 1], db, 1e-13)


# ------------------------------------------------------- fused front -----

def torch_front(x, w0, b0, w1, b1, lengths):
    B, T, F = x.shape
    C = w0.shape[2]
    L = eff_len(lengths, B, T)
    xt = torch.from_numpy(x.astype(np.float64))[:, None]                        # [B,1,T,F]
    h = Fn.conv2d(xt, torch.from_numpy(w0.astype(np.float64)).permute(2, 0, 1)[:, None],
                  torch.from_numpy(b0.astype(np.float64)), stride=2, padding=1)
    h = torch.relu(h)
    L1 = (L + 1) // 2
    m = (torch.arange(h.shape[2])[None, :] < torch.as_tensor(L1)[:, None])[:, None, :, None]
    h = torch.where(m, h, torch.zeros(()))
    y = Fn.conv2d(h, torch.from_numpy(w1.astype(np.float64)).permute(2, 0, 1)[:, None],
                  torch.from_numpy(b1.astype(np.float64)), stride=2, padding=1, groups=C)
    return y.permute(0, 2, 3, 1).numpy()


@pytest.mark.parametrize("B,T,F,C", [(2, 16, 12, 4), (3, 13, 9, 3), (1, 1, 1, 2), (2, 30, 20, 5), (1, 7, 80, 2)])
def test_front_matches_torch_chain(B, T, F, C):
    r = rng(B + T + F + C)
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    for lengths in (None, r.integers(-1, T + 2, B).astype(np.int32)):
        close(oracle.dwsub_front_fwd(x, w0, b0, w1, b1, lengths), torch_front(x, w0, b0, w1, b1, lengths))


def test_front_center_delta_closed_form():
    r = rng(31)
    B, T, F, C = 2, 21, 17, 2
    x = f32(r.standard_normal((B, T, F)))
    d = np.zeros((3, 3, C), np.float32)
    d[1, 1] = 1.0
    z = np.zeros(C, np.float32)
    lengths = np.array([21, 9], np.int32)
    y = oracle.dwsub_front_fwd(x, d, z, d, z, lengths)
    L1 = (lengths + 1) // 2
    ref = np.maximum(x[:, 0::4, 0::4].astype(np.float64), 0.0)[..., None].repeat(C, axis=3)
    for bi in range(B):
        ref[bi, (np.arange(ref.shape[1]) * 2) >= L1[bi]] = 0.0
    assert np.array_equal(y, ref)


def test_front_fully_masked_rows_equal_output_bias():
    r = rng(32)
    B, T, F, C = 1, 40, 12, 3
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    lengths = np.array([13], np.int32)  # L1 = 7: output rows with 2*t2 - 1 >= 7 see only masked h
    y = oracle.dwsub_front_fwd(x, w0, b0, w1, b1, lengths)
    for t2 in range(y.shape[1]):
        if 2 * t2 - 1 >= 7:
            assert np.all(y[0, t2] == b1.astype(np.float64)[None, :])


def test_front_input_is_not_length_masked():
    """With an odd length the last unmasked h row reads one mel frame past the length."""
    r = rng(33)
    B, T, F, C = 1, 20, 8, 2
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(np.abs(r.standard_normal((3, 3, C)))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(np.full(C, 5.0)), f32(r.standard_normal(C))
    lengths = np.array([9], np.int32)  # L1 = 5; h row 4 reads mel rows 7, 8, 9
    y = oracle.dwsub_front_fwd(x, w0, b0, w1, b1, lengths)
    x2 = x.copy()
    x2[0, 9] += 3.0
    assert not np.array_equal(y, oracle.dwsub_front_fwd(x2, w0, b0, w1, b1, lengths))
    x3 = x.copy()
    x3[0, 11:] = np.nan  # never read by an unmasked h row
    assert np.array_equal(y, oracle.dwsub_front_fwd(x3, w0, b0, w1, b1, lengths))


def test_front_positive_homogeneity():
    r = rng(34)
    B, T, F, C = 2, 16, 12, 3
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    lengths = np.array([16, 9], np.int32)
    y = oracle.dwsub_front_fwd(x, w0, b0, w1, b1, lengths) - b1.astype(np.float64)
    y2 = oracle.dwsub_front_fwd(f32(2 * x), w0, f32(2 * b0), w1, b1, lengths) - b1.astype(np.float64)
    close(y2, 2 * y, 1e-13)


# ------------------------------------------------------ causal front -----

def torch_front_causal(x, w0, b0, w1, b1, lengths, dy=None):
    """The front in causal mode: each stride-2 conv pads 2 before and 1 after
    on both axes (explicit F.pad), h masked at t1 >= floor(len/2) + 1."""
    B, T, F = x.shape
    C = w0.shape[2]
    L = eff_len(lengths, B, T)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64)).requires_grad_(dy is not None)
    tw0, tb0, tw1, tb1 = t(w0), t(b0), t(w1), t(b1)
    xt = Fn.pad(torch.from_numpy(x.astype(np.float64))[:, None], (2, 1, 2, 1))
    h = torch.relu(Fn.conv2d(xt, tw0.permute(2, 0, 1)[:, None], tb0, stride=2))
    L1 = np.where(L > 0, L // 2 + 1, 0)
    m = (torch.arange(h.shape[2])[None, :] < torch.as_tensor(L1)[:, None])[:, None, :, None]
    h = torch.where(m, h, torch.zeros(()))
    y = Fn.conv2d(Fn.pad(h, (2, 1, 2, 1)), tw1.permute(2, 0, 1)[:, None], tb1, stride=2, groups=C)
    y = y.permute(0, 2, 3, 1)
    if dy is None:
        return y.detach().numpy()
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return tw0.grad.numpy(), tb0.grad.numpy(), tw1.grad.numpy(), tb1.grad.numpy()


FRONT_CAUSAL = [(2, 16, 12, 4), (3, 13, 9, 3), (1, 1, 1, 2), (2, 30, 20, 5), (1, 7, 80, 2), (2, 2, 3, 2)]


@pytest.mark.parametrize("B,T,F,C", FRONT_CAUSAL)
def test_front_causal_matches_torch_chain(B, T, F, C):
    r = rng(50 + B + T + F + C)
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    lengths = r.integers(-1, T + 2, B).astype(np.int32)
    lengths[0] = 0
    for L in (None, lengths):
        close(oracle.dwsub_front_fwd(x, w0, b0, w1, b1, L, causal=True), torch_front_causal(x, w0, b0, w1, b1, L))


@pytest.mark.parametrize("B,T,F,C", FRONT_CAUSAL)
def test_front_causal_bwd_matches_torch_autograd(B, T, F, C):
    r = rng(60 + B + T + F + C)
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    T2 = (T // 2 + 1) // 2 + 1
    F2 = (F // 2 + 1) // 2 + 1
    dy = f32(r.standard_normal((B, T2, F2, C)))
    lengths = r.integers(-1, T + 2, B).astype(np.int32)
    lengths[-1] = 0
    for L in (None, lengths):
        got = oracle.dwsub_front_bwd(x, w0, b0, w1, L, dy, causal=True)
        for g, rf in zip(got, torch_front_causal(x, w0, b0, w1, b1, L, dy=dy)):
            close(g, rf)


def test_front_causal_present_tap_and_no_look_ahead():
    """Causal front with w0 = w1 = e_{2,2} and zero biases gives
    y[t2, f2] = [2 t2 < L1] max(0, x[4 t2, 4 f2]); and output row t2 never
    depends on mel rows after 4 t2."""
    r = rng(61)
    B, T, F, C = 3, 23, 17, 2
    x = f32(r.standard_normal((B, T, F)))
    e = np.zeros((3, 3, C), np.float32)
    e[2, 2] = 1.0
    z = np.zeros(C, np.float32)
    lengths = np.array([23, 10, 0], np.int32)
    y = oracle.dwsub_front_fwd(x, e, z, e, z, lengths, causal=True)
    T2, F2 = y.shape[1], y.shape[2]
    assert (T2, F2) == ((T // 2 + 1) // 2 + 1, (F // 2 + 1) // 2 + 1)
    ref = np.zeros_like(y)
    sub = np.maximum(x[:, 0::4, 0::4].astype(np.float64), 0.0)
    ref[:, : sub.shape[1], : sub.shape[2]] = sub[..., None]
    for bi, l in enumerate(lengths):
        L1 = l // 2 + 1 if l > 0 else 0
        ref[bi, (np.arange(T2) * 2) >= L1] = 0.0
    assert np.array_equal(y, ref)
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    y = oracle.dwsub_front_fwd(x, w0, b0, w1, b1, None, causal=True)
    for t2 in (1, 3):
        x2 = x.copy()
        x2[:, 4 * t2 + 1:] += 2.0
        y2 = oracle.dwsub_front_fwd(x2, w0, b0, w1, b1, None, causal=True)
        assert np.array_equal(y[:, : t2 + 1], y2[:, : t2 + 1])
        assert not np.array_equal(y[:, t2 + 1], y2[:, t2 + 1])


def test_front_causal_empty_item_is_output_bias():
    r = rng(62)
    B, T, F, C = 2, 12, 10, 3
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(np.abs(r.standard_normal(C)) + 1), f32(r.standard_normal(C))
    y = oracle.dwsub_front_fwd(x, w0, b0, w1, b1, np.array([0, 12], np.int32), causal=True)
    assert np.all(y[0] == b1.astype(np.float64)[None, None, :])


# ------------------------------------------------- fused front backward -----

def torch_front_grads(x, w0, b0, w1, b1, lengths, dy):
    B, T, F = x.shape
    C = w0.shape[2]
    L = eff_len(lengths, B, T)
    t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64)).requires_grad_(True)
    tw0, tb0, tw1, tb1 = t(w0), t(b0), t(w1), t(b1)
    xt = torch.from_numpy(x.astype(np.float64))[:, None]
    h = Fn.conv2d(xt, tw0.permute(2, 0, 1)[:, None], tb0, stride=2, padding=1)
    h = torch.relu(h)
    L1 = (L + 1) // 2
    m = (torch.arange(h.shape[2])[None, :] < torch.as_tensor(L1)[:, None])[:, None, :, None]
    h = torch.where(m, h, torch.zeros(()))
    y = Fn.conv2d(h, tw1.permute(2, 0, 1)[:, None], tb1, stride=2, padding=1, groups=C).permute(0, 2, 3, 1)
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return tw0.grad.numpy(), tb0.grad.numpy(), tw1.grad.numpy(), tb1.grad.numpy()


@pytest.mark.parametrize("B,T,F,C", [(2, 16, 12, 4), (3, 13, 9, 3), (1, 1, 1, 2), (2, 30, 20, 5), (1, 7, 80, 2)])
def test_front_bwd_matches_torch_autograd(B, T, F, C):
    r = rng(40 + B + T + F + C)
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    T2, F2 = (((T + 1) // 2) + 1) // 2, (((F + 1) // 2) + 1) // 2
    dy = f32(r.standard_normal((B, T2, F2, C)))
    for lengths in (None, r.integers(-1, T + 2, B).astype(np.int32)):
        got = oracle.dwsub_front_bwd(x, w0, b0, w1, lengths, dy)
        ref = torch_front_grads(x, w0, b0, w1, b1, lengths, dy)
        for g, rf in zip(got, ref):
            close(g, rf)


def test_front_bwd_closed_forms_and_linearity():
    r = rng(45)
    B, T, F, C = 2, 20, 14, 3
    x = f32(r.standard_normal((B, T, F)))
    w0 = f32(r.standard_normal((3, 3, C)))
    w1 = f32(r.integers(-4, 5, (3, 3, C)) / 4.0)  # quarter-integers: w1 +- 0.5 is exact in float32
    b0 = f32(r.standard_normal(C))
    lengths = np.array([20, 9], np.int32)
    dy1 = f32(r.integers(-4, 5, (B, 5, 4, C)))
    dy2 = f32(r.integers(-4, 5, (B, 5, 4, C)))
    g1 = oracle.dwsub_front_bwd(x, w0, b0, w1, lengths, dy1)
    g2 = oracle.dwsub_front_bwd(x, w0, b0, w1, lengths, dy2)
    g12 = oracle.dwsub_front_bwd(x, w0, b0, w1, lengths, f32(dy1 + dy2))
    for a, b_, c in zip(g1, g2, g12):
        close(c, a + b_, 1e-12)                                   # linear in dy
    close(g1[3], dy1.astype(np.float64).sum(axis=(0, 1, 2)))     # db1 = sum of dy
    # dw1 is the loss's exact derivative in w1: y is linear in w1
    loss = lambda ww1: float(np.sum((oracle.dwsub_front_fwd(x, w0, b0, ww1, np.zeros(C, np.float32), lengths))
                                    * dy1.astype(np.float64)))
    for idx in [(0, 0, 0), (1, 1, 2), (2, 1, 1)]:
        e = np.zeros_like(w1)
        e[idx] = 0.5
        fd = (loss(w1 + e) - loss(w1 - e)) / 1.0
        assert abs(fd - g1[2][idx]) <= 1e-9 * (1 + abs(fd))


def test_front_bwd_masked_input_rows_never_read():
    r = rng(46)
    B, T, F, C = 2, 24, 10, 3
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0 = f32(r.standard_normal(C))
    lengths = np.array([24, 9], np.int32)  # L1 = 5 for item 1: mel rows >= 10 feed no unmasked h row
    dy = f32(r.standard_normal((B, 6, 3, C)))
    g = oracle.dwsub_front_bwd(x, w0, b0, w1, lengths, dy)
    xp = x.copy()
    xp[1, 10:] = np.nan
    for a, b_ in zip(g, oracle.dwsub_front_bwd(xp, w0, b0, w1, lengths, dy)):
        assert np.array_equal(a, b_)


# ------------------------------------------------------ 1-D backward -----

def torch_dwconv1d_grads(x, w, b, lengths, dy, causal):
    B, T, C = x.shape
    K = w.shape[0]
    L = eff_len(lengths, B, T)
    tmask = (torch.arange(T)[None, :] < torch.as_tensor(L)[:, None])[:, :, None]
    xt = torch.from_numpy(x.astype(np.float64)).requires_grad_(True)
    wt = torch.from_numpy(w.astype(np.float64)).requires_grad_(True)
    bt = torch.from_numpy(b.astype(np.float64)).requires_grad_(True)
    xm = torch.where(tmask, xt, torch.zeros(())).permute(0, 2, 1)
    pL = K - 1 if causal else (K - 1) // 2
    xm = Fn.pad(xm, (pL, K - 1 - pL))
    y = Fn.conv1d(xm, wt.t()[:, None, :], bt, groups=C).permute(0, 2, 1)
    y = torch.where(tmask, y, torch.zeros(()))
    (y * torch.from_numpy(dy.astype(np.float64))).sum().backward()
    return xt.grad.numpy(), wt.grad.numpy(), bt.grad.numpy()


@pytest.mark.parametrize("B,T,C,K,causal", GRID_1D)
def test_1d_bwd_matches_torch_autograd(B, T, C, K, causal):
    r = rng(50 + B * 100 + T + K)
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    b = f32(r.standard_normal(C))
    dy = f32(r.standard_normal((B, T, C)))
    for lengths in (None, r.integers(-2, T + 3, B).astype(np.int32)):
        got = oracle.dwconv1d_bwd(x, w, lengths, dy, causal)
        ref = torch_dwconv1d_grads(x, w, b, lengths, dy, causal)
        for g_, r_ in zip(got, ref):
            close(g_, r_)


def test_1d_bwd_adjoint_closed_forms_and_masks():
    r = rng(51)
    B, T, C, K = 3, 30, 4, 9
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.standard_normal((K, C)))
    dy = f32(r.standard_normal((B, T, C)))
    lengths = np.array([30, 11, 0], np.int32)
    for causal in (False, True):
        dx, dw, db = oracle.dwconv1d_bwd(x, w, lengths, dy, causal)
        y_nb = oracle.dwconv1d_fwd(x, w, None, lengths, causal)
        mask = (np.arange(T)[None, :] < lengths[:, None])[:, :, None]
        g = dy.astype(np.float64) * mask
        inner = np.sum(g * y_nb)
        close(np.sum(dx * x.astype(np.float64)), inner, 1e-10)      # adjoint in x
        close(np.sum(dw * w.astype(np.float64)), inner, 1e-10)      # bilinear in (x, w)
        close(db, g.sum(axis=(0, 1)))                               # db = masked sum of dy
        assert np.all(dx[1, 11:] == 0) and np.all(dx[2] == 0)
        xn, dyn = x.copy(), dy.copy()
        xn[1, 11:] = np.nan
        dyn[1, 11:] = np.nan
        dyn[2] = np.nan
        for a, b_ in zip((dx, dw, db), oracle.dwconv1d_bwd(xn, w, lengths, dyn, causal)):
            assert np.array_equal(a, b_)


def test_1d_bwd_finite_differences_in_w():
    r = rng(52)
    B, T, C, K = 2, 20, 3, 5
    x = f32(r.standard_normal((B, T, C)))
    w = f32(r.integers(-4, 5, (K, C)) / 4.0)
    dy = f32(r.standard_normal((B, T, C)))
    lengths = np.array([20, 13], np.int32)
    _, dw, _ = oracle.dwconv1d_bwd(x, w, lengths, dy, True)
    loss = lambda ww: float(np.sum(oracle.dwconv1d_fwd(x, ww, None, lengths, True) * dy.astype(np.float64)))
    for idx in itertools.product(range(K), range(C)):
        e = np.zeros_like(w)
        e[idx] = 0.5
        assert abs((loss(w + e) - loss(w - e)) - dw[idx]) <= 1e-9 * (1 + abs(dw[idx]))


# ------------------------------------------------- streaming 1-D conv -----

def torch_causal_conv1d_seq(seq, w, b):
    """Causal depthwise conv of one whole sequence seq [T, C] (torch, fp64)."""
    T, C = seq.shape
    K = w.shape[0]
    xt = torch.from_numpy(seq.astype(np.float64)).t()[None]                 # [1, C, T]
    xt = Fn.pad(xt, (K - 1, 0))
    wt = torch.from_numpy(w.astype(np.float64)).t().contiguous()[:, None]  # [C, 1, K]
    bt = torch.from_numpy(b.astype(np.float64))
    return Fn.conv1d(xt, wt, bt, groups=C)[0].t().numpy()


def run_stream(chunks, lens, w, b, K, C):
    """Feed chunks [n][B,Tc,C] with per-stream valid lengths through the
    streaming oracle from a zero cache; returns each stream's valid outputs
    concatenated, and the final cache."""
    B = chunks[0].shape[0]
    cache = np.zeros((B, K - 1, C), np.float32)
    outs = [[] for _ in range(B)]
    for x, L in zip(chunks, lens):
        y, cache64 = oracle.dwconv1d_stream_fwd(x, w, b, L, cache)
        cache = cache64.astype(np.float32)
        assert np.array_equal(cache.astype(np.float64), cache64)   # a cache holds input values exactly
        for bi in range(B):
            l = min(max(int(L[bi]), 0), x.shape[1])
            outs[bi].append(y[bi, :l])
            assert np.all(y[bi, l:] == 0)
    return [np.concatenate(o, axis=0) for o in outs], cache


@pytest.mark.parametrize("K", [1, 2, 3, 4, 9, 15])
def test_1d_stream_chunks_equal_the_whole_causal_conv(K):
    r = rng(70 + K)
    B, C, Tc, n = 3, 5, 6, 7
    chunks = [f32(r.standard_normal((B, Tc, C))) for _ in range(n)]
    lens = [r.integers(-1, Tc + 2, B).astype(np.int32) for _ in range(n)]
    lens[2][0] = 0                           # a stream with nothing new in one chunk
    w, b = f32(r.standard_normal((K, C))), f32(r.standard_normal(C))
    got, cache = run_stream(chunks, lens, w, b, K, C)
    for bi in range(B):
        seq = np.concatenate([x[bi, :min(max(int(L[bi]), 0), Tc)] for x, L in zip(chunks, lens)], axis=0)
        close(got[bi], torch_causal_conv1d_seq(seq, w, b))
        tail = np.concatenate([np.zeros((K - 1, C), np.float32), seq], axis=0)[len(seq):]
        assert np.array_equal(cache[bi], tail)   # the last K-1 frames of the whole sequence


def test_1d_stream_single_chunk_from_zero_cache_is_the_causal_conv():
    r = rng(77)
    B, T, C, K = 3, 20, 4, 9
    x = f32(r.standard_normal((B, T, C)))
    w, b = f32(r.standard_normal((K, C))), f32(r.standard_normal(C))
    L = np.array([20, 7, 0], np.int32)
    y, _ = oracle.dwconv1d_stream_fwd(x, w, b, L, np.zeros((B, K - 1, C), np.float32))
    assert np.array_equal(y, oracle.dwconv1d_fwd(x, w, b, L, True))


def test_1d_stream_delta_kernels_read_the_cache():
    """w = e_0 returns the sequence K-1 frames back (the cache first); w =
    e_{K-1} is the identity on the chunk."""
    r = rng(78)
    B, Tc, C, K = 2, 10, 3, 5
    x = f32(r.standard_normal((B, Tc, C)))
    cache = f32(r.standard_normal((B, K - 1, C)))
    L = np.array([10, 3], np.int32)
    z = np.zeros(C, np.float32)
    e0 = np.zeros((K, C), np.float32)
    e0[0] = 1.0
    y, c2 = oracle.dwconv1d_stream_fwd(x, e0, z, L, cache)
    for bi, l in enumerate(L):
        seq = np.concatenate([cache[bi], x[bi, :l]], axis=0).astype(np.float64)
        assert np.array_equal(y[bi, :l], seq[:l]) and np.all(y[bi, l:] == 0)
        assert np.array_equal(c2[bi], seq[l:l + K - 1])
    eK = np.zeros((K, C), np.float32)
    eK[K - 1] = 1.0
    y, _ = oracle.dwconv1d_stream_fwd(x, eK, z, L, cache)
    for bi, l in enumerate(L):
        assert np.array_equal(y[bi, :l], x[bi, :l].astype(np.float64))


def test_1d_stream_empty_chunk_keeps_the_cache_and_nan_past_length_never_read():
    r = rng(79)
    B, Tc, C, K = 2, 6, 3, 4
    x = f32(r.standard_normal((B, Tc, C)))
    w, b = f32(r.standard_normal((K, C))), f32(r.standard_normal(C))
    cache = f32(r.standard_normal((B, K - 1, C)))
    L = np.array([0, 4], np.int32)
    y, c2 = oracle.dwconv1d_stream_fwd(x, w, b, L, cache)
    assert np.all(y[0] == 0) and np.array_equal(c2[0], cache[0].astype(np.float64))
    xn = x.copy()
    xn[0] = np.nan
    xn[1, 4:] = np.nan
    y2, c3 = oracle.dwconv1d_stream_fwd(xn, w, b, L, cache)
    assert np.array_equal(y, y2) and np.array_equal(c2, c3)


# ------------------------------------------------------- null biases -----

def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float64).view(np.uint64)


@pytest.mark.parametrize("causal", [False, True])
def test_null_bias_is_zero_bias_in_every_function(causal):
    """A NULL bias means zero for every operation that takes one: the result
    is bit for bit the zero-bias result (sign of zero included), and matches
    torch's chain run with zero biases."""
    r = rng(90 + causal)
    B, T, F, C = 2, 19, 11, 3
    lengths = np.array([19, 8], np.int32)
    zc = np.zeros(C, np.float32)
    # fused front, forward: either bias NULL, and both
    x = f32(r.standard_normal((B, T, F)))
    w0, w1 = f32(r.standard_normal((3, 3, C))), f32(r.standard_normal((3, 3, C)))
    b0, b1 = f32(r.standard_normal(C)), f32(r.standard_normal(C))
    tf = torch_front_causal if causal else torch_front
    for nb0, nb1 in ((True, False), (False, True), (True, True)):
        got = oracle.dwsub_front_fwd(x, w0, None if nb0 else b0, w1, None if nb1 else b1, lengths, causal=causal)
        zero = oracle.dwsub_front_fwd(x, w0, zc if nb0 else b0, w1, zc if nb1 else b1, lengths, causal=causal)
        assert np.array_equal(_bits(got), _bits(zero))
        close(got, tf(x, w0, zc if nb0 else b0, w1, zc if nb1 else b1, lengths))
    # fused front, backward: NULL b0
    T2, F2 = got.shape[1], got.shape[2]
    dy = f32(r.standard_normal((B, T2, F2, C)))
    for g, z in zip(oracle.dwsub_front_bwd(x, w0, None, w1, lengths, dy, causal=causal),
                    oracle.dwsub_front_bwd(x, w0, zc, w1, lengths, dy, causal=causal)):
        assert np.array_equal(_bits(g), _bits(z))
    # 1-D conv and the streaming conv
    x1 = f32(r.standard_normal((B, T, C)))
    w9 = f32(r.standard_normal((9, C)))
    got = oracle.dwconv1d_fwd(x1, w9, None, lengths, causal)
    assert np.array_equal(_bits(got), _bits(oracle.dwconv1d_fwd(x1, w9, zc, lengths, causal)))
    close(got, torch_dwconv1d(x1, w9, zc, lengths, causal))
    cache = f32(r.standard_normal((B, 8, C)))
    for a, z in zip(oracle.dwconv1d_stream_fwd(x1, w9, None, lengths, cache),
                    oracle.dwconv1d_stream_fwd(x1, w9, zc, lengths, cache)):
        assert np.array_equal(_bits(a), _bits(z))
    # conv2d
    x2 = f32(r.standard_normal((B, T, F, C)))
    pads = (2, 1, 2, 1) if causal else (1, 1, 1, 1)
    got = oracle.dwconv2d_fwd(x2, w0, None, lengths, pads=pads)
    assert np.array_equal(_bits(got), _bits(oracle.dwconv2d_fwd(x2, w0, zc, lengths, pads=pads)))
    close(got, torch_dwconv2d_pads(x2, w0, zc, lengths, 2, pads))
