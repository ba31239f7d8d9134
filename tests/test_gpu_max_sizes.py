"""The largest single items the kernels address (32-bit byte offsets within an
item), one frame past that rejected, and parity there: outputs sampled on
windows that the oracle computes from a slice of the input, and the weight
gradients over the whole item against their plain definitions summed in fp64."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_F32, assert_parity, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


# 1-D: (T + K + 32) * C * 4 bytes must stay below 2^31
C1, K1 = 256, 9
T1_MAX = (1 << 31) // (C1 * 4) - K1 - 32 - 1


def test_1d_largest_item_fwd_and_bwd():
    T = T1_MAX
    L = T - 5
    say(f"dwconv1d max item: T={T} C={C1} K={K1} causal, len={L}")
    x = datagen.normal((1, T, C1), 1.0, "max1/x", device=DEV)
    w = datagen.normal((K1, C1), 1.0 / K1, "max1/w", device=DEV)
    b = datagen.normal((C1,), 0.1, "max1/b", device=DEV)
    Ld = torch.tensor([L], dtype=torch.int32, device=DEV)
    y = lib().dwconv1d_fwd(x, w, b, Ld, causal=True)
    torch.cuda.synchronize()
    # windows of output frames [a, a + 64): the oracle on x[lo:a+64] with lo = a - (K-1)
    for a in (0, 1000, T // 2 + 3, L - 64, L - 30, T - 64):
        lo, hi = max(0, a - (K1 - 1)), min(T, a + 64)
        xs = x[:, lo:hi]
        ref = oracle.dwconv1d_fwd(xs, w, b, np.array([min(max(L - lo, 0), hi - lo)], np.int32), True)
        assert_parity(y[:, a:hi], ref[:, a - lo:], TOL_F32, f"y window {a}")
    assert torch.all(y[0, L:] == 0)
    del y
    dy = datagen.normal((1, T, C1), 1.0, "max1/dy", device=DEV)
    dx, dw, db = lib().dwconv1d_bwd(x, w, Ld, dy, causal=True)
    torch.cuda.synchronize()
    for a in (0, 777, T // 3, L - 64, L - 3, T - 64):
        lo, hi = max(0, a), min(T, a + 64 + K1 - 1)      # dx[u] needs dy[u .. u + K - 1] (causal)
        rdx, _, _ = oracle.dwconv1d_bwd(x[:, lo:hi], w, np.array([min(max(L - lo, 0), hi - lo)], np.int32),
                                        dy[:, lo:hi], True, want=("dx",))
        n = min(64, T - a)
        assert_parity(dx[:, a:a + n], rdx[:, :n], TOL_F32, f"dx window {a}")
    # dw[k] = sum_{t<L, t-(K-1)+k >= 0} dy[t] x[t-(K-1)+k]; db = sum_{t<L} dy[t]  (fp64 on the GPU)
    g = dy[0, :L].double()
    xd = x[0, :L].double()
    for k in range(K1):
        s = K1 - 1 - k                                     # x index = t - s
        ref = (g[s:] * xd[:L - s]).sum(dim=0)
        assert_parity(dw[k], ref.cpu().numpy(), TOL_F32, f"dw[{k}]")
    assert_parity(db, g.sum(dim=0).cpu().numpy(), TOL_F32, "db")


def test_1d_one_frame_past_the_limit_is_rejected():
    T = T1_MAX + 1
    x = torch.empty((1, T, C1), device=DEV)
    w = torch.zeros((K1, C1), device=DEV)
    with pytest.raises(lib().DwconvError, match="too large"):
        lib().dwconv1d_fwd(x, w, None, None, causal=True)
    with pytest.raises(lib().DwconvError, match="too large"):
        lib().dwconv1d_bwd(x, w, None, x.clone(), causal=True, need=("dx",))


# 2-D: (T + 4) * F * C * 4 bytes must stay below 2^31
F2, C2 = 64, 256
T2_MAX = (1 << 31) // (F2 * C2 * 4) - 4 - 1


def test_2d_largest_item_fwd_and_bwd():
    T = T2_MAX
    L = T - 3
    say(f"dwconv2d max item: [{T},{F2},{C2}] len={L}")
    s = datagen.conv2d_stage(device=DEV, B=1, T=T, F=F2, C=C2)
    x, w, b, dy = s["x"], s["w"], s["b"], s["dy"]
    Ld = torch.tensor([L], dtype=torch.int32, device=DEV)
    To = (T + 1) // 2
    y = lib().dwconv2d_fwd(x, w, b, Ld)
    torch.cuda.synchronize()
    Lo = (L + 1) // 2
    # output rows [p, p + 16): the oracle on input rows [2p - 2, 2p + 33) (an even start keeps the parity)
    for p in (0, 1, To // 2, Lo - 16, Lo - 1, To - 16):
        p = max(p, 0)
        lo, hi = max(0, 2 * p - 2), min(T, 2 * p + 33)
        ref = oracle.dwconv2d_fwd(x[:, lo:hi], w, b, np.array([min(max(L - lo, 0), hi - lo)], np.int32))
        n = min(16, To - p)
        assert_parity(y[:, p:p + n], ref[:, p - lo // 2:p - lo // 2 + n], TOL_F32, f"y rows {p}")
    assert torch.all(y[0, Lo:] == 0)
    del y
    dx, dw, db = lib().dwconv2d_bwd(x, w, Ld, dy)
    torch.cuda.synchronize()
    # dx rows [a, a + 16), a even: dy rows [a/2 - 1, a/2 + 9) and x rows [a - 2, a + 18)
    for a in (0, 2, T // 2 - 1, L - 16, L - 1, T - 16):
        a = max(0, a - (a % 2))
        lo, hi = max(0, a - 2), min(T, a + 18)
        glo = lo // 2
        ghi = glo + (hi - lo + 1) // 2
        rdx, _, _ = oracle.dwconv2d_bwd(x[:, lo:hi], w, np.array([min(max(L - lo, 0), hi - lo)], np.int32),
                                        dy[:, glo:ghi], want=("dx",))
        n = min(16, T - a)
        assert_parity(dx[:, a:a + n], rdx[:, a - lo:a - lo + n], TOL_F32, f"dx rows {a}")
    # dw[i,j] = sum over valid output rows of g[t',f'] xm[2t'+i-1, 2f'+j-1]; db = sum g  (fp64 on the GPU)
    g = dy[0, :Lo].double()                                   # [Lo, Fo, C]
    xm = torch.zeros((2 * Lo + 2, F2 + 2, C2), dtype=torch.float64, device=DEV)
    xm[1:1 + L, 1:1 + F2] = x[0, :L].double()                 # xm[r + 1, c + 1] = x[r, c], zero elsewhere
    for i in range(3):
        for j in range(3):
            xs = xm[i:i + 2 * Lo:2, j:j + F2:2]                  # rows 2t' + i - 1, columns 2f' + j - 1
            assert_parity(dw[i, j], (g * xs).sum(dim=(0, 1)).cpu().numpy(), TOL_F32, f"dw[{i},{j}]")
    assert_parity(db, g.sum(dim=(0, 1)).cpu().numpy(), TOL_F32, "db")


def test_2d_one_row_past_the_limit_is_rejected():
    T = T2_MAX + 1
    x = torch.empty((1, T, F2, C2), device=DEV)
    w = torch.zeros((3, 3, C2), device=DEV)
    with pytest.raises(lib().DwconvError, match="too large"):
        lib().dwconv2d_fwd(x, w, None, None)


# fused front: (T2 + 4) * F2 * C * 4 bytes of output per item must stay below 2^31
FF, CF = 80, 256
T2F_MAX = (1 << 31) // (20 * CF * 4) - 4 - 1
TF_MAX = 4 * T2F_MAX


def test_front_largest_item_fwd_and_windowed_bwd():
    T = TF_MAX
    L = T - 400
    say(f"dwsub_fused max item: mel [{T},{FF}] -> [{T2F_MAX},20,{CF}] len={L}")
    f = datagen.fused_front(device=DEV, B=1, T=T, F=FF, C=CF)
    x = f["x"]
    Ld = torch.tensor([L], dtype=torch.int32, device=DEV)
    y = lib().dwsub_fused_fwd(x, f["w0"], f["b0"], f["w1"], f["b1"], Ld)
    torch.cuda.synchronize()
    assert y.shape == (1, T2F_MAX, 20, CF)
    # output rows [p, p + 8): the oracle on mel rows [4p - 4, 4p + 36); slice row r = original 4(p-1) + r
    # (a multiple of 4 keeps every stage's parity; its first output row is not compared)
    L2 = ((L + 1) // 2 + 1) // 2
    for p in (1, 1000, T2F_MAX // 2, L2 - 8, L2 - 1, T2F_MAX - 8):
        lo, hi = 4 * (p - 1), min(T, 4 * p + 36)
        ref = oracle.dwsub_front_fwd(x[:, lo:hi], f["w0"], f["b0"], f["w1"], f["b1"],
                                     np.array([min(max(L - lo, 0), hi - lo)], np.int32))
        n = min(8, T2F_MAX - p)
        assert_parity(y[:, p:p + n], ref[:, 1:1 + n], TOL_F32, f"y rows {p}")
    del y
    # gradients from dy that is zero except on output rows [p, p + 8) for a few disjoint p
    # (the front has no output mask: the window past the length still adds to db1)
    dy = torch.zeros((1, T2F_MAX, 20, CF), device=DEV)
    wins = (1, T2F_MAX // 2, L2 - 4, T2F_MAX - 8)
    assert all(b_ - a >= 8 for a, b_ in zip(wins, wins[1:]))
    for p in wins:
        dy[:, p:p + 8] = datagen.normal((1, 8, 20, CF), 1.0, f"maxf/dy/{p}", device=DEV)
    got = lib().dwsub_fused_bwd(x, f["w0"], f["b0"], f["w1"], Ld, dy)
    torch.cuda.synchronize()
    ref = [np.zeros((3, 3, CF)), np.zeros(CF), np.zeros((3, 3, CF)), np.zeros(CF)]
    for p in wins:
        lo, hi = 4 * (p - 1), min(T, 4 * p + 36)
        n2 = ((hi - lo + 1) // 2 + 1) // 2
        dys = torch.zeros((1, n2, 20, CF))
        dys[:, 1:9] = dy[:, p:p + 8].cpu()
        part = oracle.dwsub_front_bwd(x[:, lo:hi], f["w0"], f["b0"], f["w1"],
                                      np.array([min(max(L - lo, 0), hi - lo)], np.int32), dys)
        ref = [a + b_ for a, b_ in zip(ref, part)]
    for name, g_, r_ in zip(("dw0", "db0", "dw1", "db1"), got, ref):
        assert_parity(g_, r_, TOL_F32, f"windowed {name}")


# streaming conv: (Tc + 2K + 32) * C * es bytes per item must stay below 2^31
TS_MAX = (1 << 31) // (C1 * 2) - 2 * K1 - 32 - 1


def test_stream_largest_chunk_bf16():
    Tc = TS_MAX
    L = Tc - 11
    say(f"dwconv1d_stream max chunk: Tc={Tc} C={C1} K={K1} bf16 len={L}")
    x = datagen.normal((1, Tc, C1), 1.0, "maxs/x", device=DEV).to(torch.bfloat16)
    w = datagen.normal((K1, C1), 1.0 / K1, "maxs/w", device=DEV).to(torch.bfloat16)
    b = datagen.normal((C1,), 0.1, "maxs/b", device=DEV).to(torch.bfloat16)
    cache = datagen.normal((1, K1 - 1, C1), 1.0, "maxs/cache", device=DEV).to(torch.bfloat16)
    y, c2 = lib().dwconv1d_stream_fwd(x, w, b, torch.tensor([L], dtype=torch.int32, device=DEV), cache)
    torch.cuda.synchronize()
    ry, rc = oracle.dwconv1d_stream_fwd(x[:, :64], w, b, np.array([64], np.int32), cache)
    assert_parity(y[:, :64], ry, 2e-2, "first frames (from the cache)")
    for a in (Tc // 2, L - 64, L - 5):
        xs = x[:, a - (K1 - 1):a + 64]
        n = min(64, L - a)
        ry, _ = oracle.dwconv1d_stream_fwd(xs[:, K1 - 1:], w, b, np.array([n], np.int32), xs[:, :K1 - 1])
        assert_parity(y[:, a:a + n], ry[:, :n], 2e-2, f"window {a}")
    assert torch.all(y[0, L:] == 0)
    assert torch.equal(c2[0], x[0, L - (K1 - 1):L])
