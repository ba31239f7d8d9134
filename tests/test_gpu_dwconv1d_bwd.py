"""GPU parity of dwconv1d_bwd (through the C ABI) against the CPU oracle."""
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_exact_zero, assert_parity, say, time_mask

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def make(B, T, C, K, seed=0, lens=None):
    tag = f"t1b/{B}/{T}/{C}/{K}/{seed}"
    x = datagen.normal((B, T, C), 1.0, tag + "/x", device=DEV)
    w = datagen.normal((K, C), 1.0 / K, tag + "/w", device=DEV)
    dy = datagen.normal((B, T, C), 1.0, tag + "/dy", device=DEV)
    if lens is None:
        lens = datagen.int_uniform(B, 0, T, tag + "/len")
    return x, w, dy, torch.as_tensor(lens, dtype=torch.int32).to(DEV)


def run(x, w, L, dy, causal, need=("dx", "dw", "db"), workspace=None):
    g = lib().dwconv1d_bwd(x, w, L, dy, causal=causal, need=need, workspace=workspace)
    torch.cuda.synchronize()
    return g


def check(x, w, L, dy, causal, what):
    B, T, C = x.shape
    say(f"dwconv1d_bwd {what}: B={B} T={T} C={C} K={w.shape[0]} causal={causal}")
    got = run(x, w, L, dy, causal)
    ref = oracle.dwconv1d_bwd(x, w, L, dy, causal)
    for name, g, r in zip(("dx", "dw", "db"), got, ref):
        assert_parity(g, r, TOL_F32, f"{what} {name}")
    Lh = L.cpu() if L is not None else torch.full((B,), T, dtype=torch.int32)
    assert_exact_zero(got[0], time_mask(Lh, B, T)[:, :, None], f"{what} dx")
    return got


GRID = [
    # (B, T, C, K, causal)
    (1, 1, 4, 3, False), (3, 1, 8, 9, True), (1, 2, 4, 5, False), (3, 7, 3, 4, False), (3, 7, 3, 4, True),
    (2, 50, 8, 15, False), (2, 50, 8, 15, True), (2, 13, 6, 7, True), (1, 33, 100, 9, False),
    (3, 45, 200, 9, True), (2, 17, 256, 3, True), (1, 100, 1, 9, False), (2, 64, 128, 31, False),
    (2, 70, 130, 31, True), (3, 49, 6, 9, False), (1, 300, 64, 5, False), (5, 97, 44, 5, True),
    (2, 129, 512, 9, True),
]


@pytest.mark.parametrize("B,T,C,K,causal", GRID)
def test_grid(B, T, C, K, causal):
    x, w, dy, L = make(B, T, C, K)
    check(x, w, L, dy, causal, "grid")


def test_null_and_clamped_lengths():
    B, T, C, K = 3, 40, 16, 9
    x, w, dy, _ = make(B, T, C, K)
    check(x, w, None, dy, False, "null lengths")
    over = torch.tensor([T + 5, -3, 17], dtype=torch.int32, device=DEV)
    got = run(x, w, over, dy, True)
    ref = oracle.dwconv1d_bwd(x, w, torch.tensor([T, 0, 17], dtype=torch.int32), dy, True)
    for g, r in zip(got, ref):
        assert_parity(g, r, TOL_F32, "clamped lengths")


def test_masked_frames_are_never_read():
    B, T, C, K = 3, 60, 32, 9
    x, w, dy, L = make(B, T, C, K, lens=[60, 21, 0])
    full = run(x, w, L, dy, False)
    xp, dyp = x.clone(), dy.clone()
    xp[1, 21:] = float("nan")
    dyp[1, 21:] = float("nan")
    xp[2] = float("nan")
    dyp[2] = float("nan")
    for a, b in zip(full, run(xp, w, L, dyp, False)):
        assert torch.equal(a, b)


def test_subsets_and_repeatable_bitwise():
    B, T, C, K = 4, 200, 64, 5
    x, w, dy, L = make(B, T, C, K)
    full = run(x, w, L, dy, True)
    again = run(x, w, L, dy, True)
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    for need in (("dx",), ("dw",), ("db",), ("dw", "db")):
        got = run(x, w, L, dy, True, need=need)
        for name, a, b in zip(("dx", "dw", "db"), got, full):
            assert (a is None) == (name not in need)
            if a is not None:
                assert torch.equal(a, b), name


def test_unaligned_pointers_take_the_narrow_path():
    B, T, C, K = 2, 30, 64, 5
    x, wt, dy, L = make(B, T, C, K)
    xs = torch.empty(B * T * C + 1, device=DEV)[1:].view(B, T, C)
    xs.copy_(x)
    check(xs, wt, L, dy, False, "unaligned x")


def test_short_workspace_raises_and_empty_batch_is_zero():
    x, w, dy, L = make(2, 16, 8, 9)
    need = lib().dwconv1d_bwd_workspace_bytes(2, 16, 8, 9)
    with pytest.raises(lib().DwconvError, match="workspace"):
        run(x, w, L, dy, False, workspace=torch.empty(need - 8, dtype=torch.uint8, device=DEV))
    dw_, db = torch.full((9, 8), 3.0, device=DEV), torch.full((8,), 3.0, device=DEV)
    lib().dwconv1d_bwd(x[:0], w, L[:0], dy[:0], dw=dw_, db=db, need=("dw", "db"))
    torch.cuda.synchronize()
    assert torch.all(dw_ == 0) and torch.all(db == 0)


def test_unsupported_width_raises():
    x, w, dy, L = make(1, 8, 4, 6)
    with pytest.raises(lib().DwconvError, match="K=6"):
        run(x, w, L, dy, False)


@pytest.mark.parametrize("K", [9, 31])
def test_conv_module_full_size(K):
    c = datagen.conv1d_causal_sweep(K, device=DEV)
    dy = datagen.normal((c["B"], c["T"], c["C"]), 1.0, f"c4/dy/K{K}/C{c['C']}", device=DEV)
    check(c["x"], c["w"], c["lengths"].to(DEV), dy, True, f"full [32,1500,512] K={K}")


# ----------------------------------------------------------- bf16 storage -----

BF16_GRID = [(1, 1, 4, 3, False), (3, 7, 3, 4, True), (2, 50, 8, 15, False), (3, 45, 200, 9, True),
             (2, 64, 128, 31, False), (5, 97, 44, 5, True), (2, 129, 512, 9, True), (2, 17, 256, 3, False)]


@pytest.mark.parametrize("B,T,C,K,causal", BF16_GRID)
def test_bf16_grid(B, T, C, K, causal):
    x, w, dy, L = make(B, T, C, K)
    x, w, dy = x.to(torch.bfloat16), w.to(torch.bfloat16), dy.to(torch.bfloat16)
    say(f"dwconv1d_bwd bf16: B={B} T={T} C={C} K={K} causal={causal}")
    gx, gw, gb = run(x, w, L, dy, causal)
    assert gx.dtype == torch.bfloat16 and gw.dtype == torch.float32
    rx, rw, rb = oracle.dwconv1d_bwd(x, w, L, dy, causal)
    assert_parity(gx, rx, TOL_BF16, "bf16 dx")
    assert_parity(gw, rw, TOL_F32, "bf16 dw")      # float outputs, fp64 sums of exact products
    assert_parity(gb, rb, TOL_F32, "bf16 db")
    assert_exact_zero(gx, time_mask(L.cpu(), B, T)[:, :, None], "bf16 dx")


@pytest.mark.parametrize("K", [5, 9])
def test_bf16_is_the_fp32_kernel_rounded(K):
    """Same arithmetic on exactly widened values: dx is the fp32 result rounded
    to nearest even, dw and db are identical."""
    x, w, dy, L = make(3, 80, 64, K)
    x, w, dy = x.to(torch.bfloat16), w.to(torch.bfloat16), dy.to(torch.bfloat16)
    a = run(x, w, L, dy, True)
    b = run(x.float(), w.float(), L, dy.float(), True)
    assert torch.equal(a[0], b[0].to(torch.bfloat16))
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


def test_bf16_conv_module_full_size():
    c = datagen.conv1d_causal_sweep(9, device=DEV)
    dy = datagen.normal((c["B"], c["T"], c["C"]), 1.0, "c4/dy/K9/C512", device=DEV).to(torch.bfloat16)
    x, w = c["x"].to(torch.bfloat16), c["w"].to(torch.bfloat16)
    L = c["lengths"].to(DEV)
    say("dwconv1d_bwd bf16 full [32,1500,512] K9")
    gx, gw, gb = run(x, w, L, dy, True)
    rx, rw, rb = oracle.dwconv1d_bwd(x, w, L, dy, True)
    assert_parity(gx, rx, TOL_BF16, "full bf16 dx")
    assert_parity(gw, rw, TOL_F32, "full bf16 dw")
    assert_parity(gb, rb, TOL_F32, "full bf16 db")


def _offset8(t):
    """A copy of t whose storage starts 8 bytes past a 16-byte-aligned address."""
    k = 8 // t.element_size()
    buf = torch.empty(t.numel() + k, dtype=t.dtype, device=t.device)
    out = buf[k:].view(t.shape)
    out.copy_(t)
    return out


@pytest.mark.parametrize("B,T,C,K,causal", [(3, 75, 512, 9, True), (2, 61, 100, 9, False), (4, 40, 20, 15, True),
                                            (2, 33, 260, 15, False), (3, 130, 8, 9, False), (1, 1, 4, 9, True),
                                            (3, 2, 4, 15, False), (2, 9, 12, 9, False), (3, 90, 64, 7, True),
                                            (2, 31, 36, 7, False), (2, 40, 128, 31, True), (3, 37, 36, 31, False),
                                            (1, 3, 4, 31, True)])
def test_paired_lanes_match_eight_byte_lanes(B, T, C, K, causal):
    """fp32 with 16-byte-aligned tensors takes the lane-group form at K = 7, 9
    and 15 (pairs of lanes, two channels each) and at K = 31 (four lanes, one
    channel each): 16-byte loads and stores, transposed through cross-lane
    swaps.  The same call 8 bytes off that alignment takes two-channel lanes
    with 8-byte accesses (one channel, 4-byte accesses at K = 31).  Both run
    the same per-element arithmetic: dx is equal bit for bit; dw and db are
    the same fp64 sums over another split of the tiles across workgroups, so
    they agree to within one float32 ulp."""
    x, w, dy, L = make(B, T, C, K, lens=[T, T // 2 + 1, 0, max(T - 9, 0)][:B])
    say(f"dwconv1d_bwd paired against 8-byte lanes B={B} T={T} C={C} K={K} causal={causal}")
    wide = run(x, w, L, dy, causal)
    x8, dy8 = _offset8(x), _offset8(dy)
    dx8 = _offset8(torch.full_like(x, float("nan")))
    _, dw8, db8 = lib().dwconv1d_bwd(x8, w, L, dy8, dx=dx8, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(wide[0], dx8), "dx"
    for a, b in ((wide[1], dw8), (wide[2], db8)):
        mag = torch.maximum(a.abs(), b.abs())
        ulp = torch.nextafter(mag, torch.full_like(mag, float("inf"))) - mag
        assert torch.all((a - b).abs() <= ulp)
    ref = oracle.dwconv1d_bwd(x, w, L, dy, causal)
    for name, g, r in zip(("dx", "dw", "db"), wide, ref):
        assert_parity(g, r, TOL_F32, f"paired {name}")


@pytest.mark.parametrize("B,T,C,K,causal", [(3, 75, 512, 9, True), (2, 61, 104, 9, False), (4, 40, 24, 15, True),
                                            (2, 33, 264, 15, False), (3, 90, 64, 7, True), (1, 3, 8, 9, True),
                                            (2, 9, 16, 7, False)])
def test_bf16_lane_groups_match_narrow_lanes(B, T, C, K, causal):
    """bf16 at K = 7, 9 and 15 with 16-byte-aligned tensors (C a multiple of
    8) takes groups of four lanes, two channels each, sharing a 16-byte piece
    of eight channels.  The same call 8 bytes off that alignment takes
    four-channel 8-byte lanes (two-channel 4-byte lanes at K = 7 and 15).  The
    arithmetic per element is the same: dx is equal bit for bit, and dw and
    db, summed over another split of the tiles, agree to one float32 ulp."""
    x, w, dy, L = make(B, T, C, K, lens=[T, T // 2 + 1, 0, max(T - 9, 0)][:B])
    x, w, dy = x.to(torch.bfloat16), w.to(torch.bfloat16), dy.to(torch.bfloat16)
    say(f"dwconv1d_bwd bf16 lane groups against narrow lanes B={B} T={T} C={C} K={K} causal={causal}")
    wide = run(x, w, L, dy, causal)
    x8, dy8 = _offset8(x), _offset8(dy)
    dx8 = _offset8(torch.full_like(x, float("nan")))
    _, dw8, db8 = lib().dwconv1d_bwd(x8, w, L, dy8, dx=dx8, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(wide[0], dx8), "dx"
    for a, b in ((wide[1], dw8), (wide[2], db8)):
        mag = torch.maximum(a.abs(), b.abs())
        ulp = torch.nextafter(mag, torch.full_like(mag, float("inf"))) - mag
        assert torch.all((a - b).abs() <= ulp)
    ref = oracle.dwconv1d_bwd(x, w, L, dy, causal)
    for name, g, r, tol in zip(("dx", "dw", "db"), wide, ref, (TOL_BF16, TOL_F32, TOL_F32)):
        assert_parity(g, r, tol, f"bf16 lane groups {name}")
