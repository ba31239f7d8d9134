"""GPU parity of dwconv1d_fwd (through the C ABI) against the CPU oracle."""
import numpy as np
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


def run(x, w, b, lengths, causal, y=None):
    y = lib().dwconv1d_fwd(x, w, b, lengths, y=y, causal=causal)
    torch.cuda.synchronize()
    return y


def check(x, w, b, lengths, causal, what):
    B, T, C = x.shape
    say(f"dwconv1d {what}: B={B} T={T} C={C} K={w.shape[0]} causal={causal} dtype={x.dtype}")
    y = run(x, w, b, lengths, causal)
    ref = oracle.dwconv1d_fwd(x, w, b, lengths, causal)
    tol = TOL_BF16 if x.dtype == torch.bfloat16 else TOL_F32
    worst = assert_parity(y, ref, tol, what)
    L = lengths if lengths is not None else torch.full((B,), T, dtype=torch.int32)
    assert_exact_zero(y, time_mask(L, B, T)[:, :, None], what)
    return y, worst


def make(B, T, C, K, dtype=torch.float32, seed=0, lens=None, bias=True):
    tag = f"t1d/{B}/{T}/{C}/{K}/{seed}"
    x = datagen.normal((B, T, C), 1.0, tag + "/x", device=DEV).to(dtype)
    w = datagen.normal((K, C), 1.0 / K, tag + "/w", device=DEV).to(dtype)
    b = datagen.normal((C,), 0.1, tag + "/b", device=DEV).to(dtype) if bias else None
    if lens is None:
        lens = datagen.int_uniform(B, 0, T, tag + "/len")
    lengths = torch.as_tensor(lens, dtype=torch.int32).to(DEV)
    return x, w, b, lengths


def test_small_config_k9_symmetric():
    c = datagen.conv1d_small(device=DEV)
    check(c["x"], c["w"], c["b"], c["lengths"].to(DEV), False, "B=2 T=64 C=8 K=9")


GRID = [
    # (B, T, C, K, causal)
    (1, 1, 8, 3, False), (3, 1, 8, 9, True), (1, 2, 4, 5, False), (3, 7, 3, 4, False),
    (3, 7, 3, 4, True), (2, 50, 8, 15, False), (2, 50, 8, 15, True), (3, 20, 5, 1, False),
    (2, 13, 4, 2, False), (2, 13, 4, 2, True), (1, 33, 100, 9, False), (3, 45, 200, 9, True),
    (2, 17, 256, 3, True), (2, 40, 12, 7, False), (2, 40, 12, 16, True), (1, 100, 1, 9, False),
    (2, 64, 128, 31, False), (3, 49, 6, 9, False), (1, 300, 64, 5, False),
    # whole 64-lane slabs of 4-channel groups at K = 9, 15 (the LDS-staged fp32 forms):
    # ragged 32-frame tiles, T below the tile and below K, several slabs
    (3, 70, 256, 9, False), (4, 31, 256, 9, True), (2, 33, 512, 15, True), (1, 5, 256, 15, False),
    (2, 97, 768, 9, True), (3, 64, 256, 15, False),
    # partial last slabs of the LDS-staged form: 50, 45 and 65 (= 64 + 1) channel groups
    (2, 70, 200, 9, True), (2, 40, 180, 15, False), (2, 70, 260, 9, True),
    # the LDS-staged form at K = 3, 4, 5: whole and partial slabs, the minimum
    # of 32 groups, T below the tile and a single frame
    (3, 70, 256, 3, False), (2, 45, 200, 4, True), (2, 33, 512, 5, True), (1, 5, 256, 4, False),
    (2, 1, 128, 3, True), (2, 65, 260, 5, False), (3, 40, 128, 4, False),
    # the persistent form (16-byte lanes, 32 or more groups): more tiles than
    # workgroups, so each workgroup walks two to four tiles through both LDS
    # buffers; one to four slabs, a partial last slab, a lone partial slab
    # (512 workgroups), 32-frame tiles at K = 15, ragged tiles
    (6, 700, 512, 9, True), (5, 900, 256, 4, False), (9, 500, 320, 3, True),
    (4, 1000, 1024, 5, False), (17, 260, 256, 9, False), (3, 999, 516, 5, True),
    (8, 900, 512, 15, True), (12, 1000, 200, 5, True), (9, 1300, 180, 15, False),
    # the fp32 register window (fewer than 32 channel groups) over longer
    # items: many tiles per item, masked tiles past each length
    (4, 1000, 64, 9, True), (3, 700, 100, 5, False), (2, 2100, 16, 15, False),
]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("B,T,C,K,causal", GRID)
def test_grid(B, T, C, K, causal, dtype):
    x, w, b, lengths = make(B, T, C, K, dtype)
    check(x, w, b, lengths, causal, "grid")


@pytest.mark.parametrize("C", [8, 512])
def test_lengths_clamped_and_null(C):
    """Out-of-range lengths clamp to [0, T], NULL means T (C = 512: the
    persistent form)."""
    B, T, K = 4, 30, 9
    x, w, b, _ = make(B, T, C, K)
    lengths = torch.tensor([-5, 0, 31, 1000], dtype=torch.int32, device=DEV)
    y, _ = check(x, w, b, lengths, False, "out-of-range lengths")
    full = torch.full((B,), T, dtype=torch.int32, device=DEV)
    y_null = run(x, w, b, None, False)
    y_full = run(x, w, b, full, False)
    assert torch.equal(y_null, y_full)
    assert torch.equal(y[2:], y_full[2:])


def test_null_bias_equals_zero_bias_bitwise():
    x, w, _, lengths = make(3, 70, 64, 9)
    z = torch.zeros(64, device=DEV)
    assert torch.equal(run(x, w, None, lengths, True), run(x, w, z, lengths, True))


@pytest.mark.parametrize("C,T", [(32, 80), (512, 80), (64, 600)])
def test_masked_input_is_never_read(C, T):
    """NaN beyond each item's length must not reach any output (C = 512 at
    fp32: the persistent form, whose tiles past a length issue no loads;
    C = 32 and 64: the register window, short and long items)."""
    for dtype in (torch.float32, torch.bfloat16):
        B, K = 3, 9
        x, w, b, _ = make(B, T, C, K, dtype)
        lengths = torch.tensor([T, 33, 0], dtype=torch.int32, device=DEV)
        y = run(x, w, b, lengths, False)
        xp = x.clone()
        xp[1, 33:] = float("nan")
        xp[2] = float("inf")
        yp = run(xp, w, b, lengths, False)
        assert torch.equal(y, yp)


def test_guard_bands_untouched():
    B, T, C, K = 2, 37, 20, 5
    x, w, b, lengths = make(B, T, C, K)
    n, G = B * T * C, 64
    buf = torch.full((n + 2 * G,), 7.25, device=DEV)
    y = buf[G:G + n].view(B, T, C)
    run(x, w, b, lengths, True, y=y)
    assert torch.all(buf[:G] == 7.25) and torch.all(buf[G + n:] == 7.25)
    assert_parity(y, oracle.dwconv1d_fwd(x, w, b, lengths, True), TOL_F32, "guard")


@pytest.mark.parametrize("C,K", [(16, 9), (256, 9), (512, 15), (128, 5)])
def test_unaligned_pointers_take_the_narrow_path(C, K):
    """A pointer off 16-byte alignment gets one-channel lanes; at C = 256 and
    512 those still fill whole 64-lane slabs, so the LDS-staged form runs with
    one channel per lane (at C = 16 the register form does)."""
    B, T = 2, 40
    x, w, b, lengths = make(B, T, C, K)
    xs = torch.empty(x.numel() + 1, device=DEV)[1:].view(B, T, C)
    xs.copy_(x)
    ys = torch.empty(x.numel() + 1, device=DEV)[1:].view(B, T, C)
    run(xs, w, b, lengths, False, y=ys)
    assert_parity(ys, oracle.dwconv1d_fwd(x, w, b, lengths, False), TOL_F32, "unaligned")


def test_repeatable_bitwise():
    x, w, b, lengths = make(4, 200, 96, 15)
    assert torch.equal(run(x, w, b, lengths, False), run(x, w, b, lengths, False))


def test_bf16_output_rounding_is_nearest_even():
    """With a unit delta kernel the fp32 sum is exact, so the bf16 output must be
    torch's own round-to-nearest-even of x + b, tie cases included."""
    B, T, C, K = 1, 6, 8, 3
    one = 1.0
    xv = torch.tensor([one, one + 2 ** -7, one + 2 ** -6, 3.0, -one - 2 ** -7, 2.0 ** -10],
                      dtype=torch.float32)
    x = xv[None, :, None].repeat(1, 1, C).to(torch.bfloat16)
    w = torch.zeros(K, C)
    w[1] = 1.0
    b = torch.full((C,), 2.0 ** -8)  # half an ulp of 1.0: ties for the first values
    exact = x.float() + b  # exact in fp32 for these values
    expect = exact.to(torch.bfloat16)
    y = run(x.to(DEV), w.to(torch.bfloat16).to(DEV), b.to(torch.bfloat16).to(DEV), None, False)
    assert torch.equal(y.cpu().view(torch.int16), expect.view(torch.int16))


def test_encoder_shape_bf16_full():
    c = datagen.conv1d_encoder_bf16(device=DEV)
    check(c["x"], c["w"], c["b"], c["lengths"].to(DEV), False, "B=16 T=750 C=1024 K=9 bf16")


@pytest.mark.parametrize("K", [3, 4, 5, 9, 15])
def test_causal_sweep_full(K):
    c = datagen.conv1d_causal_sweep(K, device=DEV)
    check(c["x"], c["w"], c["b"], c["lengths"].to(DEV), True, f"B=32 T=1500 C=512 K={K}")


def test_causal_sweep_c200_full():
    c = datagen.conv1d_causal_sweep(9, device=DEV, C=200)
    check(c["x"], c["w"], c["b"], c["lengths"].to(DEV), True, "B=32 T=1500 C=200 K=9")
    # a zero bias passed as NULL gives the same bits
    y0 = run(c["x"], c["w"], c["b"], c["lengths"].to(DEV), True)
    y1 = run(c["x"], c["w"], None, c["lengths"].to(DEV), True)
    assert torch.equal(y0, y1)
