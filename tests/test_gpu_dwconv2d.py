"""GPU parity of dwconv2d_fwd and dwconv2d_bwd (through the C ABI) against the CPU oracle."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_F32, assert_exact_zero, assert_parity, say, time_mask

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def sync():
    torch.cuda.synchronize()


def make(B, T, F, C, seed=0, lens=None):
    s = datagen.conv2d_stage(device=DEV, B=B, T=T, F=F, C=C, seed=seed)
    if lens is not None:
        s["lengths"] = torch.as_tensor(lens, dtype=torch.int32)
    s["L"] = s["lengths"].to(DEV)
    return s


SHAPES = [
    # (B, T, F, C)
    (1, 1, 1, 4), (2, 2, 2, 3), (2, 9, 7, 4), (3, 10, 8, 8), (2, 17, 13, 1), (2, 33, 16, 64),
    (1, 40, 64, 256), (2, 15, 9, 100), (2, 12, 6, 260), (3, 25, 32, 12),
    # column chunks with a shorter last chunk (31 and 23 quad / output columns)
    (2, 21, 62, 8), (2, 14, 46, 260),
]


def out_mask(L, B, To):
    Lo = (np.clip(np.asarray(L.cpu()), 0, None) + 1) // 2
    return np.arange(To)[None, :] >= Lo[:, None]


@pytest.mark.parametrize("B,T,F,C", SHAPES)
def test_fwd_grid(B, T, F, C):
    s = make(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"g2/{B}/{T}/{F}/{C}"))
    say(f"dwconv2d_fwd B={B} T={T} F={F} C={C} lengths={s['lengths'].tolist()}")
    for bias in (s["b"], None):
        y = lib().dwconv2d_fwd(s["x"], s["w"], bias, s["L"])
        sync()
        ref = oracle.dwconv2d_fwd(s["x"], s["w"], bias, s["L"])
        assert_parity(y, ref, TOL_F32, "fwd")
        To = (T + 1) // 2
        Lc = s["lengths"].clamp(0, T)
        assert_exact_zero(y, out_mask(Lc, B, To)[:, :, None, None], "fwd masked rows")


def test_fwd_null_lengths_and_masked_input_never_read():
    s = make(3, 21, 10, 16, lens=[21, 8, 0])
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"])
    xp = s["x"].clone()
    xp[1, 8:] = float("nan")
    xp[2] = float("nan")
    yp = lib().dwconv2d_fwd(xp, s["w"], s["b"], s["L"])
    y_null = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], None)
    sync()
    assert torch.equal(y, yp)
    assert torch.equal(y_null[0], y[0])
    assert_parity(y_null, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], None), TOL_F32, "null lengths")


def test_fwd_unsupported_geometry_raises():
    s = make(1, 8, 8, 4)
    with pytest.raises(lib().DwconvError, match="stride"):
        lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], stride=1)


@pytest.mark.parametrize("B,T,F,C", SHAPES)
def test_bwd_grid(B, T, F, C):
    s = make(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"g2b/{B}/{T}/{F}/{C}"))
    say(f"dwconv2d_bwd B={B} T={T} F={F} C={C} lengths={s['lengths'].tolist()}")
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"])
    sync()
    rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"])
    assert_parity(dx, rdx, TOL_F32, "dx")
    assert_parity(dw, rdw, TOL_F32, "dw")
    assert_parity(db, rdb, TOL_F32, "db")
    Lc = s["lengths"].clamp(0, T)
    assert_exact_zero(dx, time_mask(Lc, B, T)[:, :, None, None], "dx masked rows")


def test_bwd_subsets_and_masked_inputs_never_read():
    B, T, F, C = 3, 22, 11, 20
    s = make(B, T, F, C, lens=[22, 9, 0])
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"])
    xp, dyp = s["x"].clone(), s["dy"].clone()
    xp[1, 9:] = float("nan")
    xp[2] = float("inf")
    dyp[1, 5:] = float("nan")  # ceil(9/2) = 5 valid output rows
    dyp[2] = float("nan")
    dx2, dw2, db2 = lib().dwconv2d_bwd(xp, s["w"], s["L"], dyp)
    only_dx = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], need=("dx",))
    only_dw = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], need=("dw",))
    only_db = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], need=("db",))
    sync()
    assert torch.equal(dx, dx2) and torch.equal(dw, dw2) and torch.equal(db, db2)
    assert only_dx[1] is None and only_dx[2] is None and torch.equal(only_dx[0], dx)
    assert only_dw[0] is None and torch.equal(only_dw[1], dw)
    assert only_db[0] is None and torch.equal(only_db[2], db)


def test_bwd_short_workspace_raises():
    s = make(2, 10, 8, 8)
    need = lib().dwconv2d_bwd_workspace_bytes(2, 10, 8, 8)
    ws = torch.empty(need - 4, dtype=torch.uint8, device=DEV)
    with pytest.raises(lib().DwconvError, match="workspace"):
        lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], workspace=ws)


def test_bwd_empty_batch_gives_zero_gradients():
    s = make(2, 10, 8, 8)
    x0, dy0 = s["x"][:0], s["dy"][:0]
    dw = torch.full((3, 3, 8), 5.0, device=DEV)
    db = torch.full((8,), 5.0, device=DEV)
    lib().dwconv2d_bwd(x0, s["w"], s["L"][:0], dy0, dw=dw, db=db, need=("dw", "db"))
    sync()
    assert torch.all(dw == 0) and torch.all(db == 0)


def test_bwd_repeatable_bitwise():
    s = make(4, 64, 32, 64)
    a = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"])
    b = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"])
    sync()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_stage_full_size_fwd_and_bwd():
    """The full subsampler-stage workload [32,1500,64,256]: dw and db over the whole
    batch, y and dx on every item (one oracle call per item, which the oracle
    computes independently of the others)."""
    s = datagen.conv2d_stage(device=DEV)
    L = s["lengths"].to(DEV)
    say("dwconv2d full: fwd")
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], L)
    say("dwconv2d full: bwd")
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], L, s["dy"])
    sync()
    say("dwconv2d full: oracle")
    _, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["lengths"], s["dy"], want=("dw", "db"))
    assert_parity(dw, rdw, TOL_F32, "full dw")
    assert_parity(db, rdb, TOL_F32, "full db")
    B, T = s["x"].shape[:2]
    for bi in range(B):
        say(f"dwconv2d full: item {bi}")
        xs, dys, Ls = s["x"][bi:bi + 1], s["dy"][bi:bi + 1], s["lengths"][bi:bi + 1]
        assert_parity(y[bi:bi + 1], oracle.dwconv2d_fwd(xs, s["w"], s["b"], Ls), TOL_F32, f"full y item {bi}")
        rdx, _, _ = oracle.dwconv2d_bwd(xs, s["w"], Ls, dys, want=("dx",))
        assert_parity(dx[bi:bi + 1], rdx, TOL_F32, f"full dx item {bi}")
    Lc = s["lengths"].clamp(0, T)
    assert_exact_zero(dx, time_mask(Lc, B, T)[:, :, None, None], "full dx masked rows")
    assert_exact_zero(y, out_mask(Lc, B, (T + 1) // 2)[:, :, None, None], "full y masked rows")


def test_third_stage_full_size_fwd_and_bwd():
    """8x subsampling's third stride-2 stage: the 4x front output of a 15 s
    batch, [32,375,20,256] -> [32,188,10,256], lengths ~U[T/2, T] in the
    stage's own frames; whole-batch parity."""
    s = datagen.conv2d_stage(device=DEV, B=32, T=375, F=20, C=256)
    L = s["lengths"].to(DEV)
    say("dwconv2d third stage [32,375,20,256]")
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], L)
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], L, s["dy"])
    sync()
    assert y.shape == (32, 188, 10, 256)
    assert_parity(y, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], s["lengths"]), TOL_F32, "stage3 y")
    rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["lengths"], s["dy"])
    assert_parity(dx, rdx, TOL_F32, "stage3 dx")
    assert_parity(dw, rdw, TOL_F32, "stage3 dw")
    assert_parity(db, rdb, TOL_F32, "stage3 db")


def test_front_then_third_stage_lengths_compose():
    """The front (4x) followed by a third depthwise stage (8x), each masking
    with its own frame lengths: ceil(len/2), then ceil again per stage."""
    f = datagen.fused_front(device=DEV, B=3, T=96, F=40, C=32)
    f["lengths"] = torch.tensor([96, 37, 0], dtype=torch.int32)
    L = f["lengths"].to(DEV)
    h = lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], L)
    L2 = (((f["lengths"] + 1) // 2) + 1) // 2          # the front's output frames
    w3 = datagen.normal((3, 3, 32), 1.0 / 9, "t3/w", device=DEV)
    b3 = datagen.normal((32,), 0.1, "t3/b", device=DEV)
    y = lib().dwconv2d_fwd(h, w3, b3, L2.to(DEV))
    sync()
    ref_h = oracle.dwsub_front_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["lengths"])
    ref = oracle.dwconv2d_fwd(np.asarray(h.cpu()), w3, b3, L2)
    assert_parity(h, ref_h, TOL_F32, "front")
    assert_parity(y, ref, TOL_F32, "third stage")
    assert y.shape == (3, 12, 5, 32)
    assert torch.all(y[2] == 0) and torch.all(y[1, 5:] == 0)   # ceil(ceil(ceil(37/2)/2)/2) = 5
