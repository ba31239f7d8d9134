"""GPU parity of dwsub_fused_fwd (through the C ABI) against the CPU oracle."""
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


def make(B, T, F, C, lens=None, seed=0):
    f = datagen.fused_front(device=DEV, B=B, T=T, F=F, C=C, seed=seed)
    if lens is not None:
        f["lengths"] = torch.as_tensor(lens, dtype=torch.int32)
    f["L"] = f["lengths"].to(DEV)
    return f


def run(f, x=None, b0="b0", b1="b1", L="L"):
    y = lib().dwsub_fused_fwd(f["x"] if x is None else x, f["w0"], f[b0] if b0 else None, f["w1"],
                              f[b1] if b1 else None, f[L] if L else None)
    torch.cuda.synchronize()
    return y


def ref(f, b0=True, b1=True, L=True):
    return oracle.dwsub_front_fwd(f["x"], f["w0"], f["b0"] if b0 else None, f["w1"], f["b1"] if b1 else None,
                                  f["lengths"] if L else None)


SHAPES = [
    # (B, T, F, C)
    (1, 1, 1, 4), (2, 5, 3, 2), (2, 16, 12, 8), (3, 13, 9, 5), (2, 37, 80, 64), (1, 64, 80, 256),
    (2, 50, 17, 300), (2, 8, 80, 1), (3, 41, 23, 33),
]


@pytest.mark.parametrize("B,T,F,C", SHAPES)
def test_grid(B, T, F, C):
    f = make(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"gs/{B}/{T}/{F}/{C}"))
    say(f"dwsub_fused_fwd B={B} T={T} F={F} C={C} lengths={f['lengths'].tolist()}")
    assert_parity(run(f), ref(f), TOL_F32, "front")
    assert_parity(run(f, b0=None, b1=None), ref(f, b0=False, b1=False), TOL_F32, "front, null biases")
    assert_parity(run(f, L=None), ref(f, L=False), TOL_F32, "front, null lengths")


def test_odd_lengths_read_one_frame_past_the_length():
    B, T, F, C = 4, 30, 16, 32
    f = make(B, T, F, C, lens=[29, 9, 1, 0])
    y = run(f)
    assert_parity(y, ref(f), TOL_F32, "odd lengths")
    # mel rows at or past 2*ceil(len/2) feed no unmasked h row: poison them
    xp = f["x"].clone()
    for bi, l in enumerate([29, 9, 1, 0]):
        xp[bi, 2 * ((l + 1) // 2):] = float("nan")
    assert torch.equal(run(f, x=xp), y)


def test_fully_masked_rows_equal_output_bias_exactly():
    B, T, F, C = 2, 60, 20, 16
    f = make(B, T, F, C, lens=[25, 60])
    y = run(f).cpu()
    L1 = (25 + 1) // 2
    b1 = f["b1"].cpu()
    for t2 in range(y.shape[1]):
        if 2 * t2 - 1 >= L1:
            assert torch.equal(y[0, t2], b1[None, :].expand(y.shape[2], C))


def test_repeatable_bitwise():
    f = make(2, 100, 80, 256)
    assert torch.equal(run(f), run(f))


def test_front_full_size():
    f = datagen.fused_front(device=DEV)
    f["L"] = f["lengths"].to(DEV)
    say("dwsub_fused_fwd full [4,1000,80] -> [4,250,20,256]")
    assert_parity(run(f), ref(f), TOL_F32, "front full")


# ------------------------------------------------------------- backward -----

def make_bwd(B, T, F, C, lens=None, seed=0):
    f = make(B, T, F, C, lens=lens, seed=seed)
    T2, F2 = lib().out_len(lib().out_len(T)), lib().out_len(lib().out_len(F))
    f["dy"] = datagen.normal((B, T2, F2, C), 1.0, f"gsb/dy/{B}/{T}/{F}/{C}/{seed}", device=DEV)
    return f


def run_bwd(f, x=None, need=("dw0", "db0", "dw1", "db1"), b0="b0", L="L", workspace=None):
    g = lib().dwsub_fused_bwd(f["x"] if x is None else x, f["w0"], f[b0] if b0 else None, f["w1"],
                              f[L] if L else None, f["dy"], need=need, workspace=workspace)
    torch.cuda.synchronize()
    return g


def ref_bwd(f, b0=True, L=True):
    return oracle.dwsub_front_bwd(f["x"], f["w0"], f["b0"] if b0 else None, f["w1"],
                                  f["lengths"] if L else None, f["dy"])


def check_bwd(got, ref, what):
    for name, g, r in zip(("dw0", "db0", "dw1", "db1"), got, ref):
        assert_parity(g, r, TOL_F32, f"{what} {name}")


@pytest.mark.parametrize("B,T,F,C", SHAPES)
def test_bwd_grid(B, T, F, C):
    f = make_bwd(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"gsb/{B}/{T}/{F}/{C}"))
    say(f"dwsub_fused_bwd B={B} T={T} F={F} C={C} lengths={f['lengths'].tolist()}")
    check_bwd(run_bwd(f), ref_bwd(f), "front bwd")
    check_bwd(run_bwd(f, b0=None, L=None), ref_bwd(f, b0=False, L=False), "front bwd, null b0 and lengths")


def test_bwd_subsets_repeatable_and_masked_rows_never_read():
    B, T, F, C = 3, 40, 24, 64
    f = make_bwd(B, T, F, C, lens=[40, 13, 0])
    full = run_bwd(f)
    again = run_bwd(f)
    for a, b in zip(full, again):
        assert torch.equal(a, b)
    only = run_bwd(f, need=("dw1",))
    assert only[0] is None and only[1] is None and only[3] is None and torch.equal(only[2], full[2])
    xp = f["x"].clone()
    xp[1, 14:] = float("nan")  # ceil(13/2) = 7 unmasked h rows read mel rows < 14
    xp[2] = float("nan")
    for a, b in zip(full, run_bwd(f, x=xp)):
        assert torch.equal(a, b)


def test_bwd_short_workspace_raises_and_empty_batch_is_zero():
    f = make_bwd(2, 16, 12, 8)
    need = lib().dwsub_fused_bwd_workspace_bytes(2, 16, 12, 8)
    with pytest.raises(lib().DwconvError, match="workspace"):
        run_bwd(f, workspace=torch.empty(need - 8, dtype=torch.uint8, device=DEV))
    outs = [torch.full(s, 3.0, device=DEV) for s in ((3, 3, 8), (8,), (3, 3, 8), (8,))]
    lib().dwsub_fused_bwd(f["x"][:0], f["w0"], f["b0"], f["w1"], f["L"][:0], f["dy"][:0], *outs)
    torch.cuda.synchronize()
    assert all(torch.all(o == 0) for o in outs)


def test_bwd_front_full_size():
    f = datagen.fused_front(device=DEV)
    f["L"] = f["lengths"].to(DEV)
    f["dy"] = datagen.normal((4, 250, 20, 256), 1.0, "c2/dy", device=DEV)
    say("dwsub_fused_bwd full [4,1000,80], dy [4,250,20,256]")
    check_bwd(run_bwd(f), ref_bwd(f), "front bwd full")


# ----------------------------------------------------------- causal mode -----

def front_dims_oracle(T, F, causal):
    pl, ph = oracle.front_pads(causal)
    T1, F1 = oracle.conv_out_len(T, 3, 2, pl, ph), oracle.conv_out_len(F, 3, 2, pl, ph)
    return oracle.conv_out_len(T1, 3, 2, pl, ph), oracle.conv_out_len(F1, 3, 2, pl, ph)


CAUSAL_SHAPES = SHAPES + [(2, 2, 3, 8), (3, 6, 5, 7), (2, 0, 4, 4), (1, 5, 0, 4)]


@pytest.mark.parametrize("B,T,F,C", CAUSAL_SHAPES)
def test_causal_grid_fwd_bwd(B, T, F, C):
    f = make(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"gsc/{B}/{T}/{F}/{C}"))
    T2, F2 = front_dims_oracle(T, F, True)
    f["dy"] = datagen.normal((B, T2, F2, C), 1.0, f"gsc/dy/{B}/{T}/{F}/{C}", device=DEV)
    say(f"dwsub_fused causal B={B} T={T} F={F} C={C} lengths={f['lengths'].tolist()}")
    y = lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    torch.cuda.synchronize()
    assert y.shape == (B, T2, F2, C)
    ref = oracle.dwsub_front_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["lengths"], causal=True)
    assert_parity(y, ref, TOL_F32, "causal front")
    got = lib().dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], f["L"], f["dy"], causal=True)
    torch.cuda.synchronize()
    check_bwd(got, oracle.dwsub_front_bwd(f["x"], f["w0"], f["b0"], f["w1"], f["lengths"], f["dy"], causal=True),
              "causal front bwd")


def test_causal_masked_mel_rows_never_read_and_empty_item_is_bias():
    B, T, F, C = 3, 40, 24, 64
    f = make(B, T, F, C, lens=[40, 13, 0])
    T2, F2 = front_dims_oracle(T, F, True)
    f["dy"] = datagen.normal((B, T2, F2, C), 1.0, "gsc/dy/poison", device=DEV)
    y = lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    g = lib().dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], f["L"], f["dy"], causal=True)
    xp = f["x"].clone()
    # L1 = floor(13/2) + 1 = 7 unmasked h rows; h row 6 reads mel rows 10, 11, 12
    xp[1, 13:] = float("nan")
    xp[2] = float("nan")
    yp = lib().dwsub_fused_fwd(xp, f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    gp = lib().dwsub_fused_bwd(xp, f["w0"], f["b0"], f["w1"], f["L"], f["dy"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(y, yp)
    for a, b in zip(g, gp):
        assert torch.equal(a, b)
    assert torch.equal(y[2], f["b1"][None, None, :].expand(T2, F2, C))


def test_causal_output_never_looks_ahead():
    B, T, F, C = 2, 64, 20, 32
    f = make(B, T, F, C, lens=[64, 64])
    y = lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    x2 = f["x"].clone()
    x2[:, 4 * 7 + 1:] += 2.0   # output row t2 reads mel rows up to 4 t2
    y2 = lib().dwsub_fused_fwd(x2, f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :8], y2[:, :8]) and not torch.equal(y[:, 8], y2[:, 8])


def test_causal_front_full_size():
    f = datagen.fused_front(device=DEV)
    f["L"] = f["lengths"].to(DEV)
    T2, F2 = front_dims_oracle(1000, 80, True)
    assert (T2, F2) == (251, 21)
    f["dy"] = datagen.normal((4, T2, F2, 256), 1.0, "c2/dy", device=DEV)
    say("dwsub_fused causal full [4,1000,80] -> [4,251,21,256]")
    y = lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["L"], causal=True)
    got = lib().dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], f["L"], f["dy"], causal=True)
    torch.cuda.synchronize()
    assert_parity(y, oracle.dwsub_front_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], f["lengths"], causal=True),
                  TOL_F32, "causal front full")
    check_bwd(got, oracle.dwsub_front_bwd(f["x"], f["w0"], f["b0"], f["w1"], f["lengths"], f["dy"], causal=True),
              "causal front bwd full")


# ----------------------------------------------------------- bf16 storage -----

def to_bf16(f, keys=("x", "w0", "b0", "w1", "b1", "dy")):
    return dict(f, **{k: f[k].to(torch.bfloat16) for k in keys if k in f})


@pytest.mark.parametrize("causal", [False, True], ids=["symmetric", "causal"])
@pytest.mark.parametrize("B,T,F,C", [(1, 1, 1, 4), (2, 16, 12, 8), (3, 13, 9, 5), (2, 37, 80, 64), (2, 50, 17, 300)])
def test_bf16_grid_fwd_bwd(B, T, F, C, causal):
    f = make(B, T, F, C, lens=datagen.int_uniform(B, 0, T + 2, f"gsh/{B}/{T}/{F}/{C}"))
    T2, F2 = front_dims_oracle(T, F, causal)
    f["dy"] = datagen.normal((B, T2, F2, C), 1.0, f"gsh/dy/{B}/{T}/{F}/{C}", device=DEV)
    h = to_bf16(f)
    say(f"dwsub_fused bf16 causal={causal} B={B} T={T} F={F} C={C}")
    y = lib().dwsub_fused_fwd(h["x"], h["w0"], h["b0"], h["w1"], h["b1"], h["L"], causal=causal)
    got = lib().dwsub_fused_bwd(h["x"], h["w0"], h["b0"], h["w1"], h["L"], h["dy"], causal=causal)
    torch.cuda.synchronize()
    assert y.dtype == torch.bfloat16 and got[0].dtype == torch.float32
    ref = oracle.dwsub_front_fwd(h["x"], h["w0"], h["b0"], h["w1"], h["b1"], h["lengths"], causal=causal)
    assert_parity(y, ref, 2e-2, "bf16 front")
    check_bwd(got, oracle.dwsub_front_bwd(h["x"], h["w0"], h["b0"], h["w1"], h["lengths"], h["dy"], causal=causal),
              "bf16 front bwd")


@pytest.mark.parametrize("causal", [False, True], ids=["symmetric", "causal"])
def test_bf16_is_the_fp32_kernel_rounded(causal):
    f = make(3, 64, 40, 128, lens=[64, 29, 1])
    T2, F2 = front_dims_oracle(64, 40, causal)
    f["dy"] = datagen.normal((3, T2, F2, 128), 1.0, "gsh/dy/bitwise", device=DEV)
    h = to_bf16(f)
    w = {k: h[k].float() for k in ("x", "w0", "b0", "w1", "b1", "dy")}
    y16 = lib().dwsub_fused_fwd(h["x"], h["w0"], h["b0"], h["w1"], h["b1"], h["L"], causal=causal)
    y32 = lib().dwsub_fused_fwd(w["x"], w["w0"], w["b0"], w["w1"], w["b1"], h["L"], causal=causal)
    g16 = lib().dwsub_fused_bwd(h["x"], h["w0"], h["b0"], h["w1"], h["L"], h["dy"], causal=causal)
    g32 = lib().dwsub_fused_bwd(w["x"], w["w0"], w["b0"], w["w1"], h["L"], w["dy"], causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(y16, y32.to(torch.bfloat16))
    for a, b in zip(g16, g32):
        assert torch.equal(a, b)


def test_bf16_front_full_size():
    f = datagen.fused_front(device=DEV)
    f["L"] = f["lengths"].to(DEV)
    f["dy"] = datagen.normal((4, 250, 20, 256), 1.0, "c2/dy", device=DEV)
    h = to_bf16(f)
    say("dwsub_fused bf16 full [4,1000,80]")
    y = lib().dwsub_fused_fwd(h["x"], h["w0"], h["b0"], h["w1"], h["b1"], h["L"])
    got = lib().dwsub_fused_bwd(h["x"], h["w0"], h["b0"], h["w1"], h["L"], h["dy"])
    torch.cuda.synchronize()
    assert_parity(y, oracle.dwsub_front_fwd(h["x"], h["w0"], h["b0"], h["w1"], h["b1"], h["lengths"]), 2e-2,
                  "bf16 front full")
    check_bwd(got, oracle.dwsub_front_bwd(h["x"], h["w0"], h["b0"], h["w1"], h["lengths"], h["dy"]), "bf16 bwd full")
