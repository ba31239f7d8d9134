"""GPU parity of dwconv2d_fwd_ex and dwconv2d_bwd_ex (through the C ABI)
against the CPU oracle: per-side padding (the causal padding among them) and
bf16 storage."""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_exact_zero, assert_parity, say, time_mask

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)
CAUSAL = (2, 1, 2, 1)


def lib():
    import conv_subsampling_amd as dw
    return dw


def sync():
    torch.cuda.synchronize()


def out_rc(T, F, pads):
    return oracle.conv_out_len(T, 3, 2, pads[0], pads[1]), oracle.conv_out_len(F, 3, 2, pads[2], pads[3])


def make(B, T, F, C, pads, bf16=False, lens=None, seed=0):
    s = datagen.conv2d_stage(device=DEV, B=B, T=T, F=F, C=C, seed=seed, dy_rows_cols=out_rc(T, F, pads), bf16=bf16)
    if lens is not None:
        s["lengths"] = torch.as_tensor(lens, dtype=torch.int32)
    s["L"] = s["lengths"].to(DEV)
    return s


def out_mask(L, To, pads):
    L = np.clip(np.asarray(L.cpu()), 0, None)
    Lo = np.array([min(oracle.conv_out_len(int(l), 3, 2, pads[0], pads[1]), To) if l > 0 else 0 for l in L])
    return np.arange(To)[None, :] >= Lo[:, None]


PADS = [CAUSAL, (2, 1, 1, 1), (1, 1, 2, 1), (1, 0, 1, 0), (2, 2, 2, 2), (1, 2, 2, 0), (2, 0, 1, 2)]
SHAPES = [
    # (B, T, F, C)
    (1, 1, 1, 4), (2, 2, 3, 3), (2, 9, 7, 4), (3, 10, 8, 8), (2, 17, 13, 1), (2, 33, 16, 64), (2, 15, 9, 100),
    (2, 12, 6, 260), (2, 21, 62, 8),
]


@pytest.mark.parametrize("pads", PADS, ids=[str(p) for p in PADS])
@pytest.mark.parametrize("B,T,F,C", SHAPES)
def test_fwd_bwd_grid_pads(B, T, F, C, pads):
    s = make(B, T, F, C, pads, lens=datagen.int_uniform(B, 0, T + 2, f"g2p/{B}/{T}/{F}/{C}/{pads}"))
    say(f"dwconv2d_ex f32 B={B} T={T} F={F} C={C} pads={pads} lengths={s['lengths'].tolist()}")
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads)
    sync()
    assert_parity(y, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads), TOL_F32, "fwd")
    assert_exact_zero(y, out_mask(s["lengths"].clamp(0, T), y.shape[1], pads)[:, :, None, None], "fwd masked rows")
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    sync()
    rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    assert_parity(dx, rdx, TOL_F32, "dx")
    assert_parity(dw, rdw, TOL_F32, "dw")
    assert_parity(db, rdb, TOL_F32, "db")
    assert_exact_zero(dx, time_mask(s["lengths"].clamp(0, T), B, T)[:, :, None, None], "dx masked rows")


@pytest.mark.parametrize("pads", [(1, 1, 1, 1), CAUSAL], ids=["symmetric", "causal"])
@pytest.mark.parametrize("B,T,F,C", [(1, 1, 1, 4), (2, 9, 7, 4), (3, 10, 8, 8), (2, 17, 13, 2), (2, 33, 16, 64),
                                     (2, 15, 9, 100), (1, 40, 64, 256), (2, 21, 62, 8), (2, 11, 30, 64)])
def test_bf16_grid(B, T, F, C, pads):
    s = make(B, T, F, C, pads, bf16=True, lens=datagen.int_uniform(B, 0, T + 2, f"g2h/{B}/{T}/{F}/{C}"))
    say(f"dwconv2d_ex bf16 B={B} T={T} F={F} C={C} pads={pads} lengths={s['lengths'].tolist()}")
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads)
    sync()
    assert y.dtype == torch.bfloat16
    assert_parity(y, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads), TOL_BF16, "bf16 fwd")
    assert_exact_zero(y, out_mask(s["lengths"].clamp(0, T), y.shape[1], pads)[:, :, None, None], "bf16 masked")
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    sync()
    assert dx.dtype == torch.bfloat16 and dw.dtype == torch.float32
    rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    assert_parity(dx, rdx, TOL_BF16, "bf16 dx")
    # the weight gradients are float32 outputs, summed in fp64 from exact products
    assert_parity(dw, rdw, TOL_F32, "bf16 dw")
    assert_parity(db, rdb, TOL_F32, "bf16 db")
    assert_exact_zero(dx, time_mask(s["lengths"].clamp(0, T), B, T)[:, :, None, None], "bf16 dx masked")


@pytest.mark.parametrize("pads", [(1, 1, 1, 1), CAUSAL], ids=["symmetric", "causal"])
def test_bf16_is_the_fp32_kernel_rounded(pads):
    """The bf16 kernels run the fp32 kernels' arithmetic on the exactly
    widened inputs: y and dx are the fp32 results rounded to nearest even,
    bit for bit.  dw and db are the same fp64 sums of exact products, added
    in another order (the bf16 backward takes two quad rows per thread and
    its own column chunks), so they agree to within one float32 ulp."""
    s = make(3, 30, 20, 64, pads, bf16=True, lens=[30, 17, 4])
    f32 = {k: s[k].float() for k in ("x", "w", "b", "dy")}
    y16 = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads)
    y32 = lib().dwconv2d_fwd(f32["x"], f32["w"], f32["b"], s["L"], pads=pads)
    g16 = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    g32 = lib().dwconv2d_bwd(f32["x"], f32["w"], s["L"], f32["dy"], pads=pads)
    sync()
    assert torch.equal(y16, y32.to(torch.bfloat16))
    assert torch.equal(g16[0], g32[0].to(torch.bfloat16))
    for a, b in ((g16[1], g32[1]), (g16[2], g32[2])):
        mag = torch.maximum(a.abs(), b.abs())
        ulp = torch.nextafter(mag, torch.full_like(mag, float("inf"))) - mag
        assert torch.all((a - b).abs() <= ulp)


def test_causal_masked_inputs_never_read_and_repeatable():
    B, T, F, C = 3, 22, 11, 20
    s = make(B, T, F, C, CAUSAL, lens=[22, 9, 0])
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=CAUSAL)
    g = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=CAUSAL)
    g2 = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=CAUSAL)
    xp, dyp = s["x"].clone(), s["dy"].clone()
    xp[1, 9:] = float("nan")
    xp[2] = float("inf")
    dyp[1, 9 // 2 + 1:] = float("nan")  # floor(9/2) + 1 = 5 valid output rows
    dyp[2] = float("nan")
    yp = lib().dwconv2d_fwd(xp, s["w"], s["b"], s["L"], pads=CAUSAL)
    gp = lib().dwconv2d_bwd(xp, s["w"], s["L"], dyp, pads=CAUSAL)
    sync()
    assert torch.equal(y, yp)
    for a, b, c in zip(g, g2, gp):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_causal_output_never_looks_ahead():
    B, T, F, C = 2, 40, 16, 32
    s = make(B, T, F, C, CAUSAL, lens=[40, 40])
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=CAUSAL)
    x2 = s["x"].clone()
    x2[:, 21:] += 1.0
    y2 = lib().dwconv2d_fwd(x2, s["w"], s["b"], s["L"], pads=CAUSAL)
    sync()
    assert torch.equal(y[:, :11], y2[:, :11])   # rows t' with 2t' <= 20
    assert not torch.equal(y[:, 11], y2[:, 11])


def test_empty_time_axis_with_output_rows():
    """T = 0 with 2 + 2 rows of padding still has one output row: it is masked."""
    s = make(2, 1, 6, 8, (2, 2, 1, 1))
    x0 = s["x"][:, :0].contiguous()
    y = lib().dwconv2d_fwd(x0, s["w"], s["b"], None, pads=(2, 2, 1, 1))
    sync()
    assert y.shape == (2, 1, 3, 8) and torch.all(y == 0)


@pytest.mark.parametrize("pads,bf16", [(CAUSAL, False), (CAUSAL, True), ((1, 1, 1, 1), True)],
                         ids=["causal-f32", "causal-bf16", "symmetric-bf16"])
def test_stage_full_size(pads, bf16):
    """The subsampler-stage workload [32,1500,64,256] as the bench times it,
    with causal padding or bf16 storage: dw and db over the whole batch, y
    and dx on every item (one oracle call per item)."""
    T, F = 1500, 64
    s = datagen.conv2d_stage(device=DEV, dy_rows_cols=out_rc(T, F, pads), bf16=bf16)
    L = s["lengths"].to(DEV)
    tol = TOL_BF16 if bf16 else TOL_F32
    say(f"dwconv2d_ex full pads={pads} bf16={bf16}: fwd")
    y = lib().dwconv2d_fwd(s["x"], s["w"], s["b"], L, pads=pads)
    say(f"dwconv2d_ex full pads={pads} bf16={bf16}: bwd")
    dx, dw, db = lib().dwconv2d_bwd(s["x"], s["w"], L, s["dy"], pads=pads)
    sync()
    assert y.shape == (32,) + out_rc(T, F, pads) + (256,)
    say("oracle")
    _, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["lengths"], s["dy"], want=("dw", "db"), pads=pads)
    assert_parity(dw, rdw, TOL_F32, "full dw")
    assert_parity(db, rdb, TOL_F32, "full db")
    B = s["x"].shape[0]
    for bi in range(B):
        say(f"item {bi}")
        xs, dys, Ls = s["x"][bi:bi + 1], s["dy"][bi:bi + 1], s["lengths"][bi:bi + 1]
        assert_parity(y[bi:bi + 1], oracle.dwconv2d_fwd(xs, s["w"], s["b"], Ls, pads=pads), tol, f"y item {bi}")
        rdx, _, _ = oracle.dwconv2d_bwd(xs, s["w"], Ls, dys, want=("dx",), pads=pads)
        assert_parity(dx[bi:bi + 1], rdx, tol, f"dx item {bi}")
    Lc = s["lengths"].clamp(0, T)
    assert_exact_zero(dx, time_mask(Lc, B, T)[:, :, None, None], "full dx masked rows")
    assert_exact_zero(y, out_mask(Lc, y.shape[1], pads)[:, :, None, None], "full y masked rows")


def _shifted(t):
    """A copy of t whose storage starts one element past an aligned address."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    out = buf[1:].view(t.shape)
    out.copy_(t)
    return out


@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
@pytest.mark.parametrize("pads", [(1, 1, 1, 1), CAUSAL], ids=["symmetric", "causal"])
def test_unaligned_pointers_take_the_narrow_path(pads, bf16):
    """Tensors that start off 16-byte alignment get one-channel lanes, with the
    same results; no alignment is ever rejected."""
    B, T, F, C = 2, 21, 18, 64
    s = make(B, T, F, C, pads, bf16=bf16, lens=[21, 9])
    say(f"dwconv2d unaligned pads={pads} bf16={bf16}")
    x, dy = _shifted(s["x"]), _shifted(s["dy"])
    To, Fo = out_rc(T, F, pads)
    y = _shifted(torch.zeros((B, To, Fo, C), dtype=x.dtype, device=DEV))
    dx = _shifted(torch.zeros_like(s["x"]))
    lib().dwconv2d_fwd(x, s["w"], s["b"], s["L"], y=y, pads=pads)
    lib().dwconv2d_bwd(x, s["w"], s["L"], dy, dx=dx, pads=pads)
    sync()
    tol = TOL_BF16 if bf16 else TOL_F32
    assert_parity(y, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], s["L"], pads=pads), tol, "unaligned fwd")
    rdx, _, _ = oracle.dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    assert_parity(dx, rdx, tol, "unaligned dx")


def _offset8(t):
    """A copy of t whose storage starts 8 bytes past a 16-byte-aligned address."""
    k = 8 // t.element_size()
    buf = torch.empty(t.numel() + k, dtype=t.dtype, device=t.device)
    out = buf[k:].view(t.shape)
    out.copy_(t)
    return out


@pytest.mark.parametrize("pads", [(1, 1, 1, 1), CAUSAL, (2, 1, 1, 1), (1, 1, 2, 1)],
                         ids=["symmetric", "causal", "causal-time", "causal-freq"])
@pytest.mark.parametrize("B,T,F,C", [(3, 30, 21, 64), (2, 25, 64, 256), (2, 19, 9, 40), (2, 14, 33, 520),
                                     (1, 1, 1, 8), (3, 3, 2, 16), (2, 2, 3, 8)])
def test_bf16_backward_paired_lanes_match_eight_byte_lanes(B, T, F, C, pads):
    """With C a multiple of 8 and 16-byte-aligned x and dx, the bf16 backward
    moves 16 bytes per lane, two lanes sharing 8 channels of two columns.  x
    and dx 8 bytes off that alignment take 8-byte lanes instead; both forms
    run the same arithmetic in the same order, so dx, dw and db agree bit for
    bit.  Shapes: partial channel blocks (C = 40, 520), odd F (the last
    column pair has one column), masked rows."""
    s = make(B, T, F, C, pads, bf16=True, lens=[T, T // 2 + 1, 0][:B])
    say(f"dwconv2d bf16 paired against 8-byte lanes B={B} T={T} F={F} C={C} pads={pads}")
    wide = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    x8 = _offset8(s["x"])
    dx8 = _offset8(torch.full_like(s["x"], float("nan")))
    dw8, db8 = lib().dwconv2d_bwd(x8, s["w"], s["L"], s["dy"], dx=dx8, pads=pads)[1:]
    sync()
    assert torch.equal(wide[0], dx8), "dx"
    assert torch.equal(wide[1], dw8) and torch.equal(wide[2], db8), "dw, db"
    rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    assert_parity(wide[0], rdx, TOL_BF16, "paired dx")
    assert_parity(wide[1], rdw, TOL_F32, "paired dw")
    assert_parity(wide[2], rdb, TOL_F32, "paired db")
