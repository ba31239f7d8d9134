"""The allocation-free conv2d backward (dwconv2d_bwd_noalloc, through the C
ABI) against the workspace entry point (dwconv2d_bwd_ex) on the same inputs:
the same gradients, bit for bit, on two calls in a row, the second with a
smaller input, so that what the first call left in the library's scratch
array cannot leak into the second.  No device memory is allocated by the
call."""
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, TOL_F32, assert_parity, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def case(B, T, F, C, pads, bf16, seed):
    To, Fo = lib().conv2d_out_shape(T, F, pads=pads)
    s = datagen.conv2d_stage(device=DEV, B=B, T=T, F=F, C=C, dy_rows_cols=(To, Fo), bf16=bf16, seed=seed)
    s["L"] = s["lengths"].to(DEV)
    return s


def run_pair(s, pads):
    ref = lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], pads=pads)
    dx = torch.full_like(s["x"], float("nan"))
    dw = torch.full((3, 3, s["C"]), float("nan"), device=DEV)
    db = torch.full((s["C"],), float("nan"), device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    got = lib().dwconv2d_bwd_noalloc(s["x"], s["w"], s["L"], s["dy"], dx=dx, dw=dw, db=db, pads=pads)
    assert torch.cuda.memory_allocated(DEV) == before, "the allocation-free call allocated device memory"
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("bf16", [False, True], ids=["fp32", "bf16"])
def test_noalloc_matches_workspace_entry_point_on_two_calls(bf16):
    first = case(4, 90, 64, 256, (2, 1, 2, 1), bf16, seed=11)
    second = case(2, 21, 17, 72, (1, 1, 1, 1), bf16, seed=12)
    tol = TOL_BF16 if bf16 else TOL_F32
    for name, s, pads in (("first", first, (2, 1, 2, 1)), ("second, smaller", second, (1, 1, 1, 1))):
        say(f"noalloc {name}: B={s['B']} T={s['T']} F={s['F']} C={s['C']} pads={pads} bf16={bf16}")
        ref, got = run_pair(s, pads)
        for r, g, what in zip(ref, got, ("dx", "dw", "db")):
            assert torch.equal(r, g), f"{name} call: {what} differs from the workspace entry point"
        rdx, rdw, rdb = oracle.dwconv2d_bwd(s["x"], s["w"], s["lengths"], s["dy"], pads=pads)
        assert_parity(got[0], rdx, tol, f"{name} dx")
        assert_parity(got[1], rdw, TOL_F32, f"{name} dw")
        assert_parity(got[2], rdb, TOL_F32, f"{name} db")


def test_noalloc_only_some_outputs_and_full_stage_size():
    """dw and db alone, and dx alone, at the subsampler stage's shape [32,1500,64,256]."""
    s = datagen.conv2d_stage(device=DEV)
    L = s["lengths"].to(DEV)
    say("noalloc full stage")
    ref = lib().dwconv2d_bwd(s["x"], s["w"], L, s["dy"])
    dw = torch.empty((3, 3, 256), device=DEV)
    db = torch.empty((256,), device=DEV)
    lib().dwconv2d_bwd_noalloc(s["x"], s["w"], L, s["dy"], dw=dw, db=db)
    dx = torch.empty_like(s["x"])
    lib().dwconv2d_bwd_noalloc(s["x"], s["w"], L, s["dy"], dx=dx)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], dx) and torch.equal(ref[1], dw) and torch.equal(ref[2], db)


def test_noalloc_refuses_channels_past_its_scratch():
    """1024 channels over enough row groups for all 256 workgroup partials:
    (256 + 4) * 10 * 1024 * 8 bytes is more than the 16 MiB scratch."""
    s = case(32, 600, 2, 1024, (1, 1, 1, 1), False, seed=13)
    dw = torch.empty((3, 3, 1024), device=DEV)
    with pytest.raises(lib().DwconvError, match="scratch"):
        lib().dwconv2d_bwd_noalloc(s["x"], s["w"], s["L"], s["dy"], dw=dw)
    # dx alone needs no scratch, so any C is accepted
    dx = torch.empty_like(s["x"])
    lib().dwconv2d_bwd_noalloc(s["x"], s["w"], s["L"], s["dy"], dx=dx)
    torch.cuda.synchronize()
    assert torch.equal(dx, lib().dwconv2d_bwd(s["x"], s["w"], s["L"], s["dy"], need=("dx",))[0])
