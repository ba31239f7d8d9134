"""Guard bands around every output and workspace of every operation.

Each output is a window of a larger buffer whose elements, inside and around
the window, start as a NaN canary.  After a call (through the C ABI) the
canaries around the window must be untouched (no store lands outside its
tensor), every element inside must have been written (none still holds the
canary), and the window must match the CPU oracle.  Workspaces are given a
canary tail past the size the workspace query asks for, which must stay
untouched as well.  Shapes are ragged: partial tiles, partial channel lanes
and slabs, lengths of 0, mid-tile and the full extent.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, TOL_F32, Guarded, assert_parity, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def sync():
    torch.cuda.synchronize()


def written(g, what):
    g.check(what)
    assert g.untouched_inside() == 0, f"{what}: {g.untouched_inside()} elements never written"


def guarded_ws(nbytes):
    """A workspace of exactly nbytes followed by a 4 KiB canary tail."""
    return Guarded((max(nbytes, 1),), torch.uint8, DEV, G=4096)


CASES_1D = [
    # (B, T, C, K, causal, dtype): register window, persistent slab, partial slab, any-K loop, bf16,
    # LDS-staged slab, persistent form over several tiles
    (3, 45, 20, 5, True, torch.float32),
    (2, 77, 256, 9, True, torch.float32),
    (3, 41, 200, 9, False, torch.float32),
    (2, 30, 24, 7, False, torch.float32),
    (3, 53, 96, 9, False, torch.bfloat16),
    (2, 19, 1024, 15, True, torch.float32),
    (5, 900, 320, 4, False, torch.float32),  # persistent form, several tiles per workgroup
]


@pytest.mark.parametrize("B,T,C,K,causal,dt", CASES_1D)
def test_dwconv1d_fwd_and_bwd_guards(B, T, C, K, causal, dt):
    x = datagen.normal((B, T, C), 1.0, f"gb1/x/{B}/{T}/{C}/{K}", device=DEV).to(dt)
    w = datagen.normal((K, C), 1.0 / K, f"gb1/w/{C}/{K}", device=DEV).to(dt)
    b = datagen.normal((C,), 0.1, f"gb1/b/{C}", device=DEV).to(dt)
    dy = datagen.normal((B, T, C), 1.0, f"gb1/dy/{B}/{T}/{C}", device=DEV).to(dt)
    lens = torch.tensor([T, T // 2 + 1, 0, max(T - 17, 0), min(7, T)][:B], dtype=torch.int32)
    L = lens.to(DEV)
    tol = TOL_BF16 if dt == torch.bfloat16 else TOL_F32
    say(f"guards dwconv1d B={B} T={T} C={C} K={K} causal={causal} {dt}")
    y = Guarded((B, T, C), dt, DEV)
    lib().dwconv1d_fwd(x, w, b, L, y=y.t, causal=causal)
    sync()
    written(y, "1-D y")
    assert_parity(y.t, oracle.dwconv1d_fwd(x, w, b, lens, causal), tol, "1-D y")
    if K not in (3, 4, 5, 7, 9, 15, 31):
        return
    dx, gw, gb = Guarded((B, T, C), dt, DEV), Guarded((K, C), torch.float32, DEV), Guarded((C,), torch.float32, DEV)
    need = lib().dwconv1d_bwd_workspace_bytes(B, T, C, K)
    ws = guarded_ws(need)
    lib().dwconv1d_bwd(x, w, L, dy, dx=dx.t, dw=gw.t, db=gb.t, workspace=ws.t, causal=causal)
    sync()
    ws.check("1-D bwd workspace")
    for g, r, name in zip((dx, gw, gb), oracle.dwconv1d_bwd(x, w, lens, dy, causal), ("dx", "dw", "db")):
        written(g, f"1-D {name}")
        assert_parity(g.t, r, tol if name == "dx" else TOL_F32, f"1-D {name}")


@pytest.mark.parametrize("B,Tc,C,K,dt", [(5, 8, 1024, 9, torch.bfloat16), (3, 3, 40, 9, torch.float32),
                                          (4, 12, 256, 4, torch.float32), (2, 1, 64, 15, torch.bfloat16)])
def test_dwconv1d_stream_guards(B, Tc, C, K, dt):
    x = datagen.normal((B, Tc, C), 1.0, f"gbs/x/{B}/{Tc}/{C}", device=DEV).to(dt)
    w = datagen.normal((K, C), 1.0 / K, f"gbs/w/{C}/{K}", device=DEV).to(dt)
    b = datagen.normal((C,), 0.1, f"gbs/b/{C}", device=DEV).to(dt)
    cache = datagen.normal((B, K - 1, C), 1.0, f"gbs/c/{B}/{C}/{K}", device=DEV).to(dt)
    lens = datagen.int_uniform(B, 0, Tc, f"gbs/len/{B}/{Tc}")
    say(f"guards stream B={B} Tc={Tc} C={C} K={K} {dt} lengths={lens.tolist()}")
    y, co = Guarded((B, Tc, C), dt, DEV), Guarded((B, K - 1, C), dt, DEV)
    lib().dwconv1d_stream_fwd(x, w, b, lens.to(DEV), cache, cache_out=co.t, y=y.t)
    sync()
    ry, rc = oracle.dwconv1d_stream_fwd(x, w, b, lens, cache)
    written(y, "stream y")
    written(co, "stream cache_out")
    assert_parity(y.t, ry, TOL_BF16 if dt == torch.bfloat16 else TOL_F32, "stream y")
    assert np.array_equal(co.t.float().cpu().numpy().astype(np.float64), rc), "stream cache_out is a copy"


@pytest.mark.parametrize("causal", [False, True], ids=["symmetric", "causal"])
@pytest.mark.parametrize("B,T,F,C,dt", [(3, 37, 22, 72, torch.float32), (2, 61, 80, 256, torch.float32),
                                         (3, 29, 17, 64, torch.bfloat16)])
def test_front_guards(B, T, F, C, dt, causal):
    f = datagen.fused_front(device=DEV, B=B, T=T, F=F, C=C)
    for k in ("x", "w0", "b0", "w1", "b1"):
        f[k] = f[k].to(dt)
    lens = torch.tensor([T, T // 2 + 1, 0][:B], dtype=torch.int32)
    L = lens.to(DEV)
    T2, F2 = lib().front_out_shape(T, F, causal)
    tol = TOL_BF16 if dt == torch.bfloat16 else TOL_F32
    say(f"guards front B={B} T={T} F={F} C={C} {dt} causal={causal}")
    y = Guarded((B, T2, F2, C), dt, DEV)
    lib().dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], L, y=y.t, causal=causal)
    sync()
    written(y, "front y")
    assert_parity(y.t, oracle.dwsub_front_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], lens, causal=causal),
                  tol, "front y")
    dy = datagen.normal((B, T2, F2, C), 1.0, f"gbf/dy/{B}/{T}/{F}/{C}", device=DEV).to(dt)
    gs = [Guarded(s, torch.float32, DEV) for s in ((3, 3, C), (C,), (3, 3, C), (C,))]
    ws = guarded_ws(lib().dwsub_fused_bwd_workspace_bytes(B, T, F, C, causal))
    lib().dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], L, dy, dw0=gs[0].t, db0=gs[1].t, dw1=gs[2].t,
                          db1=gs[3].t, workspace=ws.t, causal=causal)
    sync()
    ws.check("front bwd workspace")
    ref = oracle.dwsub_front_bwd(f["x"], f["w0"], f["b0"], f["w1"], lens, dy, causal=causal)
    for g, r, name in zip(gs, ref, ("dw0", "db0", "dw1", "db1")):
        written(g, f"front {name}")
        assert_parity(g.t, r, TOL_F32, f"front {name}")


@pytest.mark.parametrize("pads", [(1, 1, 1, 1), (2, 1, 2, 1)], ids=["symmetric", "causal"])
@pytest.mark.parametrize("B,T,F,C,dt", [(3, 37, 21, 72, torch.float32), (2, 50, 64, 256, torch.float32),
                                         (3, 23, 11, 40, torch.bfloat16), (2, 31, 33, 256, torch.bfloat16)])
def test_dwconv2d_guards(B, T, F, C, dt, pads):
    To, Fo = lib().conv2d_out_shape(T, F, pads=pads)
    s = datagen.conv2d_stage(device=DEV, B=B, T=T, F=F, C=C, dy_rows_cols=(To, Fo), bf16=dt == torch.bfloat16)
    lens = torch.tensor([T, T // 2 + 1, 0][:B], dtype=torch.int32)
    L = lens.to(DEV)
    tol = TOL_BF16 if dt == torch.bfloat16 else TOL_F32
    say(f"guards dwconv2d B={B} T={T} F={F} C={C} {dt} pads={pads}")
    y = Guarded((B, To, Fo, C), dt, DEV)
    lib().dwconv2d_fwd(s["x"], s["w"], s["b"], L, y=y.t, pads=pads)
    sync()
    written(y, "2-D y")
    assert_parity(y.t, oracle.dwconv2d_fwd(s["x"], s["w"], s["b"], lens, pads=pads), tol, "2-D y")
    dx, gw, gb = Guarded((B, T, F, C), dt, DEV), Guarded((3, 3, C), torch.float32, DEV), \
        Guarded((C,), torch.float32, DEV)
    ws = guarded_ws(lib().dwconv2d_bwd_workspace_bytes(B, T, F, C, pads=pads))
    lib().dwconv2d_bwd(s["x"], s["w"], L, s["dy"], dx=dx.t, dw=gw.t, db=gb.t, workspace=ws.t, pads=pads)
    sync()
    ws.check("2-D bwd workspace")
    for g, r, name in zip((dx, gw, gb), oracle.dwconv2d_bwd(s["x"], s["w"], lens, s["dy"], pads=pads),
                          ("dx", "dw", "db")):
        written(g, f"2-D {name}")
        assert_parity(g.t, r, tol if name == "dx" else TOL_F32, f"2-D {name}")
