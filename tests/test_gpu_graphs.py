"""The entry points under HIP graph capture.

No entry point allocates, frees, synchronises or records a memset (every
clearing of memory is a kernel), so a sequence of calls with caller-given
outputs and workspaces can be captured into a graph and replayed.  Each
replay here is checked bit for bit against the same calls made eagerly, with
eager work and synchronisations between the replays.
"""
import pytest
import torch

import datagen
import oracle
from gpu_util import TOL_BF16, assert_parity, say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def test_streaming_chunks_captured_in_one_graph():
    """Four chunks of the streaming conv, the caches alternating between two
    buffers, captured as one graph: a whole streaming step in one launch."""
    dw = lib()
    B, Tc, C, K, n = 64, 8, 256, 9, 4
    st = datagen.conv1d_stream(device=DEV, B=B, Tc=Tc, C=C, K=K)
    xs = [datagen.normal((B, Tc, C), 1.0, f"graph/x{i}", device=DEV).to(torch.bfloat16) for i in range(n)]
    Ls = [torch.as_tensor(datagen.int_uniform(B, 0, Tc, f"graph/len{i}"), dtype=torch.int32).to(DEV) for i in range(n)]
    cache0 = st["cache"]
    caches = [torch.empty_like(cache0), torch.empty_like(cache0)]
    ys = [torch.empty_like(x) for x in xs]

    def step():
        cin = cache0
        for i in range(n):
            cout = caches[i % 2]
            dw.dwconv1d_stream_fwd(xs[i], st["w"], st["b"], Ls[i], cin, cache_out=cout, y=ys[i])
            cin = cout

    step()
    torch.cuda.synchronize()
    ref_y = [y.clone() for y in ys]
    ref_cache = caches[(n - 1) % 2].clone()
    # the eager chunks against the oracle, chunk by chunk
    cin = cache0
    for i in range(n):
        ry, rc = oracle.dwconv1d_stream_fwd(xs[i], st["w"], st["b"], Ls[i], cin)
        assert_parity(ref_y[i], ry, TOL_BF16, f"chunk {i}")
        cin = torch.as_tensor(rc, dtype=torch.float32).to(torch.bfloat16).to(DEV)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        caches[0].fill_(float("nan"))
        caches[1].fill_(float("nan"))
        torch.cuda.synchronize()
        say(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for i in range(n):
            assert torch.equal(ys[i], ref_y[i]), f"replay {rep} chunk {i}"
        assert torch.equal(caches[(n - 1) % 2], ref_cache), f"replay {rep} cache"


def test_conv2d_forward_and_backward_captured():
    dw = lib()
    s = datagen.conv2d_stage(device=DEV, B=4, T=90, F=32, C=64)
    L = s["lengths"].to(DEV)
    B, T, F, C = s["x"].shape
    y = torch.empty((B, (T + 1) // 2, (F + 1) // 2, C), device=DEV)
    dx = torch.empty_like(s["x"])
    dwt = torch.empty((3, 3, C), device=DEV)
    db = torch.empty((C,), device=DEV)
    ws = torch.empty((dw.dwconv2d_bwd_workspace_bytes(B, T, F, C),), dtype=torch.uint8, device=DEV)

    def step():
        dw.dwconv2d_fwd(s["x"], s["w"], s["b"], L, y=y)
        dw.dwconv2d_bwd(s["x"], s["w"], L, s["dy"], dx=dx, dw=dwt, db=db, workspace=ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (y, dx, dwt, db)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for t in (y, dx, dwt, db):
            t.fill_(float("nan"))
        ws.fill_(255)  # the workspace's contents must not matter
        torch.cuda.synchronize()
        say(f"conv2d graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for name, got, r in zip(("y", "dx", "dw", "db"), (y, dx, dwt, db), ref):
            assert torch.equal(got, r), f"replay {rep}: {name}"


def test_conv1d_forward_and_backward_captured():
    """The 1-D forward's persistent form (C = 512, K = 9 and K = 15) and the
    1-D backward, replayed from a graph, bit for bit against eager calls."""
    dw = lib()
    B, T, C = 6, 700, 512
    x = datagen.normal((B, T, C), 1.0, "graph1d/x", device=DEV)
    dy = datagen.normal((B, T, C), 1.0, "graph1d/dy", device=DEV)
    L = torch.as_tensor(datagen.int_uniform(B, 0, T, "graph1d/len"), dtype=torch.int32).to(DEV)
    w9 = datagen.normal((9, C), 1.0 / 9, "graph1d/w9", device=DEV)
    w15 = datagen.normal((15, C), 1.0 / 15, "graph1d/w15", device=DEV)
    b = datagen.normal((C,), 0.1, "graph1d/b", device=DEV)
    y9, y15, dx = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
    gw, gb = torch.empty((9, C), device=DEV), torch.empty((C,), device=DEV)
    ws = torch.empty((dw.dwconv1d_bwd_workspace_bytes(B, T, C, 9),), dtype=torch.uint8, device=DEV)

    def step():
        dw.dwconv1d_fwd(x, w9, b, L, y=y9, causal=True)
        dw.dwconv1d_fwd(x, w15, b, L, y=y15, causal=False)
        dw.dwconv1d_bwd(x, w9, L, dy, dx=dx, dw=gw, db=gb, workspace=ws, causal=True)

    step()
    torch.cuda.synchronize()
    outs = (y9, y15, dx, gw, gb)
    ref = [t.clone() for t in outs]
    assert_parity(y9, oracle.dwconv1d_fwd(x, w9, b, L, True), 1e-5, "eager y (K9)")
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            step()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        say(f"conv1d graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        for name, got, r in zip(("y K9", "y K15", "dx", "dw", "db"), outs, ref):
            assert torch.equal(got, r), f"replay {rep}: {name}"
