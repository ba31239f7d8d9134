"""Calls on several HIP streams at once.

The library keeps no state between calls, and every launch goes on the
stream it is given (the binding passes torch's current stream).  Operations
issued on two streams without synchronising between them must give, bit for
bit, what the same calls give one after another on the default stream.
"""
import pytest
import torch

import datagen
from gpu_util import say

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda", 0)


def lib():
    import conv_subsampling_amd as dw
    return dw


def workloads():
    s2 = datagen.conv2d_stage(device=DEV, B=4, T=120, F=32, C=64)
    s2["L"] = s2["lengths"].to(DEV)
    s1 = datagen.conv1d_causal_sweep(9, device=DEV, B=4, T=300, C=256)
    s1["L"] = s1["lengths"].to(DEV)
    s1["dy"] = datagen.normal((4, 300, 256), 1.0, "streams/dy1", device=DEV)
    fr = datagen.fused_front(device=DEV, B=2, T=120, F=40, C=64)
    fr["L"] = fr["lengths"].to(DEV)
    return s2, s1, fr


def run_a(dw, s2):
    y = dw.dwconv2d_fwd(s2["x"], s2["w"], s2["b"], s2["L"])
    g = dw.dwconv2d_bwd(s2["x"], s2["w"], s2["L"], s2["dy"])
    return (y,) + tuple(g)


def run_b(dw, s1, fr):
    y1 = dw.dwconv1d_fwd(s1["x"], s1["w"], s1["b"], s1["L"], causal=True)
    g1 = dw.dwconv1d_bwd(s1["x"], s1["w"], s1["L"], s1["dy"], causal=True)
    yf = dw.dwsub_fused_fwd(fr["x"], fr["w0"], fr["b0"], fr["w1"], fr["b1"], fr["L"])
    return (y1,) + tuple(g1) + (yf,)


def test_two_streams_match_the_default_stream_bitwise():
    dw = lib()
    s2, s1, fr = workloads()
    torch.cuda.synchronize()
    ref = run_a(dw, s2) + run_b(dw, s1, fr)
    torch.cuda.synchronize()

    sa, sb = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    outs = []
    for rep in range(3):
        say(f"streams: round {rep}")
        with torch.cuda.stream(sa):
            oa = run_a(dw, s2)
        with torch.cuda.stream(sb):
            ob = run_b(dw, s1, fr)
        outs.append(oa + ob)
    torch.cuda.synchronize()
    for got in outs:
        for i, (g, r) in enumerate(zip(got, ref)):
            assert torch.equal(g, r), f"output {i} differs on the side streams"
