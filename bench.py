#!/usr/bin/env python3
"""Throughput of the depthwise-convolution path on one MI355X.

One step runs every operation of the path once, each at its workload's full
size, on synthetic inputs resident in HBM:

  front   dwsub_fused_fwd   mel [4,1000,80] -> [4,250,20,256]           fp32
          dwsub_fused_bwd   dw0, db0, dw1, db1 of the same, dy given     fp64 sums
          dwsub_fused_*_ex  the same two in causal mode -> [4,251,21,256]
  conv1d  dwconv1d_fwd      [16,750,1024] K=9 symmetric                 bf16 storage
  sweep   dwconv1d_fwd      [32,1500,512] causal, K = 3, 4, 5, 9, 15    fp32
          dwconv1d_fwd      [32,1500,200] causal, K = 9                 fp32
  stream  dwconv1d_stream_fwd  1024 streams x 8-frame chunks, C 1024, K 9, cache  bf16
          dwconv1d_bwd      dx, dw, db of [32,1500,512] causal K = 9    fp32, fp64 sums
  stage   dwconv2d_fwd      [32,1500,64,256] -> [32,750,32,256]         fp32
          dwconv2d_bwd      dx, dw, db of the same                      fp32
          dwconv2d_fwd_ex   the same with causal padding -> [32,751,33,256]  fp32
          dwconv2d_bwd_ex   its dx, dw, db                              fp32
          dwconv2d_fwd_ex   the symmetric stage with bf16 storage       bf16
          dwconv2d_bwd_ex   its dx, dw, db (dw, db in fp32)             bf16
  stage3  dwconv2d_fwd/bwd  [32,375,20,256] -> [32,188,10,256] (8x)     fp32

The timed region is exactly --steps steps, bracketed by device
synchronisation.  Per-operation times come from HIP events recorded on the
stream the kernels run on.  The working set (about 10 GB) is far larger than
the 256 MB Infinity Cache, and the stage rows stream several GB between
consecutive uses of any other row's inputs, so every row reads cold data.

Prints one JSON line on stdout (progress goes to stderr):
  value        frames per second over the whole step (sum over operations of
               the input frames B*T each processes, divided by step time)
  hbm          algorithmic bytes per step / step time, and its fraction of
               the 8 TB/s HBM peak
  roofline     the dominant kernel's achieved algorithmic GB/s against 8 TB/s
  rows         the same figures for every operation (mean time per call, and
               its median, minimum and 90th percentile over the steps)
  cpu_baseline the CPU oracle on a bounded sample of the same workload

`python bench.py --summarize-profile DIR` turns rocprofv3 output under DIR
into the text summaries kept in profiles/.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E peak
VALU_F32_PEAK_TFLOPS = 78.6       # 256 CU x 4 SIMD x 16 lanes x 2 flop (FMA) x 2.4 GHz, unpacked fp32
DOMINANT_ROW = "stage_bwd"         # the row with the largest share of the step
DOMINANT_KERNEL = "dwconv2d_bwd_kernel"
DOMINANT_SOURCES = ["conv_subsampling_amd/csrc/dwconv2d.hip", "conv_subsampling_amd/csrc/common.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "dwconv2d_bwd_stage_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# Algorithmic work per call: valid input rows, every output element, the
# parameters and the lengths.  Masked input frames are never needed.
# --------------------------------------------------------------------------

# Each row's main kernel, as rocprofv3 names it (a prefix of the demangled
# name, through the opening parenthesis), in the order build_rows adds the
# rows.  A step launches the rows in this order, so the k-th dispatch of a
# name within a step belongs to the k-th row listing it; the profile
# summaries attribute dispatches to rows that way.
ROW_KERNELS = [
    ("front", "dw::dwsub_fused_fwd_kernel<float>("),
    ("front_bwd", "dw::dwsub_fused_bwd_kernel<float, 4>("),
    ("front_causal", "dw::dwsub_fused_fwd_kernel<float>("),
    ("front_bwd_causal", "dw::dwsub_fused_bwd_kernel<float, 5>("),
    ("conv1d_bf16", "dw::dwconv1d_fwd_kernel<unsigned short, 4, 9, 12>("),
    ("conv1d_causal_K3_C512", "dw::dwconv1d_fwd_lds_kernel<float, 4, 3, 32>("),
    ("conv1d_causal_K4_C512", "dw::dwconv1d_fwd_lds_kernel<float, 4, 4, 32>("),
    ("conv1d_causal_K5_C512", "dw::dwconv1d_fwd_lds_kernel<float, 4, 5, 32>("),
    ("conv1d_causal_K9_C512", "dw::dwconv1d_fwd_lds_kernel<float, 4, 9, 32>("),
    ("conv1d_causal_K15_C512", "dw::dwconv1d_fwd_lds_kernel<float, 4, 15, 32>("),
    ("conv1d_causal_K9_C200", "dw::dwconv1d_fwd_lds_kernel<float, 4, 9, 32>("),
    ("conv1d_stream_bf16", "dw::dwconv1d_stream_kernel<unsigned short, 8, 9, 8>("),
    ("conv1d_bwd_K9_C512", "dw::dwconv1d_bwd_kernel<float, 4, 9, true, 8>("),
    ("stage_fwd", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage_bwd", "dw::dwconv2d_bwd_kernel<float, 4, 1, 0, 0>("),
    ("stage_fwd_causal", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage_bwd_causal", "dw::dwconv2d_bwd_kernel<float, 4, 1, 1, 1>("),
    ("stage_fwd_bf16", "dw::dwconv2d_fwd_kernel<unsigned short, 8, 1, 32>("),
    ("stage_bwd_bf16", "dw::dwconv2d_bwd_kernel<unsigned short, 4, 2, 0, 0>("),
    ("stage3_fwd", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage3_bwd", "dw::dwconv2d_bwd_kernel<float, 4, 1, 0, 0>("),
]


def clamp_lengths(L, T):
    return [min(max(int(v), 0), T) for v in L]


# Each work_* function returns (algorithmic read bytes, write bytes, flops,
# dense read bytes): the last reads every frame, masked or not.

def work_conv1d(c, es):
    B, T, C, K = c["B"], c["T"], c["C"], c["K"]
    L = clamp_lengths(c["lengths"].tolist(), T)
    rd = lambda L: sum(L) * C * es + (K * C + C) * es + 4 * B
    wr = B * T * C * es
    flops = 2 * K * C * sum(L)
    return rd(L), wr, flops, rd([T] * B)


def work_conv1d_stream(c, es):
    B, Tc, C, K = c["B"], c["Tc"], c["C"], c["K"]
    L = clamp_lengths(c["lengths"].tolist(), Tc)
    rd = lambda L: sum(L) * C * es + B * (K - 1) * C * es + (K + 1) * C * es + 4 * B  # chunk, cache, w, b, lengths
    wr = B * Tc * C * es + B * (K - 1) * C * es                                       # y and the new cache
    flops = 2 * K * C * sum(L)
    return rd(L), wr, flops, rd([Tc] * B)


def work_conv1d_bwd(c):
    B, T, C, K = c["B"], c["T"], c["C"], c["K"]
    L = clamp_lengths(c["lengths"].tolist(), T)
    rd = lambda L: 2 * sum(L) * C * 4 + K * C * 4 + 4 * B   # x and dy at unmasked frames, w, lengths
    wr = B * T * C * 4 + (K + 1) * C * 4                     # dx (zeros past the length), dw, db
    flops = 2 * K * C * sum(L) * 2 + C * sum(L)
    return rd(L), wr, flops, rd([T] * B)


def front_half(n, d):
    return (n - 1 + d) // 2 + 1 if n > 0 else d


def work_front(c, d=0):
    B, T, F, C = c["B"], c["T"], c["F"], c["C"]
    T1, F1 = front_half(T, d), front_half(F, d)
    T2, F2 = front_half(T1, d), front_half(F1, d)
    L = clamp_lengths(c["lengths"].tolist(), T)
    L1 = [min(front_half(l, d), T1) if l > 0 else 0 for l in L]
    rows_read = sum(min(T, 2 * l1) for l1 in L1)  # mel rows some unmasked h row reads
    rd = rows_read * F * 4 + 20 * C * 4 + 4 * B
    wr = B * T2 * F2 * C * 4
    flops = 2 * 9 * C * F1 * sum(min(l1, T1) for l1 in L1) + 2 * 9 * B * T2 * F2 * C
    return rd, wr, flops, B * T * F * 4 + 20 * C * 4 + 4 * B


def work_front_bwd(c, d=0):
    B, T, F, C = c["B"], c["T"], c["F"], c["C"]
    T1, F1 = front_half(T, d), front_half(F, d)
    T2, F2 = front_half(T1, d), front_half(F1, d)
    L = clamp_lengths(c["lengths"].tolist(), T)
    L1 = [min(front_half(l, d), T1) if l > 0 else 0 for l in L]
    rows_read = sum(min(T, 2 * l1) for l1 in L1)
    rd = rows_read * F * 4 + B * T2 * F2 * C * 4 + 19 * C * 4 + 4 * B
    wr = 20 * C * 4
    hpos = sum(L1) * F1 * C                       # unmasked h positions
    flops = hpos * (18 + 18 + 1) + B * T2 * F2 * C * (18 + 18 + 1)
    return rd, wr, flops, B * T * F * 4 + B * T2 * F2 * C * 4 + 19 * C * 4 + 4 * B


def stage_out(n, pl, ph):
    return max(0, (n + pl + ph - 3) // 2 + 1)


def work_stage_fwd(c, pads=(1, 1, 1, 1), es=4):
    B, T, F, C = c["B"], c["T"], c["F"], c["C"]
    To, Fo = stage_out(T, pads[0], pads[1]), stage_out(F, pads[2], pads[3])
    L = clamp_lengths(c["lengths"].tolist(), T)
    Lo = [min(stage_out(l, pads[0], pads[1]), To) if l > 0 else 0 for l in L]
    rd = lambda L: sum(L) * F * C * es + 10 * C * es + 4 * B
    wr = B * To * Fo * C * es
    flops = 2 * 9 * C * Fo * sum(Lo)
    return rd(L), wr, flops, rd([T] * B)


def work_stage_bwd(c, pads=(1, 1, 1, 1), es=4):
    B, T, F, C = c["B"], c["T"], c["F"], c["C"]
    To, Fo = stage_out(T, pads[0], pads[1]), stage_out(F, pads[2], pads[3])
    L = clamp_lengths(c["lengths"].tolist(), T)
    Lo = [min(stage_out(l, pads[0], pads[1]), To) if l > 0 else 0 for l in L]
    rd = sum(L) * F * C * es + sum(Lo) * Fo * C * es + 9 * C * es + 4 * B
    wr = B * T * F * C * es + 10 * C * 4
    flops = 2 * 2 * 9 * C * Fo * sum(Lo) + C * Fo * sum(Lo)
    return rd, wr, flops, B * T * F * C * es + B * To * Fo * C * es + 9 * C * es + 4 * B


# --------------------------------------------------------------------------

def build_rows(dev):
    import torch

    import conv_subsampling_amd as dw
    import datagen

    rows = []

    def add(name, op, cfg, frames, rd, wr, flops, rd_dense, fn, bound="hbm"):
        rows.append(dict(name=name, op=op, cfg=cfg, frames=frames, read=rd, write=wr, flops=flops,
                         read_dense=rd_dense, fn=fn, bound=bound))

    f = datagen.fused_front(device=dev)
    fL = f["lengths"].to(dev)
    fy = torch.empty((f["B"], 250, 20, f["C"]), device=dev)
    add("front", "dwsub_fused_fwd", "mel [4,1000,80] -> [4,250,20,256] fp32", f["B"] * f["T"], *work_front(f),
        lambda: dw.dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], fL, y=fy), bound="alu")

    fdy = datagen.normal((f["B"], 250, 20, f["C"]), 1.0, "c2/dy", device=dev)
    fg = [torch.empty(sh, device=dev) for sh in ((3, 3, f["C"]), (f["C"],), (3, 3, f["C"]), (f["C"],))]
    fws = torch.empty((dw.dwsub_fused_bwd_workspace_bytes(f["B"], f["T"], f["F"], f["C"]),), dtype=torch.uint8,
                      device=dev)
    add("front_bwd", "dwsub_fused_bwd", "dw0,db0,dw1,db1 of the front, dy [4,250,20,256] fp64 accumulation",
        f["B"] * f["T"], *work_front_bwd(f),
        lambda: dw.dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], fL, fdy, *fg, workspace=fws), bound="alu")
    f["dy"] = fdy
    fcy = torch.empty((f["B"], 251, 21, f["C"]), device=dev)
    fcdy = datagen.normal((f["B"], 251, 21, f["C"]), 1.0, "c2/dy", device=dev)
    fcws = torch.empty((dw.dwsub_fused_bwd_workspace_bytes(f["B"], f["T"], f["F"], f["C"], causal=True),),
                       dtype=torch.uint8, device=dev)
    add("front_causal", "dwsub_fused_fwd_ex", "mel [4,1000,80] -> [4,251,21,256] causal fp32", f["B"] * f["T"],
        *work_front(f, 1),
        lambda: dw.dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], fL, y=fcy, causal=True), bound="alu")
    add("front_bwd_causal", "dwsub_fused_bwd_ex", "dw0,db0,dw1,db1 of the causal front, dy [4,251,21,256]",
        f["B"] * f["T"], *work_front_bwd(f, 1),
        lambda: dw.dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], fL, fcdy, *fg, workspace=fcws, causal=True),
        bound="alu")
    f["dy_causal"] = fcdy

    e = datagen.conv1d_encoder_bf16(device=dev)
    eL = e["lengths"].to(dev)
    ey = torch.empty_like(e["x"])
    add("conv1d_bf16", "dwconv1d_fwd", "[16,750,1024] K9 symmetric bf16", e["B"] * e["T"], *work_conv1d(e, 2),
        lambda: dw.dwconv1d_fwd(e["x"], e["w"], e["b"], eL, y=ey, causal=False))

    sweep = []
    for K, C in [(3, 512), (4, 512), (5, 512), (9, 512), (15, 512), (9, 200)]:
        s = datagen.conv1d_causal_sweep(K, device=dev, C=C)
        sweep.append(s)
        sL = s["lengths"].to(dev)
        sy = torch.empty_like(s["x"])
        add(f"conv1d_causal_K{K}_C{C}", "dwconv1d_fwd", f"[32,1500,{C}] K{K} causal fp32", s["B"] * s["T"],
            *work_conv1d(s, 4),
            (lambda s=s, sL=sL, sy=sy: dw.dwconv1d_fwd(s["x"], s["w"], s["b"], sL, y=sy, causal=True)))

    st = datagen.conv1d_stream(device=dev)
    stL = st["lengths"].to(dev)
    sty = torch.empty_like(st["x"])
    stc = torch.empty_like(st["cache"])
    add("conv1d_stream_bf16", "dwconv1d_stream_fwd", "1024 streams x 8-frame chunks, C1024 K9, K-1 frame cache, bf16",
        st["B"] * st["Tc"], *work_conv1d_stream(st, 2),
        lambda: dw.dwconv1d_stream_fwd(st["x"], st["w"], st["b"], stL, st["cache"], cache_out=stc, y=sty))

    s9 = sweep[3]
    assert s9["K"] == 9 and s9["C"] == 512
    s9["dy"] = datagen.normal((s9["B"], s9["T"], s9["C"]), 1.0, "c4/dy/K9/C512", device=dev)
    s9L = s9["lengths"].to(dev)
    bdx = torch.empty_like(s9["x"])
    bdw = torch.empty((9, s9["C"]), device=dev)
    bdb = torch.empty((s9["C"],), device=dev)
    bws = torch.empty((dw.dwconv1d_bwd_workspace_bytes(s9["B"], s9["T"], s9["C"], 9),), dtype=torch.uint8,
                      device=dev)
    add("conv1d_bwd_K9_C512", "dwconv1d_bwd", "dx,dw,db of [32,1500,512] K9 causal fp32, fp64 sums",
        s9["B"] * s9["T"], *work_conv1d_bwd(s9),
        lambda: dw.dwconv1d_bwd(s9["x"], s9["w"], s9L, s9["dy"], dx=bdx, dw=bdw, db=bdb, workspace=bws,
                                causal=True))

    g = datagen.conv2d_stage(device=dev)
    gL = g["lengths"].to(dev)
    gy = torch.empty((g["B"], 750, 32, g["C"]), device=dev)
    gdx = torch.empty_like(g["x"])
    gdw = torch.empty((3, 3, g["C"]), device=dev)
    gdb = torch.empty((g["C"],), device=dev)
    ws = torch.empty((dw.dwconv2d_bwd_workspace_bytes(g["B"], g["T"], g["F"], g["C"]),), dtype=torch.uint8,
                     device=dev)
    add("stage_fwd", "dwconv2d_fwd", "[32,1500,64,256] -> [32,750,32,256] fp32", g["B"] * g["T"],
        *work_stage_fwd(g), lambda: dw.dwconv2d_fwd(g["x"], g["w"], g["b"], gL, y=gy))
    add("stage_bwd", "dwconv2d_bwd", "dx,dw,db of [32,1500,64,256] fp32", g["B"] * g["T"], *work_stage_bwd(g),
        lambda: dw.dwconv2d_bwd(g["x"], g["w"], gL, g["dy"], dx=gdx, dw=gdw, db=gdb, workspace=ws))

    # the same stage with causal padding (fp32), and with bf16 storage (symmetric)
    causal = dw.CAUSAL_PADS_2D
    To_c, Fo_c = dw.conv2d_out_shape(g["T"], g["F"], pads=causal)
    gc = dict(g, dy=datagen.normal((g["B"], To_c, Fo_c, g["C"]), 1.0, "c5/dy", device=dev))
    gcy = torch.empty((g["B"], To_c, Fo_c, g["C"]), device=dev)
    wsc = torch.empty((dw.dwconv2d_bwd_workspace_bytes(g["B"], g["T"], g["F"], g["C"], pads=causal),),
                      dtype=torch.uint8, device=dev)
    add("stage_fwd_causal", "dwconv2d_fwd_ex", "[32,1500,64,256] -> [32,751,33,256] causal pads fp32",
        g["B"] * g["T"], *work_stage_fwd(g, causal),
        lambda: dw.dwconv2d_fwd(g["x"], g["w"], g["b"], gL, y=gcy, pads=causal))
    add("stage_bwd_causal", "dwconv2d_bwd_ex", "dx,dw,db of [32,1500,64,256] causal pads fp32", g["B"] * g["T"],
        *work_stage_bwd(g, causal),
        lambda: dw.dwconv2d_bwd(g["x"], g["w"], gL, gc["dy"], dx=gdx, dw=gdw, db=gdb, workspace=wsc, pads=causal))
    h = {k: (v.to(torch.bfloat16) if k in ("x", "w", "b", "dy") else v) for k, v in g.items()}
    hy = torch.empty((g["B"], 750, 32, g["C"]), dtype=torch.bfloat16, device=dev)
    hdx = torch.empty_like(h["x"])
    add("stage_fwd_bf16", "dwconv2d_fwd_ex", "[32,1500,64,256] -> [32,750,32,256] bf16 storage", g["B"] * g["T"],
        *work_stage_fwd(g, es=2), lambda: dw.dwconv2d_fwd(h["x"], h["w"], h["b"], gL, y=hy))
    add("stage_bwd_bf16", "dwconv2d_bwd_ex", "dx,dw,db of [32,1500,64,256] bf16 storage, fp32 dw/db",
        g["B"] * g["T"], *work_stage_bwd(g, es=2),
        lambda: dw.dwconv2d_bwd(h["x"], h["w"], gL, h["dy"], dx=hdx, dw=gdw, db=gdb, workspace=ws))
    # 8x subsampling's third stride-2 stage, on the 4x front output of a 15 s batch
    g3 = datagen.conv2d_stage(device=dev, B=32, T=375, F=20, C=256)
    g3L = g3["lengths"].to(dev)
    g3y = torch.empty((32, 188, 10, 256), device=dev)
    g3dx = torch.empty_like(g3["x"])
    ws3 = torch.empty((dw.dwconv2d_bwd_workspace_bytes(32, 375, 20, 256),), dtype=torch.uint8, device=dev)
    add("stage3_fwd", "dwconv2d_fwd", "[32,375,20,256] -> [32,188,10,256] fp32 (8x third stage)", g3["B"] * g3["T"],
        *work_stage_fwd(g3), lambda: dw.dwconv2d_fwd(g3["x"], g3["w"], g3["b"], g3L, y=g3y))
    add("stage3_bwd", "dwconv2d_bwd", "dx,dw,db of [32,375,20,256] fp32 (8x third stage)", g3["B"] * g3["T"],
        *work_stage_bwd(g3),
        lambda: dw.dwconv2d_bwd(g3["x"], g3["w"], g3L, g3["dy"], dx=g3dx, dw=gdw, db=gdb, workspace=ws3))
    data = dict(front=f, conv1d_bf16=e, sweep=sweep, stage=g, stage_causal=gc, stage_bf16=h, stream=st, stage3=g3)
    assert [r["name"] for r in rows] == [n for n, _ in ROW_KERNELS], "ROW_KERNELS is out of date"
    return rows, data


def cpu_baseline(data, target_s: float):
    """Time the CPU oracle on whole items of each workload (same shapes and
    lengths), single-threaded, and scale to frames per second."""
    import oracle

    host = lambda t, n: t[:n].detach().float().cpu()
    # parameters copied to the host once, outside the timed calls
    hp = lambda d: {k: (v.detach().float().cpu() if hasattr(v, "detach") and k != "x" and k != "dy" else v)
                    for k, v in d.items()}
    f, e, g = hp(data["front"]), hp(data["conv1d_bf16"]), hp(data["stage"])
    f["x"], f["dy"], f["dy_causal"] = data["front"]["x"], data["front"]["dy"], data["front"]["dy_causal"]
    e["x"], g["x"], g["dy"] = data["conv1d_bf16"]["x"], data["stage"]["x"], data["stage"]["dy"]
    gc = dict(g, dy=data["stage_causal"]["dy"])
    gh = hp(data["stage_bf16"])                    # bf16 values, widened exactly on the host
    gh["x"], gh["dy"] = data["stage_bf16"]["x"], data["stage_bf16"]["dy"]
    g3 = hp(data["stage3"])
    g3["x"], g3["dy"] = data["stage3"]["x"], data["stage3"]["dy"]
    sm = hp(data["stream"])
    sm["x"], sm["cache"] = data["stream"]["x"], data["stream"]["cache"]
    sweep = []
    for s in data["sweep"]:
        hs = hp(s)
        hs["x"] = s["x"]
        if "dy" in s:
            hs["dy"] = s["dy"]
        sweep.append(hs)

    def one_pass(n):
        """The oracle on the first min(n, B) items of every operation's batch."""
        secs, frames = 0.0, 0
        m = min(n, f["B"])
        xs = host(f["x"], m)
        t = time.perf_counter()
        oracle.dwsub_front_fwd(xs, f["w0"], f["b0"], f["w1"], f["b1"], f["lengths"][:m])
        secs += time.perf_counter() - t
        frames += m * f["T"]
        m = min(n, f["B"])
        xs, dys = host(f["x"], m), host(f["dy"], m)
        t = time.perf_counter()
        oracle.dwsub_front_bwd(xs, f["w0"], f["b0"], f["w1"], f["lengths"][:m], dys)
        secs += time.perf_counter() - t
        frames += m * f["T"]
        dys = host(f["dy_causal"], m)
        t = time.perf_counter()
        oracle.dwsub_front_fwd(xs, f["w0"], f["b0"], f["w1"], f["b1"], f["lengths"][:m], causal=True)
        oracle.dwsub_front_bwd(xs, f["w0"], f["b0"], f["w1"], f["lengths"][:m], dys, causal=True)
        secs += time.perf_counter() - t
        frames += 2 * m * f["T"]
        m = min(n, e["B"])
        xs = host(e["x"], m)
        t = time.perf_counter()
        oracle.dwconv1d_fwd(xs, e["w"], e["b"], e["lengths"][:m], False)
        secs += time.perf_counter() - t
        frames += m * e["T"]
        for s in sweep:
            m = min(n, s["B"])
            xs = host(s["x"], m)
            t = time.perf_counter()
            oracle.dwconv1d_fwd(xs, s["w"], s["b"], s["lengths"][:m], True)
            secs += time.perf_counter() - t
            frames += m * s["T"]
            if "dy" in s:
                dys = host(s["dy"], m)
                t = time.perf_counter()
                oracle.dwconv1d_bwd(xs, s["w"], s["lengths"][:m], dys, True)
                secs += time.perf_counter() - t
                frames += m * s["T"]
        m = min(n, sm["B"])
        xs, cs = host(sm["x"], m), host(sm["cache"], m)
        t = time.perf_counter()
        oracle.dwconv1d_stream_fwd(xs, sm["w"], sm["b"], sm["lengths"][:m], cs)
        secs += time.perf_counter() - t
        frames += m * sm["Tc"]
        m = min(n, g["B"])
        for st, pads in ((g, None), (gc, (2, 1, 2, 1)), (gh, None), (g3, None)):
            xs, dys = host(st["x"], m), host(st["dy"], m)
            t = time.perf_counter()
            oracle.dwconv2d_fwd(xs, st["w"], st["b"], st["lengths"][:m], pads=pads)
            oracle.dwconv2d_bwd(xs, st["w"], st["lengths"][:m], dys, pads=pads)
            secs += time.perf_counter() - t
            frames += 2 * m * st["T"]
        return secs, frames

    # The oracle is single-threaded C; the process is held to one core while
    # it runs, so that nothing else (numpy's own threads) lends it another.
    saved = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if saved:
        os.sched_setaffinity(0, {min(saved)})
    try:
        s1, _ = one_pass(1)
        n = int(max(1, min(g["B"], math.floor(target_s / max(s1, 1e-3)))))
        secs, frames, reps = 0.0, 0, 0
        while reps == 0 or secs < target_s:
            ds, df = one_pass(n)
            secs, frames, reps = secs + ds, frames + df, reps + 1
    finally:
        if saved:
            os.sched_setaffinity(0, saved)
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    return dict(value=round(frames / secs, 1), unit="frames/s", cores=1, kind="oracle",
                cpu_model=model, host_cpus=os.cpu_count(),
                sample=(f"every operation of the step on the first {n} items of its batch (at most its batch "
                        f"size), same shapes and lengths, {reps} pass(es): {frames} frames in {secs:.2f} s; "
                        f"the oracle is single-threaded C with fp64 accumulation, run on one pinned core"))


def read_traffic():
    """Counter-derived HBM bytes per launch of the dominant kernel, if the
    counters were taken on the current source of that kernel."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("src_sha256") != sources_sha(DOMINANT_SOURCES):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR", help="summarise rocprofv3 output under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch

    dev = torch.device("cuda", 0)
    log("building workloads ...")
    rows, data = build_rows(dev)
    torch.cuda.synchronize()
    if args.calib_copy:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        bcopy = torch.empty_like(a)
        a.fill_(1.0)
        torch.cuda.synchronize()
        bcopy.copy_(a)
        torch.cuda.synchronize()
        del a, bcopy

    for i in range(args.warmup):
        for r in rows:
            r["fn"]()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # The timed steps record events around the dominant row only: an event
    # pair around every row adds about 0.15 ms to a 4.2 ms step.  The
    # per-row table comes from a second, untimed pass of as many steps with
    # an event pair around every row.
    jdom = next(j for j, r in enumerate(rows) if r["name"] == DOMINANT_ROW)
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for j, r in enumerate(rows):
            if j == jdom:
                dev_ev[s][0].record()
            r["fn"]()
            if j == jdom:
                dev_ev[s][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")
    dom_us = sorted(a.elapsed_time(b) * 1e3 for a, b in dev_ev)

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in rows]
          for _ in range(args.steps)]
    for s in range(args.steps):
        for j, r in enumerate(rows):
            ev[s][j][0].record()
            r["fn"]()
            ev[s][j][1].record()
    torch.cuda.synchronize()
    log(f"per-row pass of {args.steps} steps done")

    ms_step = wall * 1e3 / args.steps
    frames = sum(r["frames"] for r in rows)
    alg = sum(r["read"] + r["write"] for r in rows)
    out_rows = []
    for j, r in enumerate(rows):
        ts = sorted(ev[s][j][0].elapsed_time(ev[s][j][1]) * 1e3 for s in range(args.steps))
        us = sum(ts) / len(ts)
        b = r["read"] + r["write"]
        row = dict(row=r["name"], op=r["op"], config=r["cfg"], us=round(us, 2), us_median=round(ts[len(ts) // 2], 2),
                   us_min=round(ts[0], 2), us_p90=round(ts[min(len(ts) - 1, (9 * len(ts)) // 10)], 2),
                   frames_per_s=round(r["frames"] / (us * 1e-6)), alg_bytes=b,
                   gbps=round(b / (us * 1e-6) / 1e9, 1), hbm_frac=round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                   dense_bytes=r["read_dense"] + r["write"],
                   dense_gbps=round((r["read_dense"] + r["write"]) / (us * 1e-6) / 1e9, 1))
        if r["bound"] == "alu":
            tf = r["flops"] / (us * 1e-6) / 1e12
            row.update(bound="alu", alg_flops=r["flops"], tflops=round(tf, 2),
                       alu_frac=round(tf / VALU_F32_PEAK_TFLOPS, 4))
        else:
            row.update(bound="hbm")
        out_rows.append(row)
        log(f"  {r['name']:<22} {us:9.2f} us  {row['gbps']:8.1f} GB/s  ({100 * row['hbm_frac']:.1f}% of 8 TB/s)")

    dom = next(r for r in out_rows if r["row"] == DOMINANT_ROW)
    dom_mean = sum(dom_us) / len(dom_us)
    dom_gbps = round(dom["alg_bytes"] / (dom_mean * 1e-6) / 1e9, 1)
    roofline = dict(kernel=DOMINANT_KERNEL, bound="hbm", achieved=dom_gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(dom_gbps / HBM_PEAK_GBPS, 4), traffic=read_traffic(),
                    launch_us=round(dom_mean, 2), alg_bytes_per_launch=dom["alg_bytes"])

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        cpu = cpu_baseline(data, args.cpu_seconds)
        log(f"  oracle: {cpu['value']:.0f} frames/s ({cpu['sample']})")

    line = {
        "metric": "depthwise conv frames/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": round(frames / (ms_step * 1e-3), 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; log-mel-shaped inputs, lengths ~U[T/2,T])",
        "config": {
            "workload": "encoder depthwise path: fused front [4,1000,80] fwd+bwd (symmetric and causal); conv-module dwconv1d [16,750,1024] K9 "
                        "bf16; causal dwconv1d [32,1500,512] K3/4/5/9/15 (K9 fwd+bwd) and [32,1500,200] K9; streaming dwconv1d 1024x8x1024 K9 bf16 with cache; depthwise conv2d "
                        "stage [32,1500,64,256] fwd+bwd (symmetric fp32, causal fp32, symmetric bf16); third stage "
                        "[32,375,20,256] fwd+bwd",
            "frames_per_step": frames,
            "alg_bytes_per_step": alg,
            "parallelism": "single GPU",
        },
        "hbm": {"achieved_gbps": round(alg / (ms_step * 1e-3) / 1e9, 1), "peak_gbps": HBM_PEAK_GBPS,
                "frac": round(alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "rows": out_rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


# --------------------------------------------------------------------------
# rocprofv3 summaries
# --------------------------------------------------------------------------

def _csv_rows(pattern):
    out = []
    for p in sorted(glob.glob(pattern, recursive=True)):
        with open(p, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def attribute_dispatches(disp):
    """Map each bench row to its dispatches.  disp: [(dispatch id, kernel
    name, payload)] in any order.  Returns {row: [payload, ...]}."""
    disp = sorted(disp, key=lambda t: int(t[0]))
    out = {}
    for name, prefix in ROW_KERNELS:
        same = [n for n, p in ROW_KERNELS if p == prefix]
        k, period = same.index(name), len(same)
        hits = [pl for _, kn, pl in disp if prefix in kn]
        out[name] = hits[k::period] if len(hits) % period == 0 else []
    return out


def summarize_profile(d):
    """Write profiles/ summaries from rocprofv3 output under d:
    d/stats/**/*kernel_stats.csv and *kernel_trace.csv (durations),
    d/fetch/**/*counter_collection.csv and d/write/** (HBM bytes); any may be
    missing."""
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    cmd = lambda k: (open(os.path.join(d, k, "command.txt")).read().strip()
                     if os.path.exists(os.path.join(d, k, "command.txt")) else "?")
    stats = _csv_rows(os.path.join(d, "stats", "**", "*kernel_stats.csv"))
    trace = _csv_rows(os.path.join(d, "stats", "**", "*kernel_trace.csv"))
    if stats:
        lines = ["# rocprofv3 --kernel-trace --stats, one bench.py run on one MI355X",
                 "# command: " + cmd("stats"),
                 "# per kernel name (every dispatch of the run: warm-up, timed and per-row steps):",
                 f"{'kernel':<60} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
        for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0) or 0)):
            name = r.get("Name", r.get("KernelName", "?"))
            short = (name[5:] if name.startswith("void ") else name).split("(")[0][:60]
            lines.append(f"{short:<60} {int(r.get('Calls', 0)):>6} {float(r.get('AverageNs', 0)) / 1e3:>10.2f} "
                         f"{float(r.get('MinNs', 0)) / 1e3:>10.2f} {float(r.get('MaxNs', 0)) / 1e3:>10.2f} "
                         f"{float(r.get('Percentage', 0)):>6.2f}")
        if trace:
            disp = [(r["Dispatch_Id"], r["Kernel_Name"],
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3) for r in trace]
            per_row = attribute_dispatches(disp)
            lines += ["", "# per bench row: the row's main kernel, its dispatches in this run (warm-up, timed",
                      "# and per-row steps) and their durations; a row's k-th dispatch of a kernel name within a",
                      "# step is the k-th row listing that name",
                      f"{'row':<24} {'kernel':<52} {'n':>4} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"]
            for name, prefix in ROW_KERNELS:
                v = per_row.get(name) or []
                kshort = prefix.replace("dw::", "").rstrip("(")[:52]
                if v:
                    lines.append(f"{name:<24} {kshort:<52} {len(v):>4} {sum(v) / len(v):>9.2f} {min(v):>9.2f} "
                                 f"{max(v):>9.2f}")
                else:
                    lines.append(f"{name:<24} {kshort:<52}    - (no dispatches attributed)")
        with open(os.path.join(ROOT, "profiles", "kernel_stats_bench_step.txt"), "w") as fh:
            fh.write("\n".join(lines) + "\n")
        print("\n".join(lines))

    def counter(kind, cname):
        """[(dispatch id, kernel name, value summed over the counter's instances)]."""
        per = {}
        for r in _csv_rows(os.path.join(d, kind, "**", "*counter_collection.csv")):
            if r.get("Counter_Name") != cname:
                continue
            key = r.get("Dispatch_Id")
            name, v = r.get("Kernel_Name", ""), float(r.get("Counter_Value", 0))
            per[key] = (name, per.get(key, (name, 0.0))[1] + v)
        return [(k, n, v) for k, (n, v) in per.items()]

    fetch = counter("fetch", "FETCH_SIZE")
    write = counter("write", "WRITE_SIZE")
    if not (fetch and write):
        return
    copy_bytes = float(1 << 30)

    def calib(tab):
        # the 1 GiB device copy is the largest copy-engine-kernel dispatch
        vals = [v for (_, n, v) in tab if "copyBuffer" in n]
        return max(vals) if vals else None

    cf, cw = calib(fetch), calib(write)
    f_rows, w_rows = attribute_dispatches(fetch), attribute_dispatches(write)
    mean = lambda v: sum(v) / len(v) if v else None
    kf, kw = mean(f_rows.get(DOMINANT_ROW)), mean(w_rows.get(DOMINANT_ROW))
    lines = ["# HBM traffic per launch of the dominant row's kernel, from rocprofv3 --pmc FETCH_SIZE",
             "# and WRITE_SIZE (KiB per dispatch, separate runs), each scaled by the same counter's",
             "# reading for a 1 GiB device copy (the copy reads 1 GiB and writes 1 GiB).",
             "# fetch run: " + cmd("fetch"),
             "# write run: " + cmd("write"),
             f"row={DOMINANT_ROW}",
             f"kernel={DOMINANT_KERNEL}",
             f"src_sha256={sources_sha(DOMINANT_SOURCES)}",
             f"copy_fetch_kib={cf}", f"copy_write_kib={cw}",
             f"kernel_fetch_kib={kf}", f"kernel_write_kib={kw}"]
    if cf and cw and kf is not None and kw is not None:
        sf, swr = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
        fb, wb = kf * 1024.0 * sf, kw * 1024.0 * swr
        lines += [f"scale_fetch={sf:.4f}", f"scale_write={swr:.4f}", f"fetch_bytes_per_launch={fb:.0f}",
                  f"write_bytes_per_launch={wb:.0f}", f"hbm_bytes_per_launch={fb + wb:.0f}"]
        lines.append("# every row's main kernel, HBM bytes per launch from the scaled counters: fetch, write")
        for name, _ in ROW_KERNELS:
            a, b = mean(f_rows.get(name)), mean(w_rows.get(name))
            if a is not None and b is not None:
                lines.append(f"#   {name:<24} {a * 1024.0 * sf:>16.0f} {b * 1024.0 * swr:>16.0f}")
    with open(TRAFFIC_FILE, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))

if __name__ == "__main__":
    sys.exit(main())
