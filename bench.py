#!/usr/bin/env python3
"""Throughput of the depthwise-convolution path on one MI355X.

One step runs every operation of the path once, each at its workload's full
size, on synthetic inputs resident in HBM:

  small   dwconv1d_fwd      [2,64,8] K=9 symmetric                      fp32 (µs per launch)
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
  forward_target  the lowest fraction of 8 TB/s among the forward depthwise
               rows, the row that sets it, and whether every one reaches 70%;
               kernel_only: the same from the kernels' own durations in the
               committed rocprofv3 summary (absent when that is out of date)
  rows         the same figures for every operation: mean time per call from
               HIP events (and its median, minimum and 90th percentile over
               the steps); kernel_us, the kernel-only mean from the committed
               rocprofv3 summary (null when the kernels changed since it was
               taken); for HBM-bound rows, probe_us, the time of a plain
               streaming kernel moving the row's own read and write bytes,
               timed the same way, and of_probe = probe_us / us; max_err,
               max |gpu - oracle| / (1 + |oracle|) on the items the CPU
               baseline runs, and its ratio to the row's tolerance
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
# every source the per-row kernel-only times depend on
KERNEL_SOURCES = ["conv_subsampling_amd/csrc/" + f for f in
                  ("capi.hip", "common.h", "launch.h", "dwconv1d.hip", "dwconv2d.hip", "dwsub_front.hip",
                   "reduce.hip", "probe.hip")]
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
    ("conv1d_small", "dw::dwconv1d_fwd_kernel<float, 4, 9, 8>("),
    ("front", "dw::dwsub_fused_fwd_kernel<float>("),
    ("front_bwd", "dw::dwsub_fused_bwd_kernel<float, 4>("),
    ("front_causal", "dw::dwsub_fused_fwd_kernel<float>("),
    ("front_bwd_causal", "dw::dwsub_fused_bwd_kernel<float, 5>("),
    ("conv1d_bf16", "dw::dwconv1d_fwd_kernel<unsigned short, 4, 9, 12>("),
    ("conv1d_causal_K3_C512", "dw::dwconv1d_fwd_pipe_kernel<3>("),
    ("conv1d_causal_K4_C512", "dw::dwconv1d_fwd_pipe_kernel<4>("),
    ("conv1d_causal_K5_C512", "dw::dwconv1d_fwd_pipe_kernel<5>("),
    ("conv1d_causal_K9_C512", "dw::dwconv1d_fwd_pipe_kernel<9>("),
    ("conv1d_causal_K15_C512", "dw::dwconv1d_fwd_pipe_kernel<15>("),
    ("conv1d_causal_K9_C200", "dw::dwconv1d_fwd_pipe_kernel<9>("),
    ("conv1d_stream_bf16", "dw::dwconv1d_stream_pipe_kernel<unsigned short, 9>("),
    ("conv1d_bwd_K9_C512", "dw::dwconv1d_bwd_group_kernel<float, 9, true, 8, 2>("),
    ("stage_fwd", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage_bwd", "dw::dwconv2d_bwd_kernel<float, 4, 1, 0, 0, false>("),
    ("stage_fwd_causal", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage_bwd_causal", "dw::dwconv2d_bwd_kernel<float, 4, 1, 1, 1, false>("),
    ("stage_fwd_bf16", "dw::dwconv2d_fwd_kernel<unsigned short, 8, 1, 32>("),
    ("stage_bwd_bf16", "dw::dwconv2d_bwd_kernel<unsigned short, 4, 2, 0, 0, true>("),
    ("stage3_fwd", "dw::dwconv2d_fwd_kernel<float, 4, 1, 64>("),
    ("stage3_bwd", "dw::dwconv2d_bwd_kernel<float, 4, 1, 0, 0, false>("),
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
    """Every row of the step: its work, the call the step times, and, for the
    accuracy check and the CPU baseline, the same operation on the first n
    items of its batch through the GPU path (`gpu`) and through the oracle
    (`ref`: copies those items to the host and returns a call that runs the
    oracle on them, so that only the oracle is timed)."""
    import torch

    import conv_subsampling_amd as dw
    import datagen

    rows = []
    T32, TBF = 1e-5, 2e-2     # |gpu - ref| <= tol * (1 + |ref|): fp32 storage, bf16 storage

    def add(name, op, cfg, frames, rd, wr, flops, rd_dense, fn, bound="hbm", *, items, item_frames, gpu, ref, tol):
        rows.append(dict(name=name, op=op, cfg=cfg, frames=frames, read=rd, write=wr, flops=flops,
                         read_dense=rd_dense, fn=fn, bound=bound, items=items, item_frames=item_frames,
                         gpu=gpu, ref=ref, tol=tol))

    def host(t, n=None):
        return (t if n is None else t[:n]).detach().float().cpu()

    def oracle_mod():
        import oracle
        return oracle

    # small 1-D conv: [2,64,8] K9 symmetric fp32, lengths {64, 41}
    c1 = datagen.conv1d_small(device=dev)
    c1L = c1["lengths"].to(dev)
    c1y = torch.empty_like(c1["x"])

    def c1_ref(n):
        o, xs, w, b, L = oracle_mod(), host(c1["x"], n), host(c1["w"]), host(c1["b"]), c1["lengths"][:n]
        return lambda: [o.dwconv1d_fwd(xs, w, b, L, False)]

    add("conv1d_small", "dwconv1d_fwd", "[2,64,8] K9 symmetric fp32 (launch-latency bound)", c1["B"] * c1["T"],
        *work_conv1d(c1, 4), lambda: dw.dwconv1d_fwd(c1["x"], c1["w"], c1["b"], c1L, y=c1y, causal=False),
        bound="latency", items=c1["B"], item_frames=c1["T"],
        gpu=lambda n: [dw.dwconv1d_fwd(c1["x"][:n], c1["w"], c1["b"], c1L[:n], causal=False)],
        ref=c1_ref, tol=[T32])

    # fused front, symmetric and causal, forward and backward
    f = datagen.fused_front(device=dev)
    fL = f["lengths"].to(dev)
    fy = torch.empty((f["B"], 250, 20, f["C"]), device=dev)
    fdy = datagen.normal((f["B"], 250, 20, f["C"]), 1.0, "c2/dy", device=dev)
    fcdy = datagen.normal((f["B"], 251, 21, f["C"]), 1.0, "c2/dy", device=dev)
    fg = [torch.empty(sh, device=dev) for sh in ((3, 3, f["C"]), (f["C"],), (3, 3, f["C"]), (f["C"],))]
    fws = torch.empty((dw.dwsub_fused_bwd_workspace_bytes(f["B"], f["T"], f["F"], f["C"]),), dtype=torch.uint8,
                      device=dev)
    fcy = torch.empty((f["B"], 251, 21, f["C"]), device=dev)
    fcws = torch.empty((dw.dwsub_fused_bwd_workspace_bytes(f["B"], f["T"], f["F"], f["C"], causal=True),),
                       dtype=torch.uint8, device=dev)
    fp = {k: host(f[k]) for k in ("w0", "b0", "w1", "b1")}

    def front_ref(causal):
        def make(n):
            o, xs, L = oracle_mod(), host(f["x"], n), f["lengths"][:n]
            return lambda: [o.dwsub_front_fwd(xs, fp["w0"], fp["b0"], fp["w1"], fp["b1"], L, causal=causal)]
        return make

    def front_bwd_ref(causal):
        def make(n):
            o, xs, L = oracle_mod(), host(f["x"], n), f["lengths"][:n]
            dys = host(fcdy if causal else fdy, n)
            return lambda: list(o.dwsub_front_bwd(xs, fp["w0"], fp["b0"], fp["w1"], L, dys, causal=causal))
        return make

    for causal in (False, True):
        sfx = "_causal" if causal else ""
        shape = "[4,251,21,256] causal" if causal else "[4,250,20,256]"
        add("front" + sfx, "dwsub_fused_fwd" + ("_ex" if causal else ""), f"mel [4,1000,80] -> {shape} fp32",
            f["B"] * f["T"], *work_front(f, int(causal)),
            (lambda c=causal: dw.dwsub_fused_fwd(f["x"], f["w0"], f["b0"], f["w1"], f["b1"], fL,
                                                 y=fcy if c else fy, causal=c)),
            bound="alu", items=f["B"], item_frames=f["T"],
            gpu=(lambda n, c=causal: [dw.dwsub_fused_fwd(f["x"][:n], f["w0"], f["b0"], f["w1"], f["b1"], fL[:n],
                                                         causal=c)]),
            ref=front_ref(causal), tol=[T32])
        add("front_bwd" + sfx, "dwsub_fused_bwd" + ("_ex" if causal else ""),
            f"dw0,db0,dw1,db1 of the front, dy {shape}, fp64 accumulation", f["B"] * f["T"],
            *work_front_bwd(f, int(causal)),
            (lambda c=causal: dw.dwsub_fused_bwd(f["x"], f["w0"], f["b0"], f["w1"], fL, fcdy if c else fdy, *fg,
                                                 workspace=fcws if c else fws, causal=c)),
            bound="alu", items=f["B"], item_frames=f["T"],
            gpu=(lambda n, c=causal: list(dw.dwsub_fused_bwd(f["x"][:n], f["w0"], f["b0"], f["w1"], fL[:n],
                                                             (fcdy if c else fdy)[:n], causal=c))),
            ref=front_bwd_ref(causal), tol=[T32] * 4)

    def conv1d_rows(name, cfg, d, es, tol, causal):
        L = d["lengths"].to(dev)
        y = torch.empty_like(d["x"])
        w, b = host(d["w"]), host(d["b"])

        def make(n):
            o, xs, Ls = oracle_mod(), host(d["x"], n), d["lengths"][:n]
            return lambda: [o.dwconv1d_fwd(xs, w, b, Ls, causal)]
        add(name, "dwconv1d_fwd", cfg, d["B"] * d["T"], *work_conv1d(d, es),
            lambda: dw.dwconv1d_fwd(d["x"], d["w"], d["b"], L, y=y, causal=causal),
            items=d["B"], item_frames=d["T"],
            gpu=lambda n: [dw.dwconv1d_fwd(d["x"][:n], d["w"], d["b"], L[:n], causal=causal)], ref=make, tol=[tol])

    e = datagen.conv1d_encoder_bf16(device=dev)
    conv1d_rows("conv1d_bf16", "[16,750,1024] K9 symmetric bf16", e, 2, TBF, False)

    sweep = []
    for K, C in [(3, 512), (4, 512), (5, 512), (9, 512), (15, 512), (9, 200)]:
        sd = datagen.conv1d_causal_sweep(K, device=dev, C=C)
        sweep.append(sd)
        conv1d_rows(f"conv1d_causal_K{K}_C{C}", f"[32,1500,{C}] K{K} causal fp32", sd, 4, T32, True)

    st = datagen.conv1d_stream(device=dev)
    stL = st["lengths"].to(dev)
    sty = torch.empty_like(st["x"])
    stc = torch.empty_like(st["cache"])
    stw, stb = host(st["w"]), host(st["b"])

    def stream_ref(n):
        o, xs, cs, Ls = oracle_mod(), host(st["x"], n), host(st["cache"], n), st["lengths"][:n]
        return lambda: list(o.dwconv1d_stream_fwd(xs, stw, stb, Ls, cs))

    add("conv1d_stream_bf16", "dwconv1d_stream_fwd", "1024 streams x 8-frame chunks, C1024 K9, K-1 frame cache, bf16",
        st["B"] * st["Tc"], *work_conv1d_stream(st, 2),
        lambda: dw.dwconv1d_stream_fwd(st["x"], st["w"], st["b"], stL, st["cache"], cache_out=stc, y=sty),
        items=st["B"], item_frames=st["Tc"],
        gpu=lambda n: list(dw.dwconv1d_stream_fwd(st["x"][:n], st["w"], st["b"], stL[:n], st["cache"][:n])),
        ref=stream_ref, tol=[TBF, TBF])

    s9 = sweep[3]
    assert s9["K"] == 9 and s9["C"] == 512
    s9["dy"] = datagen.normal((s9["B"], s9["T"], s9["C"]), 1.0, "c4/dy/K9/C512", device=dev)
    s9L = s9["lengths"].to(dev)
    bdx = torch.empty_like(s9["x"])
    bdw = torch.empty((9, s9["C"]), device=dev)
    bdb = torch.empty((s9["C"],), device=dev)
    bws = torch.empty((dw.dwconv1d_bwd_workspace_bytes(s9["B"], s9["T"], s9["C"], 9),), dtype=torch.uint8,
                      device=dev)
    s9w = host(s9["w"])

    def bwd1d_ref(n):
        o, xs, dys, Ls = oracle_mod(), host(s9["x"], n), host(s9["dy"], n), s9["lengths"][:n]
        return lambda: list(o.dwconv1d_bwd(xs, s9w, Ls, dys, True))

    add("conv1d_bwd_K9_C512", "dwconv1d_bwd", "dx,dw,db of [32,1500,512] K9 causal fp32, fp64 sums",
        s9["B"] * s9["T"], *work_conv1d_bwd(s9),
        lambda: dw.dwconv1d_bwd(s9["x"], s9["w"], s9L, s9["dy"], dx=bdx, dw=bdw, db=bdb, workspace=bws,
                                causal=True),
        items=s9["B"], item_frames=s9["T"],
        gpu=lambda n: list(dw.dwconv1d_bwd(s9["x"][:n], s9["w"], s9L[:n], s9["dy"][:n], causal=True)),
        ref=bwd1d_ref, tol=[T32] * 3)

    # the conv2d stage: symmetric fp32, causal fp32, symmetric bf16; then the third stage
    g = datagen.conv2d_stage(device=dev)
    gL = g["lengths"].to(dev)
    causal = dw.CAUSAL_PADS_2D
    To_c, Fo_c = dw.conv2d_out_shape(g["T"], g["F"], pads=causal)
    gc = dict(g, dy=datagen.normal((g["B"], To_c, Fo_c, g["C"]), 1.0, "c5/dy", device=dev))
    h = {k: (v.to(torch.bfloat16) if k in ("x", "w", "b", "dy") else v) for k, v in g.items()}
    g3 = datagen.conv2d_stage(device=dev, B=32, T=375, F=20, C=256)
    gdw = torch.empty((3, 3, g["C"]), device=dev)
    gdb = torch.empty((g["C"],), device=dev)
    gdx = torch.empty_like(g["x"])

    def stage_rows(name, cfg, d, pads, es, tol):
        L = d["lengths"].to(dev)
        To, Fo = dw.conv2d_out_shape(d["T"], d["F"], pads=pads)
        y = torch.empty((d["B"], To, Fo, d["C"]), dtype=d["x"].dtype, device=dev)
        dx = gdx if d["x"].shape == gdx.shape and d["x"].dtype == gdx.dtype else torch.empty_like(d["x"])
        ws = torch.empty((dw.dwconv2d_bwd_workspace_bytes(d["B"], d["T"], d["F"], d["C"], pads=pads),),
                         dtype=torch.uint8, device=dev)
        w, b = host(d["w"]), host(d["b"])
        pd = "" if pads is None and es == 4 else "_ex"

        def fref(n):
            o, xs, Ls = oracle_mod(), host(d["x"], n), d["lengths"][:n]
            return lambda: [o.dwconv2d_fwd(xs, w, b, Ls, pads=pads)]

        def bref(n):
            o, xs, dys, Ls = oracle_mod(), host(d["x"], n), host(d["dy"], n), d["lengths"][:n]
            return lambda: list(o.dwconv2d_bwd(xs, w, Ls, dys, pads=pads))

        add(f"{name}_fwd" + cfg[0], "dwconv2d_fwd" + pd, cfg[1], d["B"] * d["T"], *work_stage_fwd(d, pads or (1, 1, 1, 1), es),
            lambda: dw.dwconv2d_fwd(d["x"], d["w"], d["b"], L, y=y, pads=pads),
            items=d["B"], item_frames=d["T"],
            gpu=lambda n: [dw.dwconv2d_fwd(d["x"][:n], d["w"], d["b"], L[:n], pads=pads)], ref=fref, tol=[tol])
        add(f"{name}_bwd" + cfg[0], "dwconv2d_bwd" + pd, cfg[2], d["B"] * d["T"], *work_stage_bwd(d, pads or (1, 1, 1, 1), es),
            lambda: dw.dwconv2d_bwd(d["x"], d["w"], L, d["dy"], dx=dx, dw=gdw, db=gdb, workspace=ws, pads=pads),
            items=d["B"], item_frames=d["T"],
            gpu=lambda n: list(dw.dwconv2d_bwd(d["x"][:n], d["w"], L[:n], d["dy"][:n], pads=pads)), ref=bref,
            tol=[tol, T32, T32])

    stage_rows("stage", ("", "[32,1500,64,256] -> [32,750,32,256] fp32", "dx,dw,db of [32,1500,64,256] fp32"),
               g, None, 4, T32)
    stage_rows("stage", ("_causal", "[32,1500,64,256] -> [32,751,33,256] causal pads fp32",
                         "dx,dw,db of [32,1500,64,256] causal pads fp32"), gc, causal, 4, T32)
    stage_rows("stage", ("_bf16", "[32,1500,64,256] -> [32,750,32,256] bf16 storage",
                         "dx,dw,db of [32,1500,64,256] bf16 storage, fp32 dw/db"), h, None, 2, TBF)
    stage_rows("stage3", ("", "[32,375,20,256] -> [32,188,10,256] fp32 (8x third stage)",
                          "dx,dw,db of [32,375,20,256] fp32 (8x third stage)"), g3, None, 4, T32)
    assert [r["name"] for r in rows] == [n for n, _ in ROW_KERNELS], "ROW_KERNELS is out of date"
    return rows


def oracle_check(rows, target_s: float, time_it: bool = True):
    """Run the oracle on the first n items of every row's batch (n chosen so
    that one pass over the rows takes about target_s of CPU time), timed on
    one pinned core, and compare the GPU path on the same items with it.

    Returns (cpu_baseline dict or None, {row: max |gpu - ref| / (1 + |ref|)})."""
    import torch

    def one_pass(n, keep):
        secs, frames = 0.0, 0
        for r in rows:
            m = min(n, r["items"])
            call = r["ref"](m)
            t = time.perf_counter()
            out = call()
            secs += time.perf_counter() - t
            frames += m * r["item_frames"]
            if keep is not None:
                keep[r["name"]] = (m, out)
        return secs, frames

    # The oracle is single-threaded C; the process is held to one core while
    # it runs, so that nothing else (numpy's own threads) lends it another.
    saved = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if saved:
        os.sched_setaffinity(0, {min(saved)})
    refs = {}
    try:
        s1, _ = one_pass(1, refs if not time_it else None)
        n, secs, frames, reps = 1, 0.0, 0, 0
        if time_it:
            n = int(max(1, min(32, math.floor(target_s / max(s1, 1e-3)))))
            while reps == 0 or secs < target_s:
                ds, df = one_pass(n, refs)
                secs, frames, reps = secs + ds, frames + df, reps + 1
    finally:
        if saved:
            os.sched_setaffinity(0, saved)

    errs = {}
    for r in rows:
        m, ref = refs[r["name"]]
        got = r["gpu"](m)
        torch.cuda.synchronize()
        worst, worst_rel = 0.0, 0.0
        for gt, rf, tol in zip(got, ref, r["tol"]):
            gv = gt.detach().double().cpu().numpy()
            assert gv.shape == rf.shape, (r["name"], gv.shape, rf.shape)
            e = float((abs(gv - rf) / (1.0 + abs(rf))).max()) if gv.size else 0.0
            e = e if math.isfinite(e) else float("inf")
            worst, worst_rel = max(worst, e), max(worst_rel, e / tol)
        errs[r["name"]] = dict(items=m, max_err=worst, max_err_over_tol=worst_rel)
    if not time_it:
        return None, errs
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), None)
    except OSError:
        pass
    cpu = dict(value=round(frames / secs, 1), unit="frames/s", cores=1, kind="oracle",
               cpu_model=model, host_cpus=os.cpu_count(),
               sample=(f"every row of the step on the first {n} items of its batch (at most its batch size), "
                       f"same shapes and lengths, {reps} pass(es): {frames} frames in {secs:.2f} s; the oracle "
                       f"is single-threaded C with fp64 accumulation, run on one pinned core"))
    return cpu, errs


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


def load_probe():
    """The HBM streaming probe library (include/dwprobe.h), or None if it is
    not built."""
    import ctypes
    path = os.path.join(ROOT, "conv_subsampling_amd", "libdwprobe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dw_probe_stream.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_void_p]
    lib.dw_probe_stream.restype = ctypes.c_int
    return lib


def read_kernel_stats(path=None):
    """Per-row kernel-only mean durations (us) from the committed rocprofv3
    summary, if it was taken on the current kernel sources; else {}."""
    path = path or os.path.join(ROOT, "profiles", "kernel_stats_bench_step.txt")
    if not os.path.exists(path):
        return {}
    text = open(path).read().splitlines()
    sha = next((ln.split("=", 1)[1].strip() for ln in text if ln.startswith("# src_sha256=")), None)
    if sha != sources_sha(KERNEL_SOURCES):
        return {}
    names = {n for n, _ in ROW_KERNELS} | {"probe:" + n for n in PROBE_ROWS}
    out = {}
    for ln in text:
        parts = ln.split()  # row, kernel (may hold spaces), n, avg_us, min_us, max_us
        if len(parts) >= 6 and parts[0] in names and parts[-4].isdigit():
            try:
                out[parts[0]] = float(parts[-3])
            except ValueError:
                pass
    return out


# The rows the probe pass copies for, in the order it launches them: every
# HBM-bound row (all but the launch-bound small conv and the ALU-bound front).
PROBE_ROWS = [n for n, _ in ROW_KERNELS if n != "conv1d_small" and not n.startswith("front")]
PROBE_KERNEL = "stream_probe_kernel<2, 18>"

FORWARD_BAR = 0.70   # forward depthwise kernels: at least 70% of peak HBM bandwidth
FORWARD_ROWS = [n for n, _ in ROW_KERNELS if ("conv1d_" in n and "bwd" not in n and n != "conv1d_small")
                or n.startswith("stage") and "_fwd" in n]


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM streaming probe pass")
    ap.add_argument("--no-check", action="store_true",
                    help="skip the oracle comparison and the CPU baseline (profiling runs: only the timed, "
                         "per-row and probe passes dispatch kernels)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--summarize-profile", metavar="DIR", help="summarise rocprofv3 output under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        return 2

    import torch

    dev = torch.device("cuda", 0)
    log("building workloads ...")
    rows = build_rows(dev)
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

    # The probe pass: for every HBM-bound row, the streaming probe moves the
    # row's algorithmic read and write bytes, timed with the same events.
    # Successive probes use successive regions of two 4 GiB buffers, so every
    # probe reads and writes memory no other call touched for at least 4 GiB
    # of traffic: cold, like the rows inside the step.
    probe_us = {}
    plib = None if args.no_probe else load_probe()
    if plib is not None:
        span = 4 << 30
        psrc = torch.empty(span, dtype=torch.uint8, device=dev)
        pdst = torch.empty(span, dtype=torch.uint8, device=dev)
        psrc.fill_(1)
        stream = torch.cuda.current_stream(dev).cuda_stream
        prow = [r for r in rows if r["bound"] == "hbm" and r["read"] <= span and r["write"] <= span]
        assert [r["name"] for r in prow] == PROBE_ROWS, "PROBE_ROWS is out of date"
        pev = {r["name"]: [] for r in prow}
        off = 0
        for s in range(args.steps + 1):
            for r in prow:
                need = max(r["read"], r["write"])
                if off + need > span:
                    off = 0
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                rc = plib.dw_probe_stream(psrc.data_ptr() + off, pdst.data_ptr() + off, r["read"], r["write"], 2,
                                          stream)
                b.record()
                if rc != 0:
                    raise RuntimeError(f"dw_probe_stream failed ({rc}) for {r['name']}")
                if s > 0:  # the first round warms the probe up
                    pev[r["name"]].append((a, b))
                off += (need + 4095) // 4096 * 4096
        torch.cuda.synchronize()
        for name, evs in pev.items():
            ts = [a.elapsed_time(b) * 1e3 for a, b in evs]
            probe_us[name] = sum(ts) / len(ts)
        del psrc, pdst
        log(f"probe pass of {args.steps} steps done")

    kstats = read_kernel_stats()
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
                   kernel_us=kstats.get(r["name"]), probe_kernel_us=kstats.get("probe:" + r["name"]),
                   frames_per_s=round(r["frames"] / (us * 1e-6)), alg_bytes=b,
                   gbps=round(b / (us * 1e-6) / 1e9, 1), hbm_frac=round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                   dense_bytes=r["read_dense"] + r["write"],
                   dense_gbps=round((r["read_dense"] + r["write"]) / (us * 1e-6) / 1e9, 1))
        if r["name"] in probe_us:
            pu = probe_us[r["name"]]
            row.update(probe_us=round(pu, 2), probe_gbps=round(b / (pu * 1e-6) / 1e9, 1),
                       of_probe=round(pu / us, 4))
        row["bound"] = r["bound"]
        if r["bound"] == "alu":
            tf = r["flops"] / (us * 1e-6) / 1e12
            row.update(alg_flops=r["flops"], tflops=round(tf, 2), alu_frac=round(tf / VALU_F32_PEAK_TFLOPS, 4))
        out_rows.append(row)
        extra = f"  probe {row['probe_us']:7.2f} us ({100 * row['of_probe']:.0f}%)" if "probe_us" in row else ""
        log(f"  {r['name']:<24} {us:9.2f} us  {row['gbps']:8.1f} GB/s  ({100 * row['hbm_frac']:.1f}% of 8 TB/s)"
            + extra)

    dom = next(r for r in out_rows if r["row"] == DOMINANT_ROW)
    dom_mean = sum(dom_us) / len(dom_us)
    dom_gbps = round(dom["alg_bytes"] / (dom_mean * 1e-6) / 1e9, 1)
    roofline = dict(kernel=DOMINANT_KERNEL, bound="hbm", achieved=dom_gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                    frac=round(dom_gbps / HBM_PEAK_GBPS, 4), traffic=read_traffic(),
                    launch_us=round(dom_mean, 2), alg_bytes_per_launch=dom["alg_bytes"])
    fwd = [r for r in out_rows if r["row"] in FORWARD_ROWS]
    low = min(fwd, key=lambda r: r["hbm_frac"])
    forward_target = dict(bar=FORWARD_BAR, min_hbm_frac=low["hbm_frac"], row=low["row"],
                          rows_below=[r["row"] for r in fwd if r["hbm_frac"] < FORWARD_BAR],
                          met=all(r["hbm_frac"] >= FORWARD_BAR for r in fwd))
    # the same from the kernels' own durations (the committed rocprofv3 summary),
    # which leave out the dispatch latency that an event pair around a call adds
    kfrac = {r["row"]: round(r["alg_bytes"] / (r["kernel_us"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
             for r in fwd if r.get("kernel_us")}
    if len(kfrac) == len(fwd):
        klow = min(kfrac, key=kfrac.get)
        forward_target["kernel_only"] = dict(min_hbm_frac=kfrac[klow], row=klow,
                                             rows_below=[n for n, v in kfrac.items() if v < FORWARD_BAR],
                                             met=all(v >= FORWARD_BAR for v in kfrac.values()))

    cpu, worst = None, None
    if not args.no_check:
        log("running the oracle on a sample of every row, and the GPU path on the same items ...")
        cpu, errs = oracle_check(rows, args.cpu_seconds, time_it=not args.no_cpu_baseline)
        for row in out_rows:
            e = errs[row["row"]]
            row.update(max_err=float(f"{e['max_err']:.3e}"), max_err_over_tol=round(e["max_err_over_tol"], 4),
                       err_items=e["items"])
        if cpu:
            log(f"  oracle: {cpu['value']:.0f} frames/s ({cpu['sample']})")
        worst = max(out_rows, key=lambda r: r["max_err_over_tol"])
        log(f"  worst error against the oracle: {worst['row']} {worst['max_err']:.2e} "
            f"({worst['max_err_over_tol']:.3f} of its tolerance)")

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
        "dtype": "mixed: f32 arithmetic on f32 or bf16 storage (bf16 rows say so); f64 weight-gradient sums",
        "data": "synthetic (seeded; log-mel-shaped inputs, lengths ~U[T/2,T])",
        "config": {
            "workload": "encoder depthwise path: small dwconv1d [2,64,8] K9; fused front [4,1000,80] fwd+bwd "
                        "(symmetric and causal); conv-module dwconv1d [16,750,1024] K9 bf16; causal dwconv1d "
                        "[32,1500,512] K3/4/5/9/15 (K9 fwd+bwd) and [32,1500,200] K9; streaming dwconv1d "
                        "1024x8x1024 K9 bf16 with cache; depthwise conv2d stage [32,1500,64,256] fwd+bwd "
                        "(symmetric fp32, causal fp32, symmetric bf16); third stage [32,375,20,256] fwd+bwd",
            "frames_per_step": frames,
            "alg_bytes_per_step": alg,
            "parallelism": "single GPU",
        },
        "hbm": {"achieved_gbps": round(alg / (ms_step * 1e-3) / 1e9, 1), "peak_gbps": HBM_PEAK_GBPS,
                "frac": round(alg / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "forward_target": forward_target,
        "max_err_over_tol": worst["max_err_over_tol"] if worst else None,
        "rows": out_rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


# --------------------------------------------------------------------------
# rocprofv3 summaries
# --------------------------------------------------------------------------

def kernel_short_name(name):
    """A kernel's name without 'void ', namespaces that hide it, or its argument list."""
    name = name[5:] if name.startswith("void ") else name
    name = name.replace("(anonymous namespace)::", "")
    return name.split("(")[0]


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


FRONT_SQ_PASSES = {
    "sq1": ["SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
            "SQ_WAIT_INST_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_BUSY_CYCLES"],
    "sq2": ["SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_VALU_FMA_F64", "SQ_INSTS_VALU_CVT", "SQ_INSTS_SALU",
            "SQ_WAVE_CYCLES", "SQ_INSTS_VMEM_RD", "SQ_INSTS_VALU_MUL_F64", "SQ_INSTS_VALU_ADD_F64"],
}


def front_sq_summary(d, cmd):
    """Text summary of the front kernels' SQ counters (d/sq1, d/sq2), with the
    VALU-busy fraction against their kernel-only durations in d/stats; None if
    the counter runs are missing."""
    if not all(_csv_rows(os.path.join(d, k, "**", "*counter_collection.csv")) for k in FRONT_SQ_PASSES):
        return None
    per = {}
    for k in FRONT_SQ_PASSES:
        for r in _csv_rows(os.path.join(d, k, "**", "*counter_collection.csv")):
            name = r.get("Kernel_Name", "")
            if "dwsub_fused" not in name:
                continue
            short = kernel_short_name(name)
            per.setdefault(short, {}).setdefault((k, r["Dispatch_Id"]), {})
            dct = per[short][(k, r["Dispatch_Id"])]
            dct[r["Counter_Name"]] = dct.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    stats = {}
    for r in _csv_rows(os.path.join(d, "stats", "**", "*kernel_stats.csv")):
        name = r.get("Name", r.get("KernelName", "?"))
        stats[kernel_short_name(name)] = float(r.get("AverageNs", 0)) / 1e3
    lines = ["# SQ counters of the fused front's kernels on one MI355X, two counter passes over a short bench.py run",
             "# sq1: " + cmd("sq1"), "# sq2: " + cmd("sq2"),
             "# Values are means per dispatch (the symmetric and causal forward share one kernel name).",
             "# VALU-busy = SQ_INSTS_VALU x 4 cycles (a wave64 vector instruction on a 16-lane SIMD) / 1024",
             "# SIMDs / 2.4 GHz, against the kernel-only mean duration of the kernel-trace run (stats).", ""]
    for short in sorted(per):
        byp = {}
        for (k, did), vals in per[short].items():
            for cn, v in vals.items():
                byp.setdefault(cn, []).append(v)
        mean = {cn: sum(v) / len(v) for cn, v in byp.items()}
        ndisp = max(len(v) for v in byp.values())
        lines.append(f"kernel: {short.replace('dw::', '')}   dispatches per pass: {ndisp}")
        for cn in FRONT_SQ_PASSES["sq1"] + FRONT_SQ_PASSES["sq2"]:
            if cn in mean:
                lines.append(f"  {cn:<28} {mean[cn]:>12.4g}")
        dur = stats.get(short)
        if dur and "SQ_INSTS_VALU" in mean:
            busy = mean["SQ_INSTS_VALU"] * 4 / 1024 / 2.4e3
            lines.append(f"  VALU issue time {busy:6.2f} us of a {dur:.2f} us kernel: {100 * busy / dur:.0f}% VALU-busy")
        lines.append("")
    return "\n".join(lines) + "\n"


# Memory-side counters of every row's main kernel and of its probe copy,
# one rocprofv3 --pmc run per pass (derived counters are computed by rocprofv3).
MEM_PASSES = {
    "memA": ["VmemLatency", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES"],
    "memB": ["MeanOccupancyPerCU", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_ANY"],
    "memC": ["TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum"],
    "memD": ["TCC_EA0_WRREQ_LEVEL_sum", "TCC_EA0_WRREQ_sum"],
}


def mem_counter_summary(d, cmd):
    """Text summary of the MEM_PASSES counters per bench row (its main
    kernel's dispatches) and per probe copy; None if a pass is missing."""
    per_pass = {}
    for k in MEM_PASSES:
        rows = _csv_rows(os.path.join(d, k, "**", "*counter_collection.csv"))
        if not rows:
            return None
        disp = {}
        for r in rows:
            did = r.get("Dispatch_Id")
            name, vals = disp.get(did, (r.get("Kernel_Name", ""), {}))
            cn = r.get("Counter_Name")
            vals[cn] = vals.get(cn, 0.0) + float(r.get("Counter_Value", 0))
            disp[did] = (name, vals)
        per_pass[k] = [(did, name, vals) for did, (name, vals) in disp.items()]
        if "--no-check" not in cmd(k):
            # rows are matched to dispatches by their order (see the traffic summary)
            raise SystemExit(f"{k} counter run was taken without --no-check; take it again with --no-check")
    table = {}
    for k, disp in per_pass.items():
        for name, v in attribute_dispatches(disp).items():
            for vals in v:
                for cn, x in vals.items():
                    table.setdefault(name, {}).setdefault(cn, []).append(x)
        probes = [vals for _, kn, vals in sorted(disp, key=lambda t: int(t[0]))
                  if kernel_short_name(kn) == PROBE_KERNEL]
        if probes and len(probes) % len(PROBE_ROWS) == 0:
            for j, name in enumerate(PROBE_ROWS):
                for vals in probes[len(PROBE_ROWS) + j::len(PROBE_ROWS)]:
                    for cn, x in vals.items():
                        table.setdefault("probe:" + name, {}).setdefault(cn, []).append(x)
    mean = lambda v: sum(v) / len(v) if v else float("nan")
    lines = ["# Memory-side counters per bench row's main kernel and per probe copy, on one MI355X",
             *[f"# {k}: " + cmd(k) for k in MEM_PASSES],
             f"# src_sha256={sources_sha(KERNEL_SOURCES)}",
             "# Means per dispatch.  occ: MeanOccupancyPerCU (waves resident per CU); vmem_lat:",
             "# VmemLatency (cycles a vector memory instruction is in flight); wait: SQ_WAIT_ANY /",
             "# SQ_WAVE_CYCLES (both in quad-cycles: the share of wave time spent waiting);",
             "# rd_lat, wr_lat: TCC_EA0_RDREQ_LEVEL_sum / TCC_EA0_RDREQ_sum and the same for writes",
             "# (cycles an L2-to-memory request is in flight).",
             f"{'row':<30} {'occ':>6} {'vmem_lat':>9} {'wait':>6} {'rd_lat':>8} {'wr_lat':>8}"]
    order = [n for n, _ in ROW_KERNELS]
    names = [n for n in order if n in table]
    names += ["probe:" + n for n in PROBE_ROWS if "probe:" + n in table]
    for name in names:
        t = {cn: mean(v) for cn, v in table[name].items()}
        occ = t.get("MeanOccupancyPerCU", float("nan"))
        vl = t.get("VmemLatency", float("nan"))
        wc = t.get("SQ_WAVE_CYCLES", 0.0)
        wait = t.get("SQ_WAIT_ANY", float("nan")) / wc if wc else float("nan")
        rq, wq = t.get("TCC_EA0_RDREQ_sum", 0.0), t.get("TCC_EA0_WRREQ_sum", 0.0)
        rl = t.get("TCC_EA0_RDREQ_LEVEL_sum", float("nan")) / rq if rq else float("nan")
        wl = t.get("TCC_EA0_WRREQ_LEVEL_sum", float("nan")) / wq if wq else float("nan")
        lines.append(f"{name:<30} {occ:>6.1f} {vl:>9.0f} {wait:>6.2f} {rl:>8.0f} {wl:>8.0f}")
    return "\n".join(lines) + "\n"


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
    if stats and "--no-check" not in cmd("stats"):
        # rows are matched to dispatches by their order: the oracle check's
        # sub-batch calls would be averaged into the rows' kernel-only times
        raise SystemExit("the kernel-trace run was taken without --no-check; take it again with --no-check")
    if stats:
        lines = ["# rocprofv3 --kernel-trace --stats, one bench.py run on one MI355X",
                 "# command: " + cmd("stats"),
                 f"# src_sha256={sources_sha(KERNEL_SOURCES)}",
                 "# per kernel name (every dispatch of the run: warm-up, timed and per-row steps):",
                 f"{'kernel':<60} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}"]
        for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0) or 0)):
            name = r.get("Name", r.get("KernelName", "?"))
            short = kernel_short_name(name)[:60]
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
            # the probe pass: one probe per HBM-bound row per round, in PROBE_ROWS order; the
            # first round warms up
            probes = [du for _, kn, du in sorted(disp, key=lambda t: int(t[0]))
                      if kernel_short_name(kn) == PROBE_KERNEL]
            if probes and len(probes) % len(PROBE_ROWS) == 0:
                lines += ["", "# the probe pass: a plain copy of each HBM-bound row's read and write bytes (rounds",
                          "# after the first), kernel-only durations",
                          f"{'row':<24} {'kernel':<52} {'n':>4} {'avg_us':>9} {'min_us':>9} {'max_us':>9}"]
                for k, name in enumerate(PROBE_ROWS):
                    v = probes[len(PROBE_ROWS) + k::len(PROBE_ROWS)]
                    if v:
                        lines.append(f"probe:{name:<18} {PROBE_KERNEL:<52} {len(v):>4} {sum(v) / len(v):>9.2f} "
                                     f"{min(v):>9.2f} {max(v):>9.2f}")
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

    mem = mem_counter_summary(d, cmd)
    if mem:
        with open(os.path.join(ROOT, "profiles", "row_memory_counters.txt"), "w") as fh:
            fh.write(mem)
        print(mem)

    sq = front_sq_summary(d, cmd)
    if sq:
        with open(os.path.join(ROOT, "profiles", "dwsub_front_sq_counters.txt"), "w") as fh:
            fh.write(sq)
        print(sq)

    fetch = counter("fetch", "FETCH_SIZE")
    write = counter("write", "WRITE_SIZE")
    if not (fetch and write):
        return
    # Rows are matched to dispatches by their order, so the counter runs must
    # not include the oracle check, whose sub-batch calls dispatch the same
    # kernels on fewer items and would be averaged into the rows' bytes.
    for k in ("fetch", "write"):
        if "--no-check" not in cmd(k):
            raise SystemExit(f"{k} counter run was taken without --no-check: its per-row bytes would mix in "
                             "the oracle check's dispatches; take it again with --no-check")
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
