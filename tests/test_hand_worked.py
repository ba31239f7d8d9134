"""Hand-worked examples (tests/golden/hand_worked.json) against the oracle on
the CPU and against the HIP path on the GPU.

Each case is a tiny input whose outputs were worked out by hand from the
definition the case cites, with the working and an identity check stored
beside the values.  The values are small integers and halves: every product
and partial sum is exact in float32 and in float64, so both sides must match
them exactly, whatever their summation order.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
with open(os.path.join(HERE, "golden", "hand_worked.json")) as _f:
    CASES = json.load(_f)["cases"]
IDS = [c["name"] for c in CASES]


def _a(v):
    return np.asarray(v, dtype=np.float32)


def run_oracle(case):
    a, op = case["args"], case["op"]
    L = np.asarray(a["lengths"], dtype=np.int32)
    if op == "dwconv1d_fwd":
        return {"y": oracle.dwconv1d_fwd(_a(a["x"]), _a(a["w"]), _a(a["b"]), L, a["causal"])}
    if op == "dwconv1d_bwd":
        dx, dw, db = oracle.dwconv1d_bwd(_a(a["x"]), _a(a["w"]), L, _a(a["dy"]), a["causal"])
        return {"dx": dx, "dw": dw, "db": db}
    if op == "dwconv1d_stream_fwd":
        y, cache = oracle.dwconv1d_stream_fwd(_a(a["x"]), _a(a["w"]), _a(a["b"]), L, _a(a["cache"]))
        return {"y": y, "cache": cache}
    if op == "dwconv2d_fwd":
        return {"y": oracle.dwconv2d_fwd(_a(a["x"]), _a(a["w"]), _a(a["b"]), L, pads=a["pads"])}
    if op == "dwconv2d_bwd":
        dx, dw, db = oracle.dwconv2d_bwd(_a(a["x"]), _a(a["w"]), L, _a(a["dy"]), pads=a["pads"])
        return {"dx": dx, "dw": dw, "db": db}
    if op == "dwsub_fused_fwd":
        return {"y": oracle.dwsub_front_fwd(_a(a["x"]), _a(a["w0"]), _a(a["b0"]), _a(a["w1"]), _a(a["b1"]), L,
                                            causal=a["causal"])}
    if op == "dwsub_fused_bwd":
        dw0, db0, dw1, db1 = oracle.dwsub_front_bwd(_a(a["x"]), _a(a["w0"]), _a(a["b0"]), _a(a["w1"]), L,
                                                    _a(a["dy"]), causal=a["causal"])
        return {"dw0": dw0, "db0": db0, "dw1": dw1, "db1": db1}
    raise AssertionError(f"unknown op {op}")


def run_gpu(case, dtype):
    import conv_subsampling_amd as dw
    dev = torch.device("cuda", 0)
    a, op = case["args"], case["op"]
    t = lambda k: torch.tensor(a[k], dtype=torch.float32).to(dtype).to(dev)
    L = torch.tensor(a["lengths"], dtype=torch.int32, device=dev)
    if op == "dwconv1d_fwd":
        out = {"y": dw.dwconv1d_fwd(t("x"), t("w"), t("b"), L, causal=a["causal"])}
    elif op == "dwconv1d_bwd":
        dx, dwt, db = dw.dwconv1d_bwd(t("x"), t("w"), L, t("dy"), causal=a["causal"])
        out = {"dx": dx, "dw": dwt, "db": db}
    elif op == "dwconv1d_stream_fwd":
        y, cache = dw.dwconv1d_stream_fwd(t("x"), t("w"), t("b"), L, t("cache"))
        out = {"y": y, "cache": cache}
    elif op == "dwconv2d_fwd":
        out = {"y": dw.dwconv2d_fwd(t("x"), t("w"), t("b"), L, pads=a["pads"])}
    elif op == "dwconv2d_bwd":
        dx, dwt, db = dw.dwconv2d_bwd(t("x"), t("w"), L, t("dy"), pads=a["pads"])
        out = {"dx": dx, "dw": dwt, "db": db}
    elif op == "dwsub_fused_fwd":
        out = {"y": dw.dwsub_fused_fwd(t("x"), t("w0"), t("b0"), t("w1"), t("b1"), L, causal=a["causal"])}
    elif op == "dwsub_fused_bwd":
        dw0, db0, dw1, db1 = dw.dwsub_fused_bwd(t("x"), t("w0"), t("b0"), t("w1"), L, t("dy"), causal=a["causal"])
        out = {"dw0": dw0, "db0": db0, "dw1": dw1, "db1": db1}
    else:
        raise AssertionError(f"unknown op {op}")
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy().astype(np.float64) for k, v in out.items()}


def check(got, case, who):
    for k, want in case["expect"].items():
        w = np.asarray(want, dtype=np.float64)
        g = np.asarray(got[k])
        assert g.shape == w.shape, f"{case['name']} {who} {k}: shape {g.shape} != {w.shape}"
        assert np.array_equal(g, w), f"{case['name']} {who} {k}:\n{g}\n!=\n{w}"


def test_fixture_is_well_formed():
    names = set()
    for c in CASES:
        assert c["name"] not in names
        names.add(c["name"])
        assert c["cite"] and c["derivation"] and c["expect"]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_oracle_matches_hand_worked(case):
    check(run_oracle(case), case, "oracle")


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_gpu_matches_hand_worked(case, dtype):
    print(f"hand-worked {case['name']} {dtype}", flush=True)
    check(run_gpu(case, dtype), case, f"gpu {dtype}")
