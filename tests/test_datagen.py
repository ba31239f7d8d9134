"""The seeded input generators (CPU): draws repeat, streams are independent,
and each workload recipe has the shapes, value distributions and length mixes
it states."""
import hashlib
import subprocess
import sys
import os

import numpy as np
import pytest
import torch

import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _digest(t):
    return hashlib.sha256(t.contiguous().view(torch.uint8).numpy().tobytes()).hexdigest()


RECIPES = {
    "conv1d_small": lambda: datagen.conv1d_small(),
    "fused_front": lambda: datagen.fused_front(B=2, T=100, F=16, C=8),
    "conv1d_encoder_bf16": lambda: datagen.conv1d_encoder_bf16(B=3, T=40, C=16),
    "conv1d_causal_sweep": lambda: datagen.conv1d_causal_sweep(9, B=3, T=50, C=8),
    "conv1d_stream": lambda: datagen.conv1d_stream(B=4, Tc=8, C=16),
    "conv2d_stage": lambda: datagen.conv2d_stage(B=2, T=20, F=8, C=4),
}


def _all_digests():
    out = {}
    for name, make in RECIPES.items():
        for k, v in make().items():
            if isinstance(v, torch.Tensor):
                out[f"{name}/{k}"] = _digest(v)
    return out


def test_draws_repeat_in_one_process():
    assert _all_digests() == _all_digests()


def test_draws_repeat_in_a_fresh_process():
    """The bench and the tests draw in separate processes: the same (seed,
    stream) must give the same bits there (no dependence on global RNG state
    or hash randomisation)."""
    torch.manual_seed(1234)  # global state must not matter
    here = _all_digests()
    code = ("import sys, json; sys.path.insert(0, %r); sys.path.insert(0, %r);"
            "import test_datagen as t; print(json.dumps(t._all_digests()))") % (ROOT, os.path.join(ROOT, "tests"))
    env = dict(os.environ, PYTHONHASHSEED="12345")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    import json
    assert json.loads(r.stdout.strip().splitlines()[-1]) == here


def test_streams_and_seeds_are_independent():
    a = datagen.normal((1000,), 1.0, "s/a")
    b = datagen.normal((1000,), 1.0, "s/b")
    a1 = datagen.normal((1000,), 1.0, "s/a", seed=1)
    assert not torch.equal(a, b) and not torch.equal(a, a1)
    # distinct streams are uncorrelated draws, not shifted copies
    assert abs(float(np.corrcoef(a.numpy(), b.numpy())[0, 1])) < 0.15


def test_normal_takes_the_variance_and_uniform_its_range():
    x = datagen.normal((200_000,), 1.0 / 9, "v/x")
    assert abs(float(x.mean())) < 0.01 and abs(float(x.var()) - 1.0 / 9) < 0.005
    u = datagen.uniform((200_000,), -1.0 / 3, 1.0 / 3, "v/u")
    assert float(u.min()) >= -1.0 / 3 and float(u.max()) <= 1.0 / 3
    assert abs(float(u.var()) - (2.0 / 3) ** 2 / 12) < 0.002
    n = datagen.int_uniform(100_000, 750, 1500, "v/n")
    assert n.dtype == torch.int32 and int(n.min()) == 750 and int(n.max()) == 1500


def test_recipes_shapes_dtypes_and_lengths():
    c = datagen.conv1d_small()
    assert c["x"].shape == (2, 64, 8) and c["w"].shape == (9, 8) and c["lengths"].tolist() == [64, 41]
    assert float(c["w"].abs().max()) <= 1.0 / 3
    f = datagen.fused_front()
    assert f["x"].shape == (4, 1000, 80) and f["w0"].shape == (3, 3, 256)
    assert all(500 <= int(v) <= 1000 for v in f["lengths"])
    e = datagen.conv1d_encoder_bf16(B=4, T=750, C=64)
    assert e["x"].dtype == torch.bfloat16 and all(375 <= int(v) <= 750 for v in e["lengths"])
    # the bf16 tensors are the fp32 draws rounded to nearest even
    assert torch.equal(e["x"], datagen.normal((4, 750, 64), 1.0, "c3/x").to(torch.bfloat16))
    s = datagen.conv1d_causal_sweep(15, B=32, T=1500, C=200)
    assert s["w"].shape == (15, 200) and float(s["b"].abs().max()) == 0.0
    assert all(750 <= int(v) <= 1500 for v in s["lengths"])
    st = datagen.conv2d_stage(B=2, T=30, F=16, C=8)
    assert float(st["x"].min()) >= 0.0 and st["dy"].shape == (2, 15, 8, 8)
    stc = datagen.conv2d_stage(B=2, T=30, F=16, C=8, dy_rows_cols=(16, 9), bf16=True)
    assert stc["dy"].shape == (2, 16, 9, 8) and stc["x"].dtype == torch.bfloat16
    assert torch.equal(stc["x"], st["x"].to(torch.bfloat16))


@pytest.mark.parametrize("K", [3, 4, 5, 9, 15])
def test_causal_sweep_draws_differ_per_width(K):
    a = datagen.conv1d_causal_sweep(K, B=2, T=10, C=4)["x"]
    b = datagen.conv1d_causal_sweep(9 if K != 9 else 3, B=2, T=10, C=4)["x"]
    assert not torch.equal(a, b)
