"""Host-side logic that needs no GPU: the binding's output-shape helpers
against the oracle's definitions, and the profile summaries' attribution of
kernel dispatches to bench rows."""
import itertools

import pytest

import oracle


def lib():
    import conv_subsampling_amd as dw
    return dw


@pytest.mark.parametrize("T,F", [(0, 0), (1, 1), (2, 3), (7, 80), (1000, 80), (1500, 64), (375, 20)])
def test_conv2d_out_shape_matches_the_oracle(T, F):
    for pads in itertools.product((1, 2), (0, 1, 2), (1, 2), (0, 1, 2)):
        To, Fo = lib().conv2d_out_shape(T, F, pads=pads)
        assert To == oracle.conv_out_len(T, 3, 2, pads[0], pads[1])
        assert Fo == oracle.conv_out_len(F, 3, 2, pads[2], pads[3])
    assert lib().conv2d_out_shape(T, F) == (oracle.conv_out_len(T, 3, 2, 1), oracle.conv_out_len(F, 3, 2, 1))


@pytest.mark.parametrize("T,F", [(0, 0), (0, 4), (1, 1), (2, 3), (5, 0), (13, 9), (1000, 80), (999, 79)])
@pytest.mark.parametrize("causal", [False, True])
def test_front_out_shape_matches_the_oracle(T, F, causal):
    pl, ph = oracle.front_pads(causal)
    T1, F1 = oracle.conv_out_len(T, 3, 2, pl, ph), oracle.conv_out_len(F, 3, 2, pl, ph)
    ref = (oracle.conv_out_len(T1, 3, 2, pl, ph), oracle.conv_out_len(F1, 3, 2, pl, ph))
    assert lib().front_out_shape(T, F, causal) == ref


def test_causal_pads_constant():
    assert lib().CAUSAL_PADS_2D == (2, 1, 2, 1)


def test_dispatch_attribution_by_occurrence_within_a_step():
    import bench
    rows = bench.ROW_KERNELS
    # three steps of dispatches in row order, with unrelated kernels interleaved
    disp, i = [], 0
    for step in range(3):
        for name, prefix in rows:
            disp.append((i, "void at::native::fill_kernel(...)", None))
            disp.append((i + 1, "void " + prefix + "float const*)", (step, name)))
            i += 2
    got = bench.attribute_dispatches(list(reversed(disp)))
    for name, _ in rows:
        assert got[name] == [(s, name) for s in range(3)], name


def test_dispatch_attribution_refuses_a_partial_step():
    import bench
    name, prefix = bench.ROW_KERNELS[-1]
    same = [n for n, p in bench.ROW_KERNELS if p == prefix]
    assert len(same) > 1  # the last row shares its kernel with earlier rows
    disp = [(k, prefix + ")", k) for k in range(len(same) + 1)]   # one dispatch too many
    assert bench.attribute_dispatches(disp)[name] == []


def test_import_without_the_library_fails_loudly(tmp_path):
    """The binding has no other implementation: without libdwconv.so the
    package refuses to import, naming the missing file."""
    import os
    import shutil
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    pkg = tmp_path / "conv_subsampling_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(root, "conv_subsampling_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import conv_subsampling_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libdwconv.so is missing" in r.stderr
