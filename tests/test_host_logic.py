"""Host-side logic that needs no GPU: the binding's output-shape helpers
against the oracle's definitions, and the profile summaries' attribution of
kernel dispatches to bench rows."""
import itertools
import os

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


def test_bench_reads_kernel_only_times_of_current_sources(tmp_path):
    """Per-row kernel-only times come from the rocprofv3 summary only when it
    was taken on the current kernel sources."""
    import bench
    name, prefix = bench.ROW_KERNELS[3]
    body = [f"# src_sha256={bench.sources_sha(bench.KERNEL_SOURCES)}",
            f"{'row':<24} {'kernel':<52} {'n':>4} {'avg_us':>9} {'min_us':>9} {'max_us':>9}",
            f"{name:<24} {prefix.replace('dw::', '').rstrip('('):<52} {12:>4} {36.25:>9.2f} {35.0:>9.2f} {38.0:>9.2f}"]
    p = tmp_path / "stats.txt"
    p.write_text("\n".join(body) + "\n")
    assert bench.read_kernel_stats(str(p)) == {name: 36.25}
    p.write_text("\n".join(["# src_sha256=0000"] + body[1:]) + "\n")
    assert bench.read_kernel_stats(str(p)) == {}


def test_bench_forward_rows_are_the_forward_depthwise_kernels():
    import bench
    assert set(bench.FORWARD_ROWS) == {
        "conv1d_bf16", "conv1d_causal_K3_C512", "conv1d_causal_K4_C512", "conv1d_causal_K5_C512",
        "conv1d_causal_K9_C512", "conv1d_causal_K15_C512", "conv1d_causal_K9_C200", "conv1d_stream_bf16",
        "stage_fwd", "stage_fwd_causal", "stage_fwd_bf16", "stage3_fwd"}


def test_traffic_summary_refuses_counter_runs_taken_with_the_oracle_check(tmp_path):
    """Rows are matched to counter dispatches by their order; a run that also
    ran the oracle check has extra sub-batch dispatches, so it is refused."""
    import bench
    for kind, cname in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        d = tmp_path / kind
        d.mkdir()
        (d / "command.txt").write_text("rocprofv3 --pmc " + cname + " -- python3 bench.py --steps 1 --calib-copy\n")
        (d / "run_counter_collection.csv").write_text(
            "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n1,copyBuffer,%s,1048576\n" % cname)
    with pytest.raises(SystemExit, match="--no-check"):
        bench.summarize_profile(str(tmp_path))


def _write_mem_passes(d, with_check=False):
    """Counter CSVs for every memory-side pass: one step of row dispatches
    (dispatch i of the step carries value i + 1) and two probe rounds."""
    import bench
    rows = bench.ROW_KERNELS
    for k, counters in bench.MEM_PASSES.items():
        p = d / k
        p.mkdir()
        flags = "--steps 1" + ("" if with_check else " --no-check")
        (p / "command.txt").write_text(f"rocprofv3 --pmc {' '.join(counters)} -- python3 bench.py {flags}\n")
        lines = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        did = 0
        for i, (_, prefix) in enumerate(rows):
            did += 1
            for cn in counters:
                lines.append(f'{did},"void {prefix}float const*)",{cn},{(i + 1) * (2 if "LEVEL" in cn else 1)}')
        for _ in range(2):
            for _ in bench.PROBE_ROWS:
                did += 1
                for cn in counters:
                    lines.append(f'{did},"void {bench.PROBE_KERNEL}(uint4 const*)",{cn},{3 if "LEVEL" in cn else 1}')
        (p / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_memory_counter_summary_attributes_rows_and_probes(tmp_path):
    import bench
    _write_mem_passes(tmp_path)
    cmd = lambda k: (tmp_path / k / "command.txt").read_text().strip()
    text = bench.mem_counter_summary(str(tmp_path), cmd)
    got = {ln.split()[0]: ln.split()[1:] for ln in text.splitlines() if ln and not ln.startswith("#")}
    # a row's read latency is its LEVEL sum over its request count: 2 (i + 1) / (i + 1)
    for i, (name, prefix) in enumerate(bench.ROW_KERNELS):
        same = [n for n, p in bench.ROW_KERNELS if p == prefix]
        if len(same) == 1:
            occ, vl, wait, rd, wr = map(float, got[name])
            assert occ == i + 1 and vl == i + 1 and wait == 1.0 and rd == 2.0 and wr == 2.0, name
    for name in bench.PROBE_ROWS:
        assert list(map(float, got["probe:" + name]))[3:] == [3.0, 3.0]


def test_memory_counter_summary_refuses_runs_with_the_oracle_check(tmp_path):
    import bench
    _write_mem_passes(tmp_path, with_check=True)
    cmd = lambda k: (tmp_path / k / "command.txt").read_text().strip()
    with pytest.raises(SystemExit, match="--no-check"):
        bench.mem_counter_summary(str(tmp_path), cmd)


def test_row_kernel_names_exist_in_the_library():
    """Every bench row's kernel name (which the profile summaries match
    against rocprofv3's demangled names) names a kernel the library holds."""
    import shutil
    import subprocess
    import bench
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib = os.path.join(root, "conv_subsampling_amd", "libdwconv.so")
    plib = os.path.join(root, "conv_subsampling_amd", "libdwprobe.so")
    if not (shutil.which("nm") and os.path.exists(lib) and os.path.exists(plib)):
        pytest.skip("nm or the built libraries are missing")
    syms = subprocess.run(["nm", "-C", lib, plib], capture_output=True, text=True, check=True).stdout
    for name, prefix in bench.ROW_KERNELS:
        assert "void " + prefix in syms, (name, prefix)
    assert bench.PROBE_KERNEL + "(" in syms
