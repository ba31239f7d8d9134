"""The C-ABI library on the host: it loads, exports every entry point the
header declares, and rejects bad arguments before touching the GPU.

Argument validation happens on the host before anything is enqueued, so these
calls pass dummy non-null addresses that are never dereferenced."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dwconv.h")
LIB = os.path.join(ROOT, "conv_subsampling_amd", "libdwconv.so")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4
P = ctypes.c_void_p(0x1000)      # dummy device addresses, never dereferenced
Q = ctypes.c_void_p(0x2000)
N = None


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "libdwconv.so is not built"
    lib = ctypes.CDLL(LIB)
    i64, vp, sz, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.dw_last_error.restype = ctypes.c_char_p
    lib.dwconv1d_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i, i, vp]
    lib.dwsub_fused_fwd.argtypes = [vp] * 7 + [i64] * 4 + [vp]
    lib.dwconv2d_fwd.argtypes = [vp] * 5 + [i64] * 8 + [vp]
    lib.dwconv2d_bwd_workspace_bytes.argtypes = [i64] * 8
    lib.dwconv2d_bwd_workspace_bytes.restype = sz
    lib.dwconv2d_bwd.argtypes = [vp] * 8 + [sz] + [i64] * 8 + [vp]
    lib.dwconv2d_fwd_ex.argtypes = [vp] * 5 + [i64] * 11 + [i, vp]
    lib.dwconv2d_bwd_workspace_bytes_ex.argtypes = [i64] * 11
    lib.dwconv2d_bwd_workspace_bytes_ex.restype = sz
    lib.dwconv2d_bwd_ex.argtypes = [vp] * 8 + [sz] + [i64] * 11 + [i, vp]
    lib.dwconv1d_bwd_workspace_bytes.argtypes = [i64] * 4
    lib.dwconv1d_stream_fwd.argtypes = [vp] * 7 + [i64] * 4 + [i, vp]
    lib.dwconv1d_bwd_workspace_bytes.restype = sz
    lib.dwconv1d_bwd.argtypes = [vp] * 8 + [sz] + [i64] * 4 + [i, i, vp]
    lib.dwsub_fused_bwd_workspace_bytes.argtypes = [i64] * 4
    lib.dwsub_fused_bwd_workspace_bytes.restype = sz
    lib.dwsub_fused_bwd.argtypes = [vp] * 11 + [sz] + [i64] * 4 + [vp]
    lib.dwsub_fused_fwd_ex.argtypes = [vp] * 7 + [i64] * 4 + [i, i, vp]
    lib.dwsub_fused_bwd_workspace_bytes_ex.argtypes = [i64] * 4 + [i]
    lib.dwsub_fused_bwd_workspace_bytes_ex.restype = sz
    lib.dwsub_fused_bwd_ex.argtypes = [vp] * 11 + [sz] + [i64] * 4 + [i, i, vp]
    lib.dwconv2d_bwd_noalloc.argtypes = [vp] * 7 + [i64] * 11 + [i, vp]
    return lib


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_header_declares_the_four_operations():
    names = declared_functions()
    for f in ("dwconv1d_fwd", "dwconv1d_stream_fwd", "dwconv1d_bwd", "dwconv1d_bwd_workspace_bytes", "dwsub_fused_fwd", "dwsub_fused_bwd", "dwsub_fused_bwd_workspace_bytes",
              "dwconv2d_fwd", "dwconv2d_bwd", "dwconv2d_bwd_workspace_bytes", "dwconv2d_fwd_ex", "dwconv2d_bwd_ex",
              "dwconv2d_bwd_workspace_bytes_ex", "dwsub_fused_fwd_ex", "dwsub_fused_bwd_ex",
              "dwsub_fused_bwd_workspace_bytes_ex", "dw_abi_version", "dw_last_error"):
        assert f in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"libdwconv.so does not export {name}"


def test_abi_version(lib):
    assert lib.dw_abi_version() == 1


def err(lib):
    return lib.dw_last_error().decode()


def test_dwconv1d_validation(lib):
    f = lib.dwconv1d_fwd
    assert f(P, P, N, N, Q, 2, 8, 4, 0, 0, 0, N) == INVALID and "K=0" in err(lib)
    assert f(N, P, N, N, Q, 2, 8, 4, 3, 0, 0, N) == INVALID and "NULL" in err(lib)
    assert f(P, N, N, N, Q, 2, 8, 4, 3, 0, 0, N) == INVALID
    assert f(P, P, N, N, N, 2, 8, 4, 3, 0, 0, N) == INVALID
    assert f(P, P, N, N, P, 2, 8, 4, 3, 0, 0, N) == INVALID and "alias" in err(lib)
    assert f(P, P, N, N, Q, -1, 8, 4, 3, 0, 0, N) == INVALID and "negative" in err(lib)
    assert f(P, P, N, N, Q, 2, -8, 4, 3, 0, 0, N) == INVALID
    assert f(P, P, N, N, Q, 2, 8, 4, 3, 7, 0, N) == INVALID and "pad" in err(lib)
    assert f(P, P, N, N, Q, 2, 8, 4, 3, 0, 9, N) == INVALID and "dtype" in err(lib)
    # empty problems enqueue nothing and succeed
    assert f(P, P, N, N, Q, 0, 8, 4, 3, 0, 0, N) == OK and err(lib) == ""
    assert f(N, N, N, N, N, 0, 8, 4, 3, 0, 0, N) == OK
    assert f(P, P, N, N, Q, 2, 0, 4, 3, 1, 1, N) == OK
    assert f(P, P, N, N, Q, 2, 8, 0, 3, 1, 1, N) == OK


def test_dwconv1d_stream_validation(lib):
    f = lib.dwconv1d_stream_fwd
    R, S = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    # x, w, bias, lengths, cache_in, y, cache_out, B, Tc, C, K, dtype, stream
    assert f(P, P, N, N, R, Q, R, 4, 8, 16, 9, 0, N) == INVALID and "different" in err(lib)
    assert f(P, P, N, N, R, Q, N, 4, 8, 16, 9, 0, N) == INVALID
    assert f(P, P, N, N, R, P, S, 4, 8, 16, 9, 0, N) == INVALID and "alias" in err(lib)
    assert f(P, P, N, N, R, R, S, 4, 8, 16, 9, 0, N) == INVALID
    assert f(P, P, N, N, R, Q, S, 4, 8, 16, 0, 0, N) == INVALID and "K=0" in err(lib)
    assert f(P, P, N, N, R, Q, S, 4, 8, 16, 9, 3, N) == INVALID and "dtype" in err(lib)
    assert f(P, P, N, N, R, Q, S, -1, 8, 16, 9, 0, N) == INVALID
    assert f(P, P, N, N, R, Q, S, 0, 8, 16, 9, 0, N) == OK
    assert f(P, P, N, N, R, Q, S, 4, 8, 0, 9, 0, N) == OK


def test_dwconv1d_bwd_validation(lib):
    ws = lib.dwconv1d_bwd_workspace_bytes
    need = ws(32, 1500, 512, 9)
    assert need > 0 and ws(32, 1500, 512, 6) == 0 and ws(-1, 10, 10, 9) == 0
    f = lib.dwconv1d_bwd
    R, W = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    args = (32, 1500, 512)
    assert f(P, P, N, Q, R, W, N, W, need, *args, 6, 1, 0, N) == UNSUPPORTED and "K=6" in err(lib)
    assert f(P, P, N, Q, R, W, N, W, need, *args, 9, 1, 2, N) == INVALID and "dtype" in err(lib)
    assert f(P, P, N, Q, R, W, N, W, need - 1, *args, 9, 1, 0, N) == WORKSPACE
    assert f(P, P, N, Q, P, W, N, W, need, *args, 9, 1, 0, N) == INVALID and "alias" in err(lib)
    assert f(N, P, N, Q, R, W, N, W, need, *args, 9, 1, 0, N) == INVALID
    assert f(P, P, N, Q, R, W, N, W, need, *args, 0, 1, 0, N) == INVALID
    assert f(P, P, N, Q, R, W, N, W, need, *args, 9, 5, 0, N) == INVALID
    assert f(P, P, N, Q, N, N, N, N, 0, *args, 9, 1, 0, N) == OK  # nothing requested


def test_dwsub_fused_validation(lib):
    f = lib.dwsub_fused_fwd
    assert f(N, P, N, P, N, N, Q, 4, 100, 80, 256, N) == INVALID
    assert f(P, N, N, P, N, N, Q, 4, 100, 80, 256, N) == INVALID
    assert f(P, P, N, N, N, N, Q, 4, 100, 80, 256, N) == INVALID
    assert f(P, P, N, P, N, N, P, 4, 100, 80, 256, N) == INVALID and "alias" in err(lib)
    assert f(P, P, N, P, N, N, Q, 4, -1, 80, 256, N) == INVALID
    assert f(P, P, N, P, N, N, Q, 0, 100, 80, 256, N) == OK


def test_dwsub_fused_bwd_validation(lib):
    ws = lib.dwsub_fused_bwd_workspace_bytes
    need = ws(4, 1000, 80, 256)
    assert need > 0 and ws(-1, 10, 10, 4) == 0
    f = lib.dwsub_fused_bwd
    R, W = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    args = (4, 1000, 80, 256, N)
    assert f(P, P, N, P, N, Q, R, N, N, N, W, need - 1, *args) == WORKSPACE and "workspace" in err(lib)
    assert f(P, P, N, P, N, Q, R, N, N, N, N, need, *args) == WORKSPACE
    assert f(N, P, N, P, N, Q, R, N, N, N, W, need, *args) == INVALID
    assert f(P, P, N, P, N, N, R, N, N, N, W, need, *args) == INVALID
    assert f(P, N, N, P, N, Q, R, N, N, N, W, need, *args) == INVALID
    assert f(P, P, N, P, N, Q, R, N, N, N, W, need, 4, -1, 80, 256, N) == INVALID
    assert f(P, P, N, P, N, Q, N, N, N, N, N, 0, *args) == OK  # nothing requested


def test_dwsub_fused_ex_validation(lib):
    f = lib.dwsub_fused_fwd_ex
    assert f(P, P, N, P, N, N, Q, 4, 100, 80, 256, 2, 0, N) == INVALID and "pad" in err(lib)
    assert f(P, P, N, P, N, N, Q, 4, 100, 80, 256, 1, 5, N) == INVALID and "dtype" in err(lib)
    assert f(P, P, N, P, N, N, P, 4, 100, 80, 256, 1, 1, N) == INVALID and "alias" in err(lib)
    assert f(P, P, N, P, N, N, Q, 0, 100, 80, 256, 1, 1, N) == OK
    ws = lib.dwsub_fused_bwd_workspace_bytes_ex
    need = ws(4, 1000, 80, 256, 1)
    assert need > 0 and ws(4, 1000, 80, 256, 5) == 0
    assert ws(4, 1000, 80, 256, 0) == lib.dwsub_fused_bwd_workspace_bytes(4, 1000, 80, 256)
    g = lib.dwsub_fused_bwd_ex
    R, W = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    assert g(P, P, N, P, N, Q, R, N, N, N, W, need - 1, 4, 1000, 80, 256, 1, 1, N) == WORKSPACE
    assert g(P, P, N, P, N, Q, R, N, N, N, W, need, 4, 1000, 80, 256, 3, 0, N) == INVALID
    assert g(P, P, N, P, N, Q, R, N, N, N, W, need, 4, 1000, 80, 256, 1, 4, N) == INVALID and "dtype" in err(lib)
    assert g(P, P, N, P, N, Q, N, N, N, N, N, 0, 4, 1000, 80, 256, 1, 0, N) == OK  # nothing requested


def test_dwconv2d_fwd_validation(lib):
    f = lib.dwconv2d_fwd
    assert f(P, P, N, N, Q, 2, 8, 8, 4, 3, 3, 1, 1, N) == UNSUPPORTED and "stride" in err(lib)
    assert f(P, P, N, N, Q, 2, 8, 8, 4, 5, 5, 2, 1, N) == UNSUPPORTED
    assert f(P, P, N, N, Q, 2, 8, 8, 4, 3, 3, 2, 0, N) == UNSUPPORTED
    assert f(P, P, N, N, Q, 2, 8, 8, 4, 3, 3, 2, 3, N) == UNSUPPORTED
    assert f(N, P, N, N, Q, 2, 8, 8, 4, 3, 3, 2, 1, N) == INVALID
    assert f(P, P, N, N, P, 2, 8, 8, 4, 3, 3, 2, 1, N) == INVALID
    assert f(P, P, N, N, Q, 2, 8, -8, 4, 3, 3, 2, 1, N) == INVALID
    assert f(P, P, N, N, Q, 2, 0, 8, 4, 3, 3, 2, 1, N) == OK
    assert f(N, N, N, N, N, 0, 8, 8, 4, 3, 3, 2, 1, N) == OK  # empty: pointers unused


def test_dwconv2d_bwd_validation(lib):
    ws = lib.dwconv2d_bwd_workspace_bytes
    need = ws(32, 1500, 64, 256, 3, 3, 2, 1)
    assert need > 0
    assert ws(32, 1500, 64, 256, 3, 3, 1, 1) == 0
    assert ws(-1, 1500, 64, 256, 3, 3, 2, 1) == 0
    f = lib.dwconv2d_bwd
    R = ctypes.c_void_p(0x3000)
    W = ctypes.c_void_p(0x4000)
    args = (32, 1500, 64, 256, 3, 3, 2, 1, N)
    assert f(P, P, N, Q, R, W, N, N, 0, *args) == WORKSPACE and "workspace" in err(lib)
    assert f(P, P, N, Q, R, W, N, W, need - 1, *args) == WORKSPACE
    assert f(P, P, N, Q, P, W, N, W, need, *args) == INVALID and "alias" in err(lib)
    assert f(P, P, N, Q, Q, W, N, W, need, *args) == INVALID
    assert f(N, P, N, Q, R, W, N, W, need, *args) == INVALID
    assert f(P, P, N, Q, R, W, N, W, need, 32, 1500, 64, 256, 3, 3, 1, 1, N) == UNSUPPORTED
    # nothing requested: nothing to do
    assert f(P, P, N, Q, N, N, N, N, 0, *args) == OK


def test_dwconv2d_ex_validation(lib):
    f = lib.dwconv2d_fwd_ex
    geo = (2, 8, 8, 4, 3, 3, 2)
    for pads in ((1, 1, 1, 1), (2, 1, 2, 1), (2, 2, 1, 0), (1, 0, 2, 2)):
        for dt in (0, 1):  # empty batch: validated, nothing enqueued
            assert f(P, P, N, N, Q, 0, *geo[1:], *pads, dt, N) == OK
    assert f(P, P, N, N, Q, *geo, 0, 1, 1, 1, 0, N) == UNSUPPORTED and "pads" in err(lib)
    assert f(P, P, N, N, Q, *geo, 1, 3, 1, 1, 0, N) == UNSUPPORTED
    assert f(P, P, N, N, Q, *geo, 1, 1, 3, 1, 0, N) == UNSUPPORTED
    assert f(P, P, N, N, Q, *geo, 1, -1, 1, 1, 0, N) == INVALID
    assert f(P, P, N, N, Q, *geo, 1, 1, 1, 1, 2, N) == INVALID and "dtype" in err(lib)
    assert f(P, P, N, N, P, *geo, 2, 1, 2, 1, 1, N) == INVALID and "alias" in err(lib)
    assert f(N, P, N, N, Q, *geo, 2, 1, 2, 1, 1, N) == INVALID
    ws = lib.dwconv2d_bwd_workspace_bytes_ex
    need = ws(32, 1500, 64, 256, 3, 3, 2, 2, 1, 2, 1)
    assert need > 0 and ws(32, 1500, 64, 256, 3, 3, 2, 0, 1, 1, 1) == 0
    assert ws(32, 1500, 64, 256, 3, 3, 2, 1, 1, 1, 1) == lib.dwconv2d_bwd_workspace_bytes(32, 1500, 64, 256, 3, 3, 2, 1)
    g = lib.dwconv2d_bwd_ex
    R, W = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    args = (32, 1500, 64, 256, 3, 3, 2, 2, 1, 2, 1)
    assert g(P, P, N, Q, R, W, N, W, need - 1, *args, 1, N) == WORKSPACE
    assert g(P, P, N, Q, Q, W, N, W, need, *args, 1, N) == INVALID and "alias" in err(lib)
    assert g(P, P, N, Q, R, W, N, W, need, *args, 7, N) == INVALID
    assert g(P, P, N, Q, N, N, N, N, 0, *args, 1, N) == OK  # nothing requested


def test_last_error_is_per_thread(lib):
    import threading
    assert lib.dwconv1d_fwd(P, P, N, N, Q, 2, 8, 4, 0, 0, 0, N) == INVALID
    seen = {}

    def other():
        seen["msg"] = lib.dw_last_error().decode()

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "K=0" in err(lib)


def test_header_is_c99_and_the_library_links_from_c(tmp_path):
    """A plain C consumer: gcc -std=c99 -pedantic compiles the header, links
    libdwconv.so and runs host-side validation calls (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "abi_check")
    src = os.path.join(ROOT, "tests", "c", "abi_check.c")
    libdir = os.path.dirname(LIB)
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
                        src, "-o", exe, "-L", libdir, "-ldwconv", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "c abi check: ok" in r.stdout, r.stdout + r.stderr


HUGE = [(1 << 31), (1 << 40), (1 << 62), (1 << 63) - 1]


def test_huge_extents_are_rejected_before_any_launch(lib):
    """Extents whose byte counts overflow 64-bit products are rejected as
    too large (never wrapped into a small size that would pass), and the
    workspace queries return 0 for them."""
    R, W = ctypes.c_void_p(0x3000), ctypes.c_void_p(0x4000)
    S = ctypes.c_void_p(0x5000)
    for h in HUGE:
        for B, T, C in ((h, 8, 4), (2, h, 4), (2, 8, h), (h, h, h), (3, (1 << 31) - 1, (1 << 31) - 1)):
            assert lib.dwconv1d_fwd(P, P, N, N, Q, B, T, C, 3, 0, 0, N) == UNSUPPORTED, (B, T, C)
            assert "too large" in err(lib)
            assert lib.dwconv1d_stream_fwd(P, P, N, N, R, Q, S, B, T, C, 9, 0, N) == UNSUPPORTED
            assert lib.dwconv1d_bwd_workspace_bytes(B, T, C, 9) == 0
            assert lib.dwconv1d_bwd(P, P, N, Q, R, W, N, W, 1 << 40, B, T, C, 9, 0, 0, N) == UNSUPPORTED
        assert lib.dwconv1d_fwd(P, P, N, N, Q, 2, 8, 4, h, 0, 0, N) == UNSUPPORTED
        for B, T, F, C in ((h, 8, 8, 4), (2, h, 8, 4), (2, 8, h, 4), (2, 8, 8, h), (h, h, h, h),
                           (2, (1 << 31) - 1, (1 << 31) - 1, 2)):
            assert lib.dwconv2d_fwd(P, P, N, N, Q, B, T, F, C, 3, 3, 2, 1, N) == UNSUPPORTED, (B, T, F, C)
            assert lib.dwconv2d_bwd_workspace_bytes(B, T, F, C, 3, 3, 2, 1) == 0
            assert lib.dwconv2d_bwd(P, P, N, Q, R, W, N, W, 1 << 40, B, T, F, C, 3, 3, 2, 1, N) == UNSUPPORTED
            assert lib.dwsub_fused_fwd(P, P, N, P, N, N, Q, B, T, F, C, N) == UNSUPPORTED
            assert lib.dwsub_fused_bwd_workspace_bytes(B, T, F, C) == 0
            assert lib.dwsub_fused_bwd(P, P, N, P, N, Q, W, W, W, W, R, 1 << 40, B, T, F, C, N) == UNSUPPORTED


def test_front_forward_refuses_a_mel_item_past_2gb(lib):
    """The forward stages the mel input through a per-item buffer resource,
    so one item's mel input must stay below 2^31 bytes even when its output
    is small (one channel)."""
    T, F = 1 << 27, 8          # 2^32 bytes of fp32 mel per item; output [2^25, 2, 1]
    assert lib.dwsub_fused_fwd(P, P, N, P, N, N, Q, 1, T, F, 1, N) == UNSUPPORTED
    assert "too large" in err(lib)


PROBE_HEADER = os.path.join(ROOT, "include", "dwprobe.h")
PROBE_LIB = os.path.join(ROOT, "conv_subsampling_amd", "libdwprobe.so")


def test_probe_library_exports_its_header_and_validates():
    """The HBM streaming probe (measurement only) is its own library; its
    argument checks answer without a GPU."""
    assert os.path.exists(PROBE_LIB), "libdwprobe.so is not built"
    plib = ctypes.CDLL(PROBE_LIB)
    names = declared_functions(PROBE_HEADER)
    assert names == ["dw_probe_stream"]
    for name in names:
        assert hasattr(plib, name)
    f = plib.dw_probe_stream
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(P, Q, 0, 0, 2, N) == 0                  # nothing to move
    assert f(P, Q, 15, 15, 2, N) == 0                # rounds down to nothing
    assert f(N, Q, 64, 64, 2, N) == -1               # NULL source with bytes to read
    assert f(P, Q, -16, 16, 2, N) == -1
    assert f(P, Q, 16, 16, 3, N) == -1               # unknown policy
    assert f(ctypes.c_void_p(0x1004), Q, 16, 16, 0, N) == -1   # misaligned
    assert f(P, Q, (1 << 42) + 16, 0, 0, N) == -1
    # every header in include/ belongs to a built library that exports it
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == ["dwconv.h", "dwprobe.h"]


def test_noalloc_conv2d_bwd_validation(lib):
    """The allocation-free conv2d backward refuses, before touching a device,
    what the workspace entry point refuses, and channel counts whose partial
    sums would not fit its scratch array."""
    f = lib.dwconv2d_bwd_noalloc
    geo = [3, 3, 2, 1, 1, 1, 1]
    assert f(N, P, N, P, Q, N, N, 2, 8, 8, 4, *geo, 0, N) == INVALID                 # NULL x
    assert f(P, P, N, P, P, N, N, 2, 8, 8, 4, *geo, 0, N) == INVALID                 # dx aliases x
    assert f(P, P, N, P, Q, N, N, 2, 8, 8, 4, 3, 3, 1, 1, 1, 1, 1, 0, N) == UNSUPPORTED   # stride 1
    assert f(P, P, N, P, N, Q, N, 32, 1500, 64, 1024, *geo, 0, N) == UNSUPPORTED   # dw of 1024 channels
    assert b"scratch" in lib.dw_last_error()
    assert f(P, P, N, P, N, N, N, 32, 1500, 64, 1024, *geo, 0, N) == OK            # nothing requested
    assert f(P, P, N, P, Q, N, N, 0, 8, 8, 4, *geo, 7, N) == INVALID                 # unknown dtype
