"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two builds, each run as its own process so that the sanitizer runtime comes
first in it:
  * the oracle (oracle/oracle.c) with gcc, driven by tests/c/oracle_san.c over
    every function, tiny and degenerate shapes, and NULL optional pointers;
  * the library's host code (argument checks, size limits, launch geometry)
    with the sanitizers on the host side only (the GPU code is built without
    them: GPU sanitizers are not used here), driven by the C ABI consumer
    tests/c/abi_check.c.  Without a GPU every call there returns before a
    launch, which is exactly the host code under test.
A finding stops the process (-fno-sanitize-recover=all) with a non-zero status.
"""
import importlib.util
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLANG = "/opt/rocm/llvm/bin/clang"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nrc={r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror",
          "-o", exe, os.path.join(ROOT, "tests", "c", "oracle_san.c"), os.path.join(ROOT, "oracle", "oracle.c"),
          "-lm"])
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "0 failures" in r.stdout, r.stdout


def _builder():
    path = os.path.join(ROOT, "conv_subsampling_amd", "build.py")
    spec = importlib.util.spec_from_file_location("_dwconv_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang not found")
def test_library_host_code_under_asan_and_ubsan(tmp_path):
    b = _builder()
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    # the GPU code at -O0: it is never launched here, and builds in a fraction of the time
    flags = [f"--offload-arch={b.ARCH}", "-std=c++17", "-fPIC", "-Xarch_device", "-O0", "-Xarch_host", "-O1",
             "-Xarch_host", "-g", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", *host_san, "-I", b.INCLUDE, "-I", b.CSRC]
    procs, objs = [], []
    for src in b.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([b.hipcc(), *flags, "-c", os.path.join(b.CSRC, src), "-o", obj],
                                      stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True))
    for p in procs:
        out, _ = p.communicate()
        assert p.returncode == 0, out[-4000:]
    lib = str(tmp_path / "libdwconv_san.so")
    _run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *host_san, "-o", lib, *objs])
    exe = str(tmp_path / "abi_san")
    _run([CLANG, "-std=c99", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-I", b.INCLUDE, "-o", exe, os.path.join(ROOT, "tests", "c", "abi_check.c"),
          "-L", str(tmp_path), "-ldwconv_san", f"-Wl,-rpath,{tmp_path}"])
    r = _run([exe], env=SAN_ENV, timeout=120)
    assert "c abi check: ok" in r.stdout, r.stdout
