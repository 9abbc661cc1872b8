"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Builds the library's HIP sources with the sanitizers on their host code only
(-Xarch_host before each -fsanitize=; no device code is instrumented) and
links them with tests/sanitize/abi_driver.c, which calls every entry point of
include/tdm.h with invalid and valid-shaped arguments: each call ends in the
host validation or at the device check, so the run needs no GPU. The oracle's
C loop (oracle/oracle.c) is built the same way with gcc and driven by
tests/sanitize/oracle_driver.c through its closed forms, edge blocks and
rejected arguments. Any sanitizer report fails the test.
"""
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tiled_dense_matrix_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
HERE = os.path.join(ROOT, "tests", "sanitize")

HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _tool(name, fallback):
    path = shutil.which(name) or fallback
    if not os.path.exists(path):
        pytest.skip(f"{name} not found")
    return path


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _no_reports(r):
    text = r.stdout + r.stderr
    assert "runtime error" not in text and "AddressSanitizer" not in text, text


@pytest.fixture(scope="module")
def abi_driver(tmp_path_factory):
    hipcc = _tool("hipcc", "/opt/rocm/bin/hipcc")
    clang = _tool("amdclang", "/opt/rocm/llvm/bin/clang")
    out = tmp_path_factory.mktemp("sanitize")
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-w",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             f"-I{INCLUDE}", f"-I{CSRC}", *HOST_SAN]

    def compile_one(src):
        obj = os.path.join(out, os.path.basename(src) + ".o")
        _run([hipcc, *flags, "-c", src, "-o", obj])
        return obj

    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(out, "abi_driver.o")
    _run([clang, "-O1", "-g", "-std=c11", f"-I{INCLUDE}", "-fsanitize=address,undefined",
          "-fno-omit-frame-pointer", "-c", os.path.join(HERE, "abi_driver.c"), "-o", drv])
    exe = os.path.join(out, "abi_driver")
    _run([hipcc, "--offload-arch=gfx950", *HOST_SAN, *objs, drv, "-o", exe])
    return exe


def test_abi_validation_under_sanitizers(abi_driver):
    r = subprocess.run([abi_driver], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations held" in r.stdout
    _no_reports(r)


def test_oracle_under_sanitizers(tmp_path):
    gcc = _tool("gcc", "/usr/bin/gcc")
    exe = os.path.join(tmp_path, "oracle_driver")
    _run([gcc, "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_driver.c"),
          "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all expectations held" in r.stdout
    _no_reports(r)
