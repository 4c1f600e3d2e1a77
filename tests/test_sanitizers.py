"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The fp64 oracle is built with gcc and the library's host side with hipcc
(sanitizers on the host pass only; device code is built as usual), and two
drivers under tests/native call every host-only function and every argument
rejection path.  Any out-of-bounds access, overflow or invalid conversion
aborts the driver, which fails the test.  No call reaches a kernel launch,
so no GPU is needed.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
NATIVE = os.path.join(HERE, "native")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-o", exe,
          os.path.join(NATIVE, "oracle_sanitize_driver.c"),
          os.path.join(ROOT, "oracle", "cpmap_oracle.c"), "-lm"])
    r = _run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1"), timeout=300)
    assert "ok" in r.stdout


def test_library_host_code_under_sanitizers(tmp_path):
    if not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm toolchain not found")
    csrc = os.path.join(ROOT, "direct_coulomb_potential_amd", "csrc")
    srcs = sorted(f for f in os.listdir(csrc) if f.endswith(".hip"))

    def compile_one(name):
        obj = str(tmp_path / (name + ".o"))
        _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *HOST_SAN,
              "-c", os.path.join(csrc, name), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=4) as pool:
        objs = list(pool.map(compile_one, srcs))
    lib = str(tmp_path / "libcpmap_san.so")
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
          "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", "-o", lib,
          *objs])
    rt = _run([CLANGXX, "-print-resource-dir"]).stdout.strip() + "/lib/linux"
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", "-shared-libasan", "-o", exe,
          os.path.join(NATIVE, "abi_sanitize_driver.cpp"), f"-L{tmp_path}", "-lcpmap_san",
          f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib", f"-Wl,-rpath,{rt}"])
    r = _run([exe], env=ENV, timeout=600)
    assert "ok" in r.stdout
