"""include/cpmap.h as plain C (CPU only): a C99 program compiled with gcc
-pedantic -Werror against the header, linked to libcpmap.so, calls the
host-only entry points and the host-side argument checks."""
import os
import shutil
import subprocess

import pytest

import direct_coulomb_potential_amd as cpmap

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_header_is_plain_c_and_host_calls_link(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    libdir = os.path.dirname(cpmap.library_path())
    if not os.path.exists(cpmap.library_path()):
        pytest.fail("libcpmap.so is not built")
    exe = str(tmp_path / "c_header_driver")
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                        "-I", os.path.join(ROOT, "include"),
                        os.path.join(HERE, "native", "c_header_driver.c"), "-o", exe,
                        f"-L{libdir}", "-lcpmap", f"-Wl,-rpath,{libdir}",
                        "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath-link,/opt/rocm/lib"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
