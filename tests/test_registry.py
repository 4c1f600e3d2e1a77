"""The host-side workspace registry (CPU only).

direct_coulomb_potential_amd/csrc/workspace_registry.h is plain C++: a
driver under tests/native builds it with g++ three times -- plain, under
AddressSanitizer + UndefinedBehaviorSanitizer, and under ThreadSanitizer -- and
checks hand-picked cases (exact base, size, kind and key; writes that end
just before, start just after, touch one byte, straddle two records; ranges
past the top of the address space), 200,000 random operations against a plain
list model, and eight threads sharing one registry.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "native", "registry_driver.cpp")


@pytest.mark.parametrize("flags", [
    [],
    ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"],
    ["-fsanitize=thread"],
], ids=["plain", "asan_ubsan", "tsan"])
def test_registry_driver(tmp_path, flags):
    if shutil.which("g++") is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "registry_driver")
    r = subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-Wall", "-Wextra", "-Werror",
                        "-pthread", *flags, "-o", exe, DRIVER], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr
