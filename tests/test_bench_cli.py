"""bench.py's host side (CPU only): the one-GPU guard and the counter-summary
records it reads traffic from."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _write_profile(root, source_text, recorded_sha):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "kernel.hip"), "w") as f:
        f.write(source_text)
    rec = {"kernel": "k", "source_sha256": recorded_sha, "traffic_bytes_per_launch": 1234}
    with open(os.path.join(root, "profiles", "k.md"), "w") as f:
        f.write("# k\n\ntext\n\n```json\n" + json.dumps(rec) + "\n```\n")


def test_traffic_is_reported_only_for_the_profiled_source(tmp_path, monkeypatch):
    src = "__global__ void k() {}\n"
    sha = hashlib.sha256(src.encode()).hexdigest()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    _write_profile(str(tmp_path), src, sha)
    assert bench.measured_traffic("k.md", "kernel.hip") == 1234
    # the source changed after the counters were taken: no traffic figure
    with open(tmp_path / "kernel.hip", "a") as f:
        f.write("// edited\n")
    assert bench.measured_traffic("k.md", "kernel.hip") is None
    # missing files give no record rather than an error
    assert bench.profile_record("absent.md", "kernel.hip") is None
    assert bench.profile_record("k.md", "absent.hip") is None


def test_committed_profiles_carry_a_record():
    for name, src in [("direct_kernel_200cube_200k.md",
                       "direct_coulomb_potential_amd/csrc/direct.hip"),
                      ("cutoff_kernel_200cube_100k_rc12.md",
                       "direct_coulomb_potential_amd/csrc/cutoff.hip")]:
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
        block = text.split("```json\n")[1].split("\n```")[0]
        rec = json.loads(block)
        assert rec["source"] == src
        assert len(rec["source_sha256"]) == 64
        assert rec["traffic_bytes_per_launch"] > 0
        assert "rocprofv3 --kernel-trace --stats" in text
