"""Speed floors for the two hot kernels at the benchmark sizes, set well
below what they measure (the direct map takes 165 ms, the cutoff map about
1.47 ms), so that they only trip on a real regression (a spilling build, a
lost occupancy, a wrong launch plan), not on run-to-run noise.  Collected
last: they time full-size launches after the parity tests have passed."""
import statistics

import pytest

import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import workloads as wl

pytestmark = pytest.mark.gpu

PEAK_TFLOPS = 157.3


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


def _median_ms(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def test_direct_sum_floor_at_200cube_200k(torch):
    w = wl.large_direct()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    V = torch.empty(lat.nz, lat.ny, lat.nx, device="cuda")
    ws = torch.empty(cpmap.direct_workspace_bytes(w.n_atoms, lat), dtype=torch.uint8,
                     device="cuda")
    print("[perf floor] direct 200^3 x 200k", flush=True)
    ms = _median_ms(torch, lambda: cpmap.direct(atoms, lat, out=V, workspace=ws), 3, 1)
    frac = 10 * w.pairs / (ms * 1e-3) / 1e12 / PEAK_TFLOPS
    print(f"direct: {ms:.1f} ms, {100 * frac:.1f}% of the fp32 peak")
    assert frac >= 0.50, f"{ms:.1f} ms is {100 * frac:.1f}% of peak"


def test_cutoff_floor_at_200cube_100k_rc12(torch):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, w.bin_size, w.cutoff)
    V = torch.empty(lat.nz, lat.ny, lat.nx, device="cuda")
    print("[perf floor] cutoff 200^3 x 100k rc 12", flush=True)
    ms = _median_ms(torch, lambda: cpmap.cutoff(ws, w.n_atoms, lat, w.bin_size, w.cutoff,
                                                out=V), 10, 3)
    print(f"cutoff: {ms:.3f} ms")
    assert ms <= 2.2, f"{ms:.3f} ms"
