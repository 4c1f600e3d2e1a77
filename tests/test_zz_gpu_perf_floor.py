"""Speed floors for the hot paths at the benchmark sizes, set well below
what they measure (the direct map takes 156 ms with its workspace and 171 ms
without, the cutoff map 1.45 ms smoothed and 1.37 ms truncated, the extrema
of the 200^3 map 15-17 us per event-timed call, the k = 10 plane 28-30 us),
so that they only trip on a real regression (a spilling build, a lost
occupancy, a wrong launch plan), not on run-to-run noise.  Collected last:
they time full-size launches after the parity tests have passed."""
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


def test_truncated_cutoff_floor_at_200cube_100k_rc12(torch):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, w.bin_size, w.cutoff)
    V = torch.empty(lat.nz, lat.ny, lat.nx, device="cuda")
    print("[perf floor] truncated cutoff 200^3 x 100k rc 12", flush=True)
    ms = _median_ms(torch, lambda: cpmap.cutoff(ws, w.n_atoms, lat, w.bin_size, w.cutoff,
                                                out=V, term="truncated"), 10, 3)
    print(f"truncated cutoff: {ms:.3f} ms")
    assert ms <= 2.1, f"{ms:.3f} ms"


def test_direct_without_workspace_and_extrema_floors_at_200cube_200k(torch):
    w = wl.large_direct()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    V = torch.empty(lat.nz, lat.ny, lat.nx, device="cuda")
    print("[perf floor] cpmap_direct (no workspace) 200^3 x 200k", flush=True)
    ms = _median_ms(torch, lambda: cpmap.direct(atoms, lat, out=V, split=False), 2, 1)
    frac = 10 * w.pairs / (ms * 1e-3) / 1e12 / PEAK_TFLOPS
    print(f"direct without workspace: {ms:.1f} ms, {100 * frac:.1f}% of the fp32 peak")
    assert frac >= 0.45, f"{ms:.1f} ms is {100 * frac:.1f}% of peak"
    ext_ws = torch.empty(cpmap.library().cpmap_extrema_workspace_bytes(lat.n_points),
                         dtype=torch.uint8, device="cuda")
    out = (torch.empty(2, dtype=torch.int64, device="cuda"),
           torch.empty(2, dtype=torch.float32, device="cuda"))
    print("[perf floor] extrema of the 200^3 map", flush=True)
    ms = _median_ms(torch, lambda: cpmap.extrema(V, workspace=ext_ws, out=out), 20, 5)
    print(f"extrema: {1e3 * ms:.1f} us")
    assert ms <= 0.06, f"{1e3 * ms:.1f} us"


def test_plane_floor(torch):
    w = wl.plane_direct()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    V = torch.empty(lat.nz, lat.ny, lat.nx, device="cuda")
    ws = torch.empty(max(cpmap.direct_workspace_bytes(w.n_atoms, lat), 1), dtype=torch.uint8,
                     device="cuda")
    print("[perf floor] direct, plane k = 10", flush=True)
    ms = _median_ms(torch, lambda: cpmap.direct(atoms, lat, out=V, workspace=ws), 50, 20)
    print(f"plane: {1e3 * ms:.1f} us")
    assert ms <= 0.12, f"{1e3 * ms:.1f} us"
