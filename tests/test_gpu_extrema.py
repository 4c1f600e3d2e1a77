"""GPU parity of cpmap_extrema (ion placement) against the oracle.

Index work: the argmin/argmax indices and the values there must equal the
oracle's exactly (NaN skipped, smallest index among equal values).  Inputs are
seeded synthetic maps, never a GPU-computed potential; the end-to-end check on
a GPU potential map compares only what is unique (the oracle's potential at
the chosen node is within the parity bound of the oracle's extremum).
"""
import json
import os

import numpy as np
import pytest

import oracle
import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import Lattice
from direct_coulomb_potential_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


def _gpu_extrema(torch, V_np, offset=0):
    buf = torch.zeros(V_np.size + offset, dtype=torch.float32, device="cuda")
    V = buf[offset:]
    V.copy_(torch.from_numpy(np.ascontiguousarray(V_np, dtype=np.float32)))
    idx, val = cpmap.extrema(V)
    torch.cuda.synchronize()
    return tuple(idx.cpu().tolist()), tuple(val.cpu().tolist())


def _check(torch, V_np, offset=0):
    (gi, gv) = _gpu_extrema(torch, V_np, offset)
    (oi, ov) = oracle.extrema(V_np)
    assert gi == oi, (gi, oi)
    for a, b in zip(gv, ov):
        assert (np.isnan(a) and np.isnan(b)) or np.float32(a).tobytes() == np.float32(b).tobytes()


def test_extrema_golden(torch, golden_dir):
    with open(os.path.join(golden_dir, "extrema.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        V = np.array([float(v) for v in case["V"]], dtype=np.float32)
        (gi, _) = _gpu_extrema(torch, V)
        assert gi == (case["argmin"], case["argmax"]), case


@pytest.mark.parametrize("n", [1, 63, 4096, 4097, 65_537, 1_000_003, 8_000_000])
@pytest.mark.parametrize("offset", [0, 1])
def test_extrema_random_with_ties_and_nans(torch, n, offset):
    rng = np.random.default_rng(n + offset)
    V = np.round(rng.normal(size=n) * 8).astype(np.float32)  # many ties
    V[rng.random(n) < 0.01] = np.nan
    print(f"[extrema] n={n} offset={offset}", flush=True)
    _check(torch, V, offset)


def test_extrema_extremes_at_the_ends_and_all_nan(torch):
    n = 2_000_000
    V = np.zeros(n, dtype=np.float32)
    V[-1] = -1.0
    V[0] = 1.0
    _check(torch, V)
    _check(torch, np.full(4099, np.nan, dtype=np.float32))
    _check(torch, np.zeros(0, dtype=np.float32))
    V2 = np.full(100_000, np.inf, dtype=np.float32)
    V2[77_777] = -np.inf
    _check(torch, V2)


def test_place_ions_on_a_potential_map(torch):
    """End to end on the 100x100x50 workload: the node chosen for each ion has
    an oracle potential within the parity bound of the oracle's extremum."""
    w = wl.full_direct()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    V = cpmap.direct(atoms, lat)
    ions = cpmap.place_ions(V, lat)
    Vo, S = oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    for key, pick in (("positive_ion", np.argmin), ("negative_ion", np.argmax)):
        (i, j, k), pos, v = ions[key]
        g = (k * lat.ny + j) * lat.nx + i
        best = int(pick(Vo))
        assert abs(Vo[g] - Vo[best]) <= 1e-5 * (S[g] + S[best]), key
        assert abs(v - Vo[g]) <= 1e-5 * S[g]
        assert pos == (float(np.float32(i * np.float32(0.5))), float(np.float32(j * np.float32(0.5))),
                       float(np.float32(k * np.float32(0.5))))


@pytest.mark.parametrize("n", [5, 20_000, 8_000_000, 16_711_681])
def test_extrema_needs_no_cleared_workspace(torch, n):
    """The one-launch reduction keeps a tagged counter in its workspace: a
    workspace full of arbitrary bytes, and the same workspace reused call
    after call with maps of different sizes (the grid, and so the count the
    last workgroup waits for, changes), give the oracle's answer every time.
    16,711,681 nodes take the largest grid (512 workgroups, two slabs
    each)."""
    rng = np.random.default_rng(n)
    ws = torch.randint(0, 256, (cpmap.library().cpmap_extrema_workspace_bytes(16_711_681),),
                       dtype=torch.uint8, device="cuda")
    for m in (n, max(n // 3, 1), n):
        V_np = rng.standard_normal(m).astype(np.float32)
        V_np[rng.integers(0, m, size=max(m // 100, 1))] = np.nan
        V = torch.from_numpy(V_np).cuda()
        idx, val = cpmap.extrema(V, workspace=ws)
        torch.cuda.synchronize()
        (oi, ov) = oracle.extrema(V_np)
        assert tuple(idx.cpu().tolist()) == oi
