"""Every compute entry point is a sequence of kernel launches on the caller's
stream (no allocation, no synchronisation, no memset), so it can be captured
into a HIP graph.  Each test captures a path, changes its inputs with eager
work between replays, and checks every replay bit for bit against the eager
call on the same inputs (the kernels are deterministic), then against the
fp64 oracle.
"""
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


def _capture(torch, fn):
    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _seeds():
    return [61, 62, 63, 64]


def test_graph_bin_and_cutoff_replays(torch):
    n, lat, bs, rc = 20_000, Lattice(48, 40, 33, 0.5), 4.0, 12.0
    atoms = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    ws = torch.empty(cpmap.bin_workspace_bytes(n, lat, bs, rc), dtype=torch.uint8, device="cuda")
    sws = torch.empty(cpmap.slot_workspace_bytes(n, lat, bs, rc, 8), dtype=torch.uint8,
                      device="cuda")
    V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device="cuda")
    Vs = torch.empty_like(V)
    Vt = torch.empty_like(V)
    atoms.copy_(torch.from_numpy(wl.random_atoms(n, (-14, -14, -14), (38, 34, 30), seed=60)))

    def path():
        cpmap.bin_atoms(atoms, lat, bs, rc, workspace=ws)
        cpmap.cutoff(ws, n, lat, bs, rc, out=V)
        cpmap.cutoff(ws, n, lat, bs, rc, out=Vt, term="truncated")
        cpmap.bin_slots(ws, n, lat, bs, rc, 8, slot_workspace=sws)
        cpmap.cutoff_slots(sws, n, lat, bs, rc, 8, out=Vs)

    g = _capture(torch, path)
    for seed in _seeds():
        print(f"[graph cutoff] replay with atoms seed {seed}", flush=True)
        atoms_np = wl.random_atoms(n, (-14, -14, -14), (38, 34, 30), seed=seed)
        atoms.copy_(torch.from_numpy(atoms_np))
        g.replay()
        torch.cuda.synchronize()
        got = [V.clone(), Vt.clone(), Vs.clone()]
        for t in (V, Vt, Vs):
            t.fill_(float("nan"))
        path()  # eager, same inputs
        torch.cuda.synchronize()
        for a, b in zip(got, [V, Vt, Vs]):
            assert torch.equal(a, b)
    nodes = wl.checked_nodes(lat, n_random=2000)
    Vo, S = oracle.cutoff(atoms_np, lat.dims, lat.spacing, lat.origin, rc, nodes=nodes,
                          with_scale=True)
    err = np.abs(got[0].cpu().numpy().reshape(-1)[nodes].astype(np.float64) - Vo)
    assert np.all(err <= 1e-5 * S)


def test_graph_direct_and_extrema_replays(torch):
    n, lat = 5000, Lattice(37, 21, 13, 0.5, (1.0, -2.0, 0.25))
    atoms = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    need = cpmap.direct_workspace_bytes(n, lat)
    wsd = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device="cuda")
    V1 = torch.empty_like(V)
    exw = torch.empty(int(cpmap.library().cpmap_extrema_workspace_bytes(V.numel())),
                      dtype=torch.uint8, device="cuda")
    idx = torch.empty(2, dtype=torch.int64, device="cuda")
    val = torch.empty(2, dtype=torch.float32, device="cuda")
    idx1 = torch.empty(2, dtype=torch.int64, device="cuda")
    val1 = torch.empty(2, dtype=torch.float32, device="cuda")
    atoms.copy_(torch.from_numpy(wl.random_atoms(n, (-5, -8, -5), (25, 12, 12), seed=65)))

    def path():
        cpmap.direct(atoms, lat, out=V, workspace=wsd)
        cpmap.direct(atoms, lat, out=V1, split=False)
        cpmap.extrema(V, workspace=exw, out=(idx, val))
        # the static per-GPU slots of the allocation-free entry point, which
        # a replay (same tag) must also find cleared
        cpmap.extrema_noalloc(V1, out=(idx1, val1))

    g = _capture(torch, path)
    for seed in _seeds():
        print(f"[graph direct] replay with atoms seed {seed}", flush=True)
        atoms_np = wl.random_atoms(n, (-5, -8, -5), (25, 12, 12), seed=seed + 10)
        atoms.copy_(torch.from_numpy(atoms_np))
        g.replay()
        torch.cuda.synchronize()
        got = [V.clone(), V1.clone(), idx.clone(), val.clone(), idx1.clone(), val1.clone()]
        path()
        torch.cuda.synchronize()
        for a, b in zip(got, [V, V1, idx, val, idx1, val1]):
            assert torch.equal(a, b)
    Vo, S = oracle.direct(atoms_np, lat.dims, lat.spacing, lat.origin, with_scale=True)
    err = np.abs(got[0].cpu().numpy().reshape(-1).astype(np.float64) - Vo)
    assert np.all(err <= 1e-5 * S)
    (imin, imax), _ = oracle.extrema(got[0].cpu().numpy())
    assert got[2].cpu().tolist() == [imin, imax]
    (imin, imax), _ = oracle.extrema(got[1].cpu().numpy())
    assert got[4].cpu().tolist() == [imin, imax]
