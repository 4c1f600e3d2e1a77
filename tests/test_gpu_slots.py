"""GPU parity of fixed-capacity bins against the fp64 oracle.

cpmap_bin_slots is integer and copy work: its slots, overflow offsets and
overflow atoms must equal the oracle's sequential fill bit for bit (empty
slots included).  cpmap_cutoff_slots computes the same sum as
cpmap_cutoff_term and meets the same bound, |V_gpu - V_oracle| <= 1e-5 * S_c
at every checked node; with no overflow it must equal cpmap_cutoff_term bit
for bit (the same atoms reach every node in the same order).
"""
import numpy as np
import pytest

import oracle
import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import Lattice
from direct_coulomb_potential_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


def _slots(torch, atoms_np, lat, bs, rc, cap):
    atoms = torch.from_numpy(np.ascontiguousarray(atoms_np, dtype=np.float32)).cuda()
    n = atoms_np.shape[0]
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    sws = cpmap.bin_slots(ws, n, lat, bs, rc, cap)
    slots, starts, over = cpmap.slot_views(sws, n, lat, bs, rc, cap)
    torch.cuda.synchronize()
    return ws, sws, slots.cpu().numpy(), starts.cpu().numpy(), over.cpu().numpy()


def _check_slots(torch, atoms_np, lat, bs, rc, cap):
    ws, sws, slots, starts, over = _slots(torch, atoms_np, lat, bs, rc, cap)
    o_slots, o_starts, o_over = oracle.bin_slots(atoms_np, lat.dims, lat.spacing, lat.origin,
                                                 bs, rc, cap)
    assert slots.tobytes() == o_slots.tobytes()
    np.testing.assert_array_equal(starts, o_starts)
    n_over = int(o_starts[-1])
    assert over[:n_over].tobytes() == o_over.tobytes()
    return ws, sws, n_over


SLOT_CASES = [
    # (n, lattice, bs, rc, box_lo, box_hi, seed, capacity)
    (1, Lattice(5, 5, 5, 0.5), 1.0, 2.0, (0, 0, 0), (2, 2, 2), 21, 8),
    (777, Lattice(37, 21, 13, 0.5, (1.0, -2.0, 0.25)), 1.5, 3.0, (-5, -8, -5), (25, 12, 12), 22, 3),
    (5000, Lattice(30, 30, 30, 0.3, (-4.0, 0.0, 2.0)), 1.0, 2.5, (-8, -4, -2), (8, 13, 14), 23, 1),
    (70_000, Lattice(64, 48, 40, 0.5), 2.0, 6.0, (-10, -10, -10), (42, 34, 30), 24, 8),
    (40_000, Lattice(64, 64, 64, 0.5), 4.0, 12.0, (0, 0, 0), (32, 32, 32), 25, 64),
]


@pytest.mark.parametrize("case", SLOT_CASES, ids=[f"n{c[0]}_cap{c[7]}" for c in SLOT_CASES])
def test_bin_slots_bit_exact(torch, case):
    n, lat, bs, rc, lo, hi, seed, cap = case
    print(f"[slots] n={n} dims={lat.dims} bs={bs} rc={rc} cap={cap}", flush=True)
    _check_slots(torch, wl.random_atoms(n, lo, hi, seed=seed), lat, bs, rc, cap)


def test_bin_slots_edge_cases(torch):
    """No atoms (every slot empty); 5000 atoms in one bin (4992 overflow, in
    input order); faces, far, NaN and neutral atoms (a q = 0 atom sits in a
    slot like any other)."""
    lat = Lattice(8, 8, 8, 1.0)
    _, _, n_over = _check_slots(torch, np.zeros((0, 4), np.float32), lat, 2.0, 3.0, 8)
    assert n_over == 0
    same = wl.random_atoms(5000, (2.0, 2.0, 2.0), (2.5, 2.5, 2.5), seed=26)
    _, _, n_over = _check_slots(torch, same, lat, 2.0, 3.0, 8)
    assert n_over == 4992
    faces = np.array([[0, 0, 0, 1], [2, 0, 0, 1], [-4, -4, -4, 1], [-4.001, 0, 0, 1],
                      [13.999, 0, 0, 1], [14, 0, 0, 1], [np.nan, 0, 0, 1], [1e30, 0, 0, 1],
                      [-1e30, 0, 0, 1], [1.0, 1.0, 1.0, 0.0], [1.5, 1.0, 1.0, 0.0],
                      [0.5, 0.5, 0.5, 2.0]], dtype=np.float32)
    for cap in (1, 2, 8):
        _check_slots(torch, faces, lat, 2.0, 3.0, cap)


def test_bin_slots_config5_bit_exact(torch):
    w = wl.cutoff_binned()
    _, _, n_over = _check_slots(torch, w.atoms, w.lattice, w.bin_size, w.cutoff, 8)
    print(f"{w.name}: {n_over} of {w.n_atoms} atoms overflow 8-slot bins "
          f"({100.0 * n_over / w.n_atoms:.2f}%)")
    assert 0 < n_over < w.n_atoms // 5


def _parity(Vg, Vo, S, label):
    err = np.abs(Vg.astype(np.float64) - Vo)
    bad = ~(err <= TOL * S)
    if bad.any():
        i = int(np.argmax(np.where(bad, err, -1)))
        raise AssertionError(f"{label}: {bad.sum()} nodes out of bound; node {i}: gpu {Vg[i]!r} "
                             f"oracle {Vo[i]!r} S {S[i]!r}")
    ratio = err / np.where(S > 0, S, 1.0)
    return float(ratio.max()) if ratio.size else 0.0


def _oracle(term, atoms_np, lat, rc, nodes=None):
    fn = oracle.cutoff if term == "smoothed" else oracle.cutoff_hard
    return fn(atoms_np, lat.dims, lat.spacing, lat.origin, rc, nodes=nodes, with_scale=True)


CUT_CASES = [
    (1, Lattice(9, 9, 9, 0.5), 1.0, 2.0, (1, 1, 1), (3, 3, 3), 31),
    (2000, Lattice(37, 21, 13, 0.5, (1.0, -2.0, 0.25)), 1.5, 3.0, (-5, -8, -5), (25, 12, 12), 33),
    (4000, Lattice(30, 30, 30, 0.3, (-4.0, 0.0, 2.0)), 1.0, 2.5, (-8, -4, -2), (8, 13, 14), 34),
    (20_000, Lattice(48, 40, 33, 0.5), 4.0, 12.0, (-14, -14, -14), (38, 34, 30), 35),
]


@pytest.mark.parametrize("term", ["smoothed", "truncated"])
@pytest.mark.parametrize("cap", [1, 8])
@pytest.mark.parametrize("case", CUT_CASES, ids=[f"n{c[0]}_{c[1].nx}x{c[1].ny}x{c[1].nz}" for c in CUT_CASES])
def test_cutoff_slots_small_all_nodes(torch, case, cap, term):
    n, lat, bs, rc, lo, hi, seed = case
    print(f"[cutoff_slots] n={n} dims={lat.dims} bs={bs} rc={rc} cap={cap} {term}", flush=True)
    atoms_np = wl.random_atoms(n, lo, hi, seed=seed)
    _, sws, n_over = _check_slots(torch, atoms_np, lat, bs, rc, cap)
    out = torch.full((lat.nz, lat.ny, lat.nx), float("nan"), device="cuda")
    V = cpmap.cutoff_slots(sws, n, lat, bs, rc, cap, out=out, term=term)
    V = V.cpu().numpy().reshape(-1)
    Vo, S = _oracle(term, atoms_np, lat, rc)
    _parity(V, Vo, S, f"n={n} dims={lat.dims} cap={cap} {term} overflow={n_over}")


@pytest.mark.parametrize("term", ["smoothed", "truncated"])
def test_cutoff_slots_without_overflow_equals_csr(torch, term):
    """With capacity above every bin's count the slot pass sees the CSR's
    atoms in the CSR's order (empty slots never reach a sum), so V matches
    cpmap_cutoff_term bit for bit."""
    n, lat, bs, rc = 20_000, Lattice(48, 40, 33, 0.5), 2.0, 6.0
    atoms_np = wl.random_atoms(n, (-6, -6, -6), (30, 26, 22), seed=36)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    starts, _ = cpmap.workspace_views(ws, n, lat, bs, rc)
    cap = int(torch.diff(starts).max().item())
    assert 1 < cap <= 64
    sws = cpmap.bin_slots(ws, n, lat, bs, rc, cap)
    _, over_start, _ = cpmap.slot_views(sws, n, lat, bs, rc, cap)
    assert int(over_start[-1].item()) == 0
    a = cpmap.cutoff(ws, n, lat, bs, rc, term=term)
    b = cpmap.cutoff_slots(sws, n, lat, bs, rc, cap, term=term)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("term", ["smoothed", "truncated"])
def test_cutoff_slots_config5_checked_nodes(torch, term):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, w.bin_size, w.cutoff)
    sws = cpmap.bin_slots(ws, w.n_atoms, lat, w.bin_size, w.cutoff, 8)
    V = cpmap.cutoff_slots(sws, w.n_atoms, lat, w.bin_size, w.cutoff, 8, term=term)
    V = V.cpu().numpy().reshape(-1)
    nodes = wl.checked_nodes(lat)
    Vo, S = _oracle(term, w.atoms, lat, w.cutoff, nodes=nodes)
    worst = _parity(V[nodes], Vo, S, f"{w.name} slots {term}")
    print(f"{w.name} slots {term}: {nodes.size} nodes, worst |err|/S = {worst:.3e}")


def test_cutoff_slots_all_atoms_in_one_bin(torch):
    """Almost every atom overflows: the overflow pass carries the sum, and
    tiles out of the overflow's reach keep the slot pass's exact zeros."""
    lat = Lattice(40, 16, 16, 0.5)
    atoms_np = wl.random_atoms(3000, (2.1, 2.1, 2.1), (2.9, 2.9, 2.9), seed=37)
    _, sws, n_over = _check_slots(torch, atoms_np, lat, 1.0, 3.0, 8)
    assert n_over == 2992
    out = torch.full((16, 16, 40), float("nan"), device="cuda")
    V = cpmap.cutoff_slots(sws, 3000, lat, 1.0, 3.0, 8, out=out).cpu().numpy().reshape(-1)
    Vo, S = _oracle("smoothed", atoms_np, lat, 3.0)
    assert np.all(V[S == 0] == 0.0) and (S == 0).sum() > 1000
    _parity(V, Vo, S, "one bin")


def test_cutoff_slots_is_deterministic_and_checks_records(torch):
    atoms_np = wl.random_atoms(30_000, (0, 0, 0), (20, 20, 20), seed=38)
    lat = Lattice(40, 40, 40, 0.5)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, 2.0, 6.0)
    sws = cpmap.bin_slots(ws, 30_000, lat, 2.0, 6.0, 4)
    a = cpmap.cutoff_slots(sws, 30_000, lat, 2.0, 6.0, 4).clone()
    b = cpmap.cutoff_slots(sws, 30_000, lat, 2.0, 6.0, 4)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # a slot workspace filled for capacity 4 is refused for capacity 8 ...
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.cutoff_slots(sws, 30_000, lat, 2.0, 6.0, 8)
    assert e.value.status in (3, 4)
    # ... a CSR workspace is not a slot workspace, and the other way round
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.cutoff_slots(ws, 30_000, lat, 2.0, 6.0, 4)
    assert e.value.status in (3, 4)
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.cutoff(sws, 30_000, lat, 2.0, 6.0)
    assert e.value.status in (3, 4)
    # slots need a workspace binned for the same arguments
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.bin_slots(ws, 30_000, lat, 2.0, 5.0, 4)
    assert e.value.status in (3, 4)


@pytest.mark.parametrize("term", ["smoothed", "truncated"])
def test_cutoff_csr_and_slots_on_clustered_atoms(torch, term):
    """The 40k-atom clustered workload (20 Gaussian clusters, sigma 6 A) with
    rc = 12 A and 4 A bins: dense bins make neighbourhoods of many staging
    chunks and overflow 8-slot bins heavily; both layouts meet the bound."""
    w = wl.protein_direct()
    lat, bs, rc = w.lattice, 4.0, 12.0
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    starts, _ = cpmap.workspace_views(ws, w.n_atoms, lat, bs, rc)
    print(f"[clustered] max atoms per bin {int(torch.diff(starts).max().item())}", flush=True)
    Vc = cpmap.cutoff(ws, w.n_atoms, lat, bs, rc, term=term).cpu().numpy().reshape(-1)
    sws = cpmap.bin_slots(ws, w.n_atoms, lat, bs, rc, 8)
    n_over = int(cpmap.slot_views(sws, w.n_atoms, lat, bs, rc, 8)[1][-1].item())
    Vs = cpmap.cutoff_slots(sws, w.n_atoms, lat, bs, rc, 8, term=term).cpu().numpy().reshape(-1)
    nodes = wl.checked_nodes(lat, n_random=5000)
    Vo, S = _oracle(term, w.atoms, lat, rc, nodes=nodes)
    worst_c = _parity(Vc[nodes], Vo, S, f"clustered csr {term}")
    worst_s = _parity(Vs[nodes], Vo, S, f"clustered slots {term}")
    print(f"clustered {term}: {n_over} of {w.n_atoms} atoms overflow; worst |err|/S csr "
          f"{worst_c:.3e} slots {worst_s:.3e}")
    assert n_over > w.n_atoms // 4

