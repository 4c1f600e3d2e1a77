"""GPU parity of cpmap_direct against the fp64 oracle.

Bar: |V_gpu - V_oracle| <= 1e-5 * S at every checked node, S = sum_a |q_a|/r.
Small cases are checked at every node; the 200^3 workloads on three full
z-slices plus 10^4 seeded random nodes, in the same launch configuration the
benchmark times (the library picks it from the lattice and atom count).
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


def _run_direct(torch, atoms_np, lat, split=True):
    atoms = torch.from_numpy(np.ascontiguousarray(atoms_np, dtype=np.float32)).cuda()
    V = cpmap.direct(atoms, lat, split=split)
    torch.cuda.synchronize()
    return V.cpu().numpy().reshape(-1)


def _assert_parity(Vg, Vo, S, label):
    err = np.abs(Vg.astype(np.float64) - Vo)
    ratio = err / np.where(S > 0, S, 1.0)
    worst = int(np.argmax(ratio)) if ratio.size else 0
    assert np.all(np.isfinite(Vg)), f"{label}: non-finite output"
    assert np.all(err <= TOL * S), (
        f"{label}: max |err|/S = {ratio.max():.3e} at node {worst} "
        f"(gpu {Vg[worst]!r}, oracle {Vo[worst]!r}, S {S[worst]!r})")
    return float(ratio.max()) if ratio.size else 0.0


CASES = [
    # (n_atoms, dims, spacing, origin, box_lo, box_hi, seed)
    (1, (1, 1, 1), 0.5, (0.0, 0.0, 0.0), (-2, -2, -2), (2, 2, 2), 1),
    (3, (13, 7, 3), 0.5, (0.0, 0.0, 0.0), (0, 0, 0), (6, 3, 1), 2),
    (63, (17, 9, 5), 0.3, (-1.0, 0.5, 2.0), (-2, 0, 1), (5, 4, 4), 3),
    (65, (100, 1, 1), 0.5, (0.0, 0.0, 0.0), (-5, -1, -1), (55, 1, 1), 4),
    (257, (1, 100, 3), 0.25, (3.0, -4.0, 0.0), (0, -6, -1), (6, 22, 2), 5),
    (1000, (33, 31, 29), 0.5, (-8.0, -7.5, -7.0), (-12, -12, -12), (12, 12, 12), 6),
    (4099, (64, 64, 16), 0.5, (0.0, 0.0, 0.0), (-10, -10, -10), (42, 42, 18), 7),
    (70_000, (24, 20, 18), 1.0, (0.0, 0.0, 0.0), (-5, -5, -5), (30, 30, 30), 8),
]


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
@pytest.mark.parametrize("case", CASES, ids=[f"n{c[0]}_{c[1][0]}x{c[1][1]}x{c[1][2]}" for c in CASES])
def test_direct_small_all_nodes(torch, case, split):
    n, dims, h, origin, lo, hi, seed = case
    atoms = wl.random_atoms(n, lo, hi, seed=seed)
    lat = Lattice(*dims, h, origin)
    print(f"[direct] n={n} dims={dims} h={h} origin={origin} plan={cpmap.direct_plan(n, lat, split)}",
          flush=True)
    Vg = _run_direct(torch, atoms, lat, split)
    Vo, S = oracle.direct(atoms, dims, h, origin, with_scale=True)
    _assert_parity(Vg, Vo, S, f"n={n} dims={dims}")


def test_direct_no_atoms_writes_zeros(torch):
    lat = Lattice(9, 5, 3, 0.5)
    out = torch.full((3, 5, 9), 7.0, device="cuda")
    V = cpmap.direct(torch.zeros((0, 4), device="cuda"), lat, out=out)
    torch.cuda.synchronize()
    assert torch.all(V == 0).item()


def test_direct_zero_charges_and_far_atoms(torch):
    """q = 0 atoms add exactly nothing; atoms far outside the lattice count."""
    atoms = wl.random_atoms(300, (-50, -50, -50), (60, 60, 60), seed=9)
    atoms[::3, 3] = 0.0
    lat = Lattice(11, 10, 9, 0.5, (2.0, 2.0, 2.0))
    Vg = _run_direct(torch, atoms, lat)
    Vo, S = oracle.direct(atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    _assert_parity(Vg, Vo, S, "zero/far")
    nz = atoms[atoms[:, 3] != 0]
    Vg2 = _run_direct(torch, nz, lat)
    Vo2 = oracle.direct(nz, lat.dims, lat.spacing, lat.origin)
    _assert_parity(Vg2, Vo2, S, "zero charges removed")


# One geometry per compiled kernel variant (nodes per lane x, y, z; waves per
# workgroup), each with ragged lattice edges; the planner's choice for each
# is pinned on the CPU in test_abi.py.
VARIANT_CASES = [
    ((8, 8, 2, 4), 8000, (97, 5, 151), True),
    ((8, 8, 2, 8), 8000, (97, 73, 15), True),
    ((8, 4, 2, 4), 8000, (13, 73, 47), True),
    ((8, 4, 2, 8), 300, (57, 57, 151), True),
    ((4, 4, 2, 8), 8000, (3, 37, 151), True),
    ((4, 4, 2, 16), 300, (41, 37, 151), True),
    ((4, 4, 1, 16), 300, (97, 19, 67), True),
    ((2, 2, 1, 16), 300, (65, 11, 23), True),
    ((1, 1, 1, 16), 300, (3, 5, 1), True),
]


@pytest.mark.parametrize("variant,n,dims,split", VARIANT_CASES,
                         ids=["x".join(map(str, c[0])) for c in VARIANT_CASES])
def test_direct_each_compiled_variant_all_nodes(torch, variant, n, dims, split):
    lat = Lattice(*dims, 0.5, (-1.25, 0.5, 2.0))
    plan = cpmap.direct_plan(n, lat, split)
    print(f"[direct variant] {variant} n={n} dims={dims} plan={plan}", flush=True)
    lo = np.array(lat.origin) - 5.0
    hi = np.array(lat.origin) + np.array(dims) * lat.spacing + 5.0
    atoms = wl.random_atoms(n, lo, hi, seed=sum(dims) + n)
    Vg = _run_direct(torch, atoms, lat, split)
    Vo, S = oracle.direct(atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    _assert_parity(Vg, Vo, S, f"variant {variant}")


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_direct_same_sign_charges_large_n(torch, split):
    """All-positive charges over many atoms: the blocked fp32 sum must stay
    inside the bound even though no cancellation hides rounding."""
    atoms = wl.random_atoms(200_000, (0, 0, 0), (20, 20, 20), seed=10, q_lo=0.0, q_hi=1.0)
    lat = Lattice(16, 12, 10, 1.25, (0.1, 0.2, 0.3))
    Vg = _run_direct(torch, atoms, lat, split)
    Vo, S = oracle.direct(atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    worst = _assert_parity(Vg, Vo, S, "same sign")
    print(f"same-sign worst |err|/S = {worst:.3e}")


@pytest.mark.parametrize("split", [False, True])
def test_atom_on_a_node_gives_infinity(torch, split):
    """An atom exactly on a node (at the node's fp32 position) makes that
    node's potential +inf (positive charge) or -inf (negative), as the
    boundary documents; every other node stays finite and meets the bound,
    in the direct sum and in both cutoff terms."""
    lat = Lattice(23, 17, 11, 0.5, (1.0, -2.0, 0.25))
    atoms_np = wl.random_atoms(300, (0, -3, -1), (12, 7, 6), seed=71)
    on = {1234: 0.75, 2500: -0.5}  # node index -> charge of the atom placed on it
    for g, q in on.items():
        _, xyz = cpmap.node_position(lat, g)
        atoms_np = np.vstack([atoms_np, np.array([[*xyz, q]], dtype=np.float32)])
    Vg = _run_direct(torch, atoms_np, lat, split=split)
    keep = np.ones(lat.n_points, dtype=bool)
    for g, q in on.items():
        assert Vg[g] == (np.inf if q > 0 else -np.inf), (g, Vg[g])
        keep[g] = False
    Vo, S = oracle.direct(atoms_np, lat.dims, lat.spacing, lat.origin, with_scale=True)
    _assert_parity(Vg[keep], Vo[keep], S[keep], "atoms on nodes, direct")
    atoms = torch.from_numpy(np.ascontiguousarray(atoms_np)).cuda()
    ws = cpmap.bin_atoms(atoms, lat, 2.0, 4.0)
    for term, fn in (("smoothed", oracle.cutoff), ("truncated", oracle.cutoff_hard)):
        Vc = cpmap.cutoff(ws, atoms_np.shape[0], lat, 2.0, 4.0, term=term).cpu().numpy()
        Vc = Vc.reshape(-1)
        for g, q in on.items():
            assert Vc[g] == (np.inf if q > 0 else -np.inf), (term, g, Vc[g])
        Vo, S = fn(atoms_np, lat.dims, lat.spacing, lat.origin, 4.0, with_scale=True)
        _assert_parity(Vc[keep], Vo[keep], S[keep], f"atoms on nodes, cutoff {term}")


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
def test_direct_is_deterministic(torch, split):
    atoms = torch.from_numpy(wl.random_atoms(50_000, (0, 0, 0), (20, 20, 20), seed=12)).cuda()
    lat = Lattice(80, 60, 40, 0.25)
    a = cpmap.direct(atoms, lat, split=split).clone()
    b = cpmap.direct(atoms, lat, split=split)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_direct_planner_occupancy_table_matches_device(torch):
    """The planner's per-variant occupancy table equals what the runtime
    reports for the compiled kernels (a mismatch would only cost speed)."""
    assert cpmap.library().cpmap_direct_occupancy_check() == 0


def test_direct_split_workspace_is_used_and_reusable(torch):
    """A caller-provided workspace is accepted, reused across calls of the
    same size, and a too-small one is refused."""
    w = wl.full_direct()
    lat = w.lattice
    need = cpmap.direct_workspace_bytes(w.n_atoms, lat)
    assert need > 0
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    a = cpmap.direct(atoms, lat, workspace=ws).clone()
    b = cpmap.direct(atoms, lat, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.direct(atoms, lat, workspace=ws[: need - 256])
    assert e.value.status == 3


def test_direct_rejects_unbinned_geometry_errors(torch):
    atoms = torch.zeros((10, 4), device="cuda")
    with pytest.raises(ValueError):
        cpmap.direct(atoms, Lattice(2, 2, 2, 0.5), out=torch.zeros(7, device="cuda"))
    with pytest.raises(cpmap.CpmapError):
        cpmap.direct(atoms, Lattice(2, 2, 2, 0.0))


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
@pytest.mark.parametrize("index", [1, 2])
def test_direct_workload_all_nodes(torch, index, split):
    w = wl.workload(index)
    lat = w.lattice
    print(f"[direct] workload {w.name} plan={cpmap.direct_plan(w.n_atoms, lat, split)}", flush=True)
    Vg = _run_direct(torch, w.atoms, lat, split)
    Vo, S = oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    worst = _assert_parity(Vg, Vo, S, w.name)
    print(f"{w.name}: worst |err|/S = {worst:.3e}")


@pytest.mark.parametrize("split", [False, True], ids=["plain", "split"])
@pytest.mark.parametrize("index", [3, 4])
def test_direct_workload_checked_nodes(torch, index, split):
    w = wl.workload(index)
    lat = w.lattice
    print(f"[direct] workload {w.name} plan={cpmap.direct_plan(w.n_atoms, lat, split)}", flush=True)
    Vg = _run_direct(torch, w.atoms, lat, split)
    nodes = wl.checked_nodes(lat)
    Vo, S = oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, nodes=nodes, with_scale=True)
    worst = _assert_parity(Vg[nodes], Vo, S, w.name)
    print(f"{w.name}: {nodes.size} nodes, worst |err|/S = {worst:.3e}")


# ---------------------------------------------------------------- scatter contrast

@pytest.mark.parametrize("case", CASES[:6], ids=[f"n{c[0]}_{c[1][0]}x{c[1][1]}x{c[1][2]}" for c in CASES[:6]])
def test_scatter_small_all_nodes(torch, case):
    """The atomics-based scatter meets the same bound (its summation order
    varies from run to run)."""
    n, dims, h, origin, lo, hi, seed = case
    atoms_np = wl.random_atoms(n, lo, hi, seed=seed)
    lat = Lattice(*dims, h, origin)
    atoms = torch.from_numpy(atoms_np).cuda()
    V = cpmap.direct_scatter(atoms, lat).cpu().numpy().reshape(-1)
    Vo, S = oracle.direct(atoms_np, dims, h, origin, with_scale=True)
    _assert_parity(V, Vo, S, f"scatter n={n} dims={dims}")


@pytest.mark.parametrize("index", [1, 2])
def test_scatter_workloads(torch, index):
    w = wl.workload(index)
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    out = torch.full((lat.nz, lat.ny, lat.nx), 5.0, device="cuda")  # must be overwritten
    V = cpmap.direct_scatter(atoms, lat, out=out).cpu().numpy().reshape(-1)
    Vo, S = oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, with_scale=True)
    worst = _assert_parity(V, Vo, S, "scatter " + w.name)
    print(f"scatter {w.name}: worst |err|/S = {worst:.3e}")
