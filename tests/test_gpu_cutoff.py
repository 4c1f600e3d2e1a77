"""GPU parity of the cutoff path against the fp64 oracle.

cpmap_bin_atoms is integer work decided in fp32 (bin coordinate = fl(fl(p -
b0)/bs), the same operations on both sides): its CSR must equal the oracle's
stable counting sort bit for bit.  cpmap_cutoff must satisfy
|V_gpu - V_oracle| <= 1e-5 * S_c at every checked node, S_c = sum over
r < rc of |q|/r (so nodes with no atom inside the cutoff must be exactly 0).
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


def _bin(torch, atoms_np, lat, bs, rc):
    atoms = torch.from_numpy(np.ascontiguousarray(atoms_np, dtype=np.float32)).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    starts, srt = cpmap.workspace_views(ws, atoms_np.shape[0], lat, bs, rc)
    torch.cuda.synchronize()
    return atoms, ws, starts.cpu().numpy(), srt.cpu().numpy()


def _check_csr(torch, atoms_np, lat, bs, rc):
    _, ws, starts, srt = _bin(torch, atoms_np, lat, bs, rc)
    o_starts, o_sorted, _ = oracle.bin_atoms(atoms_np, lat.dims, lat.spacing, lat.origin, bs, rc)
    np.testing.assert_array_equal(starts, o_starts)
    kept = int(o_starts[-1])
    assert srt[:kept].tobytes() == o_sorted.tobytes()
    return ws


BIN_CASES = [
    # (n, lattice, bs, rc, box_lo, box_hi, seed)
    (1, Lattice(5, 5, 5, 0.5), 1.0, 2.0, (0, 0, 0), (2, 2, 2), 1),
    (777, Lattice(37, 21, 13, 0.5, (1.0, -2.0, 0.25)), 1.5, 3.0, (-5, -8, -5), (25, 12, 12), 2),
    (5000, Lattice(30, 30, 30, 0.3, (-4.0, 0.0, 2.0)), 1.0, 2.5, (-8, -4, -2), (8, 13, 14), 3),
    (70_000, Lattice(64, 48, 40, 0.5), 2.0, 6.0, (-10, -10, -10), (42, 34, 30), 4),
    (3000, Lattice(200, 200, 200, 0.5), 0.25, 12.0, (0, 0, 0), (100, 100, 100), 5),  # 3 radix passes
    # 196 radix tiles: the digit scan's 50,176 counts take four rounds of
    # 16,384, the last one partial, linked by the carry
    (400_000, Lattice(64, 48, 40, 0.5), 1.0, 3.0, (-4, -4, -4), (36, 28, 24), 8),
]


@pytest.mark.parametrize("case", BIN_CASES, ids=[f"n{c[0]}_bs{c[2]}" for c in BIN_CASES])
def test_bin_atoms_bit_exact(torch, case):
    n, lat, bs, rc, lo, hi, seed = case
    print(f"[bin] n={n} dims={lat.dims} bs={bs} rc={rc}", flush=True)
    atoms = wl.random_atoms(n, lo, hi, seed=seed)
    _check_csr(torch, atoms, lat, bs, rc)


def test_bin_atoms_edge_cases(torch):
    """No atoms; every atom in one bin (order kept); atoms on bin faces, outside
    the halo, and with NaN coordinates (dropped on both sides)."""
    lat = Lattice(8, 8, 8, 1.0)
    _check_csr(torch, np.zeros((0, 4), np.float32), lat, 2.0, 3.0)
    same = wl.random_atoms(5000, (2.0, 2.0, 2.0), (2.5, 2.5, 2.5), seed=6)
    _check_csr(torch, same, lat, 2.0, 3.0)
    faces = np.array([[0, 0, 0, 1], [2, 0, 0, 1], [-4, -4, -4, 1], [-4.001, 0, 0, 1],
                      [13.999, 0, 0, 1], [14, 0, 0, 1], [np.nan, 0, 0, 1], [1e30, 0, 0, 1],
                      [-1e30, 0, 0, 1], [1.0, 1.0, 1.0, 0.0]], dtype=np.float32)
    _check_csr(torch, faces, lat, 2.0, 3.0)


def test_bin_atoms_config5_bit_exact(torch):
    w = wl.cutoff_binned()
    _check_csr(torch, w.atoms, w.lattice, w.bin_size, w.cutoff)


def test_bin_atoms_is_deterministic(torch):
    atoms_np = wl.random_atoms(50_000, (0, 0, 0), (20, 20, 20), seed=7)
    lat = Lattice(40, 40, 40, 0.5)
    _, ws1, s1, a1 = _bin(torch, atoms_np, lat, 2.0, 6.0)
    _, ws2, s2, a2 = _bin(torch, atoms_np, lat, 2.0, 6.0)
    assert np.array_equal(s1, s2) and a1.tobytes() == a2.tobytes()


def _parity(Vg, Vo, S, label):
    err = np.abs(Vg.astype(np.float64) - Vo)
    bad = ~(err <= TOL * S)
    if bad.any():
        i = int(np.argmax(np.where(bad, err, -1)))
        raise AssertionError(f"{label}: {bad.sum()} nodes out of bound; node {i}: gpu {Vg[i]!r} "
                             f"oracle {Vo[i]!r} S {S[i]!r}")
    ratio = err / np.where(S > 0, S, 1.0)
    return float(ratio.max()) if ratio.size else 0.0


CUT_CASES = [
    (1, Lattice(9, 9, 9, 0.5), 1.0, 2.0, (1, 1, 1), (3, 3, 3), 11),
    (500, Lattice(19, 13, 11, 0.5), 1.0, 2.0, (-3, -3, -3), (12, 9, 8), 12),
    (2000, Lattice(37, 21, 13, 0.5, (1.0, -2.0, 0.25)), 1.5, 3.0, (-5, -8, -5), (25, 12, 12), 13),
    (4000, Lattice(30, 30, 30, 0.3, (-4.0, 0.0, 2.0)), 1.0, 2.5, (-8, -4, -2), (8, 13, 14), 14),
    (20_000, Lattice(48, 40, 33, 0.5), 4.0, 12.0, (-14, -14, -14), (38, 34, 30), 15),
    (6000, Lattice(24, 24, 24, 0.5), 0.5, 3.0, (-4, -4, -4), (16, 16, 16), 16),  # many rows per tile
]


@pytest.mark.parametrize("case", CUT_CASES, ids=[f"n{c[0]}_{c[1].nx}x{c[1].ny}x{c[1].nz}_bs{c[2]}" for c in CUT_CASES])
def test_cutoff_small_all_nodes(torch, case):
    n, lat, bs, rc, lo, hi, seed = case
    print(f"[cutoff] n={n} dims={lat.dims} bs={bs} rc={rc}", flush=True)
    atoms_np = wl.random_atoms(n, lo, hi, seed=seed)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    V = cpmap.cutoff(ws, n, lat, bs, rc).cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    _parity(V, Vo, S, f"n={n} dims={lat.dims}")


def test_cutoff_zero_far_from_atoms(torch):
    """Nodes farther than rc from every atom are exactly 0, including whole
    tiles whose neighbourhood is empty."""
    atoms_np = wl.random_atoms(400, (0, 0, 0), (6, 6, 6), seed=17)
    lat = Lattice(40, 16, 16, 0.5)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, 1.0, 3.0)
    V = cpmap.cutoff(ws, 400, lat, 1.0, 3.0).cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff(atoms_np, lat.dims, lat.spacing, lat.origin, 3.0, with_scale=True)
    assert np.all(V[S == 0] == 0.0) and (S == 0).sum() > 1000
    _parity(V, Vo, S, "far")


def test_cutoff_no_atoms(torch):
    lat = Lattice(10, 10, 10, 0.5)
    ws = cpmap.bin_atoms(torch.zeros((0, 4), device="cuda"), lat, 1.0, 2.0)
    out = torch.full((10, 10, 10), 3.0, device="cuda")
    V = cpmap.cutoff(ws, 0, lat, 1.0, 2.0, out=out)
    torch.cuda.synchronize()
    assert torch.all(V == 0).item()


# Cutoffs for which, on gfx950, no r^2 within 64 ulps below fl(rc*rc) makes
# the fp32 smoothed term exactly 0 (found with a probe of that search using
# the hardware rsq), so the kernel sums with its compare-and-select mask
# instead of the r^2 clamp; 12.0 takes the clamp.  The parity bar is the
# same either way.
FALLBACK_CUTOFFS = [1.02, 11.91, 12.55, 12.0]


@pytest.mark.parametrize("rc", FALLBACK_CUTOFFS)
def test_cutoff_select_and_clamp_cutoffs_all_nodes(torch, rc):
    print(f"[cutoff select/clamp] rc={rc}", flush=True)
    bs = rc / 3.0
    lat = Lattice(26, 22, 18, 0.5, (0.5, -1.0, 2.0))
    lo = np.array(lat.origin) - rc
    hi = np.array(lat.origin) + np.array(lat.dims) * lat.spacing + rc
    n = 3000
    atoms_np = wl.random_atoms(n, lo, hi, seed=int(rc * 100))
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    V = cpmap.cutoff(ws, n, lat, bs, rc).cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    _parity(V, Vo, S, f"rc={rc}")
    assert np.all(V[S == 0] == 0.0)


def test_cutoff_config5_checked_nodes(torch):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, w.bin_size, w.cutoff)
    V = cpmap.cutoff(ws, w.n_atoms, lat, w.bin_size, w.cutoff).cpu().numpy().reshape(-1)
    nodes = wl.checked_nodes(lat)
    Vo, S = oracle.cutoff(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=nodes,
                          with_scale=True)
    worst = _parity(V[nodes], Vo, S, w.name)
    print(f"{w.name}: {nodes.size} nodes, worst |err|/S = {worst:.3e}")


def test_cutoff_is_deterministic_and_checks_geometry(torch):
    atoms_np = wl.random_atoms(30_000, (0, 0, 0), (20, 20, 20), seed=18)
    lat = Lattice(40, 40, 40, 0.5)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, 2.0, 6.0)
    a = cpmap.cutoff(ws, 30_000, lat, 2.0, 6.0).clone()
    b = cpmap.cutoff(ws, 30_000, lat, 2.0, 6.0)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    with pytest.raises(cpmap.CpmapError) as e:
        cpmap.cutoff(ws, 30_000, Lattice(40, 40, 41, 0.5), 2.0, 6.0)
    assert e.value.status in (3, 4)  # ENOSPC or EGEOM: never a launch on a foreign layout
    with pytest.raises(cpmap.CpmapError):
        cpmap.cutoff(ws, 29_999, lat, 2.0, 6.0)


def test_cutoff_matches_direct_minus_gamma_for_huge_cutoff(torch):
    """With rc beyond every distance the cutoff path keeps every atom: compare
    with the oracle's cutoff sum, which then differs from the direct sum only
    by the smoothing polynomial."""
    atoms_np = wl.random_atoms(3000, (0, 0, 0), (8, 8, 8), seed=19)
    lat = Lattice(16, 16, 16, 0.5)
    atoms = torch.from_numpy(atoms_np).cuda()
    rc = 40.0
    ws = cpmap.bin_atoms(atoms, lat, 8.0, rc)
    V = cpmap.cutoff(ws, 3000, lat, 8.0, rc).cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    _parity(V, Vo, S, "huge rc")


# ---------------------------------------------------------------- truncated term

@pytest.mark.parametrize("case", CUT_CASES, ids=[f"n{c[0]}_{c[1].nx}x{c[1].ny}x{c[1].nz}_bs{c[2]}" for c in CUT_CASES])
def test_truncated_small_all_nodes(torch, case):
    n, lat, bs, rc, lo, hi, seed = case
    print(f"[truncated] n={n} dims={lat.dims} bs={bs} rc={rc}", flush=True)
    atoms_np = wl.random_atoms(n, lo, hi, seed=seed)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    V = cpmap.cutoff(ws, n, lat, bs, rc, term="truncated").cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff_hard(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    _parity(V, Vo, S, f"truncated n={n} dims={lat.dims}")


def test_truncated_boundary_decisions(torch):
    """Atoms one fp32 ulp inside, exactly at and one ulp outside rc of lattice
    nodes (along each axis), plus bin faces: the kernel keeps and drops
    exactly the atoms the oracle's fp32 test does."""
    h = np.float32(0.7)  # rc / h is not an integer: no atom lands on a node
    lat = Lattice(16, 16, 16, float(h))
    rc = 3.0
    pts = []
    rng = np.random.default_rng(21)
    for _ in range(300):
        node = rng.integers(0, 16, size=3).astype(np.float32) * h  # one fp32 rounding
        ax = int(rng.integers(0, 3))
        sgn = 1.0 if rng.random() < 0.5 else -1.0
        for r in (np.nextafter(np.float32(rc), np.float32(0)), np.float32(rc),
                  np.nextafter(np.float32(rc), np.float32(10))):
            p = node.astype(np.float32).copy()
            p[ax] = np.float32(p[ax] + sgn * r)
            pts.append([*p, rng.uniform(-1, 1)])
    atoms_np = np.array(pts, dtype=np.float32)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, 1.0, rc)
    V = cpmap.cutoff(ws, atoms_np.shape[0], lat, 1.0, rc, term="truncated").cpu().numpy().reshape(-1)
    Vo, S = oracle.cutoff_hard(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    _parity(V, Vo, S, "truncated boundary")


def _boundary_atoms():
    """Atoms within a few ulps of rc = 3 from a node at the origin on which the
    case-study listing's fp32 r2 = dx*dx + dy*dy + dz*dz disagrees with the
    exact distance, an fma chain or the reversed sum (tests/golden/
    truncated_boundary.json; the oracle pins re-derive each disagreement in
    exact arithmetic)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "truncated_boundary.json")) as f:
        fx = json.load(f)
    return [(c["kind"], c["atom"]) for c in fx["cases"]]


@pytest.mark.parametrize("kind,atom", _boundary_atoms(), ids=[k for k, _ in _boundary_atoms()])
@pytest.mark.parametrize("bs", [1.0, 1.5, 4.0])
def test_truncated_decision_follows_the_listing(torch, kind, atom, bs):
    print(f"[truncated listing decision] {kind} bs={bs}", flush=True)
    atoms_np = np.array([[*atom, 0.75]], dtype=np.float32)
    lat = Lattice(1, 1, 1, 1.0)
    ws = cpmap.bin_atoms(torch.from_numpy(atoms_np).cuda(), lat, bs, 3.0)
    V = cpmap.cutoff(ws, 1, lat, bs, 3.0, term="truncated").cpu().numpy().reshape(-1)
    Vo = oracle.cutoff_hard(atoms_np, lat.dims, lat.spacing, lat.origin, 3.0)
    kept = "listing_keeps" in kind
    if kept:
        assert Vo[0] != 0.0 and abs(V[0] - Vo[0]) <= 1e-5 * abs(Vo[0])
    else:
        assert Vo[0] == 0.0 and V[0] == 0.0


def _long_axis_case():
    """Atoms at every fp32 value within 4 ulps of 60 bin faces near x = 1e6 A
    on a 2^24-node axis (h = 1/16, bins of 1.3 A, rc = 1.505 A): some land,
    by their fp32 bin coordinate, in a bin whose box they lie just outside of,
    and a node within rc of them sits in a tile whose box is more than rc
    from that bin (the host test of the neighbourhood counts these pairs)."""
    nx, h, o, bs, rc = 1 << 24, 0.0625, 0.3, 1.3, 1.505
    lat = Lattice(nx, 1, 1, h, (o, 0.0, 0.0))
    _, b0, _ = oracle.bin_grid(lat.dims, h, lat.origin, bs, rc)
    c0 = int((1e6 - float(b0[0])) / bs) - 60
    rng = np.random.default_rng(23)
    pts = []
    for c in range(c0, c0 + 60):
        f = np.float32(float(b0[0]) + c * bs)
        vals = [f]
        for _ in range(4):
            vals = [np.nextafter(vals[0], np.float32(-np.inf))] + vals + \
                   [np.nextafter(vals[-1], np.float32(np.inf))]
        pts += [[float(v), float(np.float32(o)), 0.0, rng.uniform(-1, 1)] for v in vals]
    atoms = np.array(pts, dtype=np.float32)
    lo = int(np.floor((atoms[:, 0].min() - rc - np.float32(o)) / h)) - 8
    hi = int(np.ceil((atoms[:, 0].max() + rc - np.float32(o)) / h)) + 8
    near = np.arange(lo, hi, dtype=np.int64)
    far = np.random.default_rng(24).integers(0, lo - 100, size=2000).astype(np.int64)
    return lat, bs, rc, atoms, near, far


@pytest.mark.parametrize("term", ["truncated", "smoothed"])
def test_cutoff_long_axis_misbinned_atoms(torch, term):
    print(f"[cutoff long axis] term={term}", flush=True)
    lat, bs, rc, atoms_np, near, far = _long_axis_case()
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    V = cpmap.cutoff(ws, atoms_np.shape[0], lat, bs, rc, term=term).cpu().numpy().reshape(-1)
    fn = oracle.cutoff_hard if term == "truncated" else oracle.cutoff
    Vo, S = fn(atoms_np, lat.dims, lat.spacing, lat.origin, rc, nodes=near, with_scale=True)
    assert (S > 0).sum() > 1000
    _parity(V[near], Vo, S, f"long axis {term}")
    assert np.all(V[far] == 0.0)


def test_truncated_config5_checked_nodes(torch):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).cuda()
    ws = cpmap.bin_atoms(atoms, lat, w.bin_size, w.cutoff)
    V = cpmap.cutoff(ws, w.n_atoms, lat, w.bin_size, w.cutoff, term="truncated").cpu().numpy().reshape(-1)
    nodes = wl.checked_nodes(lat)
    Vo, S = oracle.cutoff_hard(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=nodes,
                               with_scale=True)
    worst = _parity(V[nodes], Vo, S, w.name + " truncated")
    print(f"{w.name} truncated: {nodes.size} nodes, worst |err|/S = {worst:.3e}")


def test_cutoff_rejects_unknown_term(torch):
    lat = Lattice(8, 8, 8, 0.5)
    ws = cpmap.bin_atoms(torch.zeros((4, 4), device="cuda"), lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.cutoff(ws, 4, lat, 1.0, 2.0, term="hard")


def test_binding_rejects_bad_buffers(torch):
    """Workspaces must be contiguous uint8 GPU tensors and extrema outputs
    int64/float32 pairs; each wrong buffer is refused before any launch."""
    lat = Lattice(8, 8, 8, 0.5)
    atoms = torch.zeros((4, 4), device="cuda")
    ws = cpmap.bin_atoms(atoms, lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.cutoff(ws.view(torch.int8), 4, lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.cutoff(ws.cpu(), 4, lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.bin_atoms(atoms, lat, 1.0, 2.0, workspace=ws[::2])
    with pytest.raises(ValueError):
        cpmap.bin_slots(ws, 4, lat, 1.0, 2.0, 2, slot_workspace=torch.empty(8, device="cuda"))
    with pytest.raises(ValueError):
        cpmap.cutoff_slots(ws.view(torch.int8), 4, lat, 1.0, 2.0, 2)
    with pytest.raises(ValueError):
        cpmap.direct(atoms, lat, split=True, workspace=torch.empty(64, device="cuda"))
    V = torch.zeros(lat.n_points, device="cuda")
    with pytest.raises(ValueError):
        cpmap.extrema(V, out=(torch.empty(2, dtype=torch.int32, device="cuda"),
                              torch.empty(2, device="cuda")))
    with pytest.raises(ValueError):
        cpmap.extrema(V, out=(torch.empty(1, dtype=torch.int64, device="cuda"),
                              torch.empty(2, device="cuda")))
    idx, val = cpmap.extrema(V, out=(torch.empty(2, dtype=torch.int64, device="cuda"),
                                     torch.empty(2, device="cuda")))
    assert val.tolist() == [0.0, 0.0]


# ---------------------------------------------------------------- workspace records

def _small_binned(torch, n=2000, seed=31):
    lat = Lattice(20, 18, 16, 0.5)
    atoms_np = wl.random_atoms(n, (-2, -2, -2), (12, 11, 10), seed=seed)
    atoms = torch.from_numpy(atoms_np).cuda()
    return lat, atoms_np, atoms


def test_workspace_overwritten_outside_the_library_gives_nan(torch):
    """A binned workspace whose header bytes changed since binning (here
    zeroed by torch) is not read: every node of V is NaN.  Rebinning it
    restores the map.  The same holds for a slot workspace built from it."""
    lat, atoms_np, atoms = _small_binned(torch)
    n = atoms_np.shape[0]
    ws = cpmap.bin_atoms(atoms, lat, 1.0, 3.0)
    good = cpmap.cutoff(ws, n, lat, 1.0, 3.0).clone()
    ws[:16].zero_()
    V = cpmap.cutoff(ws, n, lat, 1.0, 3.0)
    torch.cuda.synchronize()
    assert torch.isnan(V).all().item()
    Vt = cpmap.cutoff(ws, n, lat, 1.0, 3.0, term="truncated")
    assert torch.isnan(Vt).all().item()
    # slots built from the damaged workspace are refused by the cutoff kernels
    sws = cpmap.bin_slots(ws, n, lat, 1.0, 3.0, 4)
    Vs = cpmap.cutoff_slots(sws, n, lat, 1.0, 3.0, 4)
    torch.cuda.synchronize()
    assert torch.isnan(Vs).all().item()
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=ws)
    assert torch.equal(cpmap.cutoff(ws, n, lat, 1.0, 3.0), good)
    # a damaged slot header alone (capacity 4 overflows here, so the slot
    # map is compared with itself, not bit for bit with the CSR map)
    sws = cpmap.bin_slots(ws, n, lat, 1.0, 3.0, 4)
    slot_good = cpmap.cutoff_slots(sws, n, lat, 1.0, 3.0, 4).clone()
    torch.testing.assert_close(slot_good, good, rtol=1e-5, atol=1e-5)
    sws[8:16].fill_(1)
    assert torch.isnan(cpmap.cutoff_slots(sws, n, lat, 1.0, 3.0, 4)).all().item()


def test_writes_through_the_library_drop_overlapping_records(torch):
    """Any entry point that writes device memory drops the records of the
    workspaces it overlaps: rebinning through another base address, using the
    workspace as the direct sum's scratch or as an output, and the extrema
    outputs; afterwards the cutoff call returns CPMAP_EGEOM.  A workspace
    next to the written range keeps its record."""
    lat, atoms_np, atoms = _small_binned(torch)
    n = atoms_np.shape[0]
    need = cpmap.bin_workspace_bytes(n, lat, 1.0, 3.0)
    big = torch.empty(3 * need + 4096, dtype=torch.uint8, device="cuda")
    a = big[:need]
    b = big[need + 256: 2 * need + 256]   # after a, not touching it
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=a)
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=b)
    ref = cpmap.cutoff(a, n, lat, 1.0, 3.0).clone()

    def refused(ws):
        with pytest.raises(cpmap.CpmapError) as e:
            cpmap.cutoff(ws, n, lat, 1.0, 3.0)
        return e.value.status == 4

    # rebinning at an address inside a
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=big[256:256 + need])
    assert refused(a)
    assert torch.equal(cpmap.cutoff(b, n, lat, 1.0, 3.0), ref)  # b kept its record
    # the direct sum's output written over b's tail
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=a)
    assert torch.equal(cpmap.cutoff(a, n, lat, 1.0, 3.0), ref)
    small = Lattice(4, 4, 4, 0.5)
    out = big[2 * need:2 * need + 256].view(torch.float32).view(4, 4, 4)
    cpmap.direct(atoms[:10], small, out=out, split=False)
    assert refused(b)
    assert torch.equal(cpmap.cutoff(a, n, lat, 1.0, 3.0), ref)
    # the extrema outputs over a's first bytes
    idx = big[1024:1040].view(torch.int64)
    val = big[2048:2056].view(torch.float32)
    cpmap.extrema(ref.reshape(-1), out=(idx, val))
    assert refused(a)
    # a cutoff output over the workspace itself
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=b)
    cpmap.bin_atoms(atoms, lat, 1.0, 3.0, workspace=a)
    V = b[:256].view(torch.float32).view(4, 4, 4)
    cpmap.direct(atoms[:10], small, out=V, split=False)
    assert refused(b)
    assert torch.equal(cpmap.cutoff(a, n, lat, 1.0, 3.0), ref)


def test_reused_workspace_memory_is_refused_or_nan(torch):
    """A binned workspace freed and its memory handed to a new tensor that is
    then filled outside the library: the cutoff call either finds no record
    (CPMAP_EGEOM, new address) or finds the stale record and the kernel sees
    the changed header (NaN at every node) -- never a map computed from the
    new contents."""
    lat, atoms_np, atoms = _small_binned(torch)
    n = atoms_np.shape[0]
    need = cpmap.bin_workspace_bytes(n, lat, 1.0, 3.0)
    ws = cpmap.bin_atoms(atoms, lat, 1.0, 3.0)
    addr = ws.data_ptr()
    torch.cuda.synchronize()
    del ws
    ws2 = torch.empty(need, dtype=torch.uint8, device="cuda")
    ws2.fill_(7)
    try:
        V = cpmap.cutoff(ws2, n, lat, 1.0, 3.0)
    except cpmap.CpmapError as e:
        assert e.status == 4
        assert ws2.data_ptr() != addr
    else:
        torch.cuda.synchronize()
        assert ws2.data_ptr() == addr
        assert torch.isnan(V).all().item()


FAR = (8192.5, -4096.25, 2048.125)


@pytest.mark.parametrize("term", ["smoothed", "truncated"])
def test_far_from_the_origin(torch, term):
    """A lattice some 10^4 A from the origin, where an fp32 coordinate keeps
    about three decimal digits after the point: binning bit-exact, and both
    cutoff terms and the direct sum (plain and split) within the bound at
    every node."""
    lat = Lattice(33, 17, 9, 0.5, FAR)
    lo = (FAR[0] - 6.0, FAR[1] - 6.0, FAR[2] - 6.0)
    hi = (FAR[0] + 22.0, FAR[1] + 14.0, FAR[2] + 10.0)
    n, bs, rc = 1500, 2.0, 5.0
    print(f"[far origin] origin={FAR} dims={lat.dims} term={term}", flush=True)
    atoms_np = wl.random_atoms(n, lo, hi, seed=63)
    _check_csr(torch, atoms_np, lat, bs, rc)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    V = cpmap.cutoff(ws, n, lat, bs, rc, term=term).cpu().numpy().reshape(-1)
    ref = oracle.cutoff if term == "smoothed" else oracle.cutoff_hard
    Vo, S = ref(atoms_np, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    assert np.count_nonzero(S) > lat.n_points // 2
    _parity(V, Vo, S, f"far origin, {term}")
    Vdo, Sd = oracle.direct(atoms_np, lat.dims, lat.spacing, lat.origin, with_scale=True)
    for split in (False, True):
        Vd = cpmap.direct(atoms, lat, split=split).cpu().numpy().reshape(-1)
        _parity(Vd, Vdo, Sd, f"far origin, direct split={split}")
