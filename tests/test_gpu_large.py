"""Maximum-size cases on the GPU: lattices past 2^31 nodes (64-bit node
indices in every store and in the extrema scan) and an axis at the largest
dimension the library accepts (node coordinates exact up to 2^24).

The maps are too large to bring back whole; each check samples nodes (the
first and last, both sides of index 2^31, the nodes near the atoms, random
ones) and compares them with the fp64 oracle evaluated at exactly those
nodes, under the same bound as the other parity tests.  The extrema check
plants its extremes by construction.
"""
import numpy as np
import pytest

import oracle
import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import Lattice
from direct_coulomb_potential_amd import workloads as wl

pytestmark = pytest.mark.gpu

TOL = 1e-5
BIG = Lattice(2048, 1024, 1040, 0.5)  # 2,181,038,080 nodes (8.7 GB of V)


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


@pytest.fixture
def free_after(torch):
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _need_free_gb(torch, gb):
    """Skip (with the reason) when the device lacks the free memory a
    maximum-size case needs, rather than failing on allocation."""
    free, _ = torch.cuda.mem_get_info()
    if free < gb * 2**30:
        pytest.skip(f"needs {gb} GiB of free device memory, {free / 2**30:.0f} GiB free")


def _linear(lat, i, j, k):
    return (np.asarray(k, np.int64) * lat.ny + np.asarray(j, np.int64)) * lat.nx + np.asarray(i, np.int64)


def _sample_nodes(lat, atoms_np, seed, near=4):
    """First/last node, nodes on both sides of index 2^31, the lattice nodes
    nearest each atom and their neighbours, and random nodes."""
    n = lat.n_points
    picks = [np.array([0, 1, n - 2, n - 1], np.int64)]
    if n > 2**31 + 8:
        picks.append(np.arange(2**31 - 4, 2**31 + 4, dtype=np.int64))
    rng = np.random.default_rng(seed)
    picks.append(rng.integers(0, n, size=2000, dtype=np.int64))
    for a in atoms_np[:64]:
        c = np.floor((a[:3] - np.asarray(lat.origin)) / lat.spacing).astype(np.int64)
        off = np.arange(-near, near + 1)
        ii, jj, kk = np.meshgrid(c[0] + off, c[1] + off, c[2] + off, indexing="ij")
        ok = (ii >= 0) & (ii < lat.nx) & (jj >= 0) & (jj < lat.ny) & (kk >= 0) & (kk < lat.nz)
        picks.append(_linear(lat, ii[ok], jj[ok], kk[ok]))
    return np.unique(np.concatenate(picks))


def _gather(torch, V, nodes):
    idx = torch.from_numpy(nodes).to(V.device)
    return V.view(-1).index_select(0, idx).cpu().numpy()


def _parity(Vg, Vo, S, label):
    err = np.abs(Vg.astype(np.float64) - Vo)
    bad = ~(err <= TOL * S)
    if bad.any():
        i = int(np.argmax(np.where(bad, err, -1)))
        raise AssertionError(f"{label}: {bad.sum()} nodes out of bound; sample {i}: gpu {Vg[i]!r} "
                             f"oracle {Vo[i]!r} S {S[i]!r}")


def test_direct_past_2_31_nodes(torch, free_after):
    # atoms near the far corner (indices > 2^31) and near the origin
    far = wl.random_atoms(6, (1000.0, 480.0, 500.0), (1023.0, 511.0, 519.0), seed=51)
    near = wl.random_atoms(4, (0.3, 0.3, 0.3), (4.0, 4.0, 4.0), seed=52)
    atoms_np = np.concatenate([far, near])
    print(f"[large direct] dims={BIG.dims} nodes={BIG.n_points} atoms={len(atoms_np)}", flush=True)
    atoms = torch.from_numpy(atoms_np).cuda()
    V = cpmap.direct(atoms, BIG)
    nodes = _sample_nodes(BIG, atoms_np, seed=53)
    assert nodes.max() > 2**31 and nodes.max() == BIG.n_points - 1
    Vg = _gather(torch, V, nodes)
    del V
    Vo, S = oracle.direct(atoms_np, BIG.dims, BIG.spacing, BIG.origin, nodes=nodes, with_scale=True)
    _parity(Vg, Vo, S, "direct past 2^31")


def test_cutoff_and_slots_past_2_31_nodes(torch, free_after):
    bs, rc = 4.0, 12.0
    # z >= 512 A is k >= 1024, i.e. node index >= 2^31; ~8 atoms per 4 A bin
    far = wl.random_atoms(300, (1010.0, 500.0, 506.0), (1023.5, 511.5, 519.5), seed=54)
    near = wl.random_atoms(100, (-5.0, -5.0, -5.0), (10.0, 10.0, 10.0), seed=55)
    atoms_np = np.concatenate([far, near])
    print(f"[large cutoff] dims={BIG.dims} atoms={len(atoms_np)} bs={bs} rc={rc}", flush=True)
    atoms = torch.from_numpy(atoms_np).cuda()
    ws = cpmap.bin_atoms(atoms, BIG, bs, rc)
    nodes = _sample_nodes(BIG, atoms_np, seed=56, near=3)
    assert nodes.max() > 2**31
    V = cpmap.cutoff(ws, len(atoms_np), BIG, bs, rc)
    Vg = _gather(torch, V, nodes)
    Vo, S = oracle.cutoff(atoms_np, BIG.dims, BIG.spacing, BIG.origin, rc, nodes=nodes,
                          with_scale=True)
    _parity(Vg, Vo, S, "cutoff past 2^31")
    assert np.any(Vg[nodes > 2**31] != 0.0)
    # fixed-capacity bins on the same atoms (the far cluster overflows 4-slot bins)
    sws = cpmap.bin_slots(ws, len(atoms_np), BIG, bs, rc, 4)
    n_over = int(cpmap.slot_views(sws, len(atoms_np), BIG, bs, rc, 4)[1][-1].item())
    assert n_over > 0
    V = cpmap.cutoff_slots(sws, len(atoms_np), BIG, bs, rc, 4, out=V)
    _parity(_gather(torch, V, nodes), Vo, S, "cutoff slots past 2^31")
    del V, ws, sws


def test_extrema_past_2_31_nodes(torch, free_after):
    n = BIG.n_points
    V = torch.zeros(n, dtype=torch.float32, device="cuda")
    i_min, i_max = 2**31 + 5, n - 1
    V[i_min] = -3.0
    V[i_max] = 7.0
    V[2**31 - 1] = 7.0   # an equal maximum at a smaller index wins
    V[n - 10] = float("nan")
    idx, val = cpmap.extrema(V)
    assert idx.cpu().tolist() == [i_min, 2**31 - 1]
    assert val.cpu().tolist() == [-3.0, 7.0]
    del V


def test_direct_at_the_largest_axis(torch, free_after):
    """nx = 2^24 (the header's largest dimension): node x = fl(ox + i*h) stays
    exact at every i, and the last node is written."""
    lat = Lattice(1 << 24, 2, 2, 0.25, (-3.0, 0.0, 0.0))
    atoms_np = np.array([[1.0e6, 0.1, 0.2, 1.0], [4.0e6, 0.4, 0.3, -0.5],
                         [-1.0, 0.2, 0.1, 2.0]], dtype=np.float32)
    print(f"[largest axis] dims={lat.dims}", flush=True)
    atoms = torch.from_numpy(atoms_np).cuda()
    V = cpmap.direct(atoms, lat)
    nodes = _sample_nodes(lat, atoms_np, seed=57)
    assert nodes.max() == lat.n_points - 1
    Vg = _gather(torch, V, nodes)
    Vo, S = oracle.direct(atoms_np, lat.dims, lat.spacing, lat.origin, nodes=nodes, with_scale=True)
    _parity(Vg, Vo, S, "largest axis")
    with pytest.raises(cpmap.CpmapError):
        cpmap.direct(atoms, Lattice((1 << 24) + 1, 1, 1, 0.25))
    del V


def _positions_bins(torch, starts64, kept, nbins, p0, p1):
    """Bin of each sorted position in [p0, p1): the b with starts[b] <= p <
    starts[b + 1], and nbins for the dropped atoms past the kept ones."""
    pos = torch.arange(p0, p1, dtype=torch.int64, device="cuda")
    b = torch.searchsorted(starts64, pos, right=True) - 1
    return torch.where(pos < kept, b, torch.full_like(b, nbins))


@pytest.mark.parametrize("n", [5_000_003, 2**31 - 1], ids=["n5M", "n_max"])
def test_bin_atoms_at_the_largest_atom_count(torch, free_after, n):
    """n_atoms up to CPMAP_MAX_ATOMS (2^31 - 1): sorted positions, tile
    counts and bin starts reach the top of int32.  Each atom's charge carries
    its input index as raw bits, so every sorted atom names its origin;
    every 1000th atom lies outside the bin grid and is dropped.  Checked at
    every position: the sorted atoms are the input atoms, bit for bit, each
    input index once; bin starts rise from 0 to the kept count; every kept
    atom lies in the box of the bin its position falls in (up to the bin
    coordinate's rounding), dropped atoms sit past the kept ones, and equal
    bins keep input order.  At sampled positions the oracle's own bin of the
    input atom must contain the position."""
    lat, bs, rc = Lattice(200, 200, 200, 0.5), 1.0, 3.0  # 106^3 bins: 3 radix passes
    _need_free_gb(torch, 1 + n * 80 / 2**30)  # atoms, workspace, column copies, chunks
    bd, b0, _ = oracle.bin_grid(lat.dims, lat.spacing, lat.origin, bs, rc)
    nbx, nby, nbz = bd
    nbins = nbx * nby * nbz
    print(f"[max atoms] n={n} dims={lat.dims} bins={bd}", flush=True)
    chunk = 1 << 27
    gen = torch.Generator(device="cuda").manual_seed(58)
    atoms = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    lo = torch.tensor(b0 + 0.01, dtype=torch.float32, device="cuda")
    span = torch.tensor(np.asarray(bd, np.float32) * bs - 0.02, dtype=torch.float32,
                        device="cuda")
    ai = atoms.view(torch.int32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        atoms[s:e, :3] = lo + torch.rand((e - s, 3), generator=gen, device="cuda") * span
        ai[s:e, 3] = torch.arange(s, e, dtype=torch.int32, device="cuda")
    atoms[7::1000, 0] = 1.0e30
    kept = n - len(range(7, n, 1000))

    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    starts, srt = cpmap.workspace_views(ws, n, lat, bs, rc)
    torch.cuda.synchronize()
    print(f"[max atoms] binned n={n}", flush=True)
    assert int(starts[0]) == 0 and int(starts[-1]) == kept
    assert bool((starts[1:] >= starts[:-1]).all())
    starts64 = starts.long()

    # torch gathers from one tensor of fewer than 2^31 elements at a time:
    # the input atoms' four words and the sorted atoms' index word as columns
    si = srt.view(torch.int32)
    cols = [ai[:, k].contiguous() for k in range(4)]
    orig_all = si[:, 3].contiguous()
    seen = torch.zeros(n, dtype=torch.uint8, device="cuda")
    b0_64 = torch.tensor(b0.astype(np.float64), device="cuda")
    slack = 2.0 ** -20 * float(max(bd))  # far above the fp32 bin coordinate's error
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        e1 = min(n, e + 1)  # one position past the chunk, for the order check
        orig = orig_all[s:e1].long()
        assert int(orig.min()) >= 0 and int(orig.max()) < n
        seen[orig[:e - s]] = 1
        for k in range(4):
            assert bool((cols[k].index_select(0, orig[:e - s]) == si[s:e, k]).all()), \
                f"word {k} of the atoms in [{s}, {e})"
        bins = _positions_bins(torch, starts64, kept, nbins, s, e1)
        same = bins[1:] == bins[:-1]
        assert bool((~same | (orig[1:] > orig[:-1])).all()), f"input order in [{s}, {e1})"
        is_kept = bins[:e - s] < nbins
        t = (srt[s:e, :3].double() - b0_64) / bs
        c = torch.stack([bins[:e - s] % nbx, (bins[:e - s] // nbx) % nby,
                         bins[:e - s] // (nbx * nby)], dim=1).double()
        inside = ((t >= c - slack) & (t < c + 1 + slack)).all(dim=1)
        assert bool((inside | ~is_kept).all()), f"bin boxes in [{s}, {e})"
        assert bool(((srt[s:e, 0] == 1.0e30) | is_kept).all()), f"dropped atoms in [{s}, {e})"
    assert bool(seen.all())
    del seen

    rng = np.random.default_rng(59)
    picks = np.unique(np.concatenate([
        np.arange(0, 1 << 16), np.arange(n - (1 << 16), n),
        np.arange(kept - 512, min(n, kept + 512)),
        rng.integers(0, n, size=100_000)]).astype(np.int64))
    orig = orig_all.index_select(0, torch.from_numpy(picks).cuda()).long()
    sample = torch.stack([cols[k].index_select(0, orig) for k in range(4)], dim=1)
    sample = sample.view(torch.float32).cpu().numpy()
    _, _, bin_of = oracle.bin_atoms(sample, lat.dims, lat.spacing, lat.origin, bs, rc)
    st = starts.cpu().numpy().astype(np.int64)
    ok = np.where(bin_of >= 0,
                  (st[np.maximum(bin_of, 0)] <= picks) & (picks < st[np.maximum(bin_of, 0) + 1]),
                  picks >= kept)
    assert ok.all(), f"{(~ok).sum()} sampled positions outside their oracle bin"
    del atoms, ws, starts, srt, starts64, si, ai, cols, orig_all, orig


def test_direct_at_the_largest_atom_count(torch, free_after):
    """n_atoms = CPMAP_MAX_ATOMS (2^31 - 1) on a two-node lattice, with the
    atom split the library plans (32 parts of 16 waves): every part's and
    wave's atom slice, and the last atom index, reach the top of int32.
    Parity with the fp64 oracle at both nodes, under the usual bound."""
    n = 2**31 - 1
    lat = Lattice(2, 1, 1, 0.5)
    _need_free_gb(torch, 40)
    print(f"[max atoms direct] n={n} dims={lat.dims} plan={cpmap.direct_plan(n, lat)}",
          flush=True)
    gen = torch.Generator(device="cuda").manual_seed(60)
    atoms = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    chunk = 1 << 27
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        u = torch.rand((e - s, 4), generator=gen, device="cuda")
        atoms[s:e, :3] = u[:, :3] * 40.0 - 20.0
        atoms[s:e, 3] = u[:, 3] * 2.0 - 1.0
    V = cpmap.direct(atoms, lat)
    Vg = V.view(-1).cpu().numpy()
    atoms_np = atoms.cpu().numpy()
    del atoms, V
    print("[max atoms direct] oracle", flush=True)
    Vo, S = oracle.direct(atoms_np, lat.dims, lat.spacing, lat.origin, with_scale=True)
    _parity(Vg, Vo, S, "direct at 2^31 - 1 atoms")


def test_cutoff_neighbourhood_of_2_31_atoms(torch, free_after):
    """One tile whose bin neighbourhood holds all 2^31 - 1 atoms (an 8x8x8
    lattice, 4 A bins, rc = 2 A: the 3x3x3 bins around it), so the staging
    loop's last chunk starts at 2^31 - 256.  All but 64 atoms lie more than
    rc from every node (they are staged and tested, never summed); the 64
    near ones come last in input order and in the last bin, so they sit in
    that final chunk.  Atoms beyond rc add nothing to the smoothed term, so
    the oracle on the near atoms is the oracle on all of them."""
    n, n_near = 2**31 - 1, 64
    lat, bs, rc = Lattice(8, 8, 8, 0.5), 4.0, 2.0  # nodes in [0, 3.5]^3, bins from -4 to 8
    _need_free_gb(torch, 110)
    print(f"[max neighbourhood] n={n} dims={lat.dims} bins={cpmap.bin_grid(lat, bs, rc)}",
          flush=True)
    gen = torch.Generator(device="cuda").manual_seed(61)
    atoms = torch.empty((n, 4), dtype=torch.float32, device="cuda")
    n_far = n - n_near
    chunk = 1 << 27
    for s in range(0, n_far, chunk):
        e = min(n_far, s + chunk)
        u = torch.rand((e - s, 5), generator=gen, device="cuda")
        # x in [-3.99, -2.2] or [5.7, 7.99]: at least 2.2 A from the node box
        x = torch.where(u[:, 4] < 0.5, -3.99 + u[:, 0] * 1.79, 5.7 + u[:, 0] * 2.29)
        atoms[s:e, 0] = x
        atoms[s:e, 1:3] = -3.99 + u[:, 1:3] * 11.98
        atoms[s:e, 3] = u[:, 3] * 2.0 - 1.0
        assert float(x.abs().min()) >= 2.2 - 1e-6 and float((x - 3.5).abs().min()) >= 2.2 - 1e-6
    near = wl.random_atoms(n_near, (4.05, 4.05, 4.05), (4.6, 4.6, 4.6), seed=62)
    atoms[n_far:] = torch.from_numpy(near).cuda()
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    starts, srt = cpmap.workspace_views(ws, n, lat, bs, rc)
    # every atom is kept, and the near ones are the sorted array's last 64
    assert int(starts[-1]) == n
    assert torch.equal(srt[n_far:].cpu(), torch.from_numpy(near))
    print("[max neighbourhood] binned; cutoff", flush=True)
    V = cpmap.cutoff(ws, n, lat, bs, rc)
    Vg = V.view(-1).cpu().numpy()
    del atoms, ws, starts, srt, V
    Vo, S = oracle.cutoff(near, lat.dims, lat.spacing, lat.origin, rc, with_scale=True)
    assert np.count_nonzero(S) > 0
    _parity(Vg, Vo, S, "cutoff with 2^31 - 1 atoms in one neighbourhood")
