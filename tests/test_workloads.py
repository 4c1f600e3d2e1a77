"""The seeded input generators: determinism and the statistics each workload is
drawn to have (boxes, charge ranges, net charge, the exclusion around lattice
nodes, density).  The checks use their own arithmetic (a k-d tree for the
exclusion), not the generators' helpers."""
import numpy as np
import pytest
from scipy.spatial import cKDTree

from direct_coulomb_potential_amd import workloads as wl


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_generators_are_deterministic(index):
    a = wl.workload(index)
    b = wl.workload(index)
    assert a.atoms.tobytes() == b.atoms.tobytes()
    other = wl.WORKLOADS[index](seed=a.seed + 100)
    assert other.atoms.tobytes() != a.atoms.tobytes()
    assert a.atoms.dtype == np.float32 and a.atoms.shape[1] == 4


def _lattice_nodes(lat):
    i, j, k = np.meshgrid(np.arange(lat.nx), np.arange(lat.ny), np.arange(lat.nz), indexing="ij")
    o = np.asarray(lat.origin, np.float64)
    return np.stack([o[0] + i.ravel() * lat.spacing, o[1] + j.ravel() * lat.spacing,
                     o[2] + k.ravel() * lat.spacing], 1)


@pytest.mark.parametrize("index", [1, 2])
def test_plane_and_grid_atoms_keep_clear_of_every_node(index):
    """10k atoms in [0,50) x [0,50) x [0,25), charges in [-1, 1), none within
    0.05 A of any node of the full 100x100x50 lattice (also for the plane
    workload, which evaluates only its k = 10 plane)."""
    w = wl.workload(index)
    A = w.atoms.astype(np.float64)
    assert w.n_atoms == 10_000
    assert np.all(A[:, :3] >= 0) and np.all(A[:, 0] < 50) and np.all(A[:, 1] < 50)
    assert np.all(A[:, 2] < 25)
    assert np.all(A[:, 3] >= -1) and np.all(A[:, 3] < 1)
    d, _ = cKDTree(_lattice_nodes(wl.LATTICE_100x100x50)).query(A[:, :3], k=1)
    assert d.min() >= 0.05
    if index == 1:
        assert w.lattice.dims == (100, 100, 1) and w.lattice.origin[2] == 5.0


def test_large_direct_is_uniform_and_neutral():
    w = wl.large_direct()
    A = w.atoms.astype(np.float64)
    assert w.n_atoms == 200_000 and w.lattice.dims == (200, 200, 200)
    assert np.all(A[:, :3] >= 0) and np.all(A[:, :3] < 100)
    assert abs(A[:, 3].sum()) < 0.05            # shifted to net zero, then rounded to fp32
    assert np.all(np.abs(A[:, 3]) <= 1.01)  # U[-1, 1) minus its mean (~1e-3)
    # uniform: each of the 8 octants holds an eighth of the atoms (binomial, 5 sigma)
    octant = ((A[:, 0] >= 50).astype(int) + 2 * (A[:, 1] >= 50) + 4 * (A[:, 2] >= 50))
    counts = np.bincount(octant, minlength=8)
    assert np.all(np.abs(counts - 25_000) < 5 * np.sqrt(25_000 * 7 / 8))


def test_protein_atoms_are_clustered_and_neutral():
    w = wl.protein_direct()
    A = w.atoms.astype(np.float64)
    assert w.n_atoms == 40_000
    assert abs(A[:, 3].sum()) < 0.05
    # 20 clusters of sigma 6 A: the densest 4 A cells hold far more atoms
    # than a uniform draw would (40k atoms over the 100 A box: ~2.6 per cell)
    cells = np.floor(A[:, :3] / 4.0).astype(np.int64)
    _, per_cell = np.unique(cells, axis=0, return_counts=True)
    assert per_cell.max() > 40


def test_cutoff_workload_density_and_neighbourhoods():
    """0.1 atoms per cubic Angstrom (one per 10 A^3, the lecture's density);
    ~6.4 atoms per 4 A bin; an interior node has ~0.1 * 4/3 pi 12^3 = 724
    atoms within 12 A."""
    w = wl.cutoff_binned()
    A = w.atoms.astype(np.float64)
    assert w.n_atoms == 100_000 and w.cutoff == 12.0 and w.bin_size == 4.0
    assert np.all(A[:, :3] >= 0) and np.all(A[:, :3] < 100)
    assert np.all(A[:, 3] >= -1) and np.all(A[:, 3] < 1)
    cells = np.floor(A[:, :3] / 4.0).astype(np.int64)
    counts = np.bincount((cells[:, 2] * 25 + cells[:, 1]) * 25 + cells[:, 0], minlength=25**3)
    assert abs(counts.mean() - 6.4) < 1e-9 and 2.0 < counts.std() < 3.0
    rng = np.random.default_rng(3)
    interior = rng.uniform(20, 80, size=(500, 3))
    n_near = cKDTree(A[:, :3]).query_ball_point(interior, 12.0, return_length=True)
    assert abs(n_near.mean() - 0.1 * 4 / 3 * np.pi * 12**3) < 0.02 * 724


def test_checked_nodes_are_three_slices_plus_random():
    lat = wl.LATTICE_200
    nodes = wl.checked_nodes(lat)
    plane = lat.nx * lat.ny
    assert np.all(np.diff(nodes) > 0)
    for k in (0, 100, 199):
        assert np.isin(np.arange(k * plane, (k + 1) * plane), nodes).all()
    assert 3 * plane < nodes.size <= 3 * plane + 10_000
    assert nodes.min() >= 0 and nodes.max() < lat.n_points
    assert np.array_equal(nodes, wl.checked_nodes(lat))
