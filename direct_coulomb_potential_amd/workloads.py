"""Seeded synthetic workloads for potential-map runs.

This module only draws inputs: atom positions and charges, lattice geometry and
the sets of nodes a check samples.  It holds none of the method's arithmetic
(no distances, no potentials, no binning), so both the GPU path and the CPU
oracle's tests can take their inputs from it.

The workloads follow the pages' test systems:
  - a 100x100x50 lattice at 0.5 A with 10,000 random atoms, only the plane
    z-index 10 evaluated (the chapter-18 benchmark of the PMPP solutions
    article, section 1), and the same lattice in full;
  - 200^3 lattices at 0.5 A over a 100 A box (case-study notes, section 18.1:
    the ion-placement lattice) with protein-like clustered atoms or uniform
    atoms;
  - a cutoff system at 0.1 atoms per cubic Angstrom ("1 atom per 10 A^3", the
    binning lecture's bin-capacity slide), rc = 12 A (section 18.5), 4 A bins
    (the small-bin design slide).
The pages name no public dataset; these seeded draws stand in for the water
test systems and the 50k-1M atom structures the lecture mentions.

Every draw is fp64 from numpy's default_rng(seed), then cast to fp32.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Lattice:
    """A regular lattice: node (i,j,k) at origin + (i,j,k)*spacing, stored x-fastest."""
    nx: int
    ny: int
    nz: int
    spacing: float
    origin: Tuple[float, float, float] = (0.0, 0.0, 0.0)

    @property
    def dims(self) -> Tuple[int, int, int]:
        return (self.nx, self.ny, self.nz)

    @property
    def n_points(self) -> int:
        return self.nx * self.ny * self.nz


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    description: str
    atoms: np.ndarray            # (N, 4) float32: x, y, z, q
    lattice: Lattice             # the lattice that is evaluated
    cutoff: Optional[float] = None
    bin_size: Optional[float] = None
    seed: int = 0

    @property
    def n_atoms(self) -> int:
        return int(self.atoms.shape[0])

    @property
    def pairs(self) -> int:
        return self.n_atoms * self.lattice.n_points


def _uniform_positions(rng, n, box):
    lo = np.zeros(3)
    hi = np.asarray(box, dtype=np.float64)
    return rng.uniform(lo, hi, size=(n, 3))


def _near_node_mask(pos32, full: Lattice, min_dist: float):
    """True where a (float32-rounded) position lies within min_dist of a node of `full`.

    The nearest node along each axis is the rounded index, clamped to the lattice;
    the nearest node overall is the combination of the three.
    """
    p = pos32.astype(np.float64)
    near = np.zeros(p.shape[0], dtype=np.float64)
    for ax, n in enumerate(full.dims):
        o = full.origin[ax]
        idx = np.clip(np.rint((p[:, ax] - o) / full.spacing), 0, n - 1)
        near += (p[:, ax] - (o + idx * full.spacing)) ** 2
    return near < min_dist * min_dist


def _excluded_uniform_atoms(rng, n, box, full: Lattice, min_dist: float):
    pos = _uniform_positions(rng, n, box).astype(np.float32)
    q = rng.uniform(-1.0, 1.0, size=n)
    for _ in range(1000):
        bad = _near_node_mask(pos, full, min_dist)
        if not bad.any():
            break
        pos[bad] = _uniform_positions(rng, int(bad.sum()), box).astype(np.float32)
    else:  # pragma: no cover - probability ~0
        raise RuntimeError("exclusion resampling did not converge")
    atoms = np.empty((n, 4), dtype=np.float32)
    atoms[:, :3] = pos
    atoms[:, 3] = q.astype(np.float32)
    return atoms


def _shift_to_net_zero(q64):
    return q64 - q64.mean()


# ---- the five workloads --------------------------------------------------------

LATTICE_100x100x50 = Lattice(100, 100, 50, 0.5)
LATTICE_200 = Lattice(200, 200, 200, 0.5)


def plane_direct(seed: int = 1) -> Workload:
    """10k uniform atoms over the 50x50x25 A box; only plane k=10 (z = 5.0 A) evaluated."""
    rng = np.random.default_rng(seed)
    atoms = _excluded_uniform_atoms(rng, 10_000, (50.0, 50.0, 25.0), LATTICE_100x100x50, 0.05)
    lat = Lattice(100, 100, 1, 0.5, (0.0, 0.0, 5.0))
    return Workload("plane_100x100_k10_10k", "direct sum, plane k=10 of 100x100x50 @0.5A, 10k atoms",
                    atoms, lat, seed=seed)


def full_direct(seed: int = 2) -> Workload:
    """The same draw rule over the whole 100x100x50 lattice (500k points)."""
    rng = np.random.default_rng(seed)
    atoms = _excluded_uniform_atoms(rng, 10_000, (50.0, 50.0, 25.0), LATTICE_100x100x50, 0.05)
    return Workload("grid_100x100x50_10k", "direct sum, 100x100x50 @0.5A, 10k atoms",
                    atoms, LATTICE_100x100x50, seed=seed)


def protein_direct(seed: int = 3) -> Workload:
    """40k atoms in 20 Gaussian clusters (sigma 6 A, 2000 atoms each) around centres
    uniform in the central 60 A of the 100 A box; charges N(0, 0.4^2) shifted to net 0."""
    rng = np.random.default_rng(seed)
    n_clusters, per = 20, 2000
    centres = rng.uniform(20.0, 80.0, size=(n_clusters, 3))
    pos = np.concatenate([rng.normal(c, 6.0, size=(per, 3)) for c in centres])
    q = _shift_to_net_zero(rng.normal(0.0, 0.4, size=n_clusters * per))
    atoms = np.empty((n_clusters * per, 4), dtype=np.float32)
    atoms[:, :3] = pos.astype(np.float32)
    atoms[:, 3] = q.astype(np.float32)
    return Workload("protein_200cube_40k", "direct sum, 200^3 @0.5A, 40k clustered atoms",
                    atoms, LATTICE_200, seed=seed)


def large_direct(seed: int = 4) -> Workload:
    """200k atoms uniform in the 100 A box, charges U[-1,1] shifted to net 0; 200^3 lattice."""
    rng = np.random.default_rng(seed)
    pos = _uniform_positions(rng, 200_000, (100.0, 100.0, 100.0))
    q = _shift_to_net_zero(rng.uniform(-1.0, 1.0, size=200_000))
    atoms = np.empty((200_000, 4), dtype=np.float32)
    atoms[:, :3] = pos.astype(np.float32)
    atoms[:, 3] = q.astype(np.float32)
    return Workload("direct_200cube_200k", "direct sum, 200^3 @0.5A, 200k uniform atoms",
                    atoms, LATTICE_200, seed=seed)


def cutoff_binned(seed: int = 5) -> Workload:
    """100k atoms uniform in the 100 A box (0.1 /A^3), charges U[-1,1]; rc 12 A, 4 A bins."""
    rng = np.random.default_rng(seed)
    pos = _uniform_positions(rng, 100_000, (100.0, 100.0, 100.0))
    q = rng.uniform(-1.0, 1.0, size=100_000)
    atoms = np.empty((100_000, 4), dtype=np.float32)
    atoms[:, :3] = pos.astype(np.float32)
    atoms[:, 3] = q.astype(np.float32)
    return Workload("cutoff_200cube_100k_rc12_bin4", "smoothed cutoff, 200^3 @0.5A, 100k atoms, rc=12, bins 4A",
                    atoms, LATTICE_200, cutoff=12.0, bin_size=4.0, seed=seed)


WORKLOADS = {
    1: plane_direct,
    2: full_direct,
    3: protein_direct,
    4: large_direct,
    5: cutoff_binned,
}


def workload(index: int) -> Workload:
    return WORKLOADS[index]()


def checked_nodes(lat: Lattice, n_random: int = 10_000, seed: int = 0) -> np.ndarray:
    """Nodes a large-lattice check visits: three full z-slices (k = 0, nz/2, nz-1)
    plus n_random seeded random nodes, as sorted unique linear x-fastest indices."""
    plane = lat.nx * lat.ny
    ks = sorted({0, lat.nz // 2, lat.nz - 1})
    slices = [np.arange(k * plane, (k + 1) * plane, dtype=np.int64) for k in ks]
    rng = np.random.default_rng(10_000 + seed)
    rand = rng.integers(0, lat.n_points, size=n_random, dtype=np.int64)
    return np.unique(np.concatenate(slices + [rand]))


def random_atoms(n: int, lo, hi, seed: int, q_lo: float = -1.0, q_hi: float = 1.0) -> np.ndarray:
    """n atoms uniform in the box [lo, hi) with charges U[q_lo, q_hi), as (n, 4) float32."""
    rng = np.random.default_rng(seed)
    atoms = np.empty((n, 4), dtype=np.float32)
    atoms[:, :3] = rng.uniform(np.asarray(lo, np.float64), np.asarray(hi, np.float64),
                               size=(n, 3)).astype(np.float32)
    atoms[:, 3] = rng.uniform(q_lo, q_hi, size=n).astype(np.float32)
    return atoms
