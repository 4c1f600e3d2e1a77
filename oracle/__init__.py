"""fp64 CPU oracle for electrostatic potential maps -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this package.  The cpmap library and its Python binding never do: the oracle
and the GPU path share no code.  Each function is the plain definition from the
pages (cited in cpmap_oracle.c), evaluated one node at a time in fp64.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# CPMAP_ORACLE_LIB points the loader at another build of cpmap_oracle.c: the
# mutation test builds copies with planted mistakes and checks that the pins
# fail on each.
_LIB_PATH = os.environ.get("CPMAP_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_direct.restype = None
    lib.oracle_direct.argtypes = [_f32p, _i64, _i32, _i32, _i32, _f32, _f32, _f32, _f32,
                                  ctypes.c_void_p, _i64, _f64p, ctypes.c_void_p]
    lib.oracle_cutoff.restype = None
    lib.oracle_cutoff.argtypes = [_f32p, _i64, _i32, _i32, _i32, _f32, _f32, _f32, _f32, _f32,
                                  ctypes.c_void_p, _i64, _f64p, ctypes.c_void_p]
    lib.oracle_cutoff_hard.restype = None
    lib.oracle_cutoff_hard.argtypes = [_f32p, _i64, _i32, _i32, _i32, _f32, _f32, _f32, _f32,
                                       _f32, ctypes.c_void_p, _i64, _f64p, ctypes.c_void_p]
    lib.oracle_smoothed_term.restype = ctypes.c_double
    lib.oracle_smoothed_term.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.oracle_bin_grid.restype = _i32
    lib.oracle_bin_grid.argtypes = [_i32, _i32, _i32, _f32, _f32, _f32, _f32, _f32, _f32,
                                    _i32p, _f32p]
    lib.oracle_bin_atoms.restype = _i64
    lib.oracle_bin_atoms.argtypes = [_f32p, _i64, _i32, _i32, _i32, _f32, _f32, _f32, _f32,
                                     _f32, _f32, _i32p, _f32p, ctypes.c_void_p]
    lib.oracle_bin_slots.restype = _i64
    lib.oracle_bin_slots.argtypes = [_f32p, _i64, _i32, _i32, _i32, _f32, _f32, _f32, _f32,
                                     _f32, _f32, _i32, _f32p, _i32p, _f32p]
    lib.oracle_extrema.restype = None
    lib.oracle_extrema.argtypes = [_f32p, _i64, np.ctypeslib.ndpointer(dtype=np.int64),
                                   _f32p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _atoms(atoms):
    a = np.ascontiguousarray(atoms, dtype=np.float32)
    if a.ndim != 2 or a.shape[1] != 4:
        raise ValueError("atoms must be (N, 4) float32: x, y, z, q")
    return a


def _nodes(nodes, dims):
    if nodes is None:
        return None, int(dims[0]) * int(dims[1]) * int(dims[2])
    n = np.ascontiguousarray(nodes, dtype=np.int64)
    return n, n.size


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def direct(atoms, dims, spacing, origin=(0.0, 0.0, 0.0), nodes=None, with_scale=False):
    """fp64 direct Coulomb sum V(g) = sum_a q_a / r_ag at the lattice nodes.

    dims = (nx, ny, nz); node (i,j,k) at fp32(origin + (i,j,k)*spacing);
    nodes = linear x-fastest indices to evaluate (None = all, storage order).
    Returns V, or (V, S) with S = sum |q|/r when with_scale is set.
    """
    lib = _load()
    a = _atoms(atoms)
    idx, m = _nodes(nodes, dims)
    V = np.empty(m, dtype=np.float64)
    S = np.empty(m, dtype=np.float64) if with_scale else None
    lib.oracle_direct(a, a.shape[0], int(dims[0]), int(dims[1]), int(dims[2]), float(spacing),
                      float(origin[0]), float(origin[1]), float(origin[2]),
                      None if idx is None else idx.ctypes.data, m, V,
                      None if S is None else S.ctypes.data)
    return (V, S) if with_scale else V


def cutoff(atoms, dims, spacing, origin, rc, nodes=None, with_scale=False):
    """fp64 brute-force smoothed cutoff sum: sum over r < rc of q (1/r - gamma(r^2))."""
    lib = _load()
    a = _atoms(atoms)
    idx, m = _nodes(nodes, dims)
    V = np.empty(m, dtype=np.float64)
    S = np.empty(m, dtype=np.float64) if with_scale else None
    lib.oracle_cutoff(a, a.shape[0], int(dims[0]), int(dims[1]), int(dims[2]), float(spacing),
                      float(origin[0]), float(origin[1]), float(origin[2]), float(rc),
                      None if idx is None else idx.ctypes.data, m, V,
                      None if S is None else S.ctypes.data)
    return (V, S) if with_scale else V


def cutoff_hard(atoms, dims, spacing, origin, rc, nodes=None, with_scale=False):
    """fp64 hard-truncated cutoff sum: q/r over the atoms whose fp32 r^2 < fp32 rc^2."""
    lib = _load()
    a = _atoms(atoms)
    idx, m = _nodes(nodes, dims)
    V = np.empty(m, dtype=np.float64)
    S = np.empty(m, dtype=np.float64) if with_scale else None
    lib.oracle_cutoff_hard(a, a.shape[0], int(dims[0]), int(dims[1]), int(dims[2]),
                           float(spacing), float(origin[0]), float(origin[1]), float(origin[2]),
                           float(rc), None if idx is None else idx.ctypes.data, m, V,
                           None if S is None else S.ctypes.data)
    return (V, S) if with_scale else V


def smoothed_term(q, r, rc) -> float:
    """One atom's smoothed short-range term at distance r (0 for r >= rc)."""
    return _load().oracle_smoothed_term(float(q), float(r), float(rc))


def bin_grid(dims, spacing, origin, bin_size, cutoff_radius):
    """(bins per axis, bin-grid origin, halo) of the binning reading."""
    lib = _load()
    bd = np.zeros(3, dtype=np.int32)
    b0 = np.zeros(3, dtype=np.float32)
    halo = lib.oracle_bin_grid(int(dims[0]), int(dims[1]), int(dims[2]), float(spacing),
                               float(origin[0]), float(origin[1]), float(origin[2]),
                               float(bin_size), float(cutoff_radius), bd, b0)
    if halo < 0:
        raise ValueError("invalid bin geometry")
    return tuple(int(v) for v in bd), b0.copy(), int(halo)


def bin_atoms(atoms, dims, spacing, origin, bin_size, cutoff_radius):
    """Stable counting sort of atoms into bins.

    Returns (bin_start[nbins+1] int32, sorted atoms (n_kept, 4) float32,
    bin_of[n_atoms] int32 with -1 for dropped atoms).
    """
    lib = _load()
    a = _atoms(atoms)
    bd, _, _ = bin_grid(dims, spacing, origin, bin_size, cutoff_radius)
    nbins = bd[0] * bd[1] * bd[2]
    starts = np.zeros(nbins + 1, dtype=np.int32)
    out = np.zeros((max(a.shape[0], 1), 4), dtype=np.float32)
    bin_of = np.zeros(max(a.shape[0], 1), dtype=np.int32)
    kept = lib.oracle_bin_atoms(a, a.shape[0], int(dims[0]), int(dims[1]), int(dims[2]),
                                float(spacing), float(origin[0]), float(origin[1]),
                                float(origin[2]), float(bin_size), float(cutoff_radius),
                                starts, out, bin_of.ctypes.data)
    if kept < 0:
        raise ValueError("invalid bin geometry")
    return starts, out[:kept].copy(), bin_of[:a.shape[0]].copy()


def bin_slots(atoms, dims, spacing, origin, bin_size, cutoff_radius, capacity):
    """Fixed-capacity bins with an overflow list (reading R16).

    Returns (slots (nbins, capacity, 4) float32 with empty slots (inf, inf,
    inf, 0), over_start[nbins+1] int32, overflow atoms (n_over, 4) float32
    grouped by bin).
    """
    lib = _load()
    a = _atoms(atoms)
    bd, _, _ = bin_grid(dims, spacing, origin, bin_size, cutoff_radius)
    nbins = bd[0] * bd[1] * bd[2]
    slots = np.zeros((nbins, int(capacity), 4), dtype=np.float32)
    starts = np.zeros(nbins + 1, dtype=np.int32)
    over = np.zeros((max(a.shape[0], 1), 4), dtype=np.float32)
    n_over = lib.oracle_bin_slots(a, a.shape[0], int(dims[0]), int(dims[1]), int(dims[2]),
                                  float(spacing), float(origin[0]), float(origin[1]),
                                  float(origin[2]), float(bin_size), float(cutoff_radius),
                                  int(capacity), slots.reshape(-1, 4), starts, over)
    if n_over < 0:
        raise ValueError("invalid bin geometry or capacity")
    return slots, starts, over[:n_over].copy()


def extrema(V):
    """Ion-placement extrema of a potential map: ((argmin, argmax), (vmin, vmax)),
    smallest index among ties, NaN nodes skipped, -1 when all are NaN."""
    lib = _load()
    v = np.ascontiguousarray(V, dtype=np.float32).reshape(-1)
    idx = np.zeros(2, dtype=np.int64)
    val = np.zeros(2, dtype=np.float32)
    lib.oracle_extrema(v, v.size, idx, val)
    return (int(idx[0]), int(idx[1])), (float(val[0]), float(val[1]))
