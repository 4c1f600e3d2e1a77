"""cpmap: electrostatic potential maps on AMD Instinct MI355X (gfx950).

A thin binding over libcpmap.so (C ABI in include/cpmap.h).  It only checks
and marshals arguments: every step of the computation runs in the library's
HIP kernels.  PyTorch provides device memory and the current stream.  There
is no CPU fallback: if libcpmap.so is missing or fails to load, every call
raises.

    import direct_coulomb_potential_amd as cpmap
    lat = cpmap.Lattice(200, 200, 200, 0.5)
    V = cpmap.direct(atoms_cuda_f32_Nx4, lat)                 # direct sum
    ws = cpmap.bin_atoms(atoms, lat, bin_size=4.0, cutoff=12.0)
    Vc = cpmap.cutoff(ws, len(atoms), lat, bin_size=4.0, cutoff=12.0)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

from .workloads import Lattice

__all__ = [
    "Lattice", "CpmapError", "direct", "direct_scatter", "direct_workspace_bytes", "direct_plan", "bin_atoms", "cutoff", "bin_workspace_bytes",
    "bin_grid", "workspace_layout", "workspace_views", "neighbor_spans", "library",
    "library_path", "header_functions", "STATUS", "extrema", "place_ions", "TERMS",
    "slot_workspace_bytes", "slot_layout", "bin_slots", "slot_views", "cutoff_slots",
    "node_position", "extrema_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libcpmap.so")
_HEADER = os.path.join(os.path.dirname(_HERE), "include", "cpmap.h")

STATUS = {0: "CPMAP_OK", 1: "CPMAP_EINVAL", 2: "CPMAP_ERANGE", 3: "CPMAP_ENOSPC",
          4: "CPMAP_EGEOM", 5: "CPMAP_EHIP"}


class CpmapError(RuntimeError):
    """A cpmap_status other than CPMAP_OK; `status` holds its code."""

    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None

_i64, _i32, _f32, _vp, _sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_void_p,
                              ctypes.c_size_t)
_LAT = [_i32, _i32, _i32, _f32, _f32, _f32, _f32]

_SIGNATURES = {
    "cpmap_version": (_i32, []),
    "cpmap_status_str": (ctypes.c_char_p, [_i32]),
    "cpmap_direct": (_i32, [_vp, _i64, *_LAT, _vp, _vp]),
    "cpmap_direct_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "cpmap_direct_with_workspace": (_i32, [_vp, _i64, *_LAT, _vp, _vp, _sz, _vp]),
    "cpmap_direct_plan": (_i32, [_i64, _i32, _i32, _i32, _i32, ctypes.POINTER(_i32)]),
    "cpmap_direct_occupancy_check": (_i32, []),
    "cpmap_direct_scatter": (_i32, [_vp, _i64, *_LAT, _vp, _vp]),
    "cpmap_bin_workspace_bytes": (_sz, [_i64, *_LAT, _f32, _f32]),
    "cpmap_bin_grid": (_i32, [*_LAT, _f32, _f32, ctypes.POINTER(_i32)]),
    "cpmap_bin_atoms": (_i32, [_vp, _i64, *_LAT, _f32, _f32, _vp, _sz, _vp]),
    "cpmap_workspace_layout": (_i32, [_i64, *_LAT, _f32, _f32, ctypes.POINTER(_i64),
                                      ctypes.POINTER(_i64)]),
    "cpmap_cutoff": (_i32, [_vp, _sz, _i64, *_LAT, _f32, _f32, _vp, _vp]),
    "cpmap_cutoff_term": (_i32, [_vp, _sz, _i64, *_LAT, _f32, _f32, _i32, _vp, _vp]),
    "cpmap_extrema_workspace_bytes": (_sz, [_i64]),
    "cpmap_extrema": (_i32, [_vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "cpmap_neighbor_spans": (_i64, [*_LAT, _f32, _f32, _i32, _i32, _i32, _i32,
                                    ctypes.POINTER(_i32), _i64]),
    "cpmap_slot_workspace_bytes": (_sz, [_i64, *_LAT, _f32, _f32, _i32]),
    "cpmap_slot_layout": (_i32, [_i64, *_LAT, _f32, _f32, _i32, ctypes.POINTER(_i64),
                                 ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "cpmap_bin_slots": (_i32, [_vp, _sz, _i64, *_LAT, _f32, _f32, _i32, _vp, _sz, _vp]),
    "cpmap_cutoff_slots": (_i32, [_vp, _sz, _i64, *_LAT, _f32, _f32, _i32, _i32, _vp, _vp]),
    "cpmap_node_position": (_i32, [*_LAT, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_f32)]),
    "cpmap_extrema_noalloc": (_i32, [_vp, _i64, _vp, _vp, _vp]),
}


def library_path() -> str:
    """Path of the libcpmap.so this binding loads (next to this file)."""
    return _LIB_PATH


def library():
    """The loaded libcpmap.so (ctypes), with argument types set.  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libcpmap.so not found at {_LIB_PATH}; build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` "
            "or `python direct_coulomb_potential_amd/build.py`")
    lib = ctypes.CDLL(_LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/cpmap.h declares."""
    with open(_HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpmap_[a-z_]+)\s*\(", text)))


def _check(fn: str, status: int):
    if status != 0:
        msg = library().cpmap_status_str(status).decode()
        raise CpmapError(fn, status, msg)


def _lat_args(lat: Lattice):
    return [int(lat.nx), int(lat.ny), int(lat.nz), float(lat.spacing), float(lat.origin[0]),
            float(lat.origin[1]), float(lat.origin[2])]


def _torch():
    import torch
    return torch


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def _call(fn_name: str, device, *args):
    """Call a launching entry point with `device` current and its current
    stream as the last argument; raise on a non-zero status."""
    torch = _torch()
    with torch.cuda.device(device):
        st = getattr(library(), fn_name)(*args, _stream_ptr(device))
    _check(fn_name, st)


def _buffer(t, dtype, device, name: str, min_numel: int = 0):
    """Check that t is a contiguous GPU tensor of dtype on device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_cuda \
            or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.numel() < min_numel:
        raise ValueError(f"{name} must have at least {min_numel} elements")
    return t


def _check_atoms(atoms):
    torch = _torch()
    if not isinstance(atoms, torch.Tensor):
        raise TypeError("atoms must be a torch.Tensor")
    if atoms.dtype != torch.float32 or atoms.dim() != 2 or atoms.shape[1] != 4:
        raise ValueError("atoms must be float32 with shape (N, 4): x, y, z, q")
    if not atoms.is_cuda:
        raise ValueError("atoms must be on a GPU device")
    if not atoms.is_contiguous():
        raise ValueError("atoms must be contiguous")


def _out(lat: Lattice, device, out):
    torch = _torch()
    shape = (lat.nz, lat.ny, lat.nx)
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if out.dtype != torch.float32 or not out.is_cuda or not out.is_contiguous() \
            or out.numel() != lat.n_points:
        raise ValueError("out must be a contiguous float32 GPU tensor with nx*ny*nz elements")
    if out.device != torch.device(device):
        raise ValueError(f"out is on {out.device}, expected {device}")
    return out


def direct_workspace_bytes(n_atoms: int, lat: Lattice) -> int:
    """Bytes of the optional workspace of the split direct sum (0: not used)."""
    return int(library().cpmap_direct_workspace_bytes(int(n_atoms), int(lat.nx), int(lat.ny),
                                                      int(lat.nz)))


def direct_plan(n_atoms: int, lat: Lattice, with_workspace: bool = True):
    """(cx, cy, cz, waves per workgroup, atom parts) of a direct launch."""
    out = (_i32 * 5)()
    _check("cpmap_direct_plan", library().cpmap_direct_plan(
        int(n_atoms), int(lat.nx), int(lat.ny), int(lat.nz), int(bool(with_workspace)), out))
    return tuple(out)


def direct(atoms, lat: Lattice, out=None, split: bool = True, workspace=None):
    """Direct Coulomb sum at every node; returns V with shape (nz, ny, nx) (x fastest).

    split=True uses cpmap_direct_with_workspace with a workspace of
    direct_workspace_bytes() (allocated here unless given as a uint8 GPU
    tensor); split=False calls cpmap_direct.
    """
    torch = _torch()
    _check_atoms(atoms)
    V = _out(lat, atoms.device, out)
    a_ptr = atoms.data_ptr() if atoms.numel() else None
    v_ptr = V.data_ptr() if V.numel() else None
    if not split:
        _call("cpmap_direct", atoms.device, a_ptr, atoms.shape[0], *_lat_args(lat), v_ptr)
        return V
    need = direct_workspace_bytes(atoms.shape[0], lat)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=atoms.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _buffer(workspace, torch.uint8, atoms.device, "workspace")
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _call("cpmap_direct_with_workspace", atoms.device, a_ptr, atoms.shape[0], *_lat_args(lat),
          v_ptr, ws_ptr, ws_bytes)
    return V


def direct_scatter(atoms, lat: Lattice, out=None):
    """The scatter form of the direct sum (atomics; a contrast, not bit-reproducible)."""
    _check_atoms(atoms)
    V = _out(lat, atoms.device, out)
    _call("cpmap_direct_scatter", atoms.device, atoms.data_ptr() if atoms.numel() else None,
          atoms.shape[0], *_lat_args(lat), V.data_ptr() if V.numel() else None)
    return V


def bin_workspace_bytes(n_atoms: int, lat: Lattice, bin_size: float, cutoff: float) -> int:
    """Bytes of the workspace bin_atoms fills for this atom count and geometry
    (cpmap_bin_workspace_bytes); raises CpmapError for an invalid geometry."""
    n = library().cpmap_bin_workspace_bytes(int(n_atoms), *_lat_args(lat), float(bin_size),
                                            float(cutoff))
    if n == 0:
        raise CpmapError("cpmap_bin_workspace_bytes", 1, "invalid geometry")
    return int(n)


def bin_grid(lat: Lattice, bin_size: float, cutoff: float) -> Tuple[int, int, int]:
    """Bins per axis (x, y, z) of the bin grid for this geometry (cpmap_bin_grid)."""
    dims = (_i32 * 3)()
    _check("cpmap_bin_grid", library().cpmap_bin_grid(*_lat_args(lat), float(bin_size),
                                                       float(cutoff), dims))
    return (dims[0], dims[1], dims[2])


def workspace_layout(n_atoms: int, lat: Lattice, bin_size: float, cutoff: float):
    """Byte offsets (bin_start, sorted atoms) inside a binned workspace."""
    a, b = _i64(), _i64()
    _check("cpmap_workspace_layout",
           library().cpmap_workspace_layout(int(n_atoms), *_lat_args(lat), float(bin_size),
                                            float(cutoff), ctypes.byref(a), ctypes.byref(b)))
    return int(a.value), int(b.value)


def bin_atoms(atoms, lat: Lattice, bin_size: float, cutoff: float, workspace=None):
    """Bin atoms on the GPU into a workspace (uint8 tensor) and return it."""
    torch = _torch()
    _check_atoms(atoms)
    need = bin_workspace_bytes(atoms.shape[0], lat, bin_size, cutoff)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=atoms.device)
    _buffer(workspace, torch.uint8, atoms.device, "workspace")
    _call("cpmap_bin_atoms", atoms.device, atoms.data_ptr() if atoms.numel() else None,
          atoms.shape[0], *_lat_args(lat), float(bin_size), float(cutoff),
          workspace.data_ptr(), workspace.numel())
    return workspace


def workspace_views(workspace, n_atoms: int, lat: Lattice, bin_size: float, cutoff: float):
    """(bin_start int32[nbins+1], sorted float32[n_atoms, 4]) views into a workspace."""
    bs_off, srt_off = workspace_layout(n_atoms, lat, bin_size, cutoff)
    bx, by, bz = bin_grid(lat, bin_size, cutoff)
    nb = bx * by * bz
    torch = _torch()
    starts = workspace[bs_off:bs_off + 4 * (nb + 1)].view(torch.int32)
    srt = workspace[srt_off:srt_off + 16 * n_atoms].view(torch.float32).view(n_atoms, 4)
    return starts, srt


TERMS = {"smoothed": 0, "truncated": 1}


def cutoff(workspace, n_atoms: int, lat: Lattice, bin_size: float, cutoff: float, out=None,
           term: str = "smoothed"):
    """Cutoff sum over binned atoms; returns V (nz, ny, nx).

    term="smoothed": q (1/r - gamma(r^2)) (cpmap_cutoff); term="truncated": q/r
    with the fp32 inclusion test of cpmap_cutoff_term.
    """
    if term not in TERMS:
        raise ValueError(f"term must be one of {sorted(TERMS)}")
    torch = _torch()
    _buffer(workspace, torch.uint8, workspace.device, "workspace")
    V = _out(lat, workspace.device, out)
    _call("cpmap_cutoff_term", workspace.device, workspace.data_ptr(), workspace.numel(),
          int(n_atoms), *_lat_args(lat), float(bin_size), float(cutoff), TERMS[term],
          V.data_ptr())
    return V


def slot_workspace_bytes(n_atoms: int, lat: Lattice, bin_size: float, cutoff: float,
                         capacity: int = 8) -> int:
    """Bytes of the slot workspace bin_slots fills (cpmap_slot_workspace_bytes);
    raises CpmapError for an invalid geometry or capacity."""
    n = library().cpmap_slot_workspace_bytes(int(n_atoms), *_lat_args(lat), float(bin_size),
                                             float(cutoff), int(capacity))
    if n == 0:
        raise CpmapError("cpmap_slot_workspace_bytes", 1, "invalid geometry or capacity")
    return int(n)


def slot_layout(n_atoms: int, lat: Lattice, bin_size: float, cutoff: float, capacity: int = 8):
    """Byte offsets (slots, over_start, over_atoms) inside a slot workspace."""
    a, b, c = _i64(), _i64(), _i64()
    _check("cpmap_slot_layout",
           library().cpmap_slot_layout(int(n_atoms), *_lat_args(lat), float(bin_size),
                                       float(cutoff), int(capacity), ctypes.byref(a),
                                       ctypes.byref(b), ctypes.byref(c)))
    return int(a.value), int(b.value), int(c.value)


def bin_slots(workspace, n_atoms: int, lat: Lattice, bin_size: float, cutoff: float,
              capacity: int = 8, slot_workspace=None):
    """Fixed-capacity bins (capacity slots per bin plus an overflow list) from a
    workspace that bin_atoms filled; returns the slot workspace (uint8 tensor)."""
    torch = _torch()
    _buffer(workspace, torch.uint8, workspace.device, "workspace")
    need = slot_workspace_bytes(n_atoms, lat, bin_size, cutoff, capacity)
    if slot_workspace is None:
        slot_workspace = torch.empty(need, dtype=torch.uint8, device=workspace.device)
    _buffer(slot_workspace, torch.uint8, workspace.device, "slot_workspace")
    _call("cpmap_bin_slots", workspace.device, workspace.data_ptr(), workspace.numel(),
          int(n_atoms), *_lat_args(lat), float(bin_size), float(cutoff), int(capacity),
          slot_workspace.data_ptr(), slot_workspace.numel())
    return slot_workspace


def slot_views(slot_workspace, n_atoms: int, lat: Lattice, bin_size: float, cutoff: float,
               capacity: int = 8):
    """(slots float32[nbins, capacity, 4], over_start int32[nbins+1],
    over_atoms float32[n_atoms, 4]) views into a slot workspace."""
    torch = _torch()
    s_off, o_off, a_off = slot_layout(n_atoms, lat, bin_size, cutoff, capacity)
    bx, by, bz = bin_grid(lat, bin_size, cutoff)
    nb = bx * by * bz
    slots = slot_workspace[s_off:s_off + 16 * nb * capacity].view(torch.float32)
    starts = slot_workspace[o_off:o_off + 4 * (nb + 1)].view(torch.int32)
    over = slot_workspace[a_off:a_off + 16 * n_atoms].view(torch.float32)
    return slots.view(nb, capacity, 4), starts, over.view(n_atoms, 4)


def cutoff_slots(slot_workspace, n_atoms: int, lat: Lattice, bin_size: float, cutoff: float,
                 capacity: int = 8, out=None, term: str = "smoothed"):
    """The cutoff sum over fixed-capacity bins (slot pass, then overflow pass)."""
    if term not in TERMS:
        raise ValueError(f"term must be one of {sorted(TERMS)}")
    torch = _torch()
    _buffer(slot_workspace, torch.uint8, slot_workspace.device, "slot_workspace")
    V = _out(lat, slot_workspace.device, out)
    _call("cpmap_cutoff_slots", slot_workspace.device, slot_workspace.data_ptr(),
          slot_workspace.numel(), int(n_atoms), *_lat_args(lat), float(bin_size),
          float(cutoff), int(capacity), TERMS[term], V.data_ptr())
    return V


def neighbor_spans(lat: Lattice, bin_size: float, cutoff: float, tile: Tuple[int, int, int],
                   max_spans: int = 4096, term: str = "smoothed"):
    """x-runs of bins (cy, cz, cx_first, cx_last) the cutoff kernel walks for
    one tile with this term."""
    if term not in TERMS:
        raise ValueError(f"term must be one of {sorted(TERMS)}")
    buf = (_i32 * (4 * max_spans))()
    n = library().cpmap_neighbor_spans(*_lat_args(lat), float(bin_size), float(cutoff),
                                       TERMS[term], int(tile[0]), int(tile[1]), int(tile[2]),
                                       buf, max_spans)
    if n < 0:
        raise CpmapError("cpmap_neighbor_spans", 1, "invalid arguments")
    if n > max_spans:
        return neighbor_spans(lat, bin_size, cutoff, tile, int(n), term)
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def extrema(V, workspace=None, out=None):
    """Argmin / argmax of a GPU float32 map (cpmap_extrema).

    Returns an int64 tensor [argmin, argmax] and a float32 tensor [vmin, vmax],
    both on V's device (no synchronisation).
    """
    torch = _torch()
    if V.dtype != torch.float32 or not V.is_cuda or not V.is_contiguous():
        raise ValueError("V must be a contiguous float32 GPU tensor")
    n = V.numel()
    need = int(library().cpmap_extrema_workspace_bytes(n))
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=V.device)
    _buffer(workspace, torch.uint8, V.device, "workspace")
    if out is None:
        idx = torch.empty(2, dtype=torch.int64, device=V.device)
        val = torch.empty(2, dtype=torch.float32, device=V.device)
    else:
        idx = _buffer(out[0], torch.int64, V.device, "out[0]", 2)
        val = _buffer(out[1], torch.float32, V.device, "out[1]", 2)
    _call("cpmap_extrema", V.device, V.data_ptr() if n else None, n, idx.data_ptr(),
          val.data_ptr(), workspace.data_ptr(), workspace.numel())
    return idx, val


def extrema_noalloc(V, out=None):
    """cpmap_extrema_noalloc: as extrema(), with the library's static
    per-device scratch instead of a workspace (nothing is allocated when
    `out` is given); calls that overlap on one GPU race."""
    torch = _torch()
    if V.dtype != torch.float32 or not V.is_cuda or not V.is_contiguous():
        raise ValueError("V must be a contiguous float32 GPU tensor")
    n = V.numel()
    if out is None:
        idx = torch.empty(2, dtype=torch.int64, device=V.device)
        val = torch.empty(2, dtype=torch.float32, device=V.device)
    else:
        idx = _buffer(out[0], torch.int64, V.device, "out[0]", 2)
        val = _buffer(out[1], torch.float32, V.device, "out[1]", 2)
    _call("cpmap_extrema_noalloc", V.device, V.data_ptr() if n else None, n, idx.data_ptr(),
          val.data_ptr())
    return idx, val


def node_position(lat: Lattice, index: int):
    """((i, j, k), (x, y, z)) of the node a linear x-fastest index names
    (cpmap_node_position: the position in the kernels' fp32 values)."""
    ijk = (_i32 * 3)()
    xyz = (_f32 * 3)()
    _check("cpmap_node_position", library().cpmap_node_position(*_lat_args(lat), int(index),
                                                                ijk, xyz))
    return tuple(ijk), tuple(xyz)


def place_ions(V, lat: Lattice):
    """Nodes for a positive ion (lowest potential) and a negative ion (highest),
    as ((i, j, k), (x, y, z), value) pairs, or None for a map with no non-NaN
    node; synchronises to read the extrema back."""
    idx, val = extrema(V)
    out = []
    for g, v in zip(idx.cpu().tolist(), val.cpu().tolist()):
        out.append(None if g < 0 else (*node_position(lat, g), v))
    return {"positive_ion": out[0], "negative_ion": out[1]}
