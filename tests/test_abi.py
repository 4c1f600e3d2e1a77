"""The C ABI without a GPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import math
import subprocess

import numpy as np
import pytest

import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import Lattice

OK, EINVAL, ERANGE, ENOSPC, EGEOM = 0, 1, 2, 3, 4
LAT = [8, 8, 8, 0.5, 0.0, 0.0, 0.0]
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails its host checks


def test_header_functions_are_exported():
    names = cpmap.header_functions()
    assert {"cpmap_direct", "cpmap_bin_atoms", "cpmap_cutoff"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", cpmap.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = cpmap.library()
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_status_strings():
    lib = cpmap.library()
    assert lib.cpmap_version() >= (0 << 16) | (1 << 8)
    for s in range(6):
        assert lib.cpmap_status_str(s)
    assert lib.cpmap_status_str(99) == b"unknown status"


@pytest.mark.parametrize("args,want", [
    (dict(n=-1), EINVAL),
    (dict(n=2**31), ERANGE),
    (dict(nx=-1), EINVAL),
    (dict(nx=2**24 + 1), ERANGE),
    (dict(nx=2**24, ny=2**24, nz=2), ERANGE),
    (dict(h=0.0), EINVAL),
    (dict(h=-0.5), EINVAL),
    (dict(h=math.nan), EINVAL),
    (dict(h=math.inf), EINVAL),
    (dict(ox=math.nan), EINVAL),
    (dict(oz=math.inf), EINVAL),
    (dict(V=None), EINVAL),
    (dict(atoms=None), EINVAL),
    (dict(atoms=ctypes.c_void_p(0x1004)), EINVAL),  # not 16-byte aligned
    (dict(V=ctypes.c_void_p(0x1002)), EINVAL),      # not 4-byte aligned
    (dict(nx=0, V=None), OK),                       # empty lattice: no-op, no HIP call
    (dict(ny=0, atoms=None, V=None), OK),
])
def test_direct_argument_checks(args, want):
    a = dict(atoms=FAKE, n=10, nx=8, ny=8, nz=8, h=0.5, ox=0.0, oy=0.0, oz=0.0, V=FAKE)
    a.update(args)
    st = cpmap.library().cpmap_direct(a["atoms"], a["n"], a["nx"], a["ny"], a["nz"], a["h"],
                                      a["ox"], a["oy"], a["oz"], a["V"], None)
    assert st == want


def test_bin_geometry_queries_match_the_header_rule():
    lat = Lattice(200, 200, 200, 0.5)
    assert cpmap.bin_grid(lat, 4.0, 12.0) == (31, 31, 31)
    lat2 = Lattice(10, 3, 5, 0.5, (1.0, -2.0, 0.25))
    assert cpmap.bin_grid(lat2, 1.5, 1.5) == (6, 3, 4)
    n = cpmap.bin_workspace_bytes(100_000, lat, 4.0, 12.0)
    bs_off, srt_off = cpmap.workspace_layout(100_000, lat, 4.0, 12.0)
    assert bs_off % 256 == 0 and srt_off % 256 == 0
    assert srt_off >= bs_off + 4 * (31**3 + 1)
    assert n >= srt_off + 16 * 100_000


@pytest.mark.parametrize("bs,rc,want", [
    (0.0, 12.0, EINVAL), (4.0, 0.0, EINVAL), (math.nan, 12.0, EINVAL), (4.0, math.inf, EINVAL),
    (-1.0, 12.0, EINVAL), (1e-6, 12.0, ERANGE),
])
def test_bin_grid_rejects_bad_bins(bs, rc, want):
    dims = (ctypes.c_int32 * 3)()
    assert cpmap.library().cpmap_bin_grid(*LAT, bs, rc, dims) == want


def test_bin_and_cutoff_argument_checks():
    lib = cpmap.library()
    need = lib.cpmap_bin_workspace_bytes(100, *LAT, 1.0, 2.0)
    assert need > 0
    assert lib.cpmap_bin_workspace_bytes(-1, *LAT, 1.0, 2.0) == 0
    assert lib.cpmap_bin_workspace_bytes(100, *LAT, 0.0, 2.0) == 0
    ws = ctypes.c_void_p(0x10000)
    # too small a workspace, misaligned workspace, null atoms, bad counts
    assert lib.cpmap_bin_atoms(FAKE, 100, *LAT, 1.0, 2.0, ws, need - 1, None) == ENOSPC
    assert lib.cpmap_bin_atoms(FAKE, 100, *LAT, 1.0, 2.0, ctypes.c_void_p(0x10010), need, None) == EINVAL
    assert lib.cpmap_bin_atoms(None, 100, *LAT, 1.0, 2.0, ws, need, None) == EINVAL
    assert lib.cpmap_bin_atoms(FAKE, -5, *LAT, 1.0, 2.0, ws, need, None) == EINVAL
    assert lib.cpmap_bin_atoms(FAKE, 100, 0, 8, 8, 0.5, 0, 0, 0, 1.0, 2.0, ws, need, None) == EINVAL
    # a workspace that was never binned is rejected by cutoff, before any HIP call
    assert lib.cpmap_cutoff(ws, need, 100, *LAT, 1.0, 2.0, FAKE, None) == EGEOM
    assert lib.cpmap_cutoff(ws, need - 1, 100, *LAT, 1.0, 2.0, FAKE, None) == ENOSPC
    assert lib.cpmap_cutoff(ws, need, 100, *LAT, 1.0, 2.0, None, None) == EINVAL
    assert lib.cpmap_cutoff(None, need, 100, *LAT, 1.0, 2.0, FAKE, None) == EINVAL
    assert lib.cpmap_cutoff_term(ws, need, 100, *LAT, 1.0, 2.0, 2, FAKE, None) == EINVAL
    assert lib.cpmap_cutoff_term(ws, need, 100, *LAT, 1.0, 2.0, -1, FAKE, None) == EINVAL
    assert lib.cpmap_cutoff_term(ws, need, 100, *LAT, 1.0, 2.0, 1, FAKE, None) == EGEOM


def test_slot_argument_checks():
    """Fixed-capacity entry points: capacity range, int32 slot count, sizes,
    alignment, aliasing and the binned-for-these-arguments records, all
    refused on the host."""
    lib = cpmap.library()
    need = lib.cpmap_slot_workspace_bytes(100, *LAT, 1.0, 2.0, 8)
    bneed = lib.cpmap_bin_workspace_bytes(100, *LAT, 1.0, 2.0)
    assert need > 0 and bneed > 0
    for cap in (0, -1, 257):
        assert lib.cpmap_slot_workspace_bytes(100, *LAT, 1.0, 2.0, cap) == 0
    assert lib.cpmap_slot_workspace_bytes(100, *LAT, 1.0, 2.0, 256) > need
    assert lib.cpmap_slot_workspace_bytes(-1, *LAT, 1.0, 2.0, 8) == 0
    assert lib.cpmap_slot_workspace_bytes(100, *LAT, 0.0, 2.0, 8) == 0
    # 1002^3 bins: 2 slots per bin fit an int32 slot index, 3 do not
    big = [1000, 1000, 1000, 1.0, 0.0, 0.0, 0.0]
    assert cpmap.bin_grid(Lattice(1000, 1000, 1000, 1.0), 1.0, 1.0) == (1002, 1002, 1002)
    assert lib.cpmap_slot_workspace_bytes(10, *big, 1.0, 1.0, 2) > 0
    assert lib.cpmap_slot_workspace_bytes(10, *big, 1.0, 1.0, 3) == 0
    ws, sws = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x10000 + ((bneed + 255) // 256) * 256)
    assert lib.cpmap_bin_slots(ws, bneed, 100, *big, 1.0, 1.0, 3, sws, need, None) == ERANGE
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 0, sws, need, None) == EINVAL
    assert lib.cpmap_bin_slots(None, bneed, 100, *LAT, 1.0, 2.0, 8, sws, need, None) == EINVAL
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 8, None, need, None) == EINVAL
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 8,
                               ctypes.c_void_p(sws.value + 16), need, None) == EINVAL
    assert lib.cpmap_bin_slots(ws, bneed - 1, 100, *LAT, 1.0, 2.0, 8, sws, need, None) == ENOSPC
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 8, sws, need - 1, None) == ENOSPC
    # the slot workspace may not overlap the binned one
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 8,
                               ctypes.c_void_p(0x10000 + 256), need, None) == EINVAL
    # never binned: refused before any HIP call
    assert lib.cpmap_bin_slots(ws, bneed, 100, *LAT, 1.0, 2.0, 8, sws, need, None) == EGEOM
    assert lib.cpmap_cutoff_slots(sws, need, 100, *LAT, 1.0, 2.0, 8, 0, FAKE, None) == EGEOM
    assert lib.cpmap_cutoff_slots(sws, need, 100, *LAT, 1.0, 2.0, 8, 2, FAKE, None) == EINVAL
    assert lib.cpmap_cutoff_slots(sws, need, 100, *LAT, 1.0, 2.0, 8, 0, None, None) == EINVAL
    assert lib.cpmap_cutoff_slots(sws, need - 1, 100, *LAT, 1.0, 2.0, 8, 0, FAKE, None) == ENOSPC
    assert lib.cpmap_cutoff_slots(sws, need, 100, *LAT, 1.0, 2.0, 0, 0, FAKE, None) == EINVAL
    # layout query
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    assert lib.cpmap_slot_layout(100, *LAT, 1.0, 2.0, 8, ctypes.byref(a), ctypes.byref(b),
                                 None) == EINVAL
    assert a.value == -1 and b.value == -1
    assert lib.cpmap_slot_layout(100, *LAT, 1.0, 2.0, 8, ctypes.byref(a), ctypes.byref(b),
                                 ctypes.byref(c)) == OK
    nb = cpmap.bin_grid(Lattice(8, 8, 8, 0.5), 1.0, 2.0)
    nbins = nb[0] * nb[1] * nb[2]
    assert a.value == 256 and b.value >= a.value + 16 * 8 * nbins and c.value >= b.value + 4 * (nbins + 1)
    assert need >= c.value + 16 * 100 and a.value % 256 == b.value % 256 == c.value % 256 == 0


def test_bin_count_overflow_is_range_error():
    """Per-axis bin counts near 2^24 multiply past int64: the geometry check
    bounds the product step by step and reports ERANGE."""
    lib = cpmap.library()
    dims = (ctypes.c_int32 * 3)()
    # a 2x2x2 lattice 160 A apart in 1e-5 A bins: ~1.6e7 bins per axis
    assert lib.cpmap_bin_grid(2, 2, 2, 160.0, 0.0, 0.0, 0.0, 1e-5, 1e-5, dims) == ERANGE
    assert lib.cpmap_bin_workspace_bytes(10, 2, 2, 2, 160.0, 0.0, 0.0, 0.0, 1e-5, 1e-5) == 0
    assert lib.cpmap_slot_workspace_bytes(10, 2, 2, 2, 160.0, 0.0, 0.0, 0.0, 1e-5, 1e-5, 8) == 0


def test_layout_query_errors():
    lib = cpmap.library()
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.cpmap_workspace_layout(-1, *LAT, 1.0, 2.0, ctypes.byref(a), ctypes.byref(b)) == EINVAL
    assert a.value == -1 and b.value == -1
    assert lib.cpmap_workspace_layout(5, *LAT, 1.0, 2.0, None, ctypes.byref(b)) == EINVAL


def test_binding_rejects_cpu_and_wrong_dtype_tensors():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        cpmap.direct(torch.zeros(4, 4), Lattice(2, 2, 2, 0.5))
    with pytest.raises(ValueError):
        cpmap.direct(torch.zeros(4, 3, dtype=torch.float32), Lattice(2, 2, 2, 0.5))
    with pytest.raises(TypeError):
        cpmap.direct([[0, 0, 0, 1]], Lattice(2, 2, 2, 0.5))


def test_binding_rejects_host_buffers_before_any_launch():
    """Workspaces and outputs are checked (dtype, GPU, contiguity) before the
    library is asked to launch anything."""
    torch = pytest.importorskip("torch")
    lat = Lattice(8, 8, 8, 0.5)
    host_ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        cpmap.cutoff(host_ws, 4, lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.cutoff(host_ws.view(torch.int8), 4, lat, 1.0, 2.0)
    with pytest.raises(ValueError):
        cpmap.cutoff_slots(host_ws, 4, lat, 1.0, 2.0, 2)
    with pytest.raises(ValueError):
        cpmap.bin_slots(host_ws, 4, lat, 1.0, 2.0, 2)
    with pytest.raises(ValueError):
        cpmap.extrema(torch.zeros(16))
    with pytest.raises(ValueError):
        cpmap.cutoff(host_ws, 4, lat, 1.0, 2.0, term="hard")


def test_planner_picks_each_variant_for_its_test_geometry():
    """The GPU test that runs every compiled direct variant relies on these
    choices; a planner change that moves a geometry to another variant shows
    here first."""
    from test_gpu_direct import VARIANT_CASES
    for variant, n, dims, split in VARIANT_CASES:
        lat = Lattice(*dims, 0.5, (-1.25, 0.5, 2.0))
        assert cpmap.direct_plan(n, lat, split)[:4] == variant, (variant, n, dims)
    assert len({c[0] for c in VARIANT_CASES}) == 9


def test_direct_workspace_queries_and_checks():
    lib = cpmap.library()
    need = lib.cpmap_direct_workspace_bytes(200_000, 200, 200, 200)
    # the 200^3 lattice at 8x8x2 nodes per lane: 977 node groups; the ordered
    # split keeps a 64-word head and one count per group (4,352 bytes)
    assert need == 4352
    assert lib.cpmap_direct_workspace_bytes(-1, 200, 200, 200) == 0
    assert lib.cpmap_direct_workspace_bytes(10, -1, 2, 2) == 0
    assert cpmap.direct_plan(200_000, Lattice(200, 200, 200, 0.5), True) == (8, 8, 2, 4, 11)
    assert cpmap.direct_plan(200_000, Lattice(200, 200, 200, 0.5), False)[4] == 1
    assert cpmap.direct_plan(1, Lattice(1, 1, 1, 0.5), True)[4] == 1
    assert lib.cpmap_direct_workspace_bytes(1, 1, 1, 1) == 0
    ws = ctypes.c_void_p(0x100000)
    args = (FAKE, 200_000, 200, 200, 200, 0.5, 0.0, 0.0, 0.0, FAKE)
    assert lib.cpmap_direct_with_workspace(*args, ws, need - 1, None) == ENOSPC
    assert lib.cpmap_direct_with_workspace(*args, None, need, None) == EINVAL
    assert lib.cpmap_direct_with_workspace(*args, ctypes.c_void_p(0x100010), need, None) == EINVAL
    assert lib.cpmap_direct_with_workspace(FAKE, -1, 200, 200, 200, 0.5, 0.0, 0.0, 0.0, FAKE, ws, need, None) == EINVAL
    assert lib.cpmap_direct_with_workspace(FAKE, 10, 0, 200, 200, 0.5, 0.0, 0.0, 0.0, None, None, 0, None) == OK
    out = (ctypes.c_int32 * 5)()
    assert lib.cpmap_direct_plan(10, 2, 2, 2, 1, None) == EINVAL
    assert lib.cpmap_direct_plan(-1, 2, 2, 2, 1, out) == EINVAL


def test_extrema_argument_checks():
    lib = cpmap.library()
    need = lib.cpmap_extrema_workspace_bytes(8_000_000)
    assert 0 < need <= 64 * 1024
    assert lib.cpmap_extrema_workspace_bytes(-1) == 0
    ws = ctypes.c_void_p(0x100000)
    out_i, out_v = ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000)
    assert lib.cpmap_extrema(FAKE, 8_000_000, out_i, out_v, ws, need - 1, None) == ENOSPC
    assert lib.cpmap_extrema(FAKE, -1, out_i, out_v, ws, need, None) == EINVAL
    assert lib.cpmap_extrema(None, 10, out_i, out_v, ws, need, None) == EINVAL
    assert lib.cpmap_extrema(FAKE, 10, None, out_v, ws, need, None) == EINVAL
    assert lib.cpmap_extrema(FAKE, 10, ctypes.c_void_p(0x2004), out_v, ws, need, None) == EINVAL
    assert lib.cpmap_extrema(FAKE, 10, out_i, out_v, None, need, None) == EINVAL


def test_binding_fails_loudly_without_the_library(monkeypatch):
    """No CPU fallback: with libcpmap.so missing every call raises."""
    import numpy as np
    torch = pytest.importorskip("torch")
    monkeypatch.setattr(cpmap, "_lib", None)
    monkeypatch.setattr(cpmap, "_LIB_PATH", "/nonexistent/libcpmap.so")
    with pytest.raises(ImportError):
        cpmap.library()
    with pytest.raises(ImportError):
        cpmap.direct_workspace_bytes(10, Lattice(2, 2, 2, 0.5))
    with pytest.raises((ImportError, ValueError)):
        cpmap.direct(torch.from_numpy(np.zeros((1, 4), np.float32)), Lattice(2, 2, 2, 0.5))


def test_node_position_decodes_index_and_rounds_once():
    """cpmap_node_position: index (k*ny + j)*nx + i -> (i, j, k) and the node at
    (fl(ox + i h), fl(oy + j h), fl(oz + k h)), one fp32 rounding of the exact
    value (the header's lattice convention); out-of-range indices and invalid
    lattices are refused."""
    lat = Lattice(7, 5, 3, 0.1, (-1.25, 0.3, 1e4))
    h = float(np.float32(0.1))
    o = [float(np.float32(v)) for v in lat.origin]
    for g in [0, 1, 6, 7, 34, 35, 104]:
        ijk, xyz = cpmap.node_position(lat, g)
        i, j, k = g % 7, (g // 7) % 5, g // 35
        assert ijk == (i, j, k)
        want = tuple(float(np.float32(oo + c * h)) for oo, c in zip(o, (i, j, k)))
        assert xyz == want, (g, xyz, want)
    # 3 * 0.1f rounds once to 0.3f (0.30000001192...), not to fl(fl(3*0.1f) + 0)
    ijk, xyz = cpmap.node_position(Lattice(4, 1, 1, 0.1), 3)
    assert xyz[0] == float(np.float32(0.3))
    lib = cpmap.library()
    ijk_buf, xyz_buf = (ctypes.c_int32 * 3)(), (ctypes.c_float * 3)()
    L = [7, 5, 3, 0.1, 0.0, 0.0, 0.0]
    assert lib.cpmap_node_position(*L, 105, ijk_buf, xyz_buf) == ERANGE
    assert lib.cpmap_node_position(*L, -1, ijk_buf, xyz_buf) == ERANGE
    assert lib.cpmap_node_position(*L, 0, None, xyz_buf) == EINVAL
    assert lib.cpmap_node_position(*L, 0, ijk_buf, None) == EINVAL
    assert lib.cpmap_node_position(7, 5, 3, -0.1, 0.0, 0.0, 0.0, 0, ijk_buf, xyz_buf) == EINVAL
    assert lib.cpmap_node_position(0, 5, 3, 0.1, 0.0, 0.0, 0.0, 0, ijk_buf, xyz_buf) == ERANGE
    # the largest index of a lattice past 2^31 nodes
    big = Lattice(2048, 1024, 1040, 0.5)
    ijk, xyz = cpmap.node_position(big, big.n_points - 1)
    assert ijk == (2047, 1023, 1039) and xyz == (1023.5, 511.5, 519.5)
