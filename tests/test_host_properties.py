"""Property tests of the library's host-only queries (CPU only, no HIP call):
over random geometries, including extreme and invalid ones, every query
answers with a status instead of failing, and the sizes, layouts, plans and
neighbourhoods it returns are consistent with each other and with the
oracle's independent bin grid."""
import ctypes
import math

import numpy as np
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import direct_coulomb_potential_amd as cpmap
import oracle

OK, EINVAL, ERANGE = 0, 1, 2
# compiled direct-kernel variants (nodes per lane x, y, z; waves per
# workgroup) and their resident waves per SIMD, as the planner's table has them
OCCUPANCY = {(8, 8, 2, 4): 2, (8, 8, 2, 8): 2, (8, 4, 2, 4): 4, (8, 4, 2, 8): 4, (4, 4, 2, 8): 6,
             (4, 4, 2, 16): 4, (4, 4, 1, 16): 8, (2, 2, 1, 16): 8, (1, 1, 1, 16): 8}
VARIANTS = set(OCCUPANCY)

dims = st.integers(1, 400)
spacing = st.floats(0.05, 4.0)
origin = st.floats(-5000.0, 5000.0)
bin_size = st.floats(0.2, 16.0)
cutoff = st.floats(0.2, 30.0)
n_atoms = st.integers(0, 2_000_000)
# derandomized: every run draws the same examples; no example database
SETTINGS = settings(max_examples=300, deadline=None, derandomize=True, database=None,
                    suppress_health_check=[HealthCheck.too_slow])


def _lat(nx, ny, nz, h, ox, oy, oz):
    return [int(nx), int(ny), int(nz), float(h), float(ox), float(oy), float(oz)]


@SETTINGS
@given(nx=dims, ny=dims, nz=dims, h=spacing, ox=origin, oy=origin, oz=origin, bs=bin_size,
       rc=cutoff, n=n_atoms, cap=st.integers(1, 256))
def test_bin_and_slot_layouts_are_consistent(nx, ny, nz, h, ox, oy, oz, bs, rc, n, cap):
    lib = cpmap.library()
    L = _lat(nx, ny, nz, h, ox, oy, oz)
    bd = (ctypes.c_int32 * 3)()
    st_grid = lib.cpmap_bin_grid(*L, bs, rc, bd)
    assert st_grid in (OK, ERANGE)
    nbytes = lib.cpmap_bin_workspace_bytes(n, *L, bs, rc)
    if st_grid != OK:
        assert nbytes == 0
        return
    nbins = bd[0] * bd[1] * bd[2]
    # the oracle derives the same grid on its own
    o_dims, _, halo = oracle.bin_grid((nx, ny, nz), h, (ox, oy, oz), bs, rc)
    assert tuple(bd) == o_dims
    assert halo == math.ceil(np.float32(np.float32(rc) / np.float32(bs)))
    # the halo on both sides (the last node's bin coordinate can round to
    # just below H when the lattice is a single node thick)
    assert all(d >= 2 * halo for d in o_dims)
    assert nbins < 2**31
    assert nbytes >= 256 + 4 * (nbins + 1) + 16 * n
    a, b = ctypes.c_int64(), ctypes.c_int64()
    assert lib.cpmap_workspace_layout(n, *L, bs, rc, ctypes.byref(a), ctypes.byref(b)) == OK
    assert a.value == 256 and b.value >= a.value + 4 * (nbins + 1) and b.value % 256 == 0
    assert b.value + 16 * n <= nbytes
    # fixed-capacity slots
    sbytes = lib.cpmap_slot_workspace_bytes(n, *L, bs, rc, cap)
    s, o, v = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    st_slot = lib.cpmap_slot_layout(n, *L, bs, rc, cap, ctypes.byref(s), ctypes.byref(o),
                                    ctypes.byref(v))
    if nbins * cap >= 2**31:
        assert st_slot == ERANGE and sbytes == 0
        return
    assert st_slot == OK and sbytes > 0
    assert s.value == 256
    assert o.value >= s.value + 16 * nbins * cap and o.value % 256 == 0
    assert v.value >= o.value + 4 * (nbins + 1) and v.value % 256 == 0
    assert v.value + 16 * n <= sbytes


@SETTINGS
@given(nx=dims, ny=dims, nz=dims, h=spacing, ox=origin, oy=origin, oz=origin, bs=bin_size,
       rc=cutoff, data=st.data())
def test_neighbourhood_spans_stay_inside_the_bin_grid(nx, ny, nz, h, ox, oy, oz, bs, rc, data):
    lib = cpmap.library()
    term = data.draw(st.sampled_from([0, 1]))
    L = _lat(nx, ny, nz, h, ox, oy, oz)
    bd = (ctypes.c_int32 * 3)()
    assume(lib.cpmap_bin_grid(*L, bs, rc, bd) == OK)
    tiles = [(d + 7) // 8 for d in (nx, ny, nz)]
    t = [data.draw(st.integers(0, k - 1)) for k in tiles]
    cap = 4096
    buf = (ctypes.c_int32 * (4 * cap))()
    count = lib.cpmap_neighbor_spans(*L, bs, rc, term, t[0], t[1], t[2], buf, cap)
    assert count >= 1  # the bins under the tile itself are always within rc
    rows = set()
    for i in range(min(count, cap)):
        cy, cz, c0, c1 = buf[4 * i: 4 * i + 4]
        assert 0 <= cy < bd[1] and 0 <= cz < bd[2]
        assert 0 <= c0 <= c1 < bd[0]
        assert (cy, cz) not in rows
        rows.add((cy, cz))
    # a tile outside the lattice is refused
    assert lib.cpmap_neighbor_spans(*L, bs, rc, term, tiles[0], 0, 0, buf, cap) == -1


@SETTINGS
@given(nx=dims, ny=dims, nz=dims, n=st.integers(1, 5_000_000), ws=st.booleans())
def test_direct_plans_are_compiled_variants_with_bounded_workspace(nx, ny, nz, n, ws):
    lib = cpmap.library()
    out = (ctypes.c_int32 * 5)()
    assert lib.cpmap_direct_plan(n, nx, ny, nz, int(ws), out) == OK
    plan = tuple(out)
    assert plan[:4] in VARIANTS
    assert 1 <= plan[4] <= 32
    if not ws:
        assert plan[4] == 1
    need = lib.cpmap_direct_workspace_bytes(n, nx, ny, nz)
    with_ws = (ctypes.c_int32 * 5)()
    lib.cpmap_direct_plan(n, nx, ny, nz, 1, with_ws)
    if with_ws[4] > 1:
        cx, cy, cz, w, k = with_ws
        strips = -(-nx // cx) * -(-ny // cy) * -(-nz // cz)
        groups = -(-strips // 64)
        resident = 256 * max(1, OCCUPANCY[(cx, cy, cz, w)] * 4 // w)
        if groups >= resident:
            # ordered: the counter and one count per node group
            want = 4 * (64 + groups)
        else:
            # partial: maps of parts 1 .. K-1, at most 64 MiB
            want = 4 * (k - 1) * nx * ny * nz
            assert want <= 64 << 20
        assert need == -(-want // 256) * 256
        assert groups * k < 2**31
        assert n >= k * w * 64  # at least 64 atoms per wave
    else:
        assert need == 0


bad_float = st.sampled_from([0.0, -1.0, float("nan"), float("inf"), -float("inf")])


@SETTINGS
@given(which=st.integers(0, 2), bad=bad_float, n=n_atoms)
def test_invalid_lengths_are_refused(which, bad, n):
    lib = cpmap.library()
    args = [0.5, 4.0, 12.0]
    args[which] = bad
    h, bs, rc = args
    L = _lat(50, 40, 30, h, 0.0, 0.0, 0.0)
    bd = (ctypes.c_int32 * 3)()
    assert lib.cpmap_bin_grid(*L, bs, rc, bd) == EINVAL
    assert lib.cpmap_bin_workspace_bytes(n, *L, bs, rc) == 0
    assert lib.cpmap_slot_workspace_bytes(n, *L, bs, rc, 8) == 0


@SETTINGS
@given(big=st.integers(16_777_217, 2**31 - 1), axis=st.integers(0, 2))
def test_oversized_axes_are_refused(big, axis):
    lib = cpmap.library()
    d = [4, 4, 4]
    d[axis] = big
    out = (ctypes.c_int32 * 5)()
    assert lib.cpmap_direct_plan(1000, *d, 1, out) != OK
    assert lib.cpmap_direct_workspace_bytes(1000, *d) == 0
    bd = (ctypes.c_int32 * 3)()
    assert lib.cpmap_bin_grid(*_lat(*d, 0.5, 0.0, 0.0, 0.0), 4.0, 12.0, bd) != OK


@SETTINGS
@given(n=st.sampled_from([2**31 - 2, 2**31 - 1, 2**31, 2**40, -1]), cap=st.integers(1, 256))
def test_atom_count_limit_is_enforced(n, cap):
    """n_atoms up to 2^31 - 1 is accepted by every size query and larger or
    negative counts are refused (sizes 0, status EINVAL or ERANGE)."""
    lib = cpmap.library()
    L = _lat(64, 48, 40, 0.5, 0.0, 0.0, 0.0)
    ok = 0 <= n <= 2**31 - 1
    b = lib.cpmap_bin_workspace_bytes(n, *L, 4.0, 12.0)
    sb = lib.cpmap_slot_workspace_bytes(n, *L, 4.0, 12.0, cap)
    out = (ctypes.c_int32 * 5)()
    st_plan = lib.cpmap_direct_plan(n, 64, 48, 40, 1, out)
    if ok:
        assert b >= 16 * n and sb >= 16 * n and st_plan == OK
        assert 1 <= out[4] <= 32
    else:
        assert b == 0 and sb == 0 and st_plan != OK
