"""cpmap_extrema_noalloc, the allocation-free entry point (GPU).

Called through the C ABI (ctypes) with caller-owned outputs only; its result
must equal cpmap_extrema's -- index work, so bit for bit -- on two calls in a
row, the second with a smaller map (so the static scratch holds the first
call's slots when the second starts), then on an empty map and again on a
large one.  Collected last, so that a failure here hides no other test.
"""
import ctypes

import numpy as np
import pytest

import oracle
import direct_coulomb_potential_amd as cpmap

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


def _map(n, seed):
    rng = np.random.default_rng(seed)
    V = rng.integers(-1000, 1000, size=n).astype(np.float32)  # many ties
    V[rng.integers(0, n, size=max(n // 50, 1))] = np.nan
    V[rng.integers(0, n, size=max(n // 100, 1))] = -0.0
    return V


def _noalloc(torch, V):
    lib = cpmap.library()
    idx = torch.full((2,), 7, dtype=torch.int64, device="cuda")
    val = torch.full((2,), 7.0, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.cpmap_extrema_noalloc(V.data_ptr() if V.numel() else None, V.numel(),
                                   idx.data_ptr(), val.data_ptr(), stream)
    assert st == 0, cpmap.library().cpmap_status_str(st)
    return idx, val


def _with_workspace(torch, V):
    lib = cpmap.library()
    ws = torch.empty(lib.cpmap_extrema_workspace_bytes(V.numel()), dtype=torch.uint8,
                     device="cuda")
    return cpmap.extrema(V, workspace=ws)


@pytest.mark.parametrize("sizes", [(8_000_000, 4097), (1_000_003, 63, 0, 16_777_217)])
def test_noalloc_matches_extrema_on_calls_in_a_row(torch, sizes):
    print(f"[extrema noalloc] sizes {sizes}", flush=True)
    for k, n in enumerate(sizes):
        V_np = _map(n, seed=n + k) if n else np.zeros(0, np.float32)
        V = torch.from_numpy(V_np).cuda()
        i1, v1 = _noalloc(torch, V)
        i2, v2 = _with_workspace(torch, V)
        torch.cuda.synchronize()
        assert i1.cpu().tolist() == i2.cpu().tolist(), (n, i1, i2)
        assert v1.cpu().numpy().tobytes() == v2.cpu().numpy().tobytes(), (n, v1, v2)
        assert tuple(i1.cpu().tolist()) == oracle.extrema(V_np)[0]


def test_noalloc_rejects_bad_arguments(torch):
    lib = cpmap.library()
    idx = torch.empty(2, dtype=torch.int64, device="cuda")
    val = torch.empty(2, dtype=torch.float32, device="cuda")
    V = torch.zeros(10, device="cuda")
    assert lib.cpmap_extrema_noalloc(V.data_ptr(), -1, idx.data_ptr(), val.data_ptr(), None) == 1
    assert lib.cpmap_extrema_noalloc(V.data_ptr(), 1 << 37, idx.data_ptr(), val.data_ptr(),
                                     None) == 2
    assert lib.cpmap_extrema_noalloc(None, 10, idx.data_ptr(), val.data_ptr(), None) == 1
    assert lib.cpmap_extrema_noalloc(V.data_ptr(), 10, None, val.data_ptr(), None) == 1
    assert lib.cpmap_extrema_noalloc(V.data_ptr(), 10, idx.data_ptr() + 4, val.data_ptr(),
                                     None) == 1
