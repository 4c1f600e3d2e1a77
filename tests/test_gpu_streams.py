"""Calls on several streams at once.  The library keeps no per-call state on
the device and guards its host-side workspace records with a lock, so paths
launched concurrently on different (default-priority) streams, from different
host threads, give the same bits as the same calls made one after another.
"""
import threading

import numpy as np
import pytest

import direct_coulomb_potential_amd as cpmap
from direct_coulomb_potential_amd import Lattice
from direct_coulomb_potential_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    return torch


def _paths(torch, atoms, lat, bs, rc):
    """bin + smoothed cutoff + slots + split direct + extrema on the current stream."""
    n = atoms.shape[0]
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    vc = cpmap.cutoff(ws, n, lat, bs, rc)
    sws = cpmap.bin_slots(ws, n, lat, bs, rc, 4)
    vs = cpmap.cutoff_slots(sws, n, lat, bs, rc, 4, term="truncated")
    vd = cpmap.direct(atoms, lat)
    idx, val = cpmap.extrema(vd)
    return vc, vs, vd, idx, val


def test_concurrent_streams_match_sequential_calls(torch):
    cases = [(Lattice(40, 36, 33, 0.5, (-1.0, 0.0, 2.0)), 1.5, 4.0, 20_000, 81),
             (Lattice(27, 50, 19, 0.3, (3.0, -2.0, 0.0)), 2.0, 3.0, 8_000, 82),
             (Lattice(64, 16, 48, 0.5), 4.0, 12.0, 30_000, 83),
             (Lattice(33, 33, 33, 0.7, (0.5, 0.5, 0.5)), 1.0, 2.5, 5_000, 84)]
    inputs = []
    for lat, bs, rc, n, seed in cases:
        lo = np.array(lat.origin) - rc
        hi = np.array(lat.origin) + np.array(lat.dims) * lat.spacing + rc
        inputs.append((torch.from_numpy(wl.random_atoms(n, lo, hi, seed=seed)).cuda(), lat, bs, rc))
    print("[streams] sequential reference", flush=True)
    want = [tuple(t.clone() for t in _paths(torch, *inp)) for inp in inputs]
    torch.cuda.synchronize()

    for rep in range(3):
        print(f"[streams] concurrent repetition {rep}", flush=True)
        got = [None] * len(inputs)
        errors = []

        def worker(k):
            try:
                s = torch.cuda.Stream()  # default priority
                with torch.cuda.stream(s):
                    got[k] = _paths(torch, *inputs[k])
                s.synchronize()
            except Exception as e:  # surfaced below
                errors.append(e)

        threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(inputs))]
        for t in threads:
            t.start()
        for t in threads:
            t.join()
        assert not errors, errors
        torch.cuda.synchronize()
        for k in range(len(inputs)):
            for a, b in zip(got[k], want[k]):
                assert torch.equal(a, b), (rep, k)
