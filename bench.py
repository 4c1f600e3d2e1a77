"""Benchmark of the potential-map hot path on one MI355X.

One step = one direct-sum call (cpmap_direct_with_workspace: atoms also split
across workgroups, their sums added into V in part order) over the 200^3
lattice (0.5 A) with
200,000 uniform atoms (charges U[-1,1] shifted to net zero): 1.6e12
atom-node evaluations.  After the timed direct steps the same run times the cutoff path
(cpmap_bin_atoms + cpmap_cutoff) on the 100k-atom, rc = 12 A, 4 A-bin system
over the same lattice and reports it beside the headline number.

Prints ONE JSON line.  `value` is atom-node evaluations per second (G/s) with
inputs already resident in HBM; `roofline` prices the direct kernel against the
fp32 VALU peak at 10 FLOP per evaluation; `cpu_baseline` times the fp64 oracle
on a bounded sample of nodes on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 vector peak (256 CU x 2.4 GHz x 256 FLOP/clk)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_CLOCK_GHZ = 2.4       # engine clock the peak is quoted at
FLOP_PER_EVAL = 10
# Work of one in-cutoff atom-node pair of the cutoff kernel, counted as the
# binning lecture's slide-24 term is written: the Coulomb part as the direct
# sum's 10 FLOP, plus gamma(r^2) = GC0 + r^2 (GC1 + r^2 GC2) (two fused
# multiply-adds, 4 FLOP) and its subtraction (1) for the smoothed term; the
# hard-truncated term (the case-study section 18.5 listing) is the Coulomb
# part alone.
FLOP_PER_CUTOFF_PAIR = {"smoothed": 15, "truncated": 10}


def profile_record(profile: str, source: str):
    """The JSON record of a committed rocprofv3 counter summary, or None when
    the kernel source has changed since the counters were taken."""
    import hashlib
    import re
    try:
        with open(os.path.join(ROOT, "profiles", profile)) as f:
            block = re.search(r"```json\n(.*?)\n```", f.read(), re.S)
        rec = json.loads(block.group(1))
        with open(os.path.join(ROOT, source), "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, AttributeError, ValueError):
        return None
    if rec.get("source_sha256") != sha:
        return None
    return rec


def measured_traffic(profile: str, source: str):
    """HBM bytes per launch from a committed counter summary (None if stale)."""
    rec = profile_record(profile, source)
    return rec.get("traffic_bytes_per_launch") if rec else None


def host_cpu():
    """CPU model and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target CPU time of the oracle baseline sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-cutoff", action="store_true")
    p.add_argument("--all-configs", action="store_true",
                   help="also time the direct path on every lattice/atom configuration "
                        "(median and minimum of 10 after 3 warm-ups) and, in the CPU "
                        "baseline, the oracle on each configuration's checked nodes")
    p.add_argument("--only", choices=["direct", "cutoff", "copy", "small"], default=None,
                   help="time one path only (for profiler runs); 'copy' runs the plain "
                        "256 MiB copy kernel that calibrates the HBM byte counters; "
                        "'small' the direct sum on the single plane and the 100x100x50 "
                        "lattice (10,000 atoms each)")
    p.add_argument("--no-direct-compare", action="store_true",
                   help="skip the direct sum on the cutoff atoms (for profiler runs)")
    p.add_argument("--settle", type=float, default=SETTLE_S,
                   help="seconds of untimed calls before each side measurement; profiler "
                        "runs pass 0 so that every launch sequence has a fixed length")
    return p.parse_args()


# Untimed calls before the side measurements: after the GPU has idled (host
# work between sections), its engine clock needs some 20-40 ms of load to
# rise again, and millisecond-scale launches timed right away read it rising.
SETTLE_S = 0.25


def time_launches(torch, fn, steps, warmup, settle_s=0.0):
    """Call fn for settle_s seconds of wall time and then warmup more times,
    untimed; then `steps` times between device syncs, each launch bracketed by
    events on torch's current stream (the stream the library launches on).
    Returns (wall seconds of the timed region, per-launch ms)."""
    t_end = time.perf_counter() + settle_s
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [a.elapsed_time(b) for a, b in evs]


def cpu_baseline(oracle, w, target_s):
    """The fp64 oracle, as it stands, on a bounded node sample of the workload."""
    lat = w.lattice
    rng = np.random.default_rng(1234)
    probe = rng.integers(0, lat.n_points, size=1024, dtype=np.int64)
    oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, nodes=probe[:64])  # thread start-up
    t0 = time.perf_counter()
    oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, nodes=probe)
    rate = probe.size * w.n_atoms / max(time.perf_counter() - t0, 1e-6)
    n_nodes = int(min(max(rate * target_s / w.n_atoms, 256), lat.n_points))
    nodes = rng.integers(0, lat.n_points, size=n_nodes, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, nodes=nodes)
    dt = time.perf_counter() - t0
    return {
        "value": n_nodes * w.n_atoms / dt / 1e9,
        "unit": "G evals/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        **host_cpu(),
        "sample": f"{n_nodes} random nodes of the 200^3 lattice x all {w.n_atoms} atoms, fp64, "
                  f"{dt:.1f} s",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by lattice z-slabs, one per GPU, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import direct_coulomb_potential_amd as cpmap
    from direct_coulomb_potential_amd import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    cpmap.library()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.only == "copy":
        # calibration: one elementwise kernel reading and writing 256 MiB each
        a = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 2.0, out=b)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4}))
        return

    if args.only == "small":
        print(json.dumps(bench_small(torch, cpmap, wl, dev, args)))
        return

    w = wl.large_direct()
    lat = w.lattice
    pairs = w.pairs
    result = {
        "metric": "atom-gridpoint evals/sec (G/s) + % FP32 VALU peak, 200³ grid × 200k atoms",
        "unit": "G evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded uniform atoms, charges U[-1,1] shifted to net zero)",
        "config": {"workload": w.name, "lattice": list(lat.dims), "spacing": lat.spacing,
                   "atoms": w.n_atoms, "pairs_per_step": pairs, "parallelism": "single GPU"},
    }

    if args.only in (None, "direct"):
        atoms = torch.from_numpy(w.atoms).to(dev)
        V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device=dev)
        ws_bytes = cpmap.direct_workspace_bytes(w.n_atoms, lat)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        plan = cpmap.direct_plan(w.n_atoms, lat, True)
        result["config"]["plan"] = {"nodes_per_lane": list(plan[:3]), "waves_per_workgroup": plan[3],
                                    "atom_parts": plan[4], "workspace_bytes": ws_bytes}
        fn = lambda: cpmap.direct(atoms, lat, out=V, workspace=ws)  # noqa: E731
        wall, per = time_launches(torch, fn, args.steps, args.warmup)
        ms_step = wall / args.steps * 1e3
        kern_ms = statistics.mean(per)
        achieved = FLOP_PER_EVAL * pairs / (kern_ms * 1e-3) / 1e12
        result.update({
            "value": pairs * args.steps / wall / 1e9,
            "ms_per_step": ms_step,
            "pct_fp32_valu_peak": 100.0 * FLOP_PER_EVAL * pairs / (ms_step * 1e-3) / 1e12
            / PEAK_FP32_TFLOPS,
        })
        prof = profile_record("direct_kernel_200cube_200k.md",
                              "direct_coulomb_potential_amd/csrc/direct.hip")
        clock = prof.get("clock_ghz") if prof else None
        result["roofline"] = {
            "bound": "alu",
            "achieved": achieved,
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_FP32_TFLOPS,
            "traffic": measured_traffic("direct_kernel_200cube_200k.md",
                                        "direct_coulomb_potential_amd/csrc/direct.hip"),
            "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated)",
            "kernel": "direct_kernel (+ chain_reset, the split's counter clear, inside the same events)",
            "kernel_ms_mean": kern_ms,
            "kernel_ms_median": statistics.median(per),
            "kernel_ms_min": min(per),
            "flop_per_eval": FLOP_PER_EVAL,
            # the peak scaled to the engine clock the counters measured
            "clock_ghz_measured": clock,
            "frac_at_measured_clock": (achieved / (PEAK_FP32_TFLOPS * clock / PEAK_CLOCK_GHZ)
                                       if clock else None),
            # rocprof's VALUBusy from the committed counters (>= 100: every
            # SIMD's VALU issue saturated; null once the source has changed)
            "valu_busy_pct_from_counters": prof.get("valu_busy_pct") if prof else None,
        }
        # cpmap_direct, the call without a workspace (no atom split), on the
        # same map: timed beside the headline (two launches after one warm-up)
        _, per_plain = time_launches(torch, lambda: cpmap.direct(atoms, lat, out=V, split=False),
                                     2, 1)
        plain_ms = statistics.median(per_plain)
        result["roofline"]["no_workspace"] = {
            "entry_point": "cpmap_direct",
            "plan": list(cpmap.direct_plan(w.n_atoms, lat, False)),
            "kernel_ms_median": plain_ms,
            "achieved": FLOP_PER_EVAL * pairs / (plain_ms * 1e-3) / 1e12,
            "frac": FLOP_PER_EVAL * pairs / (plain_ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        }
        # ion placement on the map just computed: argmin / argmax over 8M nodes
        ext_ws = torch.empty(cpmap.library().cpmap_extrema_workspace_bytes(lat.n_points),
                             dtype=torch.uint8, device=dev)
        ext_out = (torch.empty(2, dtype=torch.int64, device=dev),
                   torch.empty(2, dtype=torch.float32, device=dev))
        _, per_ext = time_launches(torch, lambda: cpmap.extrema(V, workspace=ext_ws, out=ext_out),
                                   max(args.steps, 10), args.warmup)
        ext_ms = statistics.median(per_ext)
        ext_prof = profile_record("extrema_kernel_200cube.md",
                                  "direct_coulomb_potential_amd/csrc/extrema.hip")
        ext_kernel_ms = ext_prof["kernel_median_ns"] * 1e-6 if ext_prof else None
        result["ion_placement"] = {
            "op": "argmin/argmax of V (cpmap_extrema)",
            # event-timed call (includes the launch), and the kernel's own
            # median duration from the committed trace (null once stale)
            "ms_median": ext_ms,
            "hbm_gbs_algorithmic": 4 * lat.n_points / (ext_ms * 1e-3) / 1e9,
            "kernel_ms_from_trace": ext_kernel_ms,
            "kernel_hbm_gbs_algorithmic": (4 * lat.n_points / (ext_kernel_ms * 1e-3) / 1e9
                                           if ext_kernel_ms else None),
            "peak_gbs": PEAK_HBM_GBS,
        }
        del atoms, V, ws, ext_ws

    if args.only is None:
        result["gather_vs_scatter"] = bench_scatter(torch, cpmap, wl, dev, args)

    if not args.no_cutoff and args.only in (None, "cutoff"):
        result["cutoff"] = bench_cutoff(torch, cpmap, wl, dev, args)

    if args.all_configs and args.only is None:
        result["configs"] = bench_all_configs(torch, cpmap, wl, dev,
                                              result["roofline"].get("clock_ghz_measured"),
                                              args.settle)

    if not args.no_cpu_baseline and args.only is None:
        import oracle
        result["cpu_baseline"] = cpu_baseline(oracle, w, args.cpu_seconds)
        if args.all_configs:
            result["cpu_baseline"]["per_config"] = oracle_per_config(oracle, wl)

    print(json.dumps(result), flush=True)


def bench_small(torch, cpmap, wl, dev, args):
    """The direct sum on the two 10,000-atom workloads (the single plane k = 10
    and the 100x100x50 lattice): event-timed launches (median, minimum) and
    the same number of launches back to back between two events."""
    out = {}
    steps = max(args.steps, 20)
    for w in (wl.plane_direct(), wl.full_direct()):
        lat = w.lattice
        atoms = torch.from_numpy(w.atoms).to(dev)
        V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device=dev)
        ws = torch.empty(max(cpmap.direct_workspace_bytes(w.n_atoms, lat), 1), dtype=torch.uint8,
                         device=dev)
        fn = lambda: cpmap.direct(atoms, lat, out=V, workspace=ws)  # noqa: E731
        _, per = time_launches(torch, fn, steps, args.warmup, settle_s=args.settle)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        med, b2b = statistics.median(per), a.elapsed_time(b) / steps
        out[w.name] = {
            "plan": list(cpmap.direct_plan(w.n_atoms, lat, True)),
            "ms_median": med,
            "ms_min": min(per),
            "ms_back_to_back": b2b,
            "pct_fp32_peak": 100.0 * FLOP_PER_EVAL * w.pairs / (med * 1e-3) / 1e12
            / PEAK_FP32_TFLOPS,
            "pct_fp32_peak_back_to_back": 100.0 * FLOP_PER_EVAL * w.pairs / (b2b * 1e-3) / 1e12
            / PEAK_FP32_TFLOPS,
        }
    return out


def bench_all_configs(torch, cpmap, wl, dev, clock, settle_s):
    """The direct path on workloads 1-4 and on the cutoff workload's atoms:
    hipEvent-timed, 3 warm-ups, then the median and minimum of 10 calls."""
    out = {}
    for w in (wl.plane_direct(), wl.full_direct(), wl.protein_direct(), wl.large_direct(),
              wl.cutoff_binned()):
        lat = w.lattice
        atoms = torch.from_numpy(w.atoms).to(dev)
        V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device=dev)
        need = cpmap.direct_workspace_bytes(w.n_atoms, lat)
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _, per = time_launches(torch, lambda: cpmap.direct(atoms, lat, out=V, workspace=ws),
                               10, 3, settle_s=settle_s)
        med = statistics.median(per)
        tflops = FLOP_PER_EVAL * w.pairs / (med * 1e-3) / 1e12
        out[w.name] = {
            "path": "direct",
            "pairs": w.pairs,
            "ms_median": med,
            "ms_min": min(per),
            "G_evals_per_s": w.pairs / (med * 1e-3) / 1e9,
            "pct_fp32_peak": 100.0 * tflops / PEAK_FP32_TFLOPS,
            "pct_fp32_peak_at_measured_clock": (100.0 * tflops
                                                / (PEAK_FP32_TFLOPS * clock / PEAK_CLOCK_GHZ)
                                                if clock else None),
            "hbm_gbs_algorithmic": (16 * w.n_atoms + 4 * lat.n_points) / (med * 1e-3) / 1e9,
            "plan": list(cpmap.direct_plan(w.n_atoms, lat, True)),
        }
        del atoms, V, ws
    # the cutoff sum on the clustered atoms: dense bins, heavy 8-slot overflow
    w = wl.protein_direct()
    lat, bs, rc = w.lattice, 4.0, 12.0
    atoms = torch.from_numpy(w.atoms).to(dev)
    V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device=dev)
    ws = cpmap.bin_atoms(atoms, lat, bs, rc)
    sws = cpmap.bin_slots(ws, w.n_atoms, lat, bs, rc, 8)
    n_over = int(cpmap.slot_views(sws, w.n_atoms, lat, bs, rc, 8)[1][-1].item())
    _, per_bin = time_launches(torch, lambda: cpmap.bin_atoms(atoms, lat, bs, rc, workspace=ws),
                               10, 3)
    _, per_cut = time_launches(torch, lambda: cpmap.cutoff(ws, w.n_atoms, lat, bs, rc, out=V),
                               10, 3)
    _, per_slot = time_launches(
        torch, lambda: cpmap.cutoff_slots(sws, w.n_atoms, lat, bs, rc, 8, out=V), 10, 3)
    out["cutoff_" + w.name + "_rc12_bin4"] = {
        "path": "cutoff (smoothed), CSR bins and 8-slot bins",
        "bin_ms_median": statistics.median(per_bin),
        "cutoff_ms_median": statistics.median(per_cut),
        "cutoff_slots_ms_median": statistics.median(per_slot),
        "slot_overflow_fraction": n_over / w.n_atoms,
        "speedup_vs_direct": out[w.name]["ms_median"]
        / (statistics.median(per_cut) + statistics.median(per_bin)),
    }
    return out


def oracle_per_config(oracle, wl):
    """The oracle, as it stands, on each workload's checked nodes: every node
    of the two 100x100 workloads, three z-slices plus 10^4 random nodes of the
    200^3 ones (brute-force cutoff for the cutoff workload)."""
    out = {}
    for w in (wl.plane_direct(), wl.full_direct(), wl.protein_direct(), wl.large_direct(),
              wl.cutoff_binned()):
        lat = w.lattice
        nodes = None if lat.n_points <= 500_000 else wl.checked_nodes(lat)
        n_nodes = lat.n_points if nodes is None else nodes.size
        t0 = time.perf_counter()
        if w.cutoff:
            oracle.cutoff(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=nodes)
        else:
            oracle.direct(w.atoms, lat.dims, lat.spacing, lat.origin, nodes=nodes)
        dt = time.perf_counter() - t0
        out[w.name] = {
            "nodes": n_nodes,
            "pairs": n_nodes * w.n_atoms,
            "s": dt,
            "G_evals_per_s": n_nodes * w.n_atoms / dt / 1e9,
            "kind": "brute-force cutoff" if w.cutoff else "direct",
            "cores": oracle.num_threads(),
        }
    return out


def bench_scatter(torch, cpmap, wl, dev, args):
    """The gather (production) against the atomics-based scatter contrast on
    the two 100x100x50-lattice workloads."""
    out = {}
    for w in (wl.plane_direct(), wl.full_direct()):
        lat = w.lattice
        atoms = torch.from_numpy(w.atoms).to(dev)
        V = torch.empty((lat.nz, lat.ny, lat.nx), dtype=torch.float32, device=dev)
        ws = torch.empty(max(cpmap.direct_workspace_bytes(w.n_atoms, lat), 1), dtype=torch.uint8,
                         device=dev)
        _, per_g = time_launches(torch, lambda: cpmap.direct(atoms, lat, out=V, workspace=ws),
                                 max(args.steps, 5), args.warmup)
        _, per_s = time_launches(torch, lambda: cpmap.direct_scatter(atoms, lat, out=V),
                                 max(args.steps, 5), args.warmup)
        g_ms, s_ms = statistics.median(per_g), statistics.median(per_s)
        out[w.name] = {"pairs": w.pairs, "gather_ms": g_ms, "scatter_ms": s_ms,
                       "gather_G_evals_per_s": w.pairs / (g_ms * 1e-3) / 1e9,
                       "scatter_G_evals_per_s": w.pairs / (s_ms * 1e-3) / 1e9,
                       "scatter_over_gather": s_ms / g_ms}
    return out


def bench_cutoff(torch, cpmap, wl, dev, args):
    w = wl.cutoff_binned()
    lat = w.lattice
    atoms = torch.from_numpy(w.atoms).to(dev)
    bs, rc = w.bin_size, w.cutoff
    try:
        ws = cpmap.bin_atoms(atoms, lat, bs, rc)
        V = cpmap.cutoff(ws, w.n_atoms, lat, bs, rc)
        torch.cuda.synchronize()
    except cpmap.CpmapError as e:
        return {"skipped": str(e)}
    # L2 flush buffer (larger than the 8 x 4 MB of L2) between timed runs
    flush = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

    def run_bin():
        cpmap.bin_atoms(atoms, lat, bs, rc, workspace=ws)

    def run_cut():
        cpmap.cutoff(ws, w.n_atoms, lat, bs, rc, out=V)

    def run_trunc():
        cpmap.cutoff(ws, w.n_atoms, lat, bs, rc, out=V, term="truncated")

    def run_both():
        flush.zero_()
        run_bin()
        run_cut()

    steps = max(args.steps, 5)
    _, per_bin = time_launches(torch, run_bin, steps, args.warmup, settle_s=args.settle)
    _, per_cut = time_launches(torch, run_cut, steps, args.warmup, settle_s=args.settle)
    _, per_trunc = time_launches(torch, run_trunc, steps, args.warmup, settle_s=args.settle)
    wall_e2e, _ = time_launches(torch, run_both, steps, args.warmup)
    _, per_pair = time_launches(torch, lambda: (run_bin(), run_cut()), steps, args.warmup)
    graph = capture_graph(torch, lambda: (run_bin(), run_cut()))
    _, per_graph = time_launches(torch, graph.replay, steps, args.warmup)
    cut_ms = statistics.median(per_cut)
    bin_ms = statistics.median(per_bin)
    if args.no_direct_compare:
        dir_ms = float("nan")
    else:
        Vd = torch.empty_like(V)
        wsd = torch.empty(max(cpmap.direct_workspace_bytes(w.n_atoms, lat), 1), dtype=torch.uint8,
                          device=dev)
        _, per_dir = time_launches(torch, lambda: cpmap.direct(atoms, lat, out=Vd, workspace=wsd),
                                   2, 1)
        dir_ms = statistics.median(per_dir)
    bytes_alg = 16 * w.n_atoms + 4 * lat.n_points
    in_cut, in_cut_note = in_cutoff_pairs(w)
    trunc_ms = statistics.median(per_trunc)

    def tflops(term, ms):
        return in_cut * FLOP_PER_CUTOFF_PAIR[term] / (ms * 1e-3) / 1e12
    prof = profile_record("cutoff_kernel_200cube_100k_rc12.md",
                          "direct_coulomb_potential_amd/csrc/cutoff.hip")
    examined = prof.get("pairs_evaluated") if prof else None
    out = {
        "workload": w.name,
        "fixed_slots": bench_slots(torch, cpmap, w, ws, V, cut_ms, steps, args),
        "bin_ms_median": bin_ms,
        "cutoff_ms_median": cut_ms,
        "cutoff_ms_min": min(per_cut),
        "truncated_term_ms_median": trunc_ms,
        # the cutoff kernel against the same fp32 vector peak, at the FLOP per
        # in-cutoff pair above (event-timed kernel launches, median)
        "roofline": {
            "bound": "alu",
            "achieved": tflops("smoothed", cut_ms),
            "peak": PEAK_FP32_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops("smoothed", cut_ms) / PEAK_FP32_TFLOPS,
            "kernel": "cutoff_kernel (smoothed term)",
            "flop_per_in_cutoff_pair": FLOP_PER_CUTOFF_PAIR["smoothed"],
            "truncated_achieved": tflops("truncated", trunc_ms),
            "truncated_frac": tflops("truncated", trunc_ms) / PEAK_FP32_TFLOPS,
            "truncated_flop_per_in_cutoff_pair": FLOP_PER_CUTOFF_PAIR["truncated"],
        },
        "end_to_end_ms_with_l2_flush": wall_e2e / steps * 1e3,
        "bin_plus_cutoff_ms_median": statistics.median(per_pair),
        "bin_plus_cutoff_hip_graph_ms_median": statistics.median(per_graph),
        "direct_same_atoms_ms": dir_ms,
        "speedup_vs_direct": dir_ms / (cut_ms + bin_ms),
        "hbm_gbs_algorithmic": bytes_alg / (cut_ms * 1e-3) / 1e9,
        "hbm_traffic_bytes_per_launch": measured_traffic(
            "cutoff_kernel_200cube_100k_rc12.md", "direct_coulomb_potential_amd/csrc/cutoff.hip"),
        "direct_equivalent_G_evals_per_s": w.pairs / ((cut_ms + bin_ms) * 1e-3) / 1e9,
        "in_cutoff_pairs": in_cut,
        "in_cutoff_pairs_note": in_cut_note,
        "in_cutoff_G_pairs_per_s": in_cut / (cut_ms * 1e-3) / 1e9,
        "evaluated_pairs_from_counters": examined,
        "evaluated_G_pairs_per_s": examined / (cut_ms * 1e-3) / 1e9 if examined else None,
        # the cutoff kernel is VALU-bound too: rocprof's VALUBusy from the
        # committed counters (null once the source has changed)
        "valu_busy_pct_from_counters": prof.get("valu_busy_pct") if prof else None,
        "hbm_traffic_gbs_from_counters": (prof["traffic_bytes_per_launch"] / (cut_ms * 1e-3) / 1e9
                                          if prof else None),
    }
    if not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cutoff_cpu_baseline(oracle, w, in_cut / lat.n_points)
    return out


def in_cutoff_pairs(w, n_sample=20000):
    """Atom-node pairs with r < rc, estimated from a seeded sample of nodes
    (each sampled node's count is exact up to ties at r = rc; the total is the
    mean times the node count)."""
    from scipy.spatial import cKDTree
    lat = w.lattice
    rng = np.random.default_rng(4321)
    nodes = rng.integers(0, lat.n_points, size=n_sample, dtype=np.int64)
    i = nodes % lat.nx
    j = (nodes // lat.nx) % lat.ny
    k = nodes // (lat.nx * lat.ny)
    o = np.asarray(lat.origin, np.float64)
    P = np.stack([o[0] + i * lat.spacing, o[1] + j * lat.spacing, o[2] + k * lat.spacing], 1)
    tree = cKDTree(w.atoms[:, :3].astype(np.float64))
    counts = tree.query_ball_point(P, w.cutoff, return_length=True)
    mean = counts.mean()
    sem = counts.std(ddof=1) / np.sqrt(n_sample)
    return float(mean * lat.n_points), (f"estimated from {n_sample} random nodes: "
                                        f"{mean:.1f} +- {sem:.1f} atoms per node")


def cutoff_cpu_baseline(oracle, w, in_cut_per_node, target_s=4.0):
    """The oracle's brute-force cutoff sum (every atom tested at every node),
    as it stands, on a bounded node sample of the cutoff workload."""
    lat = w.lattice
    rng = np.random.default_rng(5678)
    probe = rng.integers(0, lat.n_points, size=256, dtype=np.int64)
    oracle.cutoff(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=probe[:32])
    t0 = time.perf_counter()
    oracle.cutoff(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=probe)
    per_node = max(time.perf_counter() - t0, 1e-6) / probe.size
    n_nodes = int(min(max(target_s / per_node, 256), lat.n_points))
    nodes = rng.integers(0, lat.n_points, size=n_nodes, dtype=np.int64)
    t0 = time.perf_counter()
    oracle.cutoff(w.atoms, lat.dims, lat.spacing, lat.origin, w.cutoff, nodes=nodes)
    dt = time.perf_counter() - t0
    return {
        "ms_full_map_extrapolated": dt / n_nodes * lat.n_points * 1e3,
        "G_pair_tests_per_s": n_nodes * w.n_atoms / dt / 1e9,
        "in_cutoff_G_pairs_per_s": n_nodes * in_cut_per_node / dt / 1e9,
        "cores": oracle.num_threads(),
        "kind": "oracle",
        **host_cpu(),
        "sample": f"{n_nodes} random nodes x all {w.n_atoms} atoms (brute force), fp64, {dt:.1f} s",
    }


def capture_graph(torch, fn):
    """Capture fn (library launches only) into a HIP graph on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def bench_slots(torch, cpmap, w, ws, V, csr_cut_ms, steps, args, cap=8):
    """Fixed-capacity bins (8 slots per bin, the binning lecture's layout)
    with a GPU overflow pass, timed beside the CSR cutoff on the same atoms."""
    lat, bs, rc = w.lattice, w.bin_size, w.cutoff
    try:
        sws = cpmap.bin_slots(ws, w.n_atoms, lat, bs, rc, cap)
        cpmap.cutoff_slots(sws, w.n_atoms, lat, bs, rc, cap, out=V)
        torch.cuda.synchronize()
    except cpmap.CpmapError as e:
        return {"skipped": str(e)}
    n_over = int(cpmap.slot_views(sws, w.n_atoms, lat, bs, rc, cap)[1][-1].item())
    _, per_fill = time_launches(
        torch, lambda: cpmap.bin_slots(ws, w.n_atoms, lat, bs, rc, cap, slot_workspace=sws),
        steps, args.warmup)
    _, per_cut = time_launches(
        torch, lambda: cpmap.cutoff_slots(sws, w.n_atoms, lat, bs, rc, cap, out=V),
        steps, args.warmup)
    cut_ms = statistics.median(per_cut)
    return {
        "capacity": cap,
        "overflow_atoms": n_over,
        "overflow_fraction": n_over / max(w.n_atoms, 1),
        "bin_slots_ms_median": statistics.median(per_fill),
        "cutoff_slots_ms_median": cut_ms,
        "vs_csr_cutoff": cut_ms / csr_cut_ms,
    }


if __name__ == "__main__":
    main()
