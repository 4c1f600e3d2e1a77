"""The oracle's pins catch plausible mistakes (CPU only).  Each case plants
one mistake in a copy of oracle/cpmap_oracle.c (a dropped term, a wrong sign,
index or constant, a wrong comparison, a wrong tie rule ...), builds it with
the oracle's own flags, and runs tests/test_oracle_pins.py against that build
in a subprocess: the pins must fail.  An unmodified copy built the same way
must pass.  Nothing here touches the committed oracle or its library."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "cpmap_oracle.c")
FLAGS = ["-std=c11", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
         "-shared", "-w"]

# (what the mistake is, text in the source, its replacement)
MUTATIONS = [
    ("direct: dz term dropped", "const double dz = z - (double)atoms[4 * a + 2];",
     "const double dz = 0.0*z;"),
    ("node position: origin sign", "return (double)fmaf((float)i, h, origin);",
     "return (double)origin - (double)i * (double)h;"),
    ("node position: two roundings in fp64", "return (double)fmaf((float)i, h, origin);",
     "return (double)origin + (double)i * (double)h;"),
    ("node index: y decode", "    *j = (g / nx) % ny;", "    *j = g % ny;"),
    ("node index: x decode", "    *i = g % nx;", "    *i = (g / ny) % nx;"),
    ("smoothed term: GC2", "const double gc2 = 3.0", "const double gc2 = 2.0"),
    ("smoothed term: GC1", "const double gc1 = -5.0", "const double gc1 = -4.0"),
    ("1/r^2 instead of 1/r", "v += q / r;", "v += q / (r*r);"),
    ("cutoff test too wide", "if (r2 < rc2) {", "if (r2 <= 4*rc2) {"),
    ("scale sums q, not |q|", "s += fabs(q) / r;", "s += q / r;"),
    ("bin coordinate shifted", "return d / bs;", "return d / bs + 1e-3f;"),
    ("bin index transposed",
     "return (int32_t)(((int64_t)c[2] * dims[1] + c[1]) * dims[0] + c[0]);",
     "return (int32_t)(((int64_t)c[0] * dims[1] + c[1]) * dims[0] + c[2]);"),
    ("slots: capacity one too small", "if (fill[b] < capacity) {",
     "if (fill[b] < capacity - 1) {"),
    ("slots: capacity one too large", "if (fill[b] < capacity) {",
     "if (fill[b] <= capacity && b < nbins - 1) {"),
    ("slots: overflow in input order, not grouped by bin",
     "const int64_t dst = (int64_t)over_start[b] + fill[b]++;",
     "const int64_t dst = (int64_t)fill[0]++;"),
    ("slots: charged empty-slot marker", "slots[4 * e + 3] = 0.0f;", "slots[4 * e + 3] = 1.0f;"),
    ("slots: filled from the back", "memcpy(&slots[4 * ((int64_t)b * capacity + fill[b])]",
     "memcpy(&slots[4 * ((int64_t)b * capacity + capacity - 1 - fill[b])]"),
    ("halo floored", "const int32_t halo = (int32_t)ceilf(cutoff / bin_size);",
     "const int32_t halo = (int32_t)floorf(cutoff / bin_size);"),
    ("hard instead of smoothed term", "v += smoothed_term(q, r2, rcd);", "v += q / sqrt(r2);"),
    ("extrema: last index among equal minima", "if (imin < 0 || v < V[imin])",
     "if (imin < 0 || v <= V[imin])"),
    ("extrema: last index among equal maxima", "if (imax < 0 || v > V[imax])",
     "if (imax < 0 || v >= V[imax])"),
    ("extrema: NaN not skipped", "if (isnan(v))", "if (0 && isnan(v))"),
    ("extrema: argmax reported as argmin", "    out_index[0] = imin;", "    out_index[0] = imax;"),
    ("truncated: <= instead of <", "    return r2 < rc2f;", "    return r2 <= rc2f;"),
    ("truncated: decided in fp64", "    return r2 < rc2f;",
     "    return (double)dx * dx + (double)dy * dy + (double)dz * dz < (double)rc2f;"),
    ("truncated: dz*dy for dz^2", "const float r2 = dx * dx + dy * dy + dz * dz;",
     "const float r2 = dx * dx + dy * dy + dz * dy;"),
    ("truncated: fma chain instead of the listing's sum",
     "const float r2 = dx * dx + dy * dy + dz * dz;",
     "const float r2 = fmaf(dx, dx, fmaf(dy, dy, dz * dz));"),
    ("truncated: listing's sum in reverse order",
     "const float r2 = dx * dx + dy * dy + dz * dz;",
     "const float r2 = dz * dz + dy * dy + dx * dx;"),
    ("truncated: exact distance instead of fp32",
     "    return r2 < rc2f;",
     "    return (long double)dx * dx + (long double)dy * dy + (long double)dz * dz"
     " < (long double)rc2f;"),
    ("smoothed term: r^4 coefficient", "const double gamma = gc0 + r2 * (gc1 + r2 * gc2);",
     "const double gamma = gc0 + r2 * (gc1 + r2 * gc2 * 1.0001);"),
    ("smoothed term: gamma added, not subtracted", "return q * (1.0 / sqrt(r2) - gamma);",
     "return q * (1.0 / sqrt(r2) + gamma);"),
    ("smoothed term: GC0", "const double gc0 = 15.0 / (8.0 * rc);",
     "const double gc0 = 16.0 / (8.0 * rc);"),
    ("direct: charge sign", "v += q / r;", "v -= q / r;"),
    ("node index: z decode", "*k = g / ((int64_t)nx * (int64_t)ny);",
     "*k = g / ((int64_t)nx * (int64_t)nx);"),
    ("binning: reversed order inside a bin",
     "const int64_t dst = (int64_t)bin_start[ids[a]] + fill[ids[a]]++;",
     "const int64_t dst = (int64_t)bin_start[ids[a] + 1] - 1 - fill[ids[a]]++;"),
    ("binning: atoms on the grid's lower face dropped", "if (!(t >= 0.0f && t < (float)dims[d]))",
     "if (!(t > 0.0f && t < (float)dims[d]))"),
]


def _build_and_run_pins(tmp_dir, name, text):
    src = os.path.join(tmp_dir, name + ".c")
    lib = os.path.join(tmp_dir, "lib" + name + ".so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", *FLAGS, "-o", lib, src, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, CPMAP_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(HERE, "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-400:]


def test_pins_fail_on_every_planted_mistake(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    with open(SRC) as f:
        source = f.read()
    jobs = [("control", source)]
    for k, (what, old, new) in enumerate(MUTATIONS):
        assert old in source, f"mutation {what!r} no longer applies"
        jobs.append((f"m{k:02d}", source.replace(old, new)))
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(lambda j: _build_and_run_pins(str(tmp_path), *j), jobs))
    rc, out = results[0]
    assert rc == 0, f"unmodified oracle fails its pins:\n{out}"
    survivors = [MUTATIONS[k][0] for k, (rc, _) in enumerate(results[1:]) if rc != 1]
    assert not survivors, f"mistakes the pins do not catch: {survivors}"
