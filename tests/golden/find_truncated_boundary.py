"""Writes truncated_boundary.json: atoms within a few fp32 ulps of the cutoff
sphere r = 3 around a node at the origin, chosen so that the inclusion test of
the hard-truncated term decides differently depending on how r^2 is formed.

The test that matters is the one the case-study notes print in section 18.5
(the coulomb_cutoff listing): r2 = dx*dx + dy*dy + dz*dz in fp32, kept iff
r2 < rcut2.  Each atom below is one for which that fp32 value (left to right,
every step rounded) and one other way of forming r^2 -- the exact distance,
a fused-multiply-add chain fma(dx, dx, fma(dy, dy, dz*dz)), or the sum taken in
the reverse order -- fall on opposite sides of rcut2 = 9.  The search draws
random directions in numpy and checks every candidate in exact rational
arithmetic; it calls neither the oracle nor the GPU library.  Run from the
repository root:  python tests/golden/find_truncated_boundary.py
"""
import json
import os
from fractions import Fraction as F

import numpy as np

KINDS = {
    "exact_keeps_listing_drops": "exact r^2 < 9, listing r2 >= 9",
    "exact_drops_listing_keeps": "exact r^2 >= 9, listing r2 < 9",
    "listing_keeps_fma_drops": "listing r2 < 9, fma(dx,dx,fma(dy,dy,dz*dz)) >= 9",
    "listing_drops_fma_keeps": "listing r2 >= 9, fma chain < 9",
    "listing_keeps_reversed_drops": "listing r2 < 9, (dz*dz + dy*dy) + dx*dx >= 9",
    "listing_drops_reversed_keeps": "listing r2 >= 9, reversed sum < 9",
}


def round_f32(fr):
    """The fp32 value nearest to the rational fr (ties to even)."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(F(float(c)) - fr),
                                     int(np.array(c, np.float32).view(np.uint32)) & 1))


def forms(d):
    """r^2 of the difference vector d (3 fp32 values) formed four ways."""
    sq = [round_f32(F(float(v)) ** 2) for v in d]
    listing = round_f32(F(float(round_f32(F(float(sq[0])) + F(float(sq[1]))))) + F(float(sq[2])))
    reverse = round_f32(F(float(round_f32(F(float(sq[2])) + F(float(sq[1]))))) + F(float(sq[0])))
    t = round_f32(F(float(d[1])) ** 2 + F(float(sq[2])))
    fma = round_f32(F(float(d[0])) ** 2 + F(float(t)))
    exact = sum(F(float(v)) ** 2 for v in d)
    return {"listing": listing, "fma": fma, "reversed": reverse, "exact": exact}


def classify(d):
    f = forms(d)
    keep = {k: (v < 9) for k, v in f.items()}
    out = []
    for other in ("exact", "fma", "reversed"):
        if keep["listing"] != keep[other]:
            a, b = ("keeps", "drops") if keep["listing"] else ("drops", "keeps")
            out.append(f"{other}_{b}_listing_{a}" if other == "exact"
                       else f"listing_{a}_{other}_{b}")
    return out


def main():
    rng = np.random.default_rng(7)
    found = {}
    while len(found) < len(KINDS):
        v = rng.normal(size=3)
        v *= 3.0 * (1 + rng.uniform(-3e-7, 3e-7)) / np.linalg.norm(v)
        d = v.astype(np.float32)
        for kind in classify(d):
            if kind in KINDS and kind not in found:
                found[kind] = [float(-x) for x in d]  # atom = node - d, node at 0
    fx = {
        "citation": ("Case study -- electrostatic potential map, section 18.5, the "
                     "coulomb_cutoff listing: dx = x - a.x (likewise y, z) in fp32, "
                     "r2 = dx*dx + dy*dy + dz*dz, the atom is kept iff r2 < rcut2 and adds "
                     "q * rsqrtf(r2).  Node at the origin, rc = 3 so rcut2 = 9 exactly; each "
                     "atom is exact in fp32 and the node - atom differences are exact."),
        "rc": 3.0,
        "cases": [{"kind": k, "what": KINDS[k], "atom": found[k]} for k in KINDS],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "truncated_boundary.json")
    with open(path, "w") as f:
        json.dump(fx, f, indent=1)
        f.write("\n")
    print(path)


if __name__ == "__main__":
    main()
