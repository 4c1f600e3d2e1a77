/*
 * cpmap_oracle.c -- plain fp64 CPU oracle for electrostatic potential maps.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the bench's CPU
 * baseline load this; the cpmap library never does, and it shares no code,
 * header, table or helper with the GPU path.  It is slow on purpose: every
 * function is the plain definition written out, one lattice node at a time,
 * atoms summed in input order, OpenMP over nodes only.
 *
 * Sources (the pages):
 *   - "Case study -- electrostatic potential map" (PMPP ch. 18 study notes),
 *     section 18.1: V(g) = sum_a q_a / r_{a,g} over the atoms a, evaluated at
 *     every point g of a regular 3D lattice.
 *   - same page, section 18.2 (gather kernel listing): node (gx,gy,gz) sits at
 *     (gx,gy,gz)*h, lattice stored x-fastest, idx = (gz*Ny + gy)*Nx + gx.
 *   - same page, section 18.5: cutoff binning, "r2 < rcut2" is the test, and
 *     the listing adds q/r for the kept atoms (the hard-truncated term).
 *   - "Input Binning Lecture Chapter 2", large-bin kernel slide (slide 24):
 *     the short-range term q*(1/r - g(r2)) with g(r2) = GC0 + r2*(GC1 +
 *     r2*GC2), used only when r2 < CUTOFF2.  The constants GC0..GC2 are not
 *     printed there; the workload fixes them as GC0 = 15/(8 rc),
 *     GC1 = -5/(4 rc^3), GC2 = 3/(8 rc^5) (the quadratic in r^2 that meets 1/r
 *     with value, slope and curvature at rc).
 *   - same slides, pseudo-code slide (slide 28): bin index = position / BIN_SIZE,
 *     atoms appended to their bin.
 *
 * Readings taken where the pages leave a step open (each is restated where it
 * is used):
 *   R1  node (i,j,k) sits at (fl(ox + i*h), fl(oy + j*h), fl(oz + k*h)), where
 *       fl() is one rounding to fp32 (the lattice is an fp32 object; the pages
 *       put node g at g*h with an implicit zero origin).
 *   R2  the direct sum runs over every atom, in fp64, with no Coulomb constant
 *       (units e/Angstrom).  An atom exactly on a node is outside the domain.
 *   R3  the cutoff sum keeps an atom iff r^2 < rc^2 (strict), r^2 and rc^2 in
 *       fp64 from the fp32 inputs.
 *   R4  the tolerance scale returned beside V is S = sum |q|/r over the atoms
 *       the sum keeps.
 *   R5  binning: halo H = ceil(rc/bs) bins on each side of the lattice; bin
 *       grid origin b0 = fl(o - H*bs) per axis; atom bin coordinate
 *       t = fl(fl(p - b0) / bs) in fp32; the atom is kept iff 0 <= t < nb on
 *       every axis, and then sits in bin floor(t).  nb per axis = (bin of the
 *       last lattice node) + 1 + H.  Bins are linear x-fastest; atoms sorted
 *       stably by bin (input order inside a bin).
 *   R14 the hard-truncated cutoff (the notes' section 18.5 listing: q/r added
 *       only when r2 < rcut2) decides inclusion with the listing's own fp32
 *       expression: dx, dy, dz = fl32(node - atom), r2 = dx*dx + dy*dy + dz*dz
 *       evaluated left to right, every product and sum rounded to fp32 (no
 *       contraction: the build passes -ffp-contract=off), kept iff
 *       r2 < rcut2 with rcut2 = fl32(rc*rc).  The kept terms are summed in
 *       fp64.  (An inclusion decision is integer work decided in floating
 *       point, so it is taken in the precision and order the page prints.)
 *   R15 ion placement (the notes' section 18.1: positive ions go where the
 *       potential is lowest, negative ions where it is highest): the extrema
 *       of V over its non-NaN nodes; among equal values the smallest node
 *       index; -1 when every node is NaN.
 *   R16 fixed-capacity bins ("Input Binning Lecture Chapter 2", slides 33-35:
 *       bins of 8 atom slots, 128 bytes, the atoms that do not fit go to an
 *       extra list): atoms are appended to their bin's slots in input order
 *       until the slots are full; the later atoms of that bin form its
 *       overflow, and the overflow list is kept grouped by bin (input order
 *       inside a bin).  An empty slot holds (+inf, +inf, +inf, 0): a slot is
 *       recognised as empty by its position, never by a zero charge, because
 *       a real atom may be neutral.
 *
 * Pins: tests/test_oracle_pins.py checks these functions against closed forms,
 * hand-derived values and invariants.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* R1: one rounding of the exact o + i*h to fp32 (C99 fmaf is exact-then-round). */
static double node_coord(float origin, float h, int64_t i)
{
    return (double)fmaf((float)i, h, origin);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Split a linear x-fastest node index into (i, j, k): idx = (k*ny + j)*nx + i. */
static void split_index(int64_t g, int32_t nx, int32_t ny,
                        int64_t *i, int64_t *j, int64_t *k)
{
    *i = g % nx;
    *j = (g / nx) % ny;
    *k = g / ((int64_t)nx * (int64_t)ny);
}

/*
 * Direct Coulomb sum (page 1, section 18.1, with readings R1, R2, R4).
 *   atoms   n_atoms x 4 floats (x, y, z, q), Angstrom and e.
 *   nodes   linear x-fastest node indices to evaluate, or NULL for every node
 *           of the nx*ny*nz lattice in storage order (then n_nodes must equal
 *           nx*ny*nz).
 *   V, S    n_nodes doubles each (S may be NULL): the potential and the
 *           tolerance scale sum |q|/r.
 */
void oracle_direct(const float *atoms, int64_t n_atoms,
                   int32_t nx, int32_t ny, int32_t nz, float h,
                   float ox, float oy, float oz,
                   const int64_t *nodes, int64_t n_nodes,
                   double *V, double *S)
{
    (void)nz;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_nodes; ++t) {
        int64_t g = nodes ? nodes[t] : t;
        int64_t i, j, k;
        split_index(g, nx, ny, &i, &j, &k);
        const double x = node_coord(ox, h, i);
        const double y = node_coord(oy, h, j);
        const double z = node_coord(oz, h, k);
        double v = 0.0, s = 0.0;
        for (int64_t a = 0; a < n_atoms; ++a) {
            const double dx = x - (double)atoms[4 * a + 0];
            const double dy = y - (double)atoms[4 * a + 1];
            const double dz = z - (double)atoms[4 * a + 2];
            const double q = (double)atoms[4 * a + 3];
            const double r = sqrt(dx * dx + dy * dy + dz * dz);
            v += q / r;
            s += fabs(q) / r;
        }
        V[t] = v;
        if (S)
            S[t] = s;
    }
}

/*
 * The smoothed short-range term of one atom at squared distance r2 (slide 24
 * of the binning lecture; constants as stated in the file header):
 *   q * (1/r - (GC0 + r2*(GC1 + r2*GC2)))  for r2 < rc^2, else 0.
 */
static double smoothed_term(double q, double r2, double rc)
{
    const double gc0 = 15.0 / (8.0 * rc);
    const double gc1 = -5.0 / (4.0 * rc * rc * rc);
    const double gc2 = 3.0 / (8.0 * rc * rc * rc * rc * rc);
    const double gamma = gc0 + r2 * (gc1 + r2 * gc2);
    return q * (1.0 / sqrt(r2) - gamma);
}

/* Exposed so that the pins can probe the term itself at chosen distances. */
double oracle_smoothed_term(double q, double r, double rc)
{
    const double r2 = r * r;
    if (!(r2 < rc * rc))
        return 0.0;
    return smoothed_term(q, r2, rc);
}

/*
 * Brute-force cutoff sum: every atom is visited, no bins (readings R1-R4).
 * Arguments as oracle_direct plus the cutoff radius rc (Angstrom).
 * S receives sum |q|/r over the atoms with r < rc.
 */
void oracle_cutoff(const float *atoms, int64_t n_atoms,
                   int32_t nx, int32_t ny, int32_t nz, float h,
                   float ox, float oy, float oz, float rc,
                   const int64_t *nodes, int64_t n_nodes,
                   double *V, double *S)
{
    (void)nz;
    const double rcd = (double)rc;
    const double rc2 = rcd * rcd;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_nodes; ++t) {
        int64_t g = nodes ? nodes[t] : t;
        int64_t i, j, k;
        split_index(g, nx, ny, &i, &j, &k);
        const double x = node_coord(ox, h, i);
        const double y = node_coord(oy, h, j);
        const double z = node_coord(oz, h, k);
        double v = 0.0, s = 0.0;
        for (int64_t a = 0; a < n_atoms; ++a) {
            const double dx = x - (double)atoms[4 * a + 0];
            const double dy = y - (double)atoms[4 * a + 1];
            const double dz = z - (double)atoms[4 * a + 2];
            const double r2 = dx * dx + dy * dy + dz * dz;
            if (r2 < rc2) {
                const double q = (double)atoms[4 * a + 3];
                v += smoothed_term(q, r2, rcd);
                s += fabs(q) / sqrt(r2);
            }
        }
        V[t] = v;
        if (S)
            S[t] = s;
    }
}

/* Inclusion test of the hard-truncated cutoff (reading R14): the section 18.5
 * listing's r2 = dx*dx + dy*dy + dz*dz in fp32, left to right, no contraction. */
static int hard_keep(float x, float y, float z, const float *a, float rc2f)
{
    const float dx = x - a[0];
    const float dy = y - a[1];
    const float dz = z - a[2];
    const float r2 = dx * dx + dy * dy + dz * dz;
    return r2 < rc2f;
}

/*
 * Hard-truncated cutoff sum (the notes' section 18.5 listing; reading R14):
 * V = sum of q/r over the atoms the listing's fp32 test keeps, r and the sum
 * in fp64.
 * S receives sum |q|/r over the same atoms.
 */
void oracle_cutoff_hard(const float *atoms, int64_t n_atoms,
                        int32_t nx, int32_t ny, int32_t nz, float h,
                        float ox, float oy, float oz, float rc,
                        const int64_t *nodes, int64_t n_nodes,
                        double *V, double *S)
{
    (void)nz;
    const float rc2f = rc * rc;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < n_nodes; ++t) {
        int64_t g = nodes ? nodes[t] : t;
        int64_t i, j, k;
        split_index(g, nx, ny, &i, &j, &k);
        const float xf = fmaf((float)i, h, ox);
        const float yf = fmaf((float)j, h, oy);
        const float zf = fmaf((float)k, h, oz);
        double v = 0.0, s = 0.0;
        for (int64_t a = 0; a < n_atoms; ++a) {
            if (!hard_keep(xf, yf, zf, &atoms[4 * a], rc2f))
                continue;
            const double dx = (double)xf - (double)atoms[4 * a + 0];
            const double dy = (double)yf - (double)atoms[4 * a + 1];
            const double dz = (double)zf - (double)atoms[4 * a + 2];
            const double q = (double)atoms[4 * a + 3];
            const double r = sqrt(dx * dx + dy * dy + dz * dz);
            v += q / r;
            s += fabs(q) / r;
        }
        V[t] = v;
        if (S)
            S[t] = s;
    }
}

/* ---- binning (reading R5) ------------------------------------------------ */

/* Bin coordinate of a position along one axis, fp32 as R5 states. */
static float bin_coord(float p, float b0, float bs)
{
    const float d = p - b0;
    return d / bs;
}

/*
 * Bin-grid geometry for one axis: halo H, grid origin b0 and bin count nb.
 * Returns 0 on success, -1 if the counts do not fit an int32.
 */
static int axis_bins(int32_t n, float h, float o, float bs, int32_t halo,
                     float *b0, int32_t *nb)
{
    *b0 = fmaf(-(float)halo, bs, o);
    const float last = fmaf((float)(n - 1), h, o);
    const float t = bin_coord(last, *b0, bs);
    if (!(t >= 0.0f) || t > 1.0e9f)
        return -1;
    *nb = (int32_t)floorf(t) + 1 + halo;
    return 0;
}

/*
 * Bin-grid dimensions for a lattice, bin size and cutoff (R5).
 * dims_out[0..2] = bins per axis; b0_out[0..2] = bin grid origin; returns the
 * halo H, or -1 when the inputs are invalid.
 */
int32_t oracle_bin_grid(int32_t nx, int32_t ny, int32_t nz, float h,
                        float ox, float oy, float oz,
                        float bin_size, float cutoff,
                        int32_t *dims_out, float *b0_out)
{
    if (nx <= 0 || ny <= 0 || nz <= 0 || !(h > 0.0f) || !(bin_size > 0.0f) ||
        !(cutoff > 0.0f))
        return -1;
    const int32_t halo = (int32_t)ceilf(cutoff / bin_size);
    if (axis_bins(nx, h, ox, bin_size, halo, &b0_out[0], &dims_out[0]) ||
        axis_bins(ny, h, oy, bin_size, halo, &b0_out[1], &dims_out[1]) ||
        axis_bins(nz, h, oz, bin_size, halo, &b0_out[2], &dims_out[2]))
        return -1;
    return halo;
}

/* Linear x-fastest bin of one atom (R5), or -1 when it lies outside the grid. */
static int32_t atom_bin(const float *atom, const int32_t dims[3], const float b0[3],
                        float bin_size)
{
    int32_t c[3];
    for (int d = 0; d < 3; ++d) {
        const float t = bin_coord(atom[d], b0[d], bin_size);
        if (!(t >= 0.0f && t < (float)dims[d]))
            return -1;
        c[d] = (int32_t)floorf(t);
    }
    return (int32_t)(((int64_t)c[2] * dims[1] + c[1]) * dims[0] + c[0]);
}

/*
 * Stable counting sort of atoms into the bin grid (R5; slide 28's
 * "bin[position / BIN_SIZE] += atom", kept in input order inside a bin).
 *   bin_start  nbins+1 int32: atoms of bin b are sorted[bin_start[b] ..
 *              bin_start[b+1]); bin_start[nbins] = number of kept atoms.
 *   sorted     n_atoms x 4 floats (only the first n_kept rows are written).
 *   bin_of     n_atoms int32 (may be NULL): the bin of each input atom, or -1
 *              for a dropped atom.
 * Returns the number of kept atoms, or -1 on invalid geometry.
 */
int64_t oracle_bin_atoms(const float *atoms, int64_t n_atoms,
                         int32_t nx, int32_t ny, int32_t nz, float h,
                         float ox, float oy, float oz,
                         float bin_size, float cutoff,
                         int32_t *bin_start, float *sorted, int32_t *bin_of)
{
    int32_t dims[3];
    float b0[3];
    if (oracle_bin_grid(nx, ny, nz, h, ox, oy, oz, bin_size, cutoff, dims, b0) < 0)
        return -1;
    const int64_t nbins = (int64_t)dims[0] * dims[1] * dims[2];
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_atoms > 0 ? n_atoms : 1));
    if (!ids)
        return -1;
    memset(bin_start, 0, sizeof(int32_t) * (size_t)(nbins + 1));
    for (int64_t a = 0; a < n_atoms; ++a) {
        ids[a] = atom_bin(&atoms[4 * a], dims, b0, bin_size);
        if (ids[a] >= 0)
            bin_start[ids[a] + 1] += 1;
    }
    for (int64_t b = 0; b < nbins; ++b)
        bin_start[b + 1] += bin_start[b];
    int32_t *fill = (int32_t *)calloc((size_t)nbins + 1, sizeof(int32_t));
    if (!fill) {
        free(ids);
        return -1;
    }
    for (int64_t a = 0; a < n_atoms; ++a) {
        if (ids[a] < 0)
            continue;
        const int64_t dst = (int64_t)bin_start[ids[a]] + fill[ids[a]]++;
        memcpy(&sorted[4 * dst], &atoms[4 * a], 4 * sizeof(float));
    }
    if (bin_of)
        memcpy(bin_of, ids, sizeof(int32_t) * (size_t)n_atoms);
    free(fill);
    free(ids);
    return bin_start[nbins];
}

/*
 * Fixed-capacity bins with an overflow list (R16).
 *   slots       nbins*capacity x 4 floats: slot s of bin b is row
 *               b*capacity + s; empty slots hold (+inf, +inf, +inf, 0).
 *   over_start  nbins+1 int32: the overflow atoms of bin b are rows
 *               over_start[b] .. over_start[b+1]-1 of over_atoms.
 *   over_atoms  n_atoms x 4 floats (only the first over_start[nbins] rows
 *               are written).
 * Atoms outside the bin grid are dropped, as in oracle_bin_atoms.  Returns
 * the number of overflow atoms, or -1 on invalid arguments.
 */
int64_t oracle_bin_slots(const float *atoms, int64_t n_atoms,
                         int32_t nx, int32_t ny, int32_t nz, float h,
                         float ox, float oy, float oz,
                         float bin_size, float cutoff, int32_t capacity,
                         float *slots, int32_t *over_start, float *over_atoms)
{
    int32_t dims[3];
    float b0[3];
    if (capacity < 1 ||
        oracle_bin_grid(nx, ny, nz, h, ox, oy, oz, bin_size, cutoff, dims, b0) < 0)
        return -1;
    const int64_t nbins = (int64_t)dims[0] * dims[1] * dims[2];
    int32_t *fill = (int32_t *)calloc((size_t)nbins, sizeof(int32_t));
    int32_t *over_bin = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_atoms > 0 ? n_atoms : 1));
    if (!fill || !over_bin) {
        free(fill);
        free(over_bin);
        return -1;
    }
    for (int64_t e = 0; e < nbins * capacity; ++e) {
        slots[4 * e + 0] = INFINITY;
        slots[4 * e + 1] = INFINITY;
        slots[4 * e + 2] = INFINITY;
        slots[4 * e + 3] = 0.0f;
    }
    memset(over_start, 0, sizeof(int32_t) * (size_t)(nbins + 1));
    /* the sequential fill: each atom takes the next free slot of its bin */
    for (int64_t a = 0; a < n_atoms; ++a) {
        over_bin[a] = -1;
        const int32_t b = atom_bin(&atoms[4 * a], dims, b0, bin_size);
        if (b < 0)
            continue;
        if (fill[b] < capacity) {
            memcpy(&slots[4 * ((int64_t)b * capacity + fill[b])], &atoms[4 * a],
                   4 * sizeof(float));
            fill[b] += 1;
        } else {
            over_bin[a] = b;
            over_start[b + 1] += 1;
        }
    }
    /* group the overflow list by bin, input order inside a bin */
    for (int64_t b = 0; b < nbins; ++b)
        over_start[b + 1] += over_start[b];
    memset(fill, 0, sizeof(int32_t) * (size_t)nbins);
    for (int64_t a = 0; a < n_atoms; ++a) {
        const int32_t b = over_bin[a];
        if (b < 0)
            continue;
        const int64_t dst = (int64_t)over_start[b] + fill[b]++;
        memcpy(&over_atoms[4 * dst], &atoms[4 * a], 4 * sizeof(float));
    }
    free(fill);
    free(over_bin);
    return over_start[nbins];
}

/*
 * Extrema of a potential map for ion placement (reading R15).  out_index[0] =
 * argmin, out_index[1] = argmax (smallest index among equal values, NaN
 * nodes skipped, -1 when there is no non-NaN node); out_value[0..1] = the
 * values at those nodes (NaN when the index is -1).
 */
void oracle_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value)
{
    int64_t imin = -1, imax = -1;
    for (int64_t i = 0; i < n; ++i) {
        const float v = V[i];
        if (isnan(v))
            continue;
        if (imin < 0 || v < V[imin])
            imin = i;
        if (imax < 0 || v > V[imax])
            imax = i;
    }
    out_index[0] = imin;
    out_index[1] = imax;
    out_value[0] = imin >= 0 ? V[imin] : NAN;
    out_value[1] = imax >= 0 ? V[imax] : NAN;
}
