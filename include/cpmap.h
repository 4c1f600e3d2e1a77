/*
 * cpmap.h -- electrostatic potential maps on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libcpmap.so.  Plain C: no HIP, torch or C++ types.  All calls are
 * host functions.  Unless a comment says "host", a pointer argument is a
 * device pointer (hipMalloc'd memory, or any memory the GPU can address).
 *
 * Common conventions
 *   - Atoms are n_atoms rows of 4 floats (x, y, z, q): positions in Angstrom,
 *     charges in units of e, 16-byte aligned, one float4 per atom.
 *   - The lattice has nx*ny*nz nodes; node (i,j,k) sits at
 *       (fl(ox + i*spacing), fl(oy + j*spacing), fl(oz + k*spacing))
 *     where fl() is one rounding to fp32 (the notes' gather listing puts node
 *     (gx,gy,gz) at (gx,gy,gz)*h with a zero origin; the origin is the
 *     generalisation).  V holds one fp32 per node, x-fastest:
 *       V[(k*ny + j)*nx + i]
 *     (the notes' section 18.4 on lattice index order).
 *   - Potentials are in e/Angstrom; no Coulomb constant is applied.
 *   - No call allocates or frees memory, synchronises, or prints.  Every GPU
 *     call is enqueued on `stream` (a hipStream_t; NULL = the null stream) and
 *     returns before the work finishes.  Execution faults surface at the
 *     caller's next synchronisation of that stream.
 *   - Arguments are checked on the host before any HIP call; a failed check
 *     returns a status and enqueues nothing.  Device data is not inspected:
 *     an atom placed exactly on a node gives an infinite potential there, and
 *     non-finite atom data propagates into V.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (except cpmap_direct_scatter, the atomics contrast, as stated there).
 */
#ifndef CPMAP_H
#define CPMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum cpmap_status {
    CPMAP_OK = 0,
    CPMAP_EINVAL = 1, /* null pointer, negative count, dimension < 0, spacing /
                         bin size / cutoff not finite or <= 0, misaligned ptr */
    CPMAP_ERANGE = 2, /* a count or index does not fit the library's limits */
    CPMAP_ENOSPC = 3, /* workspace smaller than cpmap_bin_workspace_bytes() */
    CPMAP_EGEOM = 4,  /* workspace was binned for another geometry or atom
                         count, was never binned, or was written since (see
                         "Workspace records" below) */
    CPMAP_EHIP = 5    /* the HIP runtime reported an error at launch */
} cpmap_status;

/* Library version, (major << 16) | (minor << 8) | patch.  Host. */
int32_t cpmap_version(void);

/* Static, human-readable name of a status code.  Host; never NULL. */
const char *cpmap_status_str(int32_t status);

/* Limits: n_atoms <= CPMAP_MAX_ATOMS; each lattice dimension <= CPMAP_MAX_DIM
 * (so that every node index is exact in fp32); nx*ny*nz <= CPMAP_MAX_POINTS. */
#define CPMAP_MAX_ATOMS 2147483647LL
#define CPMAP_MAX_DIM 16777216
#define CPMAP_MAX_POINTS 68719476736LL

/*
 * cpmap_node_position -- the node a linear index of a lattice map names, and
 * its position.  Host only, no HIP call.
 *
 * For index = (k*ny + j)*nx + i (the x-fastest order of V, the notes' section
 * 18.4) writes ijk_out (host, 3 int32) = (i, j, k) and xyz_out (host, 3
 * floats) = the node's position (fl(ox + i*spacing), fl(oy + j*spacing),
 * fl(oz + k*spacing)), the same fp32 values the kernels use (the gather
 * listing of section 18.2 puts node (gx, gy, gz) at (gx, gy, gz)*h).  With
 * cpmap_extrema it places ions at nodes (section 18.1: positive ions where
 * the potential is lowest, negative ions where it is highest).
 * Returns CPMAP_EINVAL for a null output or an invalid lattice, CPMAP_ERANGE
 * when index is outside [0, nx*ny*nz).
 */
cpmap_status cpmap_node_position(int32_t nx, int32_t ny, int32_t nz, float spacing,
                                 float ox, float oy, float oz, int64_t index,
                                 int32_t *ijk_out, float *xyz_out);

/*
 * cpmap_direct -- direct Coulomb summation over every atom.
 *
 * Computes V(g) = sum_a q_a / |g - a| at every lattice node g (the notes'
 * section 18.1 formula; section 18.2's gather mapping: each output node is
 * written once, by one GPU lane, with no atomics).  V is OVERWRITTEN with the
 * full sum (no accumulation into previous contents); n_atoms = 0 writes zeros.
 * A lattice with a zero dimension is a no-op (V may then be NULL).
 *
 *   atoms       device, n_atoms x float4 (x, y, z, q); read only
 *   n_atoms     0 <= n_atoms <= CPMAP_MAX_ATOMS
 *   nx, ny, nz  lattice dimensions, 0 <= n <= CPMAP_MAX_DIM
 *   spacing     lattice spacing h (finite, > 0)
 *   ox, oy, oz  position of node (0,0,0) (finite)
 *   V           device, nx*ny*nz floats, written
 *   stream      hipStream_t or NULL
 * Ownership: the caller owns atoms and V; both must stay valid until the
 * enqueued work completes.  Accuracy: fp32 with the hardware reciprocal
 * square root; |V - V_exact| <= 1e-5 * sum_a |q_a| / r at every node.
 */
cpmap_status cpmap_direct(const float *atoms, int64_t n_atoms,
                          int32_t nx, int32_t ny, int32_t nz, float spacing,
                          float ox, float oy, float oz,
                          float *V, void *stream);

/*
 * cpmap_direct_scatter -- the same sum in the scatter mapping, kept only as a
 * measured contrast to the gather (the case-study notes' section 18.2: a
 * thread per atom adds its q/r into every node with an atomic add).  One
 * wave per atom; its lanes add into 64 adjacent nodes at a time with
 * hardware fp32 atomics in L2.  V is zeroed, then accumulated.  The order in
 * which atoms reach a node varies, so V meets the accuracy bound of
 * cpmap_direct but is NOT bit-reproducible.  V must be ordinary device memory
 * (hipMalloc / torch), where the hardware fp32 atomics are valid.  Arguments
 * and errors as cpmap_direct.
 */
cpmap_status cpmap_direct_scatter(const float *atoms, int64_t n_atoms,
                                  int32_t nx, int32_t ny, int32_t nz, float spacing,
                                  float ox, float oy, float oz,
                                  float *V, void *stream);

/*
 * cpmap_direct_workspace_bytes -- size of the optional workspace that lets
 * cpmap_direct_with_workspace split the atom list across workgroups (0 when
 * the lattice and atom count gain nothing from it).  On lattices with at
 * least as many groups of 64 lanes' nodes as the GPU holds workgroups at
 * once, a few KB (a counter and one count per group); on smaller lattices,
 * K - 1 partial maps of the lattice, at most 64 MiB.  Host only, no HIP
 * call; depends only on n_atoms and the lattice dimensions.  0 on invalid
 * input.
 */
size_t cpmap_direct_workspace_bytes(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz);

/*
 * cpmap_direct_with_workspace -- the same direct sum as cpmap_direct, with a
 * small caller-owned workspace.  The library may then also split the atoms
 * into K contiguous parts handled by different workgroups.  On large
 * lattices part 0 of a group of nodes stores its sum into V, and part p adds
 * its sum into V once part p - 1 has added its own (the workspace holds the
 * counters that order them); on small lattices, where all parts run at
 * once, parts 1..K-1 write partial maps into the workspace that a second
 * kernel adds to V in part order.  Either way the additions happen in part
 * order on every run (no atomics on V, deterministic).  The short
 * per-workgroup atom slices run faster and even out the last round of
 * workgroups over the GPU.
 * Results agree with cpmap_direct within the accuracy bound (the summation
 * order differs).
 *
 *   workspace        device, >= cpmap_direct_workspace_bytes(...) bytes,
 *                    256-byte aligned (may be NULL when that size is 0);
 *                    overwritten, must stay valid until the work completes;
 *                    two calls that overlap on one workspace race
 *   workspace_bytes  its size; CPMAP_ENOSPC when too small
 * Other arguments, ownership and errors as cpmap_direct.
 */
cpmap_status cpmap_direct_with_workspace(const float *atoms, int64_t n_atoms,
                                         int32_t nx, int32_t ny, int32_t nz, float spacing,
                                         float ox, float oy, float oz, float *V,
                                         void *workspace, size_t workspace_bytes,
                                         void *stream);

/*
 * cpmap_direct_plan -- how a direct call of this size is launched: plan_out
 * (host, 5 int32) receives nodes per lane along x, y, z, waves per
 * workgroup, and atom parts across workgroups.  with_workspace selects the
 * plan of cpmap_direct_with_workspace (nonzero) or of cpmap_direct (0).
 * Host only, no HIP call.
 */
cpmap_status cpmap_direct_plan(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                               int32_t with_workspace, int32_t *plan_out);

/*
 * cpmap_direct_occupancy_check -- number of compiled direct-kernel variants
 * whose occupancy on the current device differs from the table the planner
 * assumes (0 when they all agree).  Calls the HIP runtime's occupancy query
 * (no device work).  A mismatch affects speed, never results.
 */
int32_t cpmap_direct_occupancy_check(void);

/*
 * Bin geometry (shared by the three cutoff calls below).  With bin size bs
 * and cutoff rc: halo H = ceil(rc/bs) bins on every side of the lattice; bin
 * grid origin b0 = fl(o - H*bs) per axis; nb per axis = floor(t_last) + 1 + H
 * with t_last the bin coordinate of the axis' last node.  An atom's bin
 * coordinate per axis is t = fl(fl(p - b0) / bs) in fp32; the atom is kept iff
 * 0 <= t < nb on every axis and then sits in bin floor(t) (the binning
 * lecture's pseudo-code slide: bin index = position / BIN_SIZE).  Atoms
 * outside the halo are at least rc from every node and are dropped.  Bins
 * are numbered x-fastest: (cz*nby + cy)*nbx + cx.
 */

/*
 * Workspace records.  cpmap_bin_atoms and cpmap_bin_slots record, on the host,
 * the range they fill, what they filled it for (atom count, lattice, bin size,
 * cutoff, capacity) and a fill number, and write a 16-byte header with that
 * number at the workspace's start (byte offset 0; the layouts below leave
 * its first 256 bytes to it).  A call that reads a filled workspace
 * (cpmap_cutoff, cpmap_cutoff_term, cpmap_bin_slots, cpmap_cutoff_slots)
 * returns CPMAP_EGEOM unless a record with the same base address, size and
 * arguments exists.  Every call that writes device memory (any V, any
 * workspace, the extrema outputs) first drops the records of the ranges it
 * writes, so a workspace rebinned through another address or used as an
 * output or scratch buffer by this library is refused afterwards.  Memory
 * written outside the library (for instance freed and reused by another
 * tensor) cannot be seen on the host: the cutoff kernels then compare the
 * device header with the record and, on a mismatch, read nothing and set
 * every node of V to NaN (cpmap_bin_slots passes the mismatch on to the slot
 * workspace).  A change that leaves the header intact but alters the bins
 * is not detected: the kernels clamp every offset they read, so it can give a
 * wrong map but never an access outside the workspace.  Records are kept
 * per process; calls from several threads are safe.
 */

/*
 * cpmap_bin_workspace_bytes -- size of the workspace that cpmap_bin_atoms
 * fills and cpmap_cutoff reads, for this atom count and geometry.  Host only,
 * no HIP call.  Returns 0 when the arguments are invalid or too large.
 */
size_t cpmap_bin_workspace_bytes(int64_t n_atoms,
                                 int32_t nx, int32_t ny, int32_t nz, float spacing,
                                 float ox, float oy, float oz,
                                 float bin_size, float cutoff);

/*
 * cpmap_bin_grid -- the bin-grid dimensions for a geometry.  Host only, no
 * HIP call.  dims_out (host, 3 int32) receives bins per axis; returns
 * CPMAP_OK or CPMAP_EINVAL / CPMAP_ERANGE.
 */
cpmap_status cpmap_bin_grid(int32_t nx, int32_t ny, int32_t nz, float spacing,
                            float ox, float oy, float oz,
                            float bin_size, float cutoff, int32_t *dims_out);

/*
 * cpmap_bin_atoms -- spatial binning of atoms (the binning lecture's
 * pseudo-code slide, step 1; the notes' section 18.5 BinTable: bins
 * flattened into one atom array with a start offset per bin).
 *
 * Sorts the atoms stably by bin on the GPU (input order kept inside a bin)
 * and writes, inside `workspace`:
 *   bin_start  (nbins + 1) int32: bin b holds sorted[bin_start[b] ..
 *              bin_start[b+1]); bin_start[nbins] = kept atoms
 *   sorted     float4 atoms in bin order
 * (offsets of both: cpmap_workspace_layout; a header occupies the first 256
 * bytes).  Records the fill as "Workspace records" above describes.
 *
 *   atoms, n_atoms, nx..oz   as in cpmap_direct
 *   bin_size, cutoff         finite, > 0 (Angstrom)
 *   workspace                device, >= cpmap_bin_workspace_bytes(...) bytes,
 *                            256-byte aligned; overwritten
 *   workspace_bytes          its size
 * Ownership: caller owns everything; the workspace must stay valid and
 * untouched until cpmap_cutoff's work on it completes.
 */
cpmap_status cpmap_bin_atoms(const float *atoms, int64_t n_atoms,
                             int32_t nx, int32_t ny, int32_t nz, float spacing,
                             float ox, float oy, float oz,
                             float bin_size, float cutoff,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * cpmap_workspace_layout -- byte offsets of bin_start and sorted inside a
 * workspace of this geometry (host only, no HIP call); -1 offsets on error.
 */
cpmap_status cpmap_workspace_layout(int64_t n_atoms,
                                    int32_t nx, int32_t ny, int32_t nz, float spacing,
                                    float ox, float oy, float oz,
                                    float bin_size, float cutoff,
                                    int64_t *bin_start_offset, int64_t *sorted_offset);

/*
 * cpmap_cutoff -- smoothed short-range potential with cutoff binning.
 *
 * For every node g: V(g) = sum over atoms with |g - a|^2 < rc^2 of
 *   q_a * (1/r - (GC0 + r^2 (GC1 + r^2 GC2))),
 *   GC0 = 15/(8 rc), GC1 = -5/(4 rc^3), GC2 = 3/(8 rc^5)
 * (the binning lecture's large-bin kernel slide gives the term's form; the
 * constants make it vanish with its first two derivatives at rc).  Each
 * workgroup owns an 8x8x8 tile of nodes, walks the neighbourhood of bins
 * whose box lies within rc of the tile (the lecture's neighbourhood offset
 * list), stages those bins' atoms in LDS and evaluates the term for each of
 * its nodes (the lecture's small-bin design).  V is OVERWRITTEN.
 *
 *   workspace, workspace_bytes   filled by cpmap_bin_atoms for the same
 *                                n_atoms and geometry; read only
 *   n_atoms, nx..cutoff          the values given to cpmap_bin_atoms
 *   V                            device, nx*ny*nz floats, written
 * Returns CPMAP_EGEOM if the workspace was not binned for these arguments
 * (its record, "Workspace records" above); V is all NaN if the workspace's
 * header no longer matches that record.
 * Accuracy: |V - V_exact| <= 1e-5 * sum_{r < rc} |q| / r at every node.
 */
cpmap_status cpmap_cutoff(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                          int32_t nx, int32_t ny, int32_t nz, float spacing,
                          float ox, float oy, float oz,
                          float bin_size, float cutoff,
                          float *V, void *stream);

/* Terms of the cutoff sum. */
enum {
    CPMAP_TERM_SMOOTHED = 0,  /* q (1/r - gamma(r^2)), as cpmap_cutoff */
    CPMAP_TERM_TRUNCATED = 1  /* q / r */
};

/*
 * cpmap_cutoff_term -- cpmap_cutoff with a choice of term.
 *
 * CPMAP_TERM_SMOOTHED is cpmap_cutoff.  CPMAP_TERM_TRUNCATED sums q / r over
 * the atoms with r^2 < rc^2 (the case-study notes' section 18.5 listing: the
 * bin scan adds q * rsqrt(r2) only when r2 < rcut2).  The inclusion test is
 * the listing's, in fp32: dx, dy, dz = fl(node - atom) and
 * r2 = dx*dx + dy*dy + dz*dz evaluated left to right with every product and
 * sum rounded (no fused multiply-add), kept iff r2 < fl(rc*rc); so an atom at
 * the boundary is kept or dropped as the listing decides it, on every call.
 * The kept terms use the hardware reciprocal square root.  The neighbourhood
 * of bins is widened for this term (cpmap_neighbor_spans) so that no kept
 * atom is missed.
 *
 *   term   CPMAP_TERM_SMOOTHED or CPMAP_TERM_TRUNCATED (else CPMAP_EINVAL)
 * Other arguments, ownership and errors as cpmap_cutoff.
 */
cpmap_status cpmap_cutoff_term(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                               int32_t nx, int32_t ny, int32_t nz, float spacing,
                               float ox, float oy, float oz,
                               float bin_size, float cutoff, int32_t term,
                               float *V, void *stream);

/*
 * cpmap_neighbor_spans -- the neighbourhood the cutoff kernel walks for one
 * tile with one term, for inspection and tests.  Host only, no HIP call.
 *
 * The tile with tile coordinates (tx, ty, tz) holds nodes
 * [8tx, 8tx+8) x [8ty, 8ty+8) x [8tz, 8tz+8) clipped to the lattice.  A bin is
 * in its neighbourhood iff the distance between the tile's node bounding box
 * and the bin's box is < R (the binning lecture's neighbourhood offset list,
 * with the box-to-box distance as the test), where R covers every atom the
 * term can keep:
 *   slack = 2^-21 * max over axes of (bins * bin_size)   (an atom's fp32 bin
 *           coordinate can place it up to 2^-23 |p - b0| outside its bin);
 *   CPMAP_TERM_SMOOTHED   R = cutoff, or cutoff + slack when slack exceeds
 *                         cutoff / 1024 (the term vanishes to third order at
 *                         the cutoff, so nearer misses add < 2^-30 |q|/rc);
 *   CPMAP_TERM_TRUNCATED  R = cutoff * (1 + 2^-16) + slack.
 * Such bins form runs along x; each run is reported as (cy, cz, cx_first,
 * cx_last) in spans_out (host, 4 int32 per span, capacity max_spans).
 * Returns the number of spans (possibly larger than max_spans, in which case
 * only max_spans were written), or -1 on invalid arguments.
 */
int64_t cpmap_neighbor_spans(int32_t nx, int32_t ny, int32_t nz, float spacing,
                             float ox, float oy, float oz,
                             float bin_size, float cutoff, int32_t term,
                             int32_t tx, int32_t ty, int32_t tz,
                             int32_t *spans_out, int64_t max_spans);

/*
 * Fixed-capacity bins (the binning lecture's slides 33-35: every bin has the
 * same number of atom slots, 8 slots of 16 bytes there, and the atoms that
 * do not fit their bin go to an extra list).  They are derived on the GPU from
 * a workspace binned by cpmap_bin_atoms, so a bin's slots hold its first
 * `capacity` atoms in input order and its later atoms are its overflow.  An
 * alternative layout for the cutoff sum, kept for measurement beside the CSR
 * (which never overflows).
 *
 * A slot workspace holds (byte offsets: cpmap_slot_layout; a header occupies
 * the first 256 bytes):
 *   slots       float4[nbins * capacity]: slot s of bin b at b*capacity + s;
 *               an empty slot is (+inf, +inf, +inf, 0).  Empty slots are told
 *               apart by their position, never by a zero charge, so a neutral
 *               atom is never taken for one.
 *   over_start  int32[nbins + 1]: the overflow atoms of bin b are
 *               over_atoms[over_start[b] .. over_start[b+1]), input order
 *   over_atoms  float4[n_atoms]; the first over_start[nbins] are written
 * 1 <= capacity <= CPMAP_MAX_SLOTS, and nbins * capacity < 2^31.
 */
#define CPMAP_MAX_SLOTS 256

/*
 * cpmap_slot_workspace_bytes -- size of a slot workspace for this atom
 * count, geometry and capacity.  Host only, no HIP call.  Returns 0 when the
 * arguments are invalid or too large.
 */
size_t cpmap_slot_workspace_bytes(int64_t n_atoms,
                                  int32_t nx, int32_t ny, int32_t nz, float spacing,
                                  float ox, float oy, float oz,
                                  float bin_size, float cutoff, int32_t capacity);

/*
 * cpmap_slot_layout -- byte offsets of slots, over_start and over_atoms inside
 * a slot workspace (host only, no HIP call); -1 offsets on error.
 */
cpmap_status cpmap_slot_layout(int64_t n_atoms,
                               int32_t nx, int32_t ny, int32_t nz, float spacing,
                               float ox, float oy, float oz,
                               float bin_size, float cutoff, int32_t capacity,
                               int64_t *slots_offset, int64_t *over_start_offset,
                               int64_t *over_atoms_offset);

/*
 * cpmap_bin_slots -- fill a slot workspace from a binned workspace.
 *
 *   workspace, workspace_bytes   filled by cpmap_bin_atoms for the same n_atoms
 *                                and geometry (else CPMAP_EGEOM); read only
 *   n_atoms, nx..cutoff          the values given to cpmap_bin_atoms
 *   capacity                     slots per bin, 1 .. CPMAP_MAX_SLOTS
 *   slot_workspace               device, >= cpmap_slot_workspace_bytes(...)
 *                                bytes, 256-byte aligned, not overlapping
 *                                workspace (else CPMAP_EINVAL); overwritten
 *   slot_workspace_bytes         its size (else CPMAP_ENOSPC)
 * Records the fill (geometry and capacity) as "Workspace records" above
 * describes.  Six stream-ordered launches; the result is the same on every
 * run.  Ownership: caller owns both workspaces; they must stay valid until
 * the work on them completes.
 */
cpmap_status cpmap_bin_slots(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                             int32_t nx, int32_t ny, int32_t nz, float spacing,
                             float ox, float oy, float oz,
                             float bin_size, float cutoff, int32_t capacity,
                             void *slot_workspace, size_t slot_workspace_bytes, void *stream);

/*
 * cpmap_cutoff_slots -- the cutoff sum of cpmap_cutoff_term over
 * fixed-capacity bins.
 *
 * Two launches of the cutoff kernel: the first walks the slots of each
 * tile's neighbourhood (a run of bins is a run of capacity-slot blocks) and
 * OVERWRITES V; the second walks the overflow list and ADDS into V, leaving
 * untouched the nodes of tiles with no overflow atom in reach (the lecture
 * computes the overflow on the CPU).  With no overflow V equals
 * cpmap_cutoff_term's bit for bit (the same atoms in the same order at every
 * node); with overflow it meets the same accuracy bound.
 *
 *   slot_workspace, bytes   filled by cpmap_bin_slots for the same n_atoms,
 *                           geometry and capacity (else CPMAP_EGEOM)
 *   term                    CPMAP_TERM_SMOOTHED or CPMAP_TERM_TRUNCATED
 * Other arguments, ownership and errors as cpmap_cutoff_term.
 */
cpmap_status cpmap_cutoff_slots(const void *slot_workspace, size_t slot_workspace_bytes,
                                int64_t n_atoms,
                                int32_t nx, int32_t ny, int32_t nz, float spacing,
                                float ox, float oy, float oz,
                                float bin_size, float cutoff, int32_t capacity, int32_t term,
                                float *V, void *stream);

/*
 * cpmap_extrema_workspace_bytes -- workspace of cpmap_extrema for n values
 * (at most 16 KB).  Host only, no HIP call; 0 on invalid n.
 */
size_t cpmap_extrema_workspace_bytes(int64_t n);

/*
 * cpmap_extrema -- ion placement on a potential map (the case-study notes'
 * section 18.1: positive ions are placed where the potential is lowest,
 * negative ions where it is highest).
 *
 * Writes, on the device, out_index[0] = argmin and out_index[1] = argmax of
 * V[0..n) and out_value[0..1] = the values there.  NaN values are skipped;
 * among equal values the smallest index wins (+0 and -0 are equal); with no
 * non-NaN value both indices are -1 and both values NaN.  For a lattice map,
 * cpmap_node_position turns an index into its node and position.
 *
 *   V          device, n floats (any layout; read only)
 *   out_index  device, 2 int64 (8-byte aligned), written
 *   out_value  device, 2 floats, written
 *   workspace  device, >= cpmap_extrema_workspace_bytes(n), 256-byte aligned;
 *              needs no clearing (its contents before the call do not matter)
 * One launch: each workgroup publishes a partial result tagged with a number
 * drawn for this call, and the last workgroup waits for all of them (a
 * bounded wait; an index of -2 would report that it ran out, which ordinary
 * runs never do).  Two calls that overlap on the same workspace race.
 * Deterministic: the result does not depend on the order in which partial
 * results are combined.
 */
cpmap_status cpmap_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * cpmap_extrema_noalloc -- cpmap_extrema without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * The same kernel as cpmap_extrema, with its scratch (512 slots of 32 bytes,
 * 16 KB) in a static device array of the library: one copy per GPU, allocated
 * when the library is loaded and held until the process ends.  The call
 * allocates and frees nothing.  Every call on one GPU shares that GPU's copy,
 * which needs no clearing between calls (each call tags its slots with a
 * fresh number); calls that overlap in time on one GPU (several streams or
 * host threads) race and may give wrong results.  Any n up to
 * CPMAP_MAX_POINTS fits the fixed scratch (the grid is capped at 512
 * workgroups); larger n is CPMAP_ERANGE.  The copy used is the current
 * device's (hipGetDevice), so the stream must belong to that device; a
 * stream of another device is CPMAP_EINVAL.
 *
 *   V, n, out_index, out_value, stream   as cpmap_extrema
 * Errors as cpmap_extrema; CPMAP_EHIP also when the scratch's device address
 * cannot be looked up.
 */
cpmap_status cpmap_extrema_noalloc(const float *V, int64_t n, int64_t *out_index,
                                   float *out_value, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CPMAP_H */
