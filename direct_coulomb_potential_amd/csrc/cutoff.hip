// Cutoff summation with spatial bins on gfx950.
//
// For every node g, over the atoms with r^2 < rc^2:
//   smoothed   V(g) = sum q * (1/r - (GC0 + r^2 (GC1 + r^2 GC2)))
//              (the binning lecture's large-bin kernel slide gives the term;
//              the constants make it vanish with two derivatives at rc);
//   truncated  V(g) = sum q / r  (the case-study notes' section 18.5 listing),
//              with the listing's inclusion test: r2 = dx*dx + dy*dy + dz*dz
//              in fp32, left to right, every step rounded (no fma), kept iff
//              r2 < fl(rc*rc).
//
// Structure (the lecture's small-bin design, re-planned for CDNA4):
//  - one workgroup per 8x8x8 tile of nodes (4 A of lattice at 0.5 A spacing,
//    the lecture's "(4 A)^3 cube of the map per thread block");
//  - the tile's neighbourhood: every bin whose box lies within rc of the
//    tile's node bounding box (the lecture's neighbourhood offset list).  The
//    qualifying bins of one (cy, cz) row form one contiguous x-run, and a
//    run's atoms are contiguous in the CSR, so the neighbourhood is a short
//    list of (start, count) spans.  The workgroup builds the list in its
//    prologue from the tile's exact node box, so it is tight for every tile
//    and needs no table;
//  - the spans' atoms are staged into LDS (the lecture's "fetch bins of data
//    into shared memory", one bin at a time there; all spans at once here, in
//    chunks of kStage atoms, small enough that LDS allows 5 resident waves
//    per SIMD);
//  - each wave owns an 8x8x4 half of the tile as four 4x4x4-node cubes of 16
//    lanes, and each cube keeps, in an LDS list of byte offsets into the
//    stage, only the staged atoms within rc of its node box (one atom per
//    lane tested against the four boxes, ballot + prefix count), which
//    removes about half of the examined pairs at 4 A bins; this is the
//    lecture's "sphere of bins" idea applied per cube at atom granularity;
//    atoms within rc of the whole cube go to the front of its list and skip
//    the cutoff test, the smoothed term's polynomial part of those atoms
//    coming from their moments (see Moments);
//  - each lane owns kNx consecutive nodes of one x-row and reads its cube's
//    listed atoms (one LDS address per cube, four per wave read; lists of
//    unequal length end under an execution mask), shares dy and dz across
//    its nodes, and
//    adds the term with r^2 clamped to the largest value <= rc^2 at which the
//    fp32 term is exactly 0 (found in the prologue; the select-based mask
//    q -> 0 is the fallback), so atoms beyond the cutoff add exactly nothing
//    and nodes beyond rc of every atom get exactly 0;
//  - V is written once per node, x-fastest.
//
// The same kernel walks fixed-capacity bins (the lecture's slides 33-35): a
// run of bins is then a run of cap-slot blocks, whose span follows from the
// geometry alone, and empty slots (at +inf) never pass the per-cube list
// test.  The bins' overflow is a CSR of its own; a second launch walks it and
// adds into V, skipping tiles whose neighbourhood holds no overflow atom.
#include <cmath>

#include "cpmap_internal.h"

namespace cpmap {

// ---- neighbourhood of a tile (host and device) -------------------------------

namespace {

struct AxisRange {
    int32_t first, last;
};

// Candidate bins along one axis: boxes that can come within rc of [lo, hi].
__host__ __device__ inline AxisRange axis_candidates(double lo, double hi, double rc, double b0,
                                                     double bs, int32_t nb)
{
    double f = floor((lo - rc - b0) / bs);
    double l = floor((hi + rc - b0) / bs);
    if (f < 0.0)
        f = 0.0;
    if (l > (double)(nb - 1))
        l = (double)(nb - 1);
    AxisRange r;
    r.first = (int32_t)f;
    r.last = (int32_t)l;
    return r;
}

// Distance between the node interval [lo, hi] and bin c's box [b0 + c bs,
// b0 + (c+1) bs] (0 when they overlap).
__host__ __device__ inline double axis_gap(double lo, double hi, double b0, double bs, int32_t c)
{
    const double blo = b0 + (double)c * bs;
    const double bhi = blo + bs;
    if (bhi < lo)
        return lo - bhi;
    if (blo > hi)
        return blo - hi;
    return 0.0;
}

// Node bounding box of tile t along one axis (nodes 8t .. min(8t+7, n-1)).
__host__ __device__ inline void tile_box(int32_t t, int32_t n, float h, float o, double *lo,
                                         double *hi)
{
    const int64_t first = (int64_t)t * kTile;
    int64_t last = first + kTile - 1;
    if (last > n - 1)
        last = n - 1;
    *lo = (double)node_coord(first, h, o);
    *hi = (double)node_coord(last, h, o);
}

// The x-run of bins of one (cy, cz) row whose box is within rc of the tile's
// box, given the row's squared y/z gap; false when the row has none.
__host__ __device__ inline bool row_run(double xlo, double xhi, double b0x, double bs,
                                        int32_t nbx, double rc, double gyz2, int32_t *cx0,
                                        int32_t *cx1)
{
    const double rc2 = rc * rc;
    if (!(gyz2 < rc2))
        return false;
    const AxisRange xr = axis_candidates(xlo, xhi, rc, b0x, bs, nbx);
    int32_t a = xr.first, b = xr.last;
    while (a <= b) {
        const double g = axis_gap(xlo, xhi, b0x, bs, a);
        if (g * g + gyz2 < rc2)
            break;
        ++a;
    }
    while (b >= a) {
        const double g = axis_gap(xlo, xhi, b0x, bs, b);
        if (g * g + gyz2 < rc2)
            break;
        --b;
    }
    if (a > b)
        return false;
    *cx0 = a;
    *cx1 = b;
    return true;
}

// A tile's node box, its candidate bin rows, and the bin geometry the rows
// are tested against (in double, as the neighbourhood is decided).
struct TileRows {
    double lo[3], hi[3];
    double b0[3], bs, rc;
    AxisRange ry, rz;
    int32_t nbx, ncy, nrows;
};

__host__ __device__ inline TileRows tile_rows(int32_t tx, int32_t ty, int32_t tz,
                                              const int32_t n[3], float h, const float o[3],
                                              const float b0[3], const int32_t nb[3], float bs,
                                              float rc)
{
    TileRows T;
    for (int a = 0; a < 3; ++a)
        T.b0[a] = (double)b0[a];
    T.bs = (double)bs;
    T.rc = (double)rc;
    T.nbx = nb[0];
    tile_box(tx, n[0], h, o[0], &T.lo[0], &T.hi[0]);
    tile_box(ty, n[1], h, o[1], &T.lo[1], &T.hi[1]);
    tile_box(tz, n[2], h, o[2], &T.lo[2], &T.hi[2]);
    T.ry = axis_candidates(T.lo[1], T.hi[1], (double)rc, (double)b0[1], (double)bs, nb[1]);
    T.rz = axis_candidates(T.lo[2], T.hi[2], (double)rc, (double)b0[2], (double)bs, nb[2]);
    T.ncy = T.ry.last - T.ry.first + 1;
    const int32_t ncz = T.rz.last - T.rz.first + 1;
    T.nrows = (T.ncy > 0 && ncz > 0) ? T.ncy * ncz : 0;
    return T;
}

// Row rr of a tile's candidate rows (z-major, then y) -> its bins' x-run.
__host__ __device__ inline bool tile_row(const TileRows &T, int32_t rr, int32_t *cy,
                                         int32_t *cz, int32_t *cx0, int32_t *cx1)
{
    *cy = T.ry.first + rr % T.ncy;
    *cz = T.rz.first + rr / T.ncy;
    const double gy = axis_gap(T.lo[1], T.hi[1], T.b0[1], T.bs, *cy);
    const double gz = axis_gap(T.lo[2], T.hi[2], T.b0[2], T.bs, *cz);
    return row_run(T.lo[0], T.hi[0], T.b0[0], T.bs, T.nbx, T.rc, gy * gy + gz * gz, cx0, cx1);
}

// ---- kernel -------------------------------------------------------------------

constexpr int kNx = 4;                                 // nodes per lane along x
constexpr int kThreads = kTile * kTile * kTile / kNx;  // 128
constexpr int kCube = 4;                               // a list group's cube of nodes
constexpr int kGroupLanes = kCube * kCube * kCube / kNx;  // 16 lanes per cube
constexpr int kGroups = 64 / kGroupLanes;              // 4 cubes per wave
constexpr int kStage = 256;                            // atoms staged per chunk (4 KB)
constexpr int kMaxRows = 256;                          // (cy, cz) rows per list chunk
// Resident waves per SIMD the kernel is built for: the sweep is latency-bound
// on its LDS reads below this (on the 100k-atom rc = 12 A map, built for 4
// waves: 1.51 / 1.46 ms for the smoothed / truncated term, against 1.45 /
// 1.38 ms at 5).  LDS per workgroup (about 14 KB: the stage and eight lists
// of kStage entries) allows 5 as well.
constexpr int kWavesPerSimd = 5;

// kRsqInside serves atoms within the cutoff of every node of the wave, which
// need neither the clamp nor the inclusion test: it adds q/r only (the
// smoothed term's polynomial part of these atoms is added from their
// moments, see Moments).
enum TermMode { kSmoothClamp = 0, kSmoothSelect = 1, kTruncated = 2, kRsqInside = 3 };

struct CutoffParams {
    float h, o[3];
    int32_t n[3];
    int32_t tiles[3];
    float b0[3];
    int32_t nb[3];
    float bs, rc, rc2;
    float list_rc;  // radius of the bin neighbourhood (neighbourhood_radius)
    float gc0, gc1, gc2;
    int32_t truncated;
    int32_t cap;  // slots per bin (fixed-capacity source)
    uint64_t magic, nonce;  // the workspace header the atoms' record expects
};

constexpr int kWaves = kThreads / 64;

// r2 as the case-study notes' section 18.5 listing forms it for its cutoff
// test: dx*dx + dy*dy + dz*dz in fp32, left to right, every product and sum
// rounded on its own.  Contraction into fused multiply-adds is switched off
// here so that the inclusion decision is the listing's, bit for bit.
__device__ __forceinline__ float listing_r2(float dx, float dy, float dz)
{
#pragma clang fp contract(off)
    const float xx = dx * dx;
    const float yy = dy * dy;
    const float zz = dz * dz;
    return (xx + yy) + zz;
}

// One staged atom against this lane's kNx nodes.  kSmoothClamp clamps r^2 to
// P.rc2, for which the kernel has checked that the fp32 smoothed term is
// exactly 0 (so atoms beyond the cutoff add exactly nothing); kSmoothSelect
// and kTruncated replace the charge by 0 outside the cutoff, kTruncated with
// the listing's r2.
template <int MODE>
__device__ __forceinline__ void add_atom(const float4 at, const float (&x)[kNx], float y, float z,
                                         const CutoffParams &P, float (&acc)[kNx])
{
    const float dy = y - at.y;
    const float dz = z - at.z;
    const float yz2 = fmaf(dy, dy, dz * dz);
#pragma unroll
    for (int c = 0; c < kNx; ++c) {
        const float dx = x[c] - at.x;
        if constexpr (MODE == kSmoothClamp) {
            const float r2 = fminf(fmaf(dx, dx, yz2), P.rc2);
            const float rs = __builtin_amdgcn_rsqf(r2);
            const float g = fmaf(fmaf(r2, P.gc2, P.gc1), r2, P.gc0);
            acc[c] = fmaf(at.w, rs - g, acc[c]);
        } else if constexpr (MODE == kSmoothSelect) {
            const float r2 = fmaf(dx, dx, yz2);
            const float rs = __builtin_amdgcn_rsqf(r2);
            const float g = fmaf(fmaf(r2, P.gc2, P.gc1), r2, P.gc0);
            const float qm = r2 < P.rc2 ? at.w : 0.0f;
            acc[c] = fmaf(qm, rs - g, acc[c]);
        } else if constexpr (MODE == kRsqInside) {
            acc[c] = fmaf(at.w, __builtin_amdgcn_rsqf(fmaf(dx, dx, yz2)), acc[c]);
        } else {
            const float r2 = listing_r2(dx, dy, dz);
            const float qm = r2 < P.rc2 ? at.w : 0.0f;
            acc[c] = fmaf(qm, __builtin_amdgcn_rsqf(r2), acc[c]);
        }
    }
}

// The same fp32 term as add_atom evaluates, at r^2 = r2.
__device__ __forceinline__ float term_at(float r2, const CutoffParams &P)
{
    return __builtin_amdgcn_rsqf(r2) - fmaf(fmaf(r2, P.gc2, P.gc1), r2, P.gc0);
}

// Largest r^2 <= rc^2 (within kClampSearch ulps) at which the fp32 term is
// exactly 0, or 0 if there is none.  The term vanishes to third order at rc,
// so it is a few ulps of 1/rc around rc^2 and some nearby r^2 rounds it to 0;
// atoms between that r^2 and rc^2 contribute O((ulp/rc)^3) in exact
// arithmetic, far below fp32 resolution.
constexpr int kClampSearch = 64;

// Every lane of the wave tests one candidate (lane k: k ulps below rc^2)
// and the wave takes the first zero, so the search is one step.  Called with
// the whole wave active.
__device__ inline float exact_zero_clamp(const CutoffParams &P)
{
    static_assert(kClampSearch == 64, "one candidate per lane of a wave");
    const uint32_t k = __lane_id();
    const float r2 = __uint_as_float(__float_as_uint(P.rc2) - k);
    const uint64_t zeros = __ballot(term_at(r2, P) == 0.0f);
    if (zeros == 0)
        return 0.0f;
    return __uint_as_float(__float_as_uint(P.rc2) - (uint32_t)(__ffsll((long long)zeros) - 1));
}

// Charge-weighted moments of a set of atoms about a centre c, with a = atom -
// c, s = |a|^2: Q = sum q, m1 = sum q a, s2 = sum q s, m2 = sum q a a^T (xx,
// yy, zz, xy, xz, yz), m3 = sum q s a, s4 = sum q s^2.  For every node x
// (relative to c) the smoothed term's polynomial part over the set is the
// exact expansion of sum q (GC0 + GC1 r^2 + GC2 r^4), r^2 = |x|^2 - 2 x.a + s:
//   sum q r^2 = Q |x|^2 - 2 x.m1 + s2,
//   sum q r^4 = Q |x|^4 + s4 + 4 x^T m2 x + 2 |x|^2 s2 - 4 |x|^2 x.m1 - 4 x.m3.
struct Moments {
    float q, m1[3], s2, m2[6], m3[3], s4;
};

__device__ __forceinline__ void moments_zero(Moments &M)
{
    M.q = M.s2 = M.s4 = 0.0f;
#pragma unroll
    for (int i = 0; i < 3; ++i)
        M.m1[i] = M.m3[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 6; ++i)
        M.m2[i] = 0.0f;
}

__device__ __forceinline__ void moments_add(Moments &M, const float4 at, const float (&c)[3])
{
    const float ax = at.x - c[0], ay = at.y - c[1], az = at.z - c[2];
    const float s = fmaf(ax, ax, fmaf(ay, ay, az * az));
    const float qx = at.w * ax, qy = at.w * ay, qz = at.w * az, qs = at.w * s;
    M.q += at.w;
    M.m1[0] += qx;
    M.m1[1] += qy;
    M.m1[2] += qz;
    M.s2 += qs;
    M.m2[0] = fmaf(qx, ax, M.m2[0]);
    M.m2[1] = fmaf(qy, ay, M.m2[1]);
    M.m2[2] = fmaf(qz, az, M.m2[2]);
    M.m2[3] = fmaf(qx, ay, M.m2[3]);
    M.m2[4] = fmaf(qx, az, M.m2[4]);
    M.m2[5] = fmaf(qy, az, M.m2[5]);
    M.m3[0] = fmaf(qs, ax, M.m3[0]);
    M.m3[1] = fmaf(qs, ay, M.m3[1]);
    M.m3[2] = fmaf(qs, az, M.m3[2]);
    M.s4 = fmaf(qs, s, M.s4);
}

// Sum over a cube's kGroupLanes lanes by an xor butterfly: both partners of
// a step add the same two values, so every lane ends with the same total.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = kGroupLanes / 2; m >= 1; m >>= 1)
        v += __shfl_xor(v, m);
    return v;
}

// Number of lanes below this one whose bit is set in mask.
__device__ __forceinline__ int32_t lanes_below(uint64_t mask)
{
    return (int32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ void moments_reduce(Moments &M)
{
    M.q = wave_sum(M.q);
    M.s2 = wave_sum(M.s2);
    M.s4 = wave_sum(M.s4);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        M.m1[i] = wave_sum(M.m1[i]);
        M.m3[i] = wave_sum(M.m3[i]);
    }
#pragma unroll
    for (int i = 0; i < 6; ++i)
        M.m2[i] = wave_sum(M.m2[i]);
}

// sum q (GC0 + GC1 r^2 + GC2 r^4) over the moments' atoms at node x (relative
// to their centre).
__device__ __forceinline__ float moments_poly(const Moments &M, float x, float y, float z,
                                              const CutoffParams &P)
{
    const float xx = fmaf(x, x, fmaf(y, y, z * z));
    const float xm1 = fmaf(x, M.m1[0], fmaf(y, M.m1[1], z * M.m1[2]));
    const float xm3 = fmaf(x, M.m3[0], fmaf(y, M.m3[1], z * M.m3[2]));
    const float diag = fmaf(M.m2[0] * x, x, fmaf(M.m2[1] * y, y, M.m2[2] * z * z));
    const float off = fmaf(M.m2[3] * x, y, fmaf(M.m2[4] * x, z, M.m2[5] * y * z));
    const float xm2x = fmaf(2.0f, off, diag);
    const float p2 = fmaf(M.q, xx, fmaf(-2.0f, xm1, M.s2));
    const float p4 = fmaf(M.q * xx, xx, M.s4) + 4.0f * xm2x + 2.0f * xx * M.s2 -
                     4.0f * xx * xm1 - 4.0f * xm3;
    return fmaf(P.gc2, p4, fmaf(P.gc1, p2, P.gc0 * M.q));
}

// The staged atom at byte offset off of the stage array.
__device__ __forceinline__ float4 staged(const float4 *stage, uint32_t off)
{
    return *reinterpret_cast<const float4 *>(reinterpret_cast<const char *>(stage) + off);
}

// Adds the staged atoms at byte offsets list[0], list[STEP], ...,
// list[STEP * (listed - 1)].
template <int MODE, int STEP>
__device__ __forceinline__ void sweep(const float4 *stage, const uint32_t *list, int32_t listed,
                                      const float (&x)[kNx], float y, float z,
                                      const CutoffParams &P, float (&acc)[kNx])
{
    int32_t i = 0;
    for (; i + 4 <= listed; i += 4) {
        const float4 a0 = staged(stage, list[STEP * (i + 0)]);
        const float4 a1 = staged(stage, list[STEP * (i + 1)]);
        const float4 a2 = staged(stage, list[STEP * (i + 2)]);
        const float4 a3 = staged(stage, list[STEP * (i + 3)]);
        add_atom<MODE>(a0, x, y, z, P, acc);
        add_atom<MODE>(a1, x, y, z, P, acc);
        add_atom<MODE>(a2, x, y, z, P, acc);
        add_atom<MODE>(a3, x, y, z, P, acc);
    }
    for (; i < listed; ++i)
        add_atom<MODE>(staged(stage, list[STEP * i]), x, y, z, P, acc);
}

// SLOTS = false: the atoms are a CSR (bin_start, sorted); SLOTS = true: they
// are fixed-capacity bins, bin b's slots at sorted[b * cap ...], and
// bin_start is not read.  ACCUM = true adds the sum into V.
// Store of this thread's kNx nodes of the tile (x-fastest rows of V); the
// indices are recomputed here rather than kept through the sweep (the empty
// asm keeps the compiler from reusing the early ones).
template <bool ACCUM>
__device__ __forceinline__ void store_nodes(const CutoffParams &P, int32_t tx, int32_t ty,
                                            int32_t tz, const float (&v)[kNx],
                                            float *__restrict__ V)
{
    int32_t te = threadIdx.x;
    asm volatile("" : "+v"(te));
    const int32_t qs = (te % 64) / kGroupLanes, ls = te % kGroupLanes;
    const int32_t i0s = tx * kTile + (qs & 1) * kCube;
    const int32_t js = ty * kTile + (qs >> 1) * kCube + ls % kCube;
    const int32_t ks = tz * kTile + (te / 64) * kCube + ls / kCube;
    if (js >= P.n[1] || ks >= P.n[2])
        return;
    float *out = V + ((int64_t)ks * P.n[1] + js) * P.n[0];
#pragma unroll
    for (int c = 0; c < kNx; ++c) {
        if (i0s + c < P.n[0]) {
            if constexpr (ACCUM)
                out[i0s + c] += v[c];
            else
                out[i0s + c] = v[c];
        }
    }
}

template <bool SLOTS, bool ACCUM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd))) void
cutoff_kernel(CutoffParams P0, const WorkspaceHeader *__restrict__ hdr,
              const int32_t *__restrict__ bin_start, const float4 *__restrict__ sorted,
              int32_t n_sorted, float *__restrict__ V)
{
    __shared__ float4 stage[kStage];
    __shared__ uint32_t cube_list[kWaves][kGroups][kStage];  // byte offsets into stage
    __shared__ int32_t span_src[kMaxRows];
    __shared__ int32_t span_off[kMaxRows + 1];
    __shared__ int32_t wave_total[kWaves];

    // Smoothed term: clamp r^2 where a clamp value with an exactly-zero term
    // exists, else select.  Truncated term: select.
    CutoffParams P = P0;
    int mode = kTruncated;
    if (!P0.truncated) {
        const float clamp = __uint_as_float(
            __builtin_amdgcn_readfirstlane(__float_as_uint(exact_zero_clamp(P0))));
        mode = clamp > 0.0f ? kSmoothClamp : kSmoothSelect;
        if (mode == kSmoothClamp)
            P.rc2 = clamp;
    }

    const int t = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(t / 64);
    const int lane = t % 64;
    const int32_t tile = blockIdx.x;
    const int32_t tx = tile % P.tiles[0];
    const int32_t ty = (tile / P.tiles[0]) % P.tiles[1];
    const int32_t tz = tile / (P.tiles[0] * P.tiles[1]);
    // A workspace whose header no longer carries the fill its record names
    // (its memory was reused and overwritten since) is not read: every node
    // becomes NaN.
    if (hdr->magic != P0.magic || hdr->nonce != P0.nonce) {
        const float nan = __builtin_nanf("");
        const float v[kNx] = {nan, nan, nan, nan};
        store_nodes<false>(P0, tx, ty, tz, v, V);
        return;
    }
    // The tile's geometry is the same for every thread: computed once and
    // kept in LDS, so its doubles do not occupy registers through the sweep.
    __shared__ TileRows T;
    if (t == 0)
        T = tile_rows(tx, ty, tz, P.n, P.h, P.o, P.b0, P.nb, P.bs, P.list_rc);
    __syncthreads();

    // This lane's nodes: an x-run of kNx nodes.  Wave w covers the tile's
    // z-half w (8 x 8 x 4 nodes) as four 4 x 4 x 4-node cubes, 16 lanes each:
    // cube q of the wave takes x-half q & 1 and y-half q >> 1, and its lanes
    // the cube's 4 x 4 (y, z) rows.  Each cube keeps its own atom list.
    const int q = lane / kGroupLanes;
    const int ql = lane % kGroupLanes;
    const int32_t i0 = tx * kTile + (q & 1) * kCube;
    const int32_t j = ty * kTile + (q >> 1) * kCube + ql % kCube;
    const int32_t k = tz * kTile + wave * kCube + ql / kCube;
    float x[kNx];
#pragma unroll
    for (int c = 0; c < kNx; ++c)
        x[c] = node_coord(i0 + c, P.h, P.o[0]);
    const float y = node_coord(j, P.h, P.o[1]);
    const float z = node_coord(k, P.h, P.o[2]);
    // atoms inside the cutoff of the whole cube and boundary atoms are summed
    // apart (each in staged order), so the order does not depend on chunking
    float acc_in[kNx], acc_bd[kNx];
#pragma unroll
    for (int c = 0; c < kNx; ++c) {
        acc_in[c] = 0.0f;
        acc_bd[c] = 0.0f;
    }
    // the smoothed term's polynomial part over the cube's inside atoms, from
    // their moments about the wave's centre: lane l of the cube accumulates
    // the cube's inside atoms number l, l + 16, ... (counted in staged order
    // over all chunks)
    Moments mom;
    moments_zero(mom);
    int32_t inside_seen = 0;

    // The cubes' node boxes (nodes past the lattice edge included: they are
    // computed and dropped, so a box only needs to contain the live ones).
    // Both x-halves, both y-halves and the wave's z-range; the same for the
    // whole wave.
    const int64_t nx0 = (int64_t)tx * kTile, ny0 = (int64_t)ty * kTile;
    const int64_t nz0 = (int64_t)tz * kTile + wave * kCube;
    const float cxlo[2] = {node_coord(nx0, P.h, P.o[0]), node_coord(nx0 + kCube, P.h, P.o[0])};
    const float cxhi[2] = {node_coord(nx0 + kCube - 1, P.h, P.o[0]),
                           node_coord(nx0 + kTile - 1, P.h, P.o[0])};
    const float cylo[2] = {node_coord(ny0, P.h, P.o[1]), node_coord(ny0 + kCube, P.h, P.o[1])};
    const float cyhi[2] = {node_coord(ny0 + kCube - 1, P.h, P.o[1]),
                           node_coord(ny0 + kTile - 1, P.h, P.o[1])};
    const float czlo = node_coord(nz0, P.h, P.o[2]);
    const float czhi = node_coord(nz0 + kCube - 1, P.h, P.o[2]);
    // a slightly widened radius keeps the lists conservative against
    // rounding; a slightly narrowed one keeps "inside" safely inside (r^2
    // below the clamp value or rc^2 at every node of the cube)
    const float keep2 = P0.rc2 * 1.0001f;
    const float inside2 = P.rc2 * 0.9999f;
    const float centre[3] = {0.5f * (cxlo[0] + cxhi[1]), 0.5f * (cylo[0] + cyhi[1]),
                             0.5f * (czlo + czhi)};
    bool any_atoms = false;

    for (int32_t row0 = 0; row0 < T.nrows; row0 += kMaxRows) {
        const int32_t rows = T.nrows - row0 < kMaxRows ? T.nrows - row0 : kMaxRows;
        // 1. size the spans: thread t takes a contiguous block of rows
        const int32_t per = (rows + kThreads - 1) / kThreads;
        const int32_t r_lo = t * per < rows ? t * per : rows;
        const int32_t r_hi = r_lo + per < rows ? r_lo + per : rows;
        int32_t local = 0;
        for (int32_t r = r_lo; r < r_hi; ++r) {
            int32_t cy, cz, cx0, cx1, cnt = 0, src = 0;
            if (tile_row(T, row0 + r, &cy, &cz, &cx0, &cx1)) {
                const int64_t base = ((int64_t)cz * P.nb[1] + cy) * P.nb[0];
                if constexpr (SLOTS) {
                    src = (int32_t)((base + cx0) * P.cap);
                    cnt = (cx1 - cx0 + 1) * P.cap;
                } else {
                    int32_t s = bin_start[base + cx0];
                    int32_t e = bin_start[base + cx1 + 1];
                    s = s < 0 ? 0 : (s > n_sorted ? n_sorted : s);
                    e = e < s ? s : (e > n_sorted ? n_sorted : e);
                    src = s;
                    cnt = e - s;
                }
            }
            span_src[r] = src;
            span_off[r] = cnt;
            local += cnt;
        }
        // 2. exclusive offsets of the spans in row order: a scan inside each
        //    wave, then the waves' totals through LDS
        // (the lane id goes through an empty asm so that the shuffle
        // addresses are formed here, not kept in registers through the sweep)
        int32_t lid = lane;
        asm volatile("" : "+v"(lid));
        int32_t incl = local;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t v = __builtin_amdgcn_ds_bpermute((lid - off) << 2, incl);
            if (lid >= off)
                incl += v;
        }
        if (lane == 63)
            wave_total[wave] = incl;
        __syncthreads();
        int32_t run = incl - local;
        int32_t sum = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int32_t wt = wave_total[w];
            run += w < wave ? wt : 0;
            sum += wt;
        }
        for (int32_t r = r_lo; r < r_hi; ++r) {
            const int32_t c = span_off[r];
            span_off[r] = run;
            run += c;
        }
        const int32_t total = __builtin_amdgcn_readfirstlane(sum);
        if (t == 0)
            span_off[rows] = total;
        any_atoms |= total > 0;
        __syncthreads();

        // 3. stage the spans' atoms in chunks; each cube lists the atoms near
        //    its nodes and its lanes sweep them
        // (64-bit chunk start: a neighbourhood can hold up to 2^31 - 1 atoms,
        // and the step past the last chunk must not wrap)
        for (int64_t c0 = 0; c0 < total; c0 += kStage) {
            const int32_t m = total - c0 < kStage ? (int32_t)(total - c0) : kStage;
            for (int32_t e = t; e < m; e += kThreads) {
                const int32_t g = (int32_t)(c0 + e);
                int32_t a = 0, b = rows;  // last row with span_off[row] <= g
                while (b - a > 1) {
                    const int32_t mid = (a + b) >> 1;
                    if (span_off[mid] <= g)
                        a = mid;
                    else
                        b = mid;
                }
                stage[e] = sorted[span_src[a] + (g - span_off[a])];
            }
            __syncthreads();
            // each cube's list: inside atoms from the front, boundary atoms
            // from the back; together at most m <= kStage entries
            int32_t n_in[kGroups], n_bd[kGroups];
#pragma unroll
            for (int g = 0; g < kGroups; ++g)
                n_in[g] = n_bd[g] = 0;
            for (int32_t e0 = 0; e0 < m; e0 += 64) {
                const int32_t e = e0 + lane;
                bool near[kGroups], inside[kGroups];
#pragma unroll
                for (int g = 0; g < kGroups; ++g)
                    near[g] = inside[g] = false;
                if (e < m) {
                    const float4 at = stage[e];
                    // per axis and half: squared gap to the box (0 inside
                    // it) and squared distance to its far face
                    float gx[2], fx[2], gy[2], fy[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const float lx = cxlo[hh] - at.x, ux = at.x - cxhi[hh];
                        const float ly = cylo[hh] - at.y, uy = at.y - cyhi[hh];
                        const float ax = fmaxf(fmaxf(lx, ux), 0.0f), bx = fmaxf(-lx, -ux);
                        const float ay = fmaxf(fmaxf(ly, uy), 0.0f), by = fmaxf(-ly, -uy);
                        gx[hh] = ax * ax;
                        fx[hh] = bx * bx;
                        gy[hh] = ay;
                        fy[hh] = by;
                    }
                    const float lz = czlo - at.z, uz = at.z - czhi;
                    const float az = fmaxf(fmaxf(lz, uz), 0.0f), bz = fmaxf(-lz, -uz);
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const float gyz = fmaf(gy[hh], gy[hh], az * az);
                        const float fyz = fmaf(fy[hh], fy[hh], bz * bz);
#pragma unroll
                        for (int xh = 0; xh < 2; ++xh) {
                            const int g = 2 * hh + xh;
                            near[g] = gx[xh] + gyz < keep2;
                            inside[g] = near[g] && fx[xh] + fyz < inside2;
                        }
                    }
                }
#pragma unroll
                for (int g = 0; g < kGroups; ++g) {
                    const uint64_t v_in = __ballot(inside[g]);
                    const uint64_t v_bd = __ballot(near[g] && !inside[g]);
                    if ((v_in | v_bd) == 0)
                        continue;
                    uint32_t *list = cube_list[wave][g];
                    if (inside[g])
                        list[n_in[g] + lanes_below(v_in)] = (uint32_t)e * 16u;
                    else if (near[g])
                        list[kStage - 1 - (n_bd[g] + lanes_below(v_bd))] = (uint32_t)e * 16u;
                    n_in[g] += __popcll(v_in);
                    n_bd[g] += __popcll(v_bd);
                }
            }
            // the lists are written and read by this wave only
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // every lane sweeps its cube's list; the lists' common length
            // without masks, the rest with the lanes whose list is longer
            int32_t my_in = n_in[0], my_bd = n_bd[0];
            int32_t min_in = n_in[0], min_bd = n_bd[0];
#pragma unroll
            for (int g = 1; g < kGroups; ++g) {
                my_in = q == g ? n_in[g] : my_in;
                my_bd = q == g ? n_bd[g] : my_bd;
                min_in = n_in[g] < min_in ? n_in[g] : min_in;
                min_bd = n_bd[g] < min_bd ? n_bd[g] : min_bd;
            }
            const uint32_t *front = cube_list[wave][q];
            const uint32_t *back = front + (kStage - 1);
            sweep<kRsqInside, 1>(stage, front, min_in, x, y, z, P, acc_in);
            for (int32_t i = min_in; i < my_in; ++i)
                add_atom<kRsqInside>(staged(stage, front[i]), x, y, z, P, acc_in);
            if (mode == kTruncated) {
                sweep<kTruncated, -1>(stage, back, min_bd, x, y, z, P, acc_bd);
                for (int32_t i = min_bd; i < my_bd; ++i)
                    add_atom<kTruncated>(staged(stage, back[-i]), x, y, z, P, acc_bd);
            } else {
                for (int32_t i = (ql - inside_seen) & (kGroupLanes - 1); i < my_in;
                     i += kGroupLanes)
                    moments_add(mom, staged(stage, front[i]), centre);
                inside_seen += my_in;
                if (mode == kSmoothClamp) {
                    sweep<kSmoothClamp, -1>(stage, back, min_bd, x, y, z, P, acc_bd);
                    for (int32_t i = min_bd; i < my_bd; ++i)
                        add_atom<kSmoothClamp>(staged(stage, back[-i]), x, y, z, P, acc_bd);
                } else {
                    sweep<kSmoothSelect, -1>(stage, back, min_bd, x, y, z, P, acc_bd);
                    for (int32_t i = min_bd; i < my_bd; ++i)
                        add_atom<kSmoothSelect>(staged(stage, back[-i]), x, y, z, P, acc_bd);
                }
            }
            __syncthreads();
        }
    }

    if (mode != kTruncated) {
        // every lane of the wave takes part in the reduction
        moments_reduce(mom);
#pragma unroll
        for (int c = 0; c < kNx; ++c)
            acc_in[c] -= moments_poly(mom, x[c] - centre[0], y - centre[1], z - centre[2], P);
    }

    float v[kNx];
#pragma unroll
    for (int c = 0; c < kNx; ++c)
        v[c] = acc_in[c] + acc_bd[c];
    // overflow pass: nothing within reach of this tile, its nodes keep their value
    if (ACCUM && !any_atoms)
        return;
    store_nodes<ACCUM>(P, tx, ty, tz, v, V);
}

int32_t ceil_div32(int32_t a, int32_t b) { return (a + b - 1) / b; }

// Radius of the bin neighbourhood a tile walks.  Two roundings can put an atom
// outside its bin's box: its bin coordinate fl(fl(p - b0) / bs) is off by at
// most 2^-23 |p - b0| per axis, and |p - b0| < nb bs for a kept atom, so the
// box is widened by slack = 2^-21 max(nb bs) (>= sqrt(3) 2^-23 max(nb bs) with
// room for the double geometry).  The truncated term's fp32 test can also
// keep an atom whose exact distance exceeds rc by an ulp or two: a relative
// 2^-16 covers that.  The smoothed term vanishes to third order at rc, so an
// atom within `slack` of the cutoff adds at most 2.5 (slack/rc)^3 |q|/rc; the
// slack is applied to it only where that bound could exceed 2^-30 |q|/rc
// (slack > rc/1024, lattices some 10^4 cutoffs long), which keeps exact-tie
// bins out of ordinary neighbourhoods.
float neighbourhood_radius(const BinGeometry &g, int32_t term)
{
    double extent = 0.0;
    for (int a = 0; a < 3; ++a)
        extent = std::fmax(extent, (double)g.ax[a].nb * (double)g.bin_size);
    const double rc = g.cutoff;
    const double slack = std::ldexp(extent, -21);
    double r = rc;
    if (term == CPMAP_TERM_TRUNCATED)
        r = rc * (1.0 + 1.0 / 65536.0) + slack;
    else if (slack > rc / 1024.0)
        r = rc + slack;
    // round up so that the fp32 radius never falls below r
    float f = (float)r;
    if ((double)f < r)
        f = std::nextafter(f, INFINITY);
    return f;
}


CutoffParams make_params(const Lattice &lat, const BinGeometry &g, int32_t term, int32_t cap,
                         uint64_t magic, uint64_t nonce)
{
    CutoffParams P;
    P.magic = magic;
    P.nonce = nonce;
    P.truncated = term == CPMAP_TERM_TRUNCATED;
    P.h = lat.h;
    for (int a = 0; a < 3; ++a) {
        P.o[a] = lat.o[a];
        P.n[a] = lat.n[a];
        P.tiles[a] = ceil_div32(lat.n[a], kTile);
        P.b0[a] = g.ax[a].b0;
        P.nb[a] = g.ax[a].nb;
    }
    const double rc = g.cutoff;
    P.bs = g.bin_size;
    P.rc = g.cutoff;
    P.rc2 = g.cutoff * g.cutoff;
    P.list_rc = neighbourhood_radius(g, term);
    P.gc0 = (float)(15.0 / (8.0 * rc));
    P.gc1 = (float)(-5.0 / (4.0 * rc * rc * rc));
    P.gc2 = (float)(3.0 / (8.0 * rc * rc * rc * rc * rc));
    P.cap = cap;
    return P;
}

int64_t tile_count(const CutoffParams &P)
{
    return (int64_t)P.tiles[0] * P.tiles[1] * P.tiles[2];
}

}  // namespace

hipError_t launch_cutoff(const void *workspace, const BinLayout &L, int64_t n_atoms,
                         const Lattice &lat, const BinGeometry &g, int32_t term, uint64_t nonce,
                         float *V, hipStream_t stream)
{
    const CutoffParams P = make_params(lat, g, term, 0, kBinMagic, nonce);
    const int64_t tiles = tile_count(P);
    if (tiles == 0)
        return hipSuccess;
    if (tiles > INT32_MAX)
        return hipErrorInvalidValue;
    const char *ws = static_cast<const char *>(workspace);
    const WorkspaceHeader *hdr = reinterpret_cast<const WorkspaceHeader *>(ws + L.header);
    const int32_t *bin_start = reinterpret_cast<const int32_t *>(ws + L.bin_start);
    const float4 *sorted = reinterpret_cast<const float4 *>(ws + L.sorted);
    hipLaunchKernelGGL((cutoff_kernel<false, false>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, P, hdr, bin_start, sorted, (int32_t)n_atoms, V);
    return hipGetLastError();
}

hipError_t launch_cutoff_slots(const void *slot_workspace, const SlotLayout &S, int64_t n_atoms,
                               const Lattice &lat, const BinGeometry &g, int32_t cap,
                               int32_t term, uint64_t nonce, float *V, hipStream_t stream)
{
    const CutoffParams Pslots = make_params(lat, g, term, cap, kSlotMagic, nonce);
    const CutoffParams Pover = make_params(lat, g, term, 0, kSlotMagic, nonce);
    const int64_t tiles = tile_count(Pslots);
    if (tiles == 0)
        return hipSuccess;
    if (tiles > INT32_MAX)
        return hipErrorInvalidValue;
    const char *ws = static_cast<const char *>(slot_workspace);
    const WorkspaceHeader *hdr = reinterpret_cast<const WorkspaceHeader *>(ws + S.header);
    const float4 *slots = reinterpret_cast<const float4 *>(ws + S.slots);
    const int32_t *over_start = reinterpret_cast<const int32_t *>(ws + S.over_start);
    const float4 *over_atoms = reinterpret_cast<const float4 *>(ws + S.over_atoms);
    const int64_t n_slots = g.nbins() * cap;
    hipLaunchKernelGGL((cutoff_kernel<true, false>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, Pslots, hdr, nullptr, slots, (int32_t)n_slots, V);
    hipLaunchKernelGGL((cutoff_kernel<false, true>), dim3((unsigned)tiles), dim3(kThreads), 0,
                       stream, Pover, hdr, over_start, over_atoms, (int32_t)n_atoms, V);
    return hipGetLastError();
}

}  // namespace cpmap

extern "C" int64_t cpmap_neighbor_spans(int32_t nx, int32_t ny, int32_t nz, float spacing,
                                        float ox, float oy, float oz, float bin_size,
                                        float cutoff, int32_t term, int32_t tx, int32_t ty,
                                        int32_t tz, int32_t *spans_out, int64_t max_spans)
{
    using namespace cpmap;
    BinGeometry g;
    if (make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g) != CPMAP_OK)
        return -1;
    if (term != CPMAP_TERM_SMOOTHED && term != CPMAP_TERM_TRUNCATED)
        return -1;
    const int32_t n[3] = {nx, ny, nz};
    const int32_t t[3] = {tx, ty, tz};
    for (int a = 0; a < 3; ++a)
        if (t[a] < 0 || t[a] >= (n[a] + kTile - 1) / kTile)
            return -1;
    if (max_spans < 0 || (max_spans > 0 && spans_out == nullptr))
        return -1;
    const float o[3] = {ox, oy, oz};
    const float b0[3] = {g.ax[0].b0, g.ax[1].b0, g.ax[2].b0};
    const int32_t nb[3] = {g.ax[0].nb, g.ax[1].nb, g.ax[2].nb};
    const TileRows T =
        tile_rows(tx, ty, tz, n, spacing, o, b0, nb, bin_size, neighbourhood_radius(g, term));
    int64_t count = 0;
    for (int32_t r = 0; r < T.nrows; ++r) {
        int32_t cy, cz, cx0, cx1;
        if (!tile_row(T, r, &cy, &cz, &cx0, &cx1))
            continue;
        if (count < max_spans) {
            spans_out[4 * count + 0] = cy;
            spans_out[4 * count + 1] = cz;
            spans_out[4 * count + 2] = cx0;
            spans_out[4 * count + 3] = cx1;
        }
        ++count;
    }
    return count;
}
