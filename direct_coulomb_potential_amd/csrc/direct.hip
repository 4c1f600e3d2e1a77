// Direct Coulomb summation on gfx950: V(g) = sum_a q_a / |g - a| for every
// lattice node g (the PMPP chapter-18 notes, section 18.1), computed as a
// gather: every node is owned by one lane and written once, with no atomics
// (same notes, section 18.2).
//
// Mapping (MI355X-first; the notes' constant-memory chunks and 4-wide
// coarsening were designed for another GPU and are not used):
//  - each lane owns a CX x CY x CZ block of nodes (x, y, z register blocking).
//    Per atom it forms dx for its CX columns, dy for its CY rows, dz^2 for its
//    CZ planes and e = dy^2 + dz^2 for its CY*CZ rows; every node then costs
//    one fma (r^2 = dx^2 + e), one v_rsq_f32 and one fma (v += q * rsq).  On
//    gfx950 v_rsq_f32 issues at half rate and does not overlap other VALU
//    work, so a node-atom pair costs 4 issue slots plus the shared work
//    (CX + CY + 2 CZ + CY*CZ) / (CX*CY*CZ) slots; the notes' coarsening
//    (section 18.3: dy, dz reused across x neighbours) is the 1D case.
//  - atoms are read wave-uniformly, four at a time, by scalar loads (one
//    s_load_dwordx16), so atom data never occupies vector registers or LDS.
//  - the W waves of a workgroup own the same 64 lanes' nodes and split the
//    atom list into W contiguous slices.  Each wave sums at most kChunk atoms
//    in registers, then the waves add their partial sums, in wave order, into
//    a running total kept in LDS.  The short register sums bound fp32
//    rounding growth for large same-sign atom sets, the fixed order keeps the
//    result deterministic, and W fills the 1024 SIMDs for small lattices.
//  - nodes are stored x-fastest, V[(k*ny + j)*nx + i] (section 18.4) from the
//    LDS total; lanes adjacent in x write adjacent 4*CX-byte runs.
#include <algorithm>
#include <atomic>
#include <cmath>

#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kWave = 64;
constexpr int64_t kChunk = 16384;

template <int CX, int CY, int CZ>
__device__ __forceinline__ void accumulate_atom(const float4 a, const float (&x)[CX],
                                                const float (&y)[CY], const float (&z)[CZ],
                                                float (&acc)[CX * CY * CZ])
{
    float dx[CX];
#pragma unroll
    for (int c = 0; c < CX; ++c)
        dx[c] = x[c] - a.x;
    float dy[CY];
#pragma unroll
    for (int d = 0; d < CY; ++d)
        dy[d] = y[d] - a.y;
#pragma unroll
    for (int e = 0; e < CZ; ++e) {
        const float dz = z[e] - a.z;
        const float dz2 = dz * dz;
#pragma unroll
        for (int d = 0; d < CY; ++d) {
            const float yz2 = fmaf(dy[d], dy[d], dz2);
#pragma unroll
            for (int c = 0; c < CX; ++c) {
                float &v = acc[(e * CY + d) * CX + c];
                v = fmaf(a.w, __builtin_amdgcn_rsqf(fmaf(dx[c], dx[c], yz2)), v);
            }
        }
    }
}

template <int CX, int CY, int CZ, int W>
__global__ __launch_bounds__(kWave *W) void direct_kernel(
    const float4 *__restrict__ atoms, int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
    int32_t nsx, int32_t nsy, int64_t n_strips, float h, float ox, float oy, float oz,
    float *__restrict__ V)
{
    constexpr int NP = CX * CY * CZ;
    __shared__ float total[NP * kWave];

    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;

    // Lane -> block of nodes.  Lanes past the last block recompute the last
    // block (they still take part in the reduction) and store nothing.
    const int64_t s_raw = (int64_t)blockIdx.x * kWave + lane;
    const bool live = s_raw < n_strips;
    const int64_t s = live ? s_raw : n_strips - 1;
    const int32_t sx = (int32_t)(s % nsx);
    const int64_t t = s / nsx;
    const int32_t sy = (int32_t)(t % nsy);
    const int32_t sz = (int32_t)(t / nsy);
    const int32_t i0 = sx * CX, j0 = sy * CY, k0 = sz * CZ;

    float x[CX], y[CY], z[CZ];
#pragma unroll
    for (int c = 0; c < CX; ++c)
        x[c] = node_coord(i0 + c, h, ox);
#pragma unroll
    for (int d = 0; d < CY; ++d)
        y[d] = node_coord(j0 + d, h, oy);
#pragma unroll
    for (int e = 0; e < CZ; ++e)
        z[e] = node_coord(k0 + e, h, oz);

    if (slice == 0) {
#pragma unroll
        for (int p = 0; p < NP; ++p)
            total[p * kWave + lane] = 0.0f;
    }

    // This wave's contiguous slice of the atoms, processed in rounds of at
    // most kChunk atoms; every wave runs the same number of rounds.
    const int64_t a_begin = n_atoms * slice / W;
    const int64_t a_end = n_atoms * (slice + 1) / W;
    const int64_t max_len = (n_atoms + W - 1) / W;
    const int64_t rounds = (max_len + kChunk - 1) / kChunk;

    for (int64_t r = 0; r < rounds; ++r) {
        float acc[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p)
            acc[p] = 0.0f;
        const int64_t lo = a_begin + r * kChunk;
        const int64_t hi = lo + kChunk < a_end ? lo + kChunk : a_end;
        int64_t a = lo;
        for (; a + 4 <= hi; a += 4) {
            const float4 t0 = atoms[a + 0];
            const float4 t1 = atoms[a + 1];
            const float4 t2 = atoms[a + 2];
            const float4 t3 = atoms[a + 3];
            accumulate_atom<CX, CY, CZ>(t0, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t1, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t2, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t3, x, y, z, acc);
        }
        for (; a < hi; ++a)
            accumulate_atom<CX, CY, CZ>(atoms[a], x, y, z, acc);
        // Add the round's partial sums into the LDS total in wave order.
        for (int w = 0; w < W; ++w) {
            __syncthreads();
            if (slice == w) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    total[p * kWave + lane] += acc[p];
            }
        }
    }
    __syncthreads();
    if (!live)
        return;

    // x-fastest store from the LDS total; the waves share the rows.  Columns
    // past nx, rows past ny and planes past nz are dropped.
    for (int row = slice; row < CY * CZ; row += W) {
        const int32_t j = j0 + row % CY;
        const int32_t k = k0 + row / CY;
        if (j >= ny || k >= nz)
            continue;
        float *out = V + ((int64_t)k * ny + j) * nx;
        const float *src = total + row * CX * kWave + lane;
#pragma unroll
        for (int c = 0; c < CX; ++c)
            if (i0 + c < nx)
                out[i0 + c] = src[c * kWave];
    }
}

__global__ void fill_zero(float *__restrict__ V, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        V[i] = 0.0f;
}

using KernelFn = void (*)(const float4 *, int64_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                          int64_t, float, float, float, float, float *);

struct Variant {
    int cx, cy, cz, w;
    KernelFn kernel;
};

#define CPMAP_VARIANT(CX, CY, CZ, W) Variant{CX, CY, CZ, W, direct_kernel<CX, CY, CZ, W>}

const Variant kVariants[] = {
    CPMAP_VARIANT(8, 8, 2, 4),  CPMAP_VARIANT(8, 8, 2, 8),  CPMAP_VARIANT(8, 4, 2, 4),
    CPMAP_VARIANT(8, 4, 2, 8),  CPMAP_VARIANT(4, 4, 2, 8),  CPMAP_VARIANT(4, 4, 2, 16),
    CPMAP_VARIANT(4, 4, 1, 16), CPMAP_VARIANT(2, 2, 1, 16), CPMAP_VARIANT(1, 1, 1, 16),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Waves of one variant that a SIMD holds at once, from the runtime's
// occupancy calculator (registers and LDS of the compiled kernel); cached.
int waves_per_simd(int idx)
{
    static std::atomic<int> cache[kNumVariants];
    int v = cache[idx].load(std::memory_order_relaxed);
    if (v > 0)
        return v;
    const Variant &var = kVariants[idx];
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, var.kernel, kWave * var.w, 0) !=
            hipSuccess ||
        blocks <= 0)
        blocks = 1;
    v = std::max(1, blocks * var.w / 4);
    cache[idx].store(v, std::memory_order_relaxed);
    return v;
}

// Modelled run time of a variant, in VALU issue slots of the busiest SIMD.
//  - a pair costs 4 slots (fma, half-rate v_rsq_f32, fma) plus the blocking's
//    shared per-atom work;
//  - workgroups spread evenly over the 256 CUs and each puts W/4 waves on
//    every SIMD of its CU; a SIMD runs `occ` waves at once, and needs two
//    resident waves to keep its VALU busy, so a lone wave runs at half rate.
double variant_cost(int idx, const Lattice &lat, int64_t n_atoms)
{
    const Variant &v = kVariants[idx];
    const int64_t strips = ceil_div(lat.n[0], v.cx) * ceil_div(lat.n[1], v.cy) *
                           ceil_div(lat.n[2], v.cz);
    const int64_t groups = ceil_div(strips, kWave);
    const double np = v.cx * v.cy * v.cz;
    const double per_pair = 4.0 + (v.cx + v.cy + 2.0 * v.cz + v.cy * v.cz) / np;
    const double wave_work = std::ceil((double)n_atoms / v.w) * np * per_pair + 64.0 * np;
    const int64_t per_simd = ceil_div(groups, 256) * std::max(1, v.w / 4);
    const int occ = waves_per_simd(idx);
    double units = 0.0;
    for (int64_t left = per_simd; left > 0; left -= occ)
        units += (double)std::max<int64_t>(std::min<int64_t>(left, occ), 2);
    return units * wave_work;
}

const Variant &pick_variant(const Lattice &lat, int64_t n_atoms)
{
    int best = 0;
    double best_cost = variant_cost(0, lat, n_atoms);
    for (int i = 1; i < kNumVariants; ++i) {
        const double c = variant_cost(i, lat, n_atoms);
        if (c < best_cost) {
            best_cost = c;
            best = i;
        }
    }
    return kVariants[best];
}

}  // namespace

hipError_t launch_direct(const float4 *atoms, int64_t n_atoms, const Lattice &lat, float *V,
                         hipStream_t stream)
{
    const int64_t points = lat.points();
    if (points == 0)
        return hipSuccess;
    if (n_atoms == 0) {
        const int64_t blocks = std::min<int64_t>(ceil_div(points, 256), 4096);
        hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, V, points);
        return hipGetLastError();
    }
    const Variant &v = pick_variant(lat, n_atoms);
    const int32_t nsx = (int32_t)ceil_div(lat.n[0], v.cx);
    const int32_t nsy = (int32_t)ceil_div(lat.n[1], v.cy);
    const int64_t nsz = ceil_div(lat.n[2], v.cz);
    const int64_t strips = (int64_t)nsx * nsy * nsz;
    const int64_t blocks = ceil_div(strips, kWave);
    hipLaunchKernelGGL(v.kernel, dim3((unsigned)blocks), dim3(kWave * v.w), 0, stream, atoms,
                       n_atoms, lat.n[0], lat.n[1], lat.n[2], nsx, nsy, strips, lat.h, lat.o[0],
                       lat.o[1], lat.o[2], V);
    return hipGetLastError();
}

}  // namespace cpmap
