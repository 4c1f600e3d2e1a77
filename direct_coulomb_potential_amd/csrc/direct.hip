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
//  - W waves of a workgroup share the same lanes' nodes and split the atom
//    list into W contiguous slices; their partial sums are added in LDS in a
//    fixed order.  This fills the 1024 SIMDs for small lattices and keeps the
//    result deterministic.
//  - sums are blocked: every kFlush atoms the running fp32 sum is added into a
//    second accumulator, which bounds rounding growth for large same-sign
//    atom sets.
//  - nodes are stored x-fastest, V[(k*ny + j)*nx + i] (section 18.4); lanes
//    adjacent in x write adjacent 4*CX-byte runs.
#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kWave = 64;
constexpr int kFlush = 512;

// Lanes per workgroup group and groups per workgroup: a workgroup always has
// at least four waves, so dispatch granularity does not change with W.
template <int W>
struct Shape {
    static constexpr int groups = W >= 4 ? 1 : 4 / W;
    static constexpr int threads = kWave * W * groups;
};

template <int CX, int CY, int CZ>
struct Block {
    static constexpr int NP = CX * CY * CZ;
};

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
                const float r2 = fmaf(dx[c], dx[c], yz2);
                float &v = acc[(e * CY + d) * CX + c];
                v = fmaf(a.w, __builtin_amdgcn_rsqf(r2), v);
            }
        }
    }
}

template <int CX, int CY, int CZ, int W>
__global__ __launch_bounds__(Shape<W>::threads) void direct_kernel(
    const float4 *__restrict__ atoms, int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
    int32_t nsx, int32_t nsy, int64_t n_strips, float h, float ox, float oy, float oz,
    float *__restrict__ V)
{
    constexpr int NP = Block<CX, CY, CZ>::NP;
    constexpr int G = Shape<W>::groups;
    __shared__ float red[W > 1 ? G * NP * kWave : 1];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;
    const int grp = wave / W;
    const int slice = wave % W;

    // Lane -> block of nodes.  Lanes past the last block recompute the last
    // block (they still take part in the LDS reduction) and store nothing.
    const int64_t s_raw = ((int64_t)blockIdx.x * G + grp) * kWave + lane;
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

    float acc[NP], hi[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        acc[p] = 0.0f;
        hi[p] = 0.0f;
    }

    // This wave's contiguous slice of the atoms (wave-uniform bounds).
    const int64_t a_begin = n_atoms * slice / W;
    const int64_t a_end = n_atoms * (slice + 1) / W;

    int64_t a = a_begin;
    while (a < a_end) {
        const int64_t blk_end = a + kFlush < a_end ? a + kFlush : a_end;
        for (; a + 4 <= blk_end; a += 4) {
            const float4 t0 = atoms[a + 0];
            const float4 t1 = atoms[a + 1];
            const float4 t2 = atoms[a + 2];
            const float4 t3 = atoms[a + 3];
            accumulate_atom<CX, CY, CZ>(t0, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t1, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t2, x, y, z, acc);
            accumulate_atom<CX, CY, CZ>(t3, x, y, z, acc);
        }
        for (; a < blk_end; ++a)
            accumulate_atom<CX, CY, CZ>(atoms[a], x, y, z, acc);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            hi[p] += acc[p];
            acc[p] = 0.0f;
        }
    }

    if constexpr (W > 1) {
        // Fixed-order reduction of the W slices: slice 0 adds slices W-1 .. 1.
        float *mine = red + grp * NP * kWave;
        for (int w = W - 1; w >= 1; --w) {
            if (slice == w) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    mine[p * kWave + lane] = hi[p];
            }
            __syncthreads();
            if (slice == 0) {
#pragma unroll
                for (int p = 0; p < NP; ++p)
                    hi[p] += mine[p * kWave + lane];
            }
            __syncthreads();
        }
        if (slice != 0)
            return;
    }
    if (!live)
        return;

    // x-fastest store; columns past nx, rows past ny, planes past nz dropped.
#pragma unroll
    for (int e = 0; e < CZ; ++e) {
        const int32_t k = k0 + e;
        if (k >= nz)
            break;
#pragma unroll
        for (int d = 0; d < CY; ++d) {
            const int32_t j = j0 + d;
            if (j >= ny)
                break;
            float *row = V + ((int64_t)k * ny + j) * nx;
            if (i0 + CX <= nx) {
#pragma unroll
                for (int c = 0; c < CX; ++c)
                    row[i0 + c] = hi[(e * CY + d) * CX + c];
            } else {
#pragma unroll
                for (int c = 0; c < CX; ++c)
                    if (i0 + c < nx)
                        row[i0 + c] = hi[(e * CY + d) * CX + c];
            }
        }
    }
}

__global__ void fill_zero(float *__restrict__ V, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        V[i] = 0.0f;
}

struct Variant {
    int cx, cy, cz, w;
    void (*kernel)(const float4 *, int64_t, int32_t, int32_t, int32_t, int32_t, int32_t, int64_t,
                   float, float, float, float, float *);
    int threads;
};

#define CPMAP_VARIANT(CX, CY, CZ, W) \
    Variant{CX, CY, CZ, W, direct_kernel<CX, CY, CZ, W>, Shape<W>::threads}

const Variant kVariants[] = {
    CPMAP_VARIANT(8, 4, 2, 1), CPMAP_VARIANT(8, 4, 2, 2), CPMAP_VARIANT(8, 4, 2, 4),
    CPMAP_VARIANT(4, 4, 2, 1), CPMAP_VARIANT(4, 4, 2, 2), CPMAP_VARIANT(4, 4, 2, 4),
    CPMAP_VARIANT(4, 4, 2, 8), CPMAP_VARIANT(4, 4, 1, 8), CPMAP_VARIANT(2, 2, 1, 16),
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Slots per useful node-atom pair for a blocking, counting the blocks' ragged
// waste and the shared per-atom work; used to pick a variant for a lattice.
double variant_cost(const Variant &v, const Lattice &lat, int64_t n_atoms)
{
    const int64_t bx = ceil_div(lat.n[0], v.cx), by = ceil_div(lat.n[1], v.cy),
                  bz = ceil_div(lat.n[2], v.cz);
    const int64_t strips = bx * by * bz;
    const double np = v.cx * v.cy * v.cz;
    const double per_pair = 4.0 + (v.cx + v.cy + 2.0 * v.cz + v.cy * v.cz) / np;
    const double waste = (double)(strips * (int64_t)np) / (double)lat.points();
    // waves in flight versus the 1024 SIMDs: one round of waves per 4 per SIMD
    const double waves = (double)ceil_div(strips, kWave) * v.w;
    const double rounds = std::ceil(waves / 4096.0);
    const double fill = waves / (rounds * 4096.0);
    const double atoms_per_wave = (double)n_atoms / v.w;
    // small per-wave atom counts pay the reduction and loop start-up
    const double startup = 1.0 + 64.0 / (atoms_per_wave + 1.0);
    return per_pair * waste * startup / fill;
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
    const Variant *best = &kVariants[0];
    double best_cost = variant_cost(*best, lat, n_atoms);
    for (const Variant &v : kVariants) {
        const double c = variant_cost(v, lat, n_atoms);
        if (c < best_cost) {
            best_cost = c;
            best = &v;
        }
    }
    const int32_t nsx = (int32_t)ceil_div(lat.n[0], best->cx);
    const int32_t nsy = (int32_t)ceil_div(lat.n[1], best->cy);
    const int64_t nsz = ceil_div(lat.n[2], best->cz);
    const int64_t strips = (int64_t)nsx * nsy * nsz;
    const int groups = best->threads / (kWave * best->w);
    const int64_t blocks = ceil_div(strips, (int64_t)kWave * groups);
    hipLaunchKernelGGL(best->kernel, dim3((unsigned)blocks), dim3(best->threads), 0, stream, atoms,
                       n_atoms, lat.n[0], lat.n[1], lat.n[2], nsx, nsy, strips, lat.h, lat.o[0],
                       lat.o[1], lat.o[2], V);
    return hipGetLastError();
}

}  // namespace cpmap
