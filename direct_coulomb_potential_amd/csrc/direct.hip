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
//  - with a caller-provided workspace the atom list is also split into K
//    contiguous parts across workgroups (short atom slices per workgroup run
//    some 9% faster than whole-atom-list ones: VALU busy 112% against 102%
//    in the counters; and the extra workgroups even out the last round of the
//    1024 SIMDs).  The parts of a node group are added in part order, in one
//    of two ways:
//      ordered   (at least as many node groups as resident workgroups) in
//                place: part 0 stores its sum, part p waits until part p - 1
//                of the same group has added its own and then adds its sum
//                to V.  Each workgroup takes a ticket from a counter when it
//                starts, and the ticket (not the workgroup's index) names its
//                part and group, parts in order; a part's predecessor
//                therefore started before it and waits only on its own
//                predecessor, so every wait ends (it is also bounded: a part
//                that ran out of it writes NaN, which no ordinary run does).
//                Tickets are G apart for the two parts, so the predecessor
//                has long finished when its successor gets to its store; the
//                workspace is the counter and one count per group.
//      partial   (fewer groups: all parts run at once, and ordered additions
//                would queue) part 0 stores into V and part p into partial
//                map p - 1 of the workspace; sum_parts then adds the maps
//                into V in part order.
//    Either way the fp32 additions happen in the same order on every run.
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
    float yz[CY * CZ];
#pragma unroll
    for (int e = 0; e < CZ; ++e) {
        const float dz = z[e] - a.z;
        const float dz2 = dz * dz;
#pragma unroll
        for (int d = 0; d < CY; ++d)
            yz[e * CY + d] = fmaf(dy[d], dy[d], dz2);
    }
    // The nodes in one sequence, one node ahead: v_rsq_f32 of node n, then
    // r^2 of node n + 1, then node n's accumulation.  The empty asm pins that
    // order (the compiler otherwise chains each node through one register:
    // fma, rsq, a wait state, fma).  Same instructions and the same sums, bit
    // for bit; on the 200^3 x 200,000 map 156 ms against 165 ms chained,
    // 159 ms when each row of CX nodes restarts the sequence, 173 ms with a
    // row's rsq grouped and 176 ms with the accumulation two nodes behind.
    constexpr int NP = CX * CY * CZ;
    float r = fmaf(dx[0], dx[0], yz[0]);
#pragma unroll
    for (int n = 0; n < NP; ++n) {
        float rs = __builtin_amdgcn_rsqf(r);
        if (n + 1 < NP) {
            r = fmaf(dx[(n + 1) % CX], dx[(n + 1) % CX], yz[(n + 1) / CX]);
            asm volatile("" : "+v"(rs), "+v"(r));
        } else {
            asm volatile("" : "+v"(rs));
        }
        acc[n] = fmaf(a.w, rs, acc[n]);
    }
}

// The ordered split's state in the workspace: chain[0] counts the
// workgroups that have started; chain[kChainHead + g] counts the parts of
// node group g already added into V.
constexpr int kChainHead = 64;

// How the parts of a node group are added (see the file comment).
enum SplitMode { kSingle = 0, kOrdered = 1, kPartial = 2 };

// Workgroup ticket t (its index unless the split is ordered, else its place
// among the started workgroups) handles node group t % n_groups against atom
// part t / n_groups.  Its nodes go to V (part 0, or every part when ordered)
// or, for a partial split, to partial map part - 1 in the workspace.  The
// workspace is the ordered split's counters (uint32) or the partial maps
// (nx*ny*nz floats each).
// OCC is the resident waves per SIMD the variant is planned for; the
// compiler keeps its registers within that budget.
template <int CX, int CY, int CZ, int W, int OCC>
__global__ __launch_bounds__(kWave *W) __attribute__((amdgpu_waves_per_eu(OCC))) void direct_kernel(
    const float4 *__restrict__ atoms, int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
    int32_t nsx, int32_t nsy, int64_t n_strips, int64_t n_groups, int32_t n_parts, float h,
    float ox, float oy, float oz, int32_t mode, void *__restrict__ ws, int64_t max_polls,
    float *__restrict__ V)
{
    constexpr int NP = CX * CY * CZ;
    __shared__ float total[NP * kWave];
    __shared__ uint32_t s_ticket;
    __shared__ int s_in_order;

    const int slice = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int lane = threadIdx.x % kWave;

    uint32_t *chain = mode == kOrdered ? static_cast<uint32_t *>(ws) : nullptr;
    uint32_t ticket = blockIdx.x;
    if (chain != nullptr) {
        if (threadIdx.x == 0)
            s_ticket = atomicAdd(&chain[0], 1u);
        __syncthreads();
        ticket = s_ticket;
    }
    // Lane -> block of nodes.  Lanes past the last block recompute the last
    // block (they still take part in the reduction) and store nothing.
    const int64_t group = (int64_t)ticket % n_groups;
    const int32_t part = (int32_t)((int64_t)ticket / n_groups);
    const int64_t s_raw = group * kWave + lane;
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

    // This wave's contiguous slice of the part's atoms, processed in rounds
    // of at most kChunk atoms; every wave runs the same number of rounds.
    const int64_t p_begin = n_atoms * part / n_parts;
    const int64_t p_len = n_atoms * (part + 1) / n_parts - p_begin;
    const int64_t a_begin = p_begin + p_len * slice / W;
    const int64_t a_end = p_begin + p_len * (slice + 1) / W;
    const int64_t max_len = (p_len + W - 1) / W;
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
        // Add the round's partial sums into the LDS total.  Up to 8 waves:
        // the nodes are cut into W chunks and in phase s wave w adds its
        // chunk (w + s) mod W, so the waves update disjoint chunks at once
        // and chunk c receives the waves in the fixed order c, c - 1, ...
        // (mod W).  16 waves (1 to 32 nodes per lane): one wave after the
        // other, in wave order; rotating there costs scalar registers and
        // halves those variants' occupancy.
        if constexpr (W <= 8) {
            constexpr int kPer = (NP + W - 1) / W;
            for (int s = 0; s < W; ++s) {
                __syncthreads();
                const int mine = (slice + s) % W;
#pragma unroll
                for (int c = 0; c < W; ++c) {
                    if (c != mine)
                        continue;
#pragma unroll
                    for (int i = 0; i < kPer; ++i) {
                        const int p = c * kPer + i;
                        if (p < NP)
                            total[p * kWave + lane] += acc[p];
                    }
                }
            }
        } else {
            for (int w = 0; w < W; ++w) {
                __syncthreads();
                if (slice == w) {
#pragma unroll
                    for (int p = 0; p < NP; ++p)
                        total[p * kWave + lane] += acc[p];
                }
            }
        }
    }
    __syncthreads();

    // Parts after the first wait for their predecessor's addition into V.
    uint32_t *done = chain != nullptr ? chain + kChainHead + group : nullptr;
    bool in_order = true;
    if (done != nullptr) {
        if (threadIdx.x == 0) {
            int64_t polls = 0;
            while (__hip_atomic_load(done, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) !=
                       (uint32_t)part &&
                   polls < max_polls) {
                __builtin_amdgcn_s_sleep(8);
                ++polls;
            }
            s_in_order = polls < max_polls;
        }
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        in_order = s_in_order != 0;
    }

    // x-fastest store (part 0) or addition (later parts) of the LDS total;
    // the waves share the rows.  Columns past nx, rows past ny and planes past
    // nz are dropped.
    if (live) {
        const bool add = done != nullptr && part > 0;
        float *dst = (mode == kPartial && part > 0)
                         ? static_cast<float *>(ws) + (int64_t)(part - 1) * nx * ny * nz
                         : V;
        for (int row = slice; row < CY * CZ; row += W) {
            const int32_t j = j0 + row % CY;
            const int32_t k = k0 + row / CY;
            if (j >= ny || k >= nz)
                continue;
            float *out = dst + ((int64_t)k * ny + j) * nx;
            const float *src = total + row * CX * kWave + lane;
#pragma unroll
            for (int c = 0; c < CX; ++c) {
                if (i0 + c < nx) {
                    const float v = add ? out[i0 + c] + src[c * kWave] : src[c * kWave];
                    out[i0 + c] = in_order ? v : __builtin_nanf("");
                }
            }
        }
    }
    if (done != nullptr) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_store(done, (uint32_t)part + 1, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void fill_zero(float *__restrict__ V, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        V[i] = 0.0f;
}

// V[i] += partial maps 1, 2, ... at i, in that order (partial map k - 1 of
// `partials` holds part k).
__global__ void sum_parts(const float *__restrict__ partials, int32_t n_maps, int64_t n,
                          float *__restrict__ V)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        float v = V[i];
        for (int32_t k = 0; k < n_maps; ++k)
            v += partials[(int64_t)k * n + i];
        V[i] = v;
    }
}

// Clears the ordered split's counter and per-group counts.
__global__ void chain_reset(uint32_t *__restrict__ chain, int64_t n_words)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += stride)
        chain[i] = 0u;
}

using KernelFn = void (*)(const float4 *, int64_t, int32_t, int32_t, int32_t, int32_t, int32_t,
                          int64_t, int64_t, int32_t, float, float, float, float, int32_t, void *,
                          int64_t, float *);

struct Variant {
    int cx, cy, cz, w;
    int occupancy;  // waves per SIMD the compiled kernel allows (registers, LDS)
    KernelFn kernel;
};

#define CPMAP_VARIANT(CX, CY, CZ, W, OCC) \
    Variant{CX, CY, CZ, W, OCC, direct_kernel<CX, CY, CZ, W, OCC>}

// Occupancies (resident waves per SIMD) are those of the gfx950 build (183,
// 111, 67, 54, 41 and 29 VGPRs; LDS never limits); a GPU test checks them
// against the runtime.
const Variant kVariants[] = {
    CPMAP_VARIANT(8, 8, 2, 4, 2),  CPMAP_VARIANT(8, 8, 2, 8, 2),  CPMAP_VARIANT(8, 4, 2, 4, 4),
    CPMAP_VARIANT(8, 4, 2, 8, 4),  CPMAP_VARIANT(4, 4, 2, 8, 6),  CPMAP_VARIANT(4, 4, 2, 16, 4),
    CPMAP_VARIANT(4, 4, 1, 16, 8), CPMAP_VARIANT(2, 2, 1, 16, 8), CPMAP_VARIANT(1, 1, 1, 16, 8),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);
constexpr int kMaxParts = 32;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t variant_groups(const Variant &v, const Lattice &lat)
{
    const int64_t strips = ceil_div(lat.n[0], v.cx) * ceil_div(lat.n[1], v.cy) *
                           ceil_div(lat.n[2], v.cz);
    return ceil_div(strips, kWave);
}

// Workgroups of a variant resident on the 256 CUs at once.
int64_t resident_workgroups(const Variant &v)
{
    return 256 * std::max(1, v.occupancy * 4 / v.w);
}

SplitMode split_mode(const Variant &v, int32_t parts, const Lattice &lat)
{
    if (parts <= 1)
        return kSingle;
    return variant_groups(v, lat) >= resident_workgroups(v) ? kOrdered : kPartial;
}

constexpr double kMaxPartialBytes = 64.0 * (1 << 20);  // cap on partial maps

struct Plan {
    int variant;
    int32_t parts;
    double seconds;
};

// Modelled run time of a variant with the atoms split into `parts` across
// workgroups:
//  - a pair costs 4 VALU issue slots (fma, half-rate v_rsq_f32, fma) plus the
//    blocking's shared per-atom work;
//  - workgroups spread evenly over the 256 CUs, each putting W/4 waves on
//    every SIMD of its CU; a SIMD runs `occupancy` waves at once and needs two
//    resident waves to keep its VALU busy, so a lone wave runs at half rate;
//    a round with fewer resident waves than the variant's occupancy also
//    hides less latency: at half the occupancy it runs ~7% slower (measured
//    on the 8x4x2 variant, whose occupancy is 4);
//  - one issue slot of a wave is 4 cycles at 2.4 GHz;
//  - with parts > 1, every part reads and writes its nodes of V once
//    (ordered), or the parts' maps are written once and summed once
//    (partial).
double plan_seconds(const Variant &v, int32_t parts, const Lattice &lat, int64_t n_atoms)
{
    const int64_t strips = ceil_div(lat.n[0], v.cx) * ceil_div(lat.n[1], v.cy) *
                           ceil_div(lat.n[2], v.cz);
    const int64_t groups = ceil_div(strips, kWave);
    const double np = v.cx * v.cy * v.cz;
    const double per_pair = 4.0 + (v.cx + v.cy + 2.0 * v.cz + v.cy * v.cz) / np;
    const double atoms_per_wave = std::ceil((double)n_atoms / ((double)parts * v.w));
    const double wave_work = atoms_per_wave * np * per_pair + 500.0;
    const int per_wg = std::max(1, v.w / 4);
    const int64_t per_simd = ceil_div(groups * parts, 256) * per_wg;
    const int occ = std::max(per_wg, v.occupancy / per_wg * per_wg);
    double units = 0.0;
    for (int64_t left = per_simd; left > 0; left -= occ) {
        const double resident = (double)std::min<int64_t>(left, occ);
        units += std::max(resident, 1.5) * (1.0 + 0.14 * (1.0 - resident / occ));
    }
    double t = units * wave_work * 4.0 / 2.4e9;
    if (parts > 1)
        t += (split_mode(v, parts, lat) == kOrdered ? 2.0 * parts : 2.0 * parts + 1.0) * 4.0 *
                 (double)lat.points() / 8.0e12 +
             3e-6;
    return t;
}

Plan make_plan(const Lattice &lat, int64_t n_atoms, bool allow_parts)
{
    Plan best{0, 1, plan_seconds(kVariants[0], 1, lat, n_atoms)};
    const int max_parts = allow_parts ? kMaxParts : 1;
    for (int i = 0; i < kNumVariants; ++i) {
        for (int32_t k = 1; k <= max_parts; ++k) {
            if (k > 1 && variant_groups(kVariants[i], lat) * k > (int64_t)INT32_MAX)
                break;  // tickets and the grid stay below 2^31
            if (split_mode(kVariants[i], k, lat) == kPartial &&
                (double)(k - 1) * 4.0 * (double)lat.points() > kMaxPartialBytes)
                break;
            if (k > 1 && n_atoms < (int64_t)k * kVariants[i].w * 64)
                break;  // keep at least 64 atoms per wave
            const double t = plan_seconds(kVariants[i], k, lat, n_atoms);
            // prefer fewer parts unless clearly faster
            if (t < best.seconds * (k > best.parts ? 0.995 : 1.0)) {
                best = Plan{i, k, t};
            }
        }
    }
    return best;
}

// The ordered split's counter and per-group counts, or the partial maps of
// parts 1 .. K-1, in 256-byte units.
size_t plan_workspace(const Plan &p, const Lattice &lat)
{
    const Variant &v = kVariants[p.variant];
    size_t bytes = 0;
    switch (split_mode(v, p.parts, lat)) {
    case kSingle:
        return 0;
    case kOrdered:
        bytes = (kChainHead + (size_t)variant_groups(v, lat)) * sizeof(uint32_t);
        break;
    case kPartial:
        bytes = (size_t)(p.parts - 1) * (size_t)lat.points() * sizeof(float);
        break;
    }
    return (bytes + 255) & ~size_t(255);
}

}  // namespace

size_t direct_workspace_bytes(int64_t n_atoms, const Lattice &lat)
{
    if (lat.points() == 0 || n_atoms == 0)
        return 0;
    return plan_workspace(make_plan(lat, n_atoms, true), lat);
}

void direct_plan(int64_t n_atoms, const Lattice &lat, bool with_workspace, int32_t out[5])
{
    const Plan p = make_plan(lat, n_atoms, with_workspace);
    const Variant &v = kVariants[p.variant];
    out[0] = v.cx;
    out[1] = v.cy;
    out[2] = v.cz;
    out[3] = v.w;
    out[4] = p.parts;
}

int direct_occupancy_mismatches()
{
    int bad = 0;
    for (const Variant &v : kVariants) {
        int blocks = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, v.kernel, kWave * v.w, 0) !=
                hipSuccess ||
            blocks * v.w / 4 != v.occupancy)
            ++bad;
    }
    return bad;
}

hipError_t launch_direct(const float4 *atoms, int64_t n_atoms, const Lattice &lat, float *V,
                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    const int64_t points = lat.points();
    if (points == 0)
        return hipSuccess;
    if (n_atoms == 0) {
        const int64_t blocks = std::min<int64_t>(ceil_div(points, 256), 4096);
        hipLaunchKernelGGL(fill_zero, dim3((unsigned)blocks), dim3(256), 0, stream, V, points);
        return hipGetLastError();
    }
    Plan plan = make_plan(lat, n_atoms, workspace != nullptr);
    if (plan_workspace(plan, lat) > workspace_bytes)
        plan = make_plan(lat, n_atoms, false);
    const Variant &v = kVariants[plan.variant];
    const int32_t nsx = (int32_t)ceil_div(lat.n[0], v.cx);
    const int32_t nsy = (int32_t)ceil_div(lat.n[1], v.cy);
    const int64_t nsz = ceil_div(lat.n[2], v.cz);
    const int64_t strips = (int64_t)nsx * nsy * nsz;
    const int64_t groups = ceil_div(strips, kWave);
    int64_t max_polls = 0;
    const SplitMode mode = split_mode(v, plan.parts, lat);
    if (mode == kOrdered) {
        // A part waits at most about as long as its predecessor's task runs
        // (it started later on equal work): bound the wait at ten modelled
        // task times, at least 2^26 polls of s_sleep(8) (about 14 s).
        const double np = v.cx * v.cy * v.cz;
        const double per_pair = 4.0 + (v.cx + v.cy + 2.0 * v.cz + v.cy * v.cz) / np;
        const double task_s = std::ceil((double)n_atoms / ((double)plan.parts * v.w)) * np *
                              per_pair * 4.0 * v.occupancy / 2.0e9;
        max_polls = std::max<int64_t>(1ll << 26, (int64_t)std::min(1e15, 10.0 * task_s / 2.0e-7));
        uint32_t *chain = static_cast<uint32_t *>(workspace);
        const int64_t words = kChainHead + groups;
        hipLaunchKernelGGL(chain_reset, dim3((unsigned)std::min<int64_t>(ceil_div(words, 256), 64)),
                           dim3(256), 0, stream, chain, words);
    }
    hipLaunchKernelGGL(v.kernel, dim3((unsigned)(groups * plan.parts)), dim3(kWave * v.w), 0,
                       stream, atoms, n_atoms, lat.n[0], lat.n[1], lat.n[2], nsx, nsy, strips,
                       groups, plan.parts, lat.h, lat.o[0], lat.o[1], lat.o[2], (int32_t)mode,
                       mode == kSingle ? nullptr : workspace, max_polls, V);
    if (mode == kPartial) {
        const int64_t blocks = std::min<int64_t>(ceil_div(points, 256), 8192);
        hipLaunchKernelGGL(sum_parts, dim3((unsigned)blocks), dim3(256), 0, stream,
                           static_cast<const float *>(workspace), plan.parts - 1, points, V);
    }
    return hipGetLastError();
}

}  // namespace cpmap
