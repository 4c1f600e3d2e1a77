// The scatter mapping of the direct sum, kept as a measured contrast to the
// gather (the case-study notes' section 18.2 and the PMPP solutions
// article's section 2: one thread per atom adds q/r into every node with an
// atomic add).
//
// Here each wave takes one atom and its 64 lanes walk the lattice in
// consecutive x-fastest node order, so one wave-wide fp32 atomic add touches
// 64 distinct adjacent nodes instead of 64 threads hitting the same node.
// Every node still receives one atomic per atom, in an order that varies
// from run to run: V agrees with the gather within the accuracy bound but is
// not bit-reproducible.  The gather (cpmap_direct) is the production path.
#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__global__ void zero_map(float *__restrict__ V, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        V[i] = 0.0f;
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(const float4 *__restrict__ atoms,
                                                           int64_t n_atoms, int32_t nx,
                                                           int32_t ny, int64_t points, float h,
                                                           float ox, float oy, float oz,
                                                           float *__restrict__ V)
{
    const int64_t a = (int64_t)blockIdx.x * kWaves + threadIdx.x / 64;
    if (a >= n_atoms)
        return;
    const float4 at = atoms[a];
    const int lane = threadIdx.x % 64;
    const int64_t rows = points / nx;
    for (int64_t row = 0; row < rows; ++row) {
        const int64_t j = row % ny;
        const int64_t k = row / ny;
        const float dy = node_coord(j, h, oy) - at.y;
        const float dz = node_coord(k, h, oz) - at.z;
        const float yz2 = fmaf(dy, dy, dz * dz);
        float *out = V + row * nx;
        for (int32_t i = lane; i < nx; i += 64) {
            const float dx = node_coord(i, h, ox) - at.x;
            // hardware fp32 atomic add in L2 (V is ordinary device memory)
            unsafeAtomicAdd(&out[i], at.w * __builtin_amdgcn_rsqf(fmaf(dx, dx, yz2)));
        }
    }
}

}  // namespace

hipError_t launch_scatter(const float4 *atoms, int64_t n_atoms, const Lattice &lat, float *V,
                          hipStream_t stream)
{
    const int64_t points = lat.points();
    if (points == 0)
        return hipSuccess;
    const int64_t zb = std::min<int64_t>((points + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_map, dim3((unsigned)zb), dim3(256), 0, stream, V, points);
    if (n_atoms > 0) {
        const int64_t blocks = (n_atoms + kWaves - 1) / kWaves;
        hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                           atoms, n_atoms, lat.n[0], lat.n[1], points, lat.h, lat.o[0], lat.o[1],
                           lat.o[2], V);
    }
    return hipGetLastError();
}

}  // namespace cpmap
