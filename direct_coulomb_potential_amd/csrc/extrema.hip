// Ion placement on a potential map (the case-study notes' section 18.1:
// positive ions go to the node of lowest potential, negative ions to the node
// of highest): argmin and argmax of V on gfx950.
//
// An HBM-bound reduction in two launches: every workgroup reduces a
// contiguous slab of V (16-byte loads when V is 16-byte aligned) to
// (min, argmin, max, argmax) and writes it to the workspace; one workgroup
// then reduces the partials.  NaN nodes are skipped; among equal values the
// smallest index wins, which makes the combine associative and commutative,
// so the result does not depend on the order partial results meet.
#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;  // floats per thread per workgroup slab
constexpr int64_t kSlab = (int64_t)kThreads * kPerThread;
constexpr int kMaxBlocks = 4096;

struct alignas(16) Ext {
    float vmin, vmax;
    int64_t imin, imax;
};

__device__ __forceinline__ Ext ext_empty()
{
    Ext e;
    e.vmin = __builtin_nanf("");
    e.vmax = __builtin_nanf("");
    e.imin = -1;
    e.imax = -1;
    return e;
}

// Adds node (v, i) to e; nodes must arrive in increasing i within one e.
__device__ __forceinline__ void ext_add(Ext &e, float v, int64_t i)
{
    if (v != v)
        return;
    if (e.imin < 0 || v < e.vmin) {
        e.vmin = v;
        e.imin = i;
    }
    if (e.imax < 0 || v > e.vmax) {
        e.vmax = v;
        e.imax = i;
    }
}

// Order-free combine: the lower value wins the min side (the higher the max
// side); equal values go to the smaller index.
__device__ __forceinline__ Ext ext_combine(Ext a, const Ext &b)
{
    if (b.imin >= 0 &&
        (a.imin < 0 || b.vmin < a.vmin || (b.vmin == a.vmin && b.imin < a.imin))) {
        a.vmin = b.vmin;
        a.imin = b.imin;
    }
    if (b.imax >= 0 &&
        (a.imax < 0 || b.vmax > a.vmax || (b.vmax == a.vmax && b.imax < a.imax))) {
        a.vmax = b.vmax;
        a.imax = b.imax;
    }
    return a;
}

__device__ __forceinline__ Ext ext_shfl_xor(const Ext &e, int mask)
{
    Ext o;
    o.vmin = __shfl_xor(e.vmin, mask);
    o.vmax = __shfl_xor(e.vmax, mask);
    o.imin = __shfl_xor(e.imin, mask);
    o.imax = __shfl_xor(e.imax, mask);
    return o;
}

// Workgroup-wide combine; the result is valid in thread 0.
__device__ Ext block_reduce(Ext e)
{
    __shared__ Ext wave_part[kThreads / 64];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        e = ext_combine(e, ext_shfl_xor(e, m));
    if (threadIdx.x % 64 == 0)
        wave_part[threadIdx.x / 64] = e;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; ++w)
            e = ext_combine(e, wave_part[w]);
    }
    return e;
}

// Pass 1: workgroup b reduces the slabs b, b + gridDim.x, ... of V.
__global__ __launch_bounds__(kThreads) void extrema_partial(const float *__restrict__ V,
                                                            int64_t n, bool vec4,
                                                            Ext *__restrict__ part)
{
    Ext e = ext_empty();
    for (int64_t base = (int64_t)blockIdx.x * kSlab; base < n;
         base += (int64_t)gridDim.x * kSlab) {
        // thread t covers kPerThread consecutive nodes starting at
        // base + t * kPerThread; its indices increase, as ext_add needs
        const int64_t first = base + (int64_t)threadIdx.x * kPerThread;
        if (vec4 && first + kPerThread <= n) {
            const float4 *p = reinterpret_cast<const float4 *>(V + first);
#pragma unroll
            for (int k = 0; k < kPerThread / 4; ++k) {
                const float4 q = p[k];
                ext_add(e, q.x, first + 4 * k + 0);
                ext_add(e, q.y, first + 4 * k + 1);
                ext_add(e, q.z, first + 4 * k + 2);
                ext_add(e, q.w, first + 4 * k + 3);
            }
        } else {
            for (int k = 0; k < kPerThread; ++k)
                if (first + k < n)
                    ext_add(e, V[first + k], first + k);
        }
    }
    e = block_reduce(e);
    if (threadIdx.x == 0)
        part[blockIdx.x] = e;
}

// Pass 2: one workgroup combines the partials and writes the result.
__global__ __launch_bounds__(kThreads) void extrema_final(const Ext *__restrict__ part,
                                                          int32_t n_part,
                                                          int64_t *__restrict__ out_index,
                                                          float *__restrict__ out_value)
{
    Ext e = ext_empty();
    for (int32_t b = threadIdx.x; b < n_part; b += kThreads)
        e = ext_combine(e, part[b]);
    e = block_reduce(e);
    if (threadIdx.x == 0) {
        out_index[0] = e.imin;
        out_index[1] = e.imax;
        out_value[0] = e.vmin;
        out_value[1] = e.vmax;
    }
}

int32_t extrema_blocks(int64_t n)
{
    const int64_t b = (n + kSlab - 1) / kSlab;
    return (int32_t)(b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b));
}

}  // namespace

size_t extrema_workspace_bytes(int64_t n) { return sizeof(Ext) * (size_t)extrema_blocks(n); }

hipError_t launch_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value,
                          void *workspace, hipStream_t stream)
{
    const int32_t blocks = extrema_blocks(n);
    Ext *part = static_cast<Ext *>(workspace);
    const bool vec4 = (reinterpret_cast<uintptr_t>(V) % 16) == 0;
    hipLaunchKernelGGL(extrema_partial, dim3(blocks), dim3(kThreads), 0, stream, V, n, vec4, part);
    hipLaunchKernelGGL(extrema_final, dim3(1), dim3(kThreads), 0, stream, part, blocks, out_index,
                       out_value);
    return hipGetLastError();
}

}  // namespace cpmap
