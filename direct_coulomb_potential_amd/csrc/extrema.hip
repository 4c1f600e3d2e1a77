// Ion placement on a potential map (the case-study notes' section 18.1:
// positive ions go to the node of lowest potential, negative ions to the node
// of highest): argmin and argmax of V on gfx950.
//
// An HBM-bound reduction in one launch.  V is read as groups of 4 consecutive
// values (one float4 when V is 16-byte aligned).  Every lane reduces each of
// its groups to its min and max (three fminf / fmaxf each) and keeps the first
// group, in its own order, holding its running extremum; the workgroup then
// reduces 64-bit keys (order-preserving value bits << 32 | the group's rank
// in the workgroup's order) with one min and one max, and publishes, per
// side, the value and the group's global number.  The last workgroup of the
// grid waits for every slot, combines them, reads the two winning groups
// again and takes the first element equal to each extremum.  Among equal
// values the smallest index wins (+0 and -0 are equal), NaN is skipped.
//
// Publication needs no fence and no shared counter: a slot is four 64-bit
// words, each (payload << 27) | tag, written with single-copy-atomic 64-bit
// stores, so a word that carries this call's tag carries this call's
// payload.  Nothing is cleared before a call: the host draws a fresh nonzero
// 27-bit tag for every call from a randomly seeded sequence, and stale memory
// passes only if all four words of a slot carry that tag (2^-108 for arbitrary
// contents).  The combining workgroup sets every word back to tag 0, which no
// call uses, so that a replay of a captured call, which repeats its tag,
// waits for fresh slots as well.  The wait is bounded (kMaxPolls rounds,
// seconds); it ends early in every ordinary run because every workgroup
// publishes its slot unconditionally and none waits on the combiner.
#include <atomic>
#include <chrono>
#include <mutex>
#include <random>
#include <vector>

#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int kLoads = 8;                          // groups per lane per slab
constexpr int64_t kWaveGroups = 64 * kLoads;       // groups per wave per slab (2048 values)
constexpr int64_t kSlabGroups = kWaveGroups * kWaves;
constexpr int kMaxBlocks = kThreads;               // one slot per combiner thread
constexpr int kTagBits = 27;
constexpr uint64_t kTagMask = (1ull << kTagBits) - 1;  // payloads fit 37 bits
constexpr int64_t kMaxPolls = 1ll << 24;
constexpr uint32_t kNoKey = 0xffffffffu;

// A workgroup's published result: (payload << 27) | tag for the minimum's
// order key, the maximum's order key, and the two groups' numbers + 1 (0: the
// workgroup saw no value).
struct alignas(32) Slot {
    uint64_t w[4];
};

// Order-preserving bits of a non-NaN value, with -0 and +0 made equal.
__device__ __forceinline__ uint32_t ordered(float v)
{
    const uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unordered(uint32_t o)
{
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m)
{
    const uint32_t lo = __shfl_xor((uint32_t)v, m);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// Values v[4g .. 4g + 3], NaN past n.
__device__ __forceinline__ float4 load_group(const float *__restrict__ V, int64_t n, int64_t g,
                                             bool vec4)
{
    const int64_t i = 4 * g;
    if (vec4 && i + 4 <= n)
        return reinterpret_cast<const float4 *>(V)[g];
    const float nan = __builtin_nanf("");
    return make_float4(i < n ? V[i] : nan, i + 1 < n ? V[i + 1] : nan,
                       i + 2 < n ? V[i + 2] : nan, i + 3 < n ? V[i + 3] : nan);
}

// (ordered value, group) of one side, combined order-free: the better value
// wins, equal values go to the smaller group; group < 0 means none.
struct Best {
    uint64_t v;
    int64_t g;
};

template <bool MIN>
__device__ __forceinline__ Best better(Best a, Best b)
{
    if (b.g < 0)
        return a;
    if (a.g < 0 || (MIN ? b.v < a.v : b.v > a.v) || (b.v == a.v && b.g < a.g))
        return b;
    return a;
}

__global__ __launch_bounds__(kThreads) void extrema_kernel(const float *__restrict__ V, int64_t n,
                                                           int32_t vec4, uint64_t tag,
                                                           Slot *__restrict__ slots,
                                                           int64_t *__restrict__ out_index,
                                                           float *__restrict__ out_value)
{
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int64_t n_groups = (n + 3) / 4;
    const int64_t G = gridDim.x;

    // Lane l of wave w takes, in slab s, the groups l, l + 64, ... of the
    // wave's 512; its local key ((s * kWaves + w) * kLoads + k) * 64 + l
    // grows with the group's number inside the workgroup's share.
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    uint32_t kmin = kNoKey, kmax = kNoKey;
    uint32_t s = 0;
    for (int64_t base = (int64_t)blockIdx.x * kSlabGroups; base < n_groups;
         base += G * kSlabGroups, ++s) {
        const int64_t wb = base + wave * kWaveGroups;
        float4 q[kLoads];
        if (vec4 && 4 * (wb + kWaveGroups) <= n) {
            // the wave's whole slab is in range: plain float4 loads
            const float4 *p = reinterpret_cast<const float4 *>(V) + wb;
#pragma unroll
            for (int k = 0; k < kLoads; ++k)
                q[k] = p[k * 64 + lane];
        } else {
#pragma unroll
            for (int k = 0; k < kLoads; ++k) {
                const int64_t g = wb + k * 64 + lane;
                q[k] = g < n_groups ? load_group(V, n, g, vec4 != 0)
                                    : make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                                  __builtin_nanf(""), __builtin_nanf(""));
            }
        }
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const float m = fminf(fminf(q[k].x, q[k].y), fminf(q[k].z, q[k].w));
            const float M = fmaxf(fmaxf(q[k].x, q[k].y), fmaxf(q[k].z, q[k].w));
            const uint32_t key = ((s * kWaves + wave) * kLoads + k) * 64 + lane;
            // an all-NaN group gives NaN, which no comparison takes; an equal
            // value replaces the starting +-inf only while no group is held
            if (m < vmin || (m == vmin && kmin == kNoKey)) {
                vmin = m;
                kmin = key;
            }
            if (M > vmax || (M == vmax && kmax == kNoKey)) {
                vmax = M;
                kmax = key;
            }
        }
    }
    // One 64-bit min (max) over (value, key) ((value, ~key)) per workgroup.
    uint64_t pmin = kmin == kNoKey ? ~0ull : ((uint64_t)ordered(vmin) << 32) | kmin;
    uint64_t pmax = kmax == kNoKey ? 0ull : ((uint64_t)ordered(vmax) << 32) | (uint32_t)~kmax;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const uint64_t a = shfl_xor64(pmin, m), b = shfl_xor64(pmax, m);
        pmin = a < pmin ? a : pmin;
        pmax = b > pmax ? b : pmax;
    }
    __shared__ uint64_t wave_min[kWaves], wave_max[kWaves];
    if (lane == 0) {
        wave_min[wave] = pmin;
        wave_max[wave] = pmax;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kWaves; ++w) {
            pmin = wave_min[w] < pmin ? wave_min[w] : pmin;
            pmax = wave_max[w] > pmax ? wave_max[w] : pmax;
        }
        // a local key back to the group's number
        auto group_of = [&](uint32_t key) -> int64_t {
            const uint32_t ln = key % 64, k = (key / 64) % kLoads;
            const uint32_t wv = (key / (64 * kLoads)) % kWaves, ss = key / (64 * kLoads * kWaves);
            return ((int64_t)blockIdx.x + (int64_t)ss * G) * kSlabGroups + (int64_t)wv * kWaveGroups +
                   (int64_t)k * 64 + ln;
        };
        const bool has_min = pmin != ~0ull, has_max = pmax != 0ull;
        const uint64_t pay[4] = {has_min ? (pmin >> 32) : 0, has_max ? (pmax >> 32) : 0,
                                 has_min ? (uint64_t)(group_of((uint32_t)pmin) + 1) : 0,
                                 has_max ? (uint64_t)(group_of(~(uint32_t)pmax) + 1) : 0};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __hip_atomic_store(&slots[blockIdx.x].w[j], (pay[j] << kTagBits) | tag,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blockIdx.x != G - 1)
        return;

    // The combiner: thread t polls slot t (threads past the grid poll the
    // last slot and count as ready) until every word carries this call's tag
    // or the bound is reached.
    const int g = (int)G;
    const int mine = (int)threadIdx.x < g ? (int)threadIdx.x : g - 1;
    __shared__ int pending;
    uint64_t w[4];
    int64_t polls = 0;
    for (;;) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            w[j] = __hip_atomic_load(&slots[mine].w[j], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        bool ready = true;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            ready = ready && (w[j] & kTagMask) == tag;
        ready = ready || (int)threadIdx.x >= g;
        if (threadIdx.x == 0)
            pending = 0;
        __syncthreads();
        if (!ready)
            pending = 1;
        __syncthreads();
        const bool done = pending == 0;
        __syncthreads();  // pending is reset by the next round
        if (done || ++polls >= kMaxPolls)
            break;
    }
    Best bmin{~0ull, -1}, bmax{0ull, -1};
    if ((int)threadIdx.x < g) {
        bmin = Best{w[0] >> kTagBits, (int64_t)(w[2] >> kTagBits) - 1};
        bmax = Best{w[1] >> kTagBits, (int64_t)(w[3] >> kTagBits) - 1};
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        bmin = better<true>(bmin, Best{shfl_xor64(bmin.v, m),
                                       (int64_t)shfl_xor64((uint64_t)bmin.g, m)});
        bmax = better<false>(bmax, Best{shfl_xor64(bmax.v, m),
                                        (int64_t)shfl_xor64((uint64_t)bmax.g, m)});
    }
    __shared__ Best wave_best[kWaves][2];
    if (lane == 0) {
        wave_best[wave][0] = bmin;
        wave_best[wave][1] = bmax;
    }
    __syncthreads();
    // leave every word at tag 0, which no call uses
    if ((int)threadIdx.x < g) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __hip_atomic_store(&slots[threadIdx.x].w[j], 0ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    if (threadIdx.x == 0) {
        for (int wv = 1; wv < kWaves; ++wv) {
            bmin = better<true>(bmin, wave_best[wv][0]);
            bmax = better<false>(bmax, wave_best[wv][1]);
        }
        // the first element of each winning group equal to its extremum
        int64_t idx[2] = {-1, -1};
        float val[2] = {__builtin_nanf(""), __builtin_nanf("")};
        const Best b2[2] = {bmin, bmax};
        for (int side = 0; side < 2; ++side) {
            if (b2[side].g < 0)
                continue;
            const float4 q = load_group(V, n, b2[side].g, vec4 != 0);
            const float c[4] = {q.x, q.y, q.z, q.w};
            const float t = unordered((uint32_t)b2[side].v);
            int j = 3;
            for (int u = 3; u >= 0; --u)
                if (c[u] == t)
                    j = u;
            idx[side] = 4 * b2[side].g + j;
            val[side] = c[j];
        }
        const bool timed_out = polls >= kMaxPolls;  // not expected: reported as index -2
        out_index[0] = timed_out ? -2 : idx[0];
        out_index[1] = timed_out ? -2 : idx[1];
        out_value[0] = val[0];
        out_value[1] = val[1];
    }
}

int32_t extrema_blocks(int64_t n)
{
    const int64_t groups = (n + 3) / 4;
    const int64_t b = (groups + kSlabGroups - 1) / kSlabGroups;
    return (int32_t)(b < 1 ? 1 : (b > kMaxBlocks ? kMaxBlocks : b));
}

// A fresh 27-bit call tag, never 0 (zeroed memory must not look like a
// published slot).  The sequence starts at a random point in every process.
uint64_t next_tag()
{
    static std::atomic<uint64_t> seq{[] {
        std::random_device rd;
        const uint64_t t = (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
        return ((uint64_t)rd() << 32) ^ (uint64_t)rd() ^ (t * 0x9e3779b97f4a7c15ull);
    }()};
    for (;;) {
        const uint64_t t = seq.fetch_add(1) & kTagMask;
        if (t != 0)
            return t;
    }
}

}  // namespace

// The allocation-free variant's slots: one copy per GPU, allocated when the
// library is loaded and held until the process ends, zero at load (tag 0: no
// call).  In host code this name is only a stand-in for the device address,
// which static_scratch() looks up.
static __device__ __align__(256) Slot scratch[kMaxBlocks];

size_t extrema_workspace_bytes(int64_t n) { return sizeof(Slot) * (size_t)extrema_blocks(n); }

size_t extrema_static_scratch_bytes() { return sizeof(scratch); }

hipError_t launch_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value,
                          void *workspace, hipStream_t stream)
{
    const int32_t blocks = extrema_blocks(n);
    const bool vec4 = (reinterpret_cast<uintptr_t>(V) % 16) == 0;
    hipLaunchKernelGGL(extrema_kernel, dim3(blocks), dim3(kThreads), 0, stream, V, n,
                       (int32_t)vec4, next_tag(), static_cast<Slot *>(workspace), out_index,
                       out_value);
    return hipGetLastError();
}

// Device address of the current device's copy of `scratch`: looked up with
// hipGetSymbolAddress the first time a device calls, with that device
// current, and kept per device.
static hipError_t static_scratch(void **out)
{
    static std::mutex mu;
    static std::vector<void *> per_device;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    std::lock_guard<std::mutex> lock(mu);
    if ((size_t)dev >= per_device.size())
        per_device.resize((size_t)dev + 1, nullptr);
    if (per_device[(size_t)dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        per_device[(size_t)dev] = p;
    }
    *out = per_device[(size_t)dev];
    return hipSuccess;
}

hipError_t launch_extrema_static(const float *V, int64_t n, int64_t *out_index,
                                 float *out_value, hipStream_t stream)
{
    if (extrema_workspace_bytes(n) > sizeof(scratch))
        return hipErrorInvalidValue;  // cannot happen: the grid never exceeds kMaxBlocks
    void *slots = nullptr;
    hipError_t e = static_scratch(&slots);
    if (e != hipSuccess)
        return e;
    return launch_extrema(V, n, out_index, out_value, slots, stream);
}

}  // namespace cpmap
