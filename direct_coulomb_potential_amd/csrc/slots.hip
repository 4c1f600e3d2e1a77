// Fixed-capacity bins with an overflow list (the binning lecture's slides
// 33-35: every bin holds the same number of atom slots, 8 slots of 16 bytes
// there, and the atoms that do not fit go to an extra list, which the
// lecture hands to the CPU).
//
// Here both are built on the GPU from the stable CSR of cpmap_bin_atoms, so
// a bin's slots take its first cap atoms in input order and its later atoms
// are its overflow, exactly as a sequential fill in input order would place
// them, and the result is the same on every run:
//   slot_fill        slots[b * cap + s] = atom s of bin b, or the empty-slot
//                    marker (+inf, +inf, +inf, 0) when bin b has fewer atoms;
//   over_chunk_sums  overflow atoms per chunk of kChunkBins bins;
//   over_chunk_scan  exclusive scan of the chunk sums (one workgroup);
//   over_starts      over_start[b] = overflow atoms in bins before b;
//   over_place       each overflow atom to over_atoms[over_start[b] + rank],
//                    rank = its position in the bin minus cap.
// The overflow list is a CSR in its own right (over_start, over_atoms), so
// the cutoff kernel walks it as it walks the full CSR.
#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kThreads = 256;
constexpr int kBinsPerThread = 16;
constexpr int64_t kChunkBins = (int64_t)kThreads * kBinsPerThread;

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

unsigned blocks_for(int64_t n, int64_t cap_blocks)
{
    int64_t b = (n + kThreads - 1) / kThreads;
    if (b > cap_blocks)
        b = cap_blocks;
    return (unsigned)(b < 1 ? 1 : b);
}

// Atoms of bin b: [*start, *start + count), with the CSR offsets clamped to
// [0, n] so that a workspace whose contents changed since it was binned can
// give wrong slots but never an access outside the sorted atoms.
__device__ __forceinline__ int32_t bin_range(const int32_t *__restrict__ bin_start, int64_t b,
                                             int32_t n, int32_t *start)
{
    int32_t s = bin_start[b], e = bin_start[b + 1];
    s = s < 0 ? 0 : (s > n ? n : s);
    e = e < s ? s : (e > n ? n : e);
    *start = s;
    return e - s;
}

__device__ __forceinline__ int32_t over_count(const int32_t *__restrict__ bin_start, int64_t b,
                                              int32_t n, int32_t cap)
{
    int32_t s;
    const int32_t c = bin_range(bin_start, b, n, &s) - cap;
    return c > 0 ? c : 0;
}

__global__ __launch_bounds__(kThreads) void slot_fill(const int32_t *__restrict__ bin_start,
                                                      const float4 *__restrict__ sorted,
                                                      int32_t n_atoms, int64_t n_slots,
                                                      int32_t cap, float4 *__restrict__ slots)
{
    const float inf = __builtin_huge_valf();
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < n_slots; e += stride) {
        const int64_t b = e / cap;
        const int32_t s = (int32_t)(e - b * cap);
        int32_t start;
        const int32_t count = bin_range(bin_start, b, n_atoms, &start);
        slots[e] = s < count ? sorted[start + s] : make_float4(inf, inf, inf, 0.0f);
    }
}

// Exclusive scan of one value per thread across the workgroup; returns the
// thread's offset and sets *total to the workgroup sum.
__device__ int32_t block_exclusive_scan(int32_t v, int32_t *total)
{
    __shared__ int32_t buf[kThreads];
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const int32_t u = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += u;
        __syncthreads();
    }
    const int32_t incl = buf[t];
    *total = buf[kThreads - 1];
    __syncthreads();  // buf is reused by the next call
    return incl - v;
}

__global__ __launch_bounds__(kThreads) void over_chunk_sums(const int32_t *__restrict__ bin_start,
                                                            int32_t n_atoms, int64_t nbins,
                                                            int32_t cap,
                                                            int32_t *__restrict__ chunk_sum)
{
    const int64_t first = (int64_t)blockIdx.x * kChunkBins + threadIdx.x * kBinsPerThread;
    int32_t local = 0;
    for (int i = 0; i < kBinsPerThread; ++i)
        if (first + i < nbins)
            local += over_count(bin_start, first + i, n_atoms, cap);
    int32_t total;
    block_exclusive_scan(local, &total);
    if (threadIdx.x == 0)
        chunk_sum[blockIdx.x] = total;
}

// chunk_sum[0 .. n) -> exclusive offsets; chunk_sum[n] = the overflow total.
__global__ __launch_bounds__(kThreads) void over_chunk_scan(int32_t *__restrict__ chunk_sum,
                                                            int64_t n)
{
    int32_t carry = 0;
    for (int64_t base = 0; base < n; base += kThreads) {
        const int64_t i = base + threadIdx.x;
        const int32_t v = i < n ? chunk_sum[i] : 0;
        int32_t total;
        const int32_t off = block_exclusive_scan(v, &total);
        if (i < n)
            chunk_sum[i] = carry + off;
        carry += total;
    }
    if (threadIdx.x == 0)
        chunk_sum[n] = carry;
}

__global__ __launch_bounds__(kThreads) void over_starts(const int32_t *__restrict__ bin_start,
                                                        int32_t n_atoms, int64_t nbins,
                                                        int32_t cap,
                                                        const int32_t *__restrict__ chunk_sum,
                                                        int64_t n_chunks,
                                                        int32_t *__restrict__ over_start)
{
    const int64_t first = (int64_t)blockIdx.x * kChunkBins + threadIdx.x * kBinsPerThread;
    int32_t c[kBinsPerThread];
    int32_t local = 0;
    for (int i = 0; i < kBinsPerThread; ++i) {
        c[i] = first + i < nbins ? over_count(bin_start, first + i, n_atoms, cap) : 0;
        local += c[i];
    }
    int32_t total;
    int32_t run = chunk_sum[blockIdx.x] + block_exclusive_scan(local, &total);
    for (int i = 0; i < kBinsPerThread; ++i) {
        if (first + i < nbins)
            over_start[first + i] = run;
        run += c[i];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0)
        over_start[nbins] = chunk_sum[n_chunks];
}

// keys[p] is the bin of sorted atom p (the radix sort's final keys; dropped
// atoms carry nbins and sort last).  Destinations outside [0, n_atoms) --
// possible only when the binned workspace changed since it was binned --
// are skipped.
__global__ __launch_bounds__(kThreads) void over_place(const int32_t *__restrict__ keys,
                                                       const int32_t *__restrict__ bin_start,
                                                       const float4 *__restrict__ sorted,
                                                       int64_t n_atoms, int64_t nbins,
                                                       int32_t cap,
                                                       const int32_t *__restrict__ over_start,
                                                       float4 *__restrict__ over_atoms)
{
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x; p < n_atoms; p += stride) {
        const int32_t b = keys[p];
        if (b < 0 || b >= nbins)
            continue;
        const int64_t rank = p - bin_start[b];
        if (rank >= cap) {
            const int64_t dst = (int64_t)over_start[b] + (rank - cap);
            if (dst >= 0 && dst < n_atoms)
                over_atoms[dst] = sorted[p];
        }
    }
}

// The slot workspace's header, written last: the slot fill's number if the
// binned workspace it read still carried the header its record expects,
// else 0, which no record holds (the cutoff kernels then refuse the slots).
__global__ void slot_header(const WorkspaceHeader *__restrict__ bin_hdr, uint64_t bin_nonce,
                            uint64_t slot_nonce, WorkspaceHeader *__restrict__ hdr)
{
    const bool ok = bin_hdr->magic == kBinMagic && bin_hdr->nonce == bin_nonce;
    hdr->magic = kSlotMagic;
    hdr->nonce = ok ? slot_nonce : 0;
}

}  // namespace

SlotLayout slot_layout(int64_t n_atoms, const BinGeometry &g, int32_t cap)
{
    SlotLayout S{};
    const size_t nbins = (size_t)g.nbins();
    S.n_chunks = ((int64_t)nbins + kChunkBins - 1) / kChunkBins;
    S.header = 0;
    S.slots = kHeaderBytes;
    S.over_start = up256(S.slots + sizeof(float4) * nbins * (size_t)cap);
    S.over_atoms = up256(S.over_start + sizeof(int32_t) * (nbins + 1));
    S.chunk_sum = up256(S.over_atoms + sizeof(float4) * (size_t)n_atoms);
    S.total = up256(S.chunk_sum + sizeof(int32_t) * (size_t)(S.n_chunks + 1));
    return S;
}

hipError_t launch_bin_slots(const void *bin_workspace, const BinLayout &L, int64_t n_atoms,
                            const BinGeometry &g, int32_t cap, uint64_t bin_nonce,
                            void *slot_workspace, const SlotLayout &S, uint64_t slot_nonce,
                            hipStream_t stream)
{
    const char *bw = static_cast<const char *>(bin_workspace);
    char *sw = static_cast<char *>(slot_workspace);
    const WorkspaceHeader *bin_hdr = reinterpret_cast<const WorkspaceHeader *>(bw + L.header);
    WorkspaceHeader *hdr = reinterpret_cast<WorkspaceHeader *>(sw + S.header);
    const int32_t n = (int32_t)n_atoms;
    const int32_t *bin_start = reinterpret_cast<const int32_t *>(bw + L.bin_start);
    const float4 *sorted = reinterpret_cast<const float4 *>(bw + L.sorted);
    const int32_t *keys = reinterpret_cast<const int32_t *>(bw + L.keys[L.passes & 1]);
    float4 *slots = reinterpret_cast<float4 *>(sw + S.slots);
    int32_t *over_start = reinterpret_cast<int32_t *>(sw + S.over_start);
    float4 *over_atoms = reinterpret_cast<float4 *>(sw + S.over_atoms);
    int32_t *chunk_sum = reinterpret_cast<int32_t *>(sw + S.chunk_sum);
    const int64_t nbins = g.nbins();
    const int64_t n_slots = nbins * cap;

    hipLaunchKernelGGL(slot_fill, dim3(blocks_for(n_slots, 8192)), dim3(kThreads), 0, stream,
                       bin_start, sorted, n, n_slots, cap, slots);
    hipLaunchKernelGGL(over_chunk_sums, dim3((unsigned)S.n_chunks), dim3(kThreads), 0, stream,
                       bin_start, n, nbins, cap, chunk_sum);
    hipLaunchKernelGGL(over_chunk_scan, dim3(1), dim3(kThreads), 0, stream, chunk_sum,
                       S.n_chunks);
    hipLaunchKernelGGL(over_starts, dim3((unsigned)S.n_chunks), dim3(kThreads), 0, stream,
                       bin_start, n, nbins, cap, chunk_sum, S.n_chunks, over_start);
    if (n_atoms > 0)
        hipLaunchKernelGGL(over_place, dim3(blocks_for(n_atoms, 8192)), dim3(kThreads), 0,
                           stream, keys, bin_start, sorted, n_atoms, nbins, cap, over_start,
                           over_atoms);
    hipLaunchKernelGGL(slot_header, dim3(1), dim3(1), 0, stream, bin_hdr, bin_nonce, slot_nonce,
                       hdr);
    return hipGetLastError();
}

}  // namespace cpmap
