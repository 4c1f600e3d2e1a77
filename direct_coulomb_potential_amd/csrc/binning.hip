// Spatial binning of atoms on gfx950 (the binning lecture's pseudo-code slide,
// step 1: bin index = position / BIN_SIZE, atoms appended to their bin; the
// notes' section 18.5 BinTable: bins flattened into one atom array with a
// start offset per bin).
//
// The lecture bins on the CPU into fixed 8-slot bins with an overflow list;
// here the GPU builds a CSR (bin_start + atoms sorted by bin), so no bin can
// overflow and the workspace size depends only on the atom count and the
// geometry.  The sort is a stable LSD radix sort on the bin id (8-bit digits,
// as many passes as the bin count needs), so atoms keep their input order
// inside a bin and the output is bit-identical from run to run:
//   keys      bin id per atom (nbins for dropped atoms, which sort last),
//             formed by the first pass's histogram kernel
//   per pass  tile histograms -> one exclusive scan (digit-major) -> stable
//             scatter, ranking equal digits inside a wave with ballots
//   finish    one launch, two jobs: bin_start[b] = lower_bound(sorted keys,
//             b), and sorted atoms = atoms[sorted indices]
#include "cpmap_internal.h"

namespace cpmap {
namespace {

constexpr int kThreads = 256;
constexpr int kItems = 8;                        // elements per thread per tile
constexpr int kTileElems = kThreads * kItems;    // elements per radix tile
constexpr int kDigits = 256;

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

struct KeyGeometry {
    float b0x, b0y, b0z, bs;
    int32_t nbx, nby, nbz, nbins;
};

// Bin id of an atom, or nbins when it lies outside the bin grid.
__device__ __forceinline__ int32_t atom_key(const float4 a, const KeyGeometry &G)
{
    const float tx = bin_coord(a.x, G.b0x, G.bs);
    const float ty = bin_coord(a.y, G.b0y, G.bs);
    const float tz = bin_coord(a.z, G.b0z, G.bs);
    const bool keep = tx >= 0.0f && tx < (float)G.nbx && ty >= 0.0f && ty < (float)G.nby &&
                      tz >= 0.0f && tz < (float)G.nbz;
    if (!keep)
        return G.nbins;
    const int32_t cx = (int32_t)floorf(tx), cy = (int32_t)floorf(ty), cz = (int32_t)floorf(tz);
    return (cz * G.nby + cy) * G.nbx + cx;
}

// Digit counts of one tile, written digit-major: hist[d * n_tiles + tile].
// FIRST: the first pass, which also forms the keys from the atoms and writes
// them with their input positions.
template <bool FIRST>
__global__ __launch_bounds__(kThreads) void k_hist(const float4 *__restrict__ atoms,
                                                   KeyGeometry G, int32_t *__restrict__ keys,
                                                   int32_t *__restrict__ vals, int32_t n,
                                                   int shift, int32_t n_tiles,
                                                   int32_t *__restrict__ hist)
{
    __shared__ int32_t cnt[kDigits];
    cnt[threadIdx.x] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kTileElems;
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int64_t e = base + it * kThreads + threadIdx.x;
        if (e < n) {
            int32_t key;
            if constexpr (FIRST) {
                key = atom_key(atoms[e], G);
                keys[e] = key;
                vals[e] = (int32_t)e;
            } else {
                key = keys[e];
            }
            atomicAdd(&cnt[(key >> shift) & 0xff], 1);
        }
    }
    __syncthreads();
    hist[(int64_t)threadIdx.x * n_tiles + blockIdx.x] = cnt[threadIdx.x];
}

// Exclusive scan of m int32 in place by one workgroup of 1024 threads, in
// rounds of 1024 x kScanPer values.  A round is read and written coalesced
// (thread t takes values t, t + 1024, ...) through an LDS copy, from which
// each thread takes kScanPer consecutive values; the threads' sums are
// scanned inside each wave with shuffles and across the 16 waves through
// LDS, and a carry links the rounds.  (Loading each thread's consecutive
// values straight from memory, 64 bytes apart across the lanes, took 2.5
// times as long for the 12,544 tile counts of 100,000 atoms.)
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 16;
constexpr int kScanRound = kScanThreads * kScanPer;

__global__ __launch_bounds__(kScanThreads) void k_scan(int32_t *__restrict__ data, int64_t m)
{
    __shared__ int32_t buf[kScanRound];
    __shared__ int32_t wave_sum[kScanThreads / 64];
    const int t = threadIdx.x;
    const int lane = t % 64;
    const int wave = t / 64;
    int32_t carry = 0;
    for (int64_t base = 0; base < m; base += kScanRound) {
        const int64_t n = m - base < kScanRound ? m - base : kScanRound;
        int32_t r[kScanPer];
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            const int64_t i = (int64_t)k * kScanThreads + t;
            r[k] = i < n ? data[base + i] : 0;
        }
#pragma unroll
        for (int k = 0; k < kScanPer; ++k)
            buf[k * kScanThreads + t] = r[k];
        __syncthreads();
        int32_t v[kScanPer];
        int32_t s = 0;
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            v[k] = buf[t * kScanPer + k];
            s += v[k];
        }
        int32_t incl = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t u = __shfl_up(incl, off);
            if (lane >= off)
                incl += u;
        }
        if (lane == 63)
            wave_sum[wave] = incl;
        __syncthreads();
        int32_t run = carry + incl - s;
        int32_t total = 0;
        for (int w = 0; w < kScanThreads / 64; ++w) {
            const int32_t ws = wave_sum[w];
            run += w < wave ? ws : 0;
            total += ws;
        }
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            buf[t * kScanPer + k] = run;
            run += v[k];
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kScanPer; ++k) {
            const int64_t i = (int64_t)k * kScanThreads + t;
            if (i < n)
                data[base + i] = buf[k * kScanThreads + t];
        }
        carry += total;
        __syncthreads();  // buf and wave_sum are rewritten by the next round
    }
}

// Stable scatter of one tile.  The tile is walked in kItems sub-tiles of 256
// consecutive elements (element base + it*256 + thread), so input order is
// (sub-tile, wave, lane).  Inside a wave, lanes with the same digit are found
// with 8 ballots; across waves and sub-tiles, per-digit counters in LDS give
// the running offsets.
__global__ __launch_bounds__(kThreads) void k_scatter(
    const int32_t *__restrict__ keys_in, const int32_t *__restrict__ vals_in, int32_t n,
    int shift, int32_t n_tiles, const int32_t *__restrict__ offsets,
    int32_t *__restrict__ keys_out, int32_t *__restrict__ vals_out)
{
    constexpr int kWaves = kThreads / 64;
    __shared__ int32_t run[kDigits];             // elements of each digit placed so far
    __shared__ int32_t wave_cnt[kWaves][kDigits];
    const int t = threadIdx.x;
    const int wave = t / 64;
    const int lane = t % 64;
    const int64_t base = (int64_t)blockIdx.x * kTileElems;
    // the tile's keys and values are loaded at once, with the tile's digit
    // offsets, before the sub-tiles' barriers (one memory latency instead of
    // one per sub-tile)
    int32_t keys_r[kItems], vals_r[kItems];
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int64_t e = base + it * kThreads + t;
        keys_r[it] = e < n ? keys_in[e] : 0;
        vals_r[it] = e < n ? vals_in[e] : 0;
    }
    run[t] = offsets[(int64_t)t * n_tiles + blockIdx.x];
    for (int w = 0; w < kWaves; ++w)
        wave_cnt[w][t] = 0;
    __syncthreads();
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int it = 0; it < kItems; ++it) {
        const int64_t e = base + it * kThreads + t;
        const bool valid = e < n;
        const int32_t key = keys_r[it];
        const int32_t val = vals_r[it];
        const int d = valid ? (key >> shift) & 0xff : kDigits;  // invalid lanes: own class
        // lanes of this wave holding the same digit (invalid lanes match none)
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t vote = __ballot(bit);
            same &= bit ? vote : ~vote;
        }
        if (!valid)
            same = 0;
        const int rank = __popcll(same & lt_mask);
        if (valid && rank == 0)
            wave_cnt[wave][d] = __popcll(same);
        __syncthreads();
        if (valid) {
            int32_t pos = run[d] + rank;
            for (int w = 0; w < wave; ++w)
                pos += wave_cnt[w][d];
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
        __syncthreads();
        int32_t added = 0;
        for (int w = 0; w < kWaves; ++w) {
            added += wave_cnt[w][t];
            wave_cnt[w][t] = 0;
        }
        run[t] += added;
        __syncthreads();
    }
}

// The binning's last launch, two independent jobs in one grid: its first
// gather_blocks workgroups gather the sorted atoms (sorted[i] =
// atoms[idx[i]]), the others set bin_start[b] = the first position whose key
// is >= b, for b in [0, nbins], and workgroup gather_blocks also writes the
// workspace header (the kernels that read the workspace run after this
// launch).
__global__ __launch_bounds__(kThreads) void k_finish(const float4 *__restrict__ atoms,
                                                     const int32_t *__restrict__ idx,
                                                     const int32_t *__restrict__ keys, int32_t n,
                                                     int32_t nbins, uint32_t gather_blocks,
                                                     float4 *__restrict__ sorted,
                                                     int32_t *__restrict__ bin_start,
                                                     WorkspaceHeader *__restrict__ hdr,
                                                     WorkspaceHeader hdr_value)
{
    if (blockIdx.x < gather_blocks) {
        const int32_t i = blockIdx.x * kThreads + threadIdx.x;
        if (i < n)
            sorted[i] = atoms[idx[i]];
        return;
    }
    const int64_t b = (int64_t)(blockIdx.x - gather_blocks) * kThreads + threadIdx.x;
    if (b == 0)
        *hdr = hdr_value;
    if (b > nbins)
        return;
    int32_t lo = 0, hi = n;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if (keys[mid] < b)
            lo = mid + 1;
        else
            hi = mid;
    }
    bin_start[b] = lo;
}

int32_t radix_passes(int64_t nbins)
{
    int bits = 0;
    while (((int64_t)1 << bits) <= nbins)  // keys take values 0 .. nbins
        ++bits;
    return (bits + 7) / 8;
}

unsigned grid_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

BinLayout bin_layout(int64_t n_atoms, const BinGeometry &g)
{
    BinLayout L{};
    const size_t n = (size_t)n_atoms;
    L.n_tiles = (n_atoms + kTileElems - 1) / kTileElems;
    L.passes = radix_passes(g.nbins());
    L.header = 0;
    L.bin_start = kHeaderBytes;
    L.sorted = up256(L.bin_start + sizeof(int32_t) * (size_t)(g.nbins() + 1));
    L.keys[0] = up256(L.sorted + 16 * n);
    L.keys[1] = up256(L.keys[0] + 4 * n);
    L.vals[0] = up256(L.keys[1] + 4 * n);
    L.vals[1] = up256(L.vals[0] + 4 * n);
    L.hist = up256(L.vals[1] + 4 * n);
    L.total = up256(L.hist + sizeof(int32_t) * kDigits * (size_t)L.n_tiles);
    return L;
}

hipError_t launch_bin_atoms(const float4 *atoms, int64_t n_atoms, const Lattice &lat,
                            const BinGeometry &g, const BinLayout &L, void *workspace,
                            uint64_t nonce, hipStream_t stream)
{
    (void)lat;
    char *ws = static_cast<char *>(workspace);
    WorkspaceHeader *hdr = reinterpret_cast<WorkspaceHeader *>(ws + L.header);
    const WorkspaceHeader hv{kBinMagic, nonce};
    const int32_t n = (int32_t)n_atoms;
    const int32_t nbins = (int32_t)g.nbins();
    int32_t *bin_start = reinterpret_cast<int32_t *>(ws + L.bin_start);
    float4 *sorted = reinterpret_cast<float4 *>(ws + L.sorted);
    int32_t *keys[2] = {reinterpret_cast<int32_t *>(ws + L.keys[0]),
                        reinterpret_cast<int32_t *>(ws + L.keys[1])};
    int32_t *vals[2] = {reinterpret_cast<int32_t *>(ws + L.vals[0]),
                        reinterpret_cast<int32_t *>(ws + L.vals[1])};
    int32_t *hist = reinterpret_cast<int32_t *>(ws + L.hist);

    if (n > 0) {
        KeyGeometry G;
        G.b0x = g.ax[0].b0;
        G.b0y = g.ax[1].b0;
        G.b0z = g.ax[2].b0;
        G.bs = g.bin_size;
        G.nbx = g.ax[0].nb;
        G.nby = g.ax[1].nb;
        G.nbz = g.ax[2].nb;
        G.nbins = nbins;
        const int32_t tiles = (int32_t)L.n_tiles;
        for (int p = 0; p < L.passes; ++p) {
            const int shift = 8 * p;
            const int src = p & 1, dst = src ^ 1;
            if (p == 0)
                hipLaunchKernelGGL(k_hist<true>, dim3(tiles), dim3(kThreads), 0, stream, atoms,
                                   G, keys[0], vals[0], n, shift, tiles, hist);
            else
                hipLaunchKernelGGL(k_hist<false>, dim3(tiles), dim3(kThreads), 0, stream, atoms,
                                   G, keys[src], vals[src], n, shift, tiles, hist);
            hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, stream, hist,
                               (int64_t)kDigits * tiles);
            hipLaunchKernelGGL(k_scatter, dim3(tiles), dim3(kThreads), 0, stream, keys[src],
                               vals[src], n, shift, tiles, hist, keys[dst], vals[dst]);
        }
        const int fin = L.passes & 1;
        const unsigned gb = grid_for(n);
        hipLaunchKernelGGL(k_finish, dim3(gb + grid_for((int64_t)nbins + 1)), dim3(kThreads), 0,
                           stream, atoms, vals[fin], keys[fin], n, nbins, gb, sorted, bin_start,
                           hdr, hv);
    } else {
        hipLaunchKernelGGL(k_finish, dim3(grid_for((int64_t)nbins + 1)), dim3(kThreads), 0,
                           stream, atoms, vals[0], keys[0], 0, nbins, 0u, sorted, bin_start, hdr,
                           hv);
    }
    return hipGetLastError();
}

}  // namespace cpmap
