// Internal declarations shared by the cpmap host code and kernels (not the oracle).
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/cpmap.h"

namespace cpmap {

// Node coordinate along one axis: one fp32 rounding of origin + i*h (the
// header's lattice convention).  Same expression on host and device.
__host__ __device__ inline float node_coord(int64_t i, float h, float origin)
{
    return fmaf(static_cast<float>(i), h, origin);
}

// Bin grid of one axis (the header's bin-geometry paragraph).
struct AxisBins {
    float b0;    // bin-grid origin
    int32_t nb;  // bins along the axis
};

struct BinGeometry {
    AxisBins ax[3];
    int32_t halo;
    float bin_size;
    float cutoff;
    int64_t nbins() const { return (int64_t)ax[0].nb * ax[1].nb * ax[2].nb; }
};

// Bin coordinate of a position: fp32 subtract, then fp32 divide (both
// correctly rounded; hipcc keeps the IEEE divide by default).
__host__ __device__ inline float bin_coord(float p, float b0, float bs)
{
    const float d = p - b0;
    return d / bs;
}

// Fills g; returns CPMAP_OK, CPMAP_EINVAL or CPMAP_ERANGE.
cpmap_status make_bin_geometry(int32_t nx, int32_t ny, int32_t nz, float h,
                               float ox, float oy, float oz, float bin_size, float cutoff,
                               BinGeometry *g);

// ---- launchers (host) -------------------------------------------------------

struct Lattice {
    int32_t n[3];
    float h;
    float o[3];
    int64_t points() const { return (int64_t)n[0] * n[1] * n[2]; }
};

// Direct sum.  With a workspace of at least direct_workspace_bytes() the atoms
// may also be split across workgroups into partial maps kept there.
hipError_t launch_direct(const float4 *atoms, int64_t n_atoms, const Lattice &lat, float *V,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);
size_t direct_workspace_bytes(int64_t n_atoms, const Lattice &lat);
// Blocking (cx, cy, cz), waves per workgroup and atom parts the launch uses.
void direct_plan(int64_t n_atoms, const Lattice &lat, bool with_workspace, int32_t out[5]);
// Variants whose runtime occupancy differs from the planning table.
int direct_occupancy_mismatches();

// First bytes of a binned or slot workspace, written on the device by the
// last kernel of the call that fills it and checked by every kernel that
// reads it: `nonce` is the fill's number in the host registry (so a
// workspace whose memory was reused and overwritten since, outside the
// library, no longer matches its record).
struct alignas(16) WorkspaceHeader {
    uint64_t magic;
    uint64_t nonce;
};
constexpr uint64_t kBinMagic = 0x4e49425f50414d43ull;   // "CMAP_BIN"
constexpr uint64_t kSlotMagic = 0x544f4c535f50414dull;  // "MAP_SLOT"
constexpr size_t kHeaderBytes = 256;

// Workspace layout of the binned atoms.
struct BinLayout {
    size_t header;      // WorkspaceHeader (kHeaderBytes reserved)
    size_t bin_start;   // offset of int32[nbins + 1]
    size_t sorted;      // offset of float4[n_atoms]
    size_t keys[2];     // int32[n_pad] radix-sort key ping-pong
    size_t vals[2];     // int32[n_pad] radix-sort value ping-pong
    size_t hist;        // int32[256 * n_tiles] digit counts per tile
    size_t total;
    int64_t n_tiles;    // radix-sort tiles
    int32_t passes;     // radix passes (8 bits each)
};

BinLayout bin_layout(int64_t n_atoms, const BinGeometry &g);

// Writes the header {kBinMagic, nonce} last.
hipError_t launch_bin_atoms(const float4 *atoms, int64_t n_atoms, const Lattice &lat,
                            const BinGeometry &g, const BinLayout &L, void *workspace,
                            uint64_t nonce, hipStream_t stream);

// Checks the header against {kBinMagic, nonce}; on a mismatch every node of V
// is set to NaN and nothing else is read.
hipError_t launch_cutoff(const void *workspace, const BinLayout &L, int64_t n_atoms,
                         const Lattice &lat, const BinGeometry &g, int32_t term, uint64_t nonce,
                         float *V, hipStream_t stream);

// Fixed-capacity bins: cap slots per bin plus an overflow list in CSR form,
// both derived from the stable CSR of a binned workspace.
struct SlotLayout {
    size_t header;      // WorkspaceHeader (kHeaderBytes reserved)
    size_t slots;       // float4[nbins * cap]
    size_t over_start;  // int32[nbins + 1]
    size_t over_atoms;  // float4[n_atoms]
    size_t chunk_sum;   // int32[n_chunks + 1] (overflow counts per chunk of bins)
    size_t total;
    int64_t n_chunks;
};

SlotLayout slot_layout(int64_t n_atoms, const BinGeometry &g, int32_t cap);

// Reads a binned workspace whose header should be {kBinMagic, bin_nonce};
// writes the slot header last: {kSlotMagic, slot_nonce}, or a nonce of 0
// (which no record holds) when the binned header did not match.
hipError_t launch_bin_slots(const void *bin_workspace, const BinLayout &L, int64_t n_atoms,
                            const BinGeometry &g, int32_t cap, uint64_t bin_nonce,
                            void *slot_workspace, const SlotLayout &S, uint64_t slot_nonce,
                            hipStream_t stream);

// The slot pass, then the overflow pass adding into V; both check the slot
// header against {kSlotMagic, nonce} (NaN at every node on a mismatch).
hipError_t launch_cutoff_slots(const void *slot_workspace, const SlotLayout &S, int64_t n_atoms,
                               const Lattice &lat, const BinGeometry &g, int32_t cap,
                               int32_t term, uint64_t nonce, float *V, hipStream_t stream);

// Scatter form of the direct sum (atomics; a measured contrast).
hipError_t launch_scatter(const float4 *atoms, int64_t n_atoms, const Lattice &lat, float *V,
                          hipStream_t stream);

// Argmin / argmax of a map (ion placement).
size_t extrema_workspace_bytes(int64_t n);
hipError_t launch_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value,
                          void *workspace, hipStream_t stream);
// The same launch with the library's static per-device scratch as workspace.
size_t extrema_static_scratch_bytes();
hipError_t launch_extrema_static(const float *V, int64_t n, int64_t *out_index,
                                 float *out_value, hipStream_t stream);

// Nodes per tile edge of the cutoff kernel.
constexpr int kTile = 8;

}  // namespace cpmap
