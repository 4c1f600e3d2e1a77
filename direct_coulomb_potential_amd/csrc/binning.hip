// Spatial binning of atoms (placeholder launcher; the GPU sort follows).
#include "cpmap_internal.h"

namespace cpmap {

BinLayout bin_layout(int64_t n_atoms, const BinGeometry &g)
{
    BinLayout L{};
    auto up = [](size_t v) { return (v + 255) & ~size_t(255); };
    L.header = 256;
    L.bin_start = L.header;
    L.sorted = up(L.bin_start + sizeof(int32_t) * (size_t)(g.nbins() + 1));
    L.total = up(L.sorted + 16 * (size_t)n_atoms);
    return L;
}

hipError_t launch_bin_atoms(const float4 *, int64_t, const Lattice &, const BinGeometry &,
                            const BinLayout &, void *, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace cpmap
