// Smoothed cutoff summation (placeholder launcher; the kernel follows).
#include "cpmap_internal.h"

namespace cpmap {

hipError_t launch_cutoff(const void *, const BinLayout &, int64_t, const Lattice &,
                         const BinGeometry &, float *, hipStream_t)
{
    return hipErrorNotSupported;
}

}  // namespace cpmap

extern "C" int64_t cpmap_neighbor_spans(int32_t, int32_t, int32_t, float, float, float, float,
                                        float, float, int32_t, int32_t, int32_t, int32_t *,
                                        int64_t)
{
    return -1;
}
