// C ABI of libcpmap: argument checks on the host, then stream-ordered launches.
// Every check happens before the first HIP call, so a rejected call enqueues
// nothing and touches no device state.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "cpmap_internal.h"
#include "workspace_registry.h"

namespace cpmap {

namespace {

bool finite_pos(float v) { return std::isfinite(v) && v > 0.0f; }

cpmap_status check_lattice(int32_t nx, int32_t ny, int32_t nz, float h, float ox, float oy,
                           float oz)
{
    if (nx < 0 || ny < 0 || nz < 0)
        return CPMAP_EINVAL;
    if (!finite_pos(h) || !std::isfinite(ox) || !std::isfinite(oy) || !std::isfinite(oz))
        return CPMAP_EINVAL;
    if (nx > CPMAP_MAX_DIM || ny > CPMAP_MAX_DIM || nz > CPMAP_MAX_DIM)
        return CPMAP_ERANGE;
    if ((int64_t)nx * ny * nz > CPMAP_MAX_POINTS)
        return CPMAP_ERANGE;
    return CPMAP_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// The workspaces the library has filled (see workspace_registry.h).
WorkspaceRegistry g_registry;

WorkspaceKey make_key(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz, float h, float ox,
                      float oy, float oz, float bs, float rc, int32_t cap = 0)
{
    return WorkspaceKey::make(n_atoms, nx, ny, nz, h, ox, oy, oz, bs, rc, cap);
}

size_t map_bytes(int32_t nx, int32_t ny, int32_t nz)
{
    return sizeof(float) * (size_t)nx * (size_t)ny * (size_t)nz;
}

Lattice make_lattice(int32_t nx, int32_t ny, int32_t nz, float h, float ox, float oy, float oz)
{
    Lattice l;
    l.n[0] = nx;
    l.n[1] = ny;
    l.n[2] = nz;
    l.h = h;
    l.o[0] = ox;
    l.o[1] = oy;
    l.o[2] = oz;
    return l;
}

// Bin grid along one axis (the header's bin-geometry paragraph).
cpmap_status axis_bins(int32_t n, float h, float o, float bs, int32_t halo, AxisBins *out)
{
    out->b0 = fmaf(-(float)halo, bs, o);
    if (!std::isfinite(out->b0))
        return CPMAP_ERANGE;
    const float last = node_coord(n - 1, h, o);
    const float t = bin_coord(last, out->b0, bs);
    if (!(t >= 0.0f) || !(t < 1.0e8f))
        return CPMAP_ERANGE;
    const int64_t nb = (int64_t)std::floor(t) + 1 + halo;
    if (nb > (1 << 24))
        return CPMAP_ERANGE;
    out->nb = (int32_t)nb;
    return CPMAP_OK;
}

// Geometry and slot layout for the fixed-capacity entry points.
cpmap_status slot_setup(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz, float h, float ox,
                        float oy, float oz, float bs, float rc, int32_t cap, BinGeometry *g,
                        SlotLayout *S);

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

}  // namespace

cpmap_status make_bin_geometry(int32_t nx, int32_t ny, int32_t nz, float h, float ox, float oy,
                               float oz, float bin_size, float cutoff, BinGeometry *g)
{
    cpmap_status st = check_lattice(nx, ny, nz, h, ox, oy, oz);
    if (st != CPMAP_OK)
        return st;
    if (nx == 0 || ny == 0 || nz == 0)
        return CPMAP_EINVAL;
    if (!finite_pos(bin_size) || !finite_pos(cutoff))
        return CPMAP_EINVAL;
    const float ratio = std::ceil(cutoff / bin_size);
    if (!(ratio <= 4096.0f))
        return CPMAP_ERANGE;
    g->halo = (int32_t)ratio;
    g->bin_size = bin_size;
    g->cutoff = cutoff;
    const int32_t n[3] = {nx, ny, nz};
    const float o[3] = {ox, oy, oz};
    for (int a = 0; a < 3; ++a) {
        st = axis_bins(n[a], h, o[a], bin_size, g->halo, &g->ax[a]);
        if (st != CPMAP_OK)
            return st;
    }
    // each axis has at most 2^24 bins, so bound the first two axes' product
    // (< 2^48) before multiplying by the third
    const int64_t plane = (int64_t)g->ax[0].nb * g->ax[1].nb;
    if (plane >= (int64_t)INT32_MAX || plane * g->ax[2].nb >= (int64_t)INT32_MAX)
        return CPMAP_ERANGE;
    return CPMAP_OK;
}

namespace {

cpmap_status slot_setup(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz, float h, float ox,
                        float oy, float oz, float bs, float rc, int32_t cap, BinGeometry *g,
                        SlotLayout *S)
{
    if (n_atoms < 0 || cap < 1 || cap > CPMAP_MAX_SLOTS)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    cpmap_status st = make_bin_geometry(nx, ny, nz, h, ox, oy, oz, bs, rc, g);
    if (st != CPMAP_OK)
        return st;
    if (g->nbins() * cap >= (int64_t)INT32_MAX)
        return CPMAP_ERANGE;
    *S = slot_layout(n_atoms, *g, cap);
    return CPMAP_OK;
}

}  // namespace

}  // namespace cpmap

using namespace cpmap;

extern "C" {

int32_t cpmap_version(void) { return (0 << 16) | (1 << 8) | 0; }

const char *cpmap_status_str(int32_t status)
{
    switch (status) {
    case CPMAP_OK:
        return "ok";
    case CPMAP_EINVAL:
        return "invalid argument";
    case CPMAP_ERANGE:
        return "size or index out of range";
    case CPMAP_ENOSPC:
        return "workspace too small";
    case CPMAP_EGEOM:
        return "workspace not binned for these arguments";
    case CPMAP_EHIP:
        return "HIP launch error";
    default:
        return "unknown status";
    }
}

cpmap_status cpmap_direct(const float *atoms, int64_t n_atoms, int32_t nx, int32_t ny,
                          int32_t nz, float spacing, float ox, float oy, float oz, float *V,
                          void *stream)
{
    if (n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    cpmap_status st = check_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (st != CPMAP_OK)
        return st;
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (lat.points() == 0)
        return CPMAP_OK;
    if (V == nullptr || (n_atoms > 0 && atoms == nullptr))
        return CPMAP_EINVAL;
    if (!aligned(V, 4) || (atoms && !aligned(atoms, 16)))
        return CPMAP_EINVAL;
    g_registry.forget(V, map_bytes(nx, ny, nz));
    hipError_t e = launch_direct(reinterpret_cast<const float4 *>(atoms), n_atoms, lat, V,
                                 nullptr, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

cpmap_status cpmap_node_position(int32_t nx, int32_t ny, int32_t nz, float spacing, float ox,
                                 float oy, float oz, int64_t index, int32_t *ijk_out,
                                 float *xyz_out)
{
    if (ijk_out == nullptr || xyz_out == nullptr)
        return CPMAP_EINVAL;
    cpmap_status st = check_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (st != CPMAP_OK)
        return st;
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (index < 0 || index >= lat.points())
        return CPMAP_ERANGE;
    const int64_t i = index % nx, j = (index / nx) % ny, k = index / ((int64_t)nx * ny);
    const int64_t c[3] = {i, j, k};
    for (int a = 0; a < 3; ++a) {
        ijk_out[a] = (int32_t)c[a];
        xyz_out[a] = node_coord(c[a], spacing, lat.o[a]);
    }
    return CPMAP_OK;
}

size_t cpmap_direct_workspace_bytes(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz)
{
    if (n_atoms < 0 || n_atoms > CPMAP_MAX_ATOMS)
        return 0;
    if (check_lattice(nx, ny, nz, 1.0f, 0.0f, 0.0f, 0.0f) != CPMAP_OK)
        return 0;
    return direct_workspace_bytes(n_atoms, make_lattice(nx, ny, nz, 1.0f, 0.0f, 0.0f, 0.0f));
}

cpmap_status cpmap_direct_with_workspace(const float *atoms, int64_t n_atoms, int32_t nx,
                                         int32_t ny, int32_t nz, float spacing, float ox,
                                         float oy, float oz, float *V, void *workspace,
                                         size_t workspace_bytes, void *stream)
{
    if (n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    cpmap_status st = check_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (st != CPMAP_OK)
        return st;
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (lat.points() == 0)
        return CPMAP_OK;
    if (V == nullptr || (n_atoms > 0 && atoms == nullptr))
        return CPMAP_EINVAL;
    if (!aligned(V, 4) || (atoms && !aligned(atoms, 16)))
        return CPMAP_EINVAL;
    const size_t need = direct_workspace_bytes(n_atoms, lat);
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 256)))
        return CPMAP_EINVAL;
    if (workspace_bytes < need)
        return CPMAP_ENOSPC;
    g_registry.forget(V, map_bytes(nx, ny, nz));
    if (need > 0)
        g_registry.forget(workspace, need);
    hipError_t e = launch_direct(reinterpret_cast<const float4 *>(atoms), n_atoms, lat, V,
                                 need > 0 ? workspace : nullptr, workspace_bytes,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

cpmap_status cpmap_direct_plan(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                               int32_t with_workspace, int32_t *plan_out)
{
    if (plan_out == nullptr || n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    cpmap_status st = check_lattice(nx, ny, nz, 1.0f, 0.0f, 0.0f, 0.0f);
    if (st != CPMAP_OK)
        return st;
    direct_plan(n_atoms, make_lattice(nx, ny, nz, 1.0f, 0.0f, 0.0f, 0.0f), with_workspace != 0,
                plan_out);
    return CPMAP_OK;
}

int32_t cpmap_direct_occupancy_check(void) { return direct_occupancy_mismatches(); }

cpmap_status cpmap_bin_grid(int32_t nx, int32_t ny, int32_t nz, float spacing, float ox, float oy,
                            float oz, float bin_size, float cutoff, int32_t *dims_out)
{
    if (dims_out == nullptr)
        return CPMAP_EINVAL;
    BinGeometry g;
    cpmap_status st = make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g);
    if (st != CPMAP_OK)
        return st;
    for (int a = 0; a < 3; ++a)
        dims_out[a] = g.ax[a].nb;
    return CPMAP_OK;
}

size_t cpmap_bin_workspace_bytes(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                                 float spacing, float ox, float oy, float oz, float bin_size,
                                 float cutoff)
{
    if (n_atoms < 0 || n_atoms > CPMAP_MAX_ATOMS)
        return 0;
    BinGeometry g;
    if (make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g) != CPMAP_OK)
        return 0;
    return bin_layout(n_atoms, g).total;
}

cpmap_status cpmap_workspace_layout(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                                    float spacing, float ox, float oy, float oz, float bin_size,
                                    float cutoff, int64_t *bin_start_offset,
                                    int64_t *sorted_offset)
{
    if (bin_start_offset)
        *bin_start_offset = -1;
    if (sorted_offset)
        *sorted_offset = -1;
    if (bin_start_offset == nullptr || sorted_offset == nullptr || n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    BinGeometry g;
    cpmap_status st = make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g);
    if (st != CPMAP_OK)
        return st;
    const BinLayout L = bin_layout(n_atoms, g);
    *bin_start_offset = (int64_t)L.bin_start;
    *sorted_offset = (int64_t)L.sorted;
    return CPMAP_OK;
}

cpmap_status cpmap_bin_atoms(const float *atoms, int64_t n_atoms, int32_t nx, int32_t ny,
                             int32_t nz, float spacing, float ox, float oy, float oz,
                             float bin_size, float cutoff, void *workspace,
                             size_t workspace_bytes, void *stream)
{
    if (n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    BinGeometry g;
    cpmap_status st = make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g);
    if (st != CPMAP_OK)
        return st;
    if (workspace == nullptr || (n_atoms > 0 && atoms == nullptr))
        return CPMAP_EINVAL;
    if (!aligned(workspace, 256) || (atoms && !aligned(atoms, 16)))
        return CPMAP_EINVAL;
    const BinLayout L = bin_layout(n_atoms, g);
    if (workspace_bytes < L.total)
        return CPMAP_ENOSPC;
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    const uint64_t nonce =
        g_registry.record(workspace, L.total, kBinnedWorkspace,
                          make_key(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff));
    hipError_t e = launch_bin_atoms(reinterpret_cast<const float4 *>(atoms), n_atoms, lat, g, L,
                                    workspace, nonce, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_registry.forget(workspace, L.total);
        return CPMAP_EHIP;
    }
    return CPMAP_OK;
}

cpmap_status cpmap_cutoff_term(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                               int32_t nx, int32_t ny, int32_t nz, float spacing, float ox,
                               float oy, float oz, float bin_size, float cutoff, int32_t term,
                               float *V, void *stream)
{
    if (n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    if (term != CPMAP_TERM_SMOOTHED && term != CPMAP_TERM_TRUNCATED)
        return CPMAP_EINVAL;
    BinGeometry g;
    cpmap_status st = make_bin_geometry(nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, &g);
    if (st != CPMAP_OK)
        return st;
    if (workspace == nullptr || V == nullptr)
        return CPMAP_EINVAL;
    if (!aligned(workspace, 256) || !aligned(V, 4))
        return CPMAP_EINVAL;
    const BinLayout L = bin_layout(n_atoms, g);
    if (workspace_bytes < L.total)
        return CPMAP_ENOSPC;
    const uint64_t nonce =
        g_registry.find(workspace, L.total, kBinnedWorkspace,
                        make_key(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff));
    if (nonce == 0)
        return CPMAP_EGEOM;
    g_registry.forget(V, map_bytes(nx, ny, nz));
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    hipError_t e = launch_cutoff(workspace, L, n_atoms, lat, g, term, nonce, V,
                                 static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

cpmap_status cpmap_cutoff(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                          int32_t nx, int32_t ny, int32_t nz, float spacing, float ox, float oy,
                          float oz, float bin_size, float cutoff, float *V, void *stream)
{
    return cpmap_cutoff_term(workspace, workspace_bytes, n_atoms, nx, ny, nz, spacing, ox, oy, oz,
                             bin_size, cutoff, CPMAP_TERM_SMOOTHED, V, stream);
}

size_t cpmap_slot_workspace_bytes(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                                  float spacing, float ox, float oy, float oz, float bin_size,
                                  float cutoff, int32_t capacity)
{
    BinGeometry g;
    SlotLayout S;
    if (slot_setup(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity, &g, &S) !=
        CPMAP_OK)
        return 0;
    return S.total;
}

cpmap_status cpmap_slot_layout(int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                               float spacing, float ox, float oy, float oz, float bin_size,
                               float cutoff, int32_t capacity, int64_t *slots_offset,
                               int64_t *over_start_offset, int64_t *over_atoms_offset)
{
    int64_t *outs[3] = {slots_offset, over_start_offset, over_atoms_offset};
    for (int64_t *o : outs)
        if (o)
            *o = -1;
    for (int64_t *o : outs)
        if (o == nullptr)
            return CPMAP_EINVAL;
    BinGeometry g;
    SlotLayout S;
    cpmap_status st =
        slot_setup(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity, &g, &S);
    if (st != CPMAP_OK)
        return st;
    *slots_offset = (int64_t)S.slots;
    *over_start_offset = (int64_t)S.over_start;
    *over_atoms_offset = (int64_t)S.over_atoms;
    return CPMAP_OK;
}

cpmap_status cpmap_bin_slots(const void *workspace, size_t workspace_bytes, int64_t n_atoms,
                             int32_t nx, int32_t ny, int32_t nz, float spacing, float ox,
                             float oy, float oz, float bin_size, float cutoff, int32_t capacity,
                             void *slot_workspace, size_t slot_workspace_bytes, void *stream)
{
    BinGeometry g;
    SlotLayout S;
    cpmap_status st =
        slot_setup(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity, &g, &S);
    if (st != CPMAP_OK)
        return st;
    if (workspace == nullptr || slot_workspace == nullptr)
        return CPMAP_EINVAL;
    if (!aligned(workspace, 256) || !aligned(slot_workspace, 256))
        return CPMAP_EINVAL;
    const BinLayout L = bin_layout(n_atoms, g);
    if (workspace_bytes < L.total || slot_workspace_bytes < S.total)
        return CPMAP_ENOSPC;
    if (overlaps(workspace, L.total, slot_workspace, S.total))
        return CPMAP_EINVAL;
    const uint64_t bin_nonce =
        g_registry.find(workspace, L.total, kBinnedWorkspace,
                        make_key(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff));
    if (bin_nonce == 0)
        return CPMAP_EGEOM;
    const uint64_t slot_nonce = g_registry.record(
        slot_workspace, S.total, kSlotWorkspace,
        make_key(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity));
    hipError_t e = launch_bin_slots(workspace, L, n_atoms, g, capacity, bin_nonce, slot_workspace,
                                    S, slot_nonce, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        g_registry.forget(slot_workspace, S.total);
        return CPMAP_EHIP;
    }
    return CPMAP_OK;
}

cpmap_status cpmap_cutoff_slots(const void *slot_workspace, size_t slot_workspace_bytes,
                                int64_t n_atoms, int32_t nx, int32_t ny, int32_t nz,
                                float spacing, float ox, float oy, float oz, float bin_size,
                                float cutoff, int32_t capacity, int32_t term, float *V,
                                void *stream)
{
    if (term != CPMAP_TERM_SMOOTHED && term != CPMAP_TERM_TRUNCATED)
        return CPMAP_EINVAL;
    BinGeometry g;
    SlotLayout S;
    cpmap_status st =
        slot_setup(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity, &g, &S);
    if (st != CPMAP_OK)
        return st;
    if (slot_workspace == nullptr || V == nullptr)
        return CPMAP_EINVAL;
    if (!aligned(slot_workspace, 256) || !aligned(V, 4))
        return CPMAP_EINVAL;
    if (slot_workspace_bytes < S.total)
        return CPMAP_ENOSPC;
    const uint64_t nonce = g_registry.find(
        slot_workspace, S.total, kSlotWorkspace,
        make_key(n_atoms, nx, ny, nz, spacing, ox, oy, oz, bin_size, cutoff, capacity));
    if (nonce == 0)
        return CPMAP_EGEOM;
    g_registry.forget(V, map_bytes(nx, ny, nz));
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    hipError_t e = launch_cutoff_slots(slot_workspace, S, n_atoms, lat, g, capacity, term, nonce,
                                       V, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

cpmap_status cpmap_direct_scatter(const float *atoms, int64_t n_atoms, int32_t nx, int32_t ny,
                                  int32_t nz, float spacing, float ox, float oy, float oz,
                                  float *V, void *stream)
{
    if (n_atoms < 0)
        return CPMAP_EINVAL;
    if (n_atoms > CPMAP_MAX_ATOMS)
        return CPMAP_ERANGE;
    cpmap_status st = check_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (st != CPMAP_OK)
        return st;
    const Lattice lat = make_lattice(nx, ny, nz, spacing, ox, oy, oz);
    if (lat.points() == 0)
        return CPMAP_OK;
    if (V == nullptr || (n_atoms > 0 && atoms == nullptr))
        return CPMAP_EINVAL;
    if (!aligned(V, 4) || (atoms && !aligned(atoms, 16)))
        return CPMAP_EINVAL;
    g_registry.forget(V, map_bytes(nx, ny, nz));
    hipError_t e = launch_scatter(reinterpret_cast<const float4 *>(atoms), n_atoms, lat, V,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

size_t cpmap_extrema_workspace_bytes(int64_t n)
{
    if (n < 0 || n > CPMAP_MAX_POINTS)
        return 0;
    return extrema_workspace_bytes(n);
}

cpmap_status cpmap_extrema(const float *V, int64_t n, int64_t *out_index, float *out_value,
                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (n < 0)
        return CPMAP_EINVAL;
    if (n > CPMAP_MAX_POINTS)
        return CPMAP_ERANGE;
    if ((n > 0 && V == nullptr) || out_index == nullptr || out_value == nullptr ||
        workspace == nullptr)
        return CPMAP_EINVAL;
    if (!aligned(V, 4) || !aligned(out_index, 8) || !aligned(out_value, 4) ||
        !aligned(workspace, 256))
        return CPMAP_EINVAL;
    if (workspace_bytes < extrema_workspace_bytes(n))
        return CPMAP_ENOSPC;
    g_registry.forget(out_index, 2 * sizeof(int64_t));
    g_registry.forget(out_value, 2 * sizeof(float));
    g_registry.forget(workspace, extrema_workspace_bytes(n));
    hipError_t e = launch_extrema(V, n, out_index, out_value, workspace,
                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

cpmap_status cpmap_extrema_noalloc(const float *V, int64_t n, int64_t *out_index,
                                   float *out_value, void *stream)
{
    if (n < 0)
        return CPMAP_EINVAL;
    if (n > CPMAP_MAX_POINTS)
        return CPMAP_ERANGE;
    if ((n > 0 && V == nullptr) || out_index == nullptr || out_value == nullptr)
        return CPMAP_EINVAL;
    if (!aligned(V, 4) || !aligned(out_index, 8) || !aligned(out_value, 4))
        return CPMAP_EINVAL;
    if (extrema_workspace_bytes(n) > extrema_static_scratch_bytes())
        return CPMAP_ERANGE;
    // the scratch is the current device's copy: the stream must run there
    int current = 0;
    if (hipGetDevice(&current) != hipSuccess)
        return CPMAP_EHIP;
    if (stream != nullptr) {
        hipDevice_t owner = 0;
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &owner) != hipSuccess)
            return CPMAP_EHIP;
        if ((int)owner != current)
            return CPMAP_EINVAL;
    }
    g_registry.forget(out_index, 2 * sizeof(int64_t));
    g_registry.forget(out_value, 2 * sizeof(float));
    hipError_t e =
        launch_extrema_static(V, n, out_index, out_value, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? CPMAP_OK : CPMAP_EHIP;
}

}  // extern "C"
