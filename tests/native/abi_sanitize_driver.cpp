// Host sanitizer driver for libcpmap's host code (test infrastructure): calls
// every host-only query over a grid of valid, degenerate, huge and non-finite
// arguments, and every entry point with arguments its host checks reject, so
// that an AddressSanitizer / UndefinedBehaviorSanitizer build of the host
// side reports any overflow, out-of-bounds access or invalid conversion.  No
// call here reaches a kernel launch.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/cpmap.h"

static int failures = 0;
#define CHECK(c)                                                                     \
    do {                                                                             \
        if (!(c)) {                                                                  \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);     \
            ++failures;                                                              \
        }                                                                            \
    } while (0)

int main()
{
    for (int s = -1; s <= 7; ++s)
        CHECK(cpmap_status_str(s) != nullptr);
    CHECK(cpmap_version() > 0);

    const float reals[] = {NAN, INFINITY, -INFINITY, -1.0f, 0.0f, 1e-30f, 0.25f, 1.0f,
                           4.0f, 12.0f, 1e6f, 3e38f};
    const int32_t dims[] = {-1, 0, 1, 7, 200, 16777216, 16777217, INT32_MAX};
    const float origins[] = {0.0f, -5.5f, 1e30f, -1e30f, NAN};
    const int64_t counts[] = {-1, 0, 1, 63, 65, 10000, 200000, INT32_MAX, INT64_MAX};

    int32_t grid[3];
    int64_t off[3];
    for (int32_t n : dims)
        for (float h : reals)
            for (float o : origins)
                for (float bs : reals)
                    for (float rc : {0.7f, 12.0f, 1e5f, NAN}) {
                        const cpmap_status st = cpmap_bin_grid(n, 5, 3, h, o, 0, 0, bs, rc, grid);
                        if (st == CPMAP_OK)
                            CHECK(grid[0] >= 1 && grid[1] >= 1 && grid[2] >= 1);
                        (void)cpmap_bin_workspace_bytes(100, n, 5, 3, h, o, 0, 0, bs, rc);
                        (void)cpmap_workspace_layout(100, n, 5, 3, h, o, 0, 0, bs, rc, &off[0],
                                                     &off[1]);
                        for (int32_t cap : {-1, 0, 1, 8, 256, 257}) {
                            (void)cpmap_slot_workspace_bytes(100, n, 5, 3, h, o, 0, 0, bs, rc, cap);
                            (void)cpmap_slot_layout(100, n, 5, 3, h, o, 0, 0, bs, rc, cap, &off[0],
                                                    &off[1], &off[2]);
                        }
                    }
    for (int64_t na : counts)
        for (int32_t n : dims) {
            int32_t plan[5];
            const cpmap_status st = cpmap_direct_plan(na, n, 3, 2, 1, plan);
            if (st == CPMAP_OK)
                CHECK(plan[0] >= 1 && plan[3] >= 1 && plan[4] >= 1);
            (void)cpmap_direct_plan(na, n, 3, 2, 0, plan);
            (void)cpmap_direct_workspace_bytes(na, n, 3, 2);
            (void)cpmap_bin_workspace_bytes(na, n, 4, 4, 0.5f, 0, 0, 0, 4.0f, 12.0f);
            (void)cpmap_extrema_workspace_bytes(na);
        }

    // the neighbourhood of every tile of a small geometry, with short buffers
    std::vector<int32_t> spans(4 * 64);
    for (int32_t tz = -1; tz <= 3; ++tz)
        for (int32_t ty = -1; ty <= 3; ++ty)
            for (int32_t tx = -1; tx <= 3; ++tx)
                for (int64_t cap : {0, 1, 64}) {
                    const int64_t k = cpmap_neighbor_spans(20, 17, 9, 0.5f, -2.0f, 1.0f, 0.25f, 1.5f,
                                                           3.0f, (tx + ty) & 1, tx, ty, tz,
                                                           cap ? spans.data() : nullptr, cap);
                    const bool valid = tx >= 0 && ty >= 0 && tz >= 0 && tx < 3 && ty < 3 && tz < 2;
                    CHECK(valid ? k >= 0 : k == -1);
                }

    // entry points: host checks reject these before any HIP call
    float *fake = reinterpret_cast<float *>(0x1000);
    void *ws = reinterpret_cast<void *>(0x10000);
    CHECK(cpmap_direct(nullptr, 10, 8, 8, 8, 0.5f, 0, 0, 0, fake, nullptr) == CPMAP_EINVAL);
    CHECK(cpmap_direct(fake, 10, 8, 8, 8, 0.5f, 0, 0, 0, nullptr, nullptr) == CPMAP_EINVAL);
    CHECK(cpmap_direct(fake, -1, 8, 8, 8, 0.5f, 0, 0, 0, fake, nullptr) == CPMAP_EINVAL);
    CHECK(cpmap_direct(fake, 10, 0, 8, 8, 0.5f, 0, 0, 0, fake, nullptr) == CPMAP_OK);
    CHECK(cpmap_direct_with_workspace(fake, 100000, 64, 64, 64, 0.5f, 0, 0, 0, fake, ws, 1,
                                      nullptr) == CPMAP_ENOSPC ||
          cpmap_direct_workspace_bytes(100000, 64, 64, 64) <= 1);
    CHECK(cpmap_direct_scatter(nullptr, 10, 8, 8, 8, 0.5f, 0, 0, 0, fake, nullptr) ==
          CPMAP_EINVAL);
    const size_t need = cpmap_bin_workspace_bytes(100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f);
    CHECK(need > 0);
    CHECK(cpmap_bin_atoms(fake, 100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, ws, need - 1, nullptr) ==
          CPMAP_ENOSPC);
    CHECK(cpmap_cutoff(ws, need, 100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, fake, nullptr) ==
          CPMAP_EGEOM);
    CHECK(cpmap_cutoff_term(ws, need, 100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, 7, fake,
                            nullptr) == CPMAP_EINVAL);
    const size_t sneed = cpmap_slot_workspace_bytes(100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, 8);
    void *sws = reinterpret_cast<void *>(0x10000 + ((need + 255) / 256) * 256);
    CHECK(cpmap_bin_slots(ws, need, 100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, 8, sws, sneed,
                          nullptr) == CPMAP_EGEOM);
    CHECK(cpmap_cutoff_slots(sws, sneed, 100, 8, 8, 8, 0.5f, 0, 0, 0, 1.0f, 2.0f, 8, 0, fake,
                             nullptr) == CPMAP_EGEOM);
    int64_t idx[2];
    float val[2];
    CHECK(cpmap_extrema(nullptr, 10, idx, val, ws, 1 << 20, nullptr) == CPMAP_EINVAL);
    CHECK(cpmap_extrema(fake, 10, idx, val, ws, 0, nullptr) == CPMAP_ENOSPC);

    if (failures)
        return 1;
    std::printf("libcpmap host sanitizer driver: ok\n");
    return 0;
}
