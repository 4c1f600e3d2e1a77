/* A C99 program against include/cpmap.h: the header must compile as plain C
 * and its host-only entry points must link and answer without a GPU. */
#include <stdio.h>
#include <string.h>

#include "cpmap.h"

static int fails = 0;
#define CHECK(cond)                                                          \
    do {                                                                     \
        if (!(cond)) {                                                       \
            printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #cond);            \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

int main(void)
{
    int32_t spans[4 * 64];
    int64_t n;
    CHECK(cpmap_version() > 0);
    CHECK(cpmap_status_str(CPMAP_OK) != NULL && strlen(cpmap_status_str(CPMAP_EINVAL)) > 0);
    CHECK(cpmap_bin_workspace_bytes(100000, 200, 200, 200, 0.5f, 0.f, 0.f, 0.f, 4.f, 12.f) > 0);
    CHECK(cpmap_bin_workspace_bytes(-1, 200, 200, 200, 0.5f, 0.f, 0.f, 0.f, 4.f, 12.f) == 0);
    /* argument checks answer on the host before any HIP call */
    CHECK(cpmap_direct(NULL, 10, 4, 4, 4, 0.5f, 0.f, 0.f, 0.f, NULL, NULL) == CPMAP_EINVAL);
    /* a lattice with a zero dimension is a documented no-op */
    CHECK(cpmap_direct(NULL, 0, 0, 4, 4, 0.5f, 0.f, 0.f, 0.f, NULL, NULL) == CPMAP_OK);
    CHECK(cpmap_direct(NULL, 0, 4, 4, 4, -0.5f, 0.f, 0.f, 0.f, NULL, NULL) == CPMAP_EINVAL);
    n = cpmap_neighbor_spans(200, 200, 200, 0.5f, 0.f, 0.f, 0.f, 4.f, 12.f, CPMAP_TERM_SMOOTHED, 10, 10, 10, spans, 64);
    CHECK(n == 48);
    CHECK(cpmap_neighbor_spans(200, 200, 200, 0.5f, 0.f, 0.f, 0.f, 4.f, 12.f, CPMAP_TERM_SMOOTHED, 25, 0, 0, spans, 64) == -1);
    if (fails == 0)
        printf("ok\n");
    return fails != 0;
}
