/*
 * Host sanitizer driver for the fp64 oracle (test infrastructure): calls every
 * oracle function on small inputs, empty inputs and atoms that binning drops,
 * so that an AddressSanitizer / UndefinedBehaviorSanitizer build reports any
 * out-of-bounds access, overflow or invalid operation.  Exits 0 when every
 * call returns the expected status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_num_threads(void);
void oracle_direct(const float *, int64_t, int32_t, int32_t, int32_t, float, float, float, float,
                   const int64_t *, int64_t, double *, double *);
void oracle_cutoff(const float *, int64_t, int32_t, int32_t, int32_t, float, float, float, float,
                   float, const int64_t *, int64_t, double *, double *);
void oracle_cutoff_hard(const float *, int64_t, int32_t, int32_t, int32_t, float, float, float,
                        float, float, const int64_t *, int64_t, double *, double *);
double oracle_smoothed_term(double, double, double);
int32_t oracle_bin_grid(int32_t, int32_t, int32_t, float, float, float, float, float, float,
                        int32_t *, float *);
int64_t oracle_bin_atoms(const float *, int64_t, int32_t, int32_t, int32_t, float, float, float,
                         float, float, float, int32_t *, float *, int32_t *);
int64_t oracle_bin_slots(const float *, int64_t, int32_t, int32_t, int32_t, float, float, float,
                         float, float, float, int32_t, float *, int32_t *, float *);
void oracle_extrema(const float *, int64_t, int64_t *, float *);

static int failures = 0;
#define CHECK(c)                                                                              \
    do {                                                                                      \
        if (!(c)) {                                                                           \
            fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__);                   \
            ++failures;                                                                       \
        }                                                                                     \
    } while (0)

int main(void)
{
    enum { N = 37 };
    float atoms[4 * N];
    for (int a = 0; a < N; ++a) {
        atoms[4 * a + 0] = -3.0f + 0.37f * (float)a;
        atoms[4 * a + 1] = 1.5f - 0.11f * (float)a;
        atoms[4 * a + 2] = 0.05f * (float)(a * a % 17);
        atoms[4 * a + 3] = (a % 3 == 0) ? 0.0f : ((a % 2) ? 0.5f : -0.75f);
    }
    atoms[4 * 5 + 0] = NAN;      /* dropped by binning */
    atoms[4 * 6 + 1] = 1.0e30f;  /* far outside the bin grid */

    const int32_t nx = 7, ny = 5, nz = 3;
    const int64_t np = (int64_t)nx * ny * nz;
    double *V = malloc(sizeof(double) * np), *S = malloc(sizeof(double) * np);
    int64_t nodes[4] = {0, 3, np / 2, np - 1};

    CHECK(oracle_num_threads() >= 1);
    /* direct and cutoffs over all nodes, a node list, and no atoms (atoms 5
     * and 6 are left out: NaN and 1e30 coordinates are outside the domain) */
    const float *clean = atoms + 4 * 7;
    const int64_t nclean = N - 7;
    oracle_direct(clean, nclean, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, NULL, np, V, S);
    oracle_direct(clean, nclean, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, nodes, 4, V, S);
    oracle_direct(clean, 0, nx, ny, nz, 0.5f, 0.0f, 0.0f, 0.0f, NULL, np, V, S);
    CHECK(V[0] == 0.0 && S[0] == 0.0);
    oracle_cutoff(clean, nclean, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 2.5f, NULL, np, V, S);
    oracle_cutoff(clean, nclean, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 2.5f, nodes, 4, V, S);
    oracle_cutoff_hard(clean, nclean, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 2.5f, NULL, np, V, S);
    CHECK(oracle_smoothed_term(1.0, 12.0, 12.0) == 0.0);
    CHECK(oracle_smoothed_term(1.0, 6.0, 12.0) > 0.0);

    /* binning: geometry, CSR, fixed-capacity slots (all atoms, NaN included) */
    int32_t dims[3];
    float b0[3];
    CHECK(oracle_bin_grid(nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 1.0f, 2.5f, dims, b0) == 3);
    CHECK(oracle_bin_grid(0, ny, nz, 0.5f, 0.0f, 0.0f, 0.0f, 1.0f, 2.5f, dims, b0) < 0);
    CHECK(oracle_bin_grid(nx, ny, nz, 0.5f, 0.0f, 0.0f, 0.0f, 0.0f, 2.5f, dims, b0) < 0);
    oracle_bin_grid(nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 1.0f, 2.5f, dims, b0);
    const int64_t nbins = (int64_t)dims[0] * dims[1] * dims[2];
    int32_t *starts = malloc(sizeof(int32_t) * (nbins + 1));
    float *sorted = malloc(sizeof(float) * 4 * N);
    int32_t *bin_of = malloc(sizeof(int32_t) * N);
    const int64_t kept = oracle_bin_atoms(atoms, N, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 1.0f,
                                          2.5f, starts, sorted, bin_of);
    CHECK(kept >= 0 && kept <= N - 2 && bin_of[5] == -1 && bin_of[6] == -1);
    CHECK(oracle_bin_atoms(atoms, 0, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 1.0f, 2.5f, starts,
                           sorted, NULL) == 0);
    for (int32_t cap = 1; cap <= 9; cap += 4) {
        float *slots = malloc(sizeof(float) * 4 * nbins * cap);
        float *over = malloc(sizeof(float) * 4 * N);
        const int64_t n_over = oracle_bin_slots(atoms, N, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f,
                                                1.0f, 2.5f, cap, slots, starts, over);
        CHECK(n_over >= 0 && n_over <= kept);
        free(slots);
        free(over);
    }
    CHECK(oracle_bin_slots(atoms, N, nx, ny, nz, 0.5f, -1.0f, 0.0f, 2.0f, 1.0f, 2.5f, 0, NULL,
                           starts, NULL) < 0);

    /* extrema: NaN skipped, empty and all-NaN maps */
    float map[6] = {1.0f, NAN, -2.0f, 3.0f, -2.0f, 3.0f};
    int64_t idx[2];
    float val[2];
    oracle_extrema(map, 6, idx, val);
    CHECK(idx[0] == 2 && idx[1] == 3);
    oracle_extrema(map, 0, idx, val);
    CHECK(idx[0] == -1 && idx[1] == -1);
    oracle_extrema(map + 1, 1, idx, val);
    CHECK(idx[0] == -1);

    free(V);
    free(S);
    free(starts);
    free(sorted);
    free(bin_of);
    if (failures)
        return 1;
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
