/*
 * Round trip through the C ABI alone (no Python, no torch): build the maps of
 * a seeded uniform system, run the coordinate and force passes in every
 * execution mode, and compare every slot bit for bit with the CPU oracle
 * (test infrastructure, linked only here). The staged exchange follows the
 * NVIDIA guide "A Practical Guide to GPU-Initiated Communication for
 * Molecular Dynamics at Scale".
 *
 * Usage: c_abi_roundtrip [n_atoms nx ny nz box rc]   (exit status 0: all equal)
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ddh.h"

/* the oracle's C entry points (oracle/ddh_oracle.c) */
int ddho_build(const float *xg, int n_atoms, const int ndom[3], const float box[3], float rc,
               float cell, void **out);
int64_t ddho_nslots(const void *h);
void ddho_coords(const void *h, float *out);
void ddho_exchange_forces(const void *h, float *ff, int nthreads);
void ddho_free(void *h);

/* seeded inputs: a 64-bit linear congruential generator, top 31 bits */
static uint64_t lcg = 20261202u;
static double uniform01(void)
{
    lcg = lcg * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(lcg >> 33) / 2147483648.0;
}

#define HIP_OK(call)                                                           \
    do {                                                                       \
        hipError_t e_ = (call);                                                \
        if (e_ != hipSuccess) {                                                \
            fprintf(stderr, "%s: %s\n", #call, hipGetErrorString(e_));         \
            return 2;                                                          \
        }                                                                      \
    } while (0)

#define DDH_OK_OR_FAIL(call)                                                   \
    do {                                                                       \
        int r_ = (call);                                                       \
        if (r_ != DDH_OK) {                                                    \
            fprintf(stderr, "%s: %d (%s)\n", #call, r_, ddh_last_error());     \
            return 3;                                                          \
        }                                                                      \
    } while (0)

static int64_t differing(const float *a, const float *b, int64_t n)
{
    int64_t bad = 0;
    for (int64_t i = 0; i < n; i++)
        if (memcmp(a + i, b + i, sizeof(float)) != 0)
            bad++;
    return bad;
}

int main(int argc, char **argv)
{
    int n = 20000, ndom[3] = {2, 2, 2};
    float box = 6.0f, rc = 1.0f;
    if (argc == 7) {
        n = atoi(argv[1]);
        ndom[0] = atoi(argv[2]);
        ndom[1] = atoi(argv[3]);
        ndom[2] = atoi(argv[4]);
        box = (float)atof(argv[5]);
        rc = (float)atof(argv[6]);
    }
    const float L[3] = {box, box, box};
    float *xg = (float *)malloc(sizeof(float) * 3 * (size_t)(n > 0 ? n : 1));
    for (int i = 0; i < 3 * n; i++) {
        float v = (float)(uniform01() * box);
        xg[i] = v < box ? v : 0.0f;
    }

    /* oracle */
    void *ref = NULL;
    if (ddho_build(xg, n, ndom, L, rc, 0.5f, &ref) != 0) {
        fprintf(stderr, "oracle build failed\n");
        return 4;
    }
    const int64_t ns = ddho_nslots(ref);
    float *x_ref = (float *)malloc(sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1));
    float *f_ref = (float *)malloc(sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1));
    float *f0 = (float *)malloc(sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1));
    float *out = (float *)malloc(sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1));
    ddho_coords(ref, x_ref);
    for (int64_t i = 0; i < 3 * ns; i++)
        f0[i] = (float)(20.0 * uniform01() - 10.0);
    memcpy(f_ref, f0, sizeof(float) * 3 * (size_t)ns);
    ddho_exchange_forces(ref, f_ref, 1);

    /* library */
    ddh_params prm;
    memset(&prm, 0, sizeof(prm));
    for (int d = 0; d < 3; d++) {
        prm.ndom[d] = ndom[d];
        prm.box[d] = L[d];
    }
    prm.rc = rc;
    prm.cell = 0.5f;
    ddh_plan *plan = NULL;
    DDH_OK_OR_FAIL(ddh_plan_create(&prm, &plan));
    float *d_xg = NULL, *d_x = NULL, *d_f = NULL;
    HIP_OK(hipMalloc((void **)&d_xg, sizeof(float) * 3 * (size_t)(n > 0 ? n : 1)));
    HIP_OK(hipMemcpy(d_xg, xg, sizeof(float) * 3 * (size_t)n, hipMemcpyHostToDevice));
    DDH_OK_OR_FAIL(ddh_build_maps(plan, d_xg, n, NULL));
    ddh_layout lay;
    DDH_OK_OR_FAIL(ddh_query(plan, &lay));
    if (lay.n_slots != ns) {
        fprintf(stderr, "slot count %lld, oracle %lld\n", (long long)lay.n_slots, (long long)ns);
        return 5;
    }
    HIP_OK(hipMalloc((void **)&d_x, sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1)));
    HIP_OK(hipMalloc((void **)&d_f, sizeof(float) * 3 * (size_t)(ns > 0 ? ns : 1)));

    const int32_t modes[] = {DDH_MODE_FUSED, DDH_MODE_PULSE, DDH_MODE_AUTO, DDH_MODE_STAGED,
                             DDH_MODE_PULSE | DDH_MODE_GRAPH, DDH_MODE_FUSED | DDH_MODE_GRAPH};
    int failures = 0;
    for (size_t m = 0; m < sizeof(modes) / sizeof(modes[0]); m++) {
        DDH_OK_OR_FAIL(ddh_set_mode(plan, modes[m]));
        for (int step = 0; step < 2; step++) {
            HIP_OK(hipMemset(d_x, 0, sizeof(float) * 3 * (size_t)ns));
            HIP_OK(hipMemcpy(d_f, f0, sizeof(float) * 3 * (size_t)ns, hipMemcpyHostToDevice));
            DDH_OK_OR_FAIL(ddh_gather_home(plan, d_xg, d_x, ns, NULL));
            DDH_OK_OR_FAIL(ddh_exchange_coords(plan, d_x, ns, NULL));
            DDH_OK_OR_FAIL(ddh_exchange_forces(plan, d_f, ns, NULL));
            DDH_OK_OR_FAIL(ddh_check(plan, NULL));
            HIP_OK(hipMemcpy(out, d_x, sizeof(float) * 3 * (size_t)ns, hipMemcpyDeviceToHost));
            const int64_t bx = differing(out, x_ref, 3 * ns);
            HIP_OK(hipMemcpy(out, d_f, sizeof(float) * 3 * (size_t)ns, hipMemcpyDeviceToHost));
            const int64_t bf = differing(out, f_ref, 3 * ns);
            printf("mode %d step %d: %lld slots, %lld halo; coordinate words differing %lld, "
                   "force words differing %lld\n",
                   (int)modes[m], step, (long long)ns, (long long)lay.n_halo, (long long)bx,
                   (long long)bf);
            failures += (bx != 0) + (bf != 0);
        }
    }
    ddh_plan_destroy(plan);
    HIP_OK(hipFree(d_xg));
    HIP_OK(hipFree(d_x));
    HIP_OK(hipFree(d_f));
    ddho_free(ref);
    free(xg);
    free(x_ref);
    free(f_ref);
    free(f0);
    free(out);
    if (failures) {
        printf("FAILED: %d comparisons differ\n", failures);
        return 1;
    }
    printf("all modes bit-identical to the oracle\n");
    return 0;
}
