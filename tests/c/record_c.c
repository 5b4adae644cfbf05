/* A plain C caller that runs gdn_record and gdn_replay on the GPU through the
 * C ABI, with device memory from the HIP C API.  With g = 1 and beta = 0 the
 * step leaves the state unchanged and y_t = S0 . q_t, which the program checks
 * against a host computation in double precision; the replay of the recorded
 * tape must give the recorded state back exactly. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

enum { B = 2, T = 3, HK = 1, HV = 2, DK = 32, DV = 16 };

static float frand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return ((float)(*s >> 8) / 16777216.0f) - 0.5f;
}

#define CHECK(x) do { if ((x) != hipSuccess) { printf("hip error at %d\n", __LINE__); return 10; } } while (0)

int main(void) {
    const size_t nqk = (size_t)B * T * HK * DK, nv = (size_t)B * T * HV * DV, ng = (size_t)B * T * HV;
    const size_t ns = (size_t)B * HV * DV * DK, nkl = (size_t)B * T * HV * DK;
    float *q = malloc(nqk * 4), *k = malloc(nqk * 4), *v = malloc(nv * 4), *g = malloc(ng * 4);
    float *beta = malloc(ng * 4), *s0 = malloc(ns * 4), *y = malloc(nv * 4), *s1 = malloc(ns * 4);
    float *s2 = malloc(ns * 4);
    unsigned seed = 12345u;
    for (size_t i = 0; i < nqk; ++i) { q[i] = frand(&seed); k[i] = frand(&seed); }
    for (size_t i = 0; i < nv; ++i) v[i] = frand(&seed);
    for (size_t i = 0; i < ng; ++i) { g[i] = 1.0f; beta[i] = 0.0f; }
    for (size_t i = 0; i < ns; ++i) s0[i] = frand(&seed);

    void *dq, *dk, *dv, *dg, *db, *ds0, *dy, *ds1, *ddl, *dkl, *dgl, *ds2;
    CHECK(hipMalloc(&dq, nqk * 4)); CHECK(hipMalloc(&dk, nqk * 4)); CHECK(hipMalloc(&dv, nv * 4));
    CHECK(hipMalloc(&dg, ng * 4)); CHECK(hipMalloc(&db, ng * 4)); CHECK(hipMalloc(&ds0, ns * 4));
    CHECK(hipMalloc(&dy, nv * 4)); CHECK(hipMalloc(&ds1, ns * 4)); CHECK(hipMalloc(&ddl, nv * 4));
    CHECK(hipMalloc(&dkl, nkl * 4)); CHECK(hipMalloc(&dgl, ng * 4)); CHECK(hipMalloc(&ds2, ns * 4));
    CHECK(hipMemcpy(dq, q, nqk * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dk, k, nqk * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dv, v, nv * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dg, g, ng * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, beta, ng * 4, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(ds0, s0, ns * 4, hipMemcpyHostToDevice));

    int rc = gdn_record(dq, dk, dv, dg, db, ds0, NULL, dy, ds1, ddl, dkl, dgl,
                        B, T, HK, HV, DK, DV, GDN_F32, GDN_GQA_BLOCK, NULL);
    if (rc != GDN_OK) { printf("gdn_record: %s\n", gdn_last_error()); return 11; }
    rc = gdn_replay(ddl, dkl, dgl, ds0, NULL, ds2, B, T, HV, DK, DV, T, GDN_F32, NULL);
    if (rc != GDN_OK) { printf("gdn_replay: %s\n", gdn_last_error()); return 12; }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(y, dy, nv * 4, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(s1, ds1, ns * 4, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(s2, ds2, ns * 4, hipMemcpyDeviceToHost));

    if (memcmp(s1, s0, ns * 4) != 0) { printf("state changed with g = 1, beta = 0\n"); return 13; }
    if (memcmp(s2, s1, ns * 4) != 0) { printf("replay differs from record\n"); return 14; }
    double worst = 0.0;
    for (int b = 0; b < B; ++b)
        for (int t = 0; t < T; ++t)
            for (int hv = 0; hv < HV; ++hv)
                for (int dv = 0; dv < DV; ++dv) {
                    const int hk = hv / (HV / HK);
                    double ref = 0.0;
                    for (int e = 0; e < DK; ++e)
                        ref += (double)s0[(((size_t)b * HV + hv) * DV + dv) * DK + e] *
                               (double)q[(((size_t)b * T + t) * HK + hk) * DK + e];
                    const double got = y[(((size_t)b * T + t) * HV + hv) * DV + dv];
                    const double err = fabs(got - ref) / (1.0 + fabs(ref));
                    if (err > worst) worst = err;
                }
    if (worst > 1e-5) { printf("y off by %g\n", worst); return 15; }
    printf("c gpu ok (worst y error %.2e)\n", worst);
    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dg); hipFree(db); hipFree(ds0);
    hipFree(dy); hipFree(ds1); hipFree(ddl); hipFree(dkl); hipFree(dgl); hipFree(ds2);
    free(q); free(k); free(v); free(g); free(beta); free(s0); free(y); free(s1); free(s2);
    return 0;
}
