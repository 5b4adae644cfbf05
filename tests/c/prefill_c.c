/* A plain C caller of gdn_prefill: bf16 inputs built on the host, device
 * memory and the workspace from the HIP C API.  The chunked prefill must agree
 * with gdn_record on the same inputs (to the bf16 tolerance, 2e-2 scaled), and
 * a workspace one byte short must be refused before any launch. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "gdn.h"

enum { B = 1, T = 70, HK = 1, HV = 2, DK = 128, DV = 16 };

static float frand(unsigned* s) {
    *s = *s * 1664525u + 1013904223u;
    return ((float)(*s >> 8) / 16777216.0f) - 0.5f;
}

/* float -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

static double from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

#define CHECK(x) do { if ((x) != hipSuccess) { printf("hip error at %d\n", __LINE__); return 10; } } while (0)

int main(void) {
    const size_t nqk = (size_t)B * T * HK * DK, nv = (size_t)B * T * HV * DV, ng = (size_t)B * T * HV;
    const size_t ns = (size_t)B * HV * DV * DK;
    uint16_t *q = malloc(nqk * 2), *k = malloc(nqk * 2), *v = malloc(nv * 2), *g = malloc(ng * 2);
    uint16_t *beta = malloc(ng * 2), *y1 = malloc(nv * 2), *y2 = malloc(nv * 2);
    float *s0 = malloc(ns * 4), *s1 = malloc(ns * 4), *s2 = malloc(ns * 4);
    unsigned seed = 777u;
    for (size_t row = 0; row < nqk / DK; ++row) {             /* unit-norm keys and queries */
        float kr[DK], qr[DK], nk = 0.f, nq = 0.f;
        for (int e = 0; e < DK; ++e) { kr[e] = frand(&seed); qr[e] = frand(&seed); nk += kr[e] * kr[e]; nq += qr[e] * qr[e]; }
        for (int e = 0; e < DK; ++e) { k[row * DK + e] = to_bf16(kr[e] / sqrtf(nk)); q[row * DK + e] = to_bf16(qr[e] / sqrtf(nq)); }
    }
    for (size_t i = 0; i < nv; ++i) v[i] = to_bf16(2.0f * frand(&seed));
    for (size_t i = 0; i < ng; ++i) { g[i] = to_bf16(0.75f + 0.4f * frand(&seed)); beta[i] = to_bf16(0.5f + frand(&seed)); }
    for (size_t i = 0; i < ns; ++i) s0[i] = 0.2f * frand(&seed);

    const uint64_t wsb = gdn_prefill_workspace_size(B, T, HV);
    void *dq, *dk, *dv, *dg, *db, *ds0, *dy1, *dy2, *ds1, *ds2, *dws;
    CHECK(hipMalloc(&dq, nqk * 2)); CHECK(hipMalloc(&dk, nqk * 2)); CHECK(hipMalloc(&dv, nv * 2));
    CHECK(hipMalloc(&dg, ng * 2)); CHECK(hipMalloc(&db, ng * 2)); CHECK(hipMalloc(&ds0, ns * 4));
    CHECK(hipMalloc(&dy1, nv * 2)); CHECK(hipMalloc(&dy2, nv * 2)); CHECK(hipMalloc(&ds1, ns * 4));
    CHECK(hipMalloc(&ds2, ns * 4)); CHECK(hipMalloc(&dws, wsb));
    CHECK(hipMemcpy(dq, q, nqk * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dk, k, nqk * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dv, v, nv * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dg, g, ng * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(db, beta, ng * 2, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(ds0, s0, ns * 4, hipMemcpyHostToDevice));

    int rc = gdn_prefill(dq, dk, dv, dg, db, ds0, NULL, dy1, ds1, NULL, NULL, NULL, dws, wsb - 1,
                         B, T, HK, HV, DK, DV, GDN_BF16, GDN_GQA_BLOCK, NULL);
    if (rc != GDN_ERR_WORKSPACE) { printf("short workspace accepted (%d)\n", rc); return 11; }
    rc = gdn_prefill(dq, dk, dv, dg, db, ds0, NULL, dy1, ds1, NULL, NULL, NULL, dws, wsb,
                     B, T, HK, HV, DK, DV, GDN_BF16, GDN_GQA_BLOCK, NULL);
    if (rc != GDN_OK) { printf("gdn_prefill: %s\n", gdn_last_error()); return 12; }
    rc = gdn_record(dq, dk, dv, dg, db, ds0, NULL, dy2, ds2, NULL, NULL, NULL,
                    B, T, HK, HV, DK, DV, GDN_BF16, GDN_GQA_BLOCK, NULL);
    if (rc != GDN_OK) { printf("gdn_record: %s\n", gdn_last_error()); return 13; }
    CHECK(hipDeviceSynchronize());
    CHECK(hipMemcpy(y1, dy1, nv * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(y2, dy2, nv * 2, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(s1, ds1, ns * 4, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(s2, ds2, ns * 4, hipMemcpyDeviceToHost));

    double worst = 0.0;
    for (size_t i = 0; i < nv; ++i) {
        const double a = from_bf16(y1[i]), r = from_bf16(y2[i]);
        const double err = fabs(a - r) / (1.0 + fabs(r));
        if (!(err <= worst)) worst = err;                     /* NaN makes worst NaN */
    }
    for (size_t i = 0; i < ns; ++i) {
        const double err = fabs((double)s1[i] - (double)s2[i]) / (1.0 + fabs((double)s2[i]));
        if (!(err <= worst)) worst = err;
    }
    if (!(worst <= 2e-2)) { printf("prefill and record differ by %g\n", worst); return 14; }
    printf("c prefill ok (worst difference %.2e)\n", worst);
    hipFree(dq); hipFree(dk); hipFree(dv); hipFree(dg); hipFree(db); hipFree(ds0);
    hipFree(dy1); hipFree(dy2); hipFree(ds1); hipFree(ds2); hipFree(dws);
    free(q); free(k); free(v); free(g); free(beta); free(y1); free(y2); free(s0); free(s1); free(s2);
    return 0;
}
