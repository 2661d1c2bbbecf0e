/*
 * One layer through the libssdscan C ABI from a plain C program (no Python): device
 * buffers from the HIP runtime, ssd_chunk_scan_fwd, and the result checked against the
 * fp64 CPU oracle (oracle_seq, the token-by-token recurrence of [分块推理 §2] of the page
 * "分块推理：解锁循环模型并行计算，实现长序列高效处理").  Test infrastructure: it links the
 * oracle, which the library itself never does.
 *
 * Exit status 0 when y and final_state are within the bf16 tolerance (max-abs error
 * normalised by the reference's max-abs <= 2e-2) and the argument checks behave.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "libssdscan.h"

int oracle_seq(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, const double *x,
               const double *dt, const double *A, const double *B, const double *C, const double *D,
               const double *init, double *y, double *final_state, int nthreads);

#define CHECK_HIP(e)                                                                   \
    do {                                                                               \
        hipError_t err_ = (e);                                                         \
        if (err_ != hipSuccess) {                                                      \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(err_), __LINE__); \
            return 2;                                                                  \
        }                                                                              \
    } while (0)

static uint64_t rng_state = 88172645463325252ull;
static double uniform(void) {            /* xorshift64, in (0, 1) */
    rng_state ^= rng_state << 13;
    rng_state ^= rng_state >> 7;
    rng_state ^= rng_state << 17;
    return ((rng_state >> 11) + 0.5) * (1.0 / 9007199254740992.0);
}
static double normal(void) {             /* Box-Muller */
    const double u = uniform(), v = uniform();
    return sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v);
}

/* float -> bfloat16 bits, round to nearest even (inputs are finite) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static double from_bf16(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* fill a bf16 tensor and its exact decoded values */
static void fill_bf16(uint16_t *h, double *d, size_t n, double scale, double shift, int kind) {
    for (size_t i = 0; i < n; ++i) {
        double v = kind == 0 ? normal() * scale : shift + uniform() * scale;
        h[i] = to_bf16((float)v);
        d[i] = from_bf16(h[i]);
    }
}

static double max_abs(const double *a, size_t n) {
    double m = 0;
    for (size_t i = 0; i < n; ++i) m = fabs(a[i]) > m ? fabs(a[i]) : m;
    return m;
}

int main(void) {
    const int64_t b = 2, L = 3 * 256 + 40, H = 4, P = 64, N = 128, G = 2;
    const int32_t Q = 256;
    const size_t nx = (size_t)(b * L * H * P), ndt = (size_t)(b * L * H), nbc = (size_t)(b * L * G * N);
    const size_t ns = (size_t)(b * H * P * N);
    uint16_t *hx = malloc(nx * 2), *hdt = malloc(ndt * 2), *hB = malloc(nbc * 2), *hC = malloc(nbc * 2);
    uint16_t *hy = malloc(nx * 2);
    double *dx = malloc(nx * 8), *ddt = malloc(ndt * 8), *dB = malloc(nbc * 8), *dC = malloc(nbc * 8);
    double *yref = malloc(nx * 8), *fref = malloc(ns * 8), *dinit = malloc(ns * 8);
    float A[4], D[4], *finit = malloc(ns * 4), *fout = malloc(ns * 4);
    double dA[4], dD[4];
    if (!hx || !hdt || !hB || !hC || !hy || !dx || !ddt || !dB || !dC || !yref || !fref || !dinit || !finit || !fout)
        return 2;
    fill_bf16(hx, dx, nx, 1.0, 0.0, 0);
    fill_bf16(hdt, ddt, ndt, 0.09, 0.01, 1);                 /* dt in [0.01, 0.1] */
    fill_bf16(hB, dB, nbc, 1.0 / sqrt((double)N), 0.0, 0);
    fill_bf16(hC, dC, nbc, 1.0 / sqrt((double)N), 0.0, 0);
    for (int h = 0; h < H; ++h) {
        A[h] = -(float)exp(uniform() * log(16.0));
        D[h] = (float)uniform();
        dA[h] = A[h];
        dD[h] = D[h];
    }
    for (size_t i = 0; i < ns; ++i) {
        finit[i] = (float)(0.3 * normal());
        dinit[i] = finit[i];
    }

    ssd_dims_t dims = {b, L, H, P, N, G, SSD_BF16, 0};
    const size_t wsb = ssd_chunk_scan_workspace_bytes(&dims, Q);
    if (wsb == 0) { fprintf(stderr, "workspace query failed: %s\n", ssd_last_error_message()); return 1; }

    void *x, *dt, *B, *C, *y, *ws;
    float *Ad, *Dd, *init, *fin;
    CHECK_HIP(hipMalloc(&x, nx * 2));
    CHECK_HIP(hipMalloc(&dt, ndt * 2));
    CHECK_HIP(hipMalloc(&B, nbc * 2));
    CHECK_HIP(hipMalloc(&C, nbc * 2));
    CHECK_HIP(hipMalloc(&y, nx * 2));
    CHECK_HIP(hipMalloc(&ws, wsb));
    CHECK_HIP(hipMalloc((void **)&Ad, sizeof(A)));
    CHECK_HIP(hipMalloc((void **)&Dd, sizeof(D)));
    CHECK_HIP(hipMalloc((void **)&init, ns * 4));
    CHECK_HIP(hipMalloc((void **)&fin, ns * 4));
    CHECK_HIP(hipMemcpy(x, hx, nx * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dt, hdt, ndt * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(B, hB, nbc * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(C, hC, nbc * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(Ad, A, sizeof(A), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(Dd, D, sizeof(D), hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(init, finit, ns * 4, hipMemcpyHostToDevice));

    /* argument checks run on the host and write nothing */
    if (ssd_chunk_scan_fwd(&dims, NULL, dt, Ad, B, C, Dd, init, Q, y, fin, 0, ws, wsb, NULL) != SSD_ERR_NULL_ARG ||
        ssd_last_error_message()[0] == 0) {
        fprintf(stderr, "null x not rejected\n");
        return 1;
    }
    if (ssd_chunk_scan_fwd(&dims, x, dt, Ad, B, C, Dd, init, Q, y, fin, 0, ws, wsb / 2, NULL) != SSD_ERR_WORKSPACE) {
        fprintf(stderr, "short workspace not rejected\n");
        return 1;
    }

    ssd_status_t st = ssd_chunk_scan_fwd(&dims, x, dt, Ad, B, C, Dd, init, Q, y, fin, 0, ws, wsb, NULL);
    if (st != SSD_OK) { fprintf(stderr, "%s: %s\n", ssd_status_string(st), ssd_last_error_message()); return 1; }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hy, y, nx * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(fout, fin, ns * 4, hipMemcpyDeviceToHost));

    if (oracle_seq(b, L, H, P, N, G, dx, ddt, dA, dB, dC, dD, dinit, yref, fref, 4) != 0) return 2;
    double ey = 0, ef = 0;
    for (size_t i = 0; i < nx; ++i) ey = fmax(ey, fabs(from_bf16(hy[i]) - yref[i]));
    for (size_t i = 0; i < ns; ++i) ef = fmax(ef, fabs((double)fout[i] - fref[i]));
    ey /= max_abs(yref, nx);
    ef /= max_abs(fref, ns);
    printf("libssdscan %d from C: y err %.3e, final_state err %.3e (tolerance 2e-2)\n", ssd_version(), ey, ef);
    return (ey <= 2e-2 && ef <= 2e-2) ? 0 : 1;
}
