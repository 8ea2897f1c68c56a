/*
 * A plain C11 program that uses the library the way a C caller would, on the
 * GPU: device buffers from the HIP runtime's C API, its own stream, the
 * entry points of include/rmsnorm.h, then the results copied back and checked
 * against properties every correct result has (no second implementation):
 *   rmsnorm_fwd (bf16, eps 0):      mean_j (y_j / w_j)^2 = 1 per row
 *   rmsnorm_residual_fwd (fp32):    h = x + residual rounded once, bit for bit,
 *                                   and the same identity for y against h
 *   rmsnorm_bwd (fp32, eps 0):      <dx, x> = 0 per row (scale invariance)
 *                                   and <dw, w> = sum of dy * y
 *   layernorm_fwd (fp32, no beta):  (y / gamma) has mean 0 and mean square 1
 * Exact parity with the oracle is the Python suite's job; this program checks
 * that the boundary works from C.  Run by tests/test_c_abi_gpu.py.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rmsnorm.h"

static int failures = 0;

#define HIP_OK(call)                                                             \
    do {                                                                         \
        hipError_t e_ = (call);                                                  \
        if (e_ != hipSuccess) {                                                  \
            printf("HIP error %d at line %d\n", (int)e_, __LINE__);              \
            exit(2);                                                             \
        }                                                                        \
    } while (0)

static void check(const char* what, int ok) {
    printf("%s %s\n", what, ok ? "ok" : "FAILED");
    if (!ok) ++failures;
}

static uint64_t state = 12345;
static float uniform(void) { /* [-1, 1) */
    state = state * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((state >> 40) & 0xFFFFFF) / 8388608.0f - 1.0f;
}
static uint16_t to_bf16(float f) { /* nearest-even; finite values */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFF + ((u >> 16) & 1)) >> 16);
}
static float from_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static void* dev_copy(const void* host, size_t n) {
    void* d = NULL;
    HIP_OK(hipMalloc(&d, n));
    HIP_OK(hipMemcpy(d, host, n, hipMemcpyHostToDevice));
    return d;
}

int main(void) {
    enum { R = 37, H = 4096, HB = 1000 };
    const size_t n = (size_t)R * H;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));

    /* rmsnorm_fwd, bf16, eps 0 */
    {
        uint16_t *x = malloc(n * 2), *w = malloc(H * 2), *y = malloc(n * 2);
        size_t i, j;
        for (i = 0; i < n; ++i) x[i] = to_bf16(2.0f * uniform());
        for (j = 0; j < H; ++j) w[j] = to_bf16(1.0f + 0.5f * uniform());
        void *dx = dev_copy(x, n * 2), *dw = dev_copy(w, H * 2), *dy = NULL;
        HIP_OK(hipMalloc(&dy, n * 2));
        check("fwd_status", rmsnorm_fwd(dx, dw, dy, R, H, 0.0f, RMSNORM_DTYPE_BF16, s) == RMSNORM_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(y, dy, n * 2, hipMemcpyDeviceToHost));
        double worst = 0.0;
        for (i = 0; i < R; ++i) {
            double m = 0.0;
            for (j = 0; j < H; ++j) {
                const double q = (double)from_bf16(y[i * H + j]) / (double)from_bf16(w[j]);
                m += q * q;
            }
            worst = fmax(worst, fabs(m / H - 1.0));
        }
        printf("fwd_rms_identity_worst %.3e\n", worst);
        check("fwd_rms_identity", worst < 1e-2); /* bf16 outputs: ~2^-8 per element, averaged */
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(dw));
        HIP_OK(hipFree(dy));
        free(x), free(w), free(y);
    }

    /* rmsnorm_residual_fwd, fp32, eps 0 */
    {
        float *x = malloc(n * 4), *r = malloc(n * 4), *w = malloc(H * 4), *h = malloc(n * 4), *y = malloc(n * 4);
        size_t i, j;
        for (i = 0; i < n; ++i) x[i] = uniform(), r[i] = 0.5f * uniform();
        for (j = 0; j < H; ++j) w[j] = 1.0f + 0.5f * uniform();
        void *dx = dev_copy(x, n * 4), *dr = dev_copy(r, n * 4), *dw = dev_copy(w, H * 4), *dh = NULL, *dy = NULL;
        HIP_OK(hipMalloc(&dh, n * 4));
        HIP_OK(hipMalloc(&dy, n * 4));
        check("residual_status",
              rmsnorm_residual_fwd(dx, dr, dw, dh, dy, R, H, 0.0f, RMSNORM_DTYPE_F32, s) == RMSNORM_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(h, dh, n * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(y, dy, n * 4, hipMemcpyDeviceToHost));
        int h_exact = 1;
        double worst = 0.0;
        for (i = 0; i < n; ++i) {
            const volatile float sum = x[i] + r[i]; /* one fp32 rounding */
            h_exact &= memcmp((const void*)&sum, &h[i], 4) == 0;
        }
        for (i = 0; i < R; ++i) {
            double m = 0.0;
            for (j = 0; j < H; ++j) {
                const double q = (double)y[i * H + j] / (double)w[j];
                m += q * q;
            }
            worst = fmax(worst, fabs(m / H - 1.0));
        }
        printf("residual_rms_identity_worst %.3e\n", worst);
        check("residual_h_bitwise", h_exact);
        check("residual_rms_identity", worst < 1e-5);
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(dr));
        HIP_OK(hipFree(dw));
        HIP_OK(hipFree(dh));
        HIP_OK(hipFree(dy));
        free(x), free(r), free(w), free(h), free(y);
    }

    /* rmsnorm_bwd, fp32, eps 0, with dweight through a queried workspace */
    {
        const size_t m = (size_t)R * HB;
        float *x = malloc(m * 4), *g = malloc(m * 4), *w = malloc(HB * 4), *dxh = malloc(m * 4), *dwh = malloc(HB * 4);
        size_t i, j, ws = 0;
        for (i = 0; i < m; ++i) x[i] = uniform(), g[i] = uniform();
        for (j = 0; j < HB; ++j) w[j] = 1.0f + 0.5f * uniform();
        check("bwd_workspace_query", rmsnorm_bwd_workspace_size(R, HB, RMSNORM_DTYPE_F32, NULL, &ws) == RMSNORM_OK);
        void *dx = dev_copy(x, m * 4), *dg = dev_copy(g, m * 4), *dw = dev_copy(w, HB * 4), *ddx = NULL, *ddw = NULL,
             *dws = NULL;
        HIP_OK(hipMalloc(&ddx, m * 4));
        HIP_OK(hipMalloc(&ddw, HB * 4));
        HIP_OK(hipMalloc(&dws, ws > 0 ? ws : 1));
        check("bwd_status", rmsnorm_bwd(dx, dw, dg, ddx, ddw, R, HB, 0.0f, RMSNORM_DTYPE_F32, dws, ws, s) ==
                                RMSNORM_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(dxh, ddx, m * 4, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(dwh, ddw, HB * 4, hipMemcpyDeviceToHost));
        double worst = 0.0, dot_dw = 0.0, dy_y = 0.0, scale = 0.0;
        for (i = 0; i < R; ++i) {
            double s2 = 0.0, dot = 0.0, nx = 0.0, nd = 0.0;
            for (j = 0; j < HB; ++j) s2 += (double)x[i * HB + j] * x[i * HB + j];
            const double rr = 1.0 / sqrt(s2 / HB);
            for (j = 0; j < HB; ++j) {
                dot += (double)dxh[i * HB + j] * x[i * HB + j];
                nx += (double)x[i * HB + j] * x[i * HB + j];
                nd += (double)dxh[i * HB + j] * dxh[i * HB + j];
                dy_y += (double)g[i * HB + j] * x[i * HB + j] * rr * w[j];
                scale += fabs((double)g[i * HB + j] * x[i * HB + j] * rr * w[j]);
            }
            worst = fmax(worst, fabs(dot) / sqrt(nx * nd));
        }
        for (j = 0; j < HB; ++j) dot_dw += (double)dwh[j] * w[j];
        printf("bwd_dx_orthogonality_worst %.3e dw_identity_err %.3e\n", worst, fabs(dot_dw - dy_y) / scale);
        check("bwd_dx_orthogonal_to_x", worst < 1e-4);
        check("bwd_dw_identity", fabs(dot_dw - dy_y) / scale < 1e-5);
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(dg));
        HIP_OK(hipFree(dw));
        HIP_OK(hipFree(ddx));
        HIP_OK(hipFree(ddw));
        HIP_OK(hipFree(dws));
        free(x), free(g), free(w), free(dxh), free(dwh);
    }

    /* layernorm_fwd, fp32, no beta */
    {
        float *x = malloc(n * 4), *gm = malloc(H * 4), *y = malloc(n * 4);
        size_t i, j;
        for (i = 0; i < n; ++i) x[i] = 3.0f + uniform();
        for (j = 0; j < H; ++j) gm[j] = 1.0f + 0.5f * uniform();
        void *dx = dev_copy(x, n * 4), *dg = dev_copy(gm, H * 4), *dy = NULL;
        HIP_OK(hipMalloc(&dy, n * 4));
        check("ln_status", layernorm_fwd(dx, dg, NULL, dy, R, H, 0.0f, RMSNORM_DTYPE_F32, s) == RMSNORM_OK);
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(y, dy, n * 4, hipMemcpyDeviceToHost));
        double worst_mean = 0.0, worst_var = 0.0;
        for (i = 0; i < R; ++i) {
            double s1 = 0.0, s2 = 0.0;
            for (j = 0; j < H; ++j) {
                const double z = (double)y[i * H + j] / gm[j];
                s1 += z;
                s2 += z * z;
            }
            worst_mean = fmax(worst_mean, fabs(s1 / H));
            worst_var = fmax(worst_var, fabs(s2 / H - 1.0));
        }
        printf("ln_moments_worst mean %.3e square %.3e\n", worst_mean, worst_var);
        check("ln_moments", worst_mean < 1e-5 && worst_var < 1e-5);
        HIP_OK(hipFree(dx));
        HIP_OK(hipFree(dg));
        HIP_OK(hipFree(dy));
        free(x), free(gm), free(y);
    }

    HIP_OK(hipStreamDestroy(s));
    printf("c abi gpu run: %d failures\n", failures);
    return failures != 0;
}
