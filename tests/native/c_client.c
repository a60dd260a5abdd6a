/*
 * c_client.c -- a plain C99 client of liblnr: the library's C ABI (include/lnr.h) used with no
 * Python and no framework, device memory and a stream from the HIP runtime directly.
 *
 *   c_client validate   argument validation only; touches no device (runs without a GPU)
 *   c_client gpu        masked causal softmax forward and backward and LayerNorm forward and
 *                       backward on device 0, checked against properties of the operations
 *
 * The GPU checks are properties that hold for any correct implementation, not a second
 * implementation of the method: softmax rows sum to 1 with exact zeros at masked and future
 * keys ("CMU 11-868 HW4 ...", section "Problem structure and scoring"), the softmax gradient's
 * rows sum to 0 and vanish where y does, LayerNorm output rows have mean 0 and second moment
 * v / (v + eps) for gamma = 1 and beta = 0, the saved mean and 1/sigma are the row's, the
 * LayerNorm input gradient's rows sum to 0 and dbeta is the column sum of dy.
 * Exit status 0 when every check passes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "lnr.h"

static int failures = 0;
static int checks = 0;

#define CHECK(cond, ...)                        \
    do {                                        \
        ++checks;                               \
        if (!(cond)) {                          \
            printf("FAIL line %d: ", __LINE__); \
            printf(__VA_ARGS__);                \
            printf("\n");                       \
            ++failures;                         \
        }                                       \
    } while (0)

#define HIP_OK(x)                                                               \
    do {                                                                        \
        hipError_t e_ = (x);                                                    \
        if (e_ != hipSuccess) {                                                 \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            exit(2);                                                            \
        }                                                                       \
    } while (0)

/* Seeded inputs: a 64-bit linear congruential generator and the Box-Muller transform. */
static uint64_t rng_state = 0x853C49E6748FEA9Bull;
static double uniform01(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) / 9007199254740992.0;
}
static float normal01(void) {
    double u1 = uniform01(), u2 = uniform01();
    if (u1 < 1e-300) u1 = 1e-300;
    return (float)(sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2));
}

/* Fake, distinct, 256-byte aligned device addresses: validation fails before any is used. */
static void *fake(int k) { return (void *)(uintptr_t)(0x7F0000000000ull + (uint64_t)k * (1ull << 30)); }

static void validate(void) {
    CHECK(attn_softmax_fw(NULL, fake(1), NULL, 2, 2, 16, 16, 0, LNR_F32, NULL) == LNR_ERR_NULL,
          "softmax fw: NULL output");
    CHECK(attn_softmax_fw(fake(0), fake(1), NULL, 2, 2, 8, 16, 1, LNR_F32, NULL) == LNR_ERR_SHAPE,
          "softmax fw: causal with Tq != Tk");
    CHECK(attn_softmax_fw(fake(0), fake(1), NULL, 2, 2, 16, 4096, 0, LNR_F32, NULL) == LNR_ERR_UNSUPPORTED,
          "softmax fw: Tk beyond the template list");
    CHECK(attn_softmax_fw(fake(0), fake(1), NULL, 2, 2, 16, 16, 0, (lnr_dtype)7, NULL) == LNR_ERR_DTYPE,
          "softmax fw: bad dtype");
    CHECK(attn_softmax_bw(fake(0), fake(1), fake(0), 2, 2, 16, 16, LNR_F16, NULL) == LNR_ERR_ALIAS,
          "softmax bw: output over y");
    CHECK(attn_softmax_fw(fake(0), fake(1), NULL, 0, 2, 16, 16, 0, LNR_F16, NULL) == LNR_OK,
          "softmax fw: B = 0 is an empty call");
    CHECK(layernorm_fw(fake(0), NULL, NULL, fake(1), fake(2), fake(3), 16, 0, 1e-8f, LNR_F16, NULL) ==
              LNR_ERR_SHAPE, "layernorm fw: C = 0");
    CHECK(layernorm_bw_workspace_bytes(16384, 1024, LNR_F16) > 0, "layernorm workspace size");
    CHECK(layernorm_bw(fake(0), fake(1), fake(2), fake(3), fake(4), fake(5), (const float *)fake(6),
                       (const float *)fake(7), 16, 64, LNR_F32, NULL, 0, NULL) == LNR_ERR_WORKSPACE,
          "layernorm bw: missing workspace");
    CHECK(strcmp(lnr_strerror(LNR_OK), "success") == 0, "strerror(OK)");
    CHECK(strstr(lnr_build_info(), "gfx950") != NULL, "build info names gfx950");
}

static void softmax_on_gpu(hipStream_t st) {
    enum { B = 2, H = 3, T = 40 };
    const size_t n = (size_t)B * H * T * T;
    const int len[B] = {25, T};
    float *x = malloc(n * sizeof(float)), *dy = malloc(n * sizeof(float));
    float *y = malloc(n * sizeof(float)), *dx = malloc(n * sizeof(float));
    float mask[B * T];
    for (size_t i = 0; i < n; ++i) {
        x[i] = normal01();
        dy[i] = normal01();
    }
    for (int b = 0; b < B; ++b)
        for (int j = 0; j < T; ++j) mask[b * T + j] = j < len[b] ? 0.0f : -INFINITY;
    float *dx_d, *x_d, *y_d, *dy_d, *m_d;
    HIP_OK(hipMalloc((void **)&x_d, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&y_d, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&dy_d, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&dx_d, n * sizeof(float)));
    HIP_OK(hipMalloc((void **)&m_d, sizeof mask));
    HIP_OK(hipMemcpy(x_d, x, n * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy_d, dy, n * sizeof(float), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(m_d, mask, sizeof mask, hipMemcpyHostToDevice));

    CHECK(attn_softmax_fw(y_d, x_d, m_d, B, H, T, T, 1, LNR_F32, st) == LNR_OK, "softmax fw status");
    CHECK(attn_softmax_bw(dx_d, dy_d, y_d, B, H, T, T, LNR_F32, st) == LNR_OK, "softmax bw status");
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(y, y_d, n * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dx, dx_d, n * sizeof(float), hipMemcpyDeviceToHost));

    int bad_sum = 0, bad_zero = 0, bad_pos = 0, bad_gsum = 0, bad_gzero = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < T; ++i) {
                const float *yr = y + (((size_t)b * H + h) * T + i) * T;
                const float *gr = dx + (((size_t)b * H + h) * T + i) * T;
                double s = 0.0, gs = 0.0, gscale = 0.0;
                for (int j = 0; j < T; ++j) {
                    const int open = j <= i && j < len[b];
                    s += yr[j];
                    gs += gr[j];
                    gscale += fabs(gr[j]);
                    if (!open && yr[j] != 0.0f) ++bad_zero;
                    if (open && !(yr[j] > 0.0f)) ++bad_pos;
                    if (!open && gr[j] != 0.0f) ++bad_gzero;
                }
                if (fabs(s - 1.0) > 1e-5) ++bad_sum;
                if (fabs(gs) > 1e-5 * (1.0 + gscale)) ++bad_gsum;
            }
    CHECK(bad_sum == 0, "softmax: %d rows do not sum to 1", bad_sum);
    CHECK(bad_zero == 0, "softmax: %d masked or future probabilities are not exactly 0", bad_zero);
    CHECK(bad_pos == 0, "softmax: %d open probabilities are not positive", bad_pos);
    CHECK(bad_gsum == 0, "softmax bw: %d gradient rows do not sum to 0", bad_gsum);
    CHECK(bad_gzero == 0, "softmax bw: %d gradients are not 0 where y is 0", bad_gzero);

    HIP_OK(hipFree(x_d));
    HIP_OK(hipFree(y_d));
    HIP_OK(hipFree(dy_d));
    HIP_OK(hipFree(dx_d));
    HIP_OK(hipFree(m_d));
    free(x);
    free(dy);
    free(y);
    free(dx);
}

static void layernorm_on_gpu(hipStream_t st) {
    enum { N = 37, C = 256 };
    const float eps = 1e-8f;
    static float x[N * C], dy[N * C], y[N * C], dx[N * C], gamma[C], beta[C], dgamma[C], dbeta[C];
    static float mean[N], rstd[N];
    for (int i = 0; i < N; ++i) {
        const float offset = 3.0f * normal01();
        for (int j = 0; j < C; ++j) {
            x[i * C + j] = offset + normal01();
            dy[i * C + j] = normal01();
        }
    }
    for (int j = 0; j < C; ++j) {
        gamma[j] = 1.0f;
        beta[j] = 0.0f;
    }
    const size_t nb = sizeof x, cb = sizeof gamma;
    float *x_d, *dy_d, *y_d, *dx_d, *g_d, *b_d, *dg_d, *db_d, *m_d, *r_d;
    void *ws_d;
    const size_t wsb = layernorm_bw_workspace_bytes(N, C, LNR_F32);
    HIP_OK(hipMalloc((void **)&x_d, nb));
    HIP_OK(hipMalloc((void **)&dy_d, nb));
    HIP_OK(hipMalloc((void **)&y_d, nb));
    HIP_OK(hipMalloc((void **)&dx_d, nb));
    HIP_OK(hipMalloc((void **)&g_d, cb));
    HIP_OK(hipMalloc((void **)&b_d, cb));
    HIP_OK(hipMalloc((void **)&dg_d, cb));
    HIP_OK(hipMalloc((void **)&db_d, cb));
    HIP_OK(hipMalloc((void **)&m_d, sizeof mean));
    HIP_OK(hipMalloc((void **)&r_d, sizeof rstd));
    HIP_OK(hipMalloc(&ws_d, wsb));
    HIP_OK(hipMemcpy(x_d, x, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dy_d, dy, nb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(g_d, gamma, cb, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(b_d, beta, cb, hipMemcpyHostToDevice));

    CHECK(layernorm_fw(y_d, m_d, r_d, x_d, g_d, b_d, N, C, eps, LNR_F32, st) == LNR_OK, "layernorm fw status");
    CHECK(layernorm_bw(dx_d, dg_d, db_d, dy_d, x_d, g_d, m_d, r_d, N, C, LNR_F32, ws_d, wsb, st) == LNR_OK,
          "layernorm bw status");
    HIP_OK(hipStreamSynchronize(st));
    HIP_OK(hipMemcpy(y, y_d, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dx, dx_d, nb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dgamma, dg_d, cb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(dbeta, db_d, cb, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(mean, m_d, sizeof mean, hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(rstd, r_d, sizeof rstd, hipMemcpyDeviceToHost));

    int bad_mean = 0, bad_m2 = 0, bad_stats = 0, bad_dx = 0, bad_db = 0;
    for (int i = 0; i < N; ++i) {
        double mu = 0.0, v = 0.0, ym = 0.0, y2 = 0.0, ds = 0.0, dscale = 0.0;
        for (int j = 0; j < C; ++j) mu += x[i * C + j];
        mu /= C;
        for (int j = 0; j < C; ++j) v += (x[i * C + j] - mu) * (x[i * C + j] - mu);
        v /= C;
        for (int j = 0; j < C; ++j) {
            ym += y[i * C + j];
            y2 += (double)y[i * C + j] * y[i * C + j];
            ds += dx[i * C + j];
            dscale += fabs(dx[i * C + j]);
        }
        ym /= C;
        y2 /= C;
        if (fabs(ym) > 1e-5) ++bad_mean;
        if (fabs(y2 - v / (v + eps)) > 1e-4) ++bad_m2;
        if (fabs(mean[i] - mu) > 1e-5 * (1.0 + fabs(mu)) || fabs(rstd[i] - 1.0 / sqrt(v + eps)) > 1e-4 / sqrt(v + eps))
            ++bad_stats;
        if (fabs(ds) > 1e-5 * (1.0 + dscale)) ++bad_dx;
    }
    for (int j = 0; j < C; ++j) {
        double s = 0.0, a = 0.0;
        for (int i = 0; i < N; ++i) {
            s += dy[i * C + j];
            a += fabs(dy[i * C + j]);
        }
        if (fabs(dbeta[j] - s) > 1e-5 * (1.0 + a)) ++bad_db;
    }
    CHECK(bad_mean == 0, "layernorm: %d rows without mean 0", bad_mean);
    CHECK(bad_m2 == 0, "layernorm: %d rows whose second moment is not v/(v+eps)", bad_m2);
    CHECK(bad_stats == 0, "layernorm: %d rows whose saved mean or 1/sigma differ from the row's", bad_stats);
    CHECK(bad_dx == 0, "layernorm bw: %d input-gradient rows do not sum to 0", bad_dx);
    CHECK(bad_db == 0, "layernorm bw: %d dbeta columns differ from the column sums of dy", bad_db);

    HIP_OK(hipFree(x_d));
    HIP_OK(hipFree(dy_d));
    HIP_OK(hipFree(y_d));
    HIP_OK(hipFree(dx_d));
    HIP_OK(hipFree(g_d));
    HIP_OK(hipFree(b_d));
    HIP_OK(hipFree(dg_d));
    HIP_OK(hipFree(db_d));
    HIP_OK(hipFree(m_d));
    HIP_OK(hipFree(r_d));
    HIP_OK(hipFree(ws_d));
}

int main(int argc, char **argv) {
    if (argc != 2 || (strcmp(argv[1], "validate") != 0 && strcmp(argv[1], "gpu") != 0)) {
        fprintf(stderr, "usage: %s validate|gpu\n", argv[0]);
        return 2;
    }
    validate();
    if (strcmp(argv[1], "gpu") == 0) {
        hipStream_t st;
        HIP_OK(hipStreamCreate(&st));
        softmax_on_gpu(st);
        layernorm_on_gpu(st);
        HIP_OK(hipStreamDestroy(st));
    }
    printf("c_client %s: %d checks, %d failed\n", argv[1], checks, failures);
    return failures == 0 ? 0 : 1;
}
