/*
 * check_c_abi.c -- the library called through its C ABI alone: no Python and
 * no torch.  Device buffers come from hipMalloc, one stream from
 * hipStreamCreate (the others run on the null stream), and every output is
 * compared element by element with the CPU oracle on the same stored inputs,
 * under the same bounds as the Python parity tests.  Also checks that bad
 * arguments come back as status codes.
 *
 * Test infrastructure: compiled by tests/c_abi/build.py, run by
 * tests/test_gpu_c_abi.py.  Exit status 0 when every case passes.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "row_wise_softmax.h"

/* The oracle (oracle/softmax_oracle.c, oracle/norm_oracle.c). */
void oracle_safe_softmax(const double *x, double *y, int64_t rows, int64_t cols);
void oracle_softmax_backward(const double *y, const double *dy, double *dx, int64_t rows,
                             int64_t cols);
void oracle_layernorm(const double *x, double *y, int64_t rows, int64_t cols, double eps,
                      const double *weight, const double *bias, double *mean_out,
                      double *rstd_out);

static int failures = 0;

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call,              \
                    hipGetErrorString(e_));                                            \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

/* Seeded inputs: splitmix64 (Vigna's published finaliser over a Weyl
 * sequence), uniform doubles in [lo, hi). */
static uint64_t rng_state;
static uint64_t splitmix64(void)
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static double uniform(double lo, double hi)
{
    return lo + (hi - lo) * (double)(splitmix64() >> 11) * 0x1.0p-53;
}

/* bfloat16 <-> float: the upper half of the binary32 pattern, rounded to
 * nearest even (inputs here are finite). */
static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* A host tensor in the dtype plus its stored values widened to double. */
typedef struct {
    int dtype;
    int64_t n;
    void *host;
    double *stored;
} Tensor;

static size_t esize(int dtype) { return dtype == RWS_F32 ? 4 : 2; }

static Tensor make_input(int dtype, int64_t n, double lo, double hi)
{
    Tensor t = {dtype, n, malloc((size_t)n * esize(dtype)), malloc((size_t)n * sizeof(double))};
    for (int64_t i = 0; i < n; ++i) {
        const float v = (float)uniform(lo, hi);
        if (dtype == RWS_F32) {
            ((float *)t.host)[i] = v;
            t.stored[i] = v;
        } else {
            const uint16_t h = float_to_bf16(v);
            ((uint16_t *)t.host)[i] = h;
            t.stored[i] = bf16_to_float(h);
        }
    }
    return t;
}

static void *to_device(const Tensor *t)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, (size_t)t->n * esize(t->dtype)));
    HIP_OK(hipMemcpy(d, t->host, (size_t)t->n * esize(t->dtype), hipMemcpyHostToDevice));
    return d;
}

static double *from_device(const void *d, int dtype, int64_t n)
{
    void *h = malloc((size_t)n * esize(dtype));
    double *out = malloc((size_t)n * sizeof(double));
    HIP_OK(hipMemcpy(h, d, (size_t)n * esize(dtype), hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == RWS_F32 ? (double)((float *)h)[i] : (double)bf16_to_float(((uint16_t *)h)[i]);
    free(h);
    return out;
}

static void report(const char *name, int ok, double worst)
{
    printf("%-44s %s (largest error %.3e)\n", name, ok ? "ok" : "FAILED", worst);
    fflush(stdout);
    if (!ok) ++failures;
}

/* Softmax bounds: fp32 |y - ref| <= 1e-5 ref + 1e-37 per element and row sums
 * within 1e-5 of 1; bf16 |y - ref| <= 8e-3 and row sums within 1e-2. */
static void check_softmax(const char *name, const double *y, const double *ref, int64_t rows,
                          int64_t cols, int dtype)
{
    int ok = 1;
    double worst = 0.0;
    for (int64_t r = 0; r < rows; ++r) {
        double sum = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            const double v = y[r * cols + j], e = fabs(v - ref[r * cols + j]);
            const double bound = dtype == RWS_F32 ? 1e-5 * ref[r * cols + j] + 1e-37 : 8e-3;
            if (!(e <= bound)) ok = 0;
            if (e > worst) worst = e;
            sum += v;
        }
        if (!(fabs(sum - 1.0) <= (dtype == RWS_F32 ? 1e-5 : 1e-2))) ok = 0;
    }
    report(name, ok, worst);
}

static void softmax_case(const char *name, int dtype, int64_t rows, int64_t cols,
                         hipStream_t stream, int kernel_id)
{
    Tensor x = make_input(dtype, rows * cols, -8.0, 8.0);
    void *dx = to_device(&x), *dy = NULL;
    HIP_OK(hipMalloc(&dy, (size_t)x.n * esize(dtype)));
    const int st = kernel_id == RWS_KERNEL_AUTO
                       ? softmax_fwd(dx, dy, rows, cols, dtype, stream)
                       : softmax_fwd_kernel(dx, dy, rows, cols, dtype, stream, kernel_id);
    if (st != RWS_OK) {
        printf("%-44s FAILED: status %d (%s)\n", name, st, softmax_last_error());
        ++failures;
    } else {
        HIP_OK(hipStreamSynchronize(stream));
        double *y = from_device(dy, dtype, x.n), *ref = malloc((size_t)x.n * sizeof(double));
        oracle_safe_softmax(x.stored, ref, rows, cols);
        check_softmax(name, y, ref, rows, cols, dtype);
        free(y);
        free(ref);
    }
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dy));
    free(x.host);
    free(x.stored);
}

/* Backward, fp32: |dx - ref| <= 2e-5 y (|dy| + sum_i |y_i dy_i|) + 1e-37. */
static void backward_case(int64_t rows, int64_t cols)
{
    Tensor z = make_input(RWS_F32, rows * cols, -4.0, 4.0), g = make_input(RWS_F32, rows * cols, -1.0, 1.0);
    double *yd = malloc((size_t)z.n * sizeof(double));
    oracle_safe_softmax(z.stored, yd, rows, cols);
    for (int64_t i = 0; i < z.n; ++i) {  /* y = the softmax, stored in fp32 */
        ((float *)z.host)[i] = (float)yd[i];
        z.stored[i] = (double)(float)yd[i];
    }
    void *dy_ = to_device(&z), *dg = to_device(&g), *ddx = NULL;
    HIP_OK(hipMalloc(&ddx, (size_t)z.n * 4));
    const int st = softmax_bwd(dy_, dg, ddx, rows, cols, RWS_F32, NULL);
    if (st != RWS_OK) {
        printf("%-44s FAILED: status %d (%s)\n", "softmax_bwd fp32", st, softmax_last_error());
        ++failures;
    } else {
        HIP_OK(hipDeviceSynchronize());
        double *dx = from_device(ddx, RWS_F32, z.n), *ref = malloc((size_t)z.n * sizeof(double));
        oracle_softmax_backward(z.stored, g.stored, ref, rows, cols);
        int ok = 1;
        double worst = 0.0;
        for (int64_t r = 0; r < rows; ++r) {
            double s = 0.0;
            for (int64_t j = 0; j < cols; ++j) s += fabs(z.stored[r * cols + j] * g.stored[r * cols + j]);
            for (int64_t j = 0; j < cols; ++j) {
                const int64_t i = r * cols + j;
                const double e = fabs(dx[i] - ref[i]);
                if (!(e <= 2e-5 * z.stored[i] * (fabs(g.stored[i]) + s) + 1e-37)) ok = 0;
                if (e > worst) worst = e;
            }
        }
        char name[64];
        snprintf(name, sizeof name, "softmax_bwd fp32 [%lld,%lld]", (long long)rows, (long long)cols);
        report(name, ok, worst);
        free(dx);
        free(ref);
    }
    HIP_OK(hipFree(dy_));
    HIP_OK(hipFree(dg));
    HIP_OK(hipFree(ddx));
    free(yd);
    free(z.host); free(z.stored); free(g.host); free(g.stored);
}

/* LayerNorm, fp32, no weight or bias: with u = 2^-24 and c = 256u,
 * e = c mean|x|, s = (e rstd)^2 / 2, n = (x - mu) rstd:
 *     |y - ref| <= c rstd mean|x| + (c + s)|n| + 2u|ref| + 1e-37,
 *     |mean - mu| <= e,  |rstd_k - rstd| <= (c + s) rstd. */
static void layernorm_case(int64_t rows, int64_t cols)
{
    Tensor x = make_input(RWS_F32, rows * cols, -3.0, 5.0);
    void *dx = to_device(&x), *dy = NULL;
    float *dmean = NULL, *drstd = NULL;
    HIP_OK(hipMalloc(&dy, (size_t)x.n * 4));
    HIP_OK(hipMalloc((void **)&dmean, (size_t)rows * 4));
    HIP_OK(hipMalloc((void **)&drstd, (size_t)rows * 4));
    const float eps = 1e-5f;
    const int st = layernorm_fwd(dx, dy, rows, cols, RWS_F32, eps, NULL, NULL, dmean, drstd, NULL);
    if (st != RWS_OK) {
        printf("%-44s FAILED: status %d (%s)\n", "layernorm_fwd fp32", st, softmax_last_error());
        ++failures;
    } else {
        HIP_OK(hipDeviceSynchronize());
        double *y = from_device(dy, RWS_F32, x.n), *ref = malloc((size_t)x.n * sizeof(double));
        double *mu = malloc((size_t)rows * sizeof(double)), *rs = malloc((size_t)rows * sizeof(double));
        double *km = from_device(dmean, RWS_F32, rows), *kr = from_device(drstd, RWS_F32, rows);
        oracle_layernorm(x.stored, ref, rows, cols, (double)eps, NULL, NULL, mu, rs);
        const double u = 0x1.0p-24, c = 256.0 * u;
        int ok = 1;
        double worst = 0.0;
        for (int64_t r = 0; r < rows; ++r) {
            double mabs = 0.0;
            for (int64_t j = 0; j < cols; ++j) mabs += fabs(x.stored[r * cols + j]);
            mabs /= (double)cols;
            const double e = c * mabs, s = 0.5 * (e * rs[r]) * (e * rs[r]);
            if (!(fabs(km[r] - mu[r]) <= e + 1e-37)) ok = 0;
            if (!(fabs(kr[r] - rs[r]) <= (c + s) * rs[r])) ok = 0;
            for (int64_t j = 0; j < cols; ++j) {
                const int64_t i = r * cols + j;
                const double err = fabs(y[i] - ref[i]);
                if (!(err <= c * rs[r] * mabs + (c + s) * fabs(ref[i]) + 2 * u * fabs(ref[i]) + 1e-37)) ok = 0;
                if (err > worst) worst = err;
            }
        }
        char name[64];
        snprintf(name, sizeof name, "layernorm_fwd fp32 [%lld,%lld]", (long long)rows, (long long)cols);
        report(name, ok, worst);
        free(y); free(ref); free(mu); free(rs); free(km); free(kr);
    }
    HIP_OK(hipFree(dx));
    HIP_OK(hipFree(dy));
    HIP_OK(hipFree(dmean));
    HIP_OK(hipFree(drstd));
    free(x.host);
    free(x.stored);
}

static void status_case(const char *name, int got, int want)
{
    const int ok = got == want;
    printf("%-44s %s (status %d, expected %d)\n", name, ok ? "ok" : "FAILED", got, want);
    if (!ok) ++failures;
}

int main(void)
{
    rng_state = 20261202u;
    int dev_count = 0;
    HIP_OK(hipGetDeviceCount(&dev_count));
    if (dev_count < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    HIP_OK(hipSetDevice(0));
    hipStream_t s = NULL;
    HIP_OK(hipStreamCreate(&s));

    softmax_case("softmax_fwd fp32 [2,3] (row 1 unaligned)", RWS_F32, 2, 3, NULL, RWS_KERNEL_AUTO);
    softmax_case("softmax_fwd fp32 [64,1000]", RWS_F32, 64, 1000, NULL, RWS_KERNEL_AUTO);
    softmax_case("softmax_fwd bf16 [4096,512]", RWS_BF16, 4096, 512, s, RWS_KERNEL_AUTO);
    softmax_case("softmax_fwd bf16 [1000,250] (tile_rows)", RWS_BF16, 1000, 250, s, RWS_KERNEL_AUTO);
    softmax_case("softmax_fwd_kernel fp32 [999,77] tile_rows", RWS_F32, 999, 77, s,
                 RWS_KERNEL_TILE_ROWS);
    softmax_case("softmax_fwd bf16 [16,300001] (split-k)", RWS_BF16, 16, 300001, s, RWS_KERNEL_AUTO);
    softmax_case("softmax_fwd_kernel fp32 [3,70001] two_pass", RWS_F32, 3, 70001, s,
                 RWS_KERNEL_TWO_PASS);
    backward_case(64, 1000);
    layernorm_case(64, 1000);

    float *buf = NULL;
    HIP_OK(hipMalloc((void **)&buf, 64 * sizeof(float)));
    status_case("rows < 0", softmax_fwd(buf, buf, -1, 4, RWS_F32, NULL), RWS_ERR_INVALID_ARG);
    status_case("unknown dtype", softmax_fwd(buf, buf, 2, 4, 7, NULL), RWS_ERR_UNSUPPORTED_DTYPE);
    status_case("pointer not element-aligned", softmax_fwd((char *)buf + 1, buf, 2, 4, RWS_F32, NULL),
                RWS_ERR_MISALIGNED);
    status_case("NULL input with data", softmax_fwd(NULL, buf, 2, 4, RWS_F32, NULL),
                RWS_ERR_INVALID_ARG);
    status_case("rows == 0 (no-op)", softmax_fwd(NULL, NULL, 0, 4, RWS_F32, NULL), RWS_OK);
    HIP_OK(hipFree(buf));
    HIP_OK(hipStreamDestroy(s));

    printf("%s: %d failure(s)\n", failures ? "FAILED" : "passed", failures);
    return failures ? 1 : 0;
}
