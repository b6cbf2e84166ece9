/*
 * norm_oracle.c -- CPU reference for row-wise LayerNorm and RMSNorm.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code,
 * header, table or constant with it.
 *
 * Plain IEEE double with libm sqrt(), one row at a time.  Inputs are the
 * values as stored in the tensor's dtype, widened exactly to double by the
 * caller.
 *
 * Sources (the pages):
 *  - DCU case-study page, section 9: LayerNorm and RMSNorm have the same
 *    read / reduce / normalise / write structure as softmax and are the
 *    natural next operators for its kernels.
 *  - Pangu-Weather profile page, section 3: a fixed-width LayerNorm with a
 *    wave per row, fp16 input and output and fp32 mean and variance; the
 *    affine parameters were folded into the following Linear, so the device
 *    kernel only normalises.
 *
 * The pages do not write the formulas out.  Readings (also listed in the
 * design notes), each the standard definition of the operator:
 *  - LayerNorm of a row x of n entries:
 *        mu = (1/n) sum_j x_j,   var = (1/n) sum_j (x_j - mu)^2   (biased),
 *        y_j = (x_j - mu) / sqrt(var + eps) * w_j + b_j.
 *    w and b are optional (absent: 1 and 0).  eps is added to the variance
 *    under the square root.
 *  - RMSNorm of a row: ms = (1/n) sum_j x_j^2,  y_j = x_j / sqrt(ms + eps) * w_j
 *    (no centring, no bias).
 *  - The statistics outputs are mu and rstd = 1/sqrt(var + eps) (LayerNorm)
 *    or rstd = 1/sqrt(ms + eps) (RMSNorm), one per row.
 *  - Plain order of evaluation: the mean first, then the centred sum of
 *    squares (the textbook two-pass form), then each output.  A row whose
 *    variance and eps are both zero gives 0 * inf = NaN, as the definition
 *    does in IEEE arithmetic; non-finite inputs propagate the same way.
 */
#include <math.h>
#include <stdint.h>

/* ---------------------------------------------------------------------------
 * LayerNorm along the last dimension.  weight, bias, mean_out, rstd_out may
 * each be NULL.
 * ------------------------------------------------------------------------- */
void oracle_layernorm(const double *x, double *y, int64_t rows, int64_t cols, double eps,
                      const double *weight, const double *bias, double *mean_out,
                      double *rstd_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double s = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            s += xr[j];
        const double mu = s / (double)cols;
        double q = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            q += (xr[j] - mu) * (xr[j] - mu);
        const double var = q / (double)cols;
        const double rstd = 1.0 / sqrt(var + eps);
        for (int64_t j = 0; j < cols; ++j) {
            double v = (xr[j] - mu) * rstd;
            if (weight)
                v = v * weight[j];
            if (bias)
                v = v + bias[j];
            yr[j] = v;
        }
        if (mean_out)
            mean_out[r] = mu;
        if (rstd_out)
            rstd_out[r] = rstd;
    }
}

/* ---------------------------------------------------------------------------
 * RMSNorm along the last dimension.  weight and rstd_out may be NULL.
 * ------------------------------------------------------------------------- */
void oracle_rmsnorm(const double *x, double *y, int64_t rows, int64_t cols, double eps,
                    const double *weight, double *rstd_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double q = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            q += xr[j] * xr[j];
        const double ms = q / (double)cols;
        const double rstd = 1.0 / sqrt(ms + eps);
        for (int64_t j = 0; j < cols; ++j) {
            double v = xr[j] * rstd;
            if (weight)
                v = v * weight[j];
            yr[j] = v;
        }
        if (rstd_out)
            rstd_out[r] = rstd;
    }
}
