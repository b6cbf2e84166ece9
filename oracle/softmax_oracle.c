/*
 * softmax_oracle.c -- CPU reference for row-wise safe softmax.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it and shares no code,
 * header, table or constant with it.
 *
 * Everything is plain IEEE double with libm exp(), one row at a time, in the
 * order the pages state the method.  No blocking, fusion or reordering beyond
 * what each routine's description names.  Inputs are the values as stored in
 * the tensor's dtype, widened exactly to double by the caller.
 *
 * Sources (the pages):
 *  - "Softmax operator definition" (HIP tutorial page, sections 1 and 5): the
 *    numerically safe form y_i = e^(x_i - max x) / sum_j e^(x_j - max x), per
 *    row of a [rows, cols] matrix, along the last dimension.
 *  - "[CUDA optimisation] safe online softmax" (section 1, the numpy
 *    safe_online_softmax): a blockwise running max m and rescaled sum d over
 *    chunks of 256, then a second pass writing e^(x - m)/d.
 *  - Same page, section 3.2 (split-k): each chunk yields a partial (m, d); the
 *    partials of a row are merged with the rule
 *        (m, d) (+) (m', d') = (M, d e^(m - M) + d' e^(m' - M)),  M = max(m, m').
 *  - Case-study page (DCU), section 4.3: the element-wise online update
 *        m' = max(m, x);  d' = d e^(m - m') + e^(x - m').
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - Merge identity is (-inf, 0).  A side whose m equals the merged M takes
 *    scale exactly 1 (no exp), so (-inf,0) (+) (-inf,0) = (-inf,0), not NaN.
 *    The page's numpy routine would produce NaN for a chunk that is entirely
 *    -inf at the start of a row; on finite input both agree exactly.
 *  - In the running forms (online, split-k partials) an entry equal to -inf
 *    adds exactly 0 to a sum, whatever the running max (its limit
 *    e^(-inf - m) = 0).  Without this a chunk made only of -inf would give
 *    e^(-inf - (-inf)) = NaN; the definition itself never meets the case
 *    unless the whole row is -inf.
 *  - Max ignores NaN (a comparison with NaN is false); a NaN element then
 *    makes its own exp NaN and so the whole row NaN.  +inf present gives
 *    inf - inf = NaN, a NaN row.  -inf entries under a finite max give 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------------
 * Safe softmax by its definition (HIP tutorial page, section 1; numpy
 * safe_softmax of the CUDA page, section 1): pass 1 the row max, pass 2 the
 * sum of exp(x - max), pass 3 each exp(x - max) divided by that sum.
 * ------------------------------------------------------------------------- */
static void safe_softmax_row(const double *x, double *y, int64_t cols)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < cols; ++j)
        if (x[j] > m)
            m = x[j];
    double d = 0.0;
    for (int64_t j = 0; j < cols; ++j)
        d += exp(x[j] - m);
    for (int64_t j = 0; j < cols; ++j)
        y[j] = exp(x[j] - m) / d;
}

void oracle_safe_softmax(const double *x, double *y, int64_t rows, int64_t cols)
{
    for (int64_t r = 0; r < rows; ++r)
        safe_softmax_row(x + r * cols, y + r * cols, cols);
}

/* Per-row statistics of the definition: m = max x, d = sum exp(x - m).
 * log(d) + m is the row's log-sum-exp. */
void oracle_row_stats(const double *x, double *m_out, double *d_out,
                      int64_t rows, int64_t cols)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double m = -INFINITY;
        for (int64_t j = 0; j < cols; ++j)
            if (xr[j] > m)
                m = xr[j];
        double d = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            d += exp(xr[j] - m);
        m_out[r] = m;
        d_out[r] = d;
    }
}

/* ---------------------------------------------------------------------------
 * The (m, d) merge rule (CUDA page, warp reduction and split-k pass 2), with
 * the guarded-identity reading stated in the header comment.
 * ------------------------------------------------------------------------- */
static void md_merge(double m_a, double d_a, double m_b, double d_b,
                     double *m_out, double *d_out)
{
    double M = (m_b > m_a) ? m_b : m_a;
    double sa = (m_a == M) ? 1.0 : exp(m_a - M);
    double sb = (m_b == M) ? 1.0 : exp(m_b - M);
    *m_out = M;
    *d_out = d_a * sa + d_b * sb;
}

void oracle_md_merge(double m_a, double d_a, double m_b, double d_b,
                     double *m_out, double *d_out)
{
    md_merge(m_a, d_a, m_b, d_b, m_out, d_out);
}

/* ---------------------------------------------------------------------------
 * Blockwise online softmax (CUDA page, section 1, safe_online_softmax):
 * for each chunk of `block` columns in order, m_new = max(m, max(chunk));
 * d = d * e^(m - m_new) + sum e^(chunk - m_new); m = m_new.  Then a second
 * pass over the row writes e^(x - m) / d.
 * ------------------------------------------------------------------------- */
void oracle_online_softmax(const double *x, double *y, int64_t rows, int64_t cols,
                           int64_t block)
{
    if (block < 1)
        block = 1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double m = -INFINITY, d = 0.0;
        for (int64_t c0 = 0; c0 < cols; c0 += block) {
            int64_t c1 = c0 + block < cols ? c0 + block : cols;
            double m_local = -INFINITY;
            for (int64_t j = c0; j < c1; ++j)
                if (xr[j] > m_local)
                    m_local = xr[j];
            double m_new = (m_local > m) ? m_local : m;
            double d_local = 0.0;
            for (int64_t j = c0; j < c1; ++j)
                d_local += (xr[j] == -INFINITY) ? 0.0 : exp(xr[j] - m_new);
            double scale = (m == m_new) ? 1.0 : exp(m - m_new);
            d = d * scale + d_local;
            m = m_new;
        }
        for (int64_t j = 0; j < cols; ++j)
            yr[j] = exp(xr[j] - m) / d;
    }
}

/* ---------------------------------------------------------------------------
 * Element-wise online update (case-study page, section 4.3):
 * m' = max(m, x_j); d' = d e^(m - m') + e^(x_j - m'), one element at a time.
 * Returns only the per-row statistics.
 * ------------------------------------------------------------------------- */
void oracle_online_stats_elementwise(const double *x, double *m_out, double *d_out,
                                     int64_t rows, int64_t cols)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double m = -INFINITY, d = 0.0;
        for (int64_t j = 0; j < cols; ++j) {
            double m_new = (xr[j] > m) ? xr[j] : m;
            double scale = (m == m_new) ? 1.0 : exp(m - m_new);
            d = d * scale + ((xr[j] == -INFINITY) ? 0.0 : exp(xr[j] - m_new));
            m = m_new;
        }
        m_out[r] = m;
        d_out[r] = d;
    }
}

/* ---------------------------------------------------------------------------
 * Split-k (CUDA page, section 3.2): the row is cut into chunks of `chunk`
 * columns; each chunk's partial (m_c, d_c) is computed on its own (max of the
 * chunk, then the sum of e^(x - m_c) over it); the partials of the row are
 * merged with the (m, d) rule in chunk order; each chunk's outputs are then
 * e^(x - M) / D with the merged (M, D).
 * ------------------------------------------------------------------------- */
void oracle_splitk_softmax(const double *x, double *y, int64_t rows, int64_t cols,
                           int64_t chunk)
{
    if (chunk < 1)
        chunk = 1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double M = -INFINITY, D = 0.0;
        for (int64_t c0 = 0; c0 < cols; c0 += chunk) {
            int64_t c1 = c0 + chunk < cols ? c0 + chunk : cols;
            double mc = -INFINITY;
            for (int64_t j = c0; j < c1; ++j)
                if (xr[j] > mc)
                    mc = xr[j];
            double dc = 0.0;
            for (int64_t j = c0; j < c1; ++j)
                dc += (xr[j] == -INFINITY) ? 0.0 : exp(xr[j] - mc);
            md_merge(M, D, mc, dc, &M, &D);
        }
        for (int64_t j = 0; j < cols; ++j)
            yr[j] = exp(xr[j] - M) / D;
    }
}

/* ---------------------------------------------------------------------------
 * Scaled, masked softmax of attention scores (DCU case-study page, section
 * 9: a mask parameter in the softmax kernel; Pangu-Weather profile page,
 * section 6: bias + mask + softmax).  For row r and column j:
 *     z_rj = scale * x_rj + mask[(r mod mask_rows), j]     (mask may be NULL)
 *     z_rj = -inf  if causal_q > 0 and j > (r mod causal_q) + cols - causal_q
 * then the definition above on z.  Reading: the causal limit aligns the last
 * query with the last key (keys may outnumber queries).
 * ------------------------------------------------------------------------- */
void oracle_masked_softmax(const double *x, double *y, int64_t rows, int64_t cols, double scale,
                           const double *mask, int64_t mask_rows, int64_t causal_q)
{
    double *z = (double *)malloc(sizeof(double) * (size_t)(cols > 0 ? cols : 1));
    if (!z)
        return;
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        const double *mr = mask ? mask + (r % mask_rows) * cols : NULL;
        for (int64_t j = 0; j < cols; ++j) {
            double v = scale * xr[j];
            if (mr)
                v += mr[j];
            if (causal_q > 0 && j > (r % causal_q) + cols - causal_q)
                v = -INFINITY;
            z[j] = v;
        }
        safe_softmax_row(z, y + r * cols, cols);
    }
    free(z);
}

/* ---------------------------------------------------------------------------
 * Softmax backward (the training step the DCU case-study page, section 5.4,
 * says needs its own check).  With y the forward output of a row and dy the
 * gradient of the loss with respect to y, the gradient with respect to the
 * row's input is the Jacobian transpose times dy:
 *     dx_j = sum_i dy_i * dy_i/dx_j = y_j * (dy_j - sum_i dy_i * y_i),
 * since dy_i/dx_j = y_i * (delta_ij - y_j).  Plain order: the dot product
 * over the row first, then each element.
 * ------------------------------------------------------------------------- */
void oracle_softmax_backward(const double *y, const double *dy, double *dx, int64_t rows,
                             int64_t cols)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *yr = y + r * cols;
        const double *gr = dy + r * cols;
        double *xr = dx + r * cols;
        double dot = 0.0;
        for (int64_t j = 0; j < cols; ++j)
            dot += gr[j] * yr[j];
        for (int64_t j = 0; j < cols; ++j)
            xr[j] = yr[j] * (gr[j] - dot);
    }
}

/* ---------------------------------------------------------------------------
 * The definition run over row ranges on several host threads: rows are
 * independent, so each thread applies safe_softmax_row to its own
 * contiguous range.  Used to time the oracle on the host's cores.
 * Returns the number of threads actually used.
 * ------------------------------------------------------------------------- */
typedef struct {
    const double *x;
    double *y;
    int64_t r0, r1, cols;
} oracle_range_t;

static void *range_worker(void *arg)
{
    oracle_range_t *a = (oracle_range_t *)arg;
    for (int64_t r = a->r0; r < a->r1; ++r)
        safe_softmax_row(a->x + r * a->cols, a->y + r * a->cols, a->cols);
    return NULL;
}

int oracle_safe_softmax_threads(const double *x, double *y, int64_t rows, int64_t cols,
                                int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if ((int64_t)nthreads > rows)
        nthreads = rows > 0 ? (int)rows : 1;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    oracle_range_t *args = (oracle_range_t *)malloc(sizeof(oracle_range_t) * (size_t)nthreads);
    char *running = (char *)calloc((size_t)nthreads, 1);
    if (!tid || !args || !running) {
        free(tid);
        free(args);
        free(running);
        oracle_safe_softmax(x, y, rows, cols);
        return 1;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        args[t].x = x;
        args[t].y = y;
        args[t].cols = cols;
        args[t].r0 = rows * t / nthreads;
        args[t].r1 = rows * (t + 1) / nthreads;
        if (pthread_create(&tid[t], NULL, range_worker, &args[t]) == 0) {
            running[t] = 1;
            ++started;
        } else {
            range_worker(&args[t]); /* run inline if a thread cannot start */
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (running[t])
            pthread_join(tid[t], NULL);
    free(tid);
    free(args);
    free(running);
    return started > 0 ? started : 1;
}
