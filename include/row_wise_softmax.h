/*
 * row_wise_softmax.h -- C ABI of the MI355X (gfx950) row-wise safe softmax
 * library (librws_softmax.so), with the softmax backward and the LayerNorm /
 * RMSNorm row normalisations on the same kernels' skeleton.
 *
 * Operation.  For a contiguous row-major matrix X[rows, cols] the library
 * writes, for every row r and column j,
 *
 *     Y[r, j] = exp(X[r, j] - m_r) / d_r,
 *     m_r     = max_j X[r, j],
 *     d_r     = sum_j exp(X[r, j] - m_r),
 *
 * i.e. softmax along the last dimension in its numerically safe form
 * (HIP softmax tutorial page, sections 1 and 5; CUDA safe-online-softmax page,
 * section 1).  Depending on the shape, the kernels obtain (m_r, d_r) directly,
 * with the running update m' = max(m, x), d' = d e^(m - m') + e^(x - m')
 * (DCU case-study page, section 4.3; CUDA safe-online-softmax page, section 1),
 * or by merging per-chunk partials with
 * (m, d) (+) (m', d') = (M, d e^(m - M) + d' e^(m' - M)), M = max(m, m')
 * (CUDA safe-online-softmax page, sections 2.1.1 and 3.2).  All of these are
 * re-associations of the same sums; every path accumulates in fp32.
 *
 * Data types (in dtype == out dtype, fp32 accumulation):
 *     RWS_F32 = 0  IEEE binary32
 *     RWS_F16 = 1  IEEE binary16
 *     RWS_BF16 = 2 bfloat16
 * Outputs are rounded to nearest-even from the fp32 result.
 *
 * Layout.  `in` and `out` point to rows*cols elements, row-major, row pitch
 * == cols (no stride argument).  Pointers must be device memory of the current
 * HIP device and aligned to the element size; 16-byte alignment is NOT
 * required (rows of any length and any start address are handled).  Exact
 * aliasing (in == out, in-place) is allowed; partial overlap is undefined.
 *
 * Streams.  `stream` is a hipStream_t passed as an opaque pointer (NULL = the
 * null stream).  All work is enqueued on it; no call synchronises the host.
 * The result is valid once the stream reaches the enqueued work.
 *
 * Ownership.  The caller owns `in` and `out`.  For the split-k paths the
 * library owns a small workspace (8 bytes per row per chunk for the two-launch
 * form, 16 bytes per row per chunk of epoch-tagged words for the single-launch
 * forms, and one 128-byte status word) that it keeps per (device, stream) and
 * grows on demand; the first call that needs a larger workspace allocates it
 * (hipMalloc; tag words and the status word are zeroed then, by a kernel on
 * the call's stream), later calls reuse it (softmax_fwd_noalloc allocates
 * nothing).  Calls on one stream are ordered, so
 * reuse is safe; the workspaces are released when the library is unloaded.
 * They are keyed by the stream handle: a destroyed stream's workspace stays
 * allocated, and a stream created later with the same handle reuses it.
 *
 * Graph capture.  Every entry point may be captured into a HIP graph.  The
 * single-launch split-k forms tell one launch's partials from the last by an
 * epoch that a replay would repeat, so while `stream` is capturing the
 * forward takes the two-launch split-k instead, and the backward and the
 * normalisations take their epoch from device memory, advanced by a small
 * kernel recorded before each of their split-k launches.  Nothing is
 * allocated during capture: capture a forward split-k call only after the
 * same call (or a larger one) has run once eagerly on the capturing stream,
 * otherwise the call returns RWS_ERR_HIP and enqueues nothing; a backward or
 * normalisation call that finds no workspace on the stream records its
 * one-workgroup-per-row form (correct, slower for few long rows).  A
 * workspace buffer that a graph captured is never freed while the library is
 * loaded (a later, larger call on that stream gets a new one), so the graph
 * stays valid; replay it on the capturing stream, or order it with that
 * stream's other split-k calls, since both use that buffer.
 *
 * Errors.  Every entry point returns a status code (below) and never exits or
 * throws.  rows == 0 or cols == 0 is a successful no-op.  A HIP launch error
 * is reported as RWS_ERR_HIP; softmax_last_error() then returns the detail
 * (thread-local, valid until the next call on the same thread).
 */
#ifndef ROW_WISE_SOFTMAX_H
#define ROW_WISE_SOFTMAX_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types. */
enum {
    RWS_F32 = 0,
    RWS_F16 = 1,
    RWS_BF16 = 2
};

/* Status codes. */
enum {
    RWS_OK = 0,
    RWS_ERR_INVALID_ARG = 1,       /* negative size, NULL pointer with data, bad id */
    RWS_ERR_UNSUPPORTED_DTYPE = 2, /* dtype not one of RWS_F32/F16/BF16 */
    RWS_ERR_MISALIGNED = 3,        /* pointer not aligned to the element size */
    RWS_ERR_HIP = 4,               /* HIP runtime error (see softmax_last_error) */
    RWS_ERR_UNSUPPORTED_SHAPE = 5, /* forced kernel cannot take this shape */
    RWS_ERR_WAIT_TIMEOUT = 6       /* softmax_stream_status: a single-launch
                                      split-k wait gave up (outputs NaN) */
};

/* Kernel families (ids for softmax_fwd_kernel / softmax_select_kernel). */
enum {
    RWS_KERNEL_AUTO = 0,      /* let the dispatcher choose */
    RWS_KERNEL_WAVE_ROW = 1,  /* one row per 64-lane wave (or per 4..32-lane
                                 group, several rows per wave); row cached in
                                 registers; cross-lane reductions without LDS
                                 (DCU case-study page, sections 4.1 and 8) */
    RWS_KERNEL_BLOCK_ONEPASS = 2, /* one workgroup per row; the row is read
                                 once and cached in registers, then LDS
                                 (CUDA safe-online-softmax page, sections 2.1
                                 and 2.2) */
    RWS_KERNEL_TWO_PASS = 3,  /* one workgroup per row, any cols: pass 1 running
                                 (m, d), pass 2 re-reads the row (CUDA
                                 safe-online-softmax page, section 3.1) */
    RWS_KERNEL_SPLITK = 4,    /* several workgroups per row: stage 1 writes a
                                 partial (m, d) per chunk, stage 2 merges a
                                 row's partials and writes the outputs (CUDA
                                 safe-online-softmax page, section 3.2) */
    RWS_KERNEL_SPLITK_FUSED = 5, /* split-k in one ordinary launch that
                                 reads the input once: each workgroup keeps
                                 its chunk in registers and waits for the
                                 row's partial (m, d), which travel as
                                 epoch-tagged words (as the ordered form
                                 below; the single-kernel form the same
                                 page, section 3.2, mentions).  Relies on the
                                 same in-order dispatch as the ordered form,
                                 and on one row's workgroups fitting on the
                                 device at once: returns
                                 RWS_ERR_UNSUPPORTED_SHAPE when they cannot.
                                 A wait that runs out of its bound writes NaN
                                 and sets the stream's status word.  The
                                 dispatcher's choice for few long rows when
                                 the whole grid fits at once (up to 64 MiB of
                                 line-aligned 16-bit input on MI355X) and the
                                 rows number at most four, exceed 32 MiB
                                 together, or need more than 512 chunks
                                 each */
    RWS_KERNEL_SPLITK_ORDERED = 6, /* split-k in one ordinary launch: the
                                 stage-1 workgroups (partial (m, d) per chunk)
                                 come first in the grid, the stage-2
                                 workgroups (merge, re-read, write) after
                                 them and poll the row's partials, which
                                 travel as epoch-tagged 64-bit words (no grid
                                 barrier, no memory fence; the single-kernel
                                 form the same page, section 3.2, mentions).
                                 Relies on workgroups being dispatched in
                                 increasing index order (within each XCD,
                                 which the hardware does but HIP does not
                                 promise); a wait that runs out of its bound
                                 writes NaN for its chunk instead of hanging
                                 and sets the stream's status word, which
                                 softmax_stream_status reports.  The
                                 dispatcher's choice for few long rows of up
                                 to 32 MiB together and 512 chunks each */
    RWS_KERNEL_TILE_ROWS = 7     /* short rows that are not line-aligned:
                                 one wave takes 4 to 64 consecutive rows
                                 (as many as fill its 64*K granule slots,
                                 K = 1..4 the variant) as one 16-byte-aligned
                                 range (every granule read and written whole
                                 by one lane, a row may start and end inside
                                 a granule) and reduces each row across the
                                 lanes that hold it, through LDS (the
                                 row-wise definition, CUDA
                                 safe-online-softmax page, section 1).  Needs
                                 in and out 16-byte aligned, rows of one
                                 granule to 1024 bytes, and a tile of at
                                 least 4 rows (RWS_ERR_UNSUPPORTED_SHAPE
                                 otherwise).  The dispatcher's choice for
                                 many such rows (plain and masked) */
};

/*
 * softmax_fwd -- Y = softmax(X) along the last dimension, kernel chosen by
 * the dispatcher from (rows, cols, dtype, pointer alignment, device).
 *   in, out : device pointers, rows*cols elements of `dtype` each
 *   rows    : number of rows (>= 0)
 *   cols    : row length (>= 0)
 *   dtype   : RWS_F32, RWS_F16 or RWS_BF16
 *   stream  : hipStream_t (NULL = null stream)
 * Returns RWS_OK or an error status.
 */
int softmax_fwd(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                void *stream);

/*
 * softmax_fwd_kernel -- as softmax_fwd, but runs the given kernel family
 * (RWS_KERNEL_*; RWS_KERNEL_AUTO behaves like softmax_fwd).  Returns
 * RWS_ERR_UNSUPPORTED_SHAPE if that family cannot take the shape (the
 * register/LDS-cached families have a maximum row length).  For tests and
 * measurement.
 */
int softmax_fwd_kernel(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                       void *stream, int kernel_id);

/*
 * softmax_fwd_noalloc -- softmax_fwd for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the library allocates nothing on this path, on the
 * first call or later.  The kernel is chosen as in softmax_fwd, except that
 * a shape the dispatcher sends to split-k runs the two-launch split-k
 * (RWS_KERNEL_SPLITK), whose per-chunk partial (m, d) pairs live in a
 * 512 KiB array that the library's code object holds on every GPU it runs
 * on, until the process ends.  Rows are launched in batches whose partials
 * fit the array (8 bytes per row per chunk); a row needing more than the
 * whole array (fp32 rows of more than 2^29 columns) is rejected with
 * RWS_ERR_UNSUPPORTED_SHAPE before any launch.  The array keeps the last
 * call's contents (nothing in it needs to start at zero).  All calls on one
 * GPU share that GPU's array: calls on that GPU that can run at the same
 * time (on different streams, or from different threads without ordering)
 * race on it and give wrong results; calls ordered on one stream are safe,
 * and so is replaying a captured call on its stream.  Arguments, layout,
 * streams and errors as softmax_fwd.
 */
int softmax_fwd_noalloc(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                        void *stream);

/*
 * softmax_fwd_masked -- softmax of attention scores with the scale and mask
 * folded in (DCU case-study page, section 9: a mask parameter in the softmax
 * kernel saves a launch; Pangu-Weather profile page, section 6: bias + mask +
 * softmax):
 *     z[r, j] = scale * X[r, j] + M[r mod mask_rows, j]      (M optional)
 *     z[r, j] = -inf   when causal_q > 0 and j > (r mod causal_q) + cols - causal_q
 *     Y[r, :] = softmax(z[r, :])  as in softmax_fwd.
 *   scale     : fp32 factor applied to X (1 for none)
 *   mask      : NULL, or an additive mask with X's dtype, mask_rows x cols,
 *               row pitch cols, aligned to the element size; row r of X uses
 *               row (r mod mask_rows), e.g. a [S, S] mask broadcast over the
 *               batch and heads of [B, H, S, S] scores (rows = B*H*S)
 *   mask_rows : rows of the mask (>= 1 when mask != NULL; ignored otherwise)
 *   causal_q  : 0 for none, else the query length q: row r is query
 *               (r mod q) and sees keys j <= (r mod q) + cols - q (the last
 *               query sees every key)
 *   kernel_id : RWS_KERNEL_AUTO, or RWS_KERNEL_WAVE_ROW / BLOCK_ONEPASS /
 *               TWO_PASS / TILE_ROWS (no split-k form;
 *               RWS_ERR_UNSUPPORTED_SHAPE); the dispatcher takes TILE_ROWS
 *               for many short rows that are not line-aligned, as for
 *               softmax_fwd
 * A row whose every entry ends up -inf becomes NaN (0/0), as the definition
 * gives.  Other arguments, layout, streams and errors as softmax_fwd.
 */
int softmax_fwd_masked(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                       float scale, const void *mask, int64_t mask_rows, int64_t causal_q,
                       void *stream, int kernel_id);

/*
 * softmax_bwd -- gradient through the row-wise softmax (the backward pass the
 * DCU case-study page, section 5.4, says training needs checked on its own):
 *     dX[r, j] = Y[r, j] * (dY[r, j] - sum_i dY[r, i] * Y[r, i])
 *   y  : the forward output Y (device, rows*cols of dtype)
 *   dy : the gradient with respect to Y (same shape and dtype)
 *   dx : the gradient with respect to the forward input (same shape and
 *        dtype); may alias dy or y exactly (in place)
 * fp32 accumulation; reads y and dy once (rows that fit a workgroup's
 * registers) and writes dx once.  Layout, alignment, streams and errors as
 * softmax_fwd.
 */
int softmax_bwd(const void *y, const void *dy, void *dx, int64_t rows, int64_t cols, int dtype,
                void *stream);

/*
 * softmax_bwd_kernel -- as softmax_bwd with a forced kernel: RWS_KERNEL_AUTO,
 * RWS_KERNEL_WAVE_ROW (row in one wave's registers), RWS_KERNEL_BLOCK_ONEPASS
 * (row in one workgroup's registers), RWS_KERNEL_TWO_PASS (any length; y
 * and dy are read twice) or RWS_KERNEL_SPLITK_ORDERED (several workgroups
 * per row in one launch: chunk dot products published as epoch-tagged
 * words, as for softmax_fwd; the dispatcher's choice for few long rows; uses
 * the per-stream tag words that the forward's ordered form allocates on
 * first use) or RWS_KERNEL_TILE_ROWS (several short rows per wave, as for
 * softmax_fwd; y, dy and dx 16-byte aligned; the dispatcher's choice for
 * many short rows that are not line-aligned).  Other ids:
 * RWS_ERR_INVALID_ARG.  softmax_bwd_describe_launch reports the choice for
 * a dy with y's 16-byte alignment.
 */
int softmax_bwd_kernel(const void *y, const void *dy, void *dx, int64_t rows, int64_t cols,
                       int dtype, void *stream, int kernel_id);

/*
 * layernorm_fwd -- LayerNorm along the last dimension, the row normalisation
 * the DCU case-study page (section 9) names as having softmax's read /
 * reduce / normalise / write structure, and the Pangu-Weather profile page
 * (section 3) runs as a wave-per-row kernel with fp16 data and fp32
 * statistics:
 *     mu_r   = (1/cols) sum_j X[r, j]
 *     var_r  = (1/cols) sum_j (X[r, j] - mu_r)^2          (biased)
 *     rstd_r = 1 / sqrt(var_r + eps)
 *     Y[r, j] = (X[r, j] - mu_r) * rstd_r * W[j] + B[j]
 *   eps    : >= 0 and finite (RWS_ERR_INVALID_ARG otherwise)
 *   weight : NULL (W = 1) or cols elements of `dtype` on the device, aligned
 *            to the element size
 *   bias   : NULL (B = 0) or as weight
 *   mean, rstd : NULL, or rows fp32 values each on the device (4-byte
 *            aligned) that receive mu_r and rstd_r (for a backward pass)
 * Statistics are accumulated in fp32 from the row held in registers (mean
 * first, then the centred sum of squares); rows longer than a workgroup's
 * registers merge per-thread (count, mean, sum of squared deviations)
 * partials pairwise.  A row with var_r + eps == 0 gives NaN (0 * inf), as the
 * definition does.  weight, bias, mean and rstd must not overlap `out`.
 * Layout, in-place use, alignment, streams and errors as softmax_fwd.
 */
int layernorm_fwd(const void *in, void *out, int64_t rows, int64_t cols, int dtype, float eps,
                  const void *weight, const void *bias, float *mean, float *rstd, void *stream);

/*
 * rmsnorm_fwd -- RMSNorm along the last dimension (named beside LayerNorm on
 * the DCU case-study page, section 9):
 *     rstd_r = 1 / sqrt((1/cols) sum_j X[r, j]^2 + eps),
 *     Y[r, j] = X[r, j] * rstd_r * W[j]
 * Arguments as layernorm_fwd (no bias, no mean).
 */
int rmsnorm_fwd(const void *in, void *out, int64_t rows, int64_t cols, int dtype, float eps,
                const void *weight, float *rstd, void *stream);

/*
 * layernorm_fwd_kernel, rmsnorm_fwd_kernel -- as above with a forced kernel:
 * RWS_KERNEL_AUTO, RWS_KERNEL_WAVE_ROW (row in one lane group's registers,
 * window up to 512 granules), RWS_KERNEL_BLOCK_ONEPASS (row in one
 * workgroup's registers, up to 4096 granules), RWS_KERNEL_TWO_PASS (any
 * length; the row is read twice) or RWS_KERNEL_SPLITK_ORDERED (several
 * workgroups per row in one launch, chunk statistics published as
 * epoch-tagged words; the dispatcher's choice for few long rows) or
 * RWS_KERNEL_TILE_ROWS (several short rows per wave, as for softmax_fwd;
 * in and out 16-byte aligned, no weight or bias; the dispatcher's choice
 * for many short rows that are not line-aligned, without weight and bias).
 * Other ids: RWS_ERR_INVALID_ARG; a row too long for the forced kernel, or
 * weight/bias with RWS_KERNEL_TILE_ROWS: RWS_ERR_UNSUPPORTED_SHAPE.
 */
int layernorm_fwd_kernel(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                         float eps, const void *weight, const void *bias, float *mean, float *rstd,
                         void *stream, int kernel_id);
int rmsnorm_fwd_kernel(const void *in, void *out, int64_t rows, int64_t cols, int dtype, float eps,
                       const void *weight, float *rstd, void *stream, int kernel_id);

/*
 * softmax_select_kernel -- the family softmax_fwd would run for this shape
 * with pointers `in` and `out` (their alignment matters), on the current
 * device.  Returns a RWS_KERNEL_* id (> 0), or a negative status on invalid
 * arguments.  Performs no GPU work.
 */
int softmax_select_kernel(int64_t rows, int64_t cols, int dtype, const void *in,
                          const void *out);

/*
 * softmax_describe_launch -- writes a one-line, NUL-terminated description of
 * the launch softmax_fwd_kernel(kernel_id) would make (variant, grid, block,
 * chunks) into buf (at most buflen bytes).  Returns RWS_OK or an error
 * status.  Performs no GPU work.
 */
int softmax_describe_launch(int64_t rows, int64_t cols, int dtype, const void *in,
                            const void *out, int kernel_id, char *buf, int64_t buflen);

/*
 * softmax_describe_launch_masked -- the same for the launch
 * softmax_fwd_masked(kernel_id) would make (the masked form may choose
 * another variant of the family).  Performs no GPU work.
 */
int softmax_describe_launch_masked(int64_t rows, int64_t cols, int dtype, const void *in,
                                   const void *out, int kernel_id, char *buf, int64_t buflen);

/*
 * softmax_fwd_variant -- as softmax_fwd_kernel(kernel_id), with entry
 * `variant` (0 .. softmax_variant_count(kernel_id) - 1) of that family's
 * compiled shapes instead of the dispatcher's choice: lane-group size and
 * granules per lane (wave_row), workgroup size and granules per thread
 * (block_onepass, two_pass), chunk shape (the split-k forms).  The
 * measurement surface that lets both candidates of a dispatcher threshold be
 * timed and profiled on one shape.  RWS_ERR_INVALID_ARG for RWS_KERNEL_AUTO
 * or variant < 0, RWS_ERR_UNSUPPORTED_SHAPE when the variant cannot hold the
 * row (or its split-k grid would not fit).  Arguments otherwise as
 * softmax_fwd_kernel.
 */
int softmax_fwd_variant(const void *in, void *out, int64_t rows, int64_t cols, int dtype,
                        void *stream, int kernel_id, int variant);

/* Number of compiled variants of a kernel family (0 for RWS_KERNEL_AUTO or an
 * unknown id).  No GPU work. */
int softmax_variant_count(int kernel_id);

/* The launch softmax_fwd_variant would make, as softmax_describe_launch.
 * No GPU work. */
int softmax_describe_variant(int64_t rows, int64_t cols, int dtype, const void *in,
                             const void *out, int kernel_id, int variant, char *buf,
                             int64_t buflen);

/*
 * softmax_bwd_describe_launch -- the same for the launch
 * softmax_bwd_kernel(kernel_id) would make with these y and dx pointers
 * (bwd_wave, bwd_block, bwd_stream or bwd_ordered, with its shape).
 * kernel_id: RWS_KERNEL_AUTO, _WAVE_ROW, _BLOCK_ONEPASS, _TWO_PASS or
 * _SPLITK_ORDERED.  Performs no GPU work.
 */
int softmax_bwd_describe_launch(int64_t rows, int64_t cols, int dtype, const void *y,
                                const void *dx, int kernel_id, char *buf, int64_t buflen);

/*
 * norm_describe_launch -- the same for the launch layernorm_fwd_kernel /
 * rmsnorm_fwd_kernel(kernel_id) would make on these tensors (both use the
 * same choice: norm_wave, norm_block, norm_stream or norm_ordered, with its
 * shape).
 * affine: nonzero when a weight and/or bias is passed (it can change the
 * lane group).  kernel_id: RWS_KERNEL_AUTO, _WAVE_ROW, _BLOCK_ONEPASS,
 * _TWO_PASS or _SPLITK_ORDERED.  Performs no GPU work.
 */
int norm_describe_launch(int64_t rows, int64_t cols, int dtype, const void *in, const void *out,
                         int affine, int kernel_id, char *buf, int64_t buflen);

/* Name of a kernel family ("wave_row", ...), or "unknown". Static storage. */
const char *softmax_kernel_name(int kernel_id);

/* Text of a status code. Static storage. */
const char *softmax_status_string(int status);

/* Detail of the last error on this thread ("" if none). */
const char *softmax_last_error(void);

/*
 * softmax_stream_status -- whether a single-launch split-k launch on `stream`
 * (RWS_KERNEL_SPLITK_ORDERED of softmax_fwd, softmax_bwd, layernorm_fwd and
 * rmsnorm_fwd, or RWS_KERNEL_SPLITK_FUSED) gave up waiting for its row's
 * partials since the last query.  Such a launch cannot report through the
 * call that enqueued it (the kernel runs after the call returns): its
 * workgroup writes NaN for its chunk and sets a status word of the stream's,
 * which this call reads.  It synchronises `stream`, reads and clears the
 * word, and returns RWS_OK, or RWS_ERR_WAIT_TIMEOUT with the detail in
 * softmax_last_error(), or RWS_ERR_HIP.  A stream that never ran such a
 * launch gives RWS_OK at once.  Not for use while `stream` is being
 * captured into a graph (it synchronises).
 */
int softmax_stream_status(void *stream);

/*
 * softmax_set_wait_limit -- tries of one poll of the single-launch split-k
 * forms before a wait gives up, for launches enqueued after this call from
 * any thread: `tries` >= 0 (0 gives up at once, so every stage-2 workgroup
 * writes NaN and reports; for tests of the reporting path), or < 0 for the
 * default (2^21 tries, at least ~0.5 s).  Returns RWS_OK, or
 * RWS_ERR_INVALID_ARG above 2^32 - 1.  No GPU work.
 */
int softmax_set_wait_limit(int64_t tries);

/*
 * softmax_copy_bytes -- plain device-to-device copy of `bytes` bytes with
 * 16-byte non-temporal loads and stores, written through when `out` is
 * 128-byte aligned (both pointers 16-byte aligned, bytes % 16 == 0), on
 * `stream`.  It is the reference point for the effective-bandwidth figure
 * (bytes read plus bytes written per unit time, DCU case-study page, sections
 * 3.2 and 5.3): the copy ceiling, and the calibration of hardware traffic
 * counters.  Returns RWS_OK or an error status.
 */
int softmax_copy_bytes(const void *in, void *out, int64_t bytes, void *stream);

/*
 * softmax_read_bytes, softmax_write_bytes -- a pure read stream (`bytes` of
 * `in` read non-temporally, nothing written) and a pure write stream
 * (`bytes` of `out` overwritten with a pattern of the 16-byte granule index,
 * written through when `out` is 128-byte aligned), with 16-byte accesses and
 * 16 KiB per workgroup, on `stream`: the HBM ceilings of reading alone and
 * of writing alone beside the copy's mixed stream.  Pointers and `bytes`
 * 16-byte aligned.  Returns RWS_OK or an error status.
 */
int softmax_read_bytes(const void *in, int64_t bytes, void *stream);
int softmax_write_bytes(void *out, int64_t bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ROW_WISE_SOFTMAX_H */
