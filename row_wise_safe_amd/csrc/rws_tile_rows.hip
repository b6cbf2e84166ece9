// rws_tile_rows.hip -- the tile_rows forms (rws_tile.hpp): several short rows
// per wave as one 16-byte-aligned range, for rows that are not line-aligned.
//
//   softmax     row max, then the exponentials against each element's row
//               maximum and their row sum, then the scaling -- the row-wise
//               definition (CUDA safe-online-softmax page, section 1) with
//               the reductions segmented by row
//   backward    dot = sum_j dy_j * y_j per row, dx_j = y_j * (dy_j - dot)
//   LayerNorm   mean, then the sum of squared deviations from it (the
//               two-pass form the other normalisation kernels use)
//   RMSNorm     mean square; no weight or bias here (those rows take the
//               other forms)
#include "rws_launch.hpp"
#include "rws_norm.hpp"
#include "rws_tile.hpp"

namespace rws {

// ---------------------------------------------------------------------------
// softmax
// ---------------------------------------------------------------------------
template <int DT, int T, int K, bool FULL>
__device__ inline void tile_softmax(const char* __restrict__ gin, char* __restrict__ gout,
                                    int nrows, int cols, uint64_t cmagic, float* part_a,
                                    float* part_b, float* row_max, float* row_rcp) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, T, K> S(nrows, cols, cmagic);
    u32x4 raw[K];
#pragma unroll
    for (int i = 0; i < K; ++i) raw[i] = tile_load<DT, FULL>(gin, S.granule(i), S.nel);

    // widen; slots past the tile are -inf (they belong to no row)
    float v[K][VEC];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        Elem<DT>::widen(raw[i], v[i]);
        const int x = S.granule(i) * VEC;
        if (x + VEC > S.nel) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i][e] = x + e < S.nel ? v[i][e] : kNegInf;
        }
    }

    // row maxima
    float pa[K], pb[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        pa[i] = kNegInf;
        pb[i] = kNegInf;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool in_a = S.in_a(i, e);
            pa[i] = vmax(pa[i], in_a ? v[i][e] : kNegInf);
            pb[i] = vmax(pb[i], in_a ? kNegInf : v[i][e]);
        }
    }
    tile_fold<T, K, OpMax>(pa, pb, part_a, part_b, row_max, cols, nrows, VEC, kNegInf,
                           [](float m) { return m; });

    // exponentials against each element's row maximum (one exp2 per element:
    // the FMA offset of the element's row is selected first; a granule with
    // a row whose maximum takes the exact form -- |max| above 2.9e6 or
    // +inf -- takes it per element), row sums
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const RowExp ea(row_max[S.ra[i]]), eb(row_max[S.rb(i)]);
        pa[i] = 0.0f;
        pb[i] = 0.0f;
        if (__builtin_expect(ea.big || eb.big, 0)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                const float y = in_a ? ea.one(v[i][e]) : eb.one(v[i][e]);
                v[i][e] = y;
                pa[i] += in_a ? y : 0.0f;
                pb[i] += in_a ? 0.0f : y;
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                const float y = __builtin_amdgcn_exp2f(
                    __builtin_fmaf(v[i][e], kLog2e, in_a ? ea.negc : eb.negc));
                v[i][e] = y;
                pa[i] += in_a ? y : 0.0f;
                pb[i] += in_a ? 0.0f : y;
            }
        }
    }
    tile_fold<T, K, OpSum>(pa, pb, part_a, part_b, row_rcp, cols, nrows, VEC, 0.0f,
                           [](float s) { return __builtin_amdgcn_rcpf(s); });

    // scale and store
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float qa = row_rcp[S.ra[i]], qb = row_rcp[S.rb(i)];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] *= S.in_a(i, e) ? qa : qb;
        tile_store<DT, FULL>(gout, S.granule(i), S.nel, v[i]);
    }
}

template <int DT, int T, int K>
__global__ __launch_bounds__(64) void k_tile_rows(const void* __restrict__ in,
                                                  void* __restrict__ out, int64_t rows, int cols,
                                                  uint64_t cmagic) {
    __shared__ float part_a[64 * K];  // per granule: its first row's partial
    __shared__ float part_b[64 * K];  // per granule: the next row's partial
    __shared__ float row_max[T];
    __shared__ float row_rcp[T];
    const int64_t row0 = (int64_t)blockIdx.x * T;
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gin = (const char*)in + off;
    char* gout = (char*)out + off;
    if (rows - row0 >= T)
        tile_softmax<DT, T, K, true>(gin, gout, T, cols, cmagic, part_a, part_b, row_max, row_rcp);
    else
        tile_softmax<DT, T, K, false>(gin, gout, (int)(rows - row0), cols, cmagic, part_a, part_b,
                                      row_max, row_rcp);
}

// ---------------------------------------------------------------------------
// softmax backward
// ---------------------------------------------------------------------------
template <int DT, int T, int K, bool FULL>
__device__ inline void tile_backward(const char* __restrict__ gy, const char* __restrict__ gdy,
                                     char* __restrict__ gdx, int nrows, int cols, uint64_t cmagic,
                                     float* part_a, float* part_b, float* row_dot) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, T, K> S(nrows, cols, cmagic);
    u32x4 ry[K], rdy[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        ry[i] = tile_load<DT, FULL>(gy, S.granule(i), S.nel);
        rdy[i] = tile_load<DT, FULL>(gdy, S.granule(i), S.nel);
    }
    // slots past the tile load as 0 and add nothing
    float y[K][VEC], d[K][VEC];
    float pa[K], pb[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        Elem<DT>::widen(ry[i], y[i]);
        Elem<DT>::widen(rdy[i], d[i]);
        pa[i] = 0.0f;
        pb[i] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float p = y[i][e] * d[i][e];
            const bool in_a = S.in_a(i, e);
            pa[i] += in_a ? p : 0.0f;
            pb[i] += in_a ? 0.0f : p;
        }
    }
    tile_fold<T, K, OpSum>(pa, pb, part_a, part_b, row_dot, cols, nrows, VEC, 0.0f,
                           [](float s) { return s; });
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float sa = row_dot[S.ra[i]], sb = row_dot[S.rb(i)];
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = y[i][e] * (d[i][e] - (S.in_a(i, e) ? sa : sb));
        tile_store<DT, FULL>(gdx, S.granule(i), S.nel, o);
    }
}

template <int DT, int T, int K>
__global__ __launch_bounds__(64) void k_bwd_tile(const void* __restrict__ y,
                                                 const void* __restrict__ dy,
                                                 void* __restrict__ dx, int64_t rows, int cols,
                                                 uint64_t cmagic) {
    __shared__ float part_a[64 * K];
    __shared__ float part_b[64 * K];
    __shared__ float row_dot[T];
    const int64_t row0 = (int64_t)blockIdx.x * T;
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gy = (const char*)y + off;
    const char* gdy = (const char*)dy + off;
    char* gdx = (char*)dx + off;
    if (rows - row0 >= T)
        tile_backward<DT, T, K, true>(gy, gdy, gdx, T, cols, cmagic, part_a, part_b, row_dot);
    else
        tile_backward<DT, T, K, false>(gy, gdy, gdx, (int)(rows - row0), cols, cmagic, part_a,
                                       part_b, row_dot);
}

// ---------------------------------------------------------------------------
// LayerNorm / RMSNorm without weight and bias
// ---------------------------------------------------------------------------
template <int DT, int T, int K, int MODE, bool FULL>
__device__ inline void tile_norm(const char* __restrict__ gin, char* __restrict__ gout, int nrows,
                                 int cols, uint64_t cmagic, const NormArgs& A, int64_t row0,
                                 float* part_a, float* part_b, float* row_mu, float* row_rstd) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, T, K> S(nrows, cols, cmagic);
    u32x4 raw[K];
#pragma unroll
    for (int i = 0; i < K; ++i) raw[i] = tile_load<DT, FULL>(gin, S.granule(i), S.nel);
    // slots past the tile load as 0; their partials are never folded into a row
    float v[K][VEC];
    float pa[K], pb[K];
    if (MODE == kLayerNorm) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
            Elem<DT>::widen(raw[i], v[i]);
            pa[i] = 0.0f;
            pb[i] = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                pa[i] += in_a ? v[i][e] : 0.0f;
                pb[i] += in_a ? 0.0f : v[i][e];
            }
        }
        const float n = A.n;
        tile_fold<T, K, OpSum>(pa, pb, part_a, part_b, row_mu, cols, nrows, VEC, 0.0f,
                               [n](float s) { return s / n; });
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const float ma = row_mu[S.ra[i]], mb = row_mu[S.rb(i)];
            pa[i] = 0.0f;
            pb[i] = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                const float c = v[i][e] - (in_a ? ma : mb);
                pa[i] = in_a ? __builtin_fmaf(c, c, pa[i]) : pa[i];
                pb[i] = in_a ? pb[i] : __builtin_fmaf(c, c, pb[i]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < K; ++i) {
            Elem<DT>::widen(raw[i], v[i]);
            pa[i] = 0.0f;
            pb[i] = 0.0f;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                pa[i] = in_a ? __builtin_fmaf(v[i][e], v[i][e], pa[i]) : pa[i];
                pb[i] = in_a ? pb[i] : __builtin_fmaf(v[i][e], v[i][e], pb[i]);
            }
        }
    }
    const NormArgs Ac = A;
    tile_fold<T, K, OpSum>(pa, pb, part_a, part_b, row_rstd, cols, nrows, VEC, 0.0f,
                           [Ac](float q) { return norm_rstd(q, Ac); });
    const int lane = threadIdx.x;
    if (lane < nrows) {
        if (MODE == kLayerNorm && A.mean) A.mean[row0 + lane] = row_mu[lane];
        if (A.rstd) A.rstd[row0 + lane] = row_rstd[lane];
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float ra = row_rstd[S.ra[i]], rb = row_rstd[S.rb(i)];
        float o[VEC];
        if (MODE == kLayerNorm) {
            const float ma = row_mu[S.ra[i]], mb = row_mu[S.rb(i)];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = S.in_a(i, e);
                o[e] = (v[i][e] - (in_a ? ma : mb)) * (in_a ? ra : rb);
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = v[i][e] * (S.in_a(i, e) ? ra : rb);
        }
        tile_store<DT, FULL>(gout, S.granule(i), S.nel, o);
    }
}

template <int DT, int T, int K, int MODE>
__global__ __launch_bounds__(64) void k_norm_tile(const void* __restrict__ in,
                                                  void* __restrict__ out, int64_t rows, int cols,
                                                  uint64_t cmagic, NormArgs A) {
    __shared__ float part_a[64 * K];
    __shared__ float part_b[64 * K];
    __shared__ float row_mu[T];
    __shared__ float row_rstd[T];
    const int64_t row0 = (int64_t)blockIdx.x * T;
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gin = (const char*)in + off;
    char* gout = (char*)out + off;
    if (rows - row0 >= T)
        tile_norm<DT, T, K, MODE, true>(gin, gout, T, cols, cmagic, A, row0, part_a, part_b, row_mu,
                                        row_rstd);
    else
        tile_norm<DT, T, K, MODE, false>(gin, gout, (int)(rows - row0), cols, cmagic, A, row0,
                                         part_a, part_b, row_mu, row_rstd);
}

// ---------------------------------------------------------------------------
// variants and launchers
// ---------------------------------------------------------------------------
// (rows per tile, granules per lane)
#define RWS_TILE_ROWS_VARIANTS(X) \
    X(4, 1) X(4, 2) X(4, 4)       \
    X(8, 1) X(8, 2) X(8, 4)       \
    X(16, 1) X(16, 2) X(16, 4)

#define RWS_ROW(t, k) {t, k},
const TileRowsVariant kTileRows[] = {RWS_TILE_ROWS_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumTileRows = sizeof(kTileRows) / sizeof(kTileRows[0]);

template <int DT, int T, int K>
static hipError_t go(const Launch& L) {
    const int64_t tiles = (L.rows + T - 1) / T;
    hipLaunchKernelGGL((k_tile_rows<DT, T, K>), dim3((unsigned)tiles), dim3(64), 0, L.stream, L.in,
                       L.out, L.rows, L.cols, remainder_magic((uint64_t)L.cols));
    return hipGetLastError();
}

template <int DT, int T, int K>
static hipError_t go_bwd(const BwdLaunch& B) {
    const int64_t tiles = (B.rows + T - 1) / T;
    hipLaunchKernelGGL((k_bwd_tile<DT, T, K>), dim3((unsigned)tiles), dim3(64), 0, B.stream, B.y,
                       B.dy, B.dx, B.rows, B.cols, remainder_magic((uint64_t)B.cols));
    return hipGetLastError();
}

template <int DT, int T, int K>
static hipError_t go_norm(const NormLaunch& N) {
    const int64_t tiles = (N.rows + T - 1) / T;
    const uint64_t M = remainder_magic((uint64_t)N.cols);
    if (N.mode == kLayerNorm)
        hipLaunchKernelGGL((k_norm_tile<DT, T, K, kLayerNorm>), dim3((unsigned)tiles), dim3(64), 0,
                           N.stream, N.in, N.out, N.rows, N.cols, M, N.args);
    else
        hipLaunchKernelGGL((k_norm_tile<DT, T, K, kRmsNorm>), dim3((unsigned)tiles), dim3(64), 0,
                           N.stream, N.in, N.out, N.rows, N.cols, M, N.args);
    return hipGetLastError();
}

template <int T, int K>
static hipError_t go_any(const Launch& L) {
    switch (L.dtype) {
        case kF32: return go<kF32, T, K>(L);
        case kF16: return go<kF16, T, K>(L);
        case kBF16: return go<kBF16, T, K>(L);
    }
    return hipErrorInvalidValue;
}

template <int T, int K>
static hipError_t go_bwd_any(const BwdLaunch& B) {
    switch (B.dtype) {
        case kF32: return go_bwd<kF32, T, K>(B);
        case kF16: return go_bwd<kF16, T, K>(B);
        case kBF16: return go_bwd<kBF16, T, K>(B);
    }
    return hipErrorInvalidValue;
}

template <int T, int K>
static hipError_t go_norm_any(const NormLaunch& N) {
    switch (N.dtype) {
        case kF32: return go_norm<kF32, T, K>(N);
        case kF16: return go_norm<kF16, T, K>(N);
        case kBF16: return go_norm<kBF16, T, K>(N);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_tile_rows(const Launch& L, int variant) {
    int i = 0;
#define RWS_CASE(t, k) \
    if (variant == i) return go_any<t, k>(L); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(const BwdLaunch& B, int variant) {
    int i = 0;
#define RWS_CASE(t, k) \
    if (variant == i) return go_bwd_any<t, k>(B); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_norm_tile(const NormLaunch& N, int variant) {
    int i = 0;
#define RWS_CASE(t, k) \
    if (variant == i) return go_norm_any<t, k>(N); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
