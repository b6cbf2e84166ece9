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

// Maxima of granule values v over its first row's elements (e < split) and
// over the next row's, each as a tree of three-operand maxima.  `ninf` is
// -inf held in a register the compiler cannot see through: with the
// constant, it rewrites max(x, e < split ? v : -inf) into a select of two
// maxima per element, which the trees avoid.
template <int VEC>
__device__ inline void split_max(const float (&v)[VEC], int split, float ninf, float& ma,
                                 float& mb) {
    float a[VEC], b[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const bool in_a = e < split;
        a[e] = in_a ? v[e] : ninf;
        b[e] = in_a ? ninf : v[e];
    }
    if (VEC == 8) {
        ma = vmax(vmax(vmax(a[0], a[1]), a[2]), vmax(vmax(a[3], a[4]), vmax(vmax(a[5], a[6]), a[7])));
        mb = vmax(vmax(vmax(b[0], b[1]), b[2]), vmax(vmax(b[3], b[4]), vmax(vmax(b[5], b[6]), b[7])));
    } else {
        ma = vmax(vmax(vmax(a[0], a[1]), a[2]), a[VEC - 1]);
        mb = vmax(vmax(vmax(b[0], b[1]), b[2]), b[VEC - 1]);
    }
}

// The exponentials of a tile against each element's row maximum (one exp2
// per element: the FMA offset of the element's row is selected first) and
// their row partials.  When a granule slot of any lane holds a row whose
// maximum takes RowExp's exact form (|max| above 2.9e6, or +inf / NaN), the
// whole wave takes, for that slot, the path where every element picks its
// row's form (a ballot keeps the branch uniform over the wave; both paths
// give the same value for a row on the FMA form).
template <int DT, int K>
__device__ inline void tile_exp(float (&v)[K][Elem<DT>::VEC], const TileSlots<DT, K>& S,
                                const float* row_max, float (&pa)[K], float (&pb)[K]) {
    constexpr int VEC = Elem<DT>::VEC;
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const RowExp ea(row_max[S.ra[i]]), eb(row_max[S.rb(i)]);
        const int sp = S.split_pass(i);
        pa[i] = 0.0f;
        pb[i] = 0.0f;
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(ea.big || eb.big) != 0, 0)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                const float y = in_a ? ea.one(v[i][e]) : eb.one(v[i][e]);
                v[i][e] = y;
                pa[i] += in_a ? y : 0.0f;
                pb[i] += in_a ? 0.0f : y;
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                const float y = __builtin_amdgcn_exp2f(
                    __builtin_fmaf(v[i][e], kLog2e, in_a ? ea.negc : eb.negc));
                v[i][e] = y;
                pa[i] += in_a ? y : 0.0f;
                pb[i] += in_a ? 0.0f : y;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// softmax
// ---------------------------------------------------------------------------
// The row-wise softmax of a tile widened into v: row maxima, the
// exponentials and row sums, the scaling, the stores.  Slots past the tile
// (and, in the tensor's last tile, elements past its end) may hold any
// value: their partials are never folded into a row and they are never
// stored.
template <int DT, int K, bool FULL>
__device__ inline void tile_softmax_rows(float (&v)[K][Elem<DT>::VEC], const TileSlots<DT, K>& S,
                                         char* __restrict__ gout, int nrows, int cols, int lg,
                                         float* part_a, float* part_b, float* row_max,
                                         float* row_rcp) {
    constexpr int VEC = Elem<DT>::VEC;
    static_assert(VEC == 8 || VEC == 4, "granule of 4 or 8 elements");
    // row maxima
    float ninf = kNegInf;
    asm volatile("" : "+v"(ninf));
    float pa[K], pb[K];
#pragma unroll
    for (int i = 0; i < K; ++i) split_max<VEC>(v[i], S.split_pass(i), ninf, pa[i], pb[i]);
    tile_fold<K, OpMax>(pa, pb, part_a, part_b, row_max, cols, nrows, lg, VEC, kNegInf,
                        [](float m) { return m; });

    // exponentials and row sums
    tile_exp<DT, K>(v, S, row_max, pa, pb);
    tile_fold<K, OpSum>(pa, pb, part_a, part_b, row_rcp, cols, nrows, lg, VEC, 0.0f,
                        [](float s) { return __builtin_amdgcn_rcpf(s); });

    // scale and store
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float qa = row_rcp[S.ra[i]], qb = row_rcp[S.rb(i)];
        const int sp = S.split_pass(i);
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] *= e < sp ? qa : qb;
        tile_store<DT, FULL>(gout, S.granule(i), S.nel, v[i]);
    }
}

template <int DT, int K, bool FULL>
__device__ inline void tile_softmax(const char* __restrict__ gin, char* __restrict__ gout,
                                    int nrows, int cols, int lg, uint64_t cmagic, float* part_a,
                                    float* part_b, float* row_max, float* row_rcp) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, K> S(nrows, cols, cmagic);
    u32x4 raw[K];
#pragma unroll
    for (int i = 0; i < K; ++i) raw[i] = tile_load<DT, FULL>(gin, S.granule(i), S.nel);
    float v[K][VEC];
#pragma unroll
    for (int i = 0; i < K; ++i) Elem<DT>::widen(raw[i], v[i]);
    tile_softmax_rows<DT, K, FULL>(v, S, gout, nrows, cols, lg, part_a, part_b, row_max, row_rcp);
}

// ---------------------------------------------------------------------------
// masked softmax: z = scale * x + mask[row mod mask_rows, col], and -inf past
// a row's causal limit (col > (row mod causal_q) + cols - causal_q), the
// prologue of the masked entry point (rws_pre.hpp gives it to the other
// forms), then the tile softmax above
// ---------------------------------------------------------------------------
struct TileMask {
    float scale;
    const char* mask;      // nullptr: no additive mask
    const char* mask_end;  // one past the mask's mask_rows * cols elements
    int64_t mask_rows;
    int64_t causal_q;      // 0: no causal limit
    int64_t row_base;      // global index of the launch's first row
    uint64_t mask_M;       // remainder_magic(mask_rows)
    uint64_t causal_M;     // remainder_magic(causal_q) when causal_q > 0
};

// Bytes [ph, ph + 16) of the 32 bytes lo ++ hi; ph in 1..15, uniform.
__device__ inline u32x4 tile_shift16(u32x4 lo, u32x4 hi, int ph) {
    const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const uint32_t b = (uint32_t)(ph & 3);
    u32x4 r;
    switch (ph >> 2) {
#define RWS_SH(q)                                                                       \
    case q:                                                                             \
        r = u32x4{__builtin_amdgcn_alignbyte(w[q + 1], w[q], b),                        \
                  __builtin_amdgcn_alignbyte(w[q + 2], w[q + 1], b),                    \
                  __builtin_amdgcn_alignbyte(w[q + 3], w[q + 2], b),                    \
                  __builtin_amdgcn_alignbyte(w[q + 4], w[q + 3], b)};                   \
        break;
        RWS_SH(0) RWS_SH(1) RWS_SH(2)
#undef RWS_SH
        default:
            r = u32x4{__builtin_amdgcn_alignbyte(w[4], w[3], b),
                      __builtin_amdgcn_alignbyte(w[5], w[4], b),
                      __builtin_amdgcn_alignbyte(w[6], w[5], b),
                      __builtin_amdgcn_alignbyte(w[7], w[6], b)};
    }
    return r;
}

// How a tile reads its mask (uniform over the wave).  A tile's mask rows
// (grow0 + r) mod mask_rows follow each other unless they wrap inside the
// tile; then the tile's mask bytes are one range laid out like the input
// tile and are read granule by granule: one aligned load (kMaskWhole), or
// two and a byte shift when the range is not 16-byte aligned (kMaskShift,
// where the aligned pairs of the whole range lie inside the mask).  A tile
// whose mask rows wrap, the tensor's partial last tile, and a shifted range
// at an end of the mask read it element by element (kMaskElem).
enum { kMaskNone = 0, kMaskWhole = 1, kMaskShift = 2, kMaskElem = 3 };

// The prologue of a tile for one way of reading the mask (MODE) and with or
// without a causal limit: loads (every load first, the input's and the
// mask's, then the arithmetic) and z into v.  Element e of granule slot i
// takes part when e < split ? e <= ta : e <= tb: ta and tb come from the
// causal limits of the granule's two rows; no element of a row past the
// tile's last one takes part, nor any of a slot past the tile.  Without a
// causal limit every element of the tile takes part, and the values the
// others get are never used.  Granules of which no element takes part
// (past the causal limit of both their rows) load neither the input nor
// the mask.
template <int DT, int K, bool FULL, int MODE, bool CAUSAL>
__device__ inline void tile_masked_prologue(float (&v)[K][Elem<DT>::VEC],
                                            const TileSlots<DT, K>& S, const char* __restrict__ gin,
                                            const TileMask& P, const char* mtile, int mph,
                                            int cols, const int* row_lim,
                                            const int64_t* row_mrow) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ES = Elem<DT>::SIZE;
    int ta[K], tb[K];
    u32x4 raw[K], mlo[K], mhi[K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int j = S.granule(i);
        const int x = j * VEC;
        const int ra = S.ra[i];
        const int c0a = x - ra * cols;  // column of element 0 in row ra
        bool any = x < S.nel;
        if (CAUSAL) {
            const int sp = S.split_pass(i);
            ta[i] = row_lim[ra] - c0a;
            tb[i] = ra < S.last ? row_lim[ra + 1] - (c0a - cols) : -1;
            any = ta[i] >= 0 || (sp < VEC && tb[i] >= sp);
        }
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        mlo[i] = u32x4{0u, 0u, 0u, 0u};
        mhi[i] = u32x4{0u, 0u, 0u, 0u};
        if (any) {
            raw[i] = tile_load<DT, FULL>(gin, j, S.nel);
            // whole granules only (a full tile: every slot inside it)
            const char* p = mtile + (int64_t)j * 16;
            if (MODE == kMaskWhole) {
                mlo[i] = load16<false>(p);
            } else if (MODE == kMaskShift) {
                mlo[i] = load16<false>(p - mph);
                mhi[i] = load16<false>(p - mph + 16);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
        Elem<DT>::widen(raw[i], v[i]);
        float mv[VEC];
        if (MODE == kMaskWhole) {
            Elem<DT>::widen(mlo[i], mv);
        } else if (MODE == kMaskShift) {
            Elem<DT>::widen(tile_shift16(mlo[i], mhi[i], mph), mv);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) mv[e] = 0.0f;
        }
        const int sp = S.split_pass(i);
        if (MODE == kMaskElem) {
            const int x = S.granule(i) * VEC;
            const int ra = S.ra[i];
            const int c0a = x - ra * cols;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                const bool ok = CAUSAL ? (in_a ? e <= ta[i] : e <= tb[i])
                                       : x < S.nel && (in_a || ra < S.last);
                if (ok) {
                    const int64_t mr = row_mrow[in_a ? ra : ra + 1];
                    const int col = (in_a ? c0a : c0a - cols) + e;
                    mv[e] = Elem<DT>::load1(P.mask + (mr * cols + col) * ES);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (CAUSAL) {
                const bool ok = e < sp ? e <= ta[i] : e <= tb[i];
                v[i][e] = ok ? __builtin_fmaf(P.scale, v[i][e], mv[e]) : kNegInf;
            } else {
                v[i][e] = __builtin_fmaf(P.scale, v[i][e], mv[e]);
            }
        }
    }
}

template <int DT, int K, bool FULL, bool CAUSAL>
__device__ inline void tile_masked_prologue_any(int mode, float (&v)[K][Elem<DT>::VEC],
                                                const TileSlots<DT, K>& S, const char* gin,
                                                const TileMask& P, const char* mtile, int mph,
                                                int cols, const int* row_lim,
                                                const int64_t* row_mrow) {
    if (mode == kMaskNone)
        tile_masked_prologue<DT, K, FULL, kMaskNone, CAUSAL>(v, S, gin, P, mtile, mph, cols,
                                                            row_lim, row_mrow);
    else if (FULL && mode == kMaskWhole)
        tile_masked_prologue<DT, K, FULL, kMaskWhole, CAUSAL>(v, S, gin, P, mtile, mph, cols,
                                                             row_lim, row_mrow);
    else if (FULL && mode == kMaskShift)
        tile_masked_prologue<DT, K, FULL, kMaskShift, CAUSAL>(v, S, gin, P, mtile, mph, cols,
                                                             row_lim, row_mrow);
    else
        tile_masked_prologue<DT, K, FULL, kMaskElem, CAUSAL>(v, S, gin, P, mtile, mph, cols,
                                                            row_lim, row_mrow);
}

template <int DT, int K, bool FULL>
__device__ inline void tile_softmax_masked(const char* __restrict__ gin, char* __restrict__ gout,
                                           int nrows, int cols, int lg, uint64_t cmagic,
                                           const TileMask& P, int64_t grow0, float* part_a,
                                           float* part_b, float* row_max, float* row_rcp,
                                           int* row_lim, int64_t* row_mrow) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ES = Elem<DT>::SIZE;
    const TileSlots<DT, K> S(nrows, cols, cmagic);
    const int lane = threadIdx.x;
    // per tile row: the last column that takes part, and the mask row
    if (lane < nrows) {
        const int64_t g = grow0 + lane;
        row_lim[lane] = P.causal_q > 0
                            ? (int)row_mod(g, P.causal_q, P.causal_M) + cols - (int)P.causal_q
                            : cols - 1;
        row_mrow[lane] = P.mask ? row_mod(g, P.mask_rows, P.mask_M) : 0;
    }
    __syncthreads();
    const int64_t m0 = row_mrow[0];
    const char* mtile = P.mask + m0 * cols * ES;
    const int mph = (int)((uintptr_t)mtile & 15);
    int mode = kMaskNone;
    if (P.mask != nullptr) {
        mode = kMaskElem;
        if (FULL && m0 + nrows <= P.mask_rows) {
            if (mph == 0)
                mode = kMaskWhole;
            else if (mtile - mph >= P.mask &&
                     mtile - mph + (int64_t)nrows * cols * ES + 32 <= P.mask_end)
                mode = kMaskShift;
        }
    }
    float v[K][VEC];
    if (P.causal_q > 0)
        tile_masked_prologue_any<DT, K, FULL, true>(mode, v, S, gin, P, mtile, mph, cols, row_lim,
                                                    row_mrow);
    else
        tile_masked_prologue_any<DT, K, FULL, false>(mode, v, S, gin, P, mtile, mph, cols,
                                                     row_lim, row_mrow);
    tile_softmax_rows<DT, K, FULL>(v, S, gout, nrows, cols, lg, part_a, part_b, row_max, row_rcp);
}

// The tile a workgroup takes (XCD runs of 2^lgrun tiles, xcd_run) and its
// first row.
__device__ inline int64_t tile_row0(int T, int lgrun) {
    return xcd_run(blockIdx.x, gridDim.x, lgrun) * T;
}

template <int DT, int K>
__global__ __launch_bounds__(64) void k_tile_rows(const void* __restrict__ in,
                                                  void* __restrict__ out, int64_t rows, int cols,
                                                  uint64_t cmagic, int T, int lg, int lgrun) {
    __shared__ float part_a[64 * K];  // per granule: its first row's partial
    __shared__ float part_b[64 * K];  // per granule: the next row's partial
    __shared__ float row_max[kTileMaxT];
    __shared__ float row_rcp[kTileMaxT];
    const int64_t row0 = tile_row0(T, lgrun);
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gin = (const char*)in + off;
    char* gout = (char*)out + off;
    if (rows - row0 >= T)
        tile_softmax<DT, K, true>(gin, gout, T, cols, lg, cmagic, part_a, part_b, row_max, row_rcp);
    else
        tile_softmax<DT, K, false>(gin, gout, (int)(rows - row0), cols, lg, cmagic, part_a, part_b,
                                   row_max, row_rcp);
}

template <int DT, int K>
__global__ __launch_bounds__(64) void k_tile_rows_masked(const void* __restrict__ in,
                                                         void* __restrict__ out, int64_t rows,
                                                         int cols, uint64_t cmagic, int T, int lg,
                                                         int lgrun, TileMask P) {
    __shared__ float part_a[64 * K];
    __shared__ float part_b[64 * K];
    __shared__ float row_max[kTileMaxT];
    __shared__ float row_rcp[kTileMaxT];
    __shared__ int row_lim[kTileMaxT];
    __shared__ int64_t row_mrow[kTileMaxT];
    const int64_t row0 = tile_row0(T, lgrun);
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gin = (const char*)in + off;
    char* gout = (char*)out + off;
    if (rows - row0 >= T)
        tile_softmax_masked<DT, K, true>(gin, gout, T, cols, lg, cmagic, P, P.row_base + row0,
                                         part_a, part_b, row_max, row_rcp, row_lim, row_mrow);
    else
        tile_softmax_masked<DT, K, false>(gin, gout, (int)(rows - row0), cols, lg, cmagic, P,
                                          P.row_base + row0, part_a, part_b, row_max, row_rcp,
                                          row_lim, row_mrow);
}

// ---------------------------------------------------------------------------
// softmax backward
// ---------------------------------------------------------------------------
template <int DT, int K, bool FULL>
__device__ inline void tile_backward(const char* __restrict__ gy, const char* __restrict__ gdy,
                                     char* __restrict__ gdx, int nrows, int cols, int lg,
                                     uint64_t cmagic, float* part_a, float* part_b,
                                     float* row_dot) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, K> S(nrows, cols, cmagic);
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
        const int sp = S.split_pass(i);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const float p = y[i][e] * d[i][e];
            const bool in_a = e < sp;
            pa[i] += in_a ? p : 0.0f;
            pb[i] += in_a ? 0.0f : p;
        }
    }
    tile_fold<K, OpSum>(pa, pb, part_a, part_b, row_dot, cols, nrows, lg, VEC, 0.0f,
                        [](float s) { return s; });
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float sa = row_dot[S.ra[i]], sb = row_dot[S.rb(i)];
        const int sp = S.split_pass(i);
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = y[i][e] * (d[i][e] - (e < sp ? sa : sb));
        tile_store<DT, FULL>(gdx, S.granule(i), S.nel, o);
    }
}

template <int DT, int K>
__global__ __launch_bounds__(64) void k_bwd_tile(const void* __restrict__ y,
                                                 const void* __restrict__ dy,
                                                 void* __restrict__ dx, int64_t rows, int cols,
                                                 uint64_t cmagic, int T, int lg, int lgrun) {
    __shared__ float part_a[64 * K];
    __shared__ float part_b[64 * K];
    __shared__ float row_dot[kTileMaxT];
    const int64_t row0 = tile_row0(T, lgrun);
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gy = (const char*)y + off;
    const char* gdy = (const char*)dy + off;
    char* gdx = (char*)dx + off;
    if (rows - row0 >= T)
        tile_backward<DT, K, true>(gy, gdy, gdx, T, cols, lg, cmagic, part_a, part_b, row_dot);
    else
        tile_backward<DT, K, false>(gy, gdy, gdx, (int)(rows - row0), cols, lg, cmagic, part_a,
                                    part_b, row_dot);
}

// ---------------------------------------------------------------------------
// LayerNorm / RMSNorm without weight and bias
// ---------------------------------------------------------------------------
template <int DT, int K, int MODE, bool FULL>
__device__ inline void tile_norm(const char* __restrict__ gin, char* __restrict__ gout, int nrows,
                                 int cols, int lg, uint64_t cmagic, const NormArgs& A,
                                 int64_t row0, float* part_a, float* part_b, float* row_mu,
                                 float* row_rstd) {
    constexpr int VEC = Elem<DT>::VEC;
    const TileSlots<DT, K> S(nrows, cols, cmagic);
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
            const int sp = S.split_pass(i);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                pa[i] += in_a ? v[i][e] : 0.0f;
                pb[i] += in_a ? 0.0f : v[i][e];
            }
        }
        const float n = A.n;
        tile_fold<K, OpSum>(pa, pb, part_a, part_b, row_mu, cols, nrows, lg, VEC, 0.0f,
                            [n](float s) { return s / n; });
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const float ma = row_mu[S.ra[i]], mb = row_mu[S.rb(i)];
            pa[i] = 0.0f;
            pb[i] = 0.0f;
            const int sp = S.split_pass(i);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
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
            const int sp = S.split_pass(i);
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                pa[i] = in_a ? __builtin_fmaf(v[i][e], v[i][e], pa[i]) : pa[i];
                pb[i] = in_a ? pb[i] : __builtin_fmaf(v[i][e], v[i][e], pb[i]);
            }
        }
    }
    const NormArgs Ac = A;
    tile_fold<K, OpSum>(pa, pb, part_a, part_b, row_rstd, cols, nrows, lg, VEC, 0.0f,
                        [Ac](float q) { return norm_rstd(q, Ac); });
    const int lane = threadIdx.x;
    if (lane < nrows) {
        if (MODE == kLayerNorm && A.mean) A.mean[row0 + lane] = row_mu[lane];
        if (A.rstd) A.rstd[row0 + lane] = row_rstd[lane];
    }
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const float ra = row_rstd[S.ra[i]], rb = row_rstd[S.rb(i)];
        const int sp = S.split_pass(i);
        float o[VEC];
        if (MODE == kLayerNorm) {
            const float ma = row_mu[S.ra[i]], mb = row_mu[S.rb(i)];
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < sp;
                o[e] = (v[i][e] - (in_a ? ma : mb)) * (in_a ? ra : rb);
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = v[i][e] * (e < sp ? ra : rb);
        }
        tile_store<DT, FULL>(gout, S.granule(i), S.nel, o);
    }
}

template <int DT, int K, int MODE>
__global__ __launch_bounds__(64) void k_norm_tile(const void* __restrict__ in,
                                                  void* __restrict__ out, int64_t rows, int cols,
                                                  uint64_t cmagic, int T, int lg, int lgrun,
                                                  NormArgs A) {
    __shared__ float part_a[64 * K];
    __shared__ float part_b[64 * K];
    __shared__ float row_mu[kTileMaxT];
    __shared__ float row_rstd[kTileMaxT];
    const int64_t row0 = tile_row0(T, lgrun);
    const int64_t off = row0 * cols * Elem<DT>::SIZE;
    const char* gin = (const char*)in + off;
    char* gout = (char*)out + off;
    if (rows - row0 >= T)
        tile_norm<DT, K, MODE, true>(gin, gout, T, cols, lg, cmagic, A, row0, part_a, part_b,
                                     row_mu, row_rstd);
    else
        tile_norm<DT, K, MODE, false>(gin, gout, (int)(rows - row0), cols, lg, cmagic, A, row0,
                                      part_a, part_b, row_mu, row_rstd);
}

// ---------------------------------------------------------------------------
// variants and launchers
// ---------------------------------------------------------------------------
// granules per lane
#define RWS_TILE_ROWS_VARIANTS(X) X(1) X(2) X(3) X(4)

#define RWS_ROW(k) {k},
const TileRowsVariant kTileRows[] = {RWS_TILE_ROWS_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumTileRows = sizeof(kTileRows) / sizeof(kTileRows[0]);

// log2 of the lanes that fold one row: the largest power of two g with
// g * T <= 64 (T >= 4, so at most 16 lanes)
static int tile_lg(int T) {
    int lg = 0;
    while (lg < 4 && (T << (lg + 1)) <= 64) ++lg;
    return lg;
}

// The shape the kernels assume: 4..64 rows per tile, tiles of whole
// granules (so every tile starts 16-byte aligned), at most 64 * K of them,
// fewer than 2^31 tiles.
static bool tile_ok(const TileShape& t, int64_t rows, int cols, int es, int K) {
    const int64_t bytes = (int64_t)t.T * cols * es;
    return t.T >= 4 && t.T <= kTileMaxT && rows > 0 && cols * es >= 16 && bytes % 16 == 0 &&
           bytes / 16 <= 64LL * K && (rows + t.T - 1) / t.T < ((int64_t)1 << 31) &&
           t.lgrun >= 0 && t.lgrun <= 10;
}

template <int DT, int K>
static hipError_t go(const Launch& L, const TileShape& t) {
    if (!tile_ok(t, L.rows, L.cols, Elem<DT>::SIZE, K)) return hipErrorInvalidValue;
    const int64_t tiles = (L.rows + t.T - 1) / t.T;
    hipLaunchKernelGGL((k_tile_rows<DT, K>), dim3((unsigned)tiles), dim3(64), 0, L.stream, L.in,
                       L.out, L.rows, L.cols, remainder_magic((uint64_t)L.cols), t.T, tile_lg(t.T),
                       t.lgrun);
    return hipGetLastError();
}

template <int DT, int K>
static hipError_t go_masked(const Launch& L, const TileShape& t, const MaskArgs& M) {
    if (!tile_ok(t, L.rows, L.cols, Elem<DT>::SIZE, K)) return hipErrorInvalidValue;
    TileMask P;
    P.scale = M.scale;
    P.mask = (const char*)M.mask;
    P.mask_rows = M.mask && M.mask_rows > 0 ? M.mask_rows : 1;
    P.mask_end = P.mask ? P.mask + P.mask_rows * L.cols * Elem<DT>::SIZE : nullptr;
    P.causal_q = M.causal_q;
    P.row_base = M.row_base;
    P.mask_M = remainder_magic((uint64_t)P.mask_rows);
    P.causal_M = M.causal_q > 0 ? remainder_magic((uint64_t)M.causal_q) : 0;
    const int64_t tiles = (L.rows + t.T - 1) / t.T;
    hipLaunchKernelGGL((k_tile_rows_masked<DT, K>), dim3((unsigned)tiles), dim3(64), 0, L.stream,
                       L.in, L.out, L.rows, L.cols, remainder_magic((uint64_t)L.cols), t.T,
                       tile_lg(t.T), t.lgrun, P);
    return hipGetLastError();
}

template <int DT, int K>
static hipError_t go_bwd(const BwdLaunch& B, const TileShape& t) {
    if (!tile_ok(t, B.rows, B.cols, Elem<DT>::SIZE, K)) return hipErrorInvalidValue;
    const int64_t tiles = (B.rows + t.T - 1) / t.T;
    hipLaunchKernelGGL((k_bwd_tile<DT, K>), dim3((unsigned)tiles), dim3(64), 0, B.stream, B.y,
                       B.dy, B.dx, B.rows, B.cols, remainder_magic((uint64_t)B.cols), t.T,
                       tile_lg(t.T), t.lgrun);
    return hipGetLastError();
}

template <int DT, int K>
static hipError_t go_norm(const NormLaunch& N, const TileShape& t) {
    if (!tile_ok(t, N.rows, N.cols, Elem<DT>::SIZE, K)) return hipErrorInvalidValue;
    const int64_t tiles = (N.rows + t.T - 1) / t.T;
    const uint64_t M = remainder_magic((uint64_t)N.cols);
    if (N.mode == kLayerNorm)
        hipLaunchKernelGGL((k_norm_tile<DT, K, kLayerNorm>), dim3((unsigned)tiles), dim3(64), 0,
                           N.stream, N.in, N.out, N.rows, N.cols, M, t.T, tile_lg(t.T), t.lgrun,
                           N.args);
    else
        hipLaunchKernelGGL((k_norm_tile<DT, K, kRmsNorm>), dim3((unsigned)tiles), dim3(64), 0,
                           N.stream, N.in, N.out, N.rows, N.cols, M, t.T, tile_lg(t.T), t.lgrun,
                           N.args);
    return hipGetLastError();
}

template <int K>
static hipError_t go_any(const Launch& L, const TileShape& t) {
    switch (L.dtype) {
        case kF32: return go<kF32, K>(L, t);
        case kF16: return go<kF16, K>(L, t);
        case kBF16: return go<kBF16, K>(L, t);
    }
    return hipErrorInvalidValue;
}

template <int K>
static hipError_t go_masked_any(const Launch& L, const TileShape& t, const MaskArgs& M) {
    switch (L.dtype) {
        case kF32: return go_masked<kF32, K>(L, t, M);
        case kF16: return go_masked<kF16, K>(L, t, M);
        case kBF16: return go_masked<kBF16, K>(L, t, M);
    }
    return hipErrorInvalidValue;
}

template <int K>
static hipError_t go_bwd_any(const BwdLaunch& B, const TileShape& t) {
    switch (B.dtype) {
        case kF32: return go_bwd<kF32, K>(B, t);
        case kF16: return go_bwd<kF16, K>(B, t);
        case kBF16: return go_bwd<kBF16, K>(B, t);
    }
    return hipErrorInvalidValue;
}

template <int K>
static hipError_t go_norm_any(const NormLaunch& N, const TileShape& t) {
    switch (N.dtype) {
        case kF32: return go_norm<kF32, K>(N, t);
        case kF16: return go_norm<kF16, K>(N, t);
        case kBF16: return go_norm<kBF16, K>(N, t);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_tile_rows(const Launch& L, int variant, const TileShape& t) {
    int i = 0;
#define RWS_CASE(k) \
    if (variant == i) return go_any<k>(L, t); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_tile_rows_masked(const Launch& L, int variant, const TileShape& t,
                                  const MaskArgs& M) {
    int i = 0;
#define RWS_CASE(k) \
    if (variant == i) return go_masked_any<k>(L, t, M); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_tile(const BwdLaunch& B, int variant, const TileShape& t) {
    int i = 0;
#define RWS_CASE(k) \
    if (variant == i) return go_bwd_any<k>(B, t); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_norm_tile(const NormLaunch& N, int variant, const TileShape& t) {
    int i = 0;
#define RWS_CASE(k) \
    if (variant == i) return go_norm_any<k>(N, t); \
    ++i;
    RWS_TILE_ROWS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
