// rws_tile_rows.hip -- short rows that do not start on a 16-byte boundary,
// several rows per wave taken as one aligned range.
//
// A row of cols elements whose byte length is not a multiple of 16 starts
// at a different 16-byte phase from its neighbours, so a per-row window
// (wave_row) has a partial granule at each end: both neighbouring rows load
// it, and each stores its own bytes of it with 2-, 4- or 8-byte stores.  For
// short rows those ends are a large share of the traffic.  But the phase
// repeats: P0 = 16 / gcd(cols * size, 16) consecutive rows (at most 8 for
// 16-bit types, 4 for fp32) span a whole number of granules, so a tile of T
// rows (T a multiple of P0) starts and ends on a 16-byte boundary whenever
// the tensor does.  One wave takes one tile: lane l holds the tile's
// granules l, l + 64, ... (coalesced 128-bit loads and stores, every granule
// read and written once and whole).  A granule holds elements of at most two
// rows (cols >= elements per granule), so each lane keeps two partial
// results per granule -- one for the row its first element belongs to, one
// for the next row -- and the row reductions go through LDS: after the
// partials are written, GL = 64 / T lanes per row fold the granules of their
// row (the first one takes its "next row" partial when the row starts inside
// it), a DPP reduction over the GL lanes finishes the row, and one lane
// publishes the row's result.  Max first, then the exponentials against each
// element's row maximum and the same fold for the sums, then the scaling:
// the row-wise definition (CUDA safe-online-softmax page, section 1), with
// the reductions segmented by row.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"

namespace rws {

// q = floor(x / d) for 32-bit x and d >= 2, with M = remainder_magic(d):
// the high 64 bits of M * x (the direct division of Lemire, Kaser and Kurz,
// exact for every 32-bit x).
__device__ inline uint32_t tile_div(uint32_t x, uint64_t M) {
    const uint64_t lo = (uint64_t)(uint32_t)M * x;
    const uint64_t hi = (uint64_t)(uint32_t)(M >> 32) * x;
    return (uint32_t)((hi + (lo >> 32)) >> 32);
}

// One tile.  FULL: T whole rows (every tile but possibly the last), so the
// tile is a whole number of granules; else the tensor's last, partial tile,
// whose last granule may stop inside (element access there).
template <int DT, int T, int K, bool FULL>
__device__ inline void tile_rows_body(const char* __restrict__ gin, char* __restrict__ gout,
                                      int nrows, int cols, uint64_t cmagic, float* part_a,
                                      float* part_b, float* row_max, float* row_rcp) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ES = Elem<DT>::SIZE;
    constexpr int GL = 64 / T;  // lanes per row in the row folds
    const int lane = threadIdx.x;
    const int nel = nrows * cols;  // elements of this tile

    // load: whole granules; element by element only where the tensor ends
    u32x4 raw[K];
    int ra[K];     // tile row of the granule's first element
    int split[K];  // elements of the granule in that row (>= VEC: all)
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int j = lane + 64 * i;
        const int x = j * VEC;
        raw[i] = u32x4{0u, 0u, 0u, 0u};
        if (x + VEC <= nel) {
            raw[i] = load16<true>(gin + (int64_t)j * 16);
        } else if (!FULL && x < nel) {
            float f[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                f[e] = x + e < nel ? Elem<DT>::load1(gin + (int64_t)(x + e) * ES) : 0.0f;
            raw[i] = Elem<DT>::narrow(f);
        }
        const int q = (int)tile_div((uint32_t)x, cmagic);
        ra[i] = q < T - 1 ? q : T - 1;  // slots past the tile: clamped, never used
        split[i] = (q + 1) * cols - x;
    }

    // widen; slots past the tile are -inf (they belong to no row)
    float v[K][VEC];
#pragma unroll
    for (int i = 0; i < K; ++i) {
        Elem<DT>::widen(raw[i], v[i]);
        const int x = (lane + 64 * i) * VEC;
        if (x + VEC > nel) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i][e] = x + e < nel ? v[i][e] : kNegInf;
        }
    }

    // the GL lanes of row r fold the partials of r's granules; the first
    // granule contributes its "next row" part when r starts inside it
    const int r = lane / GL;
    const int t = lane & (GL - 1);
    const int j0 = (r * cols) / VEC;
    const int j1 = ((r + 1) * cols - 1) / VEC;
    const bool first_in_b = j0 * VEC < r * cols;
    const bool live = FULL || r < nrows;

    // row maxima: each granule's maximum over its first row's elements (a)
    // and over the next row's (b)
#pragma unroll
    for (int i = 0; i < K; ++i) {
        float ma = kNegInf, mb = kNegInf;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool in_a = e < split[i];
            ma = vmax(ma, in_a ? v[i][e] : kNegInf);
            mb = vmax(mb, in_a ? kNegInf : v[i][e]);
        }
        part_a[lane + 64 * i] = ma;
        part_b[lane + 64 * i] = mb;
    }
    __syncthreads();
    {
        float m = kNegInf;
        if (live)
            for (int j = j0 + t; j <= j1; j += GL)
                m = vmax(m, (j == j0 && first_in_b) ? part_b[j] : part_a[j]);
        m = group_reduce<GL, OpMax>(m);
        if (t == 0) row_max[r] = live ? m : 0.0f;
    }
    __syncthreads();

    // exponentials against each element's row maximum (one exp2 per
    // element: the FMA offset of the element's row is selected first; rows
    // whose maximum takes the exact form -- |max| above 2.9e6 or +inf --
    // take it for the whole granule), row sums
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int rb = ra[i] + 1 < T ? ra[i] + 1 : T - 1;  // next row (unused past the tile)
        const RowExp ea(row_max[ra[i]]), eb(row_max[rb]);
        float sa = 0.0f, sb = 0.0f;
        if (__builtin_expect(ea.big || eb.big, 0)) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < split[i];
                const float y = in_a ? ea.one(v[i][e]) : eb.one(v[i][e]);
                v[i][e] = y;
                sa += in_a ? y : 0.0f;
                sb += in_a ? 0.0f : y;
            }
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const bool in_a = e < split[i];
                const float y =
                    __builtin_amdgcn_exp2f(__builtin_fmaf(v[i][e], kLog2e, in_a ? ea.negc : eb.negc));
                v[i][e] = y;
                sa += in_a ? y : 0.0f;
                sb += in_a ? 0.0f : y;
            }
        }
        part_a[lane + 64 * i] = sa;
        part_b[lane + 64 * i] = sb;
    }
    __syncthreads();
    {
        float s = 0.0f;
        if (live)
            for (int j = j0 + t; j <= j1; j += GL)
                s += (j == j0 && first_in_b) ? part_b[j] : part_a[j];
        s = group_reduce<GL, OpSum>(s);
        if (t == 0) row_rcp[r] = live ? __builtin_amdgcn_rcpf(s) : 0.0f;
    }
    __syncthreads();

    // scale and store: whole granules; element by element where the tensor ends
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const int j = lane + 64 * i;
        const int x = j * VEC;
        if (x >= nel) continue;
        const int rb = ra[i] + 1 < T ? ra[i] + 1 : T - 1;
        const float qa = row_rcp[ra[i]], qb = row_rcp[rb];
#pragma unroll
        for (int e = 0; e < VEC; ++e) v[i][e] *= e < split[i] ? qa : qb;
        if (x + VEC <= nel) {
            __builtin_nontemporal_store(Elem<DT>::narrow(v[i]), (u32x4*)(gout + (int64_t)j * 16));
        } else if (!FULL) {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (x + e < nel) Elem<DT>::store1(gout + (int64_t)(x + e) * ES, v[i][e]);
        }
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
    const char* gin = (const char*)in + row0 * cols * Elem<DT>::SIZE;
    char* gout = (char*)out + row0 * cols * Elem<DT>::SIZE;
    if (rows - row0 >= T)
        tile_rows_body<DT, T, K, true>(gin, gout, T, cols, cmagic, part_a, part_b, row_max, row_rcp);
    else
        tile_rows_body<DT, T, K, false>(gin, gout, (int)(rows - row0), cols, cmagic, part_a, part_b,
                                        row_max, row_rcp);
}

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

template <int T, int K>
static hipError_t go_any(const Launch& L) {
    switch (L.dtype) {
        case kF32: return go<kF32, T, K>(L);
        case kF16: return go<kF16, T, K>(L);
        case kBF16: return go<kBF16, T, K>(L);
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

}  // namespace rws
