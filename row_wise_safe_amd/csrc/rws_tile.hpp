// rws_tile.hpp -- several short rows per wave taken as one 16-byte-aligned
// range (the tile_rows forms of the softmax, its backward and the row
// normalisations).
//
// A row of cols elements whose byte length is not a multiple of 128 is not
// line-aligned, and unless it is a multiple of 16 it starts inside a 16-byte
// granule.  But P0 = 16 / gcd(cols * size, 16) consecutive rows (at most 8
// for 16-bit types, 4 for fp32) span a whole number of granules, so a tile of
// T rows, T a multiple of P0, starts and ends on a 16-byte boundary whenever
// the tensor does.  One wave takes one tile: lane l holds the tile's granules
// l, l + 64, ..., l + 64 (K - 1) -- coalesced 128-bit loads and stores,
// every granule read and written once and whole.  Rows have at least one
// granule of elements, so a granule holds elements of at most two rows: each
// lane keeps two partials per granule, one for the row of its first element
// ("a") and one for the next row ("b").  A row reduction then goes through
// LDS: the partials are written, the 64 / T lanes of each row fold the
// partials of the row's granules (the first granule gives its "b" partial
// when the row starts inside it), a DPP reduction over those lanes finishes
// the row, and one lane publishes the row's result for every lane to read.
// The last tile of the tensor may hold fewer rows; its last granule may stop
// inside, where it is read and written element by element.
#pragma once

#include "rws_kernels.hpp"

namespace rws {

// q = floor(x / d) for 32-bit x and d >= 2, with M = remainder_magic(d):
// the high 64 bits of M * x (the direct division of Lemire, Kaser and Kurz,
// exact for every 32-bit x).
__device__ inline uint32_t tile_div(uint32_t x, uint64_t M) {
    const uint64_t lo = (uint64_t)(uint32_t)M * x;
    const uint64_t hi = (uint64_t)(uint32_t)(M >> 32) * x;
    return (uint32_t)((hi + (lo >> 32)) >> 32);
}

// Where the granules a lane holds sit in its tile.
template <int DT, int T, int K>
struct TileSlots {
    static constexpr int VEC = Elem<DT>::VEC;
    int nel;        // elements of the tile
    int ra[K];      // tile row of granule i's first element (clamped to T - 1)
    int split[K];   // elements of granule i in that row (>= VEC: all of them)

    __device__ inline TileSlots(int nrows, int cols, uint64_t cmagic) {
        nel = nrows * cols;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const int x = granule(i) * VEC;
            const int q = (int)tile_div((uint32_t)x, cmagic);
            ra[i] = q < T - 1 ? q : T - 1;  // slots past the tile: clamped, never used
            split[i] = (q + 1) * cols - x;
        }
    }
    __device__ static inline int granule(int i) { return (int)threadIdx.x + 64 * i; }
    __device__ inline int rb(int i) const { return ra[i] + 1 < T ? ra[i] + 1 : T - 1; }
    __device__ inline bool in_a(int i, int e) const { return e < split[i]; }
};

// Granule i of a tile tensor (raw 16 bytes): whole, element by element where
// the tensor ends inside it (FULL: no such granule), 0 past the tile.
template <int DT, bool FULL>
__device__ inline u32x4 tile_load(const char* g, int j, int nel) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ES = Elem<DT>::SIZE;
    const int x = j * VEC;
    if (x + VEC <= nel) return load16<true>(g + (int64_t)j * 16);
    u32x4 r = {0u, 0u, 0u, 0u};
    if (!FULL && x < nel) {
        float f[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            f[e] = x + e < nel ? Elem<DT>::load1(g + (int64_t)(x + e) * ES) : 0.0f;
        r = Elem<DT>::narrow(f);
    }
    return r;
}

template <int DT, bool FULL>
__device__ inline void tile_store(char* g, int j, int nel, const float* v) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int ES = Elem<DT>::SIZE;
    const int x = j * VEC;
    if (x + VEC <= nel) {
        __builtin_nontemporal_store(Elem<DT>::narrow(v), (u32x4*)(g + (int64_t)j * 16));
    } else if (!FULL && x < nel) {
#pragma unroll
        for (int e = 0; e < VEC; ++e)
            if (x + e < nel) Elem<DT>::store1(g + (int64_t)(x + e) * ES, v[e]);
    }
}

// One row reduction over a tile: pa[i] / pb[i] are granule i's partials for
// its first row and for the next one.  On return row_out[r] holds
// fin(reduction of row r) for the tile's rows (0 for rows past a partial
// tile).  part_a / part_b: 64 * K floats of LDS each; the two barriers make
// the call safe to repeat with the same arrays.
template <int T, int K, class Op, class Fin>
__device__ inline void tile_fold(const float (&pa)[K], const float (&pb)[K], float* part_a,
                                 float* part_b, float* row_out, int cols, int nrows, int vec,
                                 float identity, Fin fin) {
    constexpr int GL = 64 / T;  // lanes per row
    static_assert(GL >= 4 && GL <= 64, "4..64 lanes per row");
    const int lane = threadIdx.x;
#pragma unroll
    for (int i = 0; i < K; ++i) {
        part_a[lane + 64 * i] = pa[i];
        part_b[lane + 64 * i] = pb[i];
    }
    __syncthreads();
    const int r = lane / GL;
    const int t = lane & (GL - 1);
    const int j0 = (r * cols) / vec;
    const int j1 = ((r + 1) * cols - 1) / vec;
    const bool first_in_b = j0 * vec < r * cols;
    const bool live = r < nrows;
    float acc = identity;
    if (live)
        for (int j = j0 + t; j <= j1; j += GL)
            acc = Op::f(acc, (j == j0 && first_in_b) ? part_b[j] : part_a[j]);
    acc = group_reduce<GL, Op>(acc);
    if (t == 0) row_out[r] = live ? fin(acc) : 0.0f;
    __syncthreads();
}

}  // namespace rws
