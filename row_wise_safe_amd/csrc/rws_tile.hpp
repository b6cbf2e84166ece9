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
// every granule read and written once and whole.  T is a launch argument
// (at most 64), chosen per row length so that the tile fills as many of the
// 64 K granule slots as it can: a slot past the tile costs the same
// instructions as a full one.  Rows have at least one granule of elements,
// so a granule holds elements of at most two rows: each lane keeps two
// partials per granule, one for the row of its first element ("a") and one
// for the next row ("b").  A row reduction then goes through LDS: the
// partials are written, the 2^lg lanes of each row (2^lg * T <= 64) fold the
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

// Where the granules a lane holds sit in its tile of nrows rows.
template <int DT, int K>
struct TileSlots {
    static constexpr int VEC = Elem<DT>::VEC;
    int nel;        // elements of the tile
    int last;       // the tile's last row
    int ra[K];      // tile row of granule i's first element (clamped to last)
    int split[K];   // elements of granule i in that row (>= VEC: all of them)

    __device__ inline TileSlots(int nrows, int cols, uint64_t cmagic) {
        nel = nrows * cols;
        last = nrows - 1;
#pragma unroll
        for (int i = 0; i < K; ++i) {
            const int x = granule(i) * VEC;
            const int q = (int)tile_div((uint32_t)x, cmagic);
            ra[i] = q < last ? q : last;  // slots past the tile: clamped, never used
            split[i] = (q + 1) * cols - x;
        }
    }
    __device__ static inline int granule(int i) { return (int)threadIdx.x + 64 * i; }
    __device__ inline int rb(int i) const { return ra[i] < last ? ra[i] + 1 : last; }
    // Element e of granule i is in row ra[i] when e < split[i], else in the
    // next row.  split[i] as a value the compiler cannot match with earlier uses: each
    // pass over the granules then compares afresh instead of keeping 2 K VEC
    // lane masks (scalar register pairs) alive across the row reductions,
    // which spilled them at K >= 3 (one compare per element and pass is
    // cheaper than the spill traffic).
    __device__ inline int split_pass(int i) const {
        int sp = split[i];
        asm volatile("" : "+v"(sp));
        return sp;
    }
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

// Reduction over aligned groups of 2^lg lanes (lg uniform, 0..4).
template <class Op>
__device__ inline float group_reduce_lg(float v, int lg) {
    if (lg >= 1) v = Op::f(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
    if (lg >= 2) v = Op::f(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
    if (lg >= 3) v = Op::f(v, dpp<0x141>(v));  // row_half_mirror: other quad of 8
    if (lg >= 4) v = Op::f(v, dpp<0x140>(v));  // row_mirror: other half of 16
    return v;
}

// One row reduction over a tile: pa[i] / pb[i] are granule i's partials for
// its first row and for the next one.  On return row_out[r] holds
// fin(reduction of row r) for the tile's rows (0 for rows past a partial
// tile).  part_a / part_b: 64 * K floats of LDS each, row_out kTileMaxT; the
// two barriers make the call safe to repeat with the same arrays.
template <int K, class Op, class Fin>
__device__ inline void tile_fold(const float (&pa)[K], const float (&pb)[K], float* part_a,
                                 float* part_b, float* row_out, int cols, int nrows, int lg,
                                 int vec, float identity, Fin fin) {
    const int lane = threadIdx.x;
#pragma unroll
    for (int i = 0; i < K; ++i) {
        part_a[lane + 64 * i] = pa[i];
        part_b[lane + 64 * i] = pb[i];
    }
    __syncthreads();
    const int r = lane >> lg;
    const int gl = 1 << lg;
    const int t = lane & (gl - 1);
    const bool live = r < nrows;
    float acc = identity;
    if (live) {
        const int j0 = (r * cols) / vec;
        const int j1 = ((r + 1) * cols - 1) / vec;
        const bool first_in_b = j0 * vec < r * cols;
        for (int j = j0 + t; j <= j1; j += gl)
            acc = Op::f(acc, (j == j0 && first_in_b) ? part_b[j] : part_a[j]);
    }
    acc = group_reduce_lg<Op>(acc, lg);
    if (t == 0) row_out[r] = live ? fin(acc) : 0.0f;
    __syncthreads();
}

}  // namespace rws
