// rws_pre.hpp -- per-element prologues applied to a row right after it is
// widened to fp32, before the row max: the identity, and the attention-score
// prologue z = scale * x + mask (+ causal limit) that the DCU case-study page
// (section 9) proposes to fold into the softmax kernel as a mask parameter.
#pragma once

#include <type_traits>

#include "rws_device.hpp"

namespace rws {

// Interface.  ctx() computes what a prologue needs per row, once per row;
// fetch() issues the loads of the prologue operand (Operand) of granule k;
// apply() rewrites the widened values and sets every slot outside the row to
// -inf (the kernels leave those slots as loaded when a prologue is active:
// RowWin::widen_in_row); needs_input() says whether granule k
// of the input can affect the result at all (a granule wholly past the
// causal limit becomes -inf whatever it holds, so its load is skipped).
struct NoPre {
    static constexpr bool kActive = false;
    using Operand = u32x4;
    struct Ctx {};
    template <class Win>
    __device__ inline Ctx ctx(int64_t, const Win&) const {
        return Ctx{};
    }
    template <class Win>
    __device__ inline bool needs_input(const Ctx&, const Win&, int) const {
        return true;
    }
    template <class Win>
    __device__ inline u32x4 fetch(const Ctx&, const Win&, int) const {
        return u32x4{0u, 0u, 0u, 0u};
    }
    template <class Win>
    __device__ inline void apply(const Ctx&, const Win&, int, float*, Operand) const {}
};

// r mod d for r >= 0, d > 0.  When both fit 32 bits, by multiplication
// with M = floor((2^64 - 1) / d) + 1, computed once on the host
// (remainder_magic): the low 64 bits of M*r are the fraction r/d scaled by
// 2^64, and their product with d, shifted right by 64, is the remainder --
// exact for every 32-bit r and d (the direct-remainder method of Lemire,
// Kaser and Kurz, "Faster remainder by direct computation", 2019).  It is a
// handful of scalar multiplies; the division it replaces sat between a row's
// start and its first load (the causal limit decides which granules are
// read): fp16 [65536,512] with a [512,512] mask and causal limit 21.4 us
// against 22.3 us.  Otherwise a plain 64-bit remainder.
__host__ __device__ inline uint64_t remainder_magic(uint64_t d) { return ~0ull / d + 1; }

__device__ inline int64_t row_mod(int64_t r, int64_t d, uint64_t M) {
    if ((((uint64_t)r | (uint64_t)d) >> 32) == 0) {
        const uint64_t frac = M * (uint64_t)r;  // modulo 2^64
        const uint64_t lo = (uint64_t)(uint32_t)frac * (uint64_t)d;
        const uint64_t hi = (uint64_t)(uint32_t)(frac >> 32) * (uint64_t)d;
        return (int64_t)(uint32_t)((hi + (lo >> 32)) >> 32);
    }
    return r % d;
}

// Bytes [ph, ph + 16) of the 32 bytes lo ++ hi, ph in 1..15 and free to
// differ between lanes: the dwords are picked by selects, then shifted.
__device__ inline u32x4 shift16_lanes(u32x4 lo, u32x4 hi, int ph) {
    const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const int q = ph >> 2;
    const uint32_t b = (uint32_t)(ph & 3);
    uint32_t s[5];
#pragma unroll
    for (int k = 0; k < 5; ++k)
        s[k] = q == 0 ? w[k] : q == 1 ? w[k + 1] : q == 2 ? w[k + 2] : w[k + 3];
    return u32x4{__builtin_amdgcn_alignbyte(s[1], s[0], b), __builtin_amdgcn_alignbyte(s[2], s[1], b),
                 __builtin_amdgcn_alignbyte(s[3], s[2], b), __builtin_amdgcn_alignbyte(s[4], s[3], b)};
}

// z = scale * x + mask[row % mask_rows, c]; columns past the causal limit
// (c > (row % causal_q) + cols - causal_q, when causal_q > 0) and slots
// outside the row become -inf.  The mask has the input's dtype and row pitch.
// fetch() issues the mask granule's loads together with the input's: one
// 128-bit load when the mask row has the input row's 16-byte phase, else
// (PAIR) the two aligned granules around it, shifted in apply().  The row's
// first and last granules take mask bytes from outside the mask row as well
// (never used: those slots become -inf); they are loaded so for mask rows
// edge_lo..edge_hi, where every such load stays inside the mask (all but the
// mask's first and last rows).  Elsewhere apply() reads the mask element by
// element.  PAIR
// doubles the registers that hold the operands in flight: kernels of 1024
// threads (128 registers a lane) leave it off.
template <int DT, bool PAIR = true>
struct MaskPre {
    static constexpr bool kActive = true;
    struct OperandPair {
        u32x4 lo;  // the mask granule, or the aligned one below it
        u32x4 hi;  // the aligned granule above it
    };
    struct OperandOne {
        u32x4 lo;  // the mask granule
    };
    using Operand = typename std::conditional<PAIR, OperandPair, OperandOne>::type;
    float scale;
    const char* mask;      // nullptr: no additive mask
    int64_t mask_rows;
    // Mask rows r with r * rowbytes >= 32 and (r + 1) * rowbytes + 32 <=
    // mask_rows * rowbytes (rowbytes = cols * size): the granule loads of a
    // row's ends reach at most 30 bytes before its mask row and 31 past it.
    int64_t edge_lo, edge_hi;
    int64_t causal_q;      // 0: no causal limit
    int64_t row_base;      // global index of the launch's first row
    uint64_t mask_M;       // remainder_magic(mask_rows)
    uint64_t causal_M;     // remainder_magic(causal_q) when causal_q > 0

    struct Ctx {
        const char* mrow;  // the row's mask row (nullptr: no mask)
        bool mvec;         // mask row has the input row's 16-byte phase
        bool mpair;        // otherwise: pairs of aligned mask granules, all in bounds
        bool medge;        // the row's partial end granules take granule loads too
        int mph;           // the mask row's 16-byte phase against the input row's
        int limit;         // last column that takes part
    };

    template <class Win>
    __device__ inline Ctx ctx(int64_t lrow, const Win& w) const {
        const int64_t row = row_base + lrow;
        Ctx c;
        c.mrow = nullptr;
        c.mvec = false;
        c.mpair = false;
        c.medge = false;
        c.mph = 0;
        if (mask) {
            constexpr int ES = Elem<DT>::SIZE;
            const int64_t r = row_mod(row, mask_rows, mask_M);
            c.mrow = mask + r * (int64_t)w.cols * ES;
            const char* xrow = w.gin + (int64_t)w.lead * ES;  // the input row start
            c.mph = (int)(((uintptr_t)c.mrow - (uintptr_t)xrow) & 15u);
            c.mvec = c.mph == 0;
            const bool in_range = r >= edge_lo && r <= edge_hi;
            c.mpair = PAIR && !c.mvec && in_range;
            c.medge = !Win::kWhole && in_range && (c.mvec || PAIR);
        }
        c.limit = w.cols - 1;
        if (causal_q > 0) c.limit = (int)row_mod(row, causal_q, causal_M) + w.cols - (int)causal_q;
        return c;
    }

    // false when every column of granule k is past the causal limit: the
    // prologue then sets the whole granule to -inf, so neither the input nor
    // the mask granule is read (about half of a square causal score matrix).
    template <class Win>
    __device__ inline bool needs_input(const Ctx& c, const Win& w, int k) const {
        return k * Elem<DT>::VEC - w.lead <= c.limit;
    }

    template <class Win>
    __device__ inline Operand fetch(const Ctx& c, const Win& w, int k) const {
        Operand g{};
        const int c0 = k * Elem<DT>::VEC - w.lead;
        const bool inside = c0 >= 0 && c0 + Elem<DT>::VEC <= w.cols;
        const bool overlaps = c0 + Elem<DT>::VEC > 0 && c0 < w.cols;
        if (c.mrow && (c.medge ? overlaps : inside)) {
            const char* p = c.mrow + (int64_t)c0 * Elem<DT>::SIZE;
            if (c.mvec) {
                g.lo = *(const u32x4*)p;
            } else if constexpr (PAIR) {
                if (c.mpair) {
                    g.lo = *(const u32x4*)(p - c.mph);
                    g.hi = *(const u32x4*)(p - c.mph + 16);
                }
            }
        }
        return g;
    }

    // The mask granule of a pair operand; (OperandOne: never called, as
    // mpair is false without PAIR.)
    __device__ static inline u32x4 shifted(const OperandPair& m, int ph) {
        return shift16_lanes(m.lo, m.hi, ph);
    }
    __device__ static inline u32x4 shifted(const OperandOne& m, int) { return m.lo; }

    template <class Win>
    __device__ inline void apply(const Ctx& c, const Win& w, int k, float* v, Operand mraw) const {
        constexpr int VEC = Elem<DT>::VEC;
        constexpr int ES = Elem<DT>::SIZE;
        const int c0 = k * VEC - w.lead;
        const bool inside = c0 >= 0 && c0 + VEC <= w.cols;
        float mv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) mv[e] = 0.0f;
        if (c.mrow) {
            // a granule past the row's ends was not loaded: its slots are
            // all dropped below, whatever mv holds
            if (c.mvec && (inside || c.medge)) {
                Elem<DT>::widen(mraw.lo, mv);
            } else if (c.mpair) {
                Elem<DT>::widen(shifted(mraw, c.mph), mv);
            } else {
                // every load issued before the first is waited for: slots
                // outside the row read the row's first element instead
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int col = c0 + e;
                    const bool in = col >= 0 && col < w.cols;
                    const float m = Elem<DT>::load1(c.mrow + (int64_t)(in ? col : 0) * ES);
                    mv[e] = in ? m : 0.0f;
                }
            }
        }
        // slots lo..hi of the granule take part (inside the row and up to the
        // causal limit).  One select per slot on every lane: the causal limit
        // falls inside most waves, where a separate whole-granule path ran
        // next to this one (fp16 [65536,512], [512,512] mask, causal: 21.0 us
        // against 21.5)
        const int lo = -c0;
        const int hi = (c.limit < w.cols - 1 ? c.limit : w.cols - 1) - c0;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const bool ok = e >= lo && e <= hi;
            v[e] = ok ? __builtin_fmaf(scale, v[e], mv[e]) : kNegInf;
        }
    }
};

}  // namespace rws
