// rws_pre.hpp -- per-element prologues applied to a row right after it is
// widened to fp32, before the row max: the identity, and the attention-score
// prologue z = scale * x + mask (+ causal limit) that the DCU case-study page
// (section 9) proposes to fold into the softmax kernel as a mask parameter.
#pragma once

#include "rws_device.hpp"

namespace rws {

struct NoPre {
    static constexpr bool kActive = false;
    template <class Win>
    __device__ inline u32x4 fetch(int64_t, const Win&, int) const {
        return u32x4{0u, 0u, 0u, 0u};
    }
    template <class Win>
    __device__ inline void apply(int64_t, const Win&, int, float*, u32x4) const {}
};

// z = scale * x + mask[row % mask_rows, c]; columns past the causal limit
// (c > (row % causal_q) + cols - causal_q, when causal_q > 0) and slots
// outside the row become -inf.  The mask has the input's dtype and row pitch.
// fetch() issues a mask granule's 128-bit load together with the input's
// (when the mask row has the input row's 16-byte phase and the granule lies
// inside the row); apply() uses it, or reads the mask element by element
// otherwise.
template <int DT>
struct MaskPre {
    static constexpr bool kActive = true;
    float scale;
    const char* mask;   // nullptr: no additive mask
    int64_t mask_rows;
    int64_t causal_q;   // 0: no causal limit
    int64_t row_base;   // global index of the launch's first row

    template <class Win>
    __device__ inline const char* mask_row(int64_t lrow, const Win& w) const {
        return mask + ((row_base + lrow) % mask_rows) * (int64_t)w.cols * Elem<DT>::SIZE;
    }
    template <class Win>
    __device__ inline bool vector_ok(const char* mrow, const Win& w, int c0) const {
        const char* xrow = w.gin + (int64_t)w.lead * Elem<DT>::SIZE;  // the input row start
        return c0 >= 0 && c0 + Elem<DT>::VEC <= w.cols &&
               (((uintptr_t)mrow - (uintptr_t)xrow) & 15u) == 0;
    }

    template <class Win>
    __device__ inline u32x4 fetch(int64_t lrow, const Win& w, int k) const {
        u32x4 g = {0u, 0u, 0u, 0u};
        if (mask) {
            const char* mrow = mask_row(lrow, w);
            const int c0 = k * Elem<DT>::VEC - w.lead;
            if (vector_ok(mrow, w, c0)) g = *(const u32x4*)(mrow + (int64_t)c0 * Elem<DT>::SIZE);
        }
        return g;
    }

    template <class Win>
    __device__ inline void apply(int64_t lrow, const Win& w, int k, float* v, u32x4 mraw) const {
        constexpr int VEC = Elem<DT>::VEC;
        constexpr int ES = Elem<DT>::SIZE;
        const int64_t row = row_base + lrow;
        const int c0 = k * VEC - w.lead;
        int limit = w.cols - 1;
        if (causal_q > 0) limit = (int)(row % causal_q) + w.cols - (int)causal_q;
        float mv[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) mv[e] = 0.0f;
        if (mask) {
            const char* mrow = mask_row(lrow, w);
            if (vector_ok(mrow, w, c0)) {
                Elem<DT>::widen(mraw, mv);
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int c = c0 + e;
                    if (c >= 0 && c < w.cols) mv[e] = Elem<DT>::load1(mrow + (int64_t)c * ES);
                }
            }
        }
        if (c0 >= 0 && c0 + VEC - 1 <= limit && c0 + VEC <= w.cols) {
            // the whole granule is inside the row and the causal limit
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[e] = __builtin_fmaf(scale, v[e], mv[e]);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int c = c0 + e;
                const bool ok = c >= 0 && c <= limit && c < w.cols;
                v[e] = ok ? __builtin_fmaf(scale, v[e], mv[e]) : kNegInf;
            }
        }
    }
};

}  // namespace rws
