// rws_device.hpp -- device primitives for the gfx950 row-wise softmax kernels.
//
//  * 16-byte "granules": every global access of a row body is one 128-bit
//    load or store per lane (DCU case-study page, sections 4.2 and 8; CUDA
//    safe-online-softmax page, section 2.1, the 128-bit pack).  A row that does
//    not start or end on a 16-byte boundary is covered by the aligned granules
//    that overlap it; the (at most two) partial granules at its ends are read
//    and written element by element, so no byte outside the row is touched
//    (InfiniTrain BF16 elementwise page: aligned vector body, scalar tail).
//  * dtype widening to fp32 (exact) and RNE narrowing (v_cvt_pk_f16_f32,
//    v_cvt_pk_bf16_f32 on gfx950) -- packed conversion as on the DCU
//    case-study page, section 4.5.
//  * Cross-lane reductions inside 4/8/16/32/64-lane groups with DPP
//    (quad_perm, row_half_mirror, row_mirror) and the gfx950 permlane16/32
//    swaps: no LDS round trip (DCU case-study page, section 5.2; CUDA
//    safe-online-softmax page, section 2.1.1, there with 32-lane shuffles).
//  * Cross-wave reductions through a few LDS words and one barrier.
//  * exp(x - m) evaluated as 2^(x*log2(e) - m*log2(e)) with v_exp_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rws {

enum DType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kFltMax = 3.40282346638528859812e+38f;

// ---------------------------------------------------------------------------
// dtype traits: VEC elements per 16-byte granule, exact widening, RNE
// narrowing, single-element access for partial granules.  Single-element
// stores are non-temporal like the 128-bit ones: a cached 2-byte store into a
// line whose other bytes arrive non-temporally measured ~12% slower on the
// unaligned fp16 [8192,4097] workload.
// ---------------------------------------------------------------------------
template <int DT>
struct Elem;

template <>
struct Elem<kF32> {
    static constexpr int VEC = 4;
    static constexpr int SIZE = 4;
    __device__ static inline void widen(u32x4 g, float* v) {
        f4_t f = __builtin_bit_cast(f4_t, g);
        v[0] = f[0]; v[1] = f[1]; v[2] = f[2]; v[3] = f[3];
    }
    __device__ static inline u32x4 narrow(const float* v) {
        f4_t f = {v[0], v[1], v[2], v[3]};
        return __builtin_bit_cast(u32x4, f);
    }
    __device__ static inline float load1(const char* p) { return *(const float*)p; }
    __device__ static inline void store1(char* p, float v) {
        __builtin_nontemporal_store(v, (float*)p);
    }
};

template <>
struct Elem<kF16> {
    static constexpr int VEC = 8;
    static constexpr int SIZE = 2;
    __device__ static inline void widen(u32x4 g, float* v) {
        f8_t f = __builtin_convertvector(__builtin_bit_cast(h8_t, g), f8_t);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = f[i];
    }
    __device__ static inline u32x4 narrow(const float* v) {
        f8_t f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
        return __builtin_bit_cast(u32x4, __builtin_convertvector(f, h8_t));
    }
    __device__ static inline float load1(const char* p) { return (float)*(const _Float16*)p; }
    __device__ static inline void store1(char* p, float v) {
        __builtin_nontemporal_store((_Float16)v, (_Float16*)p);
    }
};

template <>
struct Elem<kBF16> {
    static constexpr int VEC = 8;
    static constexpr int SIZE = 2;
    // bf16 -> fp32 is the bf16 bit pattern in the top half of the word: exact.
    __device__ static inline void widen(u32x4 g, float* v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(g[i] << 16);
            v[2 * i + 1] = __uint_as_float(g[i] & 0xffff0000u);
        }
    }
    __device__ static inline u32x4 narrow(const float* v) {
        f8_t f = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
        return __builtin_bit_cast(u32x4, __builtin_convertvector(f, b8_t));
    }
    __device__ static inline float load1(const char* p) {
        return __uint_as_float((unsigned)(*(const unsigned short*)p) << 16);
    }
    __device__ static inline void store1(char* p, float v) {
        __builtin_nontemporal_store(__builtin_bit_cast(unsigned short, (__bf16)v),
                                    (unsigned short*)p);
    }
};

// ---------------------------------------------------------------------------
// 128-bit load with a cache policy.  NT marks it non-temporal (gfx950
// `global_load_dwordx4 ... nt`): the line is not kept for reuse, in
// particular not in the 256 MB last-level cache.  Data that a kernel reads
// once is loaded NT: streams from HBM measured 3-5% faster that way on
// MI355X (fp16 [65536,512] softmax 21.7 us vs 22.4 us; a 64 MiB copy
// 22.5 us vs 23.1 us).  A first pass whose data a later pass of the same
// kernel reads again loads without it, so the re-read can hit the caches.
// ---------------------------------------------------------------------------
// 128-bit store with the non-temporal and device-scope bits
// (`global_store_dwordx4 ... nt sc1`): the line is written through past the
// XCD's L2 instead of being held there dirty.  On MI355X this moves a copy of
// HBM-resident data 2.9% faster (64 MiB: 21.1 us against 21.7 us with `nt`
// alone) and the forward wave_row kernels 1-1.7% faster on line-aligned
// rows; where two workgroups write parts of one line (rows that are not
// line-aligned) it is far slower (fp16 [8192,4097]: 40.9 us against 24.0),
// and the backward and split-k kernels measured 1.4-2% slower, so only
// callers that ask for it use it.  (No compiler builtin gives this bit
// combination for a global store, hence the one-instruction asm.)
__device__ inline void store16_wt(char* p, u32x4 v) {
    asm volatile("global_store_dwordx4 %0, %1, off nt sc1" : : "v"(p), "v"(v) : "memory");
}

// Row handled by workgroup `id` of a launch of `n` one-row workgroups when
// runs of 2^lg consecutive rows go to one XCD.  Workgroups are dispatched to
// the 8 XCDs round-robin by id, so in launch order XCD x gets rows x, x+8,
// x+16, ...; here each span of 8 * 2^lg rows is split so that XCD x gets the
// run [x * 2^lg, (x + 1) * 2^lg) of it.  A trailing partial span keeps launch
// order; lg = 0 is launch order.  (The dispatcher picks lg for the
// workgroup-per-row families; measurements are with that rule.)
__device__ inline int64_t xcd_run(int64_t id, int64_t n, int lg) {
    const int sh = 3 + lg;
    const int64_t full = (n >> sh) << sh;
    if (lg == 0 || id >= full) return id;
    const int r = (int)(id & ((1 << sh) - 1));
    return (id - r) + ((int64_t)(r & 7) << lg) + (r >> 3);
}

template <bool NT>
__device__ inline u32x4 load16(const char* p) {
    if (NT) return __builtin_nontemporal_load((const u32x4*)p);
    return *(const u32x4*)p;
}

// ---------------------------------------------------------------------------
// Bytes [lo, hi) of a packed 16-byte granule to g (16-byte aligned), lo and
// hi multiples of 2: 2-, 4- and 8-byte non-temporal stores, each naturally
// aligned -- at most three from lo up to the first 16-byte boundary or to hi,
// then at most three more below hi.  A row end inside a granule thus takes
// at most three stores instead of up to seven element stores.
// ---------------------------------------------------------------------------
__device__ inline void store_part(char* g, u32x4 w, int lo, int hi) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    int b = lo;
    if ((b & 2) && b + 2 <= hi) {
        __builtin_nontemporal_store((unsigned short)(w[b >> 2] >> 16), (unsigned short*)(g + b));
        b += 2;
    }
    if ((b & 4) && b + 4 <= hi) {
        __builtin_nontemporal_store(w[b >> 2], (unsigned*)(g + b));
        b += 4;
    }
    if ((b & 8) && b + 8 <= hi) {
        __builtin_nontemporal_store(u32x2{w[2], w[3]}, (u32x2*)(g + b));
        b += 8;
    }
    if (b + 8 <= hi) {  // b == 0 here
        __builtin_nontemporal_store(u32x2{w[0], w[1]}, (u32x2*)(g + b));
        b += 8;
    }
    if (b + 4 <= hi) {
        __builtin_nontemporal_store(w[b >> 2], (unsigned*)(g + b));
        b += 4;
    }
    if (b + 2 <= hi) {
        __builtin_nontemporal_store((unsigned short)(w[b >> 2] & 0xffffu), (unsigned short*)(g + b));
        b += 2;
    }
}

// ---------------------------------------------------------------------------
// Row window: the granules, starting on a WA-byte boundary (WA = 128, one
// cache line, or 16 for lane groups narrower than a line), that cover one row.
//   lead  = elements of the window that precede the row (0 .. WA/size - 1)
//   ngran = number of granules in the window
// Granule k holds row columns c0 = k*VEC - lead .. c0+VEC-1; it is "interior"
// (all VEC elements belong to the row) iff c0 >= 0 and c0 + VEC <= cols.
// Starting the window on a line boundary means that the 64 lanes of a wave
// writing 64 consecutive granules cover 8 whole 128-byte lines; only the
// row's first and last line are shared with the neighbouring rows.  (A window
// that started on the row's 16-byte granule would split two lines per store
// instruction for every row that is not line-aligned.)
// With ALIGNED (row start 128-byte aligned and cols*size % 128 == 0) lead == 0
// and every granule is interior.
//
// Loads are split in two so that a thread issues all of its 128-bit loads
// before it waits for any: fetch() only loads, widen() converts and masks.
//  * ALIGNED: fetch(k) reads granule min(k, ngran-1) (always inside the row);
//    widen() turns granules k >= ngran into -inf.
//  * unaligned: fetch(k) reads the whole 16-byte granule whenever it overlaps
//    the row and lies inside the tensor [tbeg, tend) -- a partial granule then
//    also holds bytes of the neighbouring row, which widen() replaces by
//    -inf.  Only the first granule of the tensor and its last one can stick
//    out of it; those two are read element by element inside widen(), so no
//    byte outside the tensor is ever read.
// ---------------------------------------------------------------------------
constexpr int kLineBytes = 128;

template <int DT, bool ALIGNED, int WA = kLineBytes>
struct RowWin {
    static_assert(WA == 16 || WA == 32 || WA == 64 || WA == 128, "window alignment");
    static constexpr int VEC = Elem<DT>::VEC;
    static constexpr int ES = Elem<DT>::SIZE;
    // each granule of the window lies wholly inside the row or wholly past it
    static constexpr bool kWhole = ALIGNED;
    const char* gin;   // first granule of the window in `in` (line aligned)
    char* gout;        // same position in `out` (used when same_phase)
    char* rout;        // row start in `out`
    int lead;
    int ngran;
    int cols;

    RowWin() = default;
    __device__ inline RowWin(const void* in, void* out, int64_t row, int cols_) {
        cols = cols_;
        const char* rin = (const char*)in + row * (int64_t)cols_ * ES;
        rout = (char*)out + row * (int64_t)cols_ * ES;
        if (ALIGNED) {
            lead = 0;
            gin = rin;
            gout = rout;
            ngran = cols_ / VEC;
        } else {
            uintptr_t a = (uintptr_t)rin;
            int mis = (int)(a & (WA - 1));
            lead = mis / ES;
            gin = rin - mis;
            gout = rout - mis;
            ngran = (mis + cols_ * ES + 15) >> 4;
        }
    }

    __device__ inline bool interior(int k) const {
        if (ALIGNED) return k < ngran;
        const int c0 = k * VEC - lead;
        return c0 >= 0 && c0 + VEC <= cols;
    }

    // Issue the 128-bit load of granule k (no wait); NT: see load16.
    template <bool NT = true>
    __device__ inline u32x4 fetch(int k, const char* tbeg, const char* tend) const {
        if (ALIGNED) {
            const int kk = k < ngran ? k : ngran - 1;
            return load16<NT>(gin + (int64_t)kk * 16);
        }
        const char* g = gin + (int64_t)k * 16;
        const int c0 = k * VEC - lead;
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (c0 + VEC > 0 && c0 < cols && g >= tbeg && g + 16 <= tend) raw = load16<NT>(g);
        return raw;
    }

    // Widen a fetched granule into v[0..VEC) for a kernel whose prologue
    // drops every slot outside the row (their values are left as they come).
    // Only a granule the tensor begins or ends inside was not loaded whole:
    // its elements in the row are read one by one, all loads issued at once.
    __device__ inline void widen_in_row(int k, u32x4 raw, float* v, const char* tbeg,
                                        const char* tend) const {
        Elem<DT>::widen(raw, v);
        if (ALIGNED) return;
        const char* g = gin + (int64_t)k * 16;
        if (!(g >= tbeg && g + 16 <= tend)) {
            const int c0 = k * VEC - lead;
            const char* rin = gin + (int64_t)lead * ES;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int c = c0 + e;
                const bool in = c >= 0 && c < cols;
                const float f = Elem<DT>::load1(in ? g + e * ES : rin);
                v[e] = in ? f : 0.0f;
            }
        }
    }

    // Widen a fetched granule into v[0..VEC); elements outside the row are -inf.
    // `full` (uniform) promises k < ngran for ALIGNED windows and skips the
    // check.
    __device__ inline void widen(int k, u32x4 raw, float* v, const char* tbeg,
                                 const char* tend, bool full = false) const {
        Elem<DT>::widen(raw, v);
        if (ALIGNED) {
            if (full) return;
            if (k >= ngran) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) v[e] = kNegInf;
            }
            return;
        }
        const int c0 = k * VEC - lead;
        if (!(c0 >= 0 && c0 + VEC <= cols)) {
            const char* g = gin + (int64_t)k * 16;
            if (g >= tbeg && g + 16 <= tend) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int c = c0 + e;
                    if (!(c >= 0 && c < cols)) v[e] = kNegInf;
                }
            } else {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int c = c0 + e;
                    v[e] = (c >= 0 && c < cols) ? Elem<DT>::load1(g + e * ES) : kNegInf;
                }
            }
        }
    }

    // Mask a fetched granule in its raw form: slots outside the row get the
    // dtype's -inf bits; a granule that sticks out of the tensor has its row
    // slots read one by one here.  Integer ops only (no widening).
    __device__ inline u32x4 mask_raw(int k, u32x4 raw, const char* tbeg, const char* tend) const {
        const int c0 = k * VEC - lead;
        const char* g = gin + (int64_t)k * 16;
        const bool whole = g >= tbeg && g + 16 <= tend;
        u32x4 o;
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
            if (ES == 4) {
                const int c = c0 + wd;
                const bool ok = c >= 0 && c < cols;
                unsigned v = raw[wd];
                if (!whole) v = ok ? *(const unsigned*)(g + 4 * wd) : 0u;
                o[wd] = ok ? v : 0xff800000u;
            } else {
                const unsigned ninf = DT == kF16 ? 0xfc00u : 0xff80u;
                const int c = c0 + 2 * wd;
                const bool ok0 = c >= 0 && c < cols;
                const bool ok1 = c + 1 >= 0 && c + 1 < cols;
                unsigned lo = raw[wd] & 0xffffu, hi = raw[wd] >> 16;
                if (!whole) {
                    lo = ok0 ? *(const unsigned short*)(g + 4 * wd) : 0u;
                    hi = ok1 ? *(const unsigned short*)(g + 4 * wd + 2) : 0u;
                }
                o[wd] = (ok0 ? lo : ninf) | ((ok1 ? hi : ninf) << 16);
            }
        }
        return o;
    }

    // Store granule k.  same_phase: `out` rows share the 16-byte phase of `in`
    // rows, so interior granules are stored as 128-bit words and a partial
    // granule as at most three naturally aligned pieces per row end
    // (store_part); otherwise every element is stored on its own.  Elements
    // outside the row are never written.  All output stores are
    // non-temporal: the output is written once and not read back by the
    // kernel, and streaming it past the caches measured 15-25% faster on
    // MI355X than ordinary stores.
    // wt (uniform): rows are line-aligned and the caller wants the 128-bit
    // stores written through (store16_wt).
    __device__ inline void store(int k, const float* v, bool same_phase, bool wt = false) const {
        if (ALIGNED) {
            if (wt)
                store16_wt(gout + (int64_t)k * 16, Elem<DT>::narrow(v));
            else
                __builtin_nontemporal_store(Elem<DT>::narrow(v), (u32x4*)(gout + (int64_t)k * 16));
            return;
        }
        const int c0 = k * VEC - lead;
        if (same_phase && c0 >= 0 && c0 + VEC <= cols) {
            __builtin_nontemporal_store(Elem<DT>::narrow(v), (u32x4*)(gout + (int64_t)k * 16));
        } else if (same_phase) {
            const int lo = (c0 < 0 ? -c0 : 0) * ES;
            const int hi = (c0 + VEC > cols ? cols - c0 : VEC) * ES;
            if (lo < hi) store_part(gout + (int64_t)k * 16, Elem<DT>::narrow(v), lo, hi);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int c = c0 + e;
                if (c >= 0 && c < cols) Elem<DT>::store1(rout + (int64_t)c * ES, v[e]);
            }
        }
    }
};

// ---------------------------------------------------------------------------
// exp(x - m) for one row.  With c = round(m * log2 e), the FMA
// x*log2e - c is exact before its single rounding, so the error is relative
// to |x - m| and the common offset delta = m*log2e - c cancels in the
// normalisation of a row taken against one maximum (sums taken against
// different maxima are merged with merge_scale, which accounts for it).  delta is at most half an ulp of c, so the form is used only
// while |c| < 2^22 (|m| < 2.9e6, delta <= 1/8, far from over/underflowing
// exp2).  Rows with a larger |m| -- possible in fp32 and bf16, and for the
// running max of a thread that has only seen masked entries -- or with
// m = +inf take (x - m)*log2e instead.  m = -inf (every entry -inf) keeps
// c = 0 so that the row becomes 0/0 = NaN like the definition, and -inf
// entries under a finite max give exactly 0.
// ---------------------------------------------------------------------------
constexpr float kFmaExpLimit = 4194304.0f;  // 2^22

struct RowExp {
    float m;
    float negc;
    bool big;
    __device__ inline explicit RowExp(float m_) : m(m_) {
        float c = m_ * kLog2e;
        big = !(__builtin_fabsf(c) < kFmaExpLimit) && (m_ != kNegInf);
        negc = (m_ == kNegInf) ? 0.0f : -c;
    }
    template <int N>
    __device__ inline void apply(float (&v)[N]) const {
        if (__builtin_expect(big, 0)) {
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_exp2f((v[i] - m) * kLog2e);
        } else {
#pragma unroll
            for (int i = 0; i < N; ++i) v[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(v[i], kLog2e, negc));
        }
    }
    __device__ inline float one(float x) const {
        return big ? __builtin_amdgcn_exp2f((x - m) * kLog2e)
                   : __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, negc));
    }
};

// Scale factor for merging a partial sum d_part, accumulated as
// sum 2^(x*log2e - off(m_part)) by RowExp(m_part), into a sum taken against
// the larger maximum M:  2^(off(m_part) - off(M)).  The offset each RowExp
// subtracts is off(m) = c = fl(m*log2e) on the FMA path and the exact
// m*log2e on the `big` path; c differs from m*log2e by the product's rounding
// error delta = m*log2e - c, which an FMA gives exactly.  A single maximum
// lets delta cancel between the sum and the outputs, but partials taken
// against different maxima each carry their own 2^delta (up to 2^(1/8) for
// |m*log2e| near 2^22), so the merge uses the offsets actually subtracted:
//   both on the FMA path:  2^(c_part - c_M)         (exact difference of the c's,
//                                                    rounded once)
//   otherwise:             2^((m_part - M)*log2e - delta_part + delta_M)
// (delta = 0 on the big path).  Exactly 1 when m_part == M, which also covers
// -inf == -inf, so the (-inf, 0) identity never produces NaN; 0 for a partial
// that saw only -inf under a larger maximum.
__device__ inline float merge_scale(float m_part, float M) {
    if (m_part == M) return 1.0f;
    if (m_part == kNegInf) return 0.0f;
    const RowExp ep(m_part), eM(M);
    if (!ep.big && !eM.big) return __builtin_amdgcn_exp2f(eM.negc - ep.negc);
    const float dp = ep.big ? 0.0f : __builtin_fmaf(m_part, kLog2e, ep.negc);
    const float dM = eM.big ? 0.0f : __builtin_fmaf(M, kLog2e, eM.negc);
    return __builtin_amdgcn_exp2f(__builtin_fmaf(m_part - M, kLog2e, dM - dp));
}

// ---------------------------------------------------------------------------
// Cross-lane reductions within aligned groups of G lanes (G = 4..64) of a
// 64-lane wave.  Every lane of a group ends with the same bits (each step
// combines a lane with its partner and the partner with it, and the ops are
// commutative).  The whole wave must be active.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ inline float dpp(float v) {
    // Every source lane of these permutations is inside the wave, so
    // bound_ctrl never applies; it only lets the move fold into its consumer.
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Maximum that propagates NaN (v_maximum3_f32 on gfx950, no operand
// canonicalisation).  A NaN input makes the row max NaN and so the whole row
// NaN, the same outcome as the definition evaluated in IEEE arithmetic.
__device__ inline float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

struct OpMax {
    __device__ static inline float f(float a, float b) { return vmax(a, b); }
};
struct OpSum {
    __device__ static inline float f(float a, float b) { return a + b; }
};

template <int G, class Op>
__device__ inline float group_reduce(float v) {
    static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
    v = Op::f(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]: partner lane ^ 1
    v = Op::f(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]: partner lane ^ 2
    if (G >= 8) v = Op::f(v, dpp<0x141>(v));  // row_half_mirror: other quad of 8
    if (G >= 16) v = Op::f(v, dpp<0x140>(v));  // row_mirror: other half of 16
    if (G >= 32) {  // rows 0<->1 and 2<->3 (lane ^ 16)
        auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    if (G >= 64) {  // halves 0-31 <-> 32-63 (lane ^ 32)
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
    }
    return v;
}

// Reduction over a whole workgroup of W waves: the wave result goes to
// slots[wave], one barrier, every lane folds the W slots in the same order.
// `slots` must not be reused by another reduction without a barrier.
template <int W, class Op>
__device__ inline float block_reduce(float v, float* slots) {
    v = group_reduce<64, Op>(v);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (W == 1) return v;
    if (lane == 0) slots[wave] = v;
    __syncthreads();
    float r = slots[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r = Op::f(r, slots[i]);
    return r;
}

}  // namespace rws
