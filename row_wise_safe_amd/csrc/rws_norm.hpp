// rws_norm.hpp -- LayerNorm and RMSNorm forward on gfx950, on the softmax
// kernels' skeleton: read a row, reduce it, normalise, write (the DCU
// case-study page, section 9, names these operators as having softmax's
// structure; the Pangu-Weather profile page, section 3, runs LayerNorm as a
// wave per row with fp16 data and fp32 statistics).
//
//   LayerNorm  mu = sum x / n,  var = sum (x - mu)^2 / n,
//              y = (x - mu) / sqrt(var + eps) [* w] [+ b]
//   RMSNorm    y = x / sqrt(sum x^2 / n + eps) [* w]
//
//   norm_wave    G lanes per row, row in registers (1 read + 1 write);
//                mean, then the centred sum of squares from the same
//                registers -- both reductions in DPP/permlane only
//   norm_block   one workgroup per row, row in registers
//   norm_stream  one workgroup per row, any length: pass 1 keeps per-thread
//                moments (count, mean, sum of squared deviations) and merges
//                them with Chan's pairwise rule -- the normalisation
//                counterpart of the (m, d) merge; pass 2 re-reads the row and
//                writes
//   norm_ordered few long rows: split-k in one launch (rws_ordered.hpp):
//                stage 1 publishes each chunk's (mean, squared deviations)
//                (RMSNorm: sum of squares), stage 2 merges the row's
//                partials with the same rule, re-reads its chunk and writes
//
// The weight and bias vectors (cols entries of the tensor's dtype, optional)
// are read on each row's granule grid: one 128-bit load per interior granule
// when the vector shares the row's 16-byte phase, element loads otherwise.
// They are small and stay in the caches; their loads are issued with the
// row's own loads (affine_fetch), and kernels are instantiated with and
// without them (AFF) so that the plain normalisation keeps its registers for
// the row.
#pragma once

#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_ordered.hpp"

namespace rws {

// A per-column vector (weight or bias) on a row window's granule grid.  PM
// (phase-matched): the windows are ALIGNED and the vector starts at the
// rows' 16-byte phase, so every granule k < ngran is one 128-bit load and
// the element-by-element fallback is not compiled.  That fallback, present
// in a kernel, costs registers even where no row takes it (fp16 norm_wave
// (16,2) LayerNorm with weight and bias: 97 VGPRs with it, 59 without).
// BATCH: the fallback issues a granule's element loads before its first
// wait (the lane groups: fp16 LayerNorm with weight and bias [131072,250]
// 105 us against 144); the workgroup form keeps one wait per load, which
// measured faster there ([55392,577] 104 us against 113.5).
template <int DT, class Win, bool PM = false, bool BATCH = false>
struct ColParam {
    static constexpr int VEC = Elem<DT>::VEC;
    static constexpr int ES = Elem<DT>::SIZE;
    const char* p;  // column 0
    bool vec;       // p has the row's 16-byte phase

    __device__ inline ColParam(const void* p_, const Win& w) : p((const char*)p_) {
        const uintptr_t rin = (uintptr_t)w.gin + (uintptr_t)(w.lead * ES);
        vec = PM || (((uintptr_t)p - rin) & 15) == 0;
    }
    // 128-bit load for an interior granule with a matching phase (no wait).
    __device__ inline u32x4 fetch(const Win& w, int k) const {
        u32x4 g = {0u, 0u, 0u, 0u};
        if (PM) {
            if (k < w.ngran) g = *(const u32x4*)(p + (int64_t)k * 16);
            return g;
        }
        const int c0 = k * VEC - w.lead;
        if (vec && c0 >= 0 && c0 + VEC <= w.cols) g = *(const u32x4*)(p + (int64_t)c0 * ES);
        return g;
    }
    // Values of granule k's columns (0 outside the row); k < ngran.
    __device__ inline void widen(const Win& w, int k, u32x4 raw, float* v) const {
        const int c0 = k * VEC - w.lead;
        if (PM || (vec && c0 >= 0 && c0 + VEC <= w.cols)) {
            Elem<DT>::widen(raw, v);
            return;
        }
        if (BATCH) {
            // slots outside the row read column 0 instead
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int c = c0 + e;
                const bool in = c >= 0 && c < w.cols;
                const float f = Elem<DT>::load1(p + (int64_t)(in ? c : 0) * ES);
                v[e] = in ? f : 0.0f;
            }
            return;
        }
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = c0 + e;
            v[e] = (c >= 0 && c < w.cols) ? Elem<DT>::load1(p + (int64_t)c * ES) : 0.0f;
        }
    }
};

// Slot e of granule k belongs to the row.
template <class Win>
__device__ inline bool in_row(const Win& w, int k, int e) {
    const int c = k * Win::VEC - w.lead + e;
    return c >= 0 && c < w.cols;
}

// Sum of squared deviations from mu over the row's slots of VEC*KG values
// (granules k0, k0 + stride, ...).
template <int DT, int KG, class Win>
__device__ inline float centred_squares(const Win& w, int k0, int stride, const float* v, float mu) {
    constexpr int VEC = Elem<DT>::VEC;
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int k = k0 + stride * i;
        const bool whole = w.interior(k);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            float d = v[i * VEC + e] - mu;
            if (!whole && !in_row(w, k, e)) d = 0.0f;
            q = __builtin_fmaf(d, d, q);
        }
    }
    return q;
}

// Issue the weight / bias loads of granules k0 + stride*i (i < KG) of one
// row (no wait).  Called with the row's own loads: issued after the
// reductions instead, the loads' cache latency lands on every row's critical
// path (LayerNorm fp16 [32768,1000] with weight and bias 35.8 us against
// 32.5 us issued early; RMSNorm with weight 31.0 against 26.9).
template <int KG, class Win, class CP>
__device__ inline void affine_fetch(const Win& w, int k0, int stride, const NormArgs& A,
                                    const CP& pw, const CP& pb, u32x4* rw, u32x4* rb) {
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int k = k0 + stride * i;
        rw[i] = A.w ? pw.fetch(w, k) : u32x4{0u, 0u, 0u, 0u};
        rb[i] = A.b ? pb.fetch(w, k) : u32x4{0u, 0u, 0u, 0u};
    }
}

// Normalise and store granules k0 + stride*i (i < KG) of one row.  AFF:
// apply A.w and/or A.b (whichever is not null) from the granules
// affine_fetch loaded into rw / rb.
template <int DT, int MODE, bool AFF, int KG, class Win, class CP>
__device__ inline void norm_store(const Win& w, int k0, int stride, const float* v, float mu,
                                  float rstd, const NormArgs& A, bool same_phase, const CP* pw,
                                  const CP* pb, const u32x4* rw, const u32x4* rb) {
    constexpr int VEC = Elem<DT>::VEC;
#pragma unroll
    for (int i = 0; i < KG; ++i) {
        const int k = k0 + stride * i;
        if (k < w.ngran) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                o[e] = MODE == kLayerNorm ? (v[i * VEC + e] - mu) * rstd : v[i * VEC + e] * rstd;
            if constexpr (AFF) {
                float fw[VEC], fb[VEC];
                if (A.w) pw->widen(w, k, rw[i], fw);
                if (A.b) pb->widen(w, k, rb[i], fb);
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (A.w) o[e] *= fw[e];
                    if (A.b) o[e] += fb[e];
                }
            }
            w.store(k, o, same_phase);
        }
    }
}

// Per-row statistics use correctly rounded divisions by n (once per row):
// a row whose sum is exact then gets its exact mean, so a constant row
// normalises to exact zeros.
__device__ inline float norm_rstd(float q, const NormArgs& A) {
    return 1.0f / __builtin_sqrtf(q / A.n + A.eps);
}

// ===========================================================================
// norm_wave: G lanes per row, 64/G rows per set, U sets per wave, K granules
// per lane (the wave_row layout of the softmax kernels).
// ===========================================================================
// AFF: 0 no weight or bias, 1 either or both, 2 the same with every row's
// phase matched (ColParam PM; ALIGNED only).
template <int DT, bool ALIGNED, int G, int K, int U, int MODE, int AFF>
__global__ __launch_bounds__(256) void k_norm_wave(const void* __restrict__ in,
                                                   void* __restrict__ out, int64_t rows, int cols,
                                                   NormArgs A, int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int RPS = 64 / G;
    constexpr int N = K * VEC;
    constexpr int WA = G * 16 >= kLineBytes ? kLineBytes : 16;
    using Win = RowWin<DT, ALIGNED, WA>;
    static_assert(AFF != 2 || ALIGNED, "phase-matched parameters need aligned rows");
    using CP = ColParam<DT, Win, AFF == 2, true>;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int sub = lane / G;
    const int64_t wave_id = (int64_t)blockIdx.x * (int64_t)(blockDim.x >> 6) +
                            __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t row0 = wave_id * (RPS * U);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);

    Win w[U];
    u32x4 raw[U][K];
    constexpr int KA = AFF ? K : 1;
    u32x4 rw[AFF ? U : 1][KA], rb[AFF ? U : 1][KA];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t row = row0 + u * RPS + sub;
        row = row < rows ? row : rows - 1;
        w[u] = Win(in, out, row, cols);
#pragma unroll
        for (int i = 0; i < K; ++i) raw[u][i] = w[u].fetch(gl + G * i, tbeg, tend);
        if constexpr (AFF != 0) affine_fetch<K>(w[u], gl, G, A, CP(A.w, w[u]), CP(A.b, w[u]), rw[u], rb[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float v[N];
#pragma unroll
        for (int i = 0; i < K; ++i) widen_zero<DT>(w[u], gl + G * i, raw[u][i], &v[i * VEC], tbeg, tend);
        float mu = 0.0f, q = 0.0f;
        if (MODE == kLayerNorm) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) s += v[j];
            mu = group_reduce<G, OpSum>(s) / A.n;
            q = centred_squares<DT, K>(w[u], gl, G, v, mu);
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) q = __builtin_fmaf(v[j], v[j], q);
        }
        q = group_reduce<G, OpSum>(q);
        const float rstd = norm_rstd(q, A);
        const int64_t row = row0 + u * RPS + sub;
        if (row < rows) {
            const CP pw(A.w, w[u]), pb(A.b, w[u]);
            norm_store<DT, MODE, (AFF != 0), K>(w[u], gl, G, v, mu, rstd, A, same_phase != 0, &pw,
                                                &pb, rw[AFF ? u : 0], rb[AFF ? u : 0]);
            if (gl == 0) {
                if (A.mean) A.mean[row] = mu;
                if (A.rstd) A.rstd[row] = rstd;
            }
        }
    }
}

// ===========================================================================
// norm_block: one workgroup of BLOCK threads per row, KR granules per thread.
// With 2-5 granules per thread the compiler is asked for six waves per SIMD
// (at most 85 VGPRs): left to itself it took 132-166 VGPRs for 3-4 granules
// (three waves per SIMD), and LayerNorm fp16 [32768,1000] with 64x3 ran
// 39.8 us against 24.9 us capped (RMSNorm 36.9 / 24.3; [8192,4097] with
// 192x3 32.0 / 24.3).  No spills at that cap.
// ===========================================================================
// Waves per SIMD asked of the compiler for a norm_block kernel (1: no
// request): six for 2-3 granules per thread, five for fp32 rows with weight
// or bias at 3 (six spilled there); none where the kernel fits anyway
// (aligned affine forms) or the workgroup size already bounds the registers.
constexpr int norm_block_waves(int dt, bool aligned, int block, int kr, bool aff) {
    if (kr != 2 && kr != 3) return 1;
    if (block == 1024 || (aff && aligned)) return 1;
    if (aff && kr == 3 && dt == kF32) return 5;
    return 6;
}

// 1024-thread workgroups have at most 128 VGPRs; holding 3-4 granules of
// weight and bias from the start spilled there, so those load them late.
constexpr bool norm_block_early_affine(int block, int kr) { return !(block == 1024 && kr >= 3); }

// AFF as for k_norm_wave.
template <int DT, bool ALIGNED, int BLOCK, int KR, int MODE, int AFF>
__global__ __launch_bounds__(BLOCK)
__attribute__((amdgpu_waves_per_eu(norm_block_waves(DT, ALIGNED, BLOCK, KR, AFF != 0)))) void k_norm_block(const void* __restrict__ in,
                                                      void* __restrict__ out, int64_t rows,
                                                      int cols, NormArgs A, int same_phase, int lgrun) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    constexpr int N = KR * VEC;
    using Win = RowWin<DT, ALIGNED>;
    static_assert(AFF != 2 || ALIGNED, "phase-matched parameters need aligned rows");
    using CP = ColParam<DT, Win, AFF == 2>;
    __shared__ float red1[W];
    __shared__ float red2[W];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const Win w(in, out, row, cols);
    u32x4 raw[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) raw[i] = w.fetch(t + BLOCK * i, tbeg, tend);
    const CP pw(A.w, w), pb(A.b, w);
    u32x4 rw[AFF ? KR : 1], rb[AFF ? KR : 1];
    constexpr bool kEarly = norm_block_early_affine(BLOCK, KR);
    if constexpr (AFF != 0 && kEarly) affine_fetch<KR>(w, t, BLOCK, A, pw, pb, rw, rb);
    float v[N];
#pragma unroll
    for (int i = 0; i < KR; ++i) widen_zero<DT>(w, t + BLOCK * i, raw[i], &v[i * VEC], tbeg, tend);
    float mu = 0.0f, q = 0.0f;
    if (MODE == kLayerNorm) {
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) s += v[j];
        mu = block_reduce<W, OpSum>(s, red1) / A.n;
        q = centred_squares<DT, KR>(w, t, BLOCK, v, mu);
    } else {
#pragma unroll
        for (int j = 0; j < N; ++j) q = __builtin_fmaf(v[j], v[j], q);
    }
    q = block_reduce<W, OpSum>(q, red2);
    const float rstd = norm_rstd(q, A);
    if constexpr (AFF != 0 && !kEarly) affine_fetch<KR>(w, t, BLOCK, A, pw, pb, rw, rb);
    norm_store<DT, MODE, (AFF != 0), KR>(w, t, BLOCK, v, mu, rstd, A, same_phase != 0, &pw, &pb, rw, rb);
    if (t == 0) {
        if (A.mean) A.mean[row] = mu;
        if (A.rstd) A.rstd[row] = rstd;
    }
}

// ===========================================================================
// norm_stream: any row length.  Moments (n, mean, M2 = sum of squared
// deviations) of two disjoint sets merge as
//     n = n_a + n_b,  delta = mean_b - mean_a,
//     mean = mean_a + delta * n_b / n,  M2 = M2_a + M2_b + delta^2 n_a n_b / n
// (Chan, Golub and LeVeque's pairwise update): no sum of x^2 is ever formed,
// so a large mean does not cancel the variance away.
// ===========================================================================
__device__ inline void moments_merge(float& n, float& m, float& q, float n2, float m2, float q2) {
    const float nn = n + n2;
    if (nn > 0.0f) {
        const float d = m2 - m;
        const float f = n2 / nn;
        m = m + d * f;
        q = q + q2 + d * d * (n * f);
    }
    n = nn;
}

template <int CTRL>
__device__ inline void moments_dpp_step(float& n, float& m, float& q) {
    moments_merge(n, m, q, dpp<CTRL>(n), dpp<CTRL>(m), dpp<CTRL>(q));
}

__device__ inline void moments_swap_step(float& n, float& m, float& q, bool b32) {
    auto sw = [&](float x) {
        return b32 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                   : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    };
    const auto rn = sw(n), rm = sw(m), rq = sw(q);
    n = __uint_as_float(rn[0]);
    m = __uint_as_float(rm[0]);
    q = __uint_as_float(rq[0]);
    moments_merge(n, m, q, __uint_as_float(rn[1]), __uint_as_float(rm[1]), __uint_as_float(rq[1]));
}

// Moments of a whole workgroup; every thread gets the same result (slots
// folded in the same order).
template <int W>
__device__ inline void moments_block(float& n, float& m, float& q, float* sn, float* sm, float* sq) {
    moments_dpp_step<0xB1>(n, m, q);
    moments_dpp_step<0x4E>(n, m, q);
    moments_dpp_step<0x141>(n, m, q);
    moments_dpp_step<0x140>(n, m, q);
    moments_swap_step(n, m, q, false);
    moments_swap_step(n, m, q, true);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (lane == 0) {
        sn[wave] = n;
        sm[wave] = m;
        sq[wave] = q;
    }
    __syncthreads();
    n = sn[0];
    m = sm[0];
    q = sq[0];
#pragma unroll
    for (int i = 1; i < W; ++i) moments_merge(n, m, q, sn[i], sm[i], sq[i]);
}

template <int DT, bool ALIGNED, int BLOCK, int U, int MODE, bool AFF>
__global__ __launch_bounds__(BLOCK) void k_norm_stream(const void* __restrict__ in,
                                                       void* __restrict__ out, int64_t rows,
                                                       int cols, NormArgs A, int same_phase, int lgrun) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    using Win = RowWin<DT, ALIGNED>;
    __shared__ float sn[W];
    __shared__ float sm[W];
    __shared__ float sq[W];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const Win w(in, out, row, cols);

    // pass 1: moments (cached loads: pass 2 reads the row again)
    float n = 0.0f, m = 0.0f, q = 0.0f;
    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = w.template fetch<false>(k0 + BLOCK * u, tbeg, tend);
        float v[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) widen_zero<DT>(w, k0 + BLOCK * u, raw[u], &v[u * VEC], tbeg, tend);
        if (MODE == kLayerNorm) {
            float cnt = 0.0f, s = 0.0f;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c0 = (k0 + BLOCK * u) * VEC - w.lead;
                const int lo = c0 > 0 ? c0 : 0;
                const int hi = c0 + VEC < cols ? c0 + VEC : cols;
                cnt += (float)(hi > lo ? hi - lo : 0);
            }
#pragma unroll
            for (int j = 0; j < U * VEC; ++j) s += v[j];
            if (cnt > 0.0f) {
                const float bm = s / cnt;
                const float bq = centred_squares<DT, U>(w, k0, BLOCK, v, bm);
                moments_merge(n, m, q, cnt, bm, bq);
            }
        } else {
#pragma unroll
            for (int j = 0; j < U * VEC; ++j) q = __builtin_fmaf(v[j], v[j], q);
        }
    }
    float mu = 0.0f;
    if (MODE == kLayerNorm) {
        moments_block<W>(n, m, q, sn, sm, sq);
        mu = m;
    } else {
        q = block_reduce<W, OpSum>(q, sq);
    }
    const float rstd = norm_rstd(q, A);

    // pass 2: normalise and write
    const ColParam<DT, Win> pw(A.w, w), pb(A.b, w);
    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) raw[u] = w.fetch(k0 + BLOCK * u, tbeg, tend);
        float v[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) widen_zero<DT>(w, k0 + BLOCK * u, raw[u], &v[u * VEC], tbeg, tend);
        u32x4 rw[AFF ? U : 1], rb[AFF ? U : 1];
        if constexpr (AFF) affine_fetch<U>(w, k0, BLOCK, A, pw, pb, rw, rb);
        norm_store<DT, MODE, AFF, U>(w, k0, BLOCK, v, mu, rstd, A, same_phase != 0, &pw, &pb, rw, rb);
    }
    if (t == 0) {
        if (A.mean) A.mean[row] = mu;
        if (A.rstd) A.rstd[row] = rstd;
    }
}

// ===========================================================================
// norm_ordered: BLOCK threads x KC granules per chunk, P chunks per row
// (workgroups: ordered_slot).  A chunk's count of row elements follows from
// its position, so LayerNorm publishes two words per chunk (mean, sum of
// squared deviations about it) and RMSNorm one (sum of squares).  Stage 2
// folds the partials in chunk order and merges across the workgroup with
// moments_block, so the statistics are the same on every call.  Without
// weight and bias the kernels are compiled for six waves per SIMD (left
// alone, 125-160 VGPRs on rows that are not line-aligned; capped, 64-78 and
// no spills; with weight and bias the cap spilled).
// ===========================================================================
template <class Win>
__device__ inline float chunk_count(const Win& w, int chunk, int span) {
    const int64_t g0 = (int64_t)chunk * span;
    const int64_t lo = g0 * Win::VEC - w.lead;
    const int64_t hi = (g0 + span) * Win::VEC - w.lead;
    const int64_t n = (hi < w.cols ? hi : w.cols) - (lo > 0 ? lo : 0);
    return n > 0 ? (float)n : 0.0f;
}

template <int DT, bool ALIGNED, int BLOCK, int KC, int MODE, bool AFF>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(AFF ? 1 : 6))) void k_norm_ordered(const void* __restrict__ in,
                                                        void* __restrict__ out, int64_t rows,
                                                        int cols, NormArgs A, int P,
                                                        OrderedSync S, int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    constexpr int N = KC * VEC;
    const unsigned epoch = launch_epoch(S.epoch, S.epoch_src);
    using Win = RowWin<DT, ALIGNED>;
    __shared__ float sn[W];
    __shared__ float sm[W];
    __shared__ float sq[W];
    const int t = threadIdx.x;
    const OrderedSlot slot = ordered_slot(blockIdx.x, rows, P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const Win w(in, out, slot.row, cols);
    const int kbase = slot.chunk * (BLOCK * KC) + t;
    uint64_t* row_tags = S.tags + 2 * slot.row * P;

    u32x4 raw[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i)
        raw[i] = slot.merge_stage ? w.template fetch<true>(kbase + BLOCK * i, tbeg, tend)
                                  : w.template fetch<false>(kbase + BLOCK * i, tbeg, tend);
    const ColParam<DT, Win> pw(A.w, w), pb(A.b, w);
    u32x4 rw[AFF ? KC : 1], rb[AFF ? KC : 1];
    if (AFF && slot.merge_stage) affine_fetch<KC>(w, kbase, BLOCK, A, pw, pb, rw, rb);
    float v[N];
#pragma unroll
    for (int i = 0; i < KC; ++i) widen_zero<DT>(w, kbase + BLOCK * i, raw[i], &v[i * VEC], tbeg, tend);

    if (!slot.merge_stage) {
        if (MODE == kLayerNorm) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) s += v[j];
            s = block_reduce<W, OpSum>(s, sm);
            const float mean = s / chunk_count(w, slot.chunk, BLOCK * KC);
            float q = centred_squares<DT, KC>(w, kbase, BLOCK, v, mean);
            q = block_reduce<W, OpSum>(q, sq);
            if (t == 0) {
                publish_word(row_tags + 2 * slot.chunk, epoch, mean);
                publish_word(row_tags + 2 * slot.chunk + 1, epoch, q);
            }
        } else {
            float q = 0.0f;
#pragma unroll
            for (int j = 0; j < N; ++j) q = __builtin_fmaf(v[j], v[j], q);
            q = block_reduce<W, OpSum>(q, sq);
            if (t == 0) publish_word(row_tags + 2 * slot.chunk, epoch, q);
        }
        return;
    }

    int late = 0;
    float mu = 0.0f, q = 0.0f;
    if (MODE == kLayerNorm) {
        float n = 0.0f, m = 0.0f;
        for (int j = t; j < P; j += BLOCK) {
            const float pm = poll_word(row_tags + 2 * j, epoch, late, S.spin_limit);
            const float pq = poll_word(row_tags + 2 * j + 1, epoch, late, S.spin_limit);
            moments_merge(n, m, q, chunk_count(w, j, BLOCK * KC), pm, pq);
        }
        moments_block<W>(n, m, q, sn, sm, sq);
        mu = m;
    } else {
        for (int j = t; j < P; j += BLOCK)
            q += poll_word(row_tags + 2 * j, epoch, late, S.spin_limit);
        q = block_reduce<W, OpSum>(q, sq);
    }
    float rstd = norm_rstd(q, A);
    if (__syncthreads_or(late) != 0) {
        mu = rstd = __builtin_nanf("");
        if (t == 0) report_late(S.status);
    }
    norm_store<DT, MODE, AFF, KC>(w, kbase, BLOCK, v, mu, rstd, A, same_phase != 0, &pw, &pb, rw, rb);
    if (t == 0 && slot.chunk == 0) {
        if (A.mean) A.mean[slot.row] = mu;
        if (A.rstd) A.rstd[slot.row] = rstd;
    }
}

}  // namespace rws
