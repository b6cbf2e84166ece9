// rws_kernels.hpp -- the four gfx950 kernel families of row-wise safe
// softmax, as templates.  Each .hip file of the library instantiates one
// family for the variants the dispatcher uses.
//
// Per row every family computes m = max x, d = sum e^(x - m) in fp32 and writes
// y = e^(x - m) * (1/d), rounded to the output dtype (HIP softmax tutorial
// page, section 1).  They differ in how a row is spread over lanes and how
// often its bytes cross HBM:
//   wave_row       one row per group of G lanes (G = 4..64), row held in
//                  registers: 1 read + 1 write, reductions in DPP/permlane only
//                  (DCU case-study page, sections 4.1, 5.2 and 8).
//   block_onepass  one workgroup per row, row held in registers then LDS:
//                  1 read + 1 write (CUDA safe-online-softmax page, 2.1-2.2).
//   two_pass       one workgroup per row, running (m, d) over the row, then a
//                  second read: any length (same page, section 3.1).
//   splitk         rows cut into chunks over many workgroups; stage 1 emits a
//                  partial (m, d) per chunk, stage 2 merges a row's partials
//                  and writes its chunk (same page, section 3.2).
// Every kernel first issues all of a thread's 128-bit loads for a batch, then
// converts, so the loads of a wave are in flight together.
#pragma once

#include "rws_device.hpp"
#include "rws_launch.hpp"
#include "rws_pre.hpp"

namespace rws {

template <int DT>
__device__ inline const char* tensor_end(const void* in, int64_t rows, int cols) {
    return (const char*)in + rows * (int64_t)cols * Elem<DT>::SIZE;
}

// Values of a fetched granule with 0 (not -inf) outside the row: the form
// that sums (dot products, moments) need.
template <int DT, class Win>
__device__ inline void widen_zero(const Win& w, int k, u32x4 raw, float* v, const char* tbeg,
                                  const char* tend) {
    w.widen(k, raw, v, tbeg, tend);
    const int c0 = k * Elem<DT>::VEC - w.lead;
    if (!(c0 >= 0 && c0 + Elem<DT>::VEC <= w.cols)) {
#pragma unroll
        for (int e = 0; e < Elem<DT>::VEC; ++e) {
            const int c = c0 + e;
            if (!(c >= 0 && c < w.cols)) v[e] = 0.0f;
        }
    }
}

// Issue the loads of input granule k and of its prologue operand, unless the
// prologue says the granule cannot affect the result (then both stay zero and
// the prologue overwrites the values).  NT: the input's load policy
// (load16); the prologue operand is shared by many rows and loads cached.
template <bool NT = true, class Pre, class Win>
__device__ inline void fetch_pre(const Pre& pre, const typename Pre::Ctx& pc, const Win& w, int k,
                                 const char* tbeg, const char* tend, u32x4& raw,
                                 typename Pre::Operand& praw) {
    if (Pre::kActive) {
        raw = u32x4{0u, 0u, 0u, 0u};
        praw = typename Pre::Operand{};
        if (pre.needs_input(pc, w, k)) {
            raw = w.template fetch<NT>(k, tbeg, tend);
            praw = pre.fetch(pc, w, k);
        }
    } else {
        raw = w.template fetch<NT>(k, tbeg, tend);
    }
}

// ===========================================================================
// wave_row: G lanes per row, 64/G rows per wave "set", U sets per wave, K
// granules per lane and row.  Lane gl of a group holds granules gl + G*i, so
// the G lanes of a group read consecutive 16-byte granules at every step.
// Rows past the end are clamped to the last row for loading (in bounds) and
// are not stored.  A workgroup holds blockDim.x / 64 waves (the launcher's
// choice, kWaveGroupWaves); wave w of workgroup b is wave b*(that) + w.
// wt: the rows are line-aligned; store through (store16_wt).
// ===========================================================================
template <int DT, bool ALIGNED, int G, int K, int U, class Pre = NoPre>
__global__ __launch_bounds__(256) void k_wave_row(const void* __restrict__ in,
                                                  void* __restrict__ out, int64_t rows,
                                                  int cols, int same_phase, int wt,
                                                  Pre pre = Pre()) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int RPS = 64 / G;  // rows per set
    constexpr int N = K * VEC;   // elements per lane per row
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int sub = lane / G;
    // The wave index is uniform: readfirstlane keeps the row arithmetic scalar.
    const int64_t wave_id = (int64_t)blockIdx.x * (int64_t)(blockDim.x >> 6) +
                            __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t row0 = wave_id * (RPS * U);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    // ALIGNED rows whose window fills all G*K slots need no masking.
    const bool full = ALIGNED && (cols / VEC >= G * K);

    constexpr int WA = softmax_window_align(G);
    RowWin<DT, ALIGNED, WA> w[U];
    typename Pre::Ctx pc[U];  // prologue context of the row each set loads
    u32x4 raw[U][K];
    typename Pre::Operand praw[Pre::kActive ? U : 1][Pre::kActive ? K : 1];  // prologue operands
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t row = row0 + u * RPS + sub;
        row = row < rows ? row : rows - 1;
        w[u] = RowWin<DT, ALIGNED, WA>(in, out, row, cols);
        pc[u] = pre.ctx(row, w[u]);
#pragma unroll
        for (int i = 0; i < K; ++i)
            fetch_pre(pre, pc[u], w[u], gl + G * i, tbeg, tend, raw[u][i],
                      praw[Pre::kActive ? u : 0][Pre::kActive ? i : 0]);
    }

    float v[U][N];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int i = 0; i < K; ++i) {
            if (Pre::kActive) {
                w[u].widen_in_row(gl + G * i, raw[u][i], &v[u][i * VEC], tbeg, tend);
                pre.apply(pc[u], w[u], gl + G * i, &v[u][i * VEC],
                          praw[Pre::kActive ? u : 0][Pre::kActive ? i : 0]);
            } else {
                w[u].widen(gl + G * i, raw[u][i], &v[u][i * VEC], tbeg, tend, full);
            }
        }
        float mx = v[u][0];
#pragma unroll
        for (int j = 1; j < N; ++j) mx = vmax(mx, v[u][j]);
        mx = group_reduce<G, OpMax>(mx);
        RowExp er(mx);
        er.apply(v[u]);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) s += v[u][j];
        s = group_reduce<G, OpSum>(s);
        const float r = __builtin_amdgcn_rcpf(s);
#pragma unroll
        for (int j = 0; j < N; ++j) v[u][j] *= r;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t row = row0 + u * RPS + sub;
        if (row < rows) {
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int k = gl + G * i;
                if (k < w[u].ngran) w[u].store(k, &v[u][i * VEC], same_phase != 0, wt != 0);
            }
        }
    }
}

// ===========================================================================
// block_onepass: one workgroup of BLOCK threads per row.  Thread t holds
// granules t + BLOCK*i (i < KR) widened in registers and parks granules
// t + BLOCK*(KR + j) (j < KL) as raw bits in LDS (only thread t touches its
// LDS slots, so they need no barrier; consecutive threads use consecutive
// 16-byte slots).  Every byte of the row crosses HBM once each way.
// ===========================================================================
template <int DT, bool ALIGNED, int BLOCK, int KR, int KL, class Pre = NoPre>
__global__ __launch_bounds__(BLOCK) void k_block_onepass(const void* __restrict__ in,
                                                         void* __restrict__ out, int64_t rows,
                                                         int cols, int same_phase, int lgrun,
                                                         Pre pre = Pre()) {
    static_assert(!Pre::kActive || KL == 0, "prologues apply to register-held rows only");
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    constexpr int N = KR * VEC;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    __shared__ u32x4 park[KL > 0 ? KL : 1][KL > 0 ? BLOCK : 1];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const typename Pre::Ctx pc = pre.ctx(row, w);

    u32x4 raw[KR];
    typename Pre::Operand praw[Pre::kActive ? KR : 1];  // prologue operands
#pragma unroll
    for (int i = 0; i < KR; ++i)
        fetch_pre(pre, pc, w, t + BLOCK * i, tbeg, tend, raw[i], praw[Pre::kActive ? i : 0]);
    u32x4 rawl[KL > 0 ? KL : 1];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) rawl[j] = w.fetch(k, tbeg, tend);
    }

    float v[N];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        if (Pre::kActive) {
            w.widen_in_row(t + BLOCK * i, raw[i], &v[i * VEC], tbeg, tend);
            pre.apply(pc, w, t + BLOCK * i, &v[i * VEC], praw[Pre::kActive ? i : 0]);
        } else {
            w.widen(t + BLOCK * i, raw[i], &v[i * VEC], tbeg, tend);
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < N; ++j) mx = vmax(mx, v[j]);
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) {
            float f[VEC];
            w.widen(k, rawl[j], f, tbeg, tend);
            // partial granules are parked with -inf outside the row
            park[j][t] = w.interior(k) ? rawl[j] : Elem<DT>::narrow(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) mx = vmax(mx, f[e]);
        }
    }
    mx = block_reduce<W, OpMax>(mx, red_max);

    const RowExp er(mx);
    er.apply(v);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) s += v[j];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(park[j][t], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) s += f[e];
        }
    }
    s = block_reduce<W, OpSum>(s, red_sum);
    const float r = __builtin_amdgcn_rcpf(s);

#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const int k = t + BLOCK * i;
        if (k < w.ngran) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i * VEC + e] *= r;
            w.store(k, &v[i * VEC], same_phase != 0);
        }
    }
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(park[j][t], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] *= r;
            w.store(k, f, same_phase != 0);
        }
    }
}

// ===========================================================================
// block_onepass for 16-bit rows with 8 register granules per thread: the row
// stays in registers as raw granules (slots outside the row set to -inf)
// and is widened again for the sum and for the store, so exp is evaluated
// twice per element.  The widened form needs more than the 128 VGPRs a
// 1024-thread workgroup has and spills (40 bytes per lane on line-aligned
// rows, 172 otherwise); this one fits.  MI355X, inputs in HBM: bf16
// [16384,50257] 625 us against 1132 widened (and 788 for two_pass); fp16
// [8192,65536] 390 against 403.  At 6 granules the widened form fits and
// stays faster (fp16 [8192,49000] 294 us against 303).
// ===========================================================================
template <int DT, bool ALIGNED, int BLOCK, int KR, int KL>
__global__ __launch_bounds__(BLOCK) void k_block_onepass_raw(const void* __restrict__ in,
                                                             void* __restrict__ out, int64_t rows,
                                                             int cols, int same_phase, int lgrun) {
    static_assert(Elem<DT>::SIZE == 2, "raw rows are for 16-bit dtypes");
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    __shared__ u32x4 park[KL > 0 ? KL : 1][KL > 0 ? BLOCK : 1];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);

    u32x4 raw[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) raw[i] = w.fetch(t + BLOCK * i, tbeg, tend);
    u32x4 rawl[KL > 0 ? KL : 1];
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) rawl[j] = w.fetch(k, tbeg, tend);
    }
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const int k = t + BLOCK * i;
        if (!ALIGNED && k < w.ngran && !w.interior(k)) raw[i] = w.mask_raw(k, raw[i], tbeg, tend);
    }

    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        if (t + BLOCK * i < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) mx = vmax(mx, f[e]);
        }
    }
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) {
            float f[VEC];
            w.widen(k, rawl[j], f, tbeg, tend);
            // partial granules are parked with -inf outside the row
            park[j][t] = w.interior(k) ? rawl[j] : Elem<DT>::narrow(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) mx = vmax(mx, f[e]);
        }
    }
    mx = block_reduce<W, OpMax>(mx, red_max);

    const RowExp er(mx);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        if (t + BLOCK * i < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) s += f[e];
        }
    }
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        if (t + BLOCK * (KR + j) < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(park[j][t], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) s += f[e];
        }
    }
    s = block_reduce<W, OpSum>(s, red_sum);
    const float r = __builtin_amdgcn_rcpf(s);

#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const int k = t + BLOCK * i;
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] *= r;
            w.store(k, f, same_phase != 0);
        }
    }
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int k = t + BLOCK * (KR + j);
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(park[j][t], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] *= r;
            w.store(k, f, same_phase != 0);
        }
    }
}

// ===========================================================================
// Running (m, d) of one thread over a batch of N values (-inf entries add 0):
//   m' = max(m, max batch);  d' = d e^(m - m') + sum e^(x - m')
// with d kept against RowExp(m)'s offset and rescaled by merge_scale.
// (DCU case-study page, section 4.3; CUDA safe-online-softmax page, section 1,
// there per chunk of 256).
// ===========================================================================
template <int N>
__device__ inline void online_update(float& m, float& d, const float (&v)[N]) {
    float lm = v[0];
#pragma unroll
    for (int j = 1; j < N; ++j) lm = vmax(lm, v[j]);
    const float mn = vmax(m, lm);
    if (mn != kNegInf) {
        const RowExp er(mn);
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) s += er.one(v[j]);
        d = d * merge_scale(m, mn) + s;
        m = mn;
    }
}

// Merge every thread's (m, d) into the row's (M, D) over the workgroup:
// M = max over threads, D = sum over threads of d e^(m - M) -- the (m, d)
// merge rule applied across the block, written as one max reduction and one
// sum reduction (CUDA safe-online-softmax page, section 2.1.1).
template <int W>
__device__ inline void block_merge(float m, float d, float& M, float& D, float* red_max,
                                   float* red_sum) {
    M = block_reduce<W, OpMax>(m, red_max);
    const float ds = (d == 0.0f) ? 0.0f : d * merge_scale(m, M);
    D = block_reduce<W, OpSum>(ds, red_sum);
}

// ===========================================================================
// two_pass: one workgroup per row, any row length.  Pass 1 streams the row in
// batches of U granules per thread with the running (m, d); the block merges
// the threads' pairs; pass 2 re-reads the row (from L2 / last-level cache when
// the row was just read) and writes e^(x - M) / D.
// ===========================================================================
template <int DT, bool ALIGNED, int BLOCK, int U, class Pre = NoPre>
__global__ __launch_bounds__(BLOCK) void k_two_pass(const void* __restrict__ in,
                                                    void* __restrict__ out, int64_t rows,
                                                    int cols, int same_phase, int lgrun,
                                                    Pre pre = Pre()) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const typename Pre::Ctx pc = pre.ctx(row, w);

    float m = kNegInf, d = 0.0f;
    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 raw[U];
        typename Pre::Operand praw[Pre::kActive ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u)  // cached: pass 2 reads the row again
            fetch_pre<false>(pre, pc, w, k0 + BLOCK * u, tbeg, tend, raw[u],
                             praw[Pre::kActive ? u : 0]);
        float v[U * VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + BLOCK * u;
            if (Pre::kActive) {
                w.widen_in_row(k, raw[u], &v[u * VEC], tbeg, tend);
                pre.apply(pc, w, k, &v[u * VEC], praw[Pre::kActive ? u : 0]);
            } else {
                w.widen(k, raw[u], &v[u * VEC], tbeg, tend);
                if (!ALIGNED && k >= w.ngran) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) v[u * VEC + e] = kNegInf;
                }
            }
        }
        online_update(m, d, v);
    }
    float M, D;
    block_merge<W>(m, d, M, D, red_max, red_sum);
    const RowExp er(M);
    const float r = __builtin_amdgcn_rcpf(D);

    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 raw[U];
        typename Pre::Operand praw[Pre::kActive ? U : 1];
#pragma unroll
        for (int u = 0; u < U; ++u)
            fetch_pre(pre, pc, w, k0 + BLOCK * u, tbeg, tend, raw[u], praw[Pre::kActive ? u : 0]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + BLOCK * u;
            if (k < w.ngran) {
                float f[VEC];
                if (Pre::kActive) {
                    w.widen_in_row(k, raw[u], f, tbeg, tend);
                    pre.apply(pc, w, k, f, praw[Pre::kActive ? u : 0]);
                } else {
                    w.widen(k, raw[u], f, tbeg, tend);
                }
#pragma unroll
                for (int e = 0; e < VEC; ++e) f[e] = er.one(f[e]) * r;
                w.store(k, f, same_phase != 0);
            }
        }
    }
}

// ===========================================================================
// split-k.  A row's window of granules is cut into P chunks of CG = BLOCK*KC
// granules; workgroup b handles chunk b % P of row b / P.
//   stage 1: chunk max, chunk sum of e^(x - m_c) -> partial (m_c, d_c)
//   stage 2: merge the row's P partials into (M, D), re-read the chunk,
//            write e^(x - M) / D.
// The two-launch form orders the stages by the launch boundary; the ordered
// single launch (rws_splitk_ordered.hip) runs both stages as workgroups of
// one grid.  Both share the stage bodies below.
// ===========================================================================

// Issue the loads of one chunk (KC granules per thread, BLOCK granules apart).
// Stage 1 loads cached (NT = false: stage 2 reads the chunk again), stage 2
// non-temporal (the last read).
template <int DT, bool ALIGNED, int BLOCK, int KC, bool NT>
__device__ inline void splitk_fetch(const RowWin<DT, ALIGNED>& w, int kbase, const char* tbeg,
                                    const char* tend, u32x4 (&raw)[KC]) {
#pragma unroll
    for (int i = 0; i < KC; ++i) raw[i] = w.template fetch<NT>(kbase + BLOCK * i, tbeg, tend);
}

// Stage 1 body: the chunk's (max, sum of e^(x - max)), in every thread.
template <int DT, bool ALIGNED, int BLOCK, int KC>
__device__ inline float2 splitk_partial(const RowWin<DT, ALIGNED>& w, int kbase,
                                        const u32x4 (&raw)[KC], const char* tbeg,
                                        const char* tend, float* red_max, float* red_sum) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    constexpr int N = KC * VEC;
    float v[N];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        w.widen(k, raw[i], &v[i * VEC], tbeg, tend);
        if (!ALIGNED && k >= w.ngran) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) v[i * VEC + e] = kNegInf;
        }
    }
    float mx = v[0];
#pragma unroll
    for (int j = 1; j < N; ++j) mx = vmax(mx, v[j]);
    mx = block_reduce<W, OpMax>(mx, red_max);
    const RowExp er(mx);
    er.apply(v);
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) s += v[j];
    s = block_reduce<W, OpSum>(s, red_sum);
    return make_float2(mx, s);
}

// Fold one partial (pm, pd) into a thread's running (m, d) (the merge rule
// with (-inf, 0) as identity: a side with d == 0 contributes nothing).
__device__ inline void md_fold(float& m, float& d, float pm, float pd) {
    const float mn = vmax(m, pm);
    const float a = (d == 0.0f) ? 0.0f : d * merge_scale(m, mn);
    const float b = (pd == 0.0f) ? 0.0f : pd * merge_scale(pm, mn);
    m = mn;
    d = a + b;
}

// Stage 2 tail: write y = e^(x - M) * r for the chunk already in `raw`.
template <int DT, bool ALIGNED, int BLOCK, int KC>
__device__ inline void splitk_write(const RowWin<DT, ALIGNED>& w, int kbase,
                                    const u32x4 (&raw)[KC], const char* tbeg, const char* tend,
                                    float M, float r, bool same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    const RowExp er(M);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        if (k < w.ngran) {
            float f[VEC];
            w.widen(k, raw[i], f, tbeg, tend);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] = er.one(f[e]) * r;
            w.store(k, f, same_phase);
        }
    }
}

template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK) void k_splitk_stage1(const void* __restrict__ in,
                                                         int64_t rows, int cols, int P,
                                                         float2* __restrict__ ws) {
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int chunk = (int)(b - row * P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, const_cast<void*>(in), row, cols);  // out unused
    const int kbase = chunk * (BLOCK * KC) + t;

    u32x4 raw[KC];
    splitk_fetch<DT, ALIGNED, BLOCK, KC, false>(w, kbase, tbeg, tend, raw);
    const float2 md =
        splitk_partial<DT, ALIGNED, BLOCK, KC>(w, kbase, raw, tbeg, tend, red_max, red_sum);
    if (t == 0) ws[row * P + chunk] = md;
}

template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK) void k_splitk_stage2(const void* __restrict__ in,
                                                         void* __restrict__ out, int64_t rows,
                                                         int cols, int P,
                                                         const float2* __restrict__ ws,
                                                         int same_phase) {
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int chunk = (int)(b - row * P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const int kbase = chunk * (BLOCK * KC) + t;

    // Issue the chunk's loads first; the partial merge overlaps their latency.
    u32x4 raw[KC];
    splitk_fetch<DT, ALIGNED, BLOCK, KC, true>(w, kbase, tbeg, tend, raw);
    float m = kNegInf, d = 0.0f;
    for (int j = t; j < P; j += BLOCK) {
        const float2 p = ws[row * P + j];
        md_fold(m, d, p.x, p.y);
    }
    float M, D;
    block_merge<W>(m, d, M, D, red_max, red_sum);
    splitk_write<DT, ALIGNED, BLOCK, KC>(w, kbase, raw, tbeg, tend, M, __builtin_amdgcn_rcpf(D),
                                        same_phase != 0);
}

}  // namespace rws
