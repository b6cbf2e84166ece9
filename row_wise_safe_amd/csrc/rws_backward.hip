// rws_backward.hip -- softmax backward on gfx950: for each row,
//     dot = sum_j dy_j * y_j,     dx_j = y_j * (dy_j - dot)
// (the gradient through y = softmax(x); the DCU case-study page, section 5.4,
// notes that training needs the backward pass checked on its own).  Same
// skeleton as the forward kernels -- read, one row reduction, elementwise
// write -- with two inputs: 2 reads + 1 write per element.
//
//   bwd_wave    G lanes per row, registers (rows up to 512 granules)
//   bwd_block   one workgroup per row, registers
//   bwd_stream  one workgroup per row, any length: pass 1 the dot product,
//               pass 2 re-reads y and dy (L2 / last-level cache) and writes
//   bwd_ordered few long rows: split-k in one launch (rws_ordered.hpp):
//               stage 1 publishes each chunk's partial dot product, stage 2
//               sums the row's partials, re-reads its chunk and writes
//
// y's row window (rws_device.hpp) drives all three tensors: dy's granule k
// is at the same offset from y's plus the constant dy - y (both have pitch
// cols), loaded as one 128-bit word when that difference is a multiple of 16
// bytes, element by element otherwise; dx is stored through the window like
// the forward output.  No byte outside a tensor is read or written.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_ordered.hpp"

namespace rws {

// The second input (dy) on the first input's granule grid.
template <int DT, class Win>
struct Second {
    static constexpr int VEC = Elem<DT>::VEC;
    static constexpr int ES = Elem<DT>::SIZE;
    const char* base;   // dy tensor
    const char* end;
    int64_t delta;      // dy - y in bytes
    bool vec;           // delta % 16 == 0

    template <bool NT = true>  // load policy: see load16
    __device__ inline u32x4 fetch(const Win& w, int k) const {
        u32x4 g = {0u, 0u, 0u, 0u};
        if (!vec) return g;
        const int c0 = k * VEC - w.lead;
        const char* p = w.gin + (int64_t)k * 16 + delta;
        if (c0 + VEC > 0 && c0 < w.cols && p >= base && p + 16 <= end) g = load16<NT>(p);
        return g;
    }
    // dy values of granule k (0 outside the row)
    __device__ inline void widen(const Win& w, int k, u32x4 raw, float* v) const {
        const int c0 = k * VEC - w.lead;
        const char* p = w.gin + (int64_t)k * 16 + delta;
        if (vec && c0 >= 0 && c0 + VEC <= w.cols) {
            Elem<DT>::widen(raw, v);
            return;
        }
        const bool whole = vec && p >= base && p + 16 <= end;
        float f[VEC];
        Elem<DT>::widen(raw, f);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int c = c0 + e;
            const bool ok = c >= 0 && c < w.cols;
            v[e] = !ok ? 0.0f : whole ? f[e] : Elem<DT>::load1(p + e * ES);
        }
    }
};

// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, int G, int K, int U>
__global__ __launch_bounds__(256) void k_bwd_wave(const void* __restrict__ y,
                                                  const void* __restrict__ dy,
                                                  void* __restrict__ dx, int64_t rows, int cols,
                                                  int dy_vec, int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int RPS = 64 / G;
    constexpr int N = K * VEC;
    constexpr int WA = G * 16 >= kLineBytes ? kLineBytes : 16;
    using Win = RowWin<DT, ALIGNED, WA>;
    const int lane = threadIdx.x & 63;
    const int gl = lane & (G - 1);
    const int sub = lane / G;
    const int64_t wave_id = (int64_t)blockIdx.x * (int64_t)(blockDim.x >> 6) +
                            __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int64_t row0 = wave_id * (RPS * U);
    const char* tbeg = (const char*)y;
    const char* tend = tensor_end<DT>(y, rows, cols);
    const Second<DT, Win> s2{(const char*)dy, tensor_end<DT>(dy, rows, cols),
                             (int64_t)((const char*)dy - (const char*)y), dy_vec != 0};

    Win w[U];
    u32x4 ry[U][K], rg[U][K];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        int64_t row = row0 + u * RPS + sub;
        row = row < rows ? row : rows - 1;
        w[u] = Win(y, dx, row, cols);
#pragma unroll
        for (int i = 0; i < K; ++i) {
            ry[u][i] = w[u].fetch(gl + G * i, tbeg, tend);
            rg[u][i] = s2.fetch(w[u], gl + G * i);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float vy[N], vg[N];
#pragma unroll
        for (int i = 0; i < K; ++i) {
            widen_zero<DT>(w[u], gl + G * i, ry[u][i], &vy[i * VEC], tbeg, tend);
            s2.widen(w[u], gl + G * i, rg[u][i], &vg[i * VEC]);
        }
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < N; ++j) dot = __builtin_fmaf(vy[j], vg[j], dot);
        dot = group_reduce<G, OpSum>(dot);
        const int64_t row = row0 + u * RPS + sub;
        if (row < rows) {
#pragma unroll
            for (int i = 0; i < K; ++i) {
                const int k = gl + G * i;
                if (k < w[u].ngran) {
                    float o[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) o[e] = vy[i * VEC + e] * (vg[i * VEC + e] - dot);
                    w[u].store(k, o, same_phase != 0);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Three granules per thread below 1024 threads compile for six waves per
// SIMD: left alone the compiler took 144 VGPRs (three waves), and fp16
// [8192,4097] with 192x3 ran 36.2 us against 33.9 us capped.
template <int DT, bool ALIGNED, int BLOCK, int KR>
__global__ __launch_bounds__(BLOCK)
__attribute__((amdgpu_waves_per_eu(KR == 3 && BLOCK < 1024 ? 6 : 1))) void k_bwd_block(const void* __restrict__ y,
                                                     const void* __restrict__ dy,
                                                     void* __restrict__ dx, int64_t rows,
                                                     int cols, int dy_vec, int same_phase,
                                                     int lgrun) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    constexpr int N = KR * VEC;
    using Win = RowWin<DT, ALIGNED>;
    __shared__ float red[W];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)y;
    const char* tend = tensor_end<DT>(y, rows, cols);
    const Second<DT, Win> s2{(const char*)dy, tensor_end<DT>(dy, rows, cols),
                             (int64_t)((const char*)dy - (const char*)y), dy_vec != 0};
    const Win w(y, dx, row, cols);
    u32x4 ry[KR], rg[KR];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        ry[i] = w.fetch(t + BLOCK * i, tbeg, tend);
        rg[i] = s2.fetch(w, t + BLOCK * i);
    }
    float vy[N], vg[N];
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        widen_zero<DT>(w, t + BLOCK * i, ry[i], &vy[i * VEC], tbeg, tend);
        s2.widen(w, t + BLOCK * i, rg[i], &vg[i * VEC]);
    }
    float dot = 0.0f;
#pragma unroll
    for (int j = 0; j < N; ++j) dot = __builtin_fmaf(vy[j], vg[j], dot);
    dot = block_reduce<W, OpSum>(dot, red);
#pragma unroll
    for (int i = 0; i < KR; ++i) {
        const int k = t + BLOCK * i;
        if (k < w.ngran) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = vy[i * VEC + e] * (vg[i * VEC + e] - dot);
            w.store(k, o, same_phase != 0);
        }
    }
}

// ---------------------------------------------------------------------------
template <int DT, bool ALIGNED, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_bwd_stream(const void* __restrict__ y,
                                                      const void* __restrict__ dy,
                                                      void* __restrict__ dx, int64_t rows,
                                                      int cols, int dy_vec, int same_phase,
                                                      int lgrun) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    using Win = RowWin<DT, ALIGNED>;
    __shared__ float red[W];
    const int t = threadIdx.x;
    const int64_t row = xcd_run(blockIdx.x, gridDim.x, lgrun);
    const char* tbeg = (const char*)y;
    const char* tend = tensor_end<DT>(y, rows, cols);
    const Second<DT, Win> s2{(const char*)dy, tensor_end<DT>(dy, rows, cols),
                             (int64_t)((const char*)dy - (const char*)y), dy_vec != 0};
    const Win w(y, dx, row, cols);
    float dot = 0.0f;
    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 ry[U], rg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {  // cached: pass 2 reads both again
            ry[u] = w.template fetch<false>(k0 + BLOCK * u, tbeg, tend);
            rg[u] = s2.template fetch<false>(w, k0 + BLOCK * u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float vy[VEC], vg[VEC];
            widen_zero<DT>(w, k0 + BLOCK * u, ry[u], vy, tbeg, tend);
            s2.widen(w, k0 + BLOCK * u, rg[u], vg);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dot = __builtin_fmaf(vy[e], vg[e], dot);
        }
    }
    dot = block_reduce<W, OpSum>(dot, red);
    for (int k0 = t; k0 < w.ngran; k0 += BLOCK * U) {
        u32x4 ry[U], rg[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            ry[u] = w.fetch(k0 + BLOCK * u, tbeg, tend);
            rg[u] = s2.fetch(w, k0 + BLOCK * u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + BLOCK * u;
            if (k < w.ngran) {
                float vy[VEC], vg[VEC], o[VEC];
                widen_zero<DT>(w, k, ry[u], vy, tbeg, tend);
                s2.widen(w, k, rg[u], vg);
#pragma unroll
                for (int e = 0; e < VEC; ++e) o[e] = vy[e] * (vg[e] - dot);
                w.store(k, o, same_phase != 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// variants and launchers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// bwd_ordered: BLOCK threads x KC granules per chunk, P chunks per row.  The
// dot product is summed chunk by chunk in a fixed order (partials 0..P-1
// folded per thread, then the block reduction), so the result is the same
// on every call.  Stage 1 loads cached (stage 2 reads the chunk again),
// stage 2 non-temporally.
template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK) void k_bwd_ordered(const void* __restrict__ y,
                                                       const void* __restrict__ dy,
                                                       void* __restrict__ dx, int64_t rows,
                                                       int cols, int P, OrderedSync S,
                                                       int dy_vec, int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    using Win = RowWin<DT, ALIGNED>;
    __shared__ float red[W];
    const int t = threadIdx.x;
    const unsigned epoch = launch_epoch(S.epoch, S.epoch_src);
    const OrderedSlot slot = ordered_slot(blockIdx.x, rows, P);
    const char* tbeg = (const char*)y;
    const char* tend = tensor_end<DT>(y, rows, cols);
    const Second<DT, Win> s2{(const char*)dy, tensor_end<DT>(dy, rows, cols),
                             (int64_t)((const char*)dy - (const char*)y), dy_vec != 0};
    const Win w(y, dx, slot.row, cols);
    const int kbase = slot.chunk * (BLOCK * KC) + t;
    uint64_t* row_tags = S.tags + 2 * slot.row * P;

    u32x4 ry[KC], rg[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        if (slot.merge_stage) {
            ry[i] = w.template fetch<true>(k, tbeg, tend);
            rg[i] = s2.template fetch<true>(w, k);
        } else {
            ry[i] = w.template fetch<false>(k, tbeg, tend);
            rg[i] = s2.template fetch<false>(w, k);
        }
    }

    if (!slot.merge_stage) {
        float dot = 0.0f;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            const int k = kbase + BLOCK * i;
            if (k < w.ngran) {
                float vy[VEC], vg[VEC];
                widen_zero<DT>(w, k, ry[i], vy, tbeg, tend);
                s2.widen(w, k, rg[i], vg);
#pragma unroll
                for (int e = 0; e < VEC; ++e) dot = __builtin_fmaf(vy[e], vg[e], dot);
            }
        }
        dot = block_reduce<W, OpSum>(dot, red);
        if (t == 0) publish_word(row_tags + 2 * slot.chunk, epoch, dot);
        return;
    }

    float dot = 0.0f;
    int late = 0;
    for (int j = t; j < P; j += BLOCK)
        dot += poll_word(row_tags + 2 * j, epoch, late, S.spin_limit);
    dot = block_reduce<W, OpSum>(dot, red);
    if (__syncthreads_or(late) != 0) {
        dot = __builtin_nanf("");
        if (t == 0) report_late(S.status);
    }
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        if (k < w.ngran) {
            float vy[VEC], vg[VEC], o[VEC];
            widen_zero<DT>(w, k, ry[i], vy, tbeg, tend);
            s2.widen(w, k, rg[i], vg);
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = vy[e] * (vg[e] - dot);
            w.store(k, o, same_phase != 0);
        }
    }
}

#define RWS_BWD_WAVE_VARIANTS(X) \
    X(4, 1, 1)                   \
    X(8, 1, 1)                   \
    X(16, 1, 1)                  \
    X(32, 1, 1)                  \
    X(64, 1, 1)                  \
    X(64, 2, 1)                  \
    X(64, 4, 1)                  \
    X(64, 8, 1)
// (threads, register granules per thread of each input): one granule per
// thread up to 1024 granules per row and the forward's three-granule shapes
// (which replace 192x1 and 576x1 at equal capacity), then 1024-thread
// workgroups.
#define RWS_BWD_BLOCK_VARIANTS(X)                                        \
    X(128, 1) X(256, 1) X(320, 1) X(384, 1) X(512, 1) X(640, 1) X(768, 1)  \
    X(1024, 1) X(64, 3) X(192, 3) X(384, 3) X(1024, 2) X(1024, 3)          \
    X(1024, 4)
#define RWS_BWD_STREAM_VARIANTS(X) \
    X(256, 4)                      \
    X(1024, 4)

#define RWS_ROW3(a, b, c) {a, b, c},
#define RWS_ROW2(a, b) {a, b},
const WaveRowVariant kBwdWave[] = {RWS_BWD_WAVE_VARIANTS(RWS_ROW3)};
const int kNumBwdWave = sizeof(kBwdWave) / sizeof(kBwdWave[0]);
const TwoPassVariant kBwdBlock[] = {RWS_BWD_BLOCK_VARIANTS(RWS_ROW2)};
const int kNumBwdBlock = sizeof(kBwdBlock) / sizeof(kBwdBlock[0]);
const TwoPassVariant kBwdStream[] = {RWS_BWD_STREAM_VARIANTS(RWS_ROW2)};
const int kNumBwdStream = sizeof(kBwdStream) / sizeof(kBwdStream[0]);
#undef RWS_ROW3
#undef RWS_ROW2

#define RWS_DT_SWITCH(CALL)                                                   \
    switch (B.dtype) {                                                        \
        case kF32: return B.aligned ? CALL(kF32, true) : CALL(kF32, false);   \
        case kF16: return B.aligned ? CALL(kF16, true) : CALL(kF16, false);   \
        case kBF16: return B.aligned ? CALL(kBF16, true) : CALL(kBF16, false); \
    }                                                                         \
    return hipErrorInvalidValue;

template <int DT, bool AL, int G, int K, int U>
static hipError_t bw(const BwdLaunch& B) {
    const WaveRowVariant v = {G, K, U};
    hipLaunchKernelGGL((k_bwd_wave<DT, AL, G, K, U>), dim3((unsigned)wave_row_grid(v, B.rows)),
                       dim3(kWaveGroupThreads), 0, B.stream, B.y, B.dy, B.dx, B.rows, B.cols, (int)B.dy_vec,
                       (int)B.same_phase);
    return hipGetLastError();
}
template <int DT, bool AL, int BL, int KR>
static hipError_t bb(const BwdLaunch& B) {
    hipLaunchKernelGGL((k_bwd_block<DT, AL, BL, KR>), dim3((unsigned)B.rows), dim3(BL), 0,
                       B.stream, B.y, B.dy, B.dx, B.rows, B.cols, (int)B.dy_vec,
                       (int)B.same_phase, B.lgrun);
    return hipGetLastError();
}
template <int DT, bool AL, int BL, int U>
static hipError_t bs(const BwdLaunch& B) {
    hipLaunchKernelGGL((k_bwd_stream<DT, AL, BL, U>), dim3((unsigned)B.rows), dim3(BL), 0,
                       B.stream, B.y, B.dy, B.dx, B.rows, B.cols, (int)B.dy_vec,
                       (int)B.same_phase, B.lgrun);
    return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t bo(const BwdLaunch& B, int P, const OrderedSync& S) {
    hipLaunchKernelGGL((k_bwd_ordered<DT, AL, kBwdOrderedBlock, kBwdOrderedKc>),
                       dim3((unsigned)(2 * B.rows * P)), dim3(kBwdOrderedBlock), 0, B.stream, B.y,
                       B.dy, B.dx, B.rows, B.cols, P, S, (int)B.dy_vec, (int)B.same_phase);
    return hipGetLastError();
}

hipError_t launch_bwd_ordered(const BwdLaunch& B, int P, const OrderedSync& S) {
    switch (B.dtype) {
        case kF32: return B.aligned ? bo<kF32, true>(B, P, S) : bo<kF32, false>(B, P, S);
        case kF16: return B.aligned ? bo<kF16, true>(B, P, S) : bo<kF16, false>(B, P, S);
        case kBF16: return B.aligned ? bo<kBF16, true>(B, P, S) : bo<kBF16, false>(B, P, S);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdLaunch& B, int family, int variant) {
    int i = 0;
    if (family == 1) {
#define RWS_CALL_W(DT_, AL_) bw<DT_, AL_, G_, K_, U_>(B)
#define RWS_CASE(g, k, u)                                                 \
    if (variant == i) {                                                   \
        constexpr int G_ = g, K_ = k, U_ = u;                             \
        RWS_DT_SWITCH(RWS_CALL_W)                                         \
    }                                                                     \
    ++i;
        RWS_BWD_WAVE_VARIANTS(RWS_CASE)
#undef RWS_CASE
#undef RWS_CALL_W
    } else if (family == 2) {
#define RWS_CALL_B(DT_, AL_) bb<DT_, AL_, BL_, KR_>(B)
#define RWS_CASE(b, kr)                                                   \
    if (variant == i) {                                                   \
        constexpr int BL_ = b, KR_ = kr;                                  \
        RWS_DT_SWITCH(RWS_CALL_B)                                         \
    }                                                                     \
    ++i;
        RWS_BWD_BLOCK_VARIANTS(RWS_CASE)
#undef RWS_CASE
#undef RWS_CALL_B
    } else if (family == 3) {
#define RWS_CALL_S(DT_, AL_) bs<DT_, AL_, BL_, U_>(B)
#define RWS_CASE(b, u)                                                    \
    if (variant == i) {                                                   \
        constexpr int BL_ = b, U_ = u;                                    \
        RWS_DT_SWITCH(RWS_CALL_S)                                         \
    }                                                                     \
    ++i;
        RWS_BWD_STREAM_VARIANTS(RWS_CASE)
#undef RWS_CASE
#undef RWS_CALL_S
    }
    return hipErrorInvalidValue;
}

}  // namespace rws
