// rws_splitk_fused.hip -- split-k in a single cooperative launch that reads
// every element once.
//
// The two-launch split-k (rws_splitk.hip) and its single-launch ordered form
// (rws_splitk_ordered.hip) read every chunk twice: once for the chunk's
// partial (m, d), again to write the outputs once the row's partials are
// merged.  Here every workgroup keeps its chunk in registers between the two
// halves: it publishes its partial, waits for the partials of the row's other
// chunks, merges them and writes its chunk from registers -- one read and one
// write per element.  The CUDA safe-online-softmax page names this
// single-kernel form (a grid-wide sync, or atomics with polling) in section
// 3.2 and leaves it unbuilt; the (m, d) merge is the same rule.
//
// Exchange: as in the ordered form (rws_ordered.hpp), a partial travels as
// two 64-bit words, (epoch << 32 | bits of m) and (epoch << 32 | bits of d),
// stored and polled with relaxed agent-scope atomics; each word carries its
// own data, so no release/acquire fence (which on this multi-XCD part writes
// back and invalidates an XCD's L2) is needed.
//
// Waiting for other workgroups of the grid is only safe when all of them are
// resident at once, so the kernel is launched with hipLaunchCooperativeKernel,
// which refuses grids that cannot be co-resident (RWS_ERR_UNSUPPORTED_SHAPE
// then).  The wait is also bounded: a workgroup that does not see a partial
// after the launch's spin limit stops waiting, writes NaN for its chunk and
// sets the stream's status word (softmax_stream_status reports it), so every
// wave always reaches the end of the kernel.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_ordered.hpp"

namespace rws {

// Max of the VEC elements of a raw granule (exact; NaN propagates).
template <int DT>
__device__ inline float granule_max(u32x4 g) {
    float f[Elem<DT>::VEC];
    Elem<DT>::widen(g, f);
    float m = f[0];
#pragma unroll
    for (int e = 1; e < Elem<DT>::VEC; ++e) m = vmax(m, f[e]);
    return m;
}

// Waves per SIMD the kernel must allow so that the grids the dispatcher
// gives it fit at once (KC 4: 8 waves, i.e. <= 64 VGPRs; KC 8: 4; KC 16: 2).
template <int KC>
constexpr int fused_min_waves() { return KC <= 4 ? 8 : KC <= 8 ? 4 : 2; }

template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK, fused_min_waves<KC>()) void k_splitk_fused(const void* __restrict__ in,
                                                        void* __restrict__ out, int64_t rows,
                                                        int cols, int P, OrderedSync S,
                                                        int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    __shared__ float red_max2[W];
    __shared__ float red_sum2[W];
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int chunk = (int)(b - row * P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const int kbase = chunk * (BLOCK * KC) + t;
    uint64_t* row_tags = S.tags + 2 * row * P;
    const unsigned epoch = launch_epoch(S.epoch, S.epoch_src);

    // The chunk stays in registers as raw 16-byte granules (half the
    // registers of fp32 for 16-bit types); granules past the window or
    // partly outside the row are rewritten with -inf in the foreign slots.
    u32x4 raw[KC];
#pragma unroll
    for (int i = 0; i < KC; ++i) raw[i] = w.fetch(kbase + BLOCK * i, tbeg, tend);
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        if (!w.interior(k)) raw[i] = w.mask_raw(k, raw[i], tbeg, tend);
    }

    // chunk max, chunk sum of e^(x - m_c)
    float mc = granule_max<DT>(raw[0]);
#pragma unroll
    for (int i = 1; i < KC; ++i) mc = vmax(mc, granule_max<DT>(raw[i]));
    mc = block_reduce<W, OpMax>(mc, red_max);
    float dc = 0.0f;
    {
        const RowExp er(mc);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
            er.apply(f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) dc += f[e];
        }
    }
    dc = block_reduce<W, OpSum>(dc, red_sum);
    if (t == 0) {
        publish_word(row_tags + 2 * chunk, epoch, mc);
        publish_word(row_tags + 2 * chunk + 1, epoch, dc);
    }
    // Keep only the raw granules live across the wait: without this the
    // compiler would reuse the widened fp32 values of the passes above and
    // hold twice the registers.  (An empty asm statement: no instruction.)
#pragma unroll
    for (int i = 0; i < KC; ++i) asm volatile("" : "+v"(raw[i]));

    // merge the row's partials (this chunk's own included): (M, D)
    float m = kNegInf, d = 0.0f;
    int late = 0;
    for (int j = t; j < P; j += BLOCK) {
        const float pm = poll_word(row_tags + 2 * j, epoch, late, S.spin_limit);
        const float pd = poll_word(row_tags + 2 * j + 1, epoch, late, S.spin_limit);
        md_fold(m, d, pm, pd);
    }
    float M, D;
    block_merge<W>(m, d, M, D, red_max2, red_sum2);
    const bool failed = __syncthreads_or(late) != 0;
    if (failed && t == 0) report_late(S.status);
    const RowExp er(M);
    const float r = failed ? __builtin_nanf("") : __builtin_amdgcn_rcpf(D);

    // y = e^(x - M) / D for the chunk held in registers
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] = er.one(f[e]) * r;
            w.store(k, f, same_phase != 0);
        }
    }
}

// (threads, granules per thread per chunk)
#define RWS_SPLITK_FUSED_VARIANTS(X) \
    X(256, 4)                        \
    X(256, 8)                        \
    X(256, 16)

#define RWS_ROW(b, kc) {b, kc},
const SplitkVariant kSplitkFused[] = {RWS_SPLITK_FUSED_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumSplitkFused = sizeof(kSplitkFused) / sizeof(kSplitkFused[0]);

template <int DT, bool AL, int B, int KC>
static const void* kernel_of() {
    return reinterpret_cast<const void*>(&k_splitk_fused<DT, AL, B, KC>);
}

template <int B, int KC>
static const void* kernel_any(int dtype, bool aligned) {
    switch (dtype) {
        case kF32: return aligned ? kernel_of<kF32, true, B, KC>() : kernel_of<kF32, false, B, KC>();
        case kF16: return aligned ? kernel_of<kF16, true, B, KC>() : kernel_of<kF16, false, B, KC>();
        case kBF16: return aligned ? kernel_of<kBF16, true, B, KC>() : kernel_of<kBF16, false, B, KC>();
    }
    return nullptr;
}

static const void* fused_kernel(int variant, int dtype, bool aligned) {
    int i = 0;
#define RWS_CASE(b, kc) \
    if (variant == i) return kernel_any<b, kc>(dtype, aligned); \
    ++i;
    RWS_SPLITK_FUSED_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return nullptr;
}

hipError_t splitk_fused_capacity(int variant, int dtype, bool aligned, int cus, int64_t* blocks) {
    const void* k = fused_kernel(variant, dtype, aligned);
    if (!k) return hipErrorInvalidValue;
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k,
                                                                kSplitkFused[variant].block, 0);
    if (e != hipSuccess) return e;
    *blocks = (int64_t)per_cu * cus;
    return hipSuccess;
}

hipError_t launch_splitk_fused(const Launch& L, int variant, int P, const OrderedSync& S) {
    const void* k = fused_kernel(variant, L.dtype, L.aligned);
    if (!k) return hipErrorInvalidValue;
    const void* in = L.in;
    void* out = L.out;
    int64_t rows = L.rows;
    int cols = L.cols;
    int same_phase = L.same_phase ? 1 : 0;
    OrderedSync sync = S;
    void* args[] = {(void*)&in, (void*)&out, (void*)&rows, (void*)&cols, (void*)&P,
                    (void*)&sync, (void*)&same_phase};
    return hipLaunchCooperativeKernel(k, dim3((unsigned)(L.rows * P)),
                                      dim3(kSplitkFused[variant].block), args, 0, L.stream);
}

}  // namespace rws
