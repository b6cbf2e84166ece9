// rws_splitk_fused.hip -- split-k in a single cooperative launch.
//
// The two-launch split-k (rws_splitk.hip) reads every chunk twice: stage 1
// for the chunk's partial (m, d), stage 2 again to write the outputs once the
// row's partials are merged.  Here every workgroup keeps its chunk in
// registers between the two halves: it publishes its partial, arrives on a
// per-row counter and waits until the row's last workgroup has arrived; then
// it merges the row's partials and writes its chunk from registers -- one
// read and one write per element.  The CUDA safe-online-softmax page names
// this single-kernel form (a grid-wide sync, or atomics with polling) in
// section 3.2 and leaves it unbuilt; the (m, d) merge is the same rule.
//
// Waiting across workgroups is only safe when all of them are resident at
// once, so the kernel is launched with hipLaunchCooperativeKernel, which
// refuses grids that cannot be co-resident (the dispatcher then uses the
// two-launch form).  The wait is also bounded: a workgroup that does not see
// its row released after kSpinLimit polls stops waiting, so every wave
// always reaches the end of the kernel; it then writes NaN for its chunk and
// sets the stream's status word (softmax_stream_status reports it).
//
// Synchronisation words (per row, in a library-owned zero-initialised
// buffer, one 256-byte line per row so that rows do not contend): count
// (arrivals of the current call; reset to 0 by the last arrival) and flag (the
// epoch of the last released call).  The host passes a per-buffer epoch that
// grows by one per call, so a flag from an earlier call never matches.
//
// Cost on MI355X: the agent-scope release (each arrival) and acquire (each
// waiter) write back and invalidate the XCD's L2, which measured about
// 34 us for fp16 [16, 1M] against 15 us for the two-launch split-k, so the
// dispatcher does not pick this family; it is available by request.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"

namespace rws {

constexpr unsigned kSpinLimit = 1u << 20;  // polls of ~500 cycles: ~0.2 s

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
                                                        int cols, int P, float2* __restrict__ ws,
                                                        unsigned* __restrict__ sync,
                                                        unsigned epoch, uint64_t* status,
                                                        int same_phase) {
    constexpr int VEC = Elem<DT>::VEC;
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    __shared__ float red_max2[W];
    __shared__ float red_sum2[W];
    __shared__ int timed_out;
    const int t = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int64_t row = b / P;
    const int chunk = (int)(b - row * P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const int kbase = chunk * (BLOCK * KC) + t;

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

    // publish the partial, arrive, wait for the row's release
    if (t == 0) {
        timed_out = 0;
        ws[row * P + chunk] = make_float2(mc, dc);
        unsigned* count = sync + kSyncWordsPerRow * row;
        unsigned* flag = count + 1;
        const unsigned old =
            __hip_atomic_fetch_add(count, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (old == (unsigned)(P - 1)) {
            __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(flag, epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            // Poll with relaxed loads (an acquire per poll would invalidate
            // the L2 every iteration); one acquire fence follows the wait.
            unsigned it = 0;
            for (; it < kSpinLimit; ++it) {
                if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == epoch)
                    break;
                __builtin_amdgcn_s_sleep(8);
            }
            if (it == kSpinLimit) {
                timed_out = 1;
                if (status)
                    __hip_atomic_fetch_or(status, kStatusLate, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // Keep only the raw granules live across the wait: without this the
    // compiler would reuse the widened fp32 values of the passes above and
    // hold twice the registers.  (An empty asm statement: no instruction.)
#pragma unroll
    for (int i = 0; i < KC; ++i) asm volatile("" : "+v"(raw[i]));

    // merge the row's partials: (M, D)
    float m = kNegInf, d = 0.0f;
    for (int j = t; j < P; j += BLOCK) {
        const float2 p = ws[row * P + j];
        const float mn = vmax(m, p.x);
        const float a = (d == 0.0f) ? 0.0f : d * merge_scale(m, mn);
        const float bb = (p.y == 0.0f) ? 0.0f : p.y * merge_scale(p.x, mn);
        m = mn;
        d = a + bb;
    }
    float M, D;
    block_merge<W>(m, d, M, D, red_max2, red_sum2);
    const RowExp er(M);
    const float r = timed_out ? __builtin_nanf("") : __builtin_amdgcn_rcpf(D);

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

hipError_t launch_splitk_fused(const Launch& L, int variant, int P, float2* ws, unsigned* sync,
                               unsigned epoch, uint64_t* status) {
    const void* k = fused_kernel(variant, L.dtype, L.aligned);
    if (!k) return hipErrorInvalidValue;
    const void* in = L.in;
    void* out = L.out;
    int64_t rows = L.rows;
    int cols = L.cols;
    int same_phase = L.same_phase ? 1 : 0;
    void* args[] = {(void*)&in, (void*)&out, (void*)&rows, (void*)&cols, (void*)&P,
                    (void*)&ws, (void*)&sync, (void*)&epoch, (void*)&status,
                    (void*)&same_phase};
    return hipLaunchCooperativeKernel(k, dim3((unsigned)(L.rows * P)),
                                      dim3(kSplitkFused[variant].block), args, 0, L.stream);
}

}  // namespace rws
