// rws_splitk_fused.hip -- split-k in a single ordinary launch that reads
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
// Waiting needs only the row's own workgroups at once, not the grid's.
// Workgroups b = row * P + chunk are handed to each XCD in increasing index
// order (the ordered form's assumption).  Take the lowest row that has not
// finished: every earlier row has finished and left its slots, and on each
// XCD no workgroup of a later row is dispatched before all of this row's
// workgroups for that XCD are, so this row's P workgroups become resident
// together provided P workgroups fit on the device -- and it finishes.  The
// dispatcher therefore checks P against the co-resident capacity of the
// variant (and, for its own choice, takes this form only when the whole grid
// fits, measured fastest).  A launch through hipLaunchCooperativeKernel,
// which guarantees the whole grid instead, cost ~17 us more per call on
// MI355X (fp16 [16,1M]: 32.9 us against 14.3-14.5).  The wait is also
// bounded: a workgroup that does not see a partial after the launch's spin
// limit stops waiting, writes NaN for its chunk and sets the stream's status
// word (softmax_stream_status reports it), so every wave always reaches the
// end of the kernel.
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

// Waves per SIMD each kernel is compiled to allow: KC 4 at 8 (<= 64 VGPRs),
// KC 8 at 4, KC 16 at 4 on line-aligned rows and 2 on the others, whose
// element-wise row ends need more registers; fp32 rows that are not
// line-aligned at 6 / 3 / 1, where the others would spill (42-236 VGPRs
// without spills; 6-14 spilled otherwise).  KC 16 at four waves per SIMD
// keeps 64 MiB of chunks resident on 256 CUs: inputs up to that size run in
// one pass of the grid.
template <int DT, bool ALIGNED, int KC>
constexpr int fused_min_waves() {
    return (DT == kF32 && !ALIGNED) ? (KC <= 4 ? 6 : KC <= 8 ? 3 : 1)
                                    : (KC <= 4 ? 8 : KC <= 8 ? 4 : ALIGNED ? 4 : 2);
}

template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK, (fused_min_waves<DT, ALIGNED, KC>())) void k_splitk_fused(const void* __restrict__ in,
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

    // chunk max, chunk sum of e^(x - m_c).  Each pass takes the granules
    // one at a time: the empty asm statements tie granule i to the running
    // result of granules < i, so the compiler cannot widen (and hold) all KC
    // granules' fp32 values at once -- KC 16 then fits 119 VGPRs instead of
    // 237.  (An empty asm statement: no instruction.)
    float mc = granule_max<DT>(raw[0]);
#pragma unroll
    for (int i = 1; i < KC; ++i) {
        asm volatile("" : "+v"(raw[i]) : "v"(mc));
        mc = vmax(mc, granule_max<DT>(raw[i]));
    }
    mc = block_reduce<W, OpMax>(mc, red_max);
    float dc = 0.0f;
    {
        const RowExp er(mc);
#pragma unroll
        for (int i = 0; i < KC; ++i) {
            asm volatile("" : "+v"(raw[i]) : "v"(dc));
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

    // One thread first waits for the row's last chunk, dispatched last and
    // so as a rule published last; the other threads wait at the barrier.
    // Only then do all threads poll their share of the row's partials (by
    // then mostly published).  Every thread polling all along multiplied the
    // agent-scope loads during the long read phase: fp16 [4,8M] 29.3 us
    // against 25.3 with this wait.  (Its result is not needed: the polls
    // below check every word, bounded as always.)
    if (t == 0) {
        int ignored = 0;
        (void)poll_word(row_tags + 2 * (P - 1) + 1, epoch, ignored, S.spin_limit);
    }
    __syncthreads();

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

    // y = e^(x - M) / D for the chunk held in registers, again one granule
    // at a time (tied to the previous granule's first output)
    float tok = r;
#pragma unroll
    for (int i = 0; i < KC; ++i) {
        const int k = kbase + BLOCK * i;
        asm volatile("" : "+v"(raw[i]) : "v"(tok));
        if (k < w.ngran) {
            float f[VEC];
            Elem<DT>::widen(raw[i], f);
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] = er.one(f[e]) * r;
            w.store(k, f, same_phase != 0);
            tok = f[0];
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

template <int KC>
static int min_waves_any(int dtype, bool aligned) {
    switch (dtype) {
        case kF32: return aligned ? fused_min_waves<kF32, true, KC>() : fused_min_waves<kF32, false, KC>();
        case kF16: return aligned ? fused_min_waves<kF16, true, KC>() : fused_min_waves<kF16, false, KC>();
        case kBF16: return aligned ? fused_min_waves<kBF16, true, KC>() : fused_min_waves<kBF16, false, KC>();
    }
    return 0;
}

int splitk_fused_min_waves(int variant, int dtype, bool aligned) {
    int i = 0;
#define RWS_CASE(b, kc) \
    if (variant == i) return min_waves_any<kc>(dtype, aligned); \
    ++i;
    RWS_SPLITK_FUSED_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return 0;
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

template <int DT, bool AL, int B, int KC>
static hipError_t go(const Launch& L, int P, const OrderedSync& S) {
    hipLaunchKernelGGL((k_splitk_fused<DT, AL, B, KC>), dim3((unsigned)(L.rows * P)), dim3(B), 0,
                       L.stream, L.in, L.out, L.rows, L.cols, P, S, (int)L.same_phase);
    return hipGetLastError();
}

template <int B, int KC>
static hipError_t go_any(const Launch& L, int P, const OrderedSync& S) {
    switch (L.dtype) {
        case kF32: return L.aligned ? go<kF32, true, B, KC>(L, P, S) : go<kF32, false, B, KC>(L, P, S);
        case kF16: return L.aligned ? go<kF16, true, B, KC>(L, P, S) : go<kF16, false, B, KC>(L, P, S);
        case kBF16: return L.aligned ? go<kBF16, true, B, KC>(L, P, S) : go<kBF16, false, B, KC>(L, P, S);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_splitk_fused(const Launch& L, int variant, int P, const OrderedSync& S) {
    int i = 0;
#define RWS_CASE(b, kc) \
    if (variant == i) return go_any<b, kc>(L, P, S); \
    ++i;
    RWS_SPLITK_FUSED_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
