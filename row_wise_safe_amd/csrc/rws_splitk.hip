// rws_splitk.hip -- instantiations and launcher of the split-k family
// (stage 1 partial (m, d) per chunk, stage 2 merge + normalise), plus the
// 16-byte copy kernel used as the bandwidth reference.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_variants.hpp"

#include <algorithm>

namespace rws {

#define RWS_ROW(b, kc) {b, kc},
const SplitkVariant kSplitk[] = {RWS_SPLITK_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumSplitk = sizeof(kSplitk) / sizeof(kSplitk[0]);

template <int DT, bool AL, int B, int KC>
static hipError_t go(const Launch& L, int P, float2* ws) {
    const dim3 grid((unsigned)(L.rows * P));
    hipLaunchKernelGGL((k_splitk_stage1<DT, AL, B, KC>), grid, dim3(B), 0, L.stream, L.in, L.rows,
                       L.cols, P, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_splitk_stage2<DT, AL, B, KC>), grid, dim3(B), 0, L.stream, L.in, L.out,
                       L.rows, L.cols, P, (const float2*)ws, (int)L.same_phase);
    return hipGetLastError();
}

template <int B, int KC>
static hipError_t go_any(const Launch& L, int P, float2* ws) {
    switch (L.dtype) {
        case kF32: return L.aligned ? go<kF32, true, B, KC>(L, P, ws) : go<kF32, false, B, KC>(L, P, ws);
        case kF16: return L.aligned ? go<kF16, true, B, KC>(L, P, ws) : go<kF16, false, B, KC>(L, P, ws);
        case kBF16: return L.aligned ? go<kBF16, true, B, KC>(L, P, ws) : go<kBF16, false, B, KC>(L, P, ws);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_splitk(const Launch& L, int variant, int P, float2* ws) {
    int i = 0;
#define RWS_CASE(b, kc) \
    if (variant == i) return go_any<b, kc>(L, P, ws); \
    ++i;
    RWS_SPLITK_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

// ===========================================================================
// Plain 16-byte copy (the copy ceiling and the calibration of the traffic
// counters): one granule per thread, non-temporal loads, one-wave
// workgroups -- like the wave_row kernels -- and, when the output starts on a
// 128-byte line, write-through stores (store16_wt).  The fastest copy of
// HBM-resident data measured on MI355X: 64 MiB in 21.1 us (21.7 us with
// plain non-temporal stores, 23.1 us with cached loads and four-wave
// workgroups).
// ===========================================================================
template <bool WT>
__global__ __launch_bounds__(64) void k_copy16(const u32x4* __restrict__ in,
                                               u32x4* __restrict__ out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
    if (i >= n) return;
    const u32x4 v = __builtin_nontemporal_load(in + i);
    if (WT)
        store16_wt((char*)(out + i), v);
    else
        __builtin_nontemporal_store(v, out + i);
}

hipError_t launch_copy16(const void* in, void* out, int64_t n16, hipStream_t stream) {
    const bool wt = (uintptr_t)out % 128 == 0;
    for (int64_t done = 0; done < n16;) {
        // at most 2^25 one-wave workgroups per launch
        const int64_t n = std::min<int64_t>(n16 - done, (int64_t)1 << 31);
        const dim3 grid((unsigned)((n + 63) / 64));
        if (wt)
            hipLaunchKernelGGL(k_copy16<true>, grid, dim3(64), 0, stream,
                               (const u32x4*)in + done, (u32x4*)out + done, n);
        else
            hipLaunchKernelGGL(k_copy16<false>, grid, dim3(64), 0, stream,
                               (const u32x4*)in + done, (u32x4*)out + done, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += n;
    }
    return hipSuccess;
}

}  // namespace rws
