// rws_splitk.hip -- instantiations and launcher of the split-k family
// (stage 1 partial (m, d) per chunk, stage 2 merge + normalise).
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

}  // namespace rws
