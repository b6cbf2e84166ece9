// rws_two_pass.hip -- instantiations and launcher of the two_pass family
// (one workgroup per row, any row length, the row is read twice).
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_variants.hpp"

namespace rws {

#define RWS_ROW(b, u) {b, u},
const TwoPassVariant kTwoPass[] = {RWS_TWO_PASS_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumTwoPass = sizeof(kTwoPass) / sizeof(kTwoPass[0]);

template <int DT, bool AL, int B, int U>
static hipError_t go(const Launch& L) {
    hipLaunchKernelGGL((k_two_pass<DT, AL, B, U>), dim3((unsigned)L.rows), dim3(B), 0, L.stream,
                       L.in, L.out, L.rows, L.cols, (int)L.same_phase, L.lgrun, NoPre());
    return hipGetLastError();
}

template <int B, int U>
static hipError_t go_any(const Launch& L) {
    switch (L.dtype) {
        case kF32: return L.aligned ? go<kF32, true, B, U>(L) : go<kF32, false, B, U>(L);
        case kF16: return L.aligned ? go<kF16, true, B, U>(L) : go<kF16, false, B, U>(L);
        case kBF16: return L.aligned ? go<kBF16, true, B, U>(L) : go<kBF16, false, B, U>(L);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_two_pass(const Launch& L, int variant) {
    int i = 0;
#define RWS_CASE(b, u) \
    if (variant == i) return go_any<b, u>(L); \
    ++i;
    RWS_TWO_PASS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
