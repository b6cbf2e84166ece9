// rws_block_onepass.hip -- instantiations and launcher of the block_onepass
// family (one workgroup per row, row cached in registers, then LDS).
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_variants.hpp"

namespace rws {

#define RWS_ROW(b, kr, kl) {b, kr, kl},
const OnepassVariant kOnepass[] = {RWS_ONEPASS_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumOnepass = sizeof(kOnepass) / sizeof(kOnepass[0]);

template <int DT, bool AL, int B, int KR, int KL>
static hipError_t go(const Launch& L) {
    if constexpr (KR >= 8 && DT != kF32)
        hipLaunchKernelGGL((k_block_onepass_raw<DT, AL, B, KR, KL>), dim3((unsigned)L.rows), dim3(B),
                           0, L.stream, L.in, L.out, L.rows, L.cols, (int)L.same_phase, L.lgrun);
    else
        hipLaunchKernelGGL((k_block_onepass<DT, AL, B, KR, KL>), dim3((unsigned)L.rows), dim3(B), 0,
                           L.stream, L.in, L.out, L.rows, L.cols, (int)L.same_phase, L.lgrun,
                           NoPre());
    return hipGetLastError();
}

template <int B, int KR, int KL>
static hipError_t go_any(const Launch& L) {
    switch (L.dtype) {
        case kF32: return L.aligned ? go<kF32, true, B, KR, KL>(L) : go<kF32, false, B, KR, KL>(L);
        case kF16: return L.aligned ? go<kF16, true, B, KR, KL>(L) : go<kF16, false, B, KR, KL>(L);
        case kBF16: return L.aligned ? go<kBF16, true, B, KR, KL>(L) : go<kBF16, false, B, KR, KL>(L);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_block_onepass(const Launch& L, int variant) {
    int i = 0;
#define RWS_CASE(b, kr, kl) \
    if (variant == i) return go_any<b, kr, kl>(L); \
    ++i;
    RWS_ONEPASS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
