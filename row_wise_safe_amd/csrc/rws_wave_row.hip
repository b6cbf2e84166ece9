// rws_wave_row.hip -- instantiations and launcher of the wave_row family.
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_variants.hpp"

namespace rws {

#define RWS_ROW(g, k, u) {g, k, u},
const WaveRowVariant kWaveRow[] = {RWS_WAVE_ROW_VARIANTS(RWS_ROW)};
#undef RWS_ROW
const int kNumWaveRow = sizeof(kWaveRow) / sizeof(kWaveRow[0]);

template <int DT, bool AL, int G, int K, int U>
static hipError_t go(const Launch& L) {
    const WaveRowVariant v = {G, K, U};
    const int64_t grid = wave_row_grid(v, L.rows);
    hipLaunchKernelGGL((k_wave_row<DT, AL, G, K, U>), dim3((unsigned)grid), dim3(kWaveGroupThreads), 0,
                       L.stream, L.in, L.out, L.rows, L.cols, (int)L.same_phase, (int)L.wt, NoPre());
    return hipGetLastError();
}

template <int G, int K, int U>
static hipError_t go_any(const Launch& L) {
    switch (L.dtype) {
        case kF32: return L.aligned ? go<kF32, true, G, K, U>(L) : go<kF32, false, G, K, U>(L);
        case kF16: return L.aligned ? go<kF16, true, G, K, U>(L) : go<kF16, false, G, K, U>(L);
        case kBF16: return L.aligned ? go<kBF16, true, G, K, U>(L) : go<kBF16, false, G, K, U>(L);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_wave_row(const Launch& L, int variant) {
    int i = 0;
#define RWS_CASE(g, k, u) \
    if (variant == i) return go_any<g, k, u>(L); \
    ++i;
    RWS_WAVE_ROW_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
