// rws_norm_wave.hip -- instantiations and launcher of norm_wave (LayerNorm
// and RMSNorm with a row per lane group, rws_norm.hpp).
#include "rws_norm.hpp"

namespace rws {

// (lanes per row G, granules per lane K, row sets per wave U).  G*K
// granules of 16 bytes hold the row window.  (16,2) and (8,6) are the
// measured choices for windows of 9-32 and 33-48 granules (the fp16 widths
// 192 and 384); the others are the narrowest group for the other lengths.
#define RWS_NORM_WAVE_VARIANTS(X) \
    X(4, 1, 1)                    \
    X(8, 1, 1)                    \
    X(16, 1, 1)                   \
    X(16, 2, 1)                   \
    X(8, 6, 1)                    \
    X(8, 3, 1)                    \
    X(16, 3, 1)                   \
    X(32, 1, 1)                   \
    X(64, 1, 1)                   \
    X(64, 2, 1)                   \
    X(64, 4, 1)                   \
    X(64, 8, 1)

#define RWS_ROW3(a, b, c) {a, b, c},
const WaveRowVariant kNormWave[] = {RWS_NORM_WAVE_VARIANTS(RWS_ROW3)};
const int kNumNormWave = sizeof(kNormWave) / sizeof(kNormWave[0]);
#undef RWS_ROW3

template <int DT, bool AL, int G, int K, int U, int MODE>
static hipError_t nw_mode(const NormLaunch& L) {
    const WaveRowVariant v = {G, K, U};
    const dim3 grid((unsigned)wave_row_grid(v, L.rows));
    const dim3 block(kWaveGroupThreads);
    if (!L.args.w && !L.args.b)
        hipLaunchKernelGGL((k_norm_wave<DT, AL, G, K, U, MODE, 0>), grid, block, 0, L.stream, L.in,
                           L.out, L.rows, L.cols, L.args, (int)L.same_phase);
    else if constexpr (AL) {
        if (L.aff_matched)
            hipLaunchKernelGGL((k_norm_wave<DT, AL, G, K, U, MODE, 2>), grid, block, 0, L.stream,
                               L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase);
        else
            hipLaunchKernelGGL((k_norm_wave<DT, AL, G, K, U, MODE, 1>), grid, block, 0, L.stream,
                               L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase);
    } else
        hipLaunchKernelGGL((k_norm_wave<DT, AL, G, K, U, MODE, 1>), grid, block, 0, L.stream, L.in,
                           L.out, L.rows, L.cols, L.args, (int)L.same_phase);
    return hipGetLastError();
}

template <int DT, bool AL, int G, int K, int U>
static hipError_t nw(const NormLaunch& L) {
    return L.mode == kLayerNorm ? nw_mode<DT, AL, G, K, U, kLayerNorm>(L)
                                : nw_mode<DT, AL, G, K, U, kRmsNorm>(L);
}

hipError_t launch_norm_wave(const NormLaunch& L, int variant) {
    int i = 0;
#define RWS_CASE(g, k, u)                                                              \
    if (variant == i) {                                                                \
        switch (L.dtype) {                                                             \
            case kF32: return L.aligned ? nw<kF32, true, g, k, u>(L) : nw<kF32, false, g, k, u>(L);    \
            case kF16: return L.aligned ? nw<kF16, true, g, k, u>(L) : nw<kF16, false, g, k, u>(L);    \
            case kBF16: return L.aligned ? nw<kBF16, true, g, k, u>(L) : nw<kBF16, false, g, k, u>(L); \
        }                                                                              \
        return hipErrorInvalidValue;                                                   \
    }                                                                                  \
    ++i;
    RWS_NORM_WAVE_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
