// rws_norm_block.hip -- instantiations and launchers of norm_block and
// norm_stream (LayerNorm and RMSNorm with a workgroup per row, rws_norm.hpp).
#include "rws_norm.hpp"

namespace rws {

// (threads, register granules per thread): the forward block_onepass shapes
// without LDS parking, and 64x2, chosen by the same rule.  A sweep of
// LayerNorm and RMSNorm over fp16 hidden sizes 768-8192 (64 MiB in, rows
// line-aligned) found the exact-fit two-granule shapes fastest at every size
// (768: 64x2 23.2 us, 1024: 64x2 23.2, 2048: 128x2 23.0, 3072: 192x2 23.1,
// 4096: 256x2 23.0, 5120: 320x2 23.5, 8192: 512x2 23.1; one granule per
// thread 24.7-173 us, one wave per row 23.1-52.6 us).
#define RWS_NORM_BLOCK_VARIANTS(X)                                       \
    X(128, 1) X(192, 1) X(256, 1) X(320, 1) X(384, 1) X(512, 1) X(640, 1) \
    X(768, 1) X(1024, 1)                                                  \
    X(64, 2) X(128, 2) X(192, 2) X(256, 2) X(320, 2) X(384, 2) X(512, 2)  \
    X(768, 2)                                                             \
    X(1024, 2)                                                            \
    X(64, 3) X(192, 3) X(384, 3) X(1024, 3) X(1024, 4) X(64, 5)
// (threads, granules per thread per batch)
#define RWS_NORM_STREAM_VARIANTS(X) \
    X(256, 4)                       \
    X(1024, 4)

#define RWS_ROW2(a, b) {a, b},
const TwoPassVariant kNormBlock[] = {RWS_NORM_BLOCK_VARIANTS(RWS_ROW2)};
const int kNumNormBlock = sizeof(kNormBlock) / sizeof(kNormBlock[0]);
const TwoPassVariant kNormStream[] = {RWS_NORM_STREAM_VARIANTS(RWS_ROW2)};
const int kNumNormStream = sizeof(kNormStream) / sizeof(kNormStream[0]);
#undef RWS_ROW2

template <int DT, bool AL, int BL, int KR, int MODE>
static hipError_t nb_mode(const NormLaunch& L) {
    const dim3 grid((unsigned)L.rows);
    if (!L.args.w && !L.args.b)
        hipLaunchKernelGGL((k_norm_block<DT, AL, BL, KR, MODE, 0>), grid, dim3(BL), 0, L.stream,
                           L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase, L.lgrun);
    else if constexpr (AL) {
        if (L.aff_matched)
            hipLaunchKernelGGL((k_norm_block<DT, AL, BL, KR, MODE, 2>), grid, dim3(BL), 0,
                               L.stream, L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase,
                               L.lgrun);
        else
            hipLaunchKernelGGL((k_norm_block<DT, AL, BL, KR, MODE, 1>), grid, dim3(BL), 0,
                               L.stream, L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase,
                               L.lgrun);
    } else
        hipLaunchKernelGGL((k_norm_block<DT, AL, BL, KR, MODE, 1>), grid, dim3(BL), 0, L.stream,
                           L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase, L.lgrun);
    return hipGetLastError();
}

template <int DT, bool AL, int BL, int KR>
static hipError_t nb(const NormLaunch& L) {
    return L.mode == kLayerNorm ? nb_mode<DT, AL, BL, KR, kLayerNorm>(L)
                                : nb_mode<DT, AL, BL, KR, kRmsNorm>(L);
}

template <int DT, bool AL, int BL, int U, int MODE>
static hipError_t ns_mode(const NormLaunch& L) {
    const dim3 grid((unsigned)L.rows);
    if (L.args.w || L.args.b)
        hipLaunchKernelGGL((k_norm_stream<DT, AL, BL, U, MODE, true>), grid, dim3(BL), 0, L.stream,
                           L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase, L.lgrun);
    else
        hipLaunchKernelGGL((k_norm_stream<DT, AL, BL, U, MODE, false>), grid, dim3(BL), 0, L.stream,
                           L.in, L.out, L.rows, L.cols, L.args, (int)L.same_phase, L.lgrun);
    return hipGetLastError();
}

template <int DT, bool AL, int BL, int U>
static hipError_t ns(const NormLaunch& L) {
    return L.mode == kLayerNorm ? ns_mode<DT, AL, BL, U, kLayerNorm>(L)
                                : ns_mode<DT, AL, BL, U, kRmsNorm>(L);
}

template <int DT, bool AL, int MODE, bool AFF>
static hipError_t no(const NormLaunch& L, int P, const OrderedSync& S) {
    hipLaunchKernelGGL((k_norm_ordered<DT, AL, kNormOrderedBlock, kNormOrderedKc, MODE, AFF>),
                       dim3((unsigned)(2 * L.rows * P)), dim3(kNormOrderedBlock), 0, L.stream, L.in,
                       L.out, L.rows, L.cols, L.args, P, S, (int)L.same_phase);
    return hipGetLastError();
}

template <int DT, bool AL>
static hipError_t no_dt(const NormLaunch& L, int P, const OrderedSync& S) {
    const bool aff = L.args.w || L.args.b;
    if (L.mode == kLayerNorm)
        return aff ? no<DT, AL, kLayerNorm, true>(L, P, S) : no<DT, AL, kLayerNorm, false>(L, P, S);
    return aff ? no<DT, AL, kRmsNorm, true>(L, P, S) : no<DT, AL, kRmsNorm, false>(L, P, S);
}

hipError_t launch_norm_ordered(const NormLaunch& L, int P, const OrderedSync& S) {
    switch (L.dtype) {
        case kF32: return L.aligned ? no_dt<kF32, true>(L, P, S) : no_dt<kF32, false>(L, P, S);
        case kF16: return L.aligned ? no_dt<kF16, true>(L, P, S) : no_dt<kF16, false>(L, P, S);
        case kBF16: return L.aligned ? no_dt<kBF16, true>(L, P, S) : no_dt<kBF16, false>(L, P, S);
    }
    return hipErrorInvalidValue;
}

#define RWS_NORM_DT_SWITCH(FN, A, B)                                                      \
    switch (L.dtype) {                                                                    \
        case kF32: return L.aligned ? FN<kF32, true, A, B>(L) : FN<kF32, false, A, B>(L);    \
        case kF16: return L.aligned ? FN<kF16, true, A, B>(L) : FN<kF16, false, A, B>(L);    \
        case kBF16: return L.aligned ? FN<kBF16, true, A, B>(L) : FN<kBF16, false, A, B>(L); \
    }                                                                                     \
    return hipErrorInvalidValue;

hipError_t launch_norm_block(const NormLaunch& L, int family, int variant) {
    int i = 0;
    if (family == 2) {
#define RWS_CASE(b, kr)                     \
    if (variant == i) {                     \
        RWS_NORM_DT_SWITCH(nb, b, kr)       \
    }                                       \
    ++i;
        RWS_NORM_BLOCK_VARIANTS(RWS_CASE)
#undef RWS_CASE
    } else if (family == 3) {
#define RWS_CASE(b, u)                      \
    if (variant == i) {                     \
        RWS_NORM_DT_SWITCH(ns, b, u)        \
    }                                       \
    ++i;
        RWS_NORM_STREAM_VARIANTS(RWS_CASE)
#undef RWS_CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace rws
