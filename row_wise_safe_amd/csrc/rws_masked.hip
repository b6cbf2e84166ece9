// rws_masked.hip -- the masked/scaled forms of wave_row, block_onepass
// (register-held rows) and two_pass: the same kernels with the
// attention-score prologue z = scale*x + mask (+ causal limit) applied right
// after each granule is widened (rws_pre.hpp).
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_variants.hpp"

namespace rws {

template <int DT, bool PAIR = true>
static MaskPre<DT, PAIR> make_pre(const MaskArgs& M, int cols) {
    MaskPre<DT, PAIR> p;
    p.scale = M.scale;
    p.mask = (const char*)M.mask;
    p.mask_rows = M.mask_rows > 0 ? M.mask_rows : 1;
    const int64_t rowbytes = (int64_t)cols * Elem<DT>::SIZE;
    p.edge_lo = (32 + rowbytes - 1) / rowbytes;
    p.edge_hi = (p.mask_rows * rowbytes - 32) / rowbytes - 1;  // below edge_lo: no such row
    p.causal_q = M.causal_q;
    p.row_base = M.row_base;
    p.mask_M = remainder_magic((uint64_t)p.mask_rows);
    p.causal_M = p.causal_q > 0 ? remainder_magic((uint64_t)p.causal_q) : 0;
    return p;
}

// ---- wave_row ------------------------------------------------------------
template <int DT, bool AL, int G, int K, int U>
static hipError_t wr(const Launch& L, const MaskArgs& M) {
    const WaveRowVariant v = {G, K, U};
    hipLaunchKernelGGL((k_wave_row<DT, AL, G, K, U, MaskPre<DT>>),
                       dim3((unsigned)wave_row_grid(v, L.rows)), dim3(kWaveGroupThreads), 0, L.stream, L.in,
                       L.out, L.rows, L.cols, (int)L.same_phase, (int)L.wt, make_pre<DT>(M, L.cols));
    return hipGetLastError();
}

template <int G, int K, int U>
static hipError_t wr_any(const Launch& L, const MaskArgs& M) {
    switch (L.dtype) {
        case kF32: return L.aligned ? wr<kF32, true, G, K, U>(L, M) : wr<kF32, false, G, K, U>(L, M);
        case kF16: return L.aligned ? wr<kF16, true, G, K, U>(L, M) : wr<kF16, false, G, K, U>(L, M);
        case kBF16: return L.aligned ? wr<kBF16, true, G, K, U>(L, M) : wr<kBF16, false, G, K, U>(L, M);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_wave_row_masked(const Launch& L, int variant, const MaskArgs& M) {
    int i = 0;
#define RWS_CASE(g, k, u) \
    if (variant == i) return wr_any<g, k, u>(L, M); \
    ++i;
    RWS_WAVE_ROW_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

// ---- block_onepass (variants without LDS parking) --------------------------
template <int DT, bool AL, int B, int KR>
static hipError_t bo(const Launch& L, const MaskArgs& M) {
    constexpr bool kPair = B < 1024;
    hipLaunchKernelGGL((k_block_onepass<DT, AL, B, KR, 0, MaskPre<DT, kPair>>), dim3((unsigned)L.rows),
                       dim3(B), 0, L.stream, L.in, L.out, L.rows, L.cols, (int)L.same_phase, L.lgrun,
                       make_pre<DT, kPair>(M, L.cols));
    return hipGetLastError();
}

template <int B, int KR, int KL>
static hipError_t bo_any(const Launch& L, const MaskArgs& M) {
    if constexpr (KL != 0) {
        return hipErrorInvalidValue;
    } else {
        switch (L.dtype) {
            case kF32: return L.aligned ? bo<kF32, true, B, KR>(L, M) : bo<kF32, false, B, KR>(L, M);
            case kF16: return L.aligned ? bo<kF16, true, B, KR>(L, M) : bo<kF16, false, B, KR>(L, M);
            case kBF16: return L.aligned ? bo<kBF16, true, B, KR>(L, M) : bo<kBF16, false, B, KR>(L, M);
        }
        return hipErrorInvalidValue;
    }
}

hipError_t launch_block_onepass_masked(const Launch& L, int variant, const MaskArgs& M) {
    int i = 0;
#define RWS_CASE(b, kr, kl) \
    if (variant == i) return bo_any<b, kr, kl>(L, M); \
    ++i;
    RWS_ONEPASS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

// ---- two_pass ----------------------------------------------------------------
template <int DT, bool AL, int B, int U>
static hipError_t tp(const Launch& L, const MaskArgs& M) {
    constexpr bool kPair = B < 1024;
    hipLaunchKernelGGL((k_two_pass<DT, AL, B, U, MaskPre<DT, kPair>>), dim3((unsigned)L.rows), dim3(B), 0,
                       L.stream, L.in, L.out, L.rows, L.cols, (int)L.same_phase, L.lgrun,
                       make_pre<DT, kPair>(M, L.cols));
    return hipGetLastError();
}

template <int B, int U>
static hipError_t tp_any(const Launch& L, const MaskArgs& M) {
    switch (L.dtype) {
        case kF32: return L.aligned ? tp<kF32, true, B, U>(L, M) : tp<kF32, false, B, U>(L, M);
        case kF16: return L.aligned ? tp<kF16, true, B, U>(L, M) : tp<kF16, false, B, U>(L, M);
        case kBF16: return L.aligned ? tp<kBF16, true, B, U>(L, M) : tp<kBF16, false, B, U>(L, M);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_two_pass_masked(const Launch& L, int variant, const MaskArgs& M) {
    int i = 0;
#define RWS_CASE(b, u) \
    if (variant == i) return tp_any<b, u>(L, M); \
    ++i;
    RWS_TWO_PASS_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
