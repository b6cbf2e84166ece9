// rws_splitk_ordered.hip -- split-k in one ordinary launch.
//
// The grid holds both stages of split-k (CUDA safe-online-softmax page,
// section 3.2): workgroups [0, rows*P) are stage 1 (one chunk's partial
// (m, d) each), workgroups [rows*P, 2*rows*P) are stage 2 (merge the row's P
// partials, re-read the chunk, write it).  The page orders the stages with a
// second launch, and names a single launch with polling as the alternative;
// this is that alternative, built so that it needs neither a grid-wide
// barrier nor any memory fence:
//
//  * No fences.  A partial travels as two 64-bit words, (epoch << 32 | bits
//    of m) and (epoch << 32 | bits of d), stored and polled with relaxed
//    agent-scope atomics.  Coherence of each single word is all the exchange
//    needs: a stage-2 thread waits until both words of a partial carry this
//    launch's epoch, and the words themselves are the data.  (A flag plus
//    separate data would need a release/acquire pair, which on this
//    multi-XCD part writes back and invalidates the XCD's L2 -- about 20 us
//    over the grid, measured.)
//  * No co-residency requirement.  Every stage-2 workgroup waits only for
//    stage-1 workgroups, and every stage-1 workgroup has a lower index than
//    every stage-2 workgroup; workgroups are handed to each XCD in increasing
//    index order, so a waiting stage-2 workgroup is never ahead of a stage-1
//    workgroup it needs, and stage-1 workgroups never wait.
//  * Bounded waiting.  A poll gives up after OrderedSync::spin_limit tries
//    (by default kOrderedSpinLimit, each a sleep plus a load round trip: at
//    least ~0.5 s in all); the workgroup then writes NaN for its chunk and
//    sets the stream's status word, which softmax_stream_status reports, so a
//    broken ordering assumption shows as NaN output and an error status,
//    never as a hang.
//
// The epoch grows by one per launch on the same tag buffer (host side), and
// the buffer is zero-filled when it is allocated and when the host's epoch
// range wraps, so a word from an earlier launch never matches.
//
// Measured on MI355X, fp16 [16, 1M] read from HBM: 14.1 us against 15.2 us
// for the two launches (the stage-2 workgroups start while the last stage-1
// workgroups finish, instead of after a kernel boundary).
#include "rws_kernels.hpp"
#include "rws_launch.hpp"
#include "rws_ordered.hpp"
#include "rws_variants.hpp"

#include <algorithm>

namespace rws {

template <int DT, bool ALIGNED, int BLOCK, int KC>
__global__ __launch_bounds__(BLOCK) void k_splitk_ordered(const void* __restrict__ in,
                                                          void* __restrict__ out, int64_t rows,
                                                          int cols, int P, OrderedSync S,
                                                          int same_phase) {
    constexpr int W = BLOCK / 64;
    __shared__ float red_max[W];
    __shared__ float red_sum[W];
    const int t = threadIdx.x;
    const int64_t RP = rows * P;
    int64_t b = blockIdx.x;
    const bool merge_stage = b >= RP;
    if (merge_stage) b -= RP;
    const int64_t row = b / P;
    const int chunk = (int)(b - row * P);
    const char* tbeg = (const char*)in;
    const char* tend = tensor_end<DT>(in, rows, cols);
    const RowWin<DT, ALIGNED> w(in, out, row, cols);
    const int kbase = chunk * (BLOCK * KC) + t;
    uint64_t* row_tags = S.tags + 2 * row * P;
    const unsigned epoch = launch_epoch(S.epoch, S.epoch_src);

    // Both stages start by loading the chunk; a stage-2 workgroup's loads
    // are then in flight while it waits for the partials.
    u32x4 raw[KC];
    if (merge_stage)
        splitk_fetch<DT, ALIGNED, BLOCK, KC, true>(w, kbase, tbeg, tend, raw);
    else
        splitk_fetch<DT, ALIGNED, BLOCK, KC, false>(w, kbase, tbeg, tend, raw);

    if (!merge_stage) {
        const float2 md =
            splitk_partial<DT, ALIGNED, BLOCK, KC>(w, kbase, raw, tbeg, tend, red_max, red_sum);
        if (t == 0) {
            publish_word(row_tags + 2 * chunk, epoch, md.x);
            publish_word(row_tags + 2 * chunk + 1, epoch, md.y);
        }
        return;
    }

    float m = kNegInf, d = 0.0f;
    int late = 0;
    for (int j = t; j < P; j += BLOCK) {
        const float pm = poll_word(row_tags + 2 * j, epoch, late, S.spin_limit);
        const float pd = poll_word(row_tags + 2 * j + 1, epoch, late, S.spin_limit);
        md_fold(m, d, pm, pd);
    }
    float M, D;
    block_merge<W>(m, d, M, D, red_max, red_sum);
    const bool failed = __syncthreads_or(late) != 0;
    if (failed && t == 0) report_late(S.status);
    const float r = failed ? __builtin_nanf("") : __builtin_amdgcn_rcpf(D);
    splitk_write<DT, ALIGNED, BLOCK, KC>(w, kbase, raw, tbeg, tend, M, r, same_phase != 0);
}

// Zero n 64-bit words (a kernel rather than a memset, so that the clear is an
// ordinary node if a caller captures the stream into a graph).
__global__ __launch_bounds__(256) void k_fill_words(uint64_t* __restrict__ p, int64_t n,
                                                    uint64_t v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

// Advance a tag buffer's device epoch (the word after its n tag words) for
// the next launch on the stream.  When the device range is used up, the
// buffer's words are zeroed first, so no word left from the range's last
// pass can match a new epoch.
__global__ __launch_bounds__(256) void k_bump_epoch(uint64_t* __restrict__ words, int64_t n) {
    const unsigned cur = (unsigned)words[n];
    const bool wrap = cur == 0xffffffffu;
    if (wrap)
        for (int64_t i = threadIdx.x; i < n; i += 256) words[i] = 0;
    __syncthreads();
    if (threadIdx.x == 0)
        words[n] = (cur < kDeviceEpochFirst || wrap) ? kDeviceEpochFirst : cur + 1;
}

hipError_t launch_bump_epoch(uint64_t* words, int64_t n, hipStream_t stream) {
    hipLaunchKernelGGL(k_bump_epoch, dim3(1), dim3(256), 0, stream, words, n);
    return hipGetLastError();
}

hipError_t launch_fill_words(uint64_t* p, int64_t n, uint64_t v, hipStream_t stream) {
    for (int64_t done = 0; done < n;) {
        const int64_t c = std::min<int64_t>(n - done, (int64_t)1 << 31);
        hipLaunchKernelGGL(k_fill_words, dim3((unsigned)((c + 255) / 256)), dim3(256), 0, stream,
                           p + done, c, v);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += c;
    }
    return hipSuccess;
}

template <int DT, bool AL, int B, int KC>
static hipError_t go(const Launch& L, int P, const OrderedSync& S) {
    hipLaunchKernelGGL((k_splitk_ordered<DT, AL, B, KC>), dim3((unsigned)(2 * L.rows * P)),
                       dim3(B), 0, L.stream, L.in, L.out, L.rows, L.cols, P, S,
                       (int)L.same_phase);
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

hipError_t launch_splitk_ordered(const Launch& L, int variant, int P, const OrderedSync& S) {
    int i = 0;
#define RWS_CASE(b, kc) \
    if (variant == i) return go_any<b, kc>(L, P, S); \
    ++i;
    RWS_SPLITK_VARIANTS(RWS_CASE)
#undef RWS_CASE
    return hipErrorInvalidValue;
}

}  // namespace rws
