// rws_ordered.hpp -- the exchange of the single-launch ("ordered") split-k
// kernels: stage-1 workgroups publish a chunk's partial as epoch-tagged
// 64-bit words, stage-2 workgroups of the same row poll them (see
// rws_splitk_ordered.hip for why this needs no fence and no co-residency).
// Shared by the softmax forward, the softmax backward and the row
// normalisations.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rws_launch.hpp"

namespace rws {

// The launch's epoch: the kernel argument, or the device word at `src`
// (launches recorded in a graph, see kDeviceEpochFirst).
__device__ inline unsigned launch_epoch(unsigned epoch, const uint64_t* src) {
    return src ? (unsigned)__hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
               : epoch;
}

__device__ inline uint64_t tag_word(unsigned epoch, float v) {
    return ((uint64_t)epoch << 32) | (uint64_t)__float_as_uint(v);
}

__device__ inline void publish_word(uint64_t* p, unsigned epoch, float v) {
    __hip_atomic_store(p, tag_word(epoch, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Poll one tagged word until it carries `epoch`; returns its value bits and
// sets `late` when `limit` tries ran out (a thread that is already late tries
// once more at most, so one thread waits at most one limit in total; a limit
// of 0 gives up without reading).
__device__ inline float poll_word(const uint64_t* p, unsigned epoch, int& late, unsigned limit) {
    const unsigned tries = late ? (limit ? 1u : 0u) : limit;
    for (unsigned it = 0; it < tries; ++it) {
        const uint64_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(v >> 32) == epoch) return __uint_as_float((unsigned)v);
        __builtin_amdgcn_s_sleep(2);
    }
    late = 1;
    return 0.0f;
}

// A workgroup whose wait gave up (its outputs are NaN) records it in the
// stream's status word; one thread per workgroup calls this.
__device__ inline void report_late(uint64_t* status) {
    if (status)
        __hip_atomic_fetch_or(status, kStatusLate, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Workgroup b of an ordered launch over rows x P chunks: [0, rows*P) are
// stage 1, [rows*P, 2*rows*P) stage 2, row-major within each stage.
struct OrderedSlot {
    bool merge_stage;
    int64_t row;
    int chunk;
};

__device__ inline OrderedSlot ordered_slot(int64_t b, int64_t rows, int P) {
    OrderedSlot s;
    const int64_t RP = rows * P;
    s.merge_stage = b >= RP;
    if (s.merge_stage) b -= RP;
    s.row = b / P;
    s.chunk = (int)(b - s.row * P);
    return s;
}

}  // namespace rws
