// rws_reference.hip -- the bandwidth references of the roofline: a 16-byte
// copy (the ceiling of a read + write stream and the calibration of the
// traffic counters), and the same kernel shape reading only and writing
// only.  The copy takes one one-wave workgroup per 1 KiB, one 16-byte
// granule per lane: among the copy forms measured on MI355X (256-thread
// workgroups, two granules per lane, persistent grid-stride loops, direct
// global-to-LDS loads) it is the fastest at every size from 16 to 256 MiB.
#include "rws_device.hpp"
#include "rws_launch.hpp"

#include <algorithm>

namespace rws {

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

// Read-only and write-only references: one 256-thread workgroup per 16 KiB,
// four 16-byte granules per thread (each load or store instruction of a wave
// covers 1 KiB).  One granule per one-wave workgroup, the copy's shape, is
// bound by workgroup dispatch when a kernel only loads or only stores
// (64 MiB in 15.2 us either way on MI355X, against 10.7 us for this read
// shape).  The read keeps its loads alive with an empty asm statement (no
// instruction, no store); the write stores a pattern of the granule index.
constexpr int kRefGranules = 4;

__global__ __launch_bounds__(256) void k_read16(const u32x4* __restrict__ in, int64_t n) {
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kRefGranules) + threadIdx.x;
    u32x4 v[kRefGranules];
#pragma unroll
    for (int u = 0; u < kRefGranules; ++u) {
        const int64_t i = i0 + 256 * u;
        v[u] = i < n ? __builtin_nontemporal_load(in + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kRefGranules; ++u) asm volatile("" : : "v"(v[u]));
}

template <bool WT>
__global__ __launch_bounds__(256) void k_write16(u32x4* __restrict__ out, int64_t n) {
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kRefGranules) + threadIdx.x;
#pragma unroll
    for (int u = 0; u < kRefGranules; ++u) {
        const int64_t i = i0 + 256 * u;
        if (i >= n) break;
        const u32x4 v = {(unsigned)i, (unsigned)(i >> 32), 0x5a5a5a5au, ~(unsigned)i};
        if (WT)
            store16_wt((char*)(out + i), v);
        else
            __builtin_nontemporal_store(v, out + i);
    }
}

hipError_t launch_read16(const void* in, int64_t n16, hipStream_t stream) {
    for (int64_t done = 0; done < n16;) {
        const int64_t n = std::min<int64_t>(n16 - done, (int64_t)1 << 31);
        hipLaunchKernelGGL(k_read16, dim3((unsigned)((n + 1023) / 1024)), dim3(256), 0, stream,
                           (const u32x4*)in + done, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += n;
    }
    return hipSuccess;
}

hipError_t launch_write16(void* out, int64_t n16, hipStream_t stream) {
    const bool wt = (uintptr_t)out % 128 == 0;
    for (int64_t done = 0; done < n16;) {
        const int64_t n = std::min<int64_t>(n16 - done, (int64_t)1 << 31);
        const dim3 grid((unsigned)((n + 1023) / 1024));
        if (wt)
            hipLaunchKernelGGL(k_write16<true>, grid, dim3(256), 0, stream, (u32x4*)out + done, n);
        else
            hipLaunchKernelGGL(k_write16<false>, grid, dim3(256), 0, stream, (u32x4*)out + done, n);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        done += n;
    }
    return hipSuccess;
}

}  // namespace rws
