// rws_api.cpp -- C ABI of the row-wise softmax library: argument checks, the
// cols-and-dtype dispatcher, the split-k workspace cache and error reporting.
// The declarations and their contract are in include/row_wise_softmax.h.
//
// Dispatch (the choice of kernel per shape is the question the CUDA
// safe-online-softmax page leaves open in its summary, section 4.3; the HIP
// tutorial page, section 7, switches by a cols threshold and notes that the
// threshold must be tuned per device):
//   * the row window (16-byte granules covering a row) fits one wave's
//     registers  -> wave_row, with the narrowest lane group that holds it;
//   * few rows of long rows                     -> split-k over many workgroups;
//   * fits a workgroup's registers (+ LDS)      -> block_onepass;
//   * otherwise                                 -> two_pass.
// The thresholds are set from measurements on MI355X.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>
#include <tuple>
#include <mutex>
#include <string>
#include <algorithm>
#include <atomic>
#include <utility>

#include "row_wise_softmax.h"
#include "rws_launch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
    g_last_error = msg;
    return status;
}

int elem_size(int dtype) { return dtype == RWS_F32 ? 4 : 2; }
const char* dtype_name(int dtype) {
    return dtype == RWS_F32 ? "f32" : dtype == RWS_F16 ? "f16" : "bf16";
}

// Longest row the kernels index with 32-bit element offsets.
constexpr int64_t kMaxCols = (int64_t)1 << 30;

struct DeviceInfo {
    int cus = 256;
    bool known = false;
};

DeviceInfo device_info() {
    static std::mutex mu;
    static std::map<int, DeviceInfo> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return DeviceInfo{};
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(dev);
    if (it != cache.end()) return it->second;
    DeviceInfo info;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        cus > 0) {
        info.cus = cus;
        info.known = true;
    } else {
        (void)hipGetLastError();
    }
    cache[dev] = info;
    return info;
}

constexpr int kOrderedMaxP = 512;
constexpr int64_t kOrderedMaxBytes = (int64_t)32 << 20;
constexpr int64_t kFusedFewRows = 4;

bool is_splitk(int family) {
    return family == RWS_KERNEL_SPLITK || family == RWS_KERNEL_SPLITK_FUSED ||
           family == RWS_KERNEL_SPLITK_ORDERED;
}

struct Plan {
    int family = 0;   // RWS_KERNEL_*
    int variant = 0;  // index into that family's variant table
    int P = 1;        // split-k chunks per row
    int64_t max_rows_per_launch = 0;
    int64_t window = 0;  // granules per row window (upper bound)
    bool aligned = false;
    bool same_phase = false;
    bool wt = false;  // write-through 128-bit stores (line-aligned wave_row)
    int lgrun = 0;    // XCD runs of 2^lgrun rows (workgroup-per-row kernels) or tiles
    int tile_t = 0;   // tile_rows: rows per tile
};

// Alignment facts of one call.
struct Geometry {
    int64_t row_bytes;
    bool a16;   // in, out and every row start 16-byte aligned
    bool a128;  // ... 128-byte (cache line) aligned
    bool same_phase;
};

Geometry geometry(int64_t cols, int dtype, const void* in, const void* out) {
    const uintptr_t ai = (uintptr_t)in, ao = (uintptr_t)out;
    Geometry g;
    g.row_bytes = cols * elem_size(dtype);
    g.a16 = ai % 16 == 0 && ao % 16 == 0 && g.row_bytes % 16 == 0;
    g.a128 = ai % 128 == 0 && ao % 128 == 0 && g.row_bytes % 128 == 0;
    g.same_phase = (ai % 16) == (ao % 16);
    return g;
}

// Granules in a row window that starts on a `wa`-byte boundary (an upper
// bound over all rows; exact when the rows are `wa`-aligned).
int64_t window_granules(const Geometry& g, int wa) {
    const bool aligned = wa == 128 ? g.a128 : g.a16;
    if (aligned) return g.row_bytes / 16;
    return (g.row_bytes + wa + 15) / 16;
}

// window alignment of the backward's and the normalisations' lane groups
int wave_row_wa(const rws::WaveRowVariant& v) { return v.G * 16 >= 128 ? 128 : 16; }
// and of the forward's (wave_row, plain and masked)
int softmax_wave_wa(const rws::WaveRowVariant& v) { return rws::softmax_window_align(v.G); }

// The dispatcher's rows for tile_rows: plain softmax over many rows of at
// most kTileMaxRowBytes that are not line-aligned -- with partial granules at
// their ends (byte length not a multiple of 16), or 16-byte multiples above
// 128 bytes -- in and out 16-byte aligned, and a tile of at least 4 rows.
// MI355X, fp16, inputs in HBM, tile_rows against the lane-group form
// (wave_row): [131072,250] 25.3 us vs 34.5, [1000000,33] 27.0 vs 55.0,
// [1048576,100] 74.6 vs 122, [64000,500] 24.9 vs 30.2, fp32 [131072,125]
// 25.0 vs 29.2; 16-byte multiples [262144,120] 25.1 vs 31.5, [131072,248]
// 25.2 vs 29.9, [65536,504] 25.5 vs 29.3, but [524288,56] 24.2 vs 20.2 (one
// granule per lane on 8 lanes, 16-byte windows, holds those rows whole).
// Tiles of eight granules per lane (spilling 374-388 scalar registers) lost
// to the lane groups and block_onepass: [65536,333] 26.2 vs 21.0,
// [32768,1022] 29.2 vs 24.8; the tile shapes stop at four.  Tile heights
// of 4, 8 or 16 rows only (a tile filling half of its slots): [1000000,33]
// 38.8 us, [1048576,100] 83.1.
constexpr int64_t kTileMaxRowBytes = 1024;
constexpr int64_t kTileMinRows = 64;

int pick_tile_rows(int64_t rows, int64_t cols, int es, int forced_variant, int* T_out);

bool tile_rows_fits(int64_t rows, int64_t cols, int dtype, const void* in, const void* out) {
    const int es = elem_size(dtype);
    const int64_t rb = cols * es;
    return rows >= kTileMinRows && rb % 128 != 0 && (rb % 16 != 0 || rb > 128) &&
           rb <= kTileMaxRowBytes && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0 &&
           pick_tile_rows(rows, cols, es, -1, nullptr) >= 0;
}

// Rows per tile with K granules per lane for rows of `cols` elements of size
// es: the largest multiple of P0 = 16 / gcd(row bytes, 16) (tiles of P0 rows
// start on a 16-byte boundary), at most rws::kTileMaxT, whose tile fits 64 K
// granules; 0 when fewer than 4 rows fit.
int tile_rows_per_tile(int64_t cols, int es, int K) {
    const int64_t rb = cols * es;
    if (cols < 16 / es || rb > kTileMaxRowBytes) return 0;
    int g = 16;
    while (rb % g) g /= 2;
    const int p0 = 16 / g;
    int64_t T = std::min<int64_t>(rws::kTileMaxT, 64LL * K * 16 / rb);
    T -= T % p0;
    return T >= 4 ? (int)T : 0;
}

// tile_rows: the variant (granules per lane K) for `rows` rows of `cols`
// elements of size es, or -1; its rows per tile in *T_out.  Every slot costs
// the same instructions whether the tile fills it or not, so the cost of a K
// is its slots per row, 64 K / T, weighted by what a K costs besides.  Up to
// kTileSmallBytes per direction the larger K cost more: more registers per
// lane (K = 4: 95 VGPRs, 5 waves per SIMD, against 8 at K = 2) and longer
// waves, so a longer tail in a launch of a few rounds of waves; at K = 1 the
// two row reductions work on one granule per lane.  Weights from sweeps of
// every feasible K on MI355X (fp16 unless noted, 63-66 MB per direction, us
// per call for K = 1/2/3/4, fill in parentheses): [262144,120] 26.6 / 23.9
// / 24.1 / 24.6 (0.94 / 0.94 / 0.94 / 1.00); [524288,60] 26.6 / 24.0 / 24.0
// / 24.8 (same fills); [1000000,33] 44.1 / 28.7 / 26.7 / 25.9 (0.52 / 0.77
// / 0.86 / 0.90); [425000,77] - / 32.9 / 26.7 / 26.2 (- / 0.60 / 0.80 /
// 0.90); [727000,45] 33.8 / 29.5 / 25.0 / 26.5 (0.70 / 0.70 / 0.94 / 0.88);
// [131072,250] - / 24.4 / 29.1 / 24.6 (- / 0.98 / 0.65 / 0.98); fp32
// [131072,125] - / 23.3 / 23.6 / 24.7 (- / 0.98 / 0.65 / 0.98); backward
// [262144,120] 31.1 us (K = 2) against 33.2 (K = 4), RMSNorm 21.8 against
// 24.8.  Larger launches run many rounds of waves and K = 4 leads at equal
// fill: [1048576,100] 75.1 (K = 2) against 73.4 (K = 4), [1048576,120] 88.0
// against 86.8, [524288,250] 89.7 against 87.1, backward [1048576,100]
// 103.1 against 100.7, LayerNorm 75.1 against 71.9; there only K = 1 carries
// a weight and the larger tile wins at equal cost.  In between the two are
// within 2 % either way ([393216,120] 34.9 against 35.6, [524288,120] 45.7
// both, [196608,250] 36.0 against 35.3, [262144,250] 46.5 against 45.8,
// [786432,100] 57.3 against 56.1), so the threshold is a round size there.
// forced_variant >= 0 asks for that K.
constexpr int64_t kTileSmallBytes = (int64_t)1 << 27;

int pick_tile_rows(int64_t rows, int64_t cols, int es, int forced_variant, int* T_out) {
    static constexpr int kWeightSmall[5] = {0, 130, 100, 102, 107};  // percent, by K
    static constexpr int kWeightLarge[5] = {0, 130, 100, 100, 100};
    const bool small = rows * cols * es <= kTileSmallBytes;
    const int* w = small ? kWeightSmall : kWeightLarge;
    int best = -1, best_t = 0;
    for (int i = 0; i < rws::kNumTileRows; ++i) {
        if (forced_variant >= 0 && i != forced_variant) continue;
        const int K = rws::kTileRows[i].K;
        const int T = tile_rows_per_tile(cols, es, K);
        if (T == 0) continue;
        if (best >= 0) {
            // cost K * w(K) / T against the best so far; at equal cost the
            // smaller K for small launches, the larger tile for large ones
            const int Kb = rws::kTileRows[best].K;
            const int64_t lhs = (int64_t)K * w[K] * best_t;
            const int64_t rhs = (int64_t)Kb * w[Kb] * T;
            if (lhs > rhs || (lhs == rhs && (small || T <= best_t))) continue;
        }
        best = i;
        best_t = T;
    }
    if (T_out) *T_out = best_t;
    return best;
}

// XCD runs of the tile kernels (log2 of tiles per run, xcd_run): adjacent
// tiles that share a cache line then share an L2 instead of each XCD
// fetching the line (fp16 RMSNorm [1000000,33] read 9% more than it wrote
// in launch order).  Runs of 64 tiles against launch order, MI355X, fp16
// unless noted, inputs in HBM: backward [1000000,33] 34.1 us vs 35.1,
// [131072,250] 33.9 vs 34.8; RMSNorm [1000000,33] 25.1 vs 25.9; LayerNorm
// [131072,250] 24.6 vs 25.5; softmax [131072,250] 25.3 vs 25.7, [262144,120]
// 25.1 vs 25.6, fp32 [131072,125] 25.0 vs 25.8 ([1000000,33] 27.0 both).
constexpr int kTileLgRunFwd = 6;
constexpr int kTileLgRunBwd = 6;
constexpr int kTileLgRunNorm = 6;

// Rows per XCD run (log2) for the one-row-per-workgroup kernels that hold the
// row in registers (block_onepass, the backward's bwd_block): on rows that are
// not line-aligned, runs of at least 128 KiB of consecutive rows per XCD
// (xcd_run in rws_device.hpp) instead of launch order.  Measured on MI355X
// with inputs in HBM, fp16: block_onepass [8192,4097] 23.3 us against 23.9
// (runs of 16 rows), [16384,2001] 24.1 against 24.8 (64), [32768,1000] 23.1
// against 24.4 (64); bwd_block [32768,1000] 34.4 against 36.4, [8192,4097]
// 37.3 against 37.6.  Not used for line-aligned rows ([8192,4096]: 23.0
// against 22.6), two_pass (no change) or the normalisations ([8192,4097]
// with 576 threads: 33.8 against 32.7).
// Chunks per row of the backward's and the normalisations' ordered split-k
// (chunks of 256 x 4 granules), and whether a call takes it: rows too long
// for their one-workgroup-per-row register form (more than 4096 granules),
// fewer rows than CUs.  MI355X, fp16, inputs in HBM, streaming form ->
// ordered: [16,1048576] backward 143 -> 25.1 us, LayerNorm 106 -> 18.0,
// RMSNorm 75 -> 14.3; [64,262144] 42.4 -> 25.2, 31.2 -> 17.6, 22.6 -> 13.7;
// [192,65536] backward 18.3 -> 16.6, LayerNorm 14.2 -> 13.0; but
// [256,65536] 23.9 -> 25.5, 16.8 -> 18.5 (256 rows fill the chip one
// workgroup per row).  Where the register form holds the row it is kept at
// every row count: [128,16384] backward 5.14 us against 7.31 ordered,
// LayerNorm 5.02 against 7.30; [64,32768] 6.52 / 5.47 against 7.17 / 7.38;
// [16,16384] 4.16 / 4.80 against 5.88 / 6.85 (the backward gives up 2 % at
// [8..16,32768]: 6.07 against 5.93).
int ordered_chunks(int64_t wline, int block, int kc) {
    const int64_t span = (int64_t)block * kc;
    return (int)((wline + span - 1) / span);
}

bool few_long_rows(int64_t rows, int64_t wline, int cus) {
    return rows < cus && wline >= 2048;
}

int xcd_run_lg(const Geometry& g) {
    if (g.a128 || g.row_bytes <= 0) return 0;
    int lg = 0;
    while (((int64_t)1 << lg) * g.row_bytes < ((int64_t)128 << 10) && lg < 12) ++lg;
    return lg;
}

int64_t onepass_capacity(const rws::OnepassVariant& v) { return (int64_t)v.block * (v.kr + v.kl); }

// Rows per launch of a workgroup-per-row kernel: the launch's thread count
// (rows x block) must stay below 2^32, the width of the dispatch's grid size;
// batches of at most 2^31 threads and 2^22 rows.
int64_t block_rows_per_launch(int block) {
    return std::min<int64_t>((int64_t)1 << 22, ((int64_t)1 << 31) / block);
}

// Choose among the wave_row variants: the narrowest lane group whose
// registers hold the window, then the form that measured fastest on MI355X
// with rows streamed from HBM.  Plain softmax: one row set per wave and one
// granule per lane where it holds the row (fp16 512 columns: 21.9 us vs 23.1
// with two row sets, 22.8 with 32 lanes x 2 granules; bf16 128 columns with
// 16-lane groups: 79.8 us vs 81.8 us with two row sets).  The masked form
// (scale, mask and causal limit): two granules per lane on 8-32 lanes where
// that holds the row, else two row sets for one-granule full-wave rows.
// fp16 [rows,cols] with a [cols,cols] mask and causal limit, about 64 MiB
// in: 128 columns 20.9 us (8x2) vs 22.9 (16x1); 192: 22.6 (16x2) vs 30.8
// (32x1); 256: 20.0 (16x2) vs 23.3 (32x1); 384: 15.1 (32x2) vs 16.5 (64x1,
// two row sets); 512: 19.8 (32x2) vs 20.7 (64x1, two row sets; 25.4 with
// one); four granules on 32 lanes lost to two on 64 (768 columns 29.0 vs
// 21.8, 1024: 26.1 vs 19.7).  Rows that are not line-aligned take the same
// two-granule groups (two to four rows per wave instead of one to two):
// fp16 [131072,250] 34.2 us (32x2) vs 42.4 (64x1), [262144,120] 28.9 (16x2)
// vs 37.4 (32x1), [524288,60] 35.4 (8x2) vs 40.6 (16x1); line-aligned rows
// keep one granule per lane ([131072,256] 21.6 (32x1) vs 22.6 (16x2)).
// Windows of 65-96 granules: three granules on 32 lanes (two rows per wave)
// instead of two on 64, for the masked form and rows that are not
// line-aligned: plain fp16 [55392,577] 26.0 us vs 30.0, [31800,600] 15.7 vs
// 16.9, [32200,700] 18.2 vs 18.7, fp32 [65400,300] 29.0 vs 29.6; masked
// (causal, [S,S] mask) 577: 38.0 vs 40.1, 768: 16.3 vs 20.7, fp32 300: 26.3
// vs 30.9.  Plain line-aligned rows keep two on 64 ([32256,768] 17.6 vs
// 17.7).  max_k limits the granules per lane.
int pick_wave_row(const Geometry& g, bool masked = false, int max_k = 1 << 30) {
    int best = -1;
    int64_t best_key = 0;
    for (int i = 0; i < rws::kNumWaveRow; ++i) {
        const rws::WaveRowVariant& v = rws::kWaveRow[i];
        const int64_t w = window_granules(g, softmax_wave_wa(v));
        if ((int64_t)v.G * v.K < w || v.K > max_k) continue;
        if (v.K == 3 && !masked && g.a128) continue;
        const int64_t cap = (int64_t)v.G * v.K;
        int pref = 2;
        if ((masked || !g.a128) && v.K == 2 && v.G < 64) pref = 0;
        else if (v.U == ((masked && v.G == 64 && v.K == 1) ? 2 : 1)) pref = 1;
        const int64_t key = cap * 4 + pref;
        if (best < 0 || key < best_key) {
            best = i;
            best_key = key;
        }
    }
    return best;
}

// A launch with few waves: at one granule per thread (and at most 16 waves
// per row) it fills each CU with at most kFewWavesPerCu waves, so it is
// latency-bound and each row is best spread over many threads.
constexpr int64_t kFewWavesPerCu = 32;

bool few_waves(int64_t rows, int64_t w, int cus) {
    return rows * std::min<int64_t>((w + 63) / 64, 16) <= kFewWavesPerCu * cus;
}

// A workgroup-per-row shape: `block` threads, `kr` granules per thread in
// registers, `kl` more parked in LDS.
struct BlockShape {
    int block, kr, kl;
};

// Choose a workgroup-per-row shape for rows of w granules (line window) among
// shapes(0..n-1), by sweeps on MI355X with inputs in HBM:
//  * few waves: the fewest granules per thread, then the smallest workgroup
//    (fp32 [64,1000]: 2.84 us with 320x1 against 4.36 us for one wave per row
//    with 8 granules per lane; fp16 [1024,2000]: 4.03 us with 320x1, 4.29
//    with 192x2, 5.66 with one wave per row);
//  * otherwise: 2-5 register granules per thread with the fewest idle slots,
//    ties to fewer granules per thread -- the fastest shape of each sweep:
//    fp16 rows of 1000 columns (window 133) 64x3, 2000 (258) 64x5, 4000 (508)
//    256x2, 4097 (521) 192x3, 8000 (1008) 512x2; the same shapes are the
//    fastest for LayerNorm and RMSNorm (1000 columns: 24.9 / 24.3 us against
//    33.2 / 30.0 with 192x1; 2000: 24.5 / 23.8 against 30.5 / 27.3 with
//    320x1; 4097: 24.3 / 23.8 against 32.7 / 30.2 with 576x1);
//  * rows longer than those shapes hold: the smallest capacity.
template <class Shape>
int pick_block_shape(int n, Shape shape, int64_t w, int64_t rows, int cus) {
    const bool few = few_waves(rows, w, cus);
    int best = -1;
    int64_t best_key = 0;
    for (int i = 0; i < n; ++i) {
        const BlockShape v = shape(i);
        if (v.block <= 0) continue;
        const int64_t cap = (int64_t)v.block * (v.kr + v.kl);
        if (cap < w) continue;
        int64_t key;
        if (few)
            key = (int64_t)(v.kr + v.kl) * (1 << 20) + cap;
        else if (v.kl == 0 && v.kr >= 2 && v.kr <= 5)
            key = (cap - w) * 8 + v.kr;
        else
            key = ((int64_t)1 << 40) + cap;
        if (best < 0 || key < best_key) {
            best = i;
            best_key = key;
        }
    }
    return best;
}

// block_onepass variant (masked: no LDS parking, and the widened kernel
// form).  On rows that are not line-aligned, 8-granule shapes whose kernel
// exceeds the 128 VGPRs of a 1024-thread workgroup and spills are left out:
// those with LDS parking (136-240 bytes per lane), and the masked 16-bit
// form (172).  They ran at ~2.9 TB/s where two_pass reaches 4.2-5.0 (fp16
// [4096,128257]: 707 us against 422).  The plain 16-bit form at 8 register
// granules holds the row as raw granules (k_block_onepass_raw) and fits.
int pick_onepass(int64_t w, int64_t rows, int cus, bool masked, bool aligned, int dtype) {
    return pick_block_shape(
        rws::kNumOnepass,
        [&](int i) {
            const rws::OnepassVariant& v = rws::kOnepass[i];
            const bool spills = !aligned && v.kr + v.kl >= 8 &&
                                (v.kl > 0 || (masked && dtype != RWS_F32));
            if ((masked && v.kl != 0) || spills) return BlockShape{0, 0, 0};
            return BlockShape{v.block, v.kr, v.kl};
        },
        w, rows, cus);
}

// Split-k chunking: the largest chunk that still gives every CU eight
// workgroups, else two, else the smallest chunk.  Measured on fp16
// [16, 1048576]: 2048 workgroups of 256x4 granules 14.8-15.0 us, 1024 of
// 256x8 15.1-15.2 us, 4096 of 256x2 17.6 us, 512 of 256x16 18.0 us.
int pick_splitk(int64_t rows, int64_t wmax, int cus, int* P_out) {
    int best = -1;
    int bestP = 1;
    for (const int per_cu : {8, 2}) {
        for (int i = 0; i < rws::kNumSplitk; ++i) {
            const rws::SplitkVariant& v = rws::kSplitk[i];
            if (v.block != 256) continue;
            const int64_t cg = (int64_t)v.block * v.kc;
            const int64_t P = (wmax + cg - 1) / cg;
            if (P > (1 << 20)) continue;
            if (rows * P >= (int64_t)per_cu * cus &&
                (best < 0 || rws::kSplitk[i].kc > rws::kSplitk[best].kc)) {
                best = i;
                bestP = (int)P;
            }
        }
        if (best >= 0) break;
    }
    if (best < 0) {
        for (int i = 0; i < rws::kNumSplitk; ++i) {
            const rws::SplitkVariant& v = rws::kSplitk[i];
            if (v.block != 256) continue;
            const int64_t cg = (int64_t)v.block * v.kc;
            const int64_t P = (wmax + cg - 1) / cg;
            if (best < 0 || v.kc < rws::kSplitk[best].kc) {
                best = i;
                bestP = (int)P;
            }
        }
    }
    *P_out = bestP;
    return best;
}

// Co-resident workgroup capacity of a fused split-k variant on the current
// device (cached); without a device, the lower bound its compiled waves per
// SIMD give (4 SIMDs per CU).
int64_t fused_capacity(int variant, int dtype, bool aligned) {
    static std::mutex mu;
    static std::map<std::tuple<int, int, int, int>, int64_t> cache;
    const DeviceInfo info = device_info();
    if (!info.known)
        return (int64_t)info.cus * 4 * rws::splitk_fused_min_waves(variant, dtype, aligned) /
               (rws::kSplitkFused[variant].block / 64);
    int dev = 0;
    (void)hipGetDevice(&dev);
    const auto key = std::make_tuple(dev, variant, dtype, aligned ? 1 : 0);
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int64_t blocks = 0;
    const hipError_t e = rws::splitk_fused_capacity(variant, dtype, aligned, info.cus, &blocks);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        blocks = -(int64_t)e;  // negative: the occupancy query failed with this error
    }
    cache[key] = blocks;
    return blocks;
}

// Fused split-k chunking: the largest chunk whose grid still gives every CU
// two workgroups and fits the co-resident capacity; else the smallest chunk
// that fits.  `fit_rows` rows must fit at once: the whole grid for the
// dispatcher's own choice, one row when the form is requested.  Returns -1
// when no variant fits.  (fp16, inputs in HBM: [4,8M] 16 granules per
// thread 25.3 us, 8 28.6, 4 34.4; [16,1M] 14.5-14.8, 15.6, 16.0.)
int pick_splitk_fused(int64_t fit_rows, int64_t rows, int64_t wmax, int dtype, bool aligned, int cus,
                      int* P_out) {
    int best = -1, bestP = 1;
    for (int pass = 0; pass < 2 && best < 0; ++pass) {
        for (int i = 0; i < rws::kNumSplitkFused; ++i) {
            const rws::SplitkVariant& v = rws::kSplitkFused[i];
            const int64_t cg = (int64_t)v.block * v.kc;
            const int64_t P = (wmax + cg - 1) / cg;
            if (P > (1 << 20) || fit_rows * P > fused_capacity(i, dtype, aligned)) continue;
            if (pass == 0 && rows * P < 2LL * cus) continue;
            const bool better = best < 0 || (pass == 0 ? v.kc > rws::kSplitkFused[best].kc
                                                       : v.kc < rws::kSplitkFused[best].kc);
            if (better) {
                best = i;
                bestP = (int)P;
            }
        }
    }
    *P_out = bestP;
    return best;
}

// forced_variant >= 0 (measurement surface, softmax_fwd_variant): that entry
// of the family's variant table instead of the dispatcher's choice, when it
// can hold the row.
int plan_launch_uncached(int64_t rows, int64_t cols, int dtype, const void* in, const void* out,
                         int kernel_id, Plan* p, bool masked, int forced_variant = -1) {
    auto bad_variant = [&](int n) {
        return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                    "variant " + std::to_string(forced_variant) + " of " +
                        std::to_string(n) + " cannot take this shape");
    };
    const Geometry g = geometry(cols, dtype, in, out);
    p->same_phase = g.same_phase;
    const int64_t wline = window_granules(g, 128);  // block-level kernels
    const int cus = device_info().cus;

    // Family: a lane group holding the row at one granule per lane ->
    // wave_row; few long rows -> split-k; many rows of up to two granules per
    // lane of a full wave -> wave_row; else one workgroup per row while its
    // registers (then LDS) hold the row; then split-k for few rows, two_pass.
    // (One wave per row with 4 or 8 granules per lane measured slower than
    // block_onepass at every row count tried: fp16 [32768,1000] 27.2 us
    // against 24.5, fp16 [16384,2000] 32.8 against 23.5.)
    // "Few long rows" (rows of >= 2048 granules) takes split-k over
    // block_onepass when block_onepass cannot hold the row, or would leave
    // more than half the CUs without a row, or leaves half of them idle and
    // parks part of the row in LDS.  MI355X, fp16, inputs in HBM, ordered
    // split-k against block_onepass: [64,65536] 7.76 against 8.98 us;
    // [128,131072] 14.4 against 18.8 (LDS parking); but [128,65536] 9.81
    // against 9.48, [256,65536] 14.5 against 14.1, [256,16384] 7.71 against
    // 5.42, [384,65536] 25.0 against 22.3, [256,131072] 32.0 against 29.9.
    int family = kernel_id;
    if (family == RWS_KERNEL_AUTO) {
        const bool few_rows = rows < 2LL * cus;
        const int ov = pick_onepass(wline, rows, cus, false, g.a128, dtype);
        const bool onepass_fits = ov >= 0;
        const bool parks = onepass_fits && rws::kOnepass[ov].kl > 0;
        const bool splitk_rows =
            !onepass_fits || 2 * rows < cus || (2 * rows <= cus && parks);
        if (tile_rows_fits(rows, cols, dtype, in, out)) {
            family = RWS_KERNEL_TILE_ROWS;
        } else if (pick_wave_row(g, masked, 1) >= 0) {
            family = RWS_KERNEL_WAVE_ROW;
        } else if (few_rows && wline >= 2048 && splitk_rows) {
            family = RWS_KERNEL_SPLITK_ORDERED;
        } else if (wline <= 128 && !few_waves(rows, wline, cus) &&
                   pick_wave_row(g, masked, 2) >= 0) {
            family = RWS_KERNEL_WAVE_ROW;
        } else if (onepass_fits) {
            family = RWS_KERNEL_BLOCK_ONEPASS;
        } else if (few_rows) {
            family = RWS_KERNEL_SPLITK_ORDERED;
        } else {
            family = RWS_KERNEL_TWO_PASS;
        }
    }
    if (masked && kernel_id == RWS_KERNEL_AUTO) {
        // the masked forms exist for tile_rows, wave_row, register-only
        // block_onepass and two_pass; long rows with few rows go to two_pass
        if (is_splitk(family)) family = RWS_KERNEL_TWO_PASS;
        if (family == RWS_KERNEL_BLOCK_ONEPASS && pick_onepass(wline, rows, cus, true, g.a128, dtype) < 0)
            family = RWS_KERNEL_TWO_PASS;
    }
    if (masked && is_splitk(family))
        return fail(RWS_ERR_UNSUPPORTED_SHAPE, "the masked form has no split-k kernel");
    p->family = family;
    // The masked form takes windows that start at the row on 16-byte aligned
    // rows (line windows otherwise lead with granules outside the row and
    // run the prologue's edge handling): fp16, [S,S] mask, causal, S = 1000
    // 26.9 us against 28.0, 2000: 45.5 against 51.5, 3000: 24.5 against
    // 25.4.  Plain softmax keeps line windows (each output line written by
    // one workgroup).
    p->aligned = masked ? g.a16 : g.a128;
    p->window = wline;
    switch (family) {
        case RWS_KERNEL_TILE_ROWS: {
            const int es = elem_size(dtype);
            if ((uintptr_t)in % 16 || (uintptr_t)out % 16)
                return fail(RWS_ERR_UNSUPPORTED_SHAPE, "tile_rows needs 16-byte aligned in and out");
            int T = 0;
            p->variant = pick_tile_rows(rows, cols, es, -1, &T);
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumTileRows) return bad_variant(rws::kNumTileRows);
                if (pick_tile_rows(rows, cols, es, forced_variant, &T) < 0) return bad_variant(rws::kNumTileRows);
                p->variant = forced_variant;
            }
            if (p->variant < 0)
                return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                            "tile_rows takes rows of one granule to 1024 bytes");
            p->aligned = false;
            p->tile_t = T;
            p->lgrun = kTileLgRunFwd;
            p->window = (int64_t)T * cols * es / 16;
            // tiles (workgroups) per launch below 2^31
            p->max_rows_per_launch = (int64_t)T * ((int64_t)1 << 30);
            break;
        }
        case RWS_KERNEL_WAVE_ROW: {
            p->variant = pick_wave_row(g, masked);
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumWaveRow) return bad_variant(rws::kNumWaveRow);
                const rws::WaveRowVariant& f = rws::kWaveRow[forced_variant];
                if ((int64_t)f.G * f.K < window_granules(g, softmax_wave_wa(f)))
                    return bad_variant(rws::kNumWaveRow);
                p->variant = forced_variant;
            }
            if (p->variant < 0)
                return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                            "wave_row holds at most 512 granules (16 bytes) per row window");
            const rws::WaveRowVariant& v = rws::kWaveRow[p->variant];
            const int wa = softmax_wave_wa(v);
            p->aligned = wa == 128 && !masked ? g.a128 : g.a16;
            p->window = window_granules(g, wa);
            // every 128-byte line of the output is written by one wave:
            // store it through (faster there; slower where lines are shared)
            p->wt = g.a128;
            // keep the threads of one launch below 2^32 (2^25 waves)
            p->max_rows_per_launch = (int64_t)(64 / v.G) * v.U * 4 * ((int64_t)1 << 23);
            break;
        }
        case RWS_KERNEL_BLOCK_ONEPASS: {
            p->variant = pick_onepass(wline, rows, cus, masked, g.a128, dtype);
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumOnepass) return bad_variant(rws::kNumOnepass);
                const rws::OnepassVariant& f = rws::kOnepass[forced_variant];
                if (onepass_capacity(f) < wline || (masked && f.kl != 0))
                    return bad_variant(rws::kNumOnepass);
                p->variant = forced_variant;
            }
            if (p->variant < 0)
                return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                            "block_onepass holds at most 16384 granules (16 bytes) per row window "
                            "on line-aligned rows, 8192 otherwise (6144 for the masked 16-bit "
                            "form)");
            p->max_rows_per_launch = block_rows_per_launch(rws::kOnepass[p->variant].block);
            p->lgrun = xcd_run_lg(g);
            break;
        }
        case RWS_KERNEL_TWO_PASS: {
            // 256 threads for short rows, 512 up to 4096 granules, then 1024
            const int want_block = wline > 4096 ? 1024 : wline > 1024 ? 512 : 256;
            p->variant = 0;
            for (int i = 0; i < rws::kNumTwoPass; ++i)
                if (rws::kTwoPass[i].block == want_block && rws::kTwoPass[i].u == 4) p->variant = i;
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumTwoPass) return bad_variant(rws::kNumTwoPass);
                p->variant = forced_variant;
            }
            p->max_rows_per_launch = block_rows_per_launch(rws::kTwoPass[p->variant].block);
            break;
        }
        case RWS_KERNEL_SPLITK_FUSED: {
            // requested: one row's workgroups must fit at once (rows beyond
            // the capacity follow in dispatch order)
            int P = 1;
            p->variant = pick_splitk_fused(1, rows, wline, dtype, g.a128, cus, &P);
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumSplitkFused) return bad_variant(rws::kNumSplitkFused);
                const int64_t cg = (int64_t)rws::kSplitkFused[forced_variant].block *
                                   rws::kSplitkFused[forced_variant].kc;
                const int64_t fp = (wline + cg - 1) / cg;
                if (fp > fused_capacity(forced_variant, dtype, g.a128))
                    return bad_variant(rws::kNumSplitkFused);
                p->variant = forced_variant;
                P = (int)fp;
            }
            if (p->variant < 0) {
                std::string caps;
                for (int i = 0; i < rws::kNumSplitkFused; ++i) {
                    const int64_t cg = (int64_t)rws::kSplitkFused[i].block * rws::kSplitkFused[i].kc;
                    caps += " " + std::to_string((wline + cg - 1) / cg) + "/" +
                            std::to_string(fused_capacity(i, dtype, g.a128));
                }
                return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                            "fused split-k: one row's workgroups cannot be resident at once on "
                            "this device (workgroups per row/capacity per variant:" + caps + ")");
            }
            p->P = P;
            // at most 2^23 workgroups per launch
            p->max_rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 23) / P);
            break;
        }
        case RWS_KERNEL_SPLITK:
        case RWS_KERNEL_SPLITK_ORDERED: {
            int P = 1;
            p->variant = pick_splitk(rows, wline, cus, &P);
            if (forced_variant >= 0) {
                if (forced_variant >= rws::kNumSplitk) return bad_variant(rws::kNumSplitk);
                const int64_t cg =
                    (int64_t)rws::kSplitk[forced_variant].block * rws::kSplitk[forced_variant].kc;
                const int64_t fp = (wline + cg - 1) / cg;
                if (fp > (1 << 20)) return bad_variant(rws::kNumSplitk);
                p->variant = forced_variant;
                P = (int)fp;
            }
            if (p->variant < 0) return fail(RWS_ERR_UNSUPPORTED_SHAPE, "split-k: no variant");
            p->P = P;
            // The ordered form saves the two-launch form's kernel boundary
            // but every stage-2 workgroup polls all P of its row's partials
            // (two tagged words each), and its stage-2 re-read overlaps the
            // last stage-1 reads only while the input fits the L2 of the
            // XCDs (8 x 4 MiB).  MI355X, fp16, inputs in HBM, ordered
            // against two launches: 32 MiB inputs [16,1M] (P 128) 14.5
            // against 15.6 us, [8,2M] (256) 14.7 against 15.7, [4,4M] (512)
            // 15.9 against 16.3, but [2,8M] (1024) 18.9 against 17.6; 64 MiB
            // inputs [32,1M] 31.9 against 31.4, [16,2M] 31.9 against 31.0,
            // [8,4M] 31.8 against 30.8, [4,8M] 33.8 against 30.1.  Past
            // either limit the dispatcher keeps the two launches.
            // The fused single launch reads the input once but writes only
            // after all of a row's chunks are read; where its whole grid
            // fits at once it beats the two launches everywhere measured and
            // the ordered form for up to four rows.  MI355X, fp16, inputs in
            // HBM, fused against the dispatcher's previous choice: 64 MiB
            // [1,32M] 28.1 against 32.9 us (two launches), [4,8M] 25.3
            // against 29.9, [32,1M] 24.4 against 31.3, [128,256K] 23.8
            // against 31.4; 32 MiB [1,16M] 16.6 against 19.0, [2,8M] 15.1
            // against 17.1, [4,4M] 14.9 against 15.8 (ordered); 8 MiB
            // [4,1M] 8.1 against 9.0 (ordered), [1,4M] 9.0 against 9.5; but
            // ordered ahead from eight rows: [8,1M] 10.3 against 11.0,
            // [16,512K] 10.1 against 10.9, [16,1M] 14.2 against 14.5,
            // [32,512K] 14.3 against 14.6 ([8,2M] 14.7 both).  Past 64 MiB
            // the grid runs in several passes and only ties the two
            // launches ([4,32M] 115.3 against 115.5), which are kept.
            const bool ordered_fits =
                P <= kOrderedMaxP && rows * cols * elem_size(dtype) <= kOrderedMaxBytes;
            if (family == RWS_KERNEL_SPLITK_ORDERED && kernel_id == RWS_KERNEL_AUTO &&
                forced_variant < 0) {
                int fP = 1;
                const int fv = pick_splitk_fused(rows, rows, wline, dtype, g.a128, cus, &fP);
                if (fv >= 0 && (!ordered_fits || rows <= kFusedFewRows)) {
                    p->family = RWS_KERNEL_SPLITK_FUSED;
                    p->variant = fv;
                    p->P = fP;
                    p->max_rows_per_launch = rows;
                    break;
                }
                if (!ordered_fits) family = p->family = RWS_KERNEL_SPLITK;
            }
            // at most 2^23 workgroups per launch (both stages of the ordered
            // form count)
            const int64_t per_row = family == RWS_KERNEL_SPLITK_ORDERED ? 2LL * P : (int64_t)P;
            p->max_rows_per_launch = std::max<int64_t>(1, ((int64_t)1 << 23) / per_row);
            break;
        }
        default:
            return fail(RWS_ERR_INVALID_ARG, "unknown kernel id " + std::to_string(kernel_id));
    }
    return RWS_OK;
}

// ---------------------------------------------------------------------------
// split-k workspace: one grow-only buffer per (device, stream).  Work on one
// stream is ordered, so a buffer is never used by two launches at once.
// ---------------------------------------------------------------------------
struct Workspace {
    void* ptr = nullptr;        // split-k partials
    size_t bytes = 0;
    uint64_t* tags = nullptr;   // single-launch split-k: epoch-tagged partial words
    int64_t tag_words = 0;
    unsigned tag_epoch = 0;     // last epoch used on `tags`
    bool captured = false;      // `ptr` is baked into a captured graph
    bool tags_captured = false; // `tags` is baked into a captured graph
    uint64_t* status = nullptr; // give-up status word of the single-launch
                                // forms (allocated once, kept until unload)
    std::vector<void*> retired; // buffers that graphs may still use
};

// Tries of one poll of the ordered forms (softmax_set_wait_limit).
std::atomic<unsigned> g_wait_limit{rws::kOrderedSpinLimit};

// Words after a tag buffer's tag words: the device epoch of launches replayed
// from graphs (rws_ordered.hpp), padded to a 128-byte line.
constexpr int64_t kTagTailWords = 16;

std::mutex g_ws_mu;
std::map<std::pair<int, hipStream_t>, Workspace>* g_ws = nullptr;

struct WorkspaceReaper {
    ~WorkspaceReaper() {
        // Buffers are released at unload; a device that is already torn down
        // reports an error here, which is ignored.
        if (!g_ws) return;
        for (auto& kv : *g_ws) {
            if (kv.second.ptr) (void)hipFree(kv.second.ptr);
            if (kv.second.tags) (void)hipFree(kv.second.tags);
            if (kv.second.status) (void)hipFree(kv.second.status);
            for (void* p : kv.second.retired) (void)hipFree(p);
        }
        delete g_ws;
        g_ws = nullptr;
    }
} g_ws_reaper;

// True while `s` is being captured into a graph.  The single-launch split-k
// forms tell one launch's partials from the last one's by an epoch passed as
// a kernel argument, which a graph would replay unchanged (a replay's stage 2
// could take the previous replay's partials).  Under capture the forward
// takes the two-launch split-k (ordered by its kernel boundary); the
// backward and the normalisations keep their ordered launch but take its
// epoch from a device word that a kernel recorded before it advances on
// every replay (launch_bump_epoch), or, when the stream has no tag buffer
// large enough, take their one-workgroup-per-row forms.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

// The give-up status word of (device, stream) (see rws::OrderedSync): one
// 128-byte line, zeroed by a kernel on `stream` when it is allocated on the
// stream's first single-launch split-k call, never moved, so launches that
// a graph recorded keep reporting into it.  nullptr when it does not exist
// yet and `cap` (nothing may be allocated while capturing; the launch then
// still writes NaN, it only cannot report).  The caller holds g_ws_mu.
int get_status_word(hipStream_t stream, bool cap, uint64_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (!g_ws) g_ws = new std::map<std::pair<int, hipStream_t>, Workspace>();
    Workspace& w = (*g_ws)[std::make_pair(dev, stream)];
    if (!w.status && !cap) {
        uint64_t* p = nullptr;
        e = hipMalloc((void**)&p, 128);
        if (e == hipSuccess) e = rws::launch_fill_words(p, 16, 0, stream);
        if (e != hipSuccess) {
            if (p) (void)hipFree(p);
            return fail(RWS_ERR_HIP, std::string("status word: ") + hipGetErrorString(e));
        }
        w.status = p;
    }
    *out = w.status;
    return RWS_OK;
}

// Grow-only workspace of (device, stream): `bytes` of partials of the
// two-launch split-k.  The caller holds
// g_ws_mu from this call until its launches are enqueued: a call from another
// host thread on the same stream that grows the buffer synchronises the
// stream and frees the old one, which is only safe once every launch that
// uses it is on the stream.  Under graph capture (`cap`: the stream is
// capturing) nothing is allocated (the call fails if the buffer is too
// small) and the buffer handed out is marked captured: when it grows later it
// is kept, not freed, since the graph's launches still name it.
int get_workspace(hipStream_t stream, bool cap, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (!g_ws) g_ws = new std::map<std::pair<int, hipStream_t>, Workspace>();
    Workspace& w = (*g_ws)[std::make_pair(dev, stream)];
    const bool grow_partials = w.bytes < bytes;
    if (grow_partials && cap)
        return fail(RWS_ERR_HIP,
                    "split-k workspace too small during graph capture: run the call once on "
                    "this stream before capturing it");
    if (grow_partials && w.ptr) {
        // the old buffers may still be in use by earlier work on this stream
        e = hipStreamSynchronize(stream);
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    }
    if (std::getenv("RWS_TEST_FAIL_ALLOC") && grow_partials)
        return fail(RWS_ERR_HIP, "workspace allocation failed (RWS_TEST_FAIL_ALLOC)");
    if (grow_partials) {
        if (w.ptr && w.captured)
            w.retired.push_back(w.ptr);
        else if (w.ptr)
            (void)hipFree(w.ptr);
        w.captured = false;
        w.ptr = nullptr;
        w.bytes = 0;
        size_t want = 4096;
        while (want < bytes) want *= 2;
        e = hipMalloc(&w.ptr, want);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return fail(RWS_ERR_HIP, std::string("hipMalloc (split-k workspace): ") + hipGetErrorString(e));
        }
        w.bytes = want;
    }
    if (cap) w.captured = true;
    *out = w.ptr;
    return RWS_OK;
}

// Tag words of the ordered split-k for (device, stream): grow-only, zeroed
// (by a kernel on `stream`) when allocated, followed by the device epoch word
// of captured launches.  Reserves `launches` consecutive host epochs and
// returns the first in *epoch0; when the host's range [1, 2^31) would run
// out, the words are zeroed again and the epochs restart at 1, so a word left
// by an earlier launch never carries a live epoch.  A buffer that a graph
// captured is kept, not freed, when it grows.  The caller holds g_ws_mu
// until its launches are enqueued (as for get_workspace).
int get_tag_workspace(hipStream_t stream, int64_t words, int64_t launches, uint64_t** out,
                      unsigned* epoch0) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (!g_ws) g_ws = new std::map<std::pair<int, hipStream_t>, Workspace>();
    Workspace& w = (*g_ws)[std::make_pair(dev, stream)];
    if (w.tag_words < words && capturing(stream))
        return fail(RWS_ERR_HIP, "split-k tag words too small during graph capture");
    if (w.tag_words < words) {
        if (w.tags && w.tags_captured) {
            w.retired.push_back(w.tags);
        } else if (w.tags) {
            // the old words may still be in use by earlier work on this stream
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return fail(RWS_ERR_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
            (void)hipFree(w.tags);
        }
        w.tags = nullptr;
        w.tag_words = 0;
        w.tags_captured = false;
        if (std::getenv("RWS_TEST_FAIL_ALLOC"))
            return fail(RWS_ERR_HIP, "workspace allocation failed (RWS_TEST_FAIL_ALLOC)");
        int64_t want = 512;
        while (want < words) want *= 2;
        e = hipMalloc((void**)&w.tags, (size_t)(want + kTagTailWords) * sizeof(uint64_t));
        if (e == hipSuccess) e = rws::launch_fill_words(w.tags, want + kTagTailWords, 0, stream);
        // test hooks: start a fresh buffer's host or device epochs just below
        // the end of their range
        const char* dev_start = std::getenv("RWS_TEST_DEVICE_EPOCH");
        if (e == hipSuccess && dev_start)
            e = rws::launch_fill_words(w.tags + want, 1, std::strtoull(dev_start, nullptr, 0),
                                       stream);
        if (e != hipSuccess) {
            if (w.tags) (void)hipFree(w.tags);
            w.tags = nullptr;
            return fail(RWS_ERR_HIP, std::string("split-k tag words: ") + hipGetErrorString(e));
        }
        w.tag_words = want;
        const char* start = std::getenv("RWS_TEST_TAG_EPOCH");
        w.tag_epoch = start ? (unsigned)std::strtoul(start, nullptr, 0) : 0u;
    }
    if ((uint64_t)w.tag_epoch + (uint64_t)launches >= (uint64_t)rws::kDeviceEpochFirst) {
        e = rws::launch_fill_words(w.tags, w.tag_words, 0, stream);
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("split-k tag words: ") + hipGetErrorString(e));
        w.tag_epoch = 0;
    }
    *out = w.tags;
    *epoch0 = w.tag_epoch + 1;
    w.tag_epoch += (unsigned)launches;
    return RWS_OK;
}

// Under graph capture: the stream's tag buffer and its word count when it
// holds `words` (it is then marked captured), else false: nothing may be
// allocated while capturing, and the caller takes a form without tags.
// Each captured ordered launch is preceded by launch_bump_epoch on the
// buffer and reads its epoch from the word after the tag words.
bool captured_tags(hipStream_t stream, int64_t words, uint64_t** tags, int64_t* n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    if (!g_ws) return false;
    auto it = g_ws->find(std::make_pair(dev, stream));
    if (it == g_ws->end() || !it->second.tags || it->second.tag_words < words) return false;
    it->second.tags_captured = true;
    *tags = it->second.tags;
    *n = it->second.tag_words;
    return true;
}

int check_args(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int kernel_id) {
    if (dtype != RWS_F32 && dtype != RWS_F16 && dtype != RWS_BF16)
        return fail(RWS_ERR_UNSUPPORTED_DTYPE, "dtype must be RWS_F32, RWS_F16 or RWS_BF16");
    if (kernel_id < RWS_KERNEL_AUTO || kernel_id > RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "unknown kernel id " + std::to_string(kernel_id));
    if (rows < 0 || cols < 0) return fail(RWS_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols > kMaxCols) return fail(RWS_ERR_UNSUPPORTED_SHAPE, "cols above 2^30");
    if (rows == 0 || cols == 0) return RWS_OK;
    if (!in || !out) return fail(RWS_ERR_INVALID_ARG, "NULL pointer with a non-empty tensor");
    const int es = elem_size(dtype);
    if ((uintptr_t)in % es || (uintptr_t)out % es)
        return fail(RWS_ERR_MISALIGNED, "pointer not aligned to the element size");
    return RWS_OK;
}

// One call: plan, get the workspace if needed, launch in row batches.
// `mask` selects the masked/scaled form (nullptr: plain softmax).
// The plan is a function of the shape, the dtype, the kernel request, the
// pointers' offsets within a 128-byte line and the device.  The last few
// plans are kept per thread, so a repeated call skips the variant searches
// (about 0.4 us of the ~4 us a small call spends on the host, measured on
// MI355X through ctypes).
struct PlanKey {
    int64_t rows, cols;
    int dtype, kernel_id, dev;
    unsigned in_line, out_line;
    bool masked;
    int variant;
    bool operator==(const PlanKey& o) const {
        return rows == o.rows && cols == o.cols && dtype == o.dtype && kernel_id == o.kernel_id &&
               dev == o.dev && in_line == o.in_line && out_line == o.out_line &&
               masked == o.masked && variant == o.variant;
    }
};

int plan_launch(int64_t rows, int64_t cols, int dtype, const void* in, const void* out,
                int kernel_id, Plan* p, bool masked = false, int forced_variant = -1) {
    struct Slot {
        PlanKey key;
        Plan plan;
        bool used = false;
    };
    constexpr int kSlots = 8;
    thread_local Slot slots[kSlots];
    thread_local int next = 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        dev = -1;
    }
    const PlanKey key{rows, cols, dtype, kernel_id, dev, (unsigned)((uintptr_t)in % 128),
                      (unsigned)((uintptr_t)out % 128), masked, forced_variant};
    for (const Slot& sl : slots)
        if (sl.used && sl.key == key) {
            *p = sl.plan;
            return RWS_OK;
        }
    const int st =
        plan_launch_uncached(rows, cols, dtype, in, out, kernel_id, p, masked, forced_variant);
    if (st == RWS_OK) {
        slots[next].key = key;
        slots[next].plan = *p;
        slots[next].used = true;
        next = (next + 1) % kSlots;
    }
    return st;
}

int run(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream,
        int kernel_id, const rws::MaskArgs* mask, int forced_variant = -1) {
    Plan p;
    int st = plan_launch(rows, cols, dtype, in, out, kernel_id, &p, mask != nullptr, forced_variant);
    if (st != RWS_OK) return st;
    const bool cap = is_splitk(p.family) && capturing((hipStream_t)stream);
    if (cap && p.family != RWS_KERNEL_SPLITK) {
        // the ordered form shares the two-launch form's variant table
        st = plan_launch(rows, cols, dtype, in, out, RWS_KERNEL_SPLITK, &p, mask != nullptr,
                         p.family == RWS_KERNEL_SPLITK_ORDERED ? forced_variant : -1);
        if (st != RWS_OK) return st;
    }

    void* ws = nullptr;
    unsigned epoch = 0;
    hipStream_t s = (hipStream_t)stream;
    // split-k: keep the workspace locked until this call's launches are enqueued
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    uint64_t* tags = nullptr;
    if (is_splitk(p.family)) ws_lock.lock();
    if (p.family == RWS_KERNEL_SPLITK_ORDERED || p.family == RWS_KERNEL_SPLITK_FUSED) {
        // size the two-launch form's partials too (rows * P pairs, a few KiB
        // for these shapes): a capture of the same call takes that form and
        // must find its workspace already allocated (sized before the
        // buffers below are taken, since growing frees the old buffer)
        Plan p2;
        if (plan_launch(rows, cols, dtype, in, out, RWS_KERNEL_SPLITK, &p2, mask != nullptr) ==
            RWS_OK) {
            void* ws2 = nullptr;
            const int64_t batch2 = std::min<int64_t>(rows, p2.max_rows_per_launch);
            st = get_workspace(s, false, (size_t)batch2 * p2.P * sizeof(float2), &ws2);
            if (st != RWS_OK) return st;
        }
    }
    if (p.family == RWS_KERNEL_SPLITK) {
        const int64_t batch = std::min<int64_t>(rows, p.max_rows_per_launch);
        st = get_workspace(s, cap, (size_t)batch * p.P * sizeof(float2), &ws);
        if (st != RWS_OK) return st;
    } else if (p.family == RWS_KERNEL_SPLITK_ORDERED || p.family == RWS_KERNEL_SPLITK_FUSED) {
        const int64_t batch = std::min<int64_t>(rows, p.max_rows_per_launch);
        const int64_t launches = (rows + p.max_rows_per_launch - 1) / p.max_rows_per_launch;
        if (launches >= ((int64_t)1 << 31))
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "single-launch split-k: too many launches for one call");
        st = get_tag_workspace(s, 2 * batch * p.P, launches, &tags, &epoch);
        if (st != RWS_OK) return st;
    }
    uint64_t* status = nullptr;
    if (p.family == RWS_KERNEL_SPLITK_FUSED || p.family == RWS_KERNEL_SPLITK_ORDERED) {
        st = get_status_word(s, cap, &status);
        if (st != RWS_OK) return st;
    }
    const unsigned wait_limit = g_wait_limit.load(std::memory_order_relaxed);
    const int64_t row_bytes = cols * elem_size(dtype);
    for (int64_t r0 = 0; r0 < rows; r0 += p.max_rows_per_launch) {
        rws::Launch L;
        L.rows = std::min<int64_t>(p.max_rows_per_launch, rows - r0);
        L.in = (const char*)in + r0 * row_bytes;
        L.out = (char*)out + r0 * row_bytes;
        L.cols = (int)cols;
        L.dtype = dtype;
        L.aligned = p.aligned;
        L.same_phase = p.same_phase;
        L.wt = p.wt;
        L.lgrun = p.lgrun;
        L.stream = s;
        hipError_t e = hipSuccess;
        if (mask) {
            rws::MaskArgs M = *mask;
            M.row_base = r0;
            switch (p.family) {
                case RWS_KERNEL_WAVE_ROW: e = rws::launch_wave_row_masked(L, p.variant, M); break;
                case RWS_KERNEL_BLOCK_ONEPASS:
                    e = rws::launch_block_onepass_masked(L, p.variant, M);
                    break;
                case RWS_KERNEL_TWO_PASS: e = rws::launch_two_pass_masked(L, p.variant, M); break;
                case RWS_KERNEL_TILE_ROWS:
                    e = rws::launch_tile_rows_masked(L, p.variant, rws::TileShape{p.tile_t, p.lgrun},
                                                     M);
                    break;
                default: e = hipErrorInvalidValue;
            }
        } else {
            switch (p.family) {
                case RWS_KERNEL_WAVE_ROW: e = rws::launch_wave_row(L, p.variant); break;
                case RWS_KERNEL_TILE_ROWS:
                    e = rws::launch_tile_rows(L, p.variant, rws::TileShape{p.tile_t, p.lgrun});
                    break;
                case RWS_KERNEL_BLOCK_ONEPASS: e = rws::launch_block_onepass(L, p.variant); break;
                case RWS_KERNEL_TWO_PASS: e = rws::launch_two_pass(L, p.variant); break;
                case RWS_KERNEL_SPLITK:
                    e = rws::launch_splitk(L, p.variant, p.P, (float2*)ws);
                    break;
                case RWS_KERNEL_SPLITK_FUSED:
                    // one epoch per launch, as below
                    e = rws::launch_splitk_fused(
                        L, p.variant, p.P,
                        rws::OrderedSync{tags, epoch + (unsigned)(r0 / p.max_rows_per_launch),
                                         nullptr, status, wait_limit});
                    break;
                case RWS_KERNEL_SPLITK_ORDERED:
                    // one epoch per launch: the batches reuse the same tag words
                    e = rws::launch_splitk_ordered(
                        L, p.variant, p.P,
                        rws::OrderedSync{tags, epoch + (unsigned)(r0 / p.max_rows_per_launch),
                                         nullptr, status, wait_limit});
                    break;
            }
        }
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    }
    return RWS_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of softmax_fwd_noalloc: split-k partials in device memory that the
// library never allocates -- a file-scope array that every GPU the library
// runs on holds from the load of its code object until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is handed to kernels.
// ---------------------------------------------------------------------------
constexpr int64_t kNoAllocScratchBytes = (int64_t)512 << 10;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> address of its copy of `scratch`

// The current device's copy of `scratch`; looked up on the first call on
// that device.
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return RWS_OK;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
        return fail(RWS_ERR_HIP, std::string("hipGetSymbolAddress (split-k scratch): ") +
                                     hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
    *out = ptr;
    return RWS_OK;
}

// softmax_fwd without device allocation: the dispatcher's plan, with a
// split-k plan run as the two-launch split-k (kernel-boundary ordering: no
// epochs, no words that must start at zero, and a captured launch replays
// correctly) on partials in `scratch`, in row batches that fit it.
int run_noalloc(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    Plan p;
    int st = plan_launch(rows, cols, dtype, in, out, RWS_KERNEL_AUTO, &p);
    if (st != RWS_OK) return st;
    if (!is_splitk(p.family)) return run(in, out, rows, cols, dtype, stream, RWS_KERNEL_AUTO, nullptr);
    st = plan_launch(rows, cols, dtype, in, out, RWS_KERNEL_SPLITK, &p);
    if (st != RWS_OK) return st;
    const int64_t per_row = (int64_t)p.P * (int64_t)sizeof(float2);
    if (per_row > kNoAllocScratchBytes)
        return fail(RWS_ERR_UNSUPPORTED_SHAPE,
                    "softmax_fwd_noalloc: a row of " + std::to_string(cols) + " columns needs " +
                        std::to_string(per_row) + " bytes of split-k partials, above the " +
                        std::to_string(kNoAllocScratchBytes) + "-byte scratch");
    void* ptr = nullptr;
    st = scratch_address(&ptr);
    if (st != RWS_OK) return st;
    const int64_t batch = std::min<int64_t>(p.max_rows_per_launch, kNoAllocScratchBytes / per_row);
    const int64_t row_bytes = cols * elem_size(dtype);
    for (int64_t r0 = 0; r0 < rows; r0 += batch) {
        rws::Launch L;
        L.rows = std::min<int64_t>(batch, rows - r0);
        L.in = (const char*)in + r0 * row_bytes;
        L.out = (char*)out + r0 * row_bytes;
        L.cols = (int)cols;
        L.dtype = dtype;
        L.aligned = p.aligned;
        L.same_phase = p.same_phase;
        L.wt = p.wt;
        L.lgrun = p.lgrun;
        L.stream = (hipStream_t)stream;
        const hipError_t e = rws::launch_splitk(L, p.variant, p.P, (float2*)ptr);
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("kernel launch: ") + hipGetErrorString(e));
    }
    return RWS_OK;
}

}  // namespace

extern "C" {

int softmax_fwd_noalloc(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                        void* stream) {
    g_last_error.clear();
    const int st = check_args(in, out, rows, cols, dtype, RWS_KERNEL_AUTO);
    if (st != RWS_OK || rows == 0 || cols == 0) return st;
    return run_noalloc(in, out, rows, cols, dtype, stream);
}

int softmax_fwd_kernel(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                       void* stream, int kernel_id) {
    g_last_error.clear();
    const int st = check_args(in, out, rows, cols, dtype, kernel_id);
    if (st != RWS_OK || rows == 0 || cols == 0) return st;
    return run(in, out, rows, cols, dtype, stream, kernel_id, nullptr);
}

int softmax_fwd_masked(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                       float scale, const void* mask, int64_t mask_rows, int64_t causal_q,
                       void* stream, int kernel_id) {
    g_last_error.clear();
    const int st = check_args(in, out, rows, cols, dtype, kernel_id);
    if (st != RWS_OK) return st;
    if (causal_q < 0) return fail(RWS_ERR_INVALID_ARG, "causal_q must be >= 0");
    if (mask && mask_rows < 1) return fail(RWS_ERR_INVALID_ARG, "mask_rows must be >= 1");
    if (mask && (uintptr_t)mask % elem_size(dtype))
        return fail(RWS_ERR_MISALIGNED, "mask not aligned to the element size");
    if (rows == 0 || cols == 0) return RWS_OK;
    rws::MaskArgs M;
    M.scale = scale;
    M.mask = mask;
    M.mask_rows = mask ? mask_rows : 1;
    M.causal_q = causal_q;
    M.row_base = 0;
    return run(in, out, rows, cols, dtype, stream, kernel_id, &M);
}

// Softmax backward: family 1 (wave, registers), 2 (block, registers) or 3
// (stream, any length), chosen like the forward kernels by the row window.
struct BwdPlan {
    int family = 0;  // 1 wave, 2 block, 3 stream, RWS_KERNEL_SPLITK_ORDERED
    int variant = 0;
    int P = 1;       // ordered split-k: chunks per row
    bool aligned = false;
    bool same_phase = false;
    int lgrun = 0;
    int tile_t = 0;  // tile_rows: rows per tile
    int64_t max_rows = 0;
};

// allow_ordered: false when a captured call finds no tag buffer large enough
// (see capturing()); a request for the ordered form then plans as
// RWS_KERNEL_AUTO without it.
// dy16: dy is 16-byte aligned (the tile form needs y, dy and dx so).
static int plan_bwd(int64_t rows, int64_t cols, int dtype, const void* y, const void* dx,
                    bool dy16, int kernel_id, BwdPlan* bp, bool allow_ordered = true) {
    if (!allow_ordered && kernel_id == RWS_KERNEL_SPLITK_ORDERED) kernel_id = RWS_KERNEL_AUTO;
    const Geometry g = geometry(cols, dtype, y, dx);
    const int64_t wline = window_granules(g, 128);
    int family = kernel_id == RWS_KERNEL_AUTO ? 0 : kernel_id;  // 1 wave, 2 block, 3 stream, 6
    int variant = -1;
    bool aligned = g.a128;
    const int cus = device_info().cus;
    // Forms, by sweeps on MI355X with inputs in HBM: one wave per row while a
    // lane group holds the row at one granule per lane, else one workgroup
    // per row (fp16 [32768,1000]: 36.3 us with 192x1 against 76.1 us for one
    // wave per row with 4 granules per lane; [131072,480]: 76.8 us against
    // 88.6 with 2 per lane; shapes below), longer rows on 1024 threads; any
    // length streams.
    auto pick_wave = [&](int max_k) {
        int best = -1;
        int64_t best_cap = 0;
        for (int i = 0; i < rws::kNumBwdWave; ++i) {
            const rws::WaveRowVariant& v = rws::kBwdWave[i];
            if ((int64_t)v.G * v.K < window_granules(g, wave_row_wa(v)) || v.K > max_k) continue;
            if (best < 0 || (int64_t)v.G * v.K < best_cap) {
                best = i;
                best_cap = (int64_t)v.G * v.K;
            }
        }
        return best;
    };
    // Block shape: the smallest capacity that holds the row; at equal
    // capacity the one with more granules per thread (fewer waves per row).
    // Sweeps on MI355X (fp16, three tensors, inputs in HBM): [8192,4097]
    // 192x3 34.1 us against 576x1 37.3; [32768,1000] 64x3 33.6 against 192x1
    // 34.7; where one granule per thread fits exactly it wins ([8192,4096]
    // 512x1 32.8 against 256x2 33.5; [16384,2048] 256x1 33.3; [32768,1024]
    // 128x1 32.7), and [16384,2000] keeps 320x1 (32.9; 128x3 33.3, 64x5 34.0).
    auto pick_block = [&]() {
        int best = -1;
        int64_t best_key = 0;
        for (int i = 0; i < rws::kNumBwdBlock; ++i) {
            const int64_t cap = (int64_t)rws::kBwdBlock[i].block * rws::kBwdBlock[i].u;
            if (cap < wline) continue;
            const int64_t key = cap * 16 - rws::kBwdBlock[i].u;
            if (best < 0 || key < best_key) {
                best = i;
                best_key = key;
            }
        }
        return best;
    };
    if (family == 0) {
        if (dy16 && tile_rows_fits(rows, cols, dtype, y, dx)) family = RWS_KERNEL_TILE_ROWS;
        else if (pick_wave(1) >= 0) family = 1;
        else if (pick_block() >= 0) family = 2;
        else if (allow_ordered && few_long_rows(rows, wline, cus)) family = RWS_KERNEL_SPLITK_ORDERED;
        else family = 3;
    }
    if (family == RWS_KERNEL_TILE_ROWS) {
        if (!dy16 || (uintptr_t)y % 16 || (uintptr_t)dx % 16)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "tile_rows needs 16-byte aligned y, dy and dx");
        int T = 0;
        const int v = pick_tile_rows(rows, cols, elem_size(dtype), -1, &T);
        if (v < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "tile_rows takes rows of one granule to 1024 bytes");
        bp->family = family;
        bp->variant = v;
        bp->aligned = false;
        bp->same_phase = true;
        bp->lgrun = kTileLgRunBwd;
        bp->tile_t = T;
        bp->max_rows = (int64_t)T * ((int64_t)1 << 30);
        return RWS_OK;
    }
    if (family == RWS_KERNEL_SPLITK_ORDERED) {
        bp->family = family;
        bp->variant = 0;
        bp->P = ordered_chunks(wline, rws::kBwdOrderedBlock, rws::kBwdOrderedKc);
        bp->aligned = aligned;
        bp->same_phase = g.same_phase;
        bp->lgrun = 0;
        // at most 2^23 workgroups per launch, both stages counted
        bp->max_rows = std::max<int64_t>(1, ((int64_t)1 << 23) / (2LL * bp->P));
        return RWS_OK;
    }
    if (family == 1) {
        variant = pick_wave(1 << 30);
        if (variant < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "backward wave kernel holds at most 512 granules");
        aligned = wave_row_wa(rws::kBwdWave[variant]) == 128 ? g.a128 : g.a16;
    } else if (family == 2) {
        variant = pick_block();
        if (variant < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "backward block kernel holds at most 4096 granules");
    } else {
        variant = 0;
        for (int i = 0; i < rws::kNumBwdStream; ++i)
            if (rws::kBwdStream[i].block == (wline > 4096 ? 1024 : 256)) variant = i;
    }
    const int64_t max_rows = family == 1
        ? (int64_t)(64 / rws::kBwdWave[variant].G) * rws::kBwdWave[variant].U * 4 * ((int64_t)1 << 23)
        : block_rows_per_launch(family == 2 ? rws::kBwdBlock[variant].block
                                            : rws::kBwdStream[variant].block);
    bp->family = family;
    bp->variant = variant;
    bp->aligned = aligned;
    bp->same_phase = g.same_phase;
    bp->lgrun = family == 2 ? xcd_run_lg(g) : 0;
    bp->max_rows = max_rows;
    return RWS_OK;
}

int softmax_bwd_kernel(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols,
                       int dtype, void* stream, int kernel_id) {
    g_last_error.clear();
    if (kernel_id != RWS_KERNEL_AUTO && kernel_id != RWS_KERNEL_WAVE_ROW &&
        kernel_id != RWS_KERNEL_BLOCK_ONEPASS && kernel_id != RWS_KERNEL_TWO_PASS &&
        kernel_id != RWS_KERNEL_SPLITK_ORDERED && kernel_id != RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "backward kernels: auto, wave_row, block_onepass, "
                                         "two_pass, splitk_ordered, tile_rows");
    int st = check_args(y, dx, rows, cols, dtype, RWS_KERNEL_AUTO);
    if (st != RWS_OK || rows == 0 || cols == 0) return st;
    if (!dy) return fail(RWS_ERR_INVALID_ARG, "NULL dy with a non-empty tensor");
    if ((uintptr_t)dy % elem_size(dtype))
        return fail(RWS_ERR_MISALIGNED, "dy not aligned to the element size");
    const bool dy16 = (uintptr_t)dy % 16 == 0;
    BwdPlan bp;
    st = plan_bwd(rows, cols, dtype, y, dx, dy16, kernel_id, &bp);
    if (st != RWS_OK) return st;
    // ordered split-k: keep the tag words locked until the launches are enqueued
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    uint64_t* tags = nullptr;
    unsigned epoch = 0;
    int64_t tag_n = 0;  // captured: epochs come from tags[tag_n]
    uint64_t* status = nullptr;
    if (bp.family == RWS_KERNEL_SPLITK_ORDERED) {
        ws_lock.lock();
        const int64_t words = 2 * std::min(rows, bp.max_rows) * bp.P;
        if (capturing((hipStream_t)stream)) {
            if (!captured_tags((hipStream_t)stream, words, &tags, &tag_n)) {
                ws_lock.unlock();
                st = plan_bwd(rows, cols, dtype, y, dx, dy16, kernel_id, &bp, false);
                if (st != RWS_OK) return st;
            } else if ((st = get_status_word((hipStream_t)stream, true, &status)) != RWS_OK) {
                return st;
            }
        } else {
            const int64_t launches = (rows + bp.max_rows - 1) / bp.max_rows;
            st = get_tag_workspace((hipStream_t)stream, words, launches, &tags, &epoch);
            if (st != RWS_OK) return st;
            st = get_status_word((hipStream_t)stream, false, &status);
            if (st != RWS_OK) return st;
        }
    }
    const unsigned wait_limit = g_wait_limit.load(std::memory_order_relaxed);
    const int family = bp.family, variant = bp.variant;
    const int64_t max_rows = bp.max_rows;
    const int64_t row_bytes = cols * elem_size(dtype);
    for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
        rws::BwdLaunch B;
        B.rows = std::min<int64_t>(max_rows, rows - r0);
        B.y = (const char*)y + r0 * row_bytes;
        B.dy = (const char*)dy + r0 * row_bytes;
        B.dx = (char*)dx + r0 * row_bytes;
        B.cols = (int)cols;
        B.dtype = dtype;
        B.aligned = bp.aligned;
        B.same_phase = bp.same_phase;
        B.dy_vec = (((uintptr_t)dy - (uintptr_t)y) % 16) == 0;
        B.lgrun = bp.lgrun;
        B.stream = (hipStream_t)stream;
        hipError_t e = hipSuccess;
        if (family == RWS_KERNEL_TILE_ROWS)
            e = rws::launch_bwd_tile(B, variant, rws::TileShape{bp.tile_t, bp.lgrun});
        else if (family != RWS_KERNEL_SPLITK_ORDERED)
            e = rws::launch_bwd(B, family, variant);
        else if (tag_n == 0)
            e = rws::launch_bwd_ordered(
                B, bp.P,
                rws::OrderedSync{tags, epoch + (unsigned)(r0 / max_rows), nullptr, status,
                                 wait_limit});
        else if ((e = rws::launch_bump_epoch(tags, tag_n, B.stream)) == hipSuccess)
            e = rws::launch_bwd_ordered(
                B, bp.P, rws::OrderedSync{tags, 0, tags + tag_n, status, wait_limit});
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("backward launch: ") + hipGetErrorString(e));
    }
    return RWS_OK;
}

int softmax_bwd(const void* y, const void* dy, void* dx, int64_t rows, int64_t cols, int dtype,
                void* stream) {
    return softmax_bwd_kernel(y, dy, dx, rows, cols, dtype, stream, RWS_KERNEL_AUTO);
}

// Row normalisations: family 1 (norm_wave), 2 (norm_block) or 3
// (norm_stream), chosen by the row window like the softmax backward.
struct NormPlan {
    int family = 0;  // 1 wave, 2 block, 3 stream, RWS_KERNEL_SPLITK_ORDERED
    int variant = 0;
    int P = 1;       // ordered split-k: chunks per row
    bool aligned = false;
    bool same_phase = false;
    int lgrun = 0;
    int tile_t = 0;  // tile_rows: rows per tile
    int64_t max_rows = 0;
};

// allow_ordered: as for plan_bwd.
static int plan_norm(int64_t rows, int64_t cols, int dtype, const void* in, const void* out,
                     bool affine, int kernel_id, NormPlan* np, bool allow_ordered = true) {
    if (!allow_ordered && kernel_id == RWS_KERNEL_SPLITK_ORDERED) kernel_id = RWS_KERNEL_AUTO;
    const Geometry g = geometry(cols, dtype, in, out);
    const int64_t wline = window_granules(g, 128);
    // Lane groups measured on MI355X (fp16 LayerNorm / RMSNorm, rotating
    // buffers): windows of 9-32 granules take (16,2,1) ([131040,192]: 17.9 us,
    // (8,3,1) 18.3 us, (32,1,1) 21.5 us), windows of 33-48 take (8,6,1)
    // ([32760,384]: 9.0 us, (16,3,1) 10.2 us, (64,1,1) 11.4 us); other
    // lengths the narrowest group that holds the window.  With weight and/or
    // bias the affine loads shift the balance to fewer rows per wave:
    // windows of 17-24 take (8,3,1) (LayerNorm [131040,192] 19.5 us against
    // 21.1 with (16,2,1); RMSNorm 18.7 either way) and 33-48 take (16,3,1)
    // ([32760,384] LayerNorm 11.9 us against 12.7 with (8,6,1), RMSNorm 11.0
    // against 11.3).
    auto norm_variant = [&](int G, int K, int U) {
        for (int i = 0; i < rws::kNumNormWave; ++i) {
            const rws::WaveRowVariant& v = rws::kNormWave[i];
            if (v.G == G && v.K == K && v.U == U &&
                (int64_t)G * K >= window_granules(g, wave_row_wa(v)))
                return i;
        }
        return -1;
    };
    // max_k limits the granules per lane of the other groups; the tuned
    // groups are taken for their windows whatever it is.
    auto pick_wave = [&](int max_k) {
        if (affine && wline > 16 && wline <= 24 && norm_variant(8, 3, 1) >= 0)
            return norm_variant(8, 3, 1);
        if (affine && wline > 32 && wline <= 48 && norm_variant(16, 3, 1) >= 0)
            return norm_variant(16, 3, 1);
        if (wline > 8 && wline <= 32 && norm_variant(16, 2, 1) >= 0) return norm_variant(16, 2, 1);
        if (wline > 32 && wline <= 48 && norm_variant(8, 6, 1) >= 0) return norm_variant(8, 6, 1);
        int best = -1;
        int64_t best_key = 0;
        for (int i = 0; i < rws::kNumNormWave; ++i) {
            const rws::WaveRowVariant& v = rws::kNormWave[i];
            const int64_t cap = (int64_t)v.G * v.K;
            if (cap < window_granules(g, wave_row_wa(v)) || v.K > max_k) continue;
            const int64_t key = cap * 64 + v.U;
            if (best < 0 || key < best_key) {
                best = i;
                best_key = key;
            }
        }
        return best;
    };
    auto pick_block = [&]() {
        return pick_block_shape(
            rws::kNumNormBlock,
            [](int i) { return BlockShape{rws::kNormBlock[i].block, rws::kNormBlock[i].u, 0}; },
            wline, rows, device_info().cus);
    };
    // Forms: the tuned lane groups above, or one wave per row while a lane
    // group holds the row at one granule per lane; else one workgroup per row
    // in the forward softmax's shapes (one wave per row with 4 or 8 granules
    // per lane measured 1.7-2.2x slower than even one granule per thread:
    // LayerNorm fp16 [32768,1000] 54.5 us against 32.9 with 192x1,
    // [16384,2000] 43.9 against 30.1 with 320x1, [8192,4000] 28.8 against 25.0
    // with 512x1); any length streams.
    int family = kernel_id == RWS_KERNEL_AUTO ? 0 : kernel_id;
    if (family == 0) {
        if (!affine && tile_rows_fits(rows, cols, dtype, in, out)) family = RWS_KERNEL_TILE_ROWS;
        else if (pick_wave(1) >= 0) family = 1;
        else if (pick_block() >= 0) family = 2;
        else if (allow_ordered && few_long_rows(rows, wline, device_info().cus))
            family = RWS_KERNEL_SPLITK_ORDERED;
        else family = 3;
    }
    if (family == RWS_KERNEL_TILE_ROWS) {
        if (affine)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "the tile_rows normalisation takes no weight or bias");
        if ((uintptr_t)in % 16 || (uintptr_t)out % 16)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "tile_rows needs 16-byte aligned in and out");
        int T = 0;
        const int v = pick_tile_rows(rows, cols, elem_size(dtype), -1, &T);
        if (v < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "tile_rows takes rows of one granule to 1024 bytes");
        np->family = family;
        np->variant = v;
        np->aligned = false;
        np->same_phase = true;
        np->lgrun = kTileLgRunNorm;
        np->tile_t = T;
        np->max_rows = (int64_t)T * ((int64_t)1 << 30);
        return RWS_OK;
    }
    if (family == RWS_KERNEL_SPLITK_ORDERED) {
        np->family = family;
        np->variant = 0;
        np->P = ordered_chunks(wline, rws::kNormOrderedBlock, rws::kNormOrderedKc);
        np->aligned = g.a128;
        np->same_phase = g.same_phase;
        np->lgrun = 0;
        // at most 2^23 workgroups per launch, both stages counted
        np->max_rows = std::max<int64_t>(1, ((int64_t)1 << 23) / (2LL * np->P));
        return RWS_OK;
    }
    int variant = -1;
    bool aligned = g.a128;
    if (family == 1) {
        // the dispatcher's choice takes one granule per lane (or a tuned
        // group); a forced wave form takes any group that holds the row
        variant = pick_wave(kernel_id == RWS_KERNEL_AUTO ? 1 : 1 << 30);
        if (variant < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "normalisation wave kernel holds at most 512 granules");
        // with weight or bias, rows 16-byte aligned take row-start windows
        // whatever the group (as the block form below)
        aligned = wave_row_wa(rws::kNormWave[variant]) == 128 && !affine ? g.a128 : g.a16;
    } else if (family == 2) {
        variant = pick_block();
        if (variant < 0)
            return fail(RWS_ERR_UNSUPPORTED_SHAPE, "normalisation block kernel holds at most 4096 granules");
        // Rows 16-byte aligned but not line-aligned, with weight or bias:
        // windows start at the row (not its line), so the weight and bias at
        // the rows' phase take the phase-matched form, which drops the
        // element fallback and its registers.  fp16 LayerNorm with weight and
        // bias: [32768,1000] 26.8 us against 31.9, [16384,2000] 27.6 against
        // 32.9, [8192,4000] 27.4 against 28.5; RMSNorm [32768,1000] 24.8
        // against 26.9.
        if (affine && g.a16) aligned = true;
    } else {
        variant = 0;
        for (int i = 0; i < rws::kNumNormStream; ++i)
            if (rws::kNormStream[i].block == (wline > 4096 ? 1024 : 256)) variant = i;
    }
    const int64_t max_rows = family == 1
        ? (int64_t)(64 / rws::kNormWave[variant].G) * rws::kNormWave[variant].U * 4 * ((int64_t)1 << 23)
        : block_rows_per_launch(family == 2 ? rws::kNormBlock[variant].block
                                            : rws::kNormStream[variant].block);
    np->family = family;
    np->variant = variant;
    np->aligned = aligned;
    np->same_phase = g.same_phase;
    np->lgrun = 0;
    np->max_rows = max_rows;
    return RWS_OK;
}

static int norm_run(int mode, const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                    float eps, const void* weight, const void* bias, float* mean, float* rstd,
                    void* stream, int kernel_id) {
    g_last_error.clear();
    if (kernel_id != RWS_KERNEL_AUTO && kernel_id != RWS_KERNEL_WAVE_ROW &&
        kernel_id != RWS_KERNEL_BLOCK_ONEPASS && kernel_id != RWS_KERNEL_TWO_PASS &&
        kernel_id != RWS_KERNEL_SPLITK_ORDERED && kernel_id != RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "normalisation kernels: auto, wave_row, block_onepass, "
                                         "two_pass, splitk_ordered, tile_rows");
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(RWS_ERR_INVALID_ARG, "eps must be finite and >= 0");
    int st = check_args(in, out, rows, cols, dtype, RWS_KERNEL_AUTO);
    if (st != RWS_OK || rows == 0 || cols == 0) return st;
    const int es = elem_size(dtype);
    if ((uintptr_t)weight % es || (uintptr_t)bias % es)
        return fail(RWS_ERR_MISALIGNED, "weight/bias not aligned to the element size");
    if ((uintptr_t)mean % 4 || (uintptr_t)rstd % 4)
        return fail(RWS_ERR_MISALIGNED, "mean/rstd not aligned to 4 bytes");
    NormPlan np;
    st = plan_norm(rows, cols, dtype, in, out, weight || bias, kernel_id, &np);
    if (st != RWS_OK) return st;
    // ordered split-k: keep the tag words locked until the launches are enqueued
    std::unique_lock<std::mutex> ws_lock(g_ws_mu, std::defer_lock);
    uint64_t* tags = nullptr;
    unsigned epoch = 0;
    int64_t tag_n = 0;  // captured: epochs come from tags[tag_n]
    uint64_t* status = nullptr;
    if (np.family == RWS_KERNEL_SPLITK_ORDERED) {
        ws_lock.lock();
        const int64_t words = 2 * std::min(rows, np.max_rows) * np.P;
        if (capturing((hipStream_t)stream)) {
            if (!captured_tags((hipStream_t)stream, words, &tags, &tag_n)) {
                ws_lock.unlock();
                st = plan_norm(rows, cols, dtype, in, out, weight || bias, kernel_id, &np, false);
                if (st != RWS_OK) return st;
            } else if ((st = get_status_word((hipStream_t)stream, true, &status)) != RWS_OK) {
                return st;
            }
        } else {
            const int64_t launches = (rows + np.max_rows - 1) / np.max_rows;
            st = get_tag_workspace((hipStream_t)stream, words, launches, &tags, &epoch);
            if (st != RWS_OK) return st;
            st = get_status_word((hipStream_t)stream, false, &status);
            if (st != RWS_OK) return st;
        }
    }
    const unsigned wait_limit = g_wait_limit.load(std::memory_order_relaxed);
    const int family = np.family, variant = np.variant;
    const int64_t max_rows = np.max_rows;
    const int64_t row_bytes = cols * es;
    for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
        rws::NormLaunch L;
        L.rows = std::min<int64_t>(max_rows, rows - r0);
        L.in = (const char*)in + r0 * row_bytes;
        L.out = (char*)out + r0 * row_bytes;
        L.cols = (int)cols;
        L.dtype = dtype;
        L.mode = mode;
        L.aligned = np.aligned;
        L.same_phase = np.same_phase;
        L.lgrun = np.lgrun;
        // aligned rows start at in's 16-byte phase; so do w and b when
        // their offset from in is a multiple of 16 bytes
        L.aff_matched = np.aligned &&
                        (!weight || ((uintptr_t)weight - (uintptr_t)in) % 16 == 0) &&
                        (!bias || ((uintptr_t)bias - (uintptr_t)in) % 16 == 0);
        L.args.w = weight;
        L.args.b = bias;
        L.args.mean = mean ? mean + r0 : nullptr;
        L.args.rstd = rstd ? rstd + r0 : nullptr;
        L.args.eps = eps;
        L.args.n = (float)cols;
        L.stream = (hipStream_t)stream;
        hipError_t e = hipSuccess;
        if (family == RWS_KERNEL_TILE_ROWS)
            e = rws::launch_norm_tile(L, variant, rws::TileShape{np.tile_t, np.lgrun});
        else if (family == 1)
            e = rws::launch_norm_wave(L, variant);
        else if (family != RWS_KERNEL_SPLITK_ORDERED)
            e = rws::launch_norm_block(L, family, variant);
        else if (tag_n == 0)
            e = rws::launch_norm_ordered(
                L, np.P,
                rws::OrderedSync{tags, epoch + (unsigned)(r0 / max_rows), nullptr, status,
                                 wait_limit});
        else if ((e = rws::launch_bump_epoch(tags, tag_n, L.stream)) == hipSuccess)
            e = rws::launch_norm_ordered(
                L, np.P, rws::OrderedSync{tags, 0, tags + tag_n, status, wait_limit});
        if (e != hipSuccess)
            return fail(RWS_ERR_HIP, std::string("normalisation launch: ") + hipGetErrorString(e));
    }
    return RWS_OK;
}

int layernorm_fwd_kernel(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                         float eps, const void* weight, const void* bias, float* mean, float* rstd,
                         void* stream, int kernel_id) {
    return norm_run(rws::kLayerNorm, in, out, rows, cols, dtype, eps, weight, bias, mean, rstd,
                    stream, kernel_id);
}

int layernorm_fwd(const void* in, void* out, int64_t rows, int64_t cols, int dtype, float eps,
                  const void* weight, const void* bias, float* mean, float* rstd, void* stream) {
    return layernorm_fwd_kernel(in, out, rows, cols, dtype, eps, weight, bias, mean, rstd, stream,
                                RWS_KERNEL_AUTO);
}

int rmsnorm_fwd_kernel(const void* in, void* out, int64_t rows, int64_t cols, int dtype, float eps,
                       const void* weight, float* rstd, void* stream, int kernel_id) {
    return norm_run(rws::kRmsNorm, in, out, rows, cols, dtype, eps, weight, nullptr, nullptr, rstd,
                    stream, kernel_id);
}

int rmsnorm_fwd(const void* in, void* out, int64_t rows, int64_t cols, int dtype, float eps,
                const void* weight, float* rstd, void* stream) {
    return rmsnorm_fwd_kernel(in, out, rows, cols, dtype, eps, weight, rstd, stream, RWS_KERNEL_AUTO);
}

int softmax_fwd(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    return softmax_fwd_kernel(in, out, rows, cols, dtype, stream, RWS_KERNEL_AUTO);
}

int softmax_select_kernel(int64_t rows, int64_t cols, int dtype, const void* in, const void* out) {
    g_last_error.clear();
    if (dtype != RWS_F32 && dtype != RWS_F16 && dtype != RWS_BF16) return -RWS_ERR_UNSUPPORTED_DTYPE;
    if (rows < 0 || cols < 0) return -RWS_ERR_INVALID_ARG;
    if (cols > kMaxCols) return -RWS_ERR_UNSUPPORTED_SHAPE;
    if (rows == 0 || cols == 0) return RWS_KERNEL_WAVE_ROW;  // nothing runs
    Plan p;
    const int st = plan_launch(rows, cols, dtype, in, out, RWS_KERNEL_AUTO, &p);
    return st == RWS_OK ? p.family : -st;
}

static int describe_launch(int64_t rows, int64_t cols, int dtype, const void* in, const void* out,
                           int kernel_id, bool masked, char* buf, int64_t buflen,
                           int forced_variant = -1) {
    g_last_error.clear();
    if (!buf || buflen <= 0) return fail(RWS_ERR_INVALID_ARG, "no output buffer");
    buf[0] = 0;
    if (dtype != RWS_F32 && dtype != RWS_F16 && dtype != RWS_BF16)
        return fail(RWS_ERR_UNSUPPORTED_DTYPE, "dtype must be RWS_F32, RWS_F16 or RWS_BF16");
    if (kernel_id < RWS_KERNEL_AUTO || kernel_id > RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "unknown kernel id " + std::to_string(kernel_id));
    if (rows < 0 || cols < 0) return fail(RWS_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols > kMaxCols) return fail(RWS_ERR_UNSUPPORTED_SHAPE, "cols above 2^30");
    if (rows == 0 || cols == 0) {
        std::snprintf(buf, (size_t)buflen, "empty: no launch");
        return RWS_OK;
    }
    Plan p;
    const int st = plan_launch(rows, cols, dtype, in, out, kernel_id, &p, masked, forced_variant);
    if (st != RWS_OK) return st;
    const char* al = p.aligned ? "aligned" : (p.same_phase ? "unaligned" : "unaligned,split-phase");
    const int64_t wmax = p.window;
    char run[32] = "";
    if (p.lgrun > 0) std::snprintf(run, sizeof run, " xcd_run=%d", 1 << p.lgrun);
    switch (p.family) {
        case RWS_KERNEL_TILE_ROWS: {
            const rws::TileRowsVariant& v = rws::kTileRows[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "tile_rows<%s,T=%d,K=%d> grid=%lld block=64 granules<=%lld%s",
                          dtype_name(dtype), p.tile_t, v.K,
                          (long long)((std::min(rows, p.max_rows_per_launch) + p.tile_t - 1) /
                                      p.tile_t),
                          (long long)wmax, run);
            break;
        }
        case RWS_KERNEL_WAVE_ROW: {
            const rws::WaveRowVariant& v = rws::kWaveRow[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "wave_row<%s,%s,G=%d,K=%d,U=%d> grid=%lld block=%d window<=%lld%s",
                          dtype_name(dtype), al, v.G, v.K, v.U,
                          (long long)rws::wave_row_grid(v, std::min(rows, p.max_rows_per_launch)),
                          rws::kWaveGroupThreads, (long long)wmax, p.wt ? " store=wt" : "");
            break;
        }
        case RWS_KERNEL_BLOCK_ONEPASS: {
            const rws::OnepassVariant& v = rws::kOnepass[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "block_onepass<%s,%s,B=%d,KR=%d,KL=%d> grid=%lld block=%d window<=%lld%s",
                          dtype_name(dtype), al, v.block, v.kr, v.kl,
                          (long long)std::min(rows, p.max_rows_per_launch), v.block, (long long)wmax,
                          run);
            break;
        }
        case RWS_KERNEL_TWO_PASS: {
            const rws::TwoPassVariant& v = rws::kTwoPass[p.variant];
            std::snprintf(buf, (size_t)buflen, "two_pass<%s,%s,B=%d,U=%d> grid=%lld block=%d window<=%lld",
                          dtype_name(dtype), al, v.block, v.u,
                          (long long)std::min(rows, p.max_rows_per_launch), v.block, (long long)wmax);
            break;
        }
        case RWS_KERNEL_SPLITK_FUSED: {
            const rws::SplitkVariant& v = rws::kSplitkFused[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "splitk_fused<%s,%s,B=%d,KC=%d> P=%d grid=%lld block=%d window<=%lld",
                          dtype_name(dtype), al, v.block, v.kc, p.P,
                          (long long)(std::min(rows, p.max_rows_per_launch) * p.P), v.block,
                          (long long)wmax);
            break;
        }
        case RWS_KERNEL_SPLITK: {
            const rws::SplitkVariant& v = rws::kSplitk[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "splitk<%s,%s,B=%d,KC=%d> P=%d grid=%lld x2 block=%d window<=%lld",
                          dtype_name(dtype), al, v.block, v.kc, p.P,
                          (long long)(std::min(rows, p.max_rows_per_launch) * p.P), v.block,
                          (long long)wmax);
            break;
        }
        case RWS_KERNEL_SPLITK_ORDERED: {
            const rws::SplitkVariant& v = rws::kSplitk[p.variant];
            std::snprintf(buf, (size_t)buflen,
                          "splitk_ordered<%s,%s,B=%d,KC=%d> P=%d grid=%lld (2 stages) block=%d "
                          "window<=%lld",
                          dtype_name(dtype), al, v.block, v.kc, p.P,
                          (long long)(2 * std::min(rows, p.max_rows_per_launch) * p.P), v.block,
                          (long long)wmax);
            break;
        }
    }
    return RWS_OK;
}

int softmax_describe_launch(int64_t rows, int64_t cols, int dtype, const void* in,
                            const void* out, int kernel_id, char* buf, int64_t buflen) {
    return describe_launch(rows, cols, dtype, in, out, kernel_id, false, buf, buflen);
}

int softmax_describe_launch_masked(int64_t rows, int64_t cols, int dtype, const void* in,
                                   const void* out, int kernel_id, char* buf, int64_t buflen) {
    return describe_launch(rows, cols, dtype, in, out, kernel_id, true, buf, buflen);
}

int softmax_describe_variant(int64_t rows, int64_t cols, int dtype, const void* in,
                             const void* out, int kernel_id, int variant, char* buf,
                             int64_t buflen) {
    if (kernel_id == RWS_KERNEL_AUTO || variant < 0) {
        g_last_error.clear();
        if (buf && buflen > 0) buf[0] = 0;
        return fail(RWS_ERR_INVALID_ARG, "a variant needs a kernel family and an index >= 0");
    }
    return describe_launch(rows, cols, dtype, in, out, kernel_id, false, buf, buflen, variant);
}

int softmax_variant_count(int kernel_id) {
    switch (kernel_id) {
        case RWS_KERNEL_WAVE_ROW: return rws::kNumWaveRow;
        case RWS_KERNEL_BLOCK_ONEPASS: return rws::kNumOnepass;
        case RWS_KERNEL_TWO_PASS: return rws::kNumTwoPass;
        case RWS_KERNEL_SPLITK:
        case RWS_KERNEL_SPLITK_ORDERED: return rws::kNumSplitk;
        case RWS_KERNEL_SPLITK_FUSED: return rws::kNumSplitkFused;
        case RWS_KERNEL_TILE_ROWS: return rws::kNumTileRows;
    }
    return 0;
}

int softmax_fwd_variant(const void* in, void* out, int64_t rows, int64_t cols, int dtype,
                        void* stream, int kernel_id, int variant) {
    g_last_error.clear();
    if (kernel_id == RWS_KERNEL_AUTO || variant < 0)
        return fail(RWS_ERR_INVALID_ARG, "a variant needs a kernel family and an index >= 0");
    const int st = check_args(in, out, rows, cols, dtype, kernel_id);
    if (st != RWS_OK || rows == 0 || cols == 0) return st;
    return run(in, out, rows, cols, dtype, stream, kernel_id, nullptr, variant);
}

int softmax_bwd_describe_launch(int64_t rows, int64_t cols, int dtype, const void* y,
                                const void* dx, int kernel_id, char* buf, int64_t buflen) {
    g_last_error.clear();
    if (!buf || buflen <= 0) return fail(RWS_ERR_INVALID_ARG, "no output buffer");
    buf[0] = 0;
    if (kernel_id != RWS_KERNEL_AUTO && kernel_id != RWS_KERNEL_WAVE_ROW &&
        kernel_id != RWS_KERNEL_BLOCK_ONEPASS && kernel_id != RWS_KERNEL_TWO_PASS &&
        kernel_id != RWS_KERNEL_SPLITK_ORDERED && kernel_id != RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "backward kernels: auto, wave_row, block_onepass, "
                                         "two_pass, splitk_ordered, tile_rows");
    if (dtype != RWS_F32 && dtype != RWS_F16 && dtype != RWS_BF16)
        return fail(RWS_ERR_UNSUPPORTED_DTYPE, "dtype must be RWS_F32, RWS_F16 or RWS_BF16");
    if (rows < 0 || cols < 0) return fail(RWS_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols > kMaxCols) return fail(RWS_ERR_UNSUPPORTED_SHAPE, "cols above 2^30");
    if (rows == 0 || cols == 0) {
        std::snprintf(buf, (size_t)buflen, "empty: no launch");
        return RWS_OK;
    }
    // dy is taken to share y's 16-byte alignment
    BwdPlan bp;
    const int st = plan_bwd(rows, cols, dtype, y, dx, (uintptr_t)y % 16 == 0, kernel_id, &bp);
    if (st != RWS_OK) return st;
    const char* al = bp.aligned ? "aligned" : (bp.same_phase ? "unaligned" : "unaligned,split-phase");
    const int64_t r = std::min(rows, bp.max_rows);
    if (bp.family == RWS_KERNEL_TILE_ROWS) {
        const rws::TileRowsVariant& v = rws::kTileRows[bp.variant];
        std::snprintf(buf, (size_t)buflen, "bwd_tile<%s,T=%d,K=%d> grid=%lld block=64 xcd_run=%d",
                      dtype_name(dtype), bp.tile_t, v.K, (long long)((r + bp.tile_t - 1) / bp.tile_t),
                      1 << bp.lgrun);
    } else if (bp.family == RWS_KERNEL_SPLITK_ORDERED) {
        std::snprintf(buf, (size_t)buflen,
                      "bwd_ordered<%s,%s,B=%d,KC=%d> P=%d grid=%lld (2 stages) block=%d",
                      dtype_name(dtype), al, rws::kBwdOrderedBlock, rws::kBwdOrderedKc, bp.P,
                      (long long)(2 * r * bp.P), rws::kBwdOrderedBlock);
    } else if (bp.family == 1) {
        const rws::WaveRowVariant& v = rws::kBwdWave[bp.variant];
        std::snprintf(buf, (size_t)buflen, "bwd_wave<%s,%s,G=%d,K=%d,U=%d> grid=%lld block=%d",
                      dtype_name(dtype), al, v.G, v.K, v.U, (long long)rws::wave_row_grid(v, r),
                      rws::kWaveGroupThreads);
    } else {
        const rws::TwoPassVariant& v =
            bp.family == 2 ? rws::kBwdBlock[bp.variant] : rws::kBwdStream[bp.variant];
        char run[32] = "";
        if (bp.lgrun > 0) std::snprintf(run, sizeof run, " xcd_run=%d", 1 << bp.lgrun);
        std::snprintf(buf, (size_t)buflen, "%s<%s,%s,B=%d,%s=%d> grid=%lld block=%d%s",
                      bp.family == 2 ? "bwd_block" : "bwd_stream", dtype_name(dtype), al, v.block,
                      bp.family == 2 ? "KR" : "U", v.u, (long long)r, v.block, run);
    }
    return RWS_OK;
}

int norm_describe_launch(int64_t rows, int64_t cols, int dtype, const void* in, const void* out,
                         int affine, int kernel_id, char* buf, int64_t buflen) {
    g_last_error.clear();
    if (!buf || buflen <= 0) return fail(RWS_ERR_INVALID_ARG, "no output buffer");
    buf[0] = 0;
    if (kernel_id != RWS_KERNEL_AUTO && kernel_id != RWS_KERNEL_WAVE_ROW &&
        kernel_id != RWS_KERNEL_BLOCK_ONEPASS && kernel_id != RWS_KERNEL_TWO_PASS &&
        kernel_id != RWS_KERNEL_SPLITK_ORDERED && kernel_id != RWS_KERNEL_TILE_ROWS)
        return fail(RWS_ERR_INVALID_ARG, "normalisation kernels: auto, wave_row, block_onepass, "
                                         "two_pass, splitk_ordered, tile_rows");
    if (dtype != RWS_F32 && dtype != RWS_F16 && dtype != RWS_BF16)
        return fail(RWS_ERR_UNSUPPORTED_DTYPE, "dtype must be RWS_F32, RWS_F16 or RWS_BF16");
    if (rows < 0 || cols < 0) return fail(RWS_ERR_INVALID_ARG, "rows and cols must be >= 0");
    if (cols > kMaxCols) return fail(RWS_ERR_UNSUPPORTED_SHAPE, "cols above 2^30");
    if (rows == 0 || cols == 0) {
        std::snprintf(buf, (size_t)buflen, "empty: no launch");
        return RWS_OK;
    }
    NormPlan np;
    const int st = plan_norm(rows, cols, dtype, in, out, affine != 0, kernel_id, &np);
    if (st != RWS_OK) return st;
    const char* al = np.aligned ? "aligned" : (np.same_phase ? "unaligned" : "unaligned,split-phase");
    const int64_t r = std::min(rows, np.max_rows);
    const long long wline = (long long)window_granules(geometry(cols, dtype, in, out), 128);
    if (np.family == RWS_KERNEL_TILE_ROWS) {
        const rws::TileRowsVariant& v = rws::kTileRows[np.variant];
        std::snprintf(buf, (size_t)buflen, "norm_tile<%s,T=%d,K=%d> grid=%lld block=64 xcd_run=%d",
                      dtype_name(dtype), np.tile_t, v.K, (long long)((r + np.tile_t - 1) / np.tile_t),
                      1 << np.lgrun);
    } else if (np.family == RWS_KERNEL_SPLITK_ORDERED) {
        std::snprintf(buf, (size_t)buflen,
                      "norm_ordered<%s,%s,B=%d,KC=%d> P=%d grid=%lld (2 stages) block=%d",
                      dtype_name(dtype), al, rws::kNormOrderedBlock, rws::kNormOrderedKc, np.P,
                      (long long)(2 * r * np.P), rws::kNormOrderedBlock);
    } else if (np.family == 1) {
        const rws::WaveRowVariant& v = rws::kNormWave[np.variant];
        std::snprintf(buf, (size_t)buflen, "norm_wave<%s,%s,G=%d,K=%d,U=%d> grid=%lld block=%d",
                      dtype_name(dtype), al, v.G, v.K, v.U, (long long)rws::wave_row_grid(v, r),
                      rws::kWaveGroupThreads);
    } else {
        const rws::TwoPassVariant& v =
            np.family == 2 ? rws::kNormBlock[np.variant] : rws::kNormStream[np.variant];
        char run[32] = "";
        if (np.lgrun > 0) std::snprintf(run, sizeof run, " xcd_run=%d", 1 << np.lgrun);
        std::snprintf(buf, (size_t)buflen, "%s<%s,%s,B=%d,%s=%d> grid=%lld block=%d window<=%lld%s",
                      np.family == 2 ? "norm_block" : "norm_stream", dtype_name(dtype), al, v.block,
                      np.family == 2 ? "KR" : "U", v.u, (long long)r, v.block, wline, run);
    }
    return RWS_OK;
}

const char* softmax_kernel_name(int kernel_id) {
    switch (kernel_id) {
        case RWS_KERNEL_AUTO: return "auto";
        case RWS_KERNEL_WAVE_ROW: return "wave_row";
        case RWS_KERNEL_BLOCK_ONEPASS: return "block_onepass";
        case RWS_KERNEL_TWO_PASS: return "two_pass";
        case RWS_KERNEL_SPLITK: return "splitk";
        case RWS_KERNEL_SPLITK_FUSED: return "splitk_fused";
        case RWS_KERNEL_SPLITK_ORDERED: return "splitk_ordered";
        case RWS_KERNEL_TILE_ROWS: return "tile_rows";
    }
    return "unknown";
}

const char* softmax_status_string(int status) {
    switch (status) {
        case RWS_OK: return "ok";
        case RWS_ERR_INVALID_ARG: return "invalid argument";
        case RWS_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
        case RWS_ERR_MISALIGNED: return "pointer misaligned for its element size";
        case RWS_ERR_HIP: return "HIP runtime error";
        case RWS_ERR_UNSUPPORTED_SHAPE: return "shape not supported by the requested kernel";
        case RWS_ERR_WAIT_TIMEOUT:
            return "a single-launch split-k wait gave up; its outputs are NaN";
    }
    return "unknown status";
}

const char* softmax_last_error(void) { return g_last_error.c_str(); }

int softmax_set_wait_limit(int64_t tries) {
    g_last_error.clear();
    if (tries > (int64_t)0xffffffffu) return fail(RWS_ERR_INVALID_ARG, "tries above 2^32 - 1");
    g_wait_limit.store(tries < 0 ? rws::kOrderedSpinLimit : (unsigned)tries,
                       std::memory_order_relaxed);
    return RWS_OK;
}

int softmax_stream_status(void* stream) {
    g_last_error.clear();
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    uint64_t* status = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mu);
        if (g_ws) {
            auto it = g_ws->find(std::make_pair(dev, (hipStream_t)stream));
            if (it != g_ws->end()) status = it->second.status;
        }
    }
    if (!status) return RWS_OK;  // no single-launch split-k call on this stream yet
    e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess)
        return fail(RWS_ERR_HIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    uint64_t v = 0;
    e = hipMemcpy(&v, status, sizeof v, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v != 0) {
        // clear it for the next query (a kernel on the stream, then wait)
        e = rws::launch_fill_words(status, 1, 0, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    }
    if (e != hipSuccess)
        return fail(RWS_ERR_HIP, std::string("status word: ") + hipGetErrorString(e));
    if (v & rws::kStatusLate)
        return fail(RWS_ERR_WAIT_TIMEOUT,
                    "a workgroup of a single-launch split-k call on this stream gave up waiting "
                    "for its row's partials and wrote NaN (workgroups were not dispatched in "
                    "index order, or the wait limit is set too low)");
    return RWS_OK;
}

int softmax_copy_bytes(const void* in, void* out, int64_t bytes, void* stream) {
    g_last_error.clear();
    if (bytes < 0) return fail(RWS_ERR_INVALID_ARG, "bytes must be >= 0");
    if (bytes == 0) return RWS_OK;
    if (!in || !out) return fail(RWS_ERR_INVALID_ARG, "NULL pointer");
    if ((uintptr_t)in % 16 || (uintptr_t)out % 16 || bytes % 16)
        return fail(RWS_ERR_MISALIGNED, "copy needs 16-byte aligned pointers and size");
    hipError_t e = rws::launch_copy16(in, out, bytes / 16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("copy launch: ") + hipGetErrorString(e));
    return RWS_OK;
}

int softmax_read_bytes(const void* in, int64_t bytes, void* stream) {
    g_last_error.clear();
    if (bytes < 0) return fail(RWS_ERR_INVALID_ARG, "bytes must be >= 0");
    if (bytes == 0) return RWS_OK;
    if (!in) return fail(RWS_ERR_INVALID_ARG, "NULL pointer");
    if ((uintptr_t)in % 16 || bytes % 16)
        return fail(RWS_ERR_MISALIGNED, "read needs a 16-byte aligned pointer and size");
    hipError_t e = rws::launch_read16(in, bytes / 16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("read launch: ") + hipGetErrorString(e));
    return RWS_OK;
}

int softmax_write_bytes(void* out, int64_t bytes, void* stream) {
    g_last_error.clear();
    if (bytes < 0) return fail(RWS_ERR_INVALID_ARG, "bytes must be >= 0");
    if (bytes == 0) return RWS_OK;
    if (!out) return fail(RWS_ERR_INVALID_ARG, "NULL pointer");
    if ((uintptr_t)out % 16 || bytes % 16)
        return fail(RWS_ERR_MISALIGNED, "write needs a 16-byte aligned pointer and size");
    hipError_t e = rws::launch_write16(out, bytes / 16, (hipStream_t)stream);
    if (e != hipSuccess) return fail(RWS_ERR_HIP, std::string("write launch: ") + hipGetErrorString(e));
    return RWS_OK;
}

}  // extern "C"
