// rws_launch.hpp -- host-side interface between the C ABI / dispatcher
// (rws_api.cpp) and the kernel translation units.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rws {

// One launch of a kernel family over `rows` rows starting at in/out.
struct Launch {
    const void* in;
    void* out;
    int64_t rows;
    int cols;
    int dtype;        // kF32 / kF16 / kBF16
    bool aligned;     // in, out 128-byte aligned and cols*size % 128 == 0
    bool same_phase;  // (in - out) % 16 == 0
    bool wt = false;  // wave_row: line-aligned rows, write-through stores
    int lgrun = 0;    // one-row-per-workgroup kernels: XCD runs of 2^lgrun rows
    hipStream_t stream;
};

// Attention-score prologue of the masked entry point: z = scale*x + mask
// (+ causal limit), see rws_pre.hpp.  row_base is the global index of the
// launch's first row (mask rows and causal queries follow global rows).
struct MaskArgs {
    float scale;
    const void* mask;
    int64_t mask_rows;
    int64_t causal_q;
    int64_t row_base;
};

struct WaveRowVariant { int G, K, U; };          // lanes per row, granules per lane, row sets

// Alignment (bytes) of the row windows of the forward's lane groups
// (wave_row, plain and masked): a 128-byte line for groups of 16 lanes or
// more, so that their lanes cover whole lines; 16 bytes for narrower groups,
// whose rows are short enough that a line-aligned window would mostly load
// neighbouring rows' bytes.  fp16 rows that are not line-aligned, 8-lane
// groups: [1000000,33] 54.9 us against 93.9 with line-aligned windows,
// [524288,60] 29.7 against 35.4 (line-aligned rows unchanged: [2097152,64]
// 80.1 both).  The backward's and the normalisations' lane groups keep
// line-aligned windows from 8 lanes.
constexpr int softmax_window_align(int G) { return G * 16 > 128 ? 128 : 16; }
struct OnepassVariant { int block, kr, kl; };    // threads, register granules, LDS granules
struct TwoPassVariant { int block, u; };         // threads, granules per batch
struct SplitkVariant { int block, kc; };         // threads, granules per thread per chunk
struct TileRowsVariant { int K; };               // granules per lane
// Tile of a tile_rows launch: T rows per one-wave workgroup (4..64, a whole
// number of granules, at most 64 * K of them), tiles in XCD runs of 2^lgrun.
struct TileShape {
    int T;
    int lgrun;
};
constexpr int kTileMaxT = 64;  // rows per tile at most (one lane per row)

extern const WaveRowVariant kWaveRow[];
extern const int kNumWaveRow;
extern const OnepassVariant kOnepass[];
extern const int kNumOnepass;
extern const TwoPassVariant kTwoPass[];
extern const int kNumTwoPass;
extern const SplitkVariant kSplitk[];
extern const int kNumSplitk;
extern const SplitkVariant kSplitkFused[];
extern const int kNumSplitkFused;
extern const TileRowsVariant kTileRows[];
extern const int kNumTileRows;

// Waves per workgroup of the wave-per-row kernels (wave_row, bwd_wave,
// norm_wave; the kernels read it from blockDim).  One-wave workgroups
// measured fastest on MI355X for rows streamed from HBM: fp16 [65536,512]
// softmax 21.7 us against 22.8 us with four waves, bf16 [1048576,128]
// 79.8 us against 81.3 us; a plain 64 MiB copy 21.9 us against 22.8 us.
constexpr int kWaveGroupWaves = 1;
constexpr int kWaveGroupThreads = 64 * kWaveGroupWaves;

// Grid of one wave-per-row launch.
inline int64_t wave_row_grid(const WaveRowVariant& v, int64_t rows) {
    const int64_t rows_per_wave = (int64_t)(64 / v.G) * v.U;
    const int64_t waves = (rows + rows_per_wave - 1) / rows_per_wave;
    return (waves + kWaveGroupWaves - 1) / kWaveGroupWaves;
}

hipError_t launch_wave_row(const Launch& L, int variant);
// Tiles of t.T rows per one-wave workgroup, K = kTileRows[variant].K
// granules per lane; in and out 16-byte aligned (hipErrorInvalidValue for a
// shape the kernels do not take).
hipError_t launch_tile_rows(const Launch& L, int variant, const TileShape& t);
hipError_t launch_block_onepass(const Launch& L, int variant);
hipError_t launch_two_pass(const Launch& L, int variant);
// Both split-k stages; ws holds rows*P (m, d) pairs.
hipError_t launch_splitk(const Launch& L, int variant, int P, float2* ws);
// Workgroups of this fused variant that can be resident at once on `cus`
// CUs (the device's occupancy query), and the waves per SIMD its kernels are
// compiled to allow (a lower bound on that occupancy without a device).
hipError_t splitk_fused_capacity(int variant, int dtype, bool aligned, int cus, int64_t* blocks);
int splitk_fused_min_waves(int variant, int dtype, bool aligned);
// What an ordered (single-launch split-k) launch needs besides its tensors,
// passed to the kernel as one argument:
//   tags       2 * rows * P epoch-tagged 64-bit words (zeroed when allocated)
//   epoch      this launch's epoch on `tags`, never 0 (unless epoch_src)
//   epoch_src  launches recorded in a graph read their epoch from this device
//              word instead (see kDeviceEpochFirst)
//   status     the stream's status word: a workgroup whose wait for a
//              partial gave up writes NaN outputs and ORs kStatusLate in
//   spin_limit tries of one poll before it gives up (kOrderedSpinLimit by
//              default: at least ~0.5 s; 0 gives up at once)
struct OrderedSync {
    uint64_t* tags;
    unsigned epoch;
    const uint64_t* epoch_src;
    uint64_t* status;
    unsigned spin_limit;
};
constexpr unsigned kOrderedSpinLimit = 1u << 21;
constexpr uint64_t kStatusLate = 1;
// Single-launch split-k that reads every element once (ordinary launch, grid
// rows*P, every workgroup keeps its chunk in registers and waits for its
// row's P partials, so P workgroups must fit on the device at once;
// OrderedSync as for the ordered form below, with 2*rows*P tag words).
hipError_t launch_splitk_fused(const Launch& L, int variant, int P, const OrderedSync& S);
// Split-k in one ordinary launch (kSplitk variants): grid 2*rows*P.
hipError_t launch_splitk_ordered(const Launch& L, int variant, int P, const OrderedSync& S);
// Epochs of eager ordered launches are handed out by the host from
// [1, 2^31).  In a captured graph a kernel argument would be replayed
// unchanged, so launches recorded there take theirs from a device word that
// a one-workgroup kernel enqueued just before advances through [2^31, 2^32).
// The two ranges never meet, so eager and replayed launches share one tag
// buffer on a stream.
constexpr unsigned kDeviceEpochFirst = 0x80000000u;
// Graph capture: advance the device epoch held in words[n] (the word after a
// tag buffer's n words) for the next ordered launch, which then reads its
// epoch from &words[n] (epoch_src) instead of a kernel argument.
hipError_t launch_bump_epoch(uint64_t* words, int64_t n, hipStream_t stream);
// Set n 64-bit words to v on `stream`.
hipError_t launch_fill_words(uint64_t* p, int64_t n, uint64_t v, hipStream_t stream);
// The masked forms (same variant tables; block_onepass only for variants
// without LDS parking).
hipError_t launch_wave_row_masked(const Launch& L, int variant, const MaskArgs& M);
hipError_t launch_block_onepass_masked(const Launch& L, int variant, const MaskArgs& M);
hipError_t launch_two_pass_masked(const Launch& L, int variant, const MaskArgs& M);
// The masked form of tile_rows (kTileRows variants, as launch_tile_rows).
hipError_t launch_tile_rows_masked(const Launch& L, int variant, const TileShape& t,
                                  const MaskArgs& M);
// Softmax backward: dx = y * (dy - sum(dy * y)) per row.
struct BwdLaunch {
    const void* y;
    const void* dy;
    void* dx;
    int64_t rows;
    int cols;
    int dtype;
    bool aligned;     // y, dx 128-byte aligned and cols*size % 128 == 0
    bool same_phase;  // (dx - y) % 16 == 0
    bool dy_vec;      // (dy - y) % 16 == 0
    int lgrun = 0;    // bwd_block / bwd_stream: XCD runs of 2^lgrun rows
    hipStream_t stream;
};
// tile_rows form of the backward (kTileRows variants): y, dy and dx
// 16-byte aligned, as launch_tile_rows.
hipError_t launch_bwd_tile(const BwdLaunch& B, int variant, const TileShape& t);
extern const WaveRowVariant kBwdWave[];
extern const int kNumBwdWave;
extern const TwoPassVariant kBwdBlock[];  // (threads, register granules per thread)
extern const int kNumBwdBlock;
extern const TwoPassVariant kBwdStream[];  // (threads, granules per thread per batch)
extern const int kNumBwdStream;
// family: 1 wave (kBwdWave), 2 block (kBwdBlock), 3 stream (kBwdStream)
hipError_t launch_bwd(const BwdLaunch& B, int family, int variant);
// Few long rows: split-k in one launch, chunks of kBwdOrderedBlock x
// kBwdOrderedKc granules, P chunks per row (OrderedSync as for the forward).
constexpr int kBwdOrderedBlock = 256;
constexpr int kBwdOrderedKc = 4;
hipError_t launch_bwd_ordered(const BwdLaunch& B, int P, const OrderedSync& S);
// Row normalisations (rws_norm.hpp).
constexpr int kLayerNorm = 0;
constexpr int kRmsNorm = 1;
struct NormArgs {
    const void* w;  // per-column weight (cols entries of the dtype) or nullptr
    const void* b;  // per-column bias or nullptr (LayerNorm only)
    float* mean;    // per-row mean out or nullptr (LayerNorm only)
    float* rstd;    // per-row 1/sqrt(var + eps) out or nullptr
    float eps;
    float n;        // cols as a float
};
struct NormLaunch {
    const void* in;
    void* out;
    int64_t rows;
    int cols;
    int dtype;
    int mode;         // kLayerNorm / kRmsNorm
    bool aligned;     // in, out 128-byte aligned and cols*size % 128 == 0
    bool same_phase;  // (out - in) % 16 == 0
    NormArgs args;    // mean/rstd already offset to the launch's first row
    bool aff_matched = false;  // aligned rows; w and b (if given) at the rows' 16-byte phase
    int lgrun = 0;    // norm_block / norm_stream: XCD runs of 2^lgrun rows
    hipStream_t stream;
};
// tile_rows form of the normalisations without weight and bias
// (kTileRows variants): in and out 16-byte aligned, as launch_tile_rows.
hipError_t launch_norm_tile(const NormLaunch& N, int variant, const TileShape& t);
extern const WaveRowVariant kNormWave[];
extern const int kNumNormWave;
extern const TwoPassVariant kNormBlock[];   // (threads, register granules per thread)
extern const int kNumNormBlock;
extern const TwoPassVariant kNormStream[];  // (threads, granules per thread per batch)
extern const int kNumNormStream;
hipError_t launch_norm_wave(const NormLaunch& L, int variant);
// family 2: block (kNormBlock), 3: stream (kNormStream)
hipError_t launch_norm_block(const NormLaunch& L, int family, int variant);
// Few long rows: split-k in one launch (as launch_bwd_ordered).
constexpr int kNormOrderedBlock = 256;
constexpr int kNormOrderedKc = 4;
hipError_t launch_norm_ordered(const NormLaunch& L, int P, const OrderedSync& S);
// n16 granules of 16 bytes: copy, read only, write only (the references of
// the roofline).
hipError_t launch_copy16(const void* in, void* out, int64_t n16, hipStream_t stream);
hipError_t launch_read16(const void* in, int64_t n16, hipStream_t stream);
hipError_t launch_write16(void* out, int64_t n16, hipStream_t stream);

}  // namespace rws
