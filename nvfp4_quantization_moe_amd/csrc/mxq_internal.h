// mxq_internal.h -- kernel argument tables and launchers shared by the C ABI
// (mxq_api.hip) and the kernels (mxq_grouped.hip, mxq_split.hip,
// mxq_fused.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"

namespace mxq {

constexpr int kThreads = 256;  // 4 waves per workgroup
constexpr int kRowsPerWave = 4;                // rows per wave in a grouped unit
constexpr int kUnitRows = 4 * kRowsPerWave;   // rows per grouped work unit
constexpr int kChunk = 512;    // row elements per wave step (8 per lane)
constexpr int kSplitThreads = 256;  // split workgroup: 4 waves

// Workgroup b of a launch runs on XCD b % 8, and each XCD has its own L2.
// Within every block of 8*G workgroups, XCD x takes units G*x .. G*x + G-1 of
// the block, so G consecutive units, which write neighbouring bytes, meet in
// one L2 while the units in flight still cover one compact window.  The tail
// past the last whole block keeps the plain order.
template <int G>
__device__ __forceinline__ int xcd_grouped_unit(int b, int n) {
    constexpr int kBlock = G * 8;
    if (b >= n / kBlock * kBlock) return b;
    return b / kBlock * kBlock + (b & 7) * G + (b >> 3) % G;
}

// Whether the XCD grouping holds for a launch of `grid` workgroups over
// `units` units: with one workgroup per unit, workgroup b takes unit b; with
// fewer, workgroup b takes units b, b + grid, b + 2 grid, ..., which all run
// on XCD b % 8 when grid is a multiple of 8.
__device__ __forceinline__ bool xcd_grouping_holds(int64_t grid, int64_t units) {
    return grid == units || (grid & 7) == 0;
}

// The same with a group size g known only at run time (g >= 1).
__device__ __forceinline__ int64_t xcd_grouped_unit(int64_t b, int64_t n, int g) {
    const int64_t block = (int64_t)g * 8;
    if (b >= n / block * block) return b;
    return b / block * block + (b & 7) * g + (b >> 3) % g;
}

// One grouped-launch descriptor.  The whole table travels in the kernel
// arguments, so a grouped call is one dispatch with no device-side table.
struct GEntry {
    const uint16_t *src;  // bf16 bits
    uint8_t *payload;
    uint8_t *scales;
    const float *g;       // NVFP4 encode scale (device scalar)
    int64_t ld;           // row stride, elements
    int32_t rows;
    int32_t unit_begin;   // index of this entry's first work unit
    int32_t slot;         // encode-scale slot (scales from the data)
    int32_t pad_;
};

struct GroupArgs {
    GEntry e[MXQ_MAX_GROUP];
    int32_t n;            // entries
    int32_t cols;
    int32_t sf_cols;      // C = cols / block
    int32_t sf_stride;    // swizzled: round_up(C, 4); linear: C
    int32_t n_cc;         // 512-column chunks per row
    int32_t total_units;
    // encode scales from the data: per-slot amax as fp32 bits (zeroed, then
    // reduced by k_amax) and the encode scales written by the quantize pass
    uint32_t *amax_bits;
    float *g_out;
    int32_t n_slots;
    int32_t uniform_units;  // units per entry when every entry has the same count, else 0
};

constexpr int kMaxSplitsPerLaunch = 256;
// Waves per row and rows per split work unit (the workgroup's 4 waves):
// swizzled, two rows of two waves (the rows' 4-byte scale slots share
// 16-byte lines, so a store of both rows' slots coalesces); linear, one row
// of four waves (shorter chains of loads per wave).
constexpr int split_wpr(int layout) { return layout == MXQ_SF_SWIZZLED ? 2 : 4; }
constexpr int split_unit_rows(int layout) { return kSplitThreads / 64 / split_wpr(layout); }

// Up to 256 consecutive non-empty splits of a concatenated activation (the
// host leaves empty splits out: they own no rows and no scale bytes).  Work units
// [0, ceil(rows / 2)) are 2 consecutive rows of the launch, across split
// boundaries.  With swizzled scales they are followed by one padding unit per
// split whose last 128-row band has 1..31 live rows (dispatched first).
struct SplitArgs {
    const uint16_t *src;  // global row 0 of this launch's first split
    uint8_t *payload;     // same row
    uint8_t *scales;      // this launch's first split's scale region
    float *row_amax;      // same row (may be null unless row-scaled)
    const float *g;       // NVFP4 encode scale; unused for MXFP8 and row-scaled
    int32_t cols;
    int32_t sf_cols;
    int32_t sf_stride;
    int32_t n;            // splits in this launch
    int32_t total_units;
    int32_t pad_;
    int32_t row_off[kMaxSplitsPerLaunch + 1];   // prefix sums of split rows
    int32_t unit_off[kMaxSplitsPerLaunch + 1];  // prefix sums of padding units
    int32_t band_off[kMaxSplitsPerLaunch + 1];  // prefix sums of 128-row bands
};

struct FusedArgs {
    const uint16_t *x;
    const uint16_t *res;
    const uint16_t *gamma;
    uint16_t *res_out;
    uint16_t *norm_out;
    uint8_t *payload;
    uint8_t *scales;
    const float *g;
    float eps;
    int32_t T;
    int32_t H;
    int32_t sf_cols;
    int32_t sf_stride;
    int32_t total_units;
    int32_t wpr;          // waves per row: 16 or 4 (with rpu 1), or 2 (with rpu 4)
    int32_t rpu;          // rows per unit
};

// Fused epilogue shape for T rows (measured at H = 7168):
//  * up to kFusedWideMaxT rows, sixteen waves per row and one-row units: each
//    wave loads one 512-column step, so a row's loads are all in flight at
//    once (T = 1 / 256: 3.8-4.3 / 4.9-5.4 us against 4.9-6.2 / 6.6-7.8 with
//    four waves); with linear scales the edge comes earlier (T = 384: 8.9
//    against 8.0 us);
//  * up to kFusedFourWaveMaxT rows, four waves per row and one-row units;
//  * beyond, two waves per row and four-row units (bandwidth bound).  The
//    last two tie near T = 1536; at T = 2048 four-row units are 1-4 us faster.
constexpr int64_t kFusedWideMaxTSwizzled = 512;
// Swizzled, H up to 16 x 512: k_fused_tiny (one workgroup per live row, no
// padding units) at T = 1 and at 17..31 rows; the general kernel from 2 to 16
// rows, where its scale-line unit order puts 4 live rows on each of up to 4
// XCDs (whole 64-byte line segments, gamma fetched by 4 L2s).  Measured at
// H = 7168, MXFP8, kernel trace (this kernel / the general one):
//   T = 1: 3.44 / 3.44 us, 1.07 / 1.44x the algorithmic bytes;
//   T = 2..16: 0.04-0.16 us slower, 1.16-1.29x / 1.08-1.27x;
//   T = 24, 31: 4.16 / 4.64 us.
// Below 32 rows every row is the only live row of its scale line.
constexpr int64_t kFusedTinyMaxT = 31;
static_assert(kFusedTinyMaxT < 32, "k_fused_tiny writes each row as the only live row of its line");
__host__ __device__ constexpr bool fused_tiny_rows(int64_t T) {
    return T == 1 || (T > 16 && T <= kFusedTinyMaxT);
}
constexpr int kFusedTinyThreads = 1024;
constexpr int64_t kFusedWideMaxTLinear = 256;
constexpr int64_t kFusedFourWaveMaxT = 1536;

// Scale swizzle unit: one 128-row band by at most this many 4-column tiles.
// Wider units (whole rows up to 512 columns) leave too few workgroups, each
// with more serial loads: 16 / 32 / 64 / 128 tiles took 9.0 / 9.5 / 11.9 /
// 16.6 us on a [31488, 448] matrix.
constexpr int kSwizzleTiles = 16;

struct SwizzleArgs {
    const uint8_t *lin;
    uint8_t *swz;
    int64_t rows;
    int64_t cols;        // scale columns C
    int64_t tiles_per_band;  // round_up(C, 4) / 4
    int32_t unit_tiles;  // tiles per unit: min(tiles_per_band, kSwizzleTiles)
    int32_t pad_;
};

// Launchers: return hipSuccess or the launch error.
hipError_t launch_grouped(int fmt, int layout, bool auto_scale, const GroupArgs &a, int64_t grid,
                          hipStream_t s, bool chain = false);
// Zero a.amax_bits[0..n_slots), then reduce each slot's amax into it.
hipError_t launch_amax(const GroupArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_split(int fmt, bool row_scaled, int layout, const SplitArgs &a, int64_t grid,
                        hipStream_t s);
hipError_t launch_fused(int fmt, int layout, const FusedArgs &a, int64_t grid, hipStream_t s);
hipError_t launch_fused_tiny(int fmt, const FusedArgs &a, hipStream_t s);
hipError_t launch_swizzle(const SwizzleArgs &a, int64_t grid, hipStream_t s);

// Largest supported row lengths.  Grouped units take 512-column chunks, so
// any width works; these are the widths tested against the oracle.  The split
// and fused kernels hold a whole row in registers, 16 steps of 512 columns
// per wave pair at most.
constexpr int64_t kMaxColsMx = 32768;
constexpr int64_t kMaxColsNv = 16384;
constexpr int64_t kMaxSplitCols = 16384;
constexpr int64_t kMaxFusedH = 16384;

// The split keeps 1/wpr of a row per wave in registers: this many 512-column
// steps per wave, rounded up to an instantiated count.
inline int split_steps(int64_t cols, int wpr) {
    const int64_t n = ((cols + kChunk - 1) / kChunk + wpr - 1) / wpr;
    if (n <= 1) return 1;
    if (n <= 2) return 2;
    if (n <= 4) return 4;
    if (n <= 7) return 7;
    if (n <= 8) return 8;
    return 16;
}

}  // namespace mxq
