// mxq_split.hip -- quantize a concatenated routed activation once and split
// it per expert: payload rows stay at their global rows, each expert's scales
// go to its own, separately padded region of one bulk buffer, and the row
// amax is emitted.  Three forms share the kernel: NVFP4 under one encode
// scale, row-scaled NVFP4 (each row under an encode scale derived from its own
// amax) and MXFP8.
//
// A work unit is consecutive rows of the activation, whatever experts they
// belong to, taken by a workgroup of 4 waves: with swizzled scales 2 rows of
// two waves each, with linear scales 1 row of four waves.  Consecutive rows
// are one contiguous stretch of memory, which HBM serves best, and many small
// workgroups keep the most loads in flight.  Linear scales of the whole
// activation are one [rows, C] matrix, so the unit's codes leave as one
// contiguous run; one row of four waves (4 steps of 512 columns per wave at
// 7168 columns, 7 waves per SIMD) ran the routed NVFP4 split in 27.3-27.6 us
// against 29.5-30.1 with two rows of two waves.  Swizzled, the same shape ran
// 0.5-1.5 us slower: one row's 4-byte scale slots lie 512 bytes apart, while
// the slots of two adjacent rows share 16-byte lines, so each store of a
// two-row unit covers both.  With swizzled scales each row's code for tile t is a
// 4-byte slot at its expert's region, band, 16-byte line p = local row % 32
// and slot q = local row / 32 % 4.  The last live row of a line also writes
// the zeros of the padding slots after it, in the same store (16 bytes for a
// line with one live row), and one unit per expert whose last band has under
// 32 live rows zeroes the lines with none.
//
// Measured on an [8192, 7168] activation, NVFP4, swizzled (246 experts of
// 19-55 rows / experts of 150 rows):
//   units of 8 rows of one expert, padding apart in 4-byte slots    39 / 39 us
//   units of a band's 2-, 4- or 8-row line segments (rows 32 apart,
//     whole 32- to 128-byte scale segments)                          40-45 / 38-42
//   8 consecutive rows (512 threads), padding apart                   37.5 / 32
//   same, padding carried by the last live row of each line           35 / 32
//   same, linear codes of partial bands reordered by a 2nd kernel     39-41 / 39-41
//   4 consecutive rows (512 or 256 threads)                           33-34.6 / 29.4-31
//   2 consecutive rows (256 threads)                                  33.3-34.4 / 29.1
//   (2 rows of four waves, 512 threads, 6-8 waves per SIMD: 35.8-37.7)
//   same, 4 consecutive units on one XCD                              32.1-32.3 / 29.3
//   same, padding units dispatched first                              30.8-31.2 / 28.7-28.9
//   same, 8, 16 or 64 units per XCD                                   30.0-30.8 / 28.8-30.1
//   same, 32 units per XCD (here)                                     30.1-30.2 / 29.0-29.1
//   (64 per XCD slows MXFP8 by 0.3-0.7 us.  Lanes on consecutive tiles of
//   one row, 64 lines per wave store instead of 32, cost about 1 us.)
//   1 row (128 threads)                                               38 / 32
//
// Splitting a band's padding over units of 16 or 4 tiles sped small
// activations up by under 1 us and slowed T = 1024 (every expert padded) by 1
// to 7 us: the padding stays one unit per expert.
//
// A wave loads its next row only after storing the current one: loading it
// earlier doubles the row registers and measured slower than leaving the
// overlap to the other resident waves.  Every byte has one writer, and no
// global atomics are used.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

// Register budgets without spills: up to 4 steps per wave in 72 VGPRs (7
// waves per SIMD) with one encode scale, in 84 (6) row-scaled, when four waves
// share a row (8 waves per SIMD spilled and ran 40 % slower); up to 7 steps in
// 96 VGPRs (5) with one encode scale, in 128 (4) row-scaled; 8 steps in 128
// or, row-scaled, 168 (3); wider rows get the whole register file.
constexpr int split_waves(int nch, bool rowsc, int wpr) {
    return nch <= 4 && wpr == 4 ? (rowsc ? 6 : 7)
           : nch <= 7           ? (rowsc ? 4 : 5)
           : nch == 8           ? (rowsc ? 3 : 4)
                                : 1;
}

template <int FMT, bool ROWSC, int LAYOUT, int NCH>
__global__ __launch_bounds__(kSplitThreads)
__attribute__((amdgpu_waves_per_eu(split_waves(NCH, ROWSC, split_wpr(LAYOUT)))))
void k_split(const SplitArgs a) {
    using Tr = FmtTraits<FMT>;
    constexpr bool kSwz = LAYOUT == MXQ_SF_SWIZZLED;
    constexpr int kWpr = split_wpr(LAYOUT);      // waves per row
    constexpr int kUnit = split_unit_rows(LAYOUT);  // rows per unit, all in flight at once
    constexpr int kPairs = kUnit;
    extern __shared__ __align__(16) uint8_t stage[];  // the unit's codes, one row per sf_stride
    __shared__ uint32_t row_max[kUnit];  // one encode scale: row amax folded by LDS atomics
    __shared__ uint32_t half_max[2][kWpr * kPairs];  // row-scaled: each wave's part-row amax, two buffers
    __shared__ int64_t row_dst[kUnit];   // swizzled: offset of each row's piece of tile 0
    __shared__ int32_t row_zero[kUnit];  // swizzled: zero slots the row's store carries
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int pair = w / kWpr, half = w % kWpr;  // the wave's row of the unit, its part of the row
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? a.cols : a.cols / 2;
    const float g = (FMT == MXQ_NVFP4 && !ROWSC) ? *a.g : 0.0f;
    const NvG G = nv_prepare(g);
    const int n_rows = a.row_off[a.n];
    const int n_row_units = (n_rows + kUnit - 1) / kUnit;
    const int tiles = a.sf_stride >> 2;
    // last split s in [0, n) with off[s] <= v (empty splits share offsets)
    auto find = [&](const int32_t *off, int v) {
        int lo = 0, hi = a.n;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (off[mid] <= v) lo = mid; else hi = mid;
        }
        return lo;
    };
    int it = 0;  // row-scaled step counter, uniform over the workgroup
    for (int u0 = blockIdx.x; u0 < a.total_units; u0 += gridDim.x) {
        // swizzled: the padding units take the first dispatch slots, so their
        // stores overlap the row units instead of trailing them; the row
        // units of 64 consecutive rows (whose codes fill the 16-byte lines of
        // half a band, or share linear 128-byte lines) meet in one L2, which
        // merges their partial-line stores
        int u = u0;
        if (kSwz) {
            const int pads = a.total_units - n_row_units;
            u = u0 < pads ? n_row_units + u0 : u0 - pads;
        }
        if (xcd_grouping_holds(gridDim.x, a.total_units) && u < n_row_units)
            u = xcd_grouped_unit<64 / kUnit>(u, n_row_units);
        if (kSwz && u >= n_row_units) {
            // padding unit of split s, whose last band has fewer than 32
            // live rows: the 16-byte chunks with no live row are zeroed
            const int s = find(a.unit_off, u - n_row_units);
            const int m = a.row_off[s + 1] - a.row_off[s];
            const int b = (m - 1) >> 7;
            const int lb = m - b * 128;  // live rows in the band, 1..31
            uint8_t *base = a.scales + (int64_t)(a.band_off[s] + b) * tiles * 512;
            const int ne = 32 - lb;  // lines p = lb..31 of every tile hold no live row
            for (int k = threadIdx.x; k < tiles * ne; k += kSplitThreads) {
                const int t = k / ne, p = lb + k - t * ne;
                *reinterpret_cast<u32x4 *>(base + (int64_t)t * 512 + p * 16) = u32x4{0, 0, 0, 0};
            }
            continue;  // uniform over the workgroup
        }
        const int r0 = u * kUnit;  // the unit's first row in the launch
        const int n_live = min(kUnit, n_rows - r0);
        auto load_row = [&](int j, u32x4 *v) {
            const uint16_t *src = a.src + (int64_t)(r0 + j) * a.cols;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int col = (kWpr * k + half) * kChunk + lane * 8;
                v[k] = u32x4{0, 0, 0, 0};
                if (col < a.cols)
                    v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + col));
            }
        };
        u32x4 cur[NCH];
        // the amax of this wave's part of the row (columns past the row were
        // loaded as zeros)
        auto half_amax = [&]() {
            uint32_t am = 0;
#pragma unroll
            for (int k = 0; k < NCH; ++k) am = max(am, amax_bits8(cur[k]));
            return wave_max(am);
        };
        // encode the wave's part of the row, in cur, as row j of the unit under
        // the encode scale Gr; whole wave.  am accumulates the part's amax bits.
        auto encode = [&](int j, const NvG &Gr, uint32_t &am) {
            uint8_t *pay_row = a.payload + (int64_t)(r0 + j) * payload_ld;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                const int col = (kWpr * k + half) * kChunk + lane * 8;
                u32x2 pay;
                const uint32_t code = quant8<FMT>(cur[k], Gr, pay);
                if (col < a.cols) {
                    store_payload<FMT>(pay_row, col, pay);
                    if (!ROWSC) am = max(am, amax_bits8(cur[k]));
                    if (leader) stage[j * a.sf_stride + col / Tr::kBlock] = (uint8_t)code;
                }
            }
        };

        if (pair < n_live) load_row(pair, cur);
        if constexpr (kSwz) {
            // each row's split, its band there, line (local row % 32) and
            // 4-byte slot (local row / 32 % 4); the splits advance in order
            int se = find(a.row_off, r0);
#pragma unroll
            for (int j = 0; j < kUnit; ++j) {
                if (j < n_live) {
                    while (a.row_off[se + 1] <= r0 + j) ++se;
                    const int rl = r0 + j - a.row_off[se];
                    const int p = rl & 31, q = (rl >> 5) & 3;
                    // live rows of the band, and the last live slot of line p
                    const int lb = min(128, a.row_off[se + 1] - a.row_off[se] - (rl & ~127));
                    const int ql = min(3, (lb - 1 - p) >> 5);
                    if ((int)threadIdx.x == j) {
                        row_dst[j] = (int64_t)(a.band_off[se] + (rl >> 7)) * tiles * 512 +
                                     p * 16 + q * 4;
                        row_zero[j] = q == ql ? 3 - q : 0;
                    }
                }
            }
            // codes of the padding columns C..round_up(C, 4) stay zero
            if (a.sf_stride != a.sf_cols) {
                for (int k = threadIdx.x * 16; k < kUnit * a.sf_stride; k += kSplitThreads * 16)
                    *reinterpret_cast<u32x4 *>(stage + k) = u32x4{0, 0, 0, 0};
            }
        }
        if (!ROWSC && threadIdx.x < kUnit) row_max[threadIdx.x] = 0;
        __syncthreads();
        if constexpr (!ROWSC) {
            for (int j = pair; j < n_live; j += kPairs) {
                uint32_t am = 0;
                encode(j, G, am);
                am = wave_max(am);
                if (lane == 0) atomicMax(&row_max[j], am);
                if (j + kPairs < n_live) load_row(j + kPairs, cur);
            }
        } else {
            // Every wave takes every step (the barrier needs all of them); a
            // row's two halves meet in half_max before either is encoded.
            for (int j0 = 0; j0 < n_live; j0 += kPairs, ++it) {
                const int j = j0 + pair;
                const uint32_t am = j < n_live ? half_amax() : 0u;
                if (lane == 0) half_max[it & 1][w] = am;
                __syncthreads();
                if (j < n_live) {
                    uint32_t ra = half_max[it & 1][kWpr * pair];
#pragma unroll
                    for (int p = 1; p < kWpr; ++p) ra = max(ra, half_max[it & 1][kWpr * pair + p]);
                    const float af = __uint_as_float(ra << 16);
                    const float gr = nv_encode_scale(af);
                    uint32_t unused = 0;
                    encode(j, nv_prepare(gr), unused);
                    if (a.row_amax && half == 0 && lane == 0) a.row_amax[r0 + j] = af;
                }
                if (j + kPairs < n_live) load_row(j + kPairs, cur);
            }
        }
        __syncthreads();
        if (!ROWSC && a.row_amax && (int)threadIdx.x < n_live)
            a.row_amax[r0 + threadIdx.x] = __uint_as_float(row_max[threadIdx.x] << 16);
        if constexpr (kSwz) {
            // row j's codes of tile t, with the zeros of the padding slots
            // after it when it is the last live row of its line: one store;
            // consecutive lanes take consecutive rows, whose lines are adjacent
            for (int k = threadIdx.x; k < n_live * tiles; k += kSplitThreads) {
                const int t = k / n_live, j = k - t * n_live;
                const uint32_t c = *reinterpret_cast<const uint32_t *>(stage + j * a.sf_stride + t * 4);
                uint8_t *dst = a.scales + row_dst[j] + (int64_t)t * 512;
                switch (row_zero[j]) {
                case 3: *reinterpret_cast<u32x4 *>(dst) = u32x4{c, 0, 0, 0}; break;
                case 2:
                    *reinterpret_cast<uint32_t *>(dst) = c;
                    *reinterpret_cast<u32x2 *>(dst + 4) = u32x2{0, 0};
                    break;
                case 1: *reinterpret_cast<u32x2 *>(dst) = u32x2{c, 0}; break;
                default: *reinterpret_cast<uint32_t *>(dst) = c; break;
                }
            }
        } else {
            uint8_t *dst = a.scales + (int64_t)r0 * a.sf_cols;
            const int nbytes = n_live * a.sf_cols;
            if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                for (int k = threadIdx.x; k < (nbytes >> 4); k += kSplitThreads)
                    *reinterpret_cast<u32x4 *>(dst + k * 16) =
                        *reinterpret_cast<const u32x4 *>(stage + k * 16);
                for (int k = (nbytes & ~15) + threadIdx.x; k < nbytes; k += kSplitThreads)
                    dst[k] = stage[k];
            } else {
                for (int k = threadIdx.x; k < nbytes; k += kSplitThreads) dst[k] = stage[k];
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Launcher.
// ---------------------------------------------------------------------------
template <int FMT, bool ROWSC, int LAYOUT>
static void split_nch(const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kSplitThreads);
    switch (split_steps(a.cols, split_wpr(LAYOUT))) {
    case 1: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 1>), gd, bd, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 2>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 4>), gd, bd, lds, s, a); break;
    case 7: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 7>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 8>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 16>), gd, bd, lds, s, a); break;
    }
}

template <int FMT, bool ROWSC>
static void split_layout(int layout, const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    if (layout == MXQ_SF_LINEAR)
        split_nch<FMT, ROWSC, MXQ_SF_LINEAR>(a, gd, lds, s);
    else
        split_nch<FMT, ROWSC, MXQ_SF_SWIZZLED>(a, gd, lds, s);
}

hipError_t launch_split(int fmt, bool row_scaled, int layout, const SplitArgs &a, int64_t grid,
                        hipStream_t s) {
    // the unit's codes; rounded up to 16 bytes, the granule of the zeroing
    // stores of the padding columns
    const size_t lds = ((size_t)split_unit_rows(layout) * a.sf_stride + 15) & ~(size_t)15;
    const dim3 gd((unsigned)(grid < 1 ? 1 : grid));
    if (fmt == MXQ_MXFP8)
        split_layout<MXQ_MXFP8, false>(layout, a, gd, lds, s);
    else if (row_scaled)
        split_layout<MXQ_NVFP4, true>(layout, a, gd, lds, s);
    else
        split_layout<MXQ_NVFP4, false>(layout, a, gd, lds, s);
    return hipGetLastError();
}

}  // namespace mxq
