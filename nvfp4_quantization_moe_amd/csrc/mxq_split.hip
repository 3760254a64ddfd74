// mxq_split.hip -- quantize a concatenated routed activation once and split
// it per expert: payload rows stay at their global rows, each expert's scales
// go to its own, separately padded region of one bulk buffer, and the row
// amax is emitted.  Three forms share the kernel: NVFP4 under one encode
// scale, row-scaled NVFP4 (each row under an encode scale derived from its own
// amax) and MXFP8.
//
// Swizzled, SUB = 2: a unit owns the 2-row segment `sub` of line h (0..3) of
// every scale tile of one 128-row band of one expert, i.e. the rows
// band*128 + 32*q + 8*h + 2*sub + i (q < 4, i < 2), so its staged scales leave
// as whole 32-byte segments, padding rows and columns zero.  Swizzled,
// SUB = 0 (scatter; for short experts, whose bands are mostly padding): a
// unit is 8 consecutive rows of one expert and writes each row's 4-byte piece
// of every tile; one more unit per expert whose last band is partial writes
// that band's padding rows as zeros (measured faster than 32-row units of
// whole 128-byte lines: 39-41 against 40-46 us on the routed activation).
// Linear: a unit is 8 consecutive rows.  The host picks SUB per call.  Only
// the unit's live rows are loaded: pairs of waves take them in turn, each
// wave holding half of a row (512-column steps 2k + half) in registers, so
// short experts keep every wave busy.  A wave loads its next row only after
// storing the current one: loading it earlier doubles the row registers and
// measured slower than leaving the overlap to the other resident waves.
// Units run in plain dispatch order; every byte has one writer, and no
// global atomics are used.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

// Up to 8 half-row steps fit in 128 VGPRs, so two workgroups share a CU;
// wider rows get the whole register file.
template <int FMT, bool ROWSC, int LAYOUT, int NCH2, int SUB>
__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(NCH2 <= 8 ? 4 : 1)))
void k_split(const SplitArgs a) {
    using Tr = FmtTraits<FMT>;
    constexpr bool kScatter = LAYOUT == MXQ_SF_SWIZZLED && SUB == 0;
    constexpr int kUnit = kScatter ? 8 : 4 * SUB;  // rows per unit
    extern __shared__ __align__(16) uint8_t stage[];
    __shared__ uint32_t row_max[kUnit];  // one encode scale: row amax folded by LDS atomics
    __shared__ uint32_t half_max[2][8];  // row-scaled: each wave's half-row amax, two buffers
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int pair = w >> 1, half = w & 1;
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? a.cols : a.cols / 2;
    const float g = (FMT == MXQ_NVFP4 && !ROWSC) ? *a.g : 0.0f;
    const float quot = (FMT == MXQ_NVFP4 && !ROWSC) ? nv_wave_quot(g) : 0.0f;
    const int stage_bytes = kUnit * a.sf_stride;
    int it = 0;  // row-scaled step counter, uniform over the workgroup
    for (int u = blockIdx.x; u < a.total_units; u += gridDim.x) {
        int lo = 0, hi = a.n;  // split s with unit_off[s] <= u < unit_off[s + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.unit_off[mid] <= u) lo = mid; else hi = mid;
        }
        const int s = lo;
        const int lu = u - a.unit_off[s];
        const int m = a.row_off[s + 1] - a.row_off[s];
        const int64_t e0 = a.row_off[s];  // expert's first row
        const int tiles = a.sf_stride >> 2;
        if constexpr (kScatter) {
            // the unit after an expert's row units zeroes the padding rows of
            // its last band: every 4-byte piece of a row at or past m
            const int n_row_units = (m + kUnit - 1) / kUnit;
            if (lu >= n_row_units) {
                const int b = (m - 1) >> 7;
                const int lb = m - b * 128;  // live rows in the band, 1..127
                uint8_t *base = a.scales + (int64_t)(a.band_off[s] + b) * tiles * 512;
                for (int k = threadIdx.x; k < tiles * 32; k += kSplitThreads) {
                    const int t = k >> 5, p = k & 31;
                    const int qf = lb > p ? min(4, (lb - p + 31) / 32) : 0;  // live q's
                    uint8_t *piece = base + (int64_t)t * 512 + p * 16;
                    if (qf == 0) {
                        *reinterpret_cast<u32x4 *>(piece) = u32x4{0, 0, 0, 0};
                    } else {
                        for (int q = qf; q < 4; ++q)
                            *reinterpret_cast<uint32_t *>(piece + q * 4) = 0u;
                    }
                }
                continue;  // uniform over the workgroup
            }
        }
        // live rows of the unit, in order; nq[q] of them in line-set row q
        constexpr int kSeg = SUB * 16;  // bytes of each tile the unit fills
        int nq[4] = {0, 0, 0, 0};
        int n_live;
        int band = 0, h = 0, sub = 0;
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED && !kScatter) {
            constexpr int kPerBand = 32 / SUB;
            band = lu / kPerBand;
            h = (lu % kPerBand) / (8 / SUB);
            sub = lu % (8 / SUB);
            const int rb = min(128, m - band * 128);
            n_live = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                nq[q] = min(SUB, max(0, rb - 32 * q - 8 * h - SUB * sub));
                n_live += nq[q];
            }
        } else {
            n_live = min(kUnit, m - lu * kUnit);
        }
        // j-th live row of the unit -> (line-set row q, slot i, row in expert)
        auto locate = [&](int j, int &q, int &i) {
            q = 0;
            i = j;
            if constexpr (LAYOUT == MXQ_SF_SWIZZLED && !kScatter) {
                while (i >= nq[q]) { i -= nq[q]; ++q; }
                return band * 128 + 32 * q + 8 * h + SUB * sub + i;
            } else {
                return lu * kUnit + j;
            }
        };
        auto load_row = [&](int j, u32x4 *v) {
            int q, i;
            const uint16_t *src = a.src + (e0 + locate(j, q, i)) * a.cols;
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                v[k] = u32x4{0, 0, 0, 0};
                if (col < a.cols)
                    v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + col));
            }
        };
        u32x4 cur[NCH2];
        // this wave's half-row amax (columns past the row were loaded as zeros)
        auto half_amax = [&]() {
            uint32_t am = 0;
#pragma unroll
            for (int k = 0; k < NCH2; ++k) am = max(am, amax_bits8(cur[k]));
            return wave_max(am);
        };
        // encode the half row in cur as live row j under (gr, qr); whole wave.
        // am accumulates the half row's amax bits over the live columns.
        auto encode = [&](int j, float gr, float qr, uint32_t &am) {
            int q, i;
            const int r = locate(j, q, i);
            uint8_t *pay_row = a.payload + (e0 + r) * payload_ld;
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                u32x2 pay;
                const uint32_t code = quant8<FMT>(cur[k], gr, qr, pay);
                if (col < a.cols) {
                    store_payload<FMT>(pay_row, col, pay);
                    if (!ROWSC) am = max(am, amax_bits8(cur[k]));
                    if (leader) {
                        const int c = col / Tr::kBlock;
                        if constexpr (kScatter)
                            stage[j * a.sf_stride + c] = (uint8_t)code;
                        else if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
                            stage[(c >> 2) * kSeg + i * 16 + q * 4 + (c & 3)] = (uint8_t)code;
                        else
                            stage[j * a.sf_cols + c] = (uint8_t)code;
                    }
                }
            }
            return r;
        };

        if (pair < n_live) load_row(pair, cur);
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            for (int k = threadIdx.x * 16; k < stage_bytes; k += kSplitThreads * 16)
                *reinterpret_cast<u32x4 *>(stage + k) = u32x4{0, 0, 0, 0};
        }
        if (!ROWSC && threadIdx.x < kUnit) row_max[threadIdx.x] = 0;
        __syncthreads();
        if constexpr (!ROWSC) {
            for (int j = pair; j < n_live; j += 4) {
                uint32_t am = 0;
                encode(j, g, quot, am);
                am = wave_max(am);
                if (lane == 0) atomicMax(&row_max[j], am);
                if (j + 4 < n_live) load_row(j + 4, cur);
            }
        } else {
            // Every wave takes every step (the barrier needs all of them); a
            // row's two halves meet in half_max before either is encoded.
            for (int j0 = 0; j0 < n_live; j0 += 4, ++it) {
                const int j = j0 + pair;
                const uint32_t am = j < n_live ? half_amax() : 0u;
                if (lane == 0) half_max[it & 1][w] = am;
                __syncthreads();
                if (j < n_live) {
                    const uint32_t ra = max(half_max[it & 1][2 * pair], half_max[it & 1][2 * pair + 1]);
                    const float af = __uint_as_float(ra << 16);
                    const float gr = nv_encode_scale(af);
                    uint32_t unused = 0;
                    const int r = encode(j, gr, nv_wave_quot(gr), unused);
                    if (a.row_amax && half == 0 && lane == 0) a.row_amax[e0 + r] = af;
                }
                if (j + 4 < n_live) load_row(j + 4, cur);
            }
        }
        __syncthreads();
        if (!ROWSC && a.row_amax && (int)threadIdx.x < n_live) {
            int q, i;
            const int r = locate(threadIdx.x, q, i);
            a.row_amax[e0 + r] = __uint_as_float(row_max[threadIdx.x] << 16);
        }
        if constexpr (kScatter) {
            // row rl's codes of tile t: the 4-byte piece (rl % 32, rl / 32 % 4)
            uint8_t *region = a.scales + (int64_t)a.band_off[s] * tiles * 512;
            for (int k = threadIdx.x; k < n_live * tiles; k += kSplitThreads) {
                const int j = k / tiles, t = k - (k / tiles) * tiles;
                const int rl = lu * kUnit + j;
                *reinterpret_cast<uint32_t *>(region + (int64_t)(rl >> 7) * tiles * 512 +
                                              (int64_t)t * 512 + (rl & 31) * 16 +
                                              ((rl >> 5) & 3) * 4) =
                    *reinterpret_cast<const uint32_t *>(stage + j * a.sf_stride + t * 4);
            }
        } else if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            const int64_t first_band = a.unit_off[s] / (32 / SUB);
            uint8_t *base = a.scales + (first_band + band) * tiles * 512 + h * 128 + sub * kSeg;
            for (int k = threadIdx.x; k < tiles * SUB; k += kSplitThreads) {
                const int t = k / SUB, part = k % SUB;
                *reinterpret_cast<u32x4 *>(base + (int64_t)t * 512 + part * 16) =
                    *reinterpret_cast<const u32x4 *>(stage + t * kSeg + part * 16);
            }
        } else {
            uint8_t *dst = a.scales + (e0 + lu * kUnit) * a.sf_cols;
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
template <int FMT, bool ROWSC, int LAYOUT, int SUB>
static void split_nch(const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kSplitThreads);
    switch (half_row_steps(a.cols)) {
    case 1: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 1, SUB>), gd, bd, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 2, SUB>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 4, SUB>), gd, bd, lds, s, a); break;
    case 7: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 7, SUB>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 8, SUB>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_split<FMT, ROWSC, LAYOUT, 16, SUB>), gd, bd, lds, s, a); break;
    }
}

template <int FMT, bool ROWSC>
static void split_layout(int layout, const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    if (layout == MXQ_SF_LINEAR)
        split_nch<FMT, ROWSC, MXQ_SF_LINEAR, 2>(a, gd, lds, s);
    else if (a.sub == 2)
        split_nch<FMT, ROWSC, MXQ_SF_SWIZZLED, 2>(a, gd, lds, s);
    else
        split_nch<FMT, ROWSC, MXQ_SF_SWIZZLED, 0>(a, gd, lds, s);
}

hipError_t launch_split(int fmt, bool row_scaled, int layout, const SplitArgs &a, int64_t grid,
                        hipStream_t s) {
    const size_t lds = (size_t)(a.sub == 0 ? 8 : 4 * a.sub) * a.sf_stride;
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
