// mxq_kernels.hip -- gfx950 kernels for grouped / split block quantization,
// the fused residual + RMSNorm + quantize epilogue, and the scale swizzle.
//
// All of this is streaming work bounded by HBM bandwidth, so the kernels are
// shaped like a well-behaved copy: many small workgroups, every load of a
// workgroup issued before any of its stores, 16 contiguous bytes per lane
// (a wave load is 1 KiB of one row), and each lane's output bytes contiguous.
//
// Grouped (k_grouped): a work unit is 4*kRowsPerWave rows x 512 columns of
// one expert, kRowsPerWave rows per wave.  A block of 32 (MXFP8) or 16 (NVFP4) elements spans 4 or 2
// adjacent lanes; its amax is reduced with DPP quad permutes, never through
// LDS.  Payload bytes go straight to HBM; scale bytes are staged in LDS.  With
// the swizzled layout the unit's rows are band*128 + 32*wave + R*h + i
// (R = kRowsPerWave, i < R) of one 128-row band, which fill one contiguous
// R*16-byte segment of each 512-byte tile the chunk touches (a whole 128-byte
// line for R = 8), so scales leave in whole segments, padding included.
//
// Split and fused (k_split, k_fused): they need whole rows (row amax, the
// RMSNorm sum of squares), so one wave owns one row and holds all of it in
// registers; a unit is 4 rows.  Fused swizzled units take rows band*128 +
// 32*wave + gi (gi = 0..31), so a unit writes one 16-byte piece of each tile
// line (8 consecutive units complete it).
// Split units take 4 consecutive rows of one expert, so short experts keep
// every wave busy.
//
// Grouped and fused: unit u runs on workgroup u, in plain dispatch order; the
// hardware spreads consecutive workgroups over the 8 XCDs, so the units in
// flight cover one contiguous stretch of every tensor (measured faster than
// giving each XCD a contiguous range).  Split: each XCD takes a contiguous
// range of units, so the 4-row units that share a scale-tile line write it
// through the same L2 (measured twice as fast there).  No atomics, no scratch, no inter-workgroup
// ordering: every byte has one writer, and the bytes do not depend on the grid
// size.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

template <int FMT>
struct FmtTraits;
template <>
struct FmtTraits<MXQ_MXFP8> {
    static constexpr int kBlock = 32;
    static constexpr int kLanesPerBlock = 4;
};
template <>
struct FmtTraits<MXQ_NVFP4> {
    static constexpr int kBlock = 16;
    static constexpr int kLanesPerBlock = 2;
};

// Quantize one lane's 8 elements; the lanes of a block cooperate through DPP
// (all lanes of a block must be active).  Returns the block's scale byte
// (every lane of the block holds it) and the lane's payload: 8 bytes (MXFP8)
// or 4 bytes in pay.x (NVFP4).
template <int FMT>
__device__ __forceinline__ uint32_t quant8(u32x4 v, float g, u32x2 &pay) {
    uint32_t a = amax_bits8(v);
    if constexpr (FMT == MXQ_MXFP8) {
        a = block_max4(a);
        const uint32_t c = mx_scale_code(a);
        pay = mx_encode8(v, c);
        return c;
    } else {
        a = block_max2(a);
        const Nv4Scale s = nv_scale(a, g);
        pay.x = nv_encode8(v, s.mult);
        pay.y = 0;
        return s.code;
    }
}

// Payload bytes are written once and not read back by this kernel: streaming
// (non-temporal) stores keep them from displacing cache lines.
template <int FMT>
__device__ __forceinline__ void store_payload(uint8_t *row_payload, int col, u32x2 pay) {
    if constexpr (FMT == MXQ_MXFP8)
        __builtin_nontemporal_store(pay, reinterpret_cast<u32x2 *>(row_payload + col));
    else
        __builtin_nontemporal_store(pay.x, reinterpret_cast<uint32_t *>(row_payload + (col >> 1)));
}

// Workgroup b -> unit such that each XCD (workgroup b runs on XCD b mod 8)
// walks a contiguous range of units; bijective on [0, n).
__device__ __forceinline__ int xcd_unit(int b, int n) {
    const int q = n >> 3, r = n & 7, x = b & 7;
    return x * q + min(x, r) + (b >> 3);
}

// Copy n staged bytes to global memory (any alignment of dst).
__device__ __forceinline__ void copy_out(uint8_t *dst, const uint8_t *src, int n) {
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        const int nv = n >> 4;
        for (int k = threadIdx.x; k < nv; k += kThreads)
            *reinterpret_cast<u32x4 *>(dst + k * 16) = *reinterpret_cast<const u32x4 *>(src + k * 16);
        for (int k = (nv << 4) + threadIdx.x; k < n; k += kThreads) dst[k] = src[k];
    } else {
        for (int k = threadIdx.x; k < n; k += kThreads) dst[k] = src[k];
    }
}

// ---------------------------------------------------------------------------
// Grouped: 1..16 experts, one launch, the descriptor table in kernel args.
// ---------------------------------------------------------------------------
// Row groups of a 128-row band (swizzled): 32 / kRowsPerWave.
constexpr int kGroupsPerBand = 32 / kRowsPerWave;

template <int LAYOUT>
__device__ __forceinline__ int group_row(int rg, int q, int i) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        return (rg / kGroupsPerBand) * 128 + 32 * q + kRowsPerWave * (rg % kGroupsPerBand) + i;
    else
        return rg * kUnitRows + kRowsPerWave * q + i;
}

template <int FMT, int LAYOUT>
__global__ __launch_bounds__(kThreads) void k_grouped(const GroupArgs a) {
    using Tr = FmtTraits<FMT>;
    constexpr int kCodes = kChunk / Tr::kBlock;  // scale codes per row per unit: 16 or 32
    constexpr int kSegBytes = kRowsPerWave * 16;   // bytes of one tile line the unit fills
    __shared__ __align__(16) uint8_t stage[kUnitRows * kCodes];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    const int cl = lane * 8 / Tr::kBlock;  // this lane's code column inside the unit
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? a.cols : a.cols / 2;
    for (int u = blockIdx.x; u < a.total_units; u += gridDim.x) {
        int ei = 0;
        while (ei + 1 < a.n && u >= a.e[ei + 1].unit_begin) ++ei;
        const GEntry &E = a.e[ei];
        const int lu = u - E.unit_begin;
        const int rg = lu / a.n_cc;
        const int cc = lu - rg * a.n_cc;
        const int col = cc * kChunk + lane * 8;
        const bool live_col = col < a.cols;
        const float g = FMT == MXQ_NVFP4 ? *E.g : 0.0f;

        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            if (r < E.rows && live_col)
                v[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(E.src + (int64_t)r * E.ld + col));
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            uint32_t code = 0;  // rows and columns past the tensor stage zeros
            if (r < E.rows && live_col) {
                u32x2 pay;
                code = quant8<FMT>(v[i], g, pay);
                store_payload<FMT>(E.payload + (int64_t)r * payload_ld, col, pay);
            }
            if (leader) {
                if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
                    stage[(cl >> 2) * kSegBytes + i * 16 + q * 4 + (cl & 3)] = (uint8_t)code;
                else
                    stage[(kRowsPerWave * q + i) * kCodes + cl] = (uint8_t)code;
            }
        }
        __syncthreads();
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            // the unit's segment of each tile this chunk touches:
            // (kCodes/4) tiles x kRowsPerWave x 16 bytes
            const int tiles = a.sf_stride >> 2;
            const int t0 = cc * (kCodes / 4);
            const int k = threadIdx.x;
            if (k < (kCodes / 4) * kRowsPerWave) {
                const int tl = k / kRowsPerWave, part = k % kRowsPerWave;
                if (t0 + tl < tiles) {
                    uint8_t *dst = E.scales +
                                   ((int64_t)(rg / kGroupsPerBand) * tiles + t0 + tl) * 512 +
                                   (rg % kGroupsPerBand) * kSegBytes + part * 16;
                    *reinterpret_cast<u32x4 *>(dst) =
                        *reinterpret_cast<const u32x4 *>(stage + tl * kSegBytes + part * 16);
                }
            }
        } else {
            const int c0 = cc * kCodes;
            const int ncodes = min(kCodes, a.sf_cols - c0);
            constexpr int kParts = kCodes / 16;
            for (int k = threadIdx.x; k < kUnitRows * kParts; k += kThreads) {
                const int rl = k / kParts, part = k % kParts;
                const int r = rg * kUnitRows + rl;
                if (r >= E.rows) continue;
                uint8_t *dst = E.scales + (int64_t)r * a.sf_cols + c0 + part * 16;
                const uint8_t *src = stage + rl * kCodes + part * 16;
                if (ncodes == kCodes && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
                    *reinterpret_cast<u32x4 *>(dst) = *reinterpret_cast<const u32x4 *>(src);
                } else {
                    for (int j = 0; j < 16 && part * 16 + j < ncodes; ++j) dst[j] = src[j];
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Row-per-wave units (split, fused): 4 rows per workgroup, one per wave.
// Staged scales: swizzled [tile][wave][4] (16 bytes per tile), linear
// [wave][C].
// ---------------------------------------------------------------------------
template <int LAYOUT>
__device__ __forceinline__ int wave_row(int lu, int q) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        return (lu >> 5) * 128 + 32 * q + (lu & 31);
    else
        return lu * 4 + q;
}

template <int LAYOUT>
__device__ __forceinline__ void stage_code(uint8_t *stage, int q, int c, int sf_cols,
                                           uint32_t code) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        stage[(c >> 2) * 16 + q * 4 + (c & 3)] = (uint8_t)code;
    else
        stage[q * sf_cols + c] = (uint8_t)code;
}

// Write a 4-row unit's staged scales into a scale matrix region of `rows` rows.
template <int LAYOUT>
__device__ __forceinline__ void flush_rows4(const uint8_t *stage, uint8_t *region, int lu,
                                            int rows, int sf_cols, int sf_stride) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
        const int tiles = sf_stride >> 2;
        uint8_t *base = region + (int64_t)(lu >> 5) * tiles * 512 + (lu & 31) * 16;
        for (int t = threadIdx.x; t < tiles; t += kThreads)
            *reinterpret_cast<u32x4 *>(base + (int64_t)t * 512) =
                *reinterpret_cast<const u32x4 *>(stage + t * 16);
    } else {
        const int live = min(4, rows - lu * 4);
        copy_out(region + (int64_t)lu * 4 * sf_cols, stage, live * sf_cols);
    }
}

// Split units are 4 consecutive rows of one expert (short experts would leave
// waves idle under the interleaved order).  Swizzled scales of such a unit
// form one dword per row in each tile.
__device__ __forceinline__ void flush_split_swz(const uint8_t *stage, uint8_t *region, int lu,
                                                int sf_stride) {
    const int tiles = sf_stride >> 2;
    const int r0 = lu * 4;
    uint8_t *base = region + (int64_t)(r0 >> 7) * tiles * 512 + ((r0 & 127) >> 5) * 4;
    for (int k = threadIdx.x; k < tiles * 4; k += kThreads) {
        const int t = k >> 2, qq = k & 3;
        *reinterpret_cast<uint32_t *>(base + (int64_t)t * 512 + ((r0 & 31) + qq) * 16) =
            *reinterpret_cast<const uint32_t *>(stage + t * 16 + qq * 4);
    }
}

// Split: quantize rows of one expert's slice; NCH 512-column steps per row.
template <int LAYOUT, int NCH>
__global__ __launch_bounds__(kThreads) void k_split(const SplitArgs a) {
    extern __shared__ __align__(16) uint8_t stage[];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    const int64_t payload_ld = a.cols / 2;
    const float g = *a.g;
    for (int b = blockIdx.x; b < a.total_units; b += gridDim.x) {
        const int u = (int)gridDim.x == a.total_units ? xcd_unit(b, a.total_units) : b;
        int lo = 0, hi = a.n;  // split s with unit_off[s] <= u < unit_off[s + 1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.unit_off[mid] <= u) lo = mid; else hi = mid;
        }
        const int s = lo;
        const int lu = u - a.unit_off[s];
        const int m = a.row_off[s + 1] - a.row_off[s];
        const int64_t r0 = a.row_off[s];
        const int r = lu * 4 + q;
        if (r < m) {
            const uint16_t *src = a.src + (r0 + r) * a.cols;
            u32x4 v[NCH];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < a.cols)
                    v[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src + col));
            }
            uint8_t *pay_row = a.payload + (r0 + r) * payload_ld;
            uint32_t amax = 0;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < a.cols) {
                    u32x2 pay;
                    const uint32_t code = quant8<MXQ_NVFP4>(v[ch], g, pay);
                    store_payload<MXQ_NVFP4>(pay_row, col, pay);
                    amax = max(amax, amax_bits8(v[ch]));
                    if ((lane & 1) == 0) stage_code<LAYOUT>(stage, q, col / 16, a.sf_cols, code);
                } else if ((lane & 1) == 0 && col / 16 < a.sf_stride) {
                    stage_code<LAYOUT>(stage, q, col / 16, a.sf_cols, 0);
                }
            }
            amax = wave_max(amax);
            if (a.row_amax && lane == 0) a.row_amax[r0 + r] = __uint_as_float(amax << 16);
        } else if (LAYOUT == MXQ_SF_SWIZZLED) {
            for (int c = lane; c < a.sf_stride; c += kWave) stage_code<LAYOUT>(stage, q, c, a.sf_cols, 0);
        }
        __syncthreads();
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
            flush_split_swz(stage, a.scales + (int64_t)a.unit_off[s] * 4 * a.sf_stride, lu,
                            a.sf_stride);
        else
            flush_rows4<LAYOUT>(stage, a.scales + r0 * a.sf_cols, lu, m, a.sf_cols, a.sf_stride);
        __syncthreads();
    }
}

// Fused residual add + RMSNorm + quantize, one row per wave.  The row's bf16
// residual sum stays in registers; the sum of squares is reduced across the
// wave in a fixed order; norm_out and the quantized form come from the same
// bf16 values.
template <int FMT, int LAYOUT, int NCH>
__global__ __launch_bounds__(kThreads) void k_fused(const FusedArgs a) {
    using Tr = FmtTraits<FMT>;
    extern __shared__ __align__(16) uint8_t stage[];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    const int H = a.H;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? H : H / 2;
    const float g = FMT == MXQ_NVFP4 ? *a.g : 0.0f;
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    for (int lu = blockIdx.x; lu < a.total_units; lu += gridDim.x) {
        const int r = wave_row<LAYOUT>(lu, q);
        if (r < a.T) {
            const int64_t rb = (int64_t)r * H;
            u32x4 xv[NCH], rv[NCH];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < H) {
                    xv[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + rb + col));
                    rv[ch] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.res + rb + col));
                }
            }
            float acc = 0.0f;
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < H) {
                    u32x4 sum;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t blo = f32_to_bf16(bf16_lo(xv[ch][j]) + bf16_lo(rv[ch][j]));
                        const uint32_t bhi = f32_to_bf16(bf16_hi(xv[ch][j]) + bf16_hi(rv[ch][j]));
                        const float flo = __uint_as_float(blo << 16);
                        const float fhi = __uint_as_float(bhi << 16);
                        acc = __builtin_fmaf(flo, flo, acc);
                        acc = __builtin_fmaf(fhi, fhi, acc);
                        sum[j] = blo | (bhi << 16);
                    }
                    xv[ch] = sum;  // the bf16 residual sum
                    *reinterpret_cast<u32x4 *>(a.res_out + rb + col) = sum;
                }
            }
            const float inv = 1.0f / __builtin_sqrtf(wave_sum(acc) / (float)H + a.eps);
            u32x4 gm[NCH];
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < H) gm[ch] = *reinterpret_cast<const u32x4 *>(a.gamma + col);
            }
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < H) {
                    u32x4 nv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float nlo = (bf16_lo(xv[ch][j]) * bf16_lo(gm[ch][j])) * inv;
                        const float nhi = (bf16_hi(xv[ch][j]) * bf16_hi(gm[ch][j])) * inv;
                        nv[j] = pack_bf16(nlo, nhi);
                    }
                    *reinterpret_cast<u32x4 *>(a.norm_out + rb + col) = nv;
                    u32x2 pay;
                    const uint32_t code = quant8<FMT>(nv, g, pay);
                    store_payload<FMT>(a.payload + (int64_t)r * payload_ld, col, pay);
                    if (leader) stage_code<LAYOUT>(stage, q, col / Tr::kBlock, a.sf_cols, code);
                }
            }
        } else if (LAYOUT == MXQ_SF_SWIZZLED) {
            for (int c = lane; c < a.sf_stride; c += kWave) stage_code<LAYOUT>(stage, q, c, a.sf_cols, 0);
        }
        __syncthreads();
        flush_rows4<LAYOUT>(stage, a.scales, lu, a.T, a.sf_cols, a.sf_stride);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Linear -> swizzled scale layout.  One thread per 16-byte output vector:
// rows 32*q + i (q = 0..3) of a 128-row band, 4 columns each; padding is 0.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_swizzle(const SwizzleArgs a) {
    for (int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x; k < a.n_vec;
         k += (int64_t)gridDim.x * kThreads) {
        const int64_t tile = k >> 5;
        const int i = (int)(k & 31);
        const int64_t band = tile / a.tiles_per_band;
        const int64_t c0 = (tile % a.tiles_per_band) * 4;
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t r = band * 128 + 32 * q + i;
            uint32_t word = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t c = c0 + j;
                if (r < a.rows && c < a.cols) word |= (uint32_t)a.lin[r * a.cols + c] << (8 * j);
            }
            w[q] = word;
        }
        *reinterpret_cast<u32x4 *>(a.swz + k * 16) = u32x4{w[0], w[1], w[2], w[3]};
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static inline unsigned grid_of(int64_t g) { return (unsigned)(g < 1 ? 1 : g); }

hipError_t launch_grouped(int fmt, int layout, const GroupArgs &a, int64_t grid, hipStream_t s) {
    const dim3 gd(grid_of(grid)), bd(kThreads);
    if (fmt == MXQ_MXFP8 && layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_LINEAR>), gd, bd, 0, s, a);
    else if (fmt == MXQ_MXFP8)
        hipLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_SWIZZLED>), gd, bd, 0, s, a);
    else if (layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_LINEAR>), gd, bd, 0, s, a);
    else
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_SWIZZLED>), gd, bd, 0, s, a);
    return hipGetLastError();
}

// Row-per-wave kernels keep the whole row in registers: NCH 512-column steps.
int row_steps(int64_t cols) {
    const int64_t n = (cols + kChunk - 1) / kChunk;
    if (n <= 2) return 2;
    if (n <= 4) return 4;
    if (n <= 8) return 8;
    if (n <= 14) return 14;
    if (n <= 16) return 16;
    return 32;
}

template <int LAYOUT>
static void split_nch(const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kThreads);
    switch (row_steps(a.cols)) {
    case 2: hipLaunchKernelGGL((k_split<LAYOUT, 2>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_split<LAYOUT, 4>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_split<LAYOUT, 8>), gd, bd, lds, s, a); break;
    case 14: hipLaunchKernelGGL((k_split<LAYOUT, 14>), gd, bd, lds, s, a); break;
    case 16: hipLaunchKernelGGL((k_split<LAYOUT, 16>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_split<LAYOUT, 32>), gd, bd, lds, s, a); break;
    }
}

hipError_t launch_split(int layout, const SplitArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)4 * a.sf_stride;
    const dim3 gd(grid_of(grid));
    if (layout == MXQ_SF_LINEAR)
        split_nch<MXQ_SF_LINEAR>(a, gd, lds, s);
    else
        split_nch<MXQ_SF_SWIZZLED>(a, gd, lds, s);
    return hipGetLastError();
}

template <int FMT, int LAYOUT>
static void fused_nch(const FusedArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kThreads);
    switch (row_steps(a.H)) {
    case 2: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 2>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 4>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 8>), gd, bd, lds, s, a); break;
    case 14: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 14>), gd, bd, lds, s, a); break;
    case 16: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 16>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 32>), gd, bd, lds, s, a); break;
    }
}

hipError_t launch_fused(int fmt, int layout, const FusedArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)4 * a.sf_stride;
    const dim3 gd(grid_of(grid));
    if (fmt == MXQ_MXFP8 && layout == MXQ_SF_LINEAR)
        fused_nch<MXQ_MXFP8, MXQ_SF_LINEAR>(a, gd, lds, s);
    else if (fmt == MXQ_MXFP8)
        fused_nch<MXQ_MXFP8, MXQ_SF_SWIZZLED>(a, gd, lds, s);
    else if (layout == MXQ_SF_LINEAR)
        fused_nch<MXQ_NVFP4, MXQ_SF_LINEAR>(a, gd, lds, s);
    else
        fused_nch<MXQ_NVFP4, MXQ_SF_SWIZZLED>(a, gd, lds, s);
    return hipGetLastError();
}

hipError_t launch_swizzle(const SwizzleArgs &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL(k_swizzle, dim3(grid_of(grid)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace mxq
