// mxq_kernels.hip -- gfx950 kernels for grouped / split block quantization,
// the fused residual + RMSNorm + quantize epilogue, and the scale swizzle.
//
// Work decomposition (all quantize kernels): a workgroup of 4 waves takes a
// 32-row work unit; each wave owns 8 rows and streams them in 512-element
// steps, each lane loading 16 contiguous bytes (8 bf16), so a wave load is
// 1 KiB of one row.  A block of 32 (MXFP8) or 16 (NVFP4) elements spans 4 or
// 2 adjacent lanes; its amax is reduced with DPP quad permutes, never through
// LDS.  Payload bytes go straight to HBM (8 or 4 contiguous bytes per lane);
// scale bytes are staged in LDS and written out once per unit.  With the
// swizzled layout a unit takes rows band*128 + 32*wave + 8*g + i of one
// 128-row band, which fill exactly one full 128-byte line of every 512-byte
// tile, so the staged scales leave as whole lines, padding included.  No
// atomics, no scratch buffers, no inter-workgroup ordering: every byte has
// exactly one writer, and the result does not depend on the grid size.
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

// Quantize one lane's 8 elements; the lanes of a block cooperate through DPP.
// Returns the block's scale byte (every lane of the block holds it) and the
// lane's payload: 8 bytes (MXFP8) or 4 bytes in pay.x (NVFP4).
template <int FMT>
__device__ __forceinline__ uint32_t quant8(u32x4 v, float g, u32x2 &pay) {
    uint32_t a = amax_bits8(v);
    if constexpr (FMT == MXQ_MXFP8) {
        a = block_max4(a);
        uint32_t c = mx_scale_code(a);
        pay = mx_encode8(v, mx_multiplier(c));
        return c;
    } else {
        a = block_max2(a);
        Nv4Scale s = nv_scale(a, g);
        pay.x = nv_encode8(v, s.mult);
        pay.y = 0;
        return s.code;
    }
}

template <int FMT>
__device__ __forceinline__ void store_payload(uint8_t *row_payload, int col, u32x2 pay) {
    if constexpr (FMT == MXQ_MXFP8)
        *reinterpret_cast<u32x2 *>(row_payload + col) = pay;
    else
        *reinterpret_cast<uint32_t *>(row_payload + (col >> 1)) = pay.x;
}

// Row of the unit handled by wave q at slot i.
template <int LAYOUT>
__device__ __forceinline__ int unit_row(int lu, int q, int i) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        return (lu >> 2) * 128 + 32 * q + 8 * (lu & 3) + i;
    else
        return lu * kUnitRows + 8 * q + i;
}

template <int LAYOUT>
__device__ __forceinline__ int stage_index(int q, int i, int c, int sf_stride) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        return stage_index_swz(q, i, c);
    else
        return (8 * q + i) * sf_stride + c;
}

__device__ __forceinline__ void stage_zero(uint8_t *stage, int bytes) {
    for (int k = threadIdx.x * 16; k < bytes; k += kThreads * 16)
        *reinterpret_cast<u32x4 *>(stage + k) = u32x4{0, 0, 0, 0};
}

// Write a unit's staged scales.  Swizzled: line g of each of the band's
// tiles.  Linear: the unit's live rows, contiguous in the scale matrix.
template <int LAYOUT>
__device__ __forceinline__ void stage_flush(const uint8_t *stage, uint8_t *scales, int lu,
                                            int live_rows, int sf_cols, int sf_stride) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
        const int tiles = sf_stride >> 2;
        uint8_t *dst = scales + ((int64_t)(lu >> 2) * tiles) * 512 + (lu & 3) * 128;
        for (int k = threadIdx.x; k < tiles * 8; k += kThreads) {
            const int t = k >> 3, part = k & 7;
            *reinterpret_cast<u32x4 *>(dst + (int64_t)t * 512 + part * 16) =
                *reinterpret_cast<const u32x4 *>(stage + t * 128 + part * 16);
        }
    } else {
        const int n = live_rows * sf_cols;
        uint8_t *dst = scales + (int64_t)lu * kUnitRows * sf_cols;
        if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            const int nv = n >> 4;
            for (int k = threadIdx.x; k < nv; k += kThreads)
                *reinterpret_cast<u32x4 *>(dst + k * 16) =
                    *reinterpret_cast<const u32x4 *>(stage + k * 16);
            for (int k = (nv << 4) + threadIdx.x; k < n; k += kThreads) dst[k] = stage[k];
        } else {
            for (int k = threadIdx.x; k < n; k += kThreads) dst[k] = stage[k];
        }
    }
}

// Quantize the rows of one unit (wave q's 8 rows), staging scales.
// rows: live rows of the tensor; src/payload point at row 0.
template <int FMT, int LAYOUT, bool kRowAmax>
__device__ __forceinline__ void quant_unit_rows(const uint16_t *src, int64_t ld, uint8_t *payload,
                                                int64_t payload_ld, int rows, int cols, int lu,
                                                float g, uint8_t *stage, int sf_stride,
                                                float *row_amax) {
    using Tr = FmtTraits<FMT>;
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    uint32_t amax_row[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) amax_row[i] = 0;

    for (int c0 = 0; c0 < cols; c0 += kChunk) {
        const int col = c0 + lane * 8;
        const bool live_col = col < cols;
        u32x4 v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = unit_row<LAYOUT>(lu, q, i);
            if (r < rows && live_col)
                v[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(src + (int64_t)r * ld + col));
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = unit_row<LAYOUT>(lu, q, i);
            if (r < rows && live_col) {
                u32x2 pay;
                const uint32_t code = quant8<FMT>(v[i], g, pay);
                store_payload<FMT>(payload + (int64_t)r * payload_ld, col, pay);
                if ((lane & (Tr::kLanesPerBlock - 1)) == 0)
                    stage[stage_index<LAYOUT>(q, i, col / Tr::kBlock, sf_stride)] = (uint8_t)code;
                if constexpr (kRowAmax) amax_row[i] = max(amax_row[i], amax_bits8(v[i]));
            }
        }
    }
    if constexpr (kRowAmax) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int r = unit_row<LAYOUT>(lu, q, i);
            if (r < rows) {
                const uint32_t m = wave_max(amax_row[i]);
                if (lane == 0) row_amax[r] = __uint_as_float(m << 16);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Grouped: 1..16 experts, one launch, the descriptor table in kernel args.
// ---------------------------------------------------------------------------
template <int FMT, int LAYOUT>
__global__ __launch_bounds__(kThreads) void k_grouped(const GroupArgs a) {
    extern __shared__ __align__(16) uint8_t stage[];
    const int stage_bytes = kUnitRows * a.sf_stride;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? a.cols : a.cols / 2;
    for (int u = blockIdx.x; u < a.total_units; u += gridDim.x) {
        int ei = 0;
        while (ei + 1 < a.n && u >= a.e[ei + 1].unit_begin) ++ei;
        const GEntry &E = a.e[ei];
        const int lu = u - E.unit_begin;
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) stage_zero(stage, stage_bytes);
        __syncthreads();
        const float g = FMT == MXQ_NVFP4 ? *E.g : 0.0f;
        quant_unit_rows<FMT, LAYOUT, false>(E.src, E.ld, E.payload, payload_ld, E.rows, a.cols, lu,
                                            g, stage, a.sf_stride, nullptr);
        __syncthreads();
        stage_flush<LAYOUT>(stage, E.scales, lu, min(kUnitRows, E.rows - lu * kUnitRows),
                            a.sf_cols, a.sf_stride);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Split: one concatenated activation, per-expert units and scale regions.
// ---------------------------------------------------------------------------
template <int LAYOUT>
__global__ __launch_bounds__(kThreads) void k_split(const SplitArgs a) {
    extern __shared__ __align__(16) uint8_t stage[];
    const int stage_bytes = kUnitRows * a.sf_stride;
    const int64_t payload_ld = a.cols / 2;
    const float g = *a.g;
    for (int u = blockIdx.x; u < a.total_units; u += gridDim.x) {
        // split s with unit_off[s] <= u < unit_off[s+1] (binary search)
        int lo = 0, hi = a.n;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (a.unit_off[mid] <= u) lo = mid; else hi = mid;
        }
        const int s = lo;
        const int lu = u - a.unit_off[s];
        const int m = a.row_off[s + 1] - a.row_off[s];
        const int64_t r0 = a.row_off[s];
        uint8_t *scales = LAYOUT == MXQ_SF_SWIZZLED
                              ? a.scales + (int64_t)a.unit_off[s] * kUnitRows * a.sf_stride
                              : a.scales + r0 * a.sf_cols;
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) stage_zero(stage, stage_bytes);
        __syncthreads();
        if (a.row_amax)
            quant_unit_rows<MXQ_NVFP4, LAYOUT, true>(a.src + r0 * a.cols, a.cols,
                                                     a.payload + r0 * payload_ld, payload_ld, m,
                                                     a.cols, lu, g, stage, a.sf_stride,
                                                     a.row_amax + r0);
        else
            quant_unit_rows<MXQ_NVFP4, LAYOUT, false>(a.src + r0 * a.cols, a.cols,
                                                      a.payload + r0 * payload_ld, payload_ld, m,
                                                      a.cols, lu, g, stage, a.sf_stride, nullptr);
        __syncthreads();
        stage_flush<LAYOUT>(stage, scales, lu, min(kUnitRows, m - lu * kUnitRows), a.sf_cols,
                            a.sf_stride);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Fused residual add + RMSNorm + quantize.  A wave owns whole rows: it keeps
// the row's bf16 residual sum in registers (NCH 512-element steps), reduces
// the sum of squares across the wave in a fixed order, then writes norm_out
// and quantizes the same bf16 values.
// ---------------------------------------------------------------------------
template <int FMT, int LAYOUT, int NCH>
__global__ __launch_bounds__(kThreads) void k_fused(const FusedArgs a) {
    using Tr = FmtTraits<FMT>;
    extern __shared__ __align__(16) uint8_t stage[];
    const int stage_bytes = kUnitRows * a.sf_stride;
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    const int H = a.H;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? H : H / 2;
    const float g = FMT == MXQ_NVFP4 ? *a.g : 0.0f;
    for (int u = blockIdx.x; u < a.total_units; u += gridDim.x) {
        const int lu = u;
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) stage_zero(stage, stage_bytes);
        __syncthreads();
        for (int i = 0; i < 8; ++i) {
            const int r = unit_row<LAYOUT>(lu, q, i);
            if (r >= a.T) continue;  // uniform across the wave
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
                    xv[ch] = sum;  // keep the bf16 residual sum
                    *reinterpret_cast<u32x4 *>(a.res_out + rb + col) = sum;
                }
            }
            const float ss = wave_sum(acc);
            const float inv = 1.0f / __builtin_sqrtf(ss / (float)H + a.eps);
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
                const int col = ch * kChunk + lane * 8;
                if (col < H) {
                    const u32x4 gm = *reinterpret_cast<const u32x4 *>(a.gamma + col);
                    u32x4 nv;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float nlo = (bf16_lo(xv[ch][j]) * bf16_lo(gm[j])) * inv;
                        const float nhi = (bf16_hi(xv[ch][j]) * bf16_hi(gm[j])) * inv;
                        nv[j] = pack_bf16(nlo, nhi);
                    }
                    *reinterpret_cast<u32x4 *>(a.norm_out + rb + col) = nv;
                    u32x2 pay;
                    const uint32_t code = quant8<FMT>(nv, g, pay);
                    store_payload<FMT>(a.payload + (int64_t)r * payload_ld, col, pay);
                    if ((lane & (Tr::kLanesPerBlock - 1)) == 0)
                        stage[stage_index<LAYOUT>(q, i, col / Tr::kBlock, a.sf_stride)] =
                            (uint8_t)code;
                }
            }
        }
        __syncthreads();
        stage_flush<LAYOUT>(stage, a.scales, lu, min(kUnitRows, a.T - lu * kUnitRows), a.sf_cols,
                            a.sf_stride);
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
    const size_t lds = (size_t)kUnitRows * a.sf_stride;
    const dim3 gd(grid_of(grid)), bd(kThreads);
    if (fmt == MXQ_MXFP8 && layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_LINEAR>), gd, bd, lds, s, a);
    else if (fmt == MXQ_MXFP8)
        hipLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_SWIZZLED>), gd, bd, lds, s, a);
    else if (layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_LINEAR>), gd, bd, lds, s, a);
    else
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_SWIZZLED>), gd, bd, lds, s, a);
    return hipGetLastError();
}

hipError_t launch_split(int layout, const SplitArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)kUnitRows * a.sf_stride;
    const dim3 gd(grid_of(grid)), bd(kThreads);
    if (layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_split<MXQ_SF_LINEAR>), gd, bd, lds, s, a);
    else
        hipLaunchKernelGGL((k_split<MXQ_SF_SWIZZLED>), gd, bd, lds, s, a);
    return hipGetLastError();
}

template <int FMT, int LAYOUT>
static void fused_nch(const FusedArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const int nch = (a.H + kChunk - 1) / kChunk;
    const dim3 bd(kThreads);
    if (nch <= 2)
        hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 2>), gd, bd, lds, s, a);
    else if (nch <= 4)
        hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 4>), gd, bd, lds, s, a);
    else if (nch <= 8)
        hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 8>), gd, bd, lds, s, a);
    else if (nch <= 16)
        hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 16>), gd, bd, lds, s, a);
    else
        hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 32>), gd, bd, lds, s, a);
}

hipError_t launch_fused(int fmt, int layout, const FusedArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)kUnitRows * a.sf_stride;
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
