// mxq_fused.hip -- the fused residual add + RMSNorm + quantize epilogue, and
// the linear -> swizzled scale conversion.
//
// The epilogue needs whole rows (the RMSNorm sum of squares): two, four or
// sixteen waves own one row and hold it in registers.  A unit is RPU
// consecutive rows; swizzled units cover the padding rows up to the next
// multiple of 128 too.  Every byte has one writer.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

// ---------------------------------------------------------------------------
// WPR waves share each row, wave `part` holding the 512-column steps
// WPR*k + part of it in registers.  gamma is staged in LDS by the
// workgroup's first unit with a live row, after that unit's row loads are
// issued (measured 0.6-0.9 us faster at T = 1024-4096 than staging first);
// units that hold only padding rows never load it.  Each unit's codes are
// staged in LDS too, one row per sf_stride bytes.
// ---------------------------------------------------------------------------

// Copy n staged bytes to global memory with the whole workgroup (NT threads).
template <int NT>
__device__ __forceinline__ void copy_out_rows(uint8_t *dst, const uint8_t *src, int n) {
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        const int nv = n >> 4;
        for (int k = threadIdx.x; k < nv; k += NT)
            *reinterpret_cast<u32x4 *>(dst + k * 16) = *reinterpret_cast<const u32x4 *>(src + k * 16);
        for (int k = (nv << 4) + threadIdx.x; k < n; k += NT) dst[k] = src[k];
    } else {
        for (int k = threadIdx.x; k < n; k += NT) dst[k] = src[k];
    }
}

// Fused residual add + RMSNorm + quantize.  The row's bf16 residual sum stays
// in registers; the sum of squares is each wave's fixed-order partial, the
// row's WPR partials added in wave order; norm_out and the quantized form come
// from the same bf16 values.  NCHW: 512-column steps per wave.  A unit is RPU
// consecutive rows; swizzled codes leave as each row's 4-byte slot of every
// tile, consecutive lanes taking consecutive rows (whose slots share 16-byte
// lines), and the units that share lines run on one XCD.  With two waves per
// row the kernel is held to 128 VGPRs.
template <int FMT, int LAYOUT, int NCHW, int WPR, int RPU>
__global__ __launch_bounds__(RPU * WPR * kWave)
__attribute__((amdgpu_waves_per_eu(WPR == 2 ? 4 : 1)))
void k_fused(const FusedArgs a) {
    using Tr = FmtTraits<FMT>;
    constexpr int kNT = RPU * WPR * kWave;
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ float red[RPU * WPR];
    const int H = a.H;
    uint16_t *gamma_s = reinterpret_cast<uint16_t *>(smem);
    uint8_t *stage = smem + ((2 * H + 15) & ~15);
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int q = RPU == 1 ? 0 : w / WPR;  // the unit's row of this wave (0: scalar addresses)
    const int part = w % WPR;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? H : H / 2;
    const float g = FMT == MXQ_NVFP4 ? *a.g : 0.0f;
    const NvG G = nv_prepare(g);
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    bool staged = false;  // gamma is in LDS (uniform)
    for (int lu0 = blockIdx.x; lu0 < a.total_units; lu0 += gridDim.x) {
        int lu = lu0;
        int r;
        if (LAYOUT == MXQ_SF_SWIZZLED && RPU == 1) {
            // one-row units, a 128-row band's 128 units in the order of its
            // scale lines: the 16 units of each XCD group are the rows whose
            // codes fill 4 whole 16-byte lines (64 contiguous bytes of every
            // tile), rows p + 32 q for 4 consecutive p and q = 0..3, so one
            // L2 writes them whole
            if (xcd_grouping_holds(gridDim.x, a.total_units))
                lu = xcd_grouped_unit<16>(lu0, a.total_units);
            const int i = lu & 127, k = i >> 5, j = i & 31;
            r = (lu & ~127) + 8 * k + (j >> 2) + 32 * (j & 3);
        } else {
            // four-row units: the 8 consecutive rows whose codes share
            // 128-byte lines on one XCD
            if (LAYOUT == MXQ_SF_SWIZZLED && xcd_grouping_holds(gridDim.x, a.total_units))
                lu = xcd_grouped_unit<8 / RPU>(lu0, a.total_units);
            r = lu * RPU + q;
        }
        const bool live = r < a.T;
        const int r0 = RPU == 1 ? r : lu * RPU;  // the unit's first row
        const bool unit_live = r0 < a.T;  // uniform: any live row in the unit
        const bool stage_now = !staged && unit_live;
        const int64_t rb = (int64_t)r * H;
        u32x4 xv[NCHW];
        float acc = 0.0f;
        if (live) {
            u32x4 rv[NCHW];
#pragma unroll
            for (int k = 0; k < NCHW; ++k) {
                const int col = (WPR * k + part) * kChunk + lane * 8;
                if (col < H) {
                    xv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + rb + col));
                    rv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.res + rb + col));
                }
            }
            if (stage_now)  // H is a multiple of 16
                for (int k = threadIdx.x * 8; k < H; k += kNT * 8)
                    *reinterpret_cast<u32x4 *>(gamma_s + k) = *reinterpret_cast<const u32x4 *>(a.gamma + k);
#pragma unroll
            for (int k = 0; k < NCHW; ++k) {
                const int col = (WPR * k + part) * kChunk + lane * 8;
                if (col < H) {
                    u32x4 sum;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t blo = f32_to_bf16(bf16_lo(xv[k][j]) + bf16_lo(rv[k][j]));
                        const uint32_t bhi = f32_to_bf16(bf16_hi(xv[k][j]) + bf16_hi(rv[k][j]));
                        const float flo = __uint_as_float(blo << 16);
                        const float fhi = __uint_as_float(bhi << 16);
                        acc = __builtin_fmaf(flo, flo, acc);
                        acc = __builtin_fmaf(fhi, fhi, acc);
                        sum[j] = blo | (bhi << 16);
                    }
                    xv[k] = sum;  // the bf16 residual sum
                    __builtin_nontemporal_store(sum, reinterpret_cast<u32x4 *>(a.res_out + rb + col));
                }
            }
            acc = wave_sum(acc);
        } else if (stage_now) {  // a dead row of a unit with live rows
            for (int k = threadIdx.x * 8; k < H; k += kNT * 8)
                *reinterpret_cast<u32x4 *>(gamma_s + k) = *reinterpret_cast<const u32x4 *>(a.gamma + k);
        }
        staged = staged || unit_live;
        if (lane == 0) red[w] = acc;
        __syncthreads();  // the partial sums, and gamma in LDS
        if (live) {
            float ss = red[q * WPR];
#pragma unroll
            for (int p = 1; p < WPR; ++p) ss += red[q * WPR + p];
            const float inv = 1.0f / __builtin_sqrtf(ss / (float)H + a.eps);
#pragma unroll
            for (int k = 0; k < NCHW; ++k) {
                const int col = (WPR * k + part) * kChunk + lane * 8;
                u32x4 nv = u32x4{0, 0, 0, 0};
                if (col < H) {
                    const u32x4 gm = *reinterpret_cast<const u32x4 *>(gamma_s + col);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float nlo = (bf16_lo(xv[k][j]) * bf16_lo(gm[j])) * inv;
                        const float nhi = (bf16_hi(xv[k][j]) * bf16_hi(gm[j])) * inv;
                        nv[j] = pack_bf16(nlo, nhi);
                    }
                    __builtin_nontemporal_store(nv, reinterpret_cast<u32x4 *>(a.norm_out + rb + col));
                }
                u32x2 pay;
                const uint32_t code = quant8<FMT>(nv, G, pay);  // whole wave
                if (col < H) {
                    store_payload<FMT>(a.payload + (int64_t)r * payload_ld, col, pay);
                    if (leader) stage[q * a.sf_stride + col / Tr::kBlock] = (uint8_t)code;
                }
            }
        } else if (LAYOUT == MXQ_SF_SWIZZLED && part == 0) {
            for (int c = lane; c < a.sf_stride; c += kWave) stage[q * a.sf_stride + c] = 0;
        }
        __syncthreads();
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            // row r0 + j's 4 codes of tile t: one 4-byte slot per tile
            const int tiles = a.sf_stride >> 2;
            for (int k = threadIdx.x; k < tiles * RPU; k += kNT) {
                const int t = k / RPU, j = k % RPU, rr = r0 + j;
                uint8_t *dst = a.scales + ((int64_t)(rr >> 7) * tiles + t) * 512 + (rr & 31) * 16 +
                               ((rr >> 5) & 3) * 4;
                *reinterpret_cast<uint32_t *>(dst) =
                    *reinterpret_cast<const uint32_t *>(stage + j * a.sf_stride + t * 4);
            }
        } else if (r0 < a.T) {
            // linear: sf_stride == sf_cols, so the live rows' codes are contiguous
            copy_out_rows<kNT>(a.scales + (int64_t)r0 * a.sf_cols, stage,
                               min(RPU, a.T - r0) * a.sf_cols);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// A few rows, swizzled scales: one 1024-thread workgroup per live row (fewer
// than 32 rows, H up to 16 x 512), sixteen waves of one 512-column step each,
// and no units for the padding rows.  Each row is the only live row of its
// 16-byte scale line (line p = the row), so it writes its 4 codes of a tile
// with the zeros of the line's three padding slots in one store; the lines
// T..31 of every tile, which hold no live row, are zeroed by the same
// workgroups.  Only the XCDs that run a live row then fetch the code and
// gamma: at T = 1 one XCD instead of eight, FETCH + WRITE 1.07x the
// algorithmic bytes instead of 1.44-1.57x, in the same time.  A kernel of its
// own: the general kernel's code is larger, and at a few rows a launch costs
// little more than its instruction fetch and memory latency (the general
// kernel with this logic added ran 0.3 us slower at T = 1).  The arithmetic
// and the sum order are the general kernel's with sixteen waves per row.
// ---------------------------------------------------------------------------
template <int FMT>
__global__ __launch_bounds__(kFusedTinyThreads) void k_fused_tiny(const FusedArgs a) {
    using Tr = FmtTraits<FMT>;
    constexpr int kWaves = kFusedTinyThreads / kWave;
    constexpr int kLanesPerTile = 4 * Tr::kLanesPerBlock;  // 4 blocks of codes per tile
    __shared__ float red[kWaves];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int r = blockIdx.x;
    const int H = a.H;
    const int col = w * kChunk + lane * 8;
    const bool has = col < H;
    const int64_t rb = (int64_t)r * H;
    const float g = FMT == MXQ_NVFP4 ? *a.g : 0.0f;
    const NvG G = nv_prepare(g);
    u32x4 xv = u32x4{0, 0, 0, 0}, rv = u32x4{0, 0, 0, 0}, gm = u32x4{0, 0, 0, 0};
    if (has) {
        xv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + rb + col));
        rv = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.res + rb + col));
        gm = *reinterpret_cast<const u32x4 *>(a.gamma + col);
    }
    // lines T..31 of every tile hold no live row: zeroed here, between the
    // row's loads and their first use.  One counter tracks a wave's loads and
    // stores, so the wave waits for these stores with its loads, under whose
    // latency they complete; issued after the row (measured 0.1-0.2 us
    // slower) they would lengthen the launch's tail.
    const int tiles = a.sf_stride >> 2;
    const int ne = 32 - a.T;
    for (int k = r * kFusedTinyThreads + (int)threadIdx.x; k < tiles * ne;
         k += a.T * kFusedTinyThreads) {
        const int t = k / ne, p = a.T + k - t * ne;
        *reinterpret_cast<u32x4 *>(a.scales + (int64_t)t * 512 + p * 16) = u32x4{0, 0, 0, 0};
    }
    float acc = 0.0f;
    if (has) {
        u32x4 sum;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t blo = f32_to_bf16(bf16_lo(xv[j]) + bf16_lo(rv[j]));
            const uint32_t bhi = f32_to_bf16(bf16_hi(xv[j]) + bf16_hi(rv[j]));
            const float flo = __uint_as_float(blo << 16);
            const float fhi = __uint_as_float(bhi << 16);
            acc = __builtin_fmaf(flo, flo, acc);
            acc = __builtin_fmaf(fhi, fhi, acc);
            sum[j] = blo | (bhi << 16);
        }
        xv = sum;  // the bf16 residual sum
        __builtin_nontemporal_store(sum, reinterpret_cast<u32x4 *>(a.res_out + rb + col));
    }
    acc = wave_sum(acc);
    if (lane == 0) red[w] = acc;
    __syncthreads();
    float ss = red[0];
#pragma unroll
    for (int p = 1; p < kWaves; ++p) ss += red[p];
    const float inv = 1.0f / __builtin_sqrtf(ss / (float)H + a.eps);
    u32x4 nv = u32x4{0, 0, 0, 0};
    if (has) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float nlo = (bf16_lo(xv[j]) * bf16_lo(gm[j])) * inv;
            const float nhi = (bf16_hi(xv[j]) * bf16_hi(gm[j])) * inv;
            nv[j] = pack_bf16(nlo, nhi);
        }
        __builtin_nontemporal_store(nv, reinterpret_cast<u32x4 *>(a.norm_out + rb + col));
    }
    u32x2 pay;
    const uint32_t code = quant8<FMT>(nv, G, pay);  // whole wave
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? H : H / 2;
    if (has) store_payload<FMT>(a.payload + (int64_t)r * payload_ld, col, pay);
    // a tile's 4 codes come from the first lanes of its 4 blocks; its first
    // lane writes them with the line's zero slots (a tile lies wholly inside
    // or outside the row: C is a multiple of 4)
    const uint32_t c1 = __shfl(code, lane + Tr::kLanesPerBlock);
    const uint32_t c2 = __shfl(code, lane + 2 * Tr::kLanesPerBlock);
    const uint32_t c3 = __shfl(code, lane + 3 * Tr::kLanesPerBlock);
    if (has && lane % kLanesPerTile == 0) {
        const int t = (w * kChunk + lane * 8) / (4 * Tr::kBlock);
        *reinterpret_cast<u32x4 *>(a.scales + (int64_t)t * 512 + r * 16) =
            u32x4{code | (c1 << 8) | (c2 << 16) | (c3 << 24), 0, 0, 0};
    }
}

// ---------------------------------------------------------------------------
// Linear -> swizzled scale layout.  A unit is one 128-row band by up to
// kSwizzleTiles tiles (4 scale columns each): its linear codes are read row
// by row into LDS, then its tiles leave as one contiguous run of 16-byte
// lines.  Rows and columns past the matrix read as 0, which is the padding.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_swizzle(const SwizzleArgs a) {
    // the unit's 128 rows x (4 * nt) codes, one word (4 codes of a tile) per
    // entry; the odd row pitch nt + 1 keeps the column reads on distinct banks
    extern __shared__ uint32_t codes[];
    const int nt = a.unit_tiles, pitch = nt + 1;
    // rows of a multiple of 4 codes from a 4-byte aligned base: each row's 4
    // codes of a tile are one aligned word (the usual case; uniform)
    const bool words = (a.cols & 3) == 0 && (reinterpret_cast<uintptr_t>(a.lin) & 3) == 0;
    const int64_t groups = (a.tiles_per_band + nt - 1) / nt;
    const int64_t n_units = (a.rows + 127) / 128 * groups;
    // the units of one band (up to 16) run on one XCD: each 128-byte line of
    // the band's rows is read by several of them, and one L2 then fetches it
    // once (measured 2.0x -> 1.02x the input on 128-column rows)
    const int g = groups < 16 ? (int)groups : 16;
    for (int64_t u0 = blockIdx.x; u0 < n_units; u0 += gridDim.x) {
        const int64_t u = xcd_grouping_holds(gridDim.x, n_units) ? xcd_grouped_unit(u0, n_units, g) : u0;
        const int64_t band = u / groups, t0 = (u - band * groups) * nt;
        // kBatch loads in flight per thread before any LDS write
        constexpr int kBatch = 8;
        for (int k0 = 0; k0 < 128 * nt; k0 += kBatch * kThreads) {
            uint32_t w[kBatch];
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int k = k0 + b * kThreads + (int)threadIdx.x;
                const int row = k / nt, wc = k - row * nt;
                const int64_t r = band * 128 + row, c0 = (t0 + wc) * 4;
                w[b] = 0;
                if (k < 128 * nt && r < a.rows && c0 < a.cols) {
                    if (words) {
                        w[b] = *reinterpret_cast<const uint32_t *>(a.lin + r * a.cols + c0);
                    } else {
                        for (int j = 0; j < 4 && c0 + j < a.cols; ++j)
                            w[b] |= (uint32_t)a.lin[r * a.cols + c0 + j] << (8 * j);
                    }
                }
            }
#pragma unroll
            for (int b = 0; b < kBatch; ++b) {
                const int k = k0 + b * kThreads + (int)threadIdx.x;
                const int row = k / nt;
                if (k < 128 * nt) codes[row * pitch + (k - row * nt)] = w[b];
            }
        }
        __syncthreads();
        // the unit's tiles are contiguous in the output: 512 bytes each, 16
        // bytes per line p holding rows p, p+32, p+64, p+96
        const int n_t = (int)min((int64_t)nt, a.tiles_per_band - t0);
        uint8_t *dst = a.swz + (band * a.tiles_per_band + t0) * 512;
        for (int k = threadIdx.x; k < n_t * 32; k += kThreads) {
            const int t = k >> 5, p = k & 31;
            *reinterpret_cast<u32x4 *>(dst + k * 16) =
                u32x4{codes[p * pitch + t], codes[(p + 32) * pitch + t],
                      codes[(p + 64) * pitch + t], codes[(p + 96) * pitch + t]};
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static inline unsigned grid_of(int64_t g) { return (unsigned)(g < 1 ? 1 : g); }

// 512-column steps per wave for a row of H columns shared by wpr waves,
// rounded up to an instantiated count.
static int fused_steps(int64_t H, int wpr) {
    const int64_t n = ((H + kChunk - 1) / kChunk + wpr - 1) / wpr;
    return n <= 1 ? 1 : n <= 2 ? 2 : n <= 4 ? 4 : n <= 7 ? 7 : n <= 8 ? 8 : 16;
}

template <int FMT, int LAYOUT, int WPR, int RPU>
static void fused_nch(const FusedArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(RPU * WPR * kWave);
    switch (fused_steps(a.H, WPR)) {
    case 1: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 1, WPR, RPU>), gd, bd, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 2, WPR, RPU>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 4, WPR, RPU>), gd, bd, lds, s, a); break;
    case 7: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 7, WPR, RPU>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 8, WPR, RPU>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 16, WPR, RPU>), gd, bd, lds, s, a); break;
    }
}

// The shape is the host's choice (a.wpr, a.rpu): sixteen or four waves per
// row and one-row units for latency-bound calls (the more waves, the shorter
// each row's chain of dependent loads), two waves per row and four-row units
// for large ones.  Units of rows 32 apart (whole 16-byte swizzled pieces per
// unit) measured 3-6 % slower at T = 4096 than these consecutive rows.
template <int FMT, int LAYOUT>
static void fused_wpr(const FusedArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    if (a.wpr == 2)
        fused_nch<FMT, LAYOUT, 2, 4>(a, gd, lds, s);
    else if (a.wpr == 16)
        fused_nch<FMT, LAYOUT, 16, 1>(a, gd, lds, s);
    else
        fused_nch<FMT, LAYOUT, 4, 1>(a, gd, lds, s);
}

hipError_t launch_fused(int fmt, int layout, const FusedArgs &a, int64_t grid, hipStream_t s) {
    // gamma (bf16 [H], 16-byte rounded) then the staged scales of a unit
    const size_t lds = (size_t)((2 * a.H + 15) & ~15) + (size_t)a.rpu * a.sf_stride;
    const dim3 gd(grid_of(grid));
    if (fmt == MXQ_MXFP8 && layout == MXQ_SF_LINEAR)
        fused_wpr<MXQ_MXFP8, MXQ_SF_LINEAR>(a, gd, lds, s);
    else if (fmt == MXQ_MXFP8)
        fused_wpr<MXQ_MXFP8, MXQ_SF_SWIZZLED>(a, gd, lds, s);
    else if (layout == MXQ_SF_LINEAR)
        fused_wpr<MXQ_NVFP4, MXQ_SF_LINEAR>(a, gd, lds, s);
    else
        fused_wpr<MXQ_NVFP4, MXQ_SF_SWIZZLED>(a, gd, lds, s);
    return hipGetLastError();
}

hipError_t launch_fused_tiny(int fmt, const FusedArgs &a, hipStream_t s) {
    const dim3 gd(grid_of(a.T)), bd(kFusedTinyThreads);
    if (fmt == MXQ_MXFP8)
        hipLaunchKernelGGL(k_fused_tiny<MXQ_MXFP8>, gd, bd, 0, s, a);
    else
        hipLaunchKernelGGL(k_fused_tiny<MXQ_NVFP4>, gd, bd, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_swizzle(const SwizzleArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)128 * (a.unit_tiles + 1) * 4;  // 8.5 KiB at 16 tiles
    hipLaunchKernelGGL(k_swizzle, dim3(grid_of(grid)), dim3(kThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace mxq
