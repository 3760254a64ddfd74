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
// Fused (k_fused) needs whole rows (the RMSNorm sum of squares): two waves
// own one row and hold it in registers; a unit is 4 rows.  Swizzled units take
// rows band*128 + 32*q + gi (gi = 0..31), so a unit writes one 16-byte piece
// of each tile line (8 consecutive units complete it).
// Split (k_split): a unit owns one line of every scale tile of a 128-row band
// of one expert and loads only that line-set's live rows, whole rows, two
// waves per row.
//
// Grouped and fused: unit u runs on workgroup u, in plain dispatch order; the
// hardware spreads consecutive workgroups over the 8 XCDs, so the units in
// flight cover one contiguous stretch of every tensor (measured faster than
// giving each XCD a contiguous range).  No global atomics, no scratch, no inter-workgroup
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

// Quantize one lane's 8 elements; the lanes of a block cooperate through DPP,
// and NVFP4 fetches its multiplier quotient across the wave (nv_wave_quot),
// so every lane of the wave must call it (lanes past the tensor pass zeros
// and discard the result).  Returns the block's scale byte (every lane of the
// block holds it) and the lane's payload: 8 bytes (MXFP8) or 4 bytes in pay.x
// (NVFP4).
template <int FMT>
__device__ __forceinline__ uint32_t quant8(u32x4 v, float g, float quot, u32x2 &pay) {
    uint32_t a = amax_bits8(v);
    if constexpr (FMT == MXQ_MXFP8) {
        a = block_max4(a);
        const uint32_t c = mx_scale_code(a);
        pay = mx_encode8(v, c);
        return c;
    } else {
        a = block_max2(a);
        const Nv4Scale s = nv_scale(a, g, quot);
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
        const float quot = FMT == MXQ_NVFP4 ? nv_wave_quot(g) : 0.0f;

        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            v[i] = u32x4{0, 0, 0, 0};
            if (r < E.rows && live_col)
                v[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(E.src + (int64_t)r * E.ld + col));
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            uint32_t code = 0;  // rows and columns past the tensor stage zeros
            if (r < E.rows) {  // uniform: the whole wave quantizes
                u32x2 pay;
                const uint32_t c = quant8<FMT>(v[i], g, quot, pay);
                if (live_col) {
                    code = c;
                    store_payload<FMT>(E.payload + (int64_t)r * payload_ld, col, pay);
                }
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
// Whole-row units (split, fused): 4 rows per workgroup of 8 waves, two waves
// per row; each wave holds half of its row in registers (512-column steps
// 2k + half).  Row-wide reductions combine the two halves through LDS in a
// fixed order.  Staged scales: swizzled [tile][row][4] (16 bytes per tile),
// linear [row][C].
// ---------------------------------------------------------------------------
template <int LAYOUT>
__device__ __forceinline__ void stage_code(uint8_t *stage, int q, int c, int sf_cols,
                                           uint32_t code) {
    if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
        stage[(c >> 2) * 16 + q * 4 + (c & 3)] = (uint8_t)code;
    else
        stage[q * sf_cols + c] = (uint8_t)code;
}

// Zero the staged codes of a row with no data (swizzled padding rows).
template <int LAYOUT>
__device__ __forceinline__ void stage_zero_row(uint8_t *stage, int q, int lane, int sf_cols,
                                               int sf_stride) {
    for (int c = lane; c < sf_stride; c += kWave) stage_code<LAYOUT>(stage, q, c, sf_cols, 0);
}

// Copy n staged bytes to global memory with kRowThreads threads.
__device__ __forceinline__ void copy_out_rows(uint8_t *dst, const uint8_t *src, int n) {
    if ((reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
        const int nv = n >> 4;
        for (int k = threadIdx.x; k < nv; k += kRowThreads)
            *reinterpret_cast<u32x4 *>(dst + k * 16) = *reinterpret_cast<const u32x4 *>(src + k * 16);
        for (int k = (nv << 4) + threadIdx.x; k < n; k += kRowThreads) dst[k] = src[k];
    } else {
        for (int k = threadIdx.x; k < n; k += kRowThreads) dst[k] = src[k];
    }
}

// Fused swizzled units take rows band*128 + 32*q + gi (gi = lu mod 32): one
// 16-byte piece per tile line.
__device__ __forceinline__ void flush_interleaved_swz(const uint8_t *stage, uint8_t *region,
                                                      int lu, int sf_stride) {
    const int tiles = sf_stride >> 2;
    uint8_t *base = region + (int64_t)(lu >> 5) * tiles * 512 + (lu & 31) * 16;
    for (int t = threadIdx.x; t < tiles; t += kRowThreads)
        *reinterpret_cast<u32x4 *>(base + (int64_t)t * 512) =
            *reinterpret_cast<const u32x4 *>(stage + t * 16);
}

// Split.  Swizzled: a unit owns line h (0..3) of every scale tile of one
// 128-row band of one expert, i.e. the rows band*128 + 32*q + 8*h + i
// (q < 4, i < 8), so its staged scales leave as whole 128-byte lines, padding
// rows and columns zero.  Linear: a unit is 32 consecutive rows.  Only the
// unit's live rows are loaded: pairs of waves take them in turn, each wave
// holding half of a row (512-column steps 2k + half) in registers, so short
// experts keep every wave busy.  The row amax is the max over the two halves,
// folded in LDS; no global atomics.
// At most 128 VGPRs, so two workgroups share a CU (short experts give each
// workgroup little work).
template <int LAYOUT, int NCH2>
__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(4)))
void k_split(const SplitArgs a) {
    extern __shared__ __align__(16) uint8_t stage[];
    __shared__ uint32_t row_max[32];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int pair = w >> 1, half = w & 1;
    const int64_t payload_ld = a.cols / 2;
    const float g = *a.g;
    const float quot = nv_wave_quot(g);
    const int stage_bytes = 32 * a.sf_stride;
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
        // live rows of the unit, in order; nq[q] of them in line-set row q
        int nq[4] = {0, 0, 0, 0};
        int n_live;
        int band = 0, h = 0;
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            band = lu >> 2;
            h = lu & 3;
            const int rb = min(128, m - band * 128);
            n_live = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                nq[q] = min(8, max(0, rb - 32 * q - 8 * h));
                n_live += nq[q];
            }
        } else {
            n_live = min(32, m - lu * 32);
        }
        // j-th live row of the unit -> (line-set row q, slot i, row in expert)
        auto locate = [&](int j, int &q, int &i) {
            q = 0;
            i = j;
            if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
                while (i >= nq[q]) { i -= nq[q]; ++q; }
                return band * 128 + 32 * q + 8 * h + i;
            } else {
                return lu * 32 + j;
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
        u32x4 cur[NCH2], nxt[NCH2];
        if (pair < n_live) load_row(pair, cur);
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            for (int k = threadIdx.x * 16; k < stage_bytes; k += kSplitThreads * 16)
                *reinterpret_cast<u32x4 *>(stage + k) = u32x4{0, 0, 0, 0};
        }
        if (threadIdx.x < 32) row_max[threadIdx.x] = 0;
        __syncthreads();
        for (int j = pair; j < n_live; j += 4) {
            if (j + 4 < n_live) load_row(j + 4, nxt);  // next row's loads in flight
            int q, i;
            const int r = locate(j, q, i);
            uint8_t *pay_row = a.payload + (e0 + r) * payload_ld;
            uint32_t amax = 0;
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                u32x2 pay;
                const uint32_t code = quant8<MXQ_NVFP4>(cur[k], g, quot, pay);  // whole wave
                if (col < a.cols) {
                    store_payload<MXQ_NVFP4>(pay_row, col, pay);
                    amax = max(amax, amax_bits8(cur[k]));
                    if ((lane & 1) == 0) {
                        const int c = col / 16;
                        if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
                            stage[(c >> 2) * 128 + i * 16 + q * 4 + (c & 3)] = (uint8_t)code;
                        else
                            stage[j * a.sf_cols + c] = (uint8_t)code;
                    }
                }
            }
            amax = wave_max(amax);
            if (lane == 0) atomicMax(&row_max[j], amax);
#pragma unroll
            for (int k = 0; k < NCH2; ++k) cur[k] = nxt[k];
        }
        __syncthreads();
        if (a.row_amax && (int)threadIdx.x < n_live) {
            int q, i;
            const int r = locate(threadIdx.x, q, i);
            a.row_amax[e0 + r] = __uint_as_float(row_max[threadIdx.x] << 16);
        }
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED) {
            const int tiles = a.sf_stride >> 2;
            uint8_t *base = a.scales + (int64_t)(a.unit_off[s] >> 2) * tiles * 512 +
                            (int64_t)band * tiles * 512 + h * 128;
            for (int k = threadIdx.x; k < tiles * 8; k += kSplitThreads) {
                const int t = k >> 3, part = k & 7;
                *reinterpret_cast<u32x4 *>(base + (int64_t)t * 512 + part * 16) =
                    *reinterpret_cast<const u32x4 *>(stage + t * 128 + part * 16);
            }
        } else {
            uint8_t *dst = a.scales + (e0 + lu * 32) * a.sf_cols;
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

// Fused residual add + RMSNorm + quantize.  The row's bf16 residual sum stays
// in registers; the sum of squares is each wave's fixed-order partial,
// combined lower half + upper half; norm_out and the quantized form come
// from the same bf16 values.
template <int FMT, int LAYOUT, int NCH2>
__global__ __launch_bounds__(kRowThreads) void k_fused(const FusedArgs a) {
    using Tr = FmtTraits<FMT>;
    extern __shared__ __align__(16) uint8_t stage[];
    __shared__ float red[8];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x >> 6;
    const int q = w >> 1, half = w & 1;
    const int H = a.H;
    const int64_t payload_ld = FMT == MXQ_MXFP8 ? H : H / 2;
    const float g = FMT == MXQ_NVFP4 ? *a.g : 0.0f;
    const float quot = FMT == MXQ_NVFP4 ? nv_wave_quot(g) : 0.0f;
    const bool leader = (lane & (Tr::kLanesPerBlock - 1)) == 0;
    for (int lu = blockIdx.x; lu < a.total_units; lu += gridDim.x) {
        const int r = LAYOUT == MXQ_SF_SWIZZLED ? (lu >> 5) * 128 + 32 * q + (lu & 31)
                                                : lu * 4 + q;
        const bool live = r < a.T;
        const int64_t rb = (int64_t)r * H;
        u32x4 xv[NCH2];
        float acc = 0.0f;
        if (live) {
            u32x4 rv[NCH2];
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                if (col < H) {
                    xv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.x + rb + col));
                    rv[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.res + rb + col));
                }
            }
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
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
        }
        if (lane == 0) red[w] = acc;
        __syncthreads();
        if (live) {
            const float inv = 1.0f / __builtin_sqrtf((red[2 * q] + red[2 * q + 1]) / (float)H + a.eps);
            u32x4 gm[NCH2];
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                if (col < H) gm[k] = *reinterpret_cast<const u32x4 *>(a.gamma + col);
            }
#pragma unroll
            for (int k = 0; k < NCH2; ++k) {
                const int col = (2 * k + half) * kChunk + lane * 8;
                u32x4 nv = u32x4{0, 0, 0, 0};
                if (col < H) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float nlo = (bf16_lo(xv[k][j]) * bf16_lo(gm[k][j])) * inv;
                        const float nhi = (bf16_hi(xv[k][j]) * bf16_hi(gm[k][j])) * inv;
                        nv[j] = pack_bf16(nlo, nhi);
                    }
                    __builtin_nontemporal_store(nv, reinterpret_cast<u32x4 *>(a.norm_out + rb + col));
                }
                u32x2 pay;
                const uint32_t code = quant8<FMT>(nv, g, quot, pay);  // whole wave
                if (col < H) {
                    store_payload<FMT>(a.payload + (int64_t)r * payload_ld, col, pay);
                    if (leader) stage_code<LAYOUT>(stage, q, col / Tr::kBlock, a.sf_cols, code);
                }
            }
        } else if (LAYOUT == MXQ_SF_SWIZZLED && half == 0) {
            stage_zero_row<LAYOUT>(stage, q, lane, a.sf_cols, a.sf_stride);
        }
        __syncthreads();
        if constexpr (LAYOUT == MXQ_SF_SWIZZLED)
            flush_interleaved_swz(stage, a.scales, lu, a.sf_stride);
        else
            copy_out_rows(a.scales + (int64_t)lu * 4 * a.sf_cols, stage,
                          min(4, a.T - lu * 4) * a.sf_cols);
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

// Whole-row kernels keep half a row per wave in registers: NCH2 512-column
// steps per wave.
int half_row_steps(int64_t cols) {
    const int64_t n = ((cols + kChunk - 1) / kChunk + 1) / 2;
    if (n <= 1) return 1;
    if (n <= 2) return 2;
    if (n <= 4) return 4;
    if (n <= 7) return 7;
    if (n <= 8) return 8;
    return 16;
}

template <int LAYOUT>
static void split_nch(const SplitArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kSplitThreads);
    switch (half_row_steps(a.cols)) {
    case 1: hipLaunchKernelGGL((k_split<LAYOUT, 1>), gd, bd, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_split<LAYOUT, 2>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_split<LAYOUT, 4>), gd, bd, lds, s, a); break;
    case 7: hipLaunchKernelGGL((k_split<LAYOUT, 7>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_split<LAYOUT, 8>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_split<LAYOUT, 16>), gd, bd, lds, s, a); break;
    }
}

hipError_t launch_split(int layout, const SplitArgs &a, int64_t grid, hipStream_t s) {
    const size_t lds = (size_t)32 * a.sf_stride;
    const dim3 gd(grid_of(grid));
    if (layout == MXQ_SF_LINEAR)
        split_nch<MXQ_SF_LINEAR>(a, gd, lds, s);
    else
        split_nch<MXQ_SF_SWIZZLED>(a, gd, lds, s);
    return hipGetLastError();
}

template <int FMT, int LAYOUT>
static void fused_nch(const FusedArgs &a, dim3 gd, size_t lds, hipStream_t s) {
    const dim3 bd(kRowThreads);
    switch (half_row_steps(a.H)) {
    case 1: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 1>), gd, bd, lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 2>), gd, bd, lds, s, a); break;
    case 4: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 4>), gd, bd, lds, s, a); break;
    case 7: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 7>), gd, bd, lds, s, a); break;
    case 8: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 8>), gd, bd, lds, s, a); break;
    default: hipLaunchKernelGGL((k_fused<FMT, LAYOUT, 16>), gd, bd, lds, s, a); break;
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
