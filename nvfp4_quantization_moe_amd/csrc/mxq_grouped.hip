// mxq_grouped.hip -- grouped block quantization: 1..16 expert tensors that
// share a row length, one launch, the descriptor table in the kernel
// arguments.
//
// Streaming work bounded by HBM bandwidth, so the kernel is shaped like a
// well-behaved copy: many small workgroups, every load of a workgroup issued
// before any of its stores, 16 contiguous bytes per lane (a wave load is
// 1 KiB of one row), each lane's output bytes contiguous.
//
// A work unit is 4*kRowsPerWave rows x 512 columns of one expert,
// kRowsPerWave rows per wave.  A block of 32 (MXFP8) or 16 (NVFP4) elements
// spans 4 or 2 adjacent lanes; its amax is reduced with DPP quad permutes,
// never through LDS.  Payload bytes go straight to HBM; scale bytes are staged
// in LDS.  With the swizzled layout the unit's rows are band*128 + 32*wave +
// R*h + i (R = kRowsPerWave, i < R) of one 128-row band, which fill one
// contiguous R*16-byte segment of each 512-byte tile the chunk touches, so
// scales leave in whole segments, padding included.
//
// Unit u runs on workgroup u, in plain dispatch order; the hardware spreads
// consecutive workgroups over the 8 XCDs, so the units in flight cover one
// contiguous stretch of every tensor (measured faster than giving each XCD a
// contiguous range).  No global atomics, no scratch, no inter-workgroup
// ordering: every byte has one writer, and the bytes do not depend on the
// grid size.
#include "mxq_device.h"
#include "mxq_internal.h"

namespace mxq {

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
// Launcher.
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

}  // namespace mxq
