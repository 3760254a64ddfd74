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
// scales leave in whole segments, padding included.  Measured alternatives
// that lost: 2 rows per wave (4 or 8 waves), scale codes stored from
// registers as 4-byte pieces instead of LDS-staged 16-byte segments, a
// persistent grid with software-pipelined loads.
//
// Unit u runs on workgroup u, in plain dispatch order, except that with
// linear scales every 8 consecutive units run on one XCD (1-3 % faster).
// Swizzled, the same grouping made the Qwen3-235B gate_up launches 2 % slower,
// and on rows of 1.5 chunks (768 columns), where the plain order puts every
// full chunk on an even XCD and every half chunk on an odd one, evening out
// the XCDs left the launch time unchanged: the launch is bound by HBM, not by
// the busiest XCD.  The units in flight
// cover one contiguous stretch of every tensor (measured faster than giving
// each XCD a contiguous range).  The quantize kernel uses no global atomics, no scratch
// and no inter-workgroup ordering: every byte has one writer, and the bytes
// do not depend on the grid size.  (k_amax, for encode scales from the data,
// folds each workgroup's maximum into its slot with one atomic max.)
#include <hip/hip_ext.h>

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

// AUTO (NVFP4 only): the encode scale of entry e is nv_encode_scale of its
// slot's amax, reduced beforehand by k_amax; workgroup 0 publishes every
// slot's encode scale.
template <int FMT, int LAYOUT, bool AUTO>
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
    if (AUTO && blockIdx.x == 0 && (int)threadIdx.x < a.n_slots)
        a.g_out[threadIdx.x] = nv_encode_scale(__uint_as_float(a.amax_bits[threadIdx.x]));
    for (int u0 = blockIdx.x; u0 < a.total_units; u0 += gridDim.x) {
        // linear: 8 consecutive units (the column chunks of a row group) share
        // 128-byte scale lines; meeting in one L2 merges their partial lines
        const int u = LAYOUT == MXQ_SF_LINEAR && xcd_grouping_holds(gridDim.x, a.total_units)
                          ? xcd_grouped_unit<8>(u0, a.total_units)
                          : u0;
        // the unit's entry: one scalar division when every entry has the same
        // number of units (every launch of a model layer; 0.5-1.2 us per
        // launch faster than the walk), else a walk of the table
        int ei = 0;
        if (a.uniform_units > 0)
            ei = u / a.uniform_units;
        else
            while (ei + 1 < a.n && u >= a.e[ei + 1].unit_begin) ++ei;
        const GEntry &E = a.e[ei];
        // the entry's fields, read once per unit into scalar registers (reading
        // them through E in the row loops reloaded them from the kernel
        // arguments each row: 21 scalar loads instead of 8; 0.5-1 % slower)
        const uint16_t *const e_src = E.src;
        uint8_t *const e_payload = E.payload;
        uint8_t *const e_scales = E.scales;
        const int64_t e_ld = E.ld;
        const int e_rows = E.rows;
        const int lu = u - E.unit_begin;
        const int rg = lu / a.n_cc;
        const int cc = lu - rg * a.n_cc;
        const int col = cc * kChunk + lane * 8;
        const bool live_col = col < a.cols;
        const float g = FMT != MXQ_NVFP4 ? 0.0f
                        : AUTO ? nv_encode_scale(__uint_as_float(a.amax_bits[E.slot]))
                               : *E.g;
        const NvG G = nv_prepare(g);

        u32x4 v[kRowsPerWave];
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            v[i] = u32x4{0, 0, 0, 0};
            if (r < e_rows && live_col)
                v[i] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4 *>(e_src + (int64_t)r * e_ld + col));
        }
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) {
            const int r = group_row<LAYOUT>(rg, q, i);
            uint32_t code = 0;  // rows and columns past the tensor stage zeros
            if (r < e_rows) {  // uniform: the whole wave quantizes
                u32x2 pay;
                const uint32_t c = quant8<FMT>(v[i], G, pay);
                if (live_col) {
                    code = c;
                    store_payload<FMT>(e_payload + (int64_t)r * payload_ld, col, pay);
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
                    uint8_t *dst = e_scales +
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
                if (r >= e_rows) continue;
                uint8_t *dst = e_scales + (int64_t)r * a.sf_cols + c0 + part * 16;
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
// Per-slot amax for encode scales from the data.  A workgroup folds a run of
// kAmaxUnits k_grouped units of one entry into one value and makes one atomic
// max on its slot: atomics on one address from every workgroup serialize (one
// per unit measured 4x slower than the whole read), so the run length sets
// their number.  A run takes every W-th unit of its entry (W = the entry's
// run count), so the runs in flight read a compact window of each entry:
// runs of consecutive units, which spread the workgroups in flight over the
// whole tensor, read 7% slower.  The amax is kept as fp32 bits (a bf16
// magnitude shifted up), whose unsigned order is the value order.  The
// quantize pass reads the input again from HBM: no unit order, call size (1
// to 16 experts) or load kind showed reuse from the last-level cache.
// ---------------------------------------------------------------------------
constexpr int kAmaxUnits = 32;

// Runs of an amax launch: ceil(units / kAmaxUnits) per entry.
__host__ __device__ inline int amax_runs(const GroupArgs &a) {
    int n_runs = 0;
    for (int e = 0; e < a.n; ++e) {
        const int nu = (e + 1 < a.n ? a.e[e + 1].unit_begin : a.total_units) - a.e[e].unit_begin;
        n_runs += (nu + kAmaxUnits - 1) / kAmaxUnits;
    }
    return n_runs;
}

__global__ __launch_bounds__(64) void k_zero_slots(uint32_t *amax_bits, int n) {
    if ((int)threadIdx.x < n) amax_bits[threadIdx.x] = 0;
}

__global__ __launch_bounds__(kThreads) void k_amax(const GroupArgs a) {
    __shared__ uint32_t red[kThreads / kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x >> 6;
    // fold the workgroup's running max m into slot `slot` (uniform call)
    auto flush = [&](uint32_t m, int slot) {
        m = wave_max(m);
        if (lane == 0) red[q] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            m = max(max(red[0], red[1]), max(red[2], red[3]));
            if (m != 0) atomicMax(a.amax_bits + slot, m << 16);
        }
        __syncthreads();
    };
    // runs: each entry's units are split into ceil(n / kAmaxUnits) runs; run lr
    // of an entry with W runs takes its units lr, lr + W, lr + 2W, ... so that
    // the runs in flight cover a compact window of every entry
    const int n_runs = amax_runs(a);
    for (int run = blockIdx.x; run < n_runs; run += gridDim.x) {
        int ei = 0, rb = 0, W = 0, nu = 0;
        for (;; ++ei) {
            nu = (ei + 1 < a.n ? a.e[ei + 1].unit_begin : a.total_units) - a.e[ei].unit_begin;
            W = (nu + kAmaxUnits - 1) / kAmaxUnits;
            if (run < rb + W) break;
            rb += W;
        }
        const GEntry &E = a.e[ei];
        const int lr = run - rb;
        uint32_t m = 0;
        for (int lu = lr; lu < nu; lu += W) {
            const int rg = lu / a.n_cc;
            const int col = (lu - rg * a.n_cc) * kChunk + lane * 8;
            u32x4 v[kRowsPerWave];
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) {
                const int r = rg * kUnitRows + kRowsPerWave * q + i;
                v[i] = u32x4{0, 0, 0, 0};
                if (r < E.rows && col < a.cols)
                    v[i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(E.src + (int64_t)r * E.ld + col));
            }
#pragma unroll
            for (int i = 0; i < kRowsPerWave; ++i) m = max(m, amax_bits8(v[i]));
        }
        const int slot = E.slot;
        flush(m, slot);
    }
}

// ---------------------------------------------------------------------------
// Launcher.
// ---------------------------------------------------------------------------
static inline unsigned grid_of(int64_t g) { return (unsigned)(g < 1 ? 1 : g); }

// chain: the dispatch packet's barrier bit is cleared (HIP's any-order
// launch), so the launch may start while the stream's previous launch drains.
hipError_t launch_grouped(int fmt, int layout, bool auto_scale, const GroupArgs &a, int64_t grid,
                          hipStream_t s, bool chain) {
    const dim3 gd(grid_of(grid)), bd(kThreads);
    const uint32_t fl = chain ? hipExtAnyOrderLaunch : 0;
    if (fmt == MXQ_MXFP8 && layout == MXQ_SF_LINEAR)
        hipExtLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_LINEAR, false>), gd, bd, 0, s, nullptr,
                              nullptr, fl, a);
    else if (fmt == MXQ_MXFP8)
        hipExtLaunchKernelGGL((k_grouped<MXQ_MXFP8, MXQ_SF_SWIZZLED, false>), gd, bd, 0, s, nullptr,
                              nullptr, fl, a);
    else if (layout == MXQ_SF_LINEAR && !auto_scale)
        hipExtLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_LINEAR, false>), gd, bd, 0, s, nullptr,
                              nullptr, fl, a);
    else if (!auto_scale)
        hipExtLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_SWIZZLED, false>), gd, bd, 0, s, nullptr,
                              nullptr, fl, a);
    else if (layout == MXQ_SF_LINEAR)
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_LINEAR, true>), gd, bd, 0, s, a);
    else
        hipLaunchKernelGGL((k_grouped<MXQ_NVFP4, MXQ_SF_SWIZZLED, true>), gd, bd, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_amax(const GroupArgs &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL(k_zero_slots, dim3(1), dim3(64), 0, s, a.amax_bits, a.n_slots);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || a.total_units == 0) return err;
    const int64_t runs = amax_runs(a);
    hipLaunchKernelGGL(k_amax, dim3(grid_of(grid < runs ? grid : runs)), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace mxq
