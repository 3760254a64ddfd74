// mxq_api.hip -- the C ABI declared in include/mxq.h: argument validation,
// descriptor-table packing and kernel launches.  Every check runs on the host
// before any launch; a call that fails a check enqueues nothing.
#include <stdint.h>
#include <string.h>

#include "mxq_internal.h"

using namespace mxq;

namespace {

int64_t g_max_workgroups = 0;  // debug grid cap; 0 = one workgroup per unit

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline bool valid_fmt(int f) { return f == MXQ_MXFP8 || f == MXQ_NVFP4; }
inline bool valid_layout(int l) { return l == MXQ_SF_LINEAR || l == MXQ_SF_SWIZZLED; }
inline int64_t block_of(int fmt) { return fmt == MXQ_MXFP8 ? 32 : 16; }
inline int64_t max_cols(int fmt) { return fmt == MXQ_MXFP8 ? kMaxColsMx : kMaxColsNv; }

// Row groups of `per` rows for a tensor of `rows` rows.  Swizzled groups
// cover the padded rows too, so the padding is written by the kernel.
inline int64_t row_groups(int64_t rows, int layout, int per) {
    if (rows <= 0) return 0;
    return layout == MXQ_SF_SWIZZLED ? round_up(rows, 128) / per : (rows + per - 1) / per;
}

inline int64_t grid_for(int64_t units) {
    if (g_max_workgroups > 0 && g_max_workgroups < units) return g_max_workgroups;
    return units;
}

inline int64_t sf_bytes(int64_t rows, int64_t C, int layout) {
    if (layout == MXQ_SF_LINEAR) return rows * C;
    return round_up(rows, 128) * round_up(C, 4);
}

}  // namespace

extern "C" {

const char *mxq_status_str(int status) {
    switch (status) {
    case MXQ_OK: return "ok";
    case MXQ_EINVAL: return "invalid argument (null pointer, enum, count, split or eps)";
    case MXQ_ESHAPE: return "unsupported shape or alignment";
    case MXQ_EUNSUPPORTED: return "combination not implemented";
    case MXQ_ELAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

void mxq_set_max_workgroups(int64_t n) { g_max_workgroups = n > 0 ? n : 0; }

int64_t mxq_scale_bytes(int64_t rows, int64_t cols, int fmt, int layout) {
    if (!valid_fmt(fmt) || !valid_layout(layout) || rows < 0 || cols <= 0 ||
        cols % block_of(fmt) != 0)
        return -1;
    return sf_bytes(rows, cols / block_of(fmt), layout);
}

int64_t mxq_split_scale_offset(const int64_t *split_rows, int n_splits, int i, int64_t cols,
                               int fmt, int layout) {
    if ((!split_rows && n_splits > 0) || n_splits < 0 || i < 0 || i > n_splits) return -1;
    if (!valid_fmt(fmt) || !valid_layout(layout) || cols <= 0 || cols % block_of(fmt) != 0)
        return -1;
    int64_t off = 0;
    for (int j = 0; j < n_splits; ++j)
        if (split_rows[j] < 0) return -1;
    for (int j = 0; j < i; ++j) off += sf_bytes(split_rows[j], cols / block_of(fmt), layout);
    return off;
}

}  // extern "C"

namespace {

// Validate and pack a grouped call.  Returns MXQ_OK and fills `a`, or the
// status of the first failed check.
int pack_grouped(int fmt, int layout, int64_t cols, const mxq_entry *entries, int n_entries,
                 bool need_g, GroupArgs &a) {
    if (!valid_fmt(fmt) || !valid_layout(layout) || !entries || n_entries < 1 ||
        n_entries > MXQ_MAX_GROUP)
        return MXQ_EINVAL;
    if (cols <= 0 || cols % block_of(fmt) != 0 || cols > max_cols(fmt)) return MXQ_ESHAPE;
    memset(&a, 0, sizeof(a));
    a.n = n_entries;
    a.cols = (int32_t)cols;
    a.sf_cols = (int32_t)(cols / block_of(fmt));
    a.sf_stride = layout == MXQ_SF_SWIZZLED ? (int32_t)round_up(a.sf_cols, 4) : a.sf_cols;
    a.n_cc = (int32_t)((cols + kChunk - 1) / kChunk);
    int64_t units = 0;
    for (int i = 0; i < n_entries; ++i) {
        const mxq_entry &e = entries[i];
        // rows padded to 128 must still index as int32
        if (e.rows < 0 || e.rows > ((int64_t)1 << 31) - 128) return MXQ_EINVAL;
        if (e.rows > 0) {
            if (!e.src || !e.payload || !e.scales) return MXQ_EINVAL;
            if (need_g && !e.global_scale) return MXQ_EINVAL;
            if (e.src_ld < cols || e.src_ld % 8 != 0 || e.src_ld >= (int64_t)1 << 31)
                return MXQ_ESHAPE;
            if (!aligned16(e.src) || !aligned16(e.payload)) return MXQ_ESHAPE;
            if (layout == MXQ_SF_SWIZZLED && !aligned16(e.scales)) return MXQ_ESHAPE;
        }
        a.e[i].src = static_cast<const uint16_t *>(e.src);
        a.e[i].payload = static_cast<uint8_t *>(e.payload);
        a.e[i].scales = static_cast<uint8_t *>(e.scales);
        a.e[i].g = e.global_scale;
        a.e[i].ld = e.src_ld;
        a.e[i].rows = (int32_t)e.rows;
        a.e[i].unit_begin = (int32_t)units;
        a.e[i].slot = i;
        units += row_groups(e.rows, layout, kUnitRows) * a.n_cc;
        if (units >= (int64_t)1 << 31) return MXQ_ESHAPE;
    }
    a.total_units = (int32_t)units;
    // every entry the same number of units: the kernel finds a unit's entry
    // by one division
    a.uniform_units = units > 0 && units % n_entries == 0 ? (int32_t)(units / n_entries) : 0;
    for (int i = 0; i < n_entries && a.uniform_units; ++i)
        if (a.e[i].unit_begin != i * a.uniform_units) a.uniform_units = 0;
    return MXQ_OK;
}

}  // namespace

extern "C" {

int mx_quant_grouped(int fmt, int layout, int64_t cols, const mxq_entry *entries, int n_entries,
                     void *stream) {
    GroupArgs a;
    const int st = pack_grouped(fmt, layout, cols, entries, n_entries, fmt == MXQ_NVFP4, a);
    if (st != MXQ_OK) return st;
    if (a.total_units == 0) return MXQ_OK;
    hipError_t err =
        launch_grouped(fmt, layout, false, a, grid_for(a.total_units), (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_ELAUNCH;
}

int mx_quant_grouped_batch(int fmt, int layout, int64_t cols, const mxq_entry *entries,
                           int n_entries, int per_launch, unsigned flags, void *stream) {
    if (n_entries < 1 || per_launch < 1 || per_launch > MXQ_MAX_GROUP || !entries ||
        (flags & ~(unsigned)MXQ_CHAIN) != 0)
        return MXQ_EINVAL;
    // every launch's entries are checked before the first launch
    GroupArgs a;
    for (int b = 0; b < n_entries; b += per_launch) {
        const int n = n_entries - b < per_launch ? n_entries - b : per_launch;
        const int st = pack_grouped(fmt, layout, cols, entries + b, n, fmt == MXQ_NVFP4, a);
        if (st != MXQ_OK) return st;
    }
    hipStream_t s = (hipStream_t)stream;
    // a stream being captured into a graph gets ordinary launches
    bool chain = (flags & MXQ_CHAIN) != 0;
    if (chain) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
            chain = false;
    }
    bool first = true;  // the first launch keeps the stream's order
    for (int b = 0; b < n_entries; b += per_launch) {
        const int n = n_entries - b < per_launch ? n_entries - b : per_launch;
        pack_grouped(fmt, layout, cols, entries + b, n, fmt == MXQ_NVFP4, a);
        if (a.total_units == 0) continue;
        if (launch_grouped(fmt, layout, false, a, grid_for(a.total_units), s, chain && !first) !=
            hipSuccess)
            return MXQ_ELAUNCH;
        first = false;
    }
    return MXQ_OK;
}

int nvfp4_quant_grouped_auto(int layout, int64_t cols, const mxq_entry *entries, int n_entries,
                             const int *scale_slot, int n_slots, float *global_scale_out,
                             float *amax_out, void *stream) {
    GroupArgs a;
    const int st = pack_grouped(MXQ_NVFP4, layout, cols, entries, n_entries, false, a);
    if (st != MXQ_OK) return st;
    if (n_slots < 1 || n_slots > MXQ_MAX_GROUP || !global_scale_out || !amax_out)
        return MXQ_EINVAL;
    if (!scale_slot && n_slots != n_entries) return MXQ_EINVAL;
    if ((reinterpret_cast<uintptr_t>(global_scale_out) & 3) != 0 ||
        (reinterpret_cast<uintptr_t>(amax_out) & 3) != 0)
        return MXQ_ESHAPE;
    for (int i = 0; i < n_entries; ++i) {
        const int sl = scale_slot ? scale_slot[i] : i;
        if (sl < 0 || sl >= n_slots) return MXQ_EINVAL;
        a.e[i].slot = sl;
    }
    a.amax_bits = reinterpret_cast<uint32_t *>(amax_out);
    a.g_out = global_scale_out;
    a.n_slots = n_slots;
    hipStream_t s = (hipStream_t)stream;
    const int64_t grid = grid_for(a.total_units);
    if (launch_amax(a, grid, s) != hipSuccess) return MXQ_ELAUNCH;
    // the quantize pass always runs: its workgroup 0 publishes the encode scales
    hipError_t err = launch_grouped(MXQ_NVFP4, layout, true, a, grid, s);
    return err == hipSuccess ? MXQ_OK : MXQ_ELAUNCH;
}

}  // extern "C"

namespace {

// The three split forms share validation and launch packing.  row_scaled
// implies NVFP4; g is read only for tensor-scaled NVFP4.
int quant_split(int fmt, bool row_scaled, const void *src, int64_t total_rows, int64_t cols,
                const int64_t *split_rows, int n_splits, const float *global_scale,
                void *payload, void *scales, float *row_amax, int layout, void *stream) {
    if (!valid_layout(layout) || (!split_rows && n_splits > 0) || n_splits < 0 ||
        total_rows < 0 || total_rows >= (int64_t)1 << 31)
        return MXQ_EINVAL;
    int64_t sum = 0;
    for (int i = 0; i < n_splits; ++i) {
        if (split_rows[i] < 0) return MXQ_EINVAL;
        sum += split_rows[i];
    }
    if (sum != total_rows) return MXQ_EINVAL;
    if (cols <= 0 || cols % block_of(fmt) != 0 || cols > kMaxSplitCols) return MXQ_ESHAPE;
    if (total_rows == 0) return MXQ_OK;
    if (!src || !payload || !scales) return MXQ_EINVAL;
    if (fmt == MXQ_NVFP4 && !row_scaled && !global_scale) return MXQ_EINVAL;
    if (row_scaled && !row_amax) return MXQ_EINVAL;
    if (!aligned16(src) || !aligned16(payload)) return MXQ_ESHAPE;
    if (layout == MXQ_SF_SWIZZLED && !aligned16(scales)) return MXQ_ESHAPE;

    const int64_t C = cols / block_of(fmt);
    const int64_t Cs = layout == MXQ_SF_SWIZZLED ? round_up(C, 4) : C;
    const int64_t payload_ld = fmt == MXQ_MXFP8 ? cols : cols / 2;
    // Linear scales need no per-expert padding: expert i's region starts at
    // o_i * C and its local row r - o_i sits at r * C, so the bulk buffer is
    // the [total_rows, C] scale matrix of the whole activation and the split
    // is one tensor's quantization (units then span expert boundaries).
    const int64_t whole[1] = {total_rows};
    if (layout == MXQ_SF_LINEAR) {
        split_rows = whole;
        n_splits = 1;
    }
    // Empty splits own no rows and no scale bytes, so the launches' tables
    // list only the others: the prefix sums of rows, bands and padding units
    // are the same, and a row's expert is then found in a few steps even when
    // most experts are empty (decode-sized activations).
    int64_t row_base = 0, scale_base = 0;
    int next = 0;  // the next split to place
    while (next < n_splits) {
        SplitArgs a;
        memset(&a, 0, sizeof(a));
        a.src = static_cast<const uint16_t *>(src) + row_base * cols;
        a.payload = static_cast<uint8_t *>(payload) + row_base * payload_ld;
        a.scales = static_cast<uint8_t *>(scales) + scale_base;
        a.row_amax = row_amax ? row_amax + row_base : nullptr;
        a.g = global_scale;
        a.cols = (int32_t)cols;
        a.sf_cols = (int32_t)C;
        a.sf_stride = (int32_t)Cs;
        int n = 0;
        int64_t rows = 0, pads = 0, sbytes = 0, bands = 0;
        for (; next < n_splits && n < kMaxSplitsPerLaunch; ++next) {
            const int64_t m = split_rows[next];
            if (m == 0) continue;
            a.row_off[n] = (int32_t)rows;
            a.unit_off[n] = (int32_t)pads;
            a.band_off[n] = (int32_t)bands;
            ++n;
            rows += m;
            bands += (m + 127) / 128;
            pads += layout == MXQ_SF_SWIZZLED && m % 128 != 0 && m % 128 < 32 ? 1 : 0;
            sbytes += sf_bytes(m, C, layout);
        }
        if (n == 0) break;  // only empty splits were left
        a.n = n;
        a.row_off[n] = (int32_t)rows;
        a.unit_off[n] = (int32_t)pads;
        a.band_off[n] = (int32_t)bands;
        const int64_t ur = split_unit_rows(layout);
        const int64_t units = (rows + ur - 1) / ur + pads;
        a.total_units = (int32_t)units;
        if (units > 0) {
            hipError_t err =
                launch_split(fmt, row_scaled, layout, a, grid_for(units), (hipStream_t)stream);
            if (err != hipSuccess) return MXQ_ELAUNCH;
        }
        row_base += rows;
        scale_base += sbytes;
    }
    return MXQ_OK;
}

}  // namespace

extern "C" {

int nvfp4_quant_split(const void *src, int64_t total_rows, int64_t cols, const int64_t *split_rows,
                      int n_splits, const float *global_scale, void *payload, void *scales,
                      float *row_amax, int layout, void *stream) {
    return quant_split(MXQ_NVFP4, false, src, total_rows, cols, split_rows, n_splits,
                       global_scale, payload, scales, row_amax, layout, stream);
}

int nvfp4_quant_split_row_scaled(const void *src, int64_t total_rows, int64_t cols,
                                 const int64_t *split_rows, int n_splits, void *payload,
                                 void *scales, float *row_amax, int layout, void *stream) {
    return quant_split(MXQ_NVFP4, true, src, total_rows, cols, split_rows, n_splits, nullptr,
                       payload, scales, row_amax, layout, stream);
}

int mxfp8_quant_split(const void *src, int64_t total_rows, int64_t cols, const int64_t *split_rows,
                      int n_splits, void *payload, void *scales, float *row_amax, int layout,
                      void *stream) {
    return quant_split(MXQ_MXFP8, false, src, total_rows, cols, split_rows, n_splits, nullptr,
                       payload, scales, row_amax, layout, stream);
}

int rmsnorm_quant_fused(int fmt, int layout, const void *x, const void *residual,
                        const void *gamma, float eps, int64_t T, int64_t H,
                        const float *global_scale, void *residual_out, void *norm_out,
                        void *payload, void *scales, void *stream) {
    if (!valid_fmt(fmt) || !valid_layout(layout)) return MXQ_EINVAL;
    // eps a normal fp32 (a subnormal eps would let the fp32 sum of squares of
    // a row of tiny values lose accuracy); rows padded to 128 must still index
    // as int32
    if (!(eps >= 0x1p-126f) || !(eps < 3.4e38f) || T < 0 || T > ((int64_t)1 << 31) - 128)
        return MXQ_EINVAL;
    if (H <= 0 || H % block_of(fmt) != 0 || H > kMaxFusedH) return MXQ_ESHAPE;
    const int64_t C = H / block_of(fmt);
    // The swizzled tile needs four scale columns; a hidden size that would pad
    // scale columns is refused rather than leaving unreachable padding.
    if (layout == MXQ_SF_SWIZZLED && C % 4 != 0) return MXQ_ESHAPE;
    if (T == 0) return MXQ_OK;
    if (!x || !residual || !gamma || !residual_out || !norm_out || !payload || !scales)
        return MXQ_EINVAL;
    if (fmt == MXQ_NVFP4 && !global_scale) return MXQ_EINVAL;
    if (!aligned16(x) || !aligned16(residual) || !aligned16(gamma) || !aligned16(residual_out) ||
        !aligned16(norm_out) || !aligned16(payload) || !aligned16(scales))
        return MXQ_ESHAPE;
    FusedArgs a;
    memset(&a, 0, sizeof(a));
    a.x = static_cast<const uint16_t *>(x);
    a.res = static_cast<const uint16_t *>(residual);
    a.gamma = static_cast<const uint16_t *>(gamma);
    a.res_out = static_cast<uint16_t *>(residual_out);
    a.norm_out = static_cast<uint16_t *>(norm_out);
    a.payload = static_cast<uint8_t *>(payload);
    a.scales = static_cast<uint8_t *>(scales);
    a.g = global_scale;
    a.eps = eps;
    a.T = (int32_t)T;
    a.H = (int32_t)H;
    a.sf_cols = (int32_t)C;
    a.sf_stride = (int32_t)(layout == MXQ_SF_SWIZZLED ? round_up(C, 4) : C);
    const int64_t wide_max =
        layout == MXQ_SF_SWIZZLED ? kFusedWideMaxTSwizzled : kFusedWideMaxTLinear;
    a.wpr = T <= wide_max ? 16 : T <= kFusedFourWaveMaxT ? 4 : 2;
    a.rpu = a.wpr == 2 ? 4 : 1;
    hipError_t err;
    if (layout == MXQ_SF_SWIZZLED && fused_tiny_rows(T) && H <= 16 * kChunk &&
        grid_for(T) == T) {
        // a few rows: one workgroup per live row, no padding units
        a.wpr = 16;
        a.total_units = (int32_t)T;
        err = launch_fused_tiny(fmt, a, (hipStream_t)stream);
    } else {
        const int64_t units = row_groups(T, layout, a.rpu);
        a.total_units = (int32_t)units;
        err = launch_fused(fmt, layout, a, grid_for(units), (hipStream_t)stream);
    }
    return err == hipSuccess ? MXQ_OK : MXQ_ELAUNCH;
}

int scale_swizzle(const void *linear, int64_t rows, int64_t sf_cols, void *swizzled, void *stream) {
    if (rows < 0 || sf_cols <= 0 || rows >= (int64_t)1 << 40 || sf_cols >= (int64_t)1 << 31)
        return MXQ_EINVAL;
    if (rows == 0) return MXQ_OK;
    if (!linear || !swizzled) return MXQ_EINVAL;
    if (!aligned16(swizzled)) return MXQ_ESHAPE;
    SwizzleArgs a;
    a.lin = static_cast<const uint8_t *>(linear);
    a.swz = static_cast<uint8_t *>(swizzled);
    a.rows = rows;
    a.cols = sf_cols;
    a.tiles_per_band = round_up(sf_cols, 4) / 4;
    a.unit_tiles = (int32_t)(a.tiles_per_band < kSwizzleTiles ? a.tiles_per_band : kSwizzleTiles);
    // units: 128-row bands x groups of unit_tiles tiles
    int64_t grid = (rows + 127) / 128 * ((a.tiles_per_band + a.unit_tiles - 1) / a.unit_tiles);
    if (grid > 65536) grid = 65536;
    hipError_t err = launch_swizzle(a, grid_for(grid), (hipStream_t)stream);
    return err == hipSuccess ? MXQ_OK : MXQ_ELAUNCH;
}

}  // extern "C"
