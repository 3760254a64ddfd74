/*
 * mxq.h -- C ABI of the MI355X (gfx950) block-scaled quantization library
 * for Mixture-of-Experts tensors: MXFP8 and NVFP4, grouped over experts or
 * split per expert, with linear or swizzled 128x4 scale layouts, and a fused
 * residual-add + RMSNorm + quantize epilogue.
 *
 * Pages the operations come from (cited by title and section):
 *   [RL-3804]   NVIDIA-NeMo/RL #3804 "perf(refit): batch MXFP8 expert
 *               prequantization" (Summary; Why; Self-review > Verified clean)
 *   [MO-2750]   NVIDIA/Model-Optimizer #2750 "Fold fused experts' quantizers
 *               into their weights shard-locally" (commits; review)
 *   [TRT-17452] NVIDIA/TensorRT-LLM #17452 "NVFP4 linear-SF AllReduce
 *               epilogue" (layout, fold and exactness-test commits)
 *   [TE-3800]   NVIDIA/TransformerEngine #3800, split quantization of
 *               row-scaled NVFP4 activations (Description; Changes; diagram)
 *   [TRT-17453] NVIDIA/TensorRT-LLM #17453 "MXFP8 carrier and quantize
 *               folds" (Triton func, merge kernel, invariance-test and
 *               AllReduce-epilogue commits)
 *
 * Formats.  Input elements are bf16.  MXFP8: blocks of 32 contiguous row
 * elements, one E8M0 scale byte per block (code c means 2^(c-127); c is the
 * smallest code with amax <= 448 * 2^(c-127)), E4M3 elements (OCP, largest
 * finite 448, round to nearest even, sign of zero kept; the reciprocal of the
 * block scale is flushed to zero when the scale or the reciprocal is not a
 * normal fp32 number).  NVFP4: blocks of 16, one E4M3 scale byte per block
 * under an fp32 encode scale g (block scale s = fp32(fp32(amax/6) * g)
 * rounded to E4M3 with saturation; element multiplier fp32(g / s_q)), E2M1
 * elements saturating at 6, two per byte, element 2j in the low nibble of
 * byte j; the multiplier is flushed to 0 when it is not a normal fp32 number
 * (subnormal, or infinite after overflow), the NVFP4 form of the flush on the
 * block-scale reciprocal.  An NVFP4 encode scale g may be any positive finite
 * fp32 number, subnormal included (it is a device value the library cannot
 * check: zero, negative, infinite or NaN g give unspecified bytes).  Results
 * are bit-identical to the definitions above, whatever the grouping, split or
 * launch shape.
 *
 * Scale layouts [TRT-17452, layout commit; TRT-17453, AllReduce epilogue
 * commit].  LINEAR: byte (r, c) of an [R, C] scale matrix at r*C + c.
 * SWIZZLED_128x4: rows padded to a multiple of 128, columns to a multiple of
 * 4; each 128x4 tile is 512 contiguous bytes, tiles in row-tile-major order;
 * inside a tile (r, c) is at (r%32)*16 + ((r%128)/32)*4 + c%4.  Every padding
 * byte is written as 0, so scale buffers need no prior zeroing
 * [TRT-17453, merge-kernel commit].
 *
 * Ownership and streams.  The caller owns every buffer; the library keeps no
 * allocation, stream, cache or mutable state other than the debug grid cap
 * below.  Pointers marked "device" are device memory; everything else is host
 * memory read during the call only.  All GPU work is enqueued on `stream`
 * (a hipStream_t; NULL is the null stream) and the call returns without
 * synchronizing; the caller makes the inputs ready on that stream.  No call
 * allocates, copies or synchronizes, so every call may be captured in a HIP
 * graph.  Outputs must not alias inputs or each other.
 *
 * Errors.  Every call validates all arguments on the host first; when a check
 * fails it returns a nonzero mxq_status, launches nothing and writes nothing.
 * MXQ_ELAUNCH reports a kernel launch that the HIP runtime rejected after
 * validation passed.  A call that issues several launches
 * (mx_quant_grouped_batch; nvfp4_quant_grouped_auto; a split with more than
 * 256 non-empty experts)
 * may then have enqueued the launches before the failed one, so after
 * MXQ_ELAUNCH every output of the call is unspecified.
 */
#ifndef MXQ_H
#define MXQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MXQ_OK = 0,
    MXQ_EINVAL = 1,       /* null pointer, bad enum, bad count or split, bad eps       */
    MXQ_ESHAPE = 2,       /* cols not a multiple of the block, misaligned pointer ... */
    MXQ_EUNSUPPORTED = 3, /* a combination the library does not implement           */
    MXQ_ELAUNCH = 4       /* the HIP runtime rejected a kernel launch                 */
} mxq_status;

typedef enum { MXQ_MXFP8 = 0, MXQ_NVFP4 = 1 } mxq_format;
typedef enum { MXQ_SF_LINEAR = 0, MXQ_SF_SWIZZLED = 1 } mxq_sf_layout;

#define MXQ_MAX_GROUP 16 /* experts per grouped call [RL-3804, Summary] */

/* One expert tensor of a grouped call. */
typedef struct {
    const void *src;          /* device bf16 [rows, src_ld], 16-byte aligned; the
                                 first `cols` elements of each row are read     */
    void *payload;            /* device u8, dense: MXFP8 [rows, cols], NVFP4
                                 [rows, cols/2]; 16-byte aligned                 */
    void *scales;             /* device u8, mxq_scale_bytes(rows, cols, fmt,
                                 layout) bytes; 16-byte aligned if swizzled     */
    const float *global_scale;/* device fp32 scalar: NVFP4 encode scale g,
                                 positive and finite; ignored for MXFP8         */
    int64_t rows;             /* 0 .. 2^31 - 128; 0 writes nothing             */
    int64_t src_ld;           /* row stride in elements: >= cols, multiple of 8 */
} mxq_entry;

/*
 * mx_quant_grouped -- quantize 1..16 expert tensors that share `cols` in ONE
 * kernel launch driven by a descriptor table [RL-3804, Summary; Why;
 * Self-review > Verified clean: batched quantization is bit-identical to the
 * per-tensor path because the format is row-independent; a per-call cap of
 * 16, where one entry is exactly the per-expert path].
 *   fmt, layout  mxq_format, mxq_sf_layout
 *   cols         elements per row; a multiple of 32 (MXFP8) or 16 (NVFP4),
 *                at most 32768 (MXFP8) or 16384 (NVFP4)
 *   entries      host array of n_entries descriptors; each entry's rows may
 *                differ
 * Returns MXQ_EINVAL for n_entries outside [1, 16], a null pointer or a bad
 * enum; MXQ_ESHAPE for a bad cols, src_ld or alignment.
 */
int mx_quant_grouped(int fmt, int layout, int64_t cols, const mxq_entry *entries, int n_entries,
                     void *stream);

/*
 * mx_quant_grouped_batch -- mx_quant_grouped over any number of entries that
 * share `cols` (a model's experts of one projection, say): ceil(n_entries /
 * per_launch) launches of up to per_launch (1..16) entries, in entry order,
 * on `stream` [RL-3804, Summary: batches of at most 16 experts; Why: the
 * per-launch cost is what batching removes].  The bytes are those of
 * mx_quant_grouped on each batch.
 *   flags  0, or MXQ_CHAIN: every launch after the first is dispatched with
 *          HIP's any-order launch (the barrier bit of its dispatch packet
 *          clear), so it may start while the previous launch drains, hiding
 *          that launch's ramp and tail.  The first launch is ordinary, so the
 *          whole call still follows everything queued before it, and work
 *          queued after the call still follows all of its launches.  The
 *          launches of one call read only inputs and write only distinct
 *          outputs (outputs must not alias inputs or each other, across the
 *          whole call), so their order does not matter.  On a stream being
 *          captured into a graph the launches are ordinary.  Measured: a
 *          Qwen3-30B-A3B-shaped layer's 2 x 8 launches of 76-153 MB take
 *          348 -> 328 us; launches of 300 MB and more gain nothing (about 1 %
 *          slower), so leave it off there.
 * Every batch is validated before the first launch; errors as
 * mx_quant_grouped, plus MXQ_EINVAL for n_entries < 1, per_launch outside
 * [1, 16] or an unknown flag.
 */
#define MXQ_CHAIN 1u
int mx_quant_grouped_batch(int fmt, int layout, int64_t cols, const mxq_entry *entries,
                           int n_entries, int per_launch, unsigned flags, void *stream);

/*
 * nvfp4_quant_grouped_auto -- mx_quant_grouped for NVFP4 with the encode
 * scales computed from the data in the same call [MO-2750, review: the
 * second-level scale is a per-expert scalar, shared by gate and up because
 * the fused gate/up slice has one amax].  Entry i belongs to scale slot
 * scale_slot[i]; a slot's amax is the max |x| over all of its entries and its
 * encode scale is
 *     g_s = 1 if amax_s = 0, else min(fp32(2688 / amax_s), FLT_MAX * 2^-9)
 * (2688 = 448 * 6; the pages print no formula; the cap is the largest g for
 * which every multiplier g / s_q, s_q >= 2^-9, is finite, and only amax below
 * about 2^-107.6 reaches it).  Every entry is then
 * quantized exactly as mx_quant_grouped(MXQ_NVFP4, ...) with g = g_s of its
 * slot.  entries[i].global_scale is ignored.
 *   scale_slot        host int[n_entries], values in [0, n_slots), or NULL
 *                     for one slot per entry (then n_slots == n_entries)
 *   n_slots           1..16
 *   global_scale_out  device fp32 [n_slots]: g_s (every slot written; a slot
 *                     with no rows gets amax 0 and g 1)
 *   amax_out          device fp32 [n_slots]: amax_s; also the reduction's
 *                     accumulator, so it must not alias anything else
 * Three kernels on `stream` (zero the accumulators, per-slot amax, quantize):
 * the input is read twice.  On MXQ_ELAUNCH the outputs are unspecified.
 */
int nvfp4_quant_grouped_auto(int layout, int64_t cols, const mxq_entry *entries, int n_entries,
                             const int *scale_slot, int n_slots, float *global_scale_out,
                             float *amax_out, void *stream);

/*
 * nvfp4_quant_split -- quantize a concatenated routed activation once and
 * split it per expert [TE-3800, Description; Changes: independent per-expert
 * scale padding including uneven and empty splits; requantizing one expert
 * does not modify another expert's storage; diagram: split packed values and
 * row amax, split scales with separate expert padding].
 *   src          device bf16 [total_rows, cols], contiguous, 16-byte aligned
 *   split_rows   host int64[n_splits], each >= 0, summing to total_rows;
 *                expert i owns rows [o_i, o_i + m_i), o_i = sum_{j<i} m_j
 *   global_scale device fp32 scalar g shared by all rows (as for entries)
 *   payload      device u8 [total_rows, cols/2]; expert i's rows are rows
 *                [o_i, o_i + m_i) (16-byte aligned base)
 *   scales       device u8 bulk buffer; expert i's scale matrix [m_i, cols/16]
 *                in `layout` starts at mxq_split_scale_offset(..., i, ...) and
 *                holds mxq_scale_bytes(m_i, cols, MXQ_NVFP4, layout) bytes:
 *                swizzled pads each expert to a multiple of 128 rows; an empty
 *                expert owns no bytes (16-byte aligned base if swizzled)
 *   row_amax     device fp32 [total_rows]: max_j |src[r, j]| (NULL to skip)
 * cols is a multiple of 16, at most 16384.  Any number of splits is allowed,
 * none included (then total_rows must be 0 and split_rows may be NULL).
 * 0 <= total_rows < 2^31, else MXQ_EINVAL; total_rows == 0 is MXQ_OK with no
 * launch.
 */
int nvfp4_quant_split(const void *src, int64_t total_rows, int64_t cols,
                      const int64_t *split_rows, int n_splits, const float *global_scale,
                      void *payload, void *scales, float *row_amax, int layout, void *stream);

/*
 * nvfp4_quant_split_row_scaled -- the split of nvfp4_quant_split with a
 * second-level scale per row instead of one per tensor [TE-3800,
 * Description: row-scaled NVFP4 activations are quantized once and their
 * payload and row-scale metadata partitioned per expert; diagram: split
 * packed values and row amax].  Row r is quantized under its own encode scale
 *     g_r = 1                                        if a_r = 0,
 *     g_r = min(fp32(2688 / a_r), FLT_MAX * 2^-9)    otherwise,
 * a_r = max_j |src[r, j]| (2688 = 448 * 6: the row amax lands on the largest
 * E4M3 block scale times the largest E2M1 element; the pages print no
 * formula, this is the per-tensor convention applied per row; the cap keeps
 * every block multiplier finite, and no lower bound is needed because
 * 2688 / a_r >= 2688 / FLT_MAX keeps every multiplier normal).  The decode scale of row r
 * is 1 / g_r, which a consumer recomputes from row_amax.
 *   row_amax     device fp32 [total_rows], REQUIRED: a_r of every row
 * Everything else as nvfp4_quant_split (no global_scale).
 */
int nvfp4_quant_split_row_scaled(const void *src, int64_t total_rows, int64_t cols,
                                 const int64_t *split_rows, int n_splits, void *payload,
                                 void *scales, float *row_amax, int layout, void *stream);

/*
 * mxfp8_quant_split -- the same quantize-once-and-split for MXFP8 [TE-3800,
 * Description: MXFP8 is the control of the split measurements].
 *   payload      device u8 [total_rows, cols]; expert i's rows [o_i, o_i + m_i)
 *   scales       bulk buffer as in nvfp4_quant_split with fmt MXQ_MXFP8:
 *                expert i at mxq_split_scale_offset(..., i, cols, MXQ_MXFP8,
 *                layout), [m_i, cols/32] in `layout`, swizzled rows padded per
 *                expert to 128
 *   row_amax     device fp32 [total_rows] or NULL
 * cols is a multiple of 32, at most 16384.
 */
int mxfp8_quant_split(const void *src, int64_t total_rows, int64_t cols,
                      const int64_t *split_rows, int n_splits, void *payload, void *scales,
                      float *row_amax, int layout, void *stream);

/*
 * rmsnorm_quant_fused -- residual add + RMSNorm + block quantization in one
 * pass [TRT-17452, fold commit: the epilogue quantizes the same bf16 values
 * it writes to norm_out; TRT-17453, AllReduce epilogue commit: bitwise equal
 * to quantizing norm_out afterwards, the invented scale rows past the last
 * live row are zeroed by the kernel, a hidden size that would pad scale
 * columns is rejected on the host].  Single GPU; no collective.
 *   x, residual  device bf16 [T, H]; gamma device bf16 [H]
 *   residual_out device bf16 [T, H] = bf16(x + residual)
 *   norm_out     device bf16 [T, H] = bf16(r * gamma / sqrt(mean(r^2) + eps)),
 *                fp32 arithmetic, within 1 bf16 ulp of the exact value while
 *                every |r| < 2^64 / sqrt(H) and |r * gamma| < 2^127 (the fp32
 *                sum of squares and products stay finite); beyond that the
 *                value is unspecified
 *   payload, scales  fmt/layout quantization of norm_out (as mx_quant_grouped
 *                with rows = T, cols = H); swizzled scale rows T..round_up(T,128)
 *                are written as zero
 *   global_scale device fp32 g for NVFP4; ignored for MXFP8
 * H is a multiple of 32 (MXFP8) or 16 (NVFP4) and at most 16384; with the
 * swizzled layout H must also give a multiple of 4 scale columns (H % 128 == 0
 * for MXFP8, H % 64 == 0 for NVFP4), else MXQ_ESHAPE.  eps must be finite and
 * at least 2^-126 (a normal fp32); 0 <= T <= 2^31 - 128, else MXQ_EINVAL.  T == 0 is MXQ_OK with no
 * launch.  All pointers 16-byte aligned.
 */
int rmsnorm_quant_fused(int fmt, int layout, const void *x, const void *residual,
                        const void *gamma, float eps, int64_t T, int64_t H,
                        const float *global_scale, void *residual_out, void *norm_out,
                        void *payload, void *scales, void *stream);

/*
 * scale_swizzle -- convert a linear [rows, sf_cols] scale matrix to the
 * swizzled 128x4 layout, zero padded [RL-3804, Summary: receiver-side layout
 * conversion; TRT-17453, invariance-test commit: the two layouts agree].
 *   linear    device u8 [rows, sf_cols], any alignment
 *   swizzled  device u8 [round_up(rows,128) * round_up(sf_cols,4)], 16-byte
 *             aligned
 * 0 <= rows < 2^40 and 1 <= sf_cols < 2^31, else MXQ_EINVAL; rows == 0 is
 * MXQ_OK with no launch.
 */
int scale_swizzle(const void *linear, int64_t rows, int64_t sf_cols, void *swizzled,
                  void *stream);

/* Size of one scale matrix for a [rows, cols] tensor; -1 on bad arguments. */
int64_t mxq_scale_bytes(int64_t rows, int64_t cols, int fmt, int layout);

/* Byte offset of split i's scales in the bulk buffer (i == n_splits gives the
 * total size; split_rows may be NULL when n_splits == 0); -1 on bad
 * arguments. */
int64_t mxq_split_scale_offset(const int64_t *split_rows, int n_splits, int i, int64_t cols,
                               int fmt, int layout);

/* Static description of a status code. */
const char *mxq_status_str(int status);

/* Debug and test knob: cap the number of workgroups a launch may use
 * (0 restores the default).  Outputs do not depend on it; the tests use it to
 * show that.  Process-wide; not thread-safe. */
void mxq_set_max_workgroups(int64_t n);

#ifdef __cplusplus
}
#endif
#endif /* MXQ_H */
