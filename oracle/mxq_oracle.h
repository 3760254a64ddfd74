/*
 * mxq_oracle.h -- plain, slow, CPU-only reference for block-scaled (MXFP8 /
 * NVFP4) quantization of MoE expert tensors.
 *
 * THIS IS TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no source, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * Sources (pages, cited by title and section):
 *   [RL-3804]  NVIDIA-NeMo/RL #3804 "perf(refit): batch MXFP8 expert
 *              prequantization" -- Summary; Self-review > Verified clean.
 *   [MO-2750]  NVIDIA/Model-Optimizer #2750 "Fold fused experts' quantizers
 *              into their weights shard-locally" -- commit messages; review.
 *   [TRT-17452] NVIDIA/TensorRT-LLM #17452 "NVFP4 linear-SF AllReduce
 *              epilogue" -- commit messages (layout; fold; exactness test).
 *   [TE-3800]  NVIDIA/TransformerEngine #3800 (split quantization of
 *              row-scaled NVFP4 activations) -- Description; Changes.
 *   [TRT-17453] NVIDIA/TensorRT-LLM #17453 "MXFP8 carrier and quantize
 *              folds" -- commit messages (Triton func; merge kernel; sweep
 *              and invariance tests; AllReduce epilogue).
 * Format definitions follow the public OCP 8-bit floating point (OFP8) spec
 * (E4M3, the no-infinity variant with largest finite 448), the OCP
 * Microscaling (MX) v1.0 spec (E8M0, E2M1, 32-element blocks), and the public
 * NVFP4 description (16-element blocks, E4M3 block scale, fp32 second-level
 * scale).
 *
 * Everything is computed in double precision except where a reading below
 * fixes an fp32 operation; each such operation is written as a C float
 * operation (IEEE-754 binary32, round-to-nearest-even, no contraction).
 *
 * Readings the pages leave open: the 128x4 swizzle permutation, the E2M1
 * nibble order, the NVFP4 arithmetic order and the encode-scale formula.  Each
 * is taken as stated at its function and pinned by hand-derived fixtures
 * (tests/golden/), so no function here is left without a pin.
 */
#ifndef MXQ_ORACLE_H
#define MXQ_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_MXFP8 = 0, ORC_NVFP4 = 1 };
enum { ORC_LINEAR = 0, ORC_SWIZZLED = 1 };

/* ---- element formats ------------------------------------------------- */
double   orc_bf16_value(uint16_t bits);
uint16_t orc_bf16_round(double v);        /* nearest bf16, ties to even       */
double   orc_e4m3_value(uint8_t code);    /* NaN codes 0x7F / 0xFF -> NaN     */
uint8_t  orc_e4m3_encode(double v);       /* nearest, ties even, sat. +-448   */
double   orc_e2m1_value(uint8_t code);    /* low nibble of code               */
uint8_t  orc_e2m1_encode(double v);       /* nearest, ties even, sat. +-6     */
double   orc_e8m0_value(uint8_t code);    /* 2^(code-127); 0xFF -> NaN        */

/* ---- block rules ------------------------------------------------------ */
uint8_t orc_mxfp8_scale_code(double amax);
double  orc_mxfp8_multiplier(uint8_t code);
void    orc_mxfp8_block(const uint16_t *x, int n, uint8_t *payload, uint8_t *scale);
void    orc_nvfp4_block(const uint16_t *x, int n, float g, uint8_t *payload, uint8_t *scale);

/* ---- scale layouts ---------------------------------------------------- */
int64_t orc_sf_cols(int64_t cols, int fmt);
int64_t orc_sf_bytes(int64_t rows, int64_t sf_cols, int layout);
int64_t orc_sf_offset(int64_t r, int64_t c, int64_t sf_cols, int layout);

/* ---- whole tensors ---------------------------------------------------- */
/* One expert tensor: bf16 [rows, cols] with row stride ld (elements).  The
 * payload is dense: [rows, cols] (MXFP8) or [rows, cols/2] (NVFP4).  The scale
 * region holds orc_sf_bytes(rows, sf_cols, layout) bytes, every one written. */
int orc_quantize(int fmt, int layout, const uint16_t *src, int64_t rows, int64_t cols,
                 int64_t ld, float g, uint8_t *payload, uint8_t *scales);

/* Concatenated activation bf16 [total_rows, cols] split into n experts. */
int64_t orc_split_scale_offset(const int64_t *split_rows, int n, int i, int64_t cols,
                               int fmt, int layout);
int orc_nvfp4_split(const uint16_t *src, int64_t total_rows, int64_t cols,
                    const int64_t *split_rows, int n, float g, int layout,
                    uint8_t *payload, uint8_t *scales, float *row_amax);
/* Any format: MXFP8 (g ignored), NVFP4 under one encode scale g, or, with
 * row_scaled != 0, NVFP4 where row r uses orc_nvfp4_encode_scale(row_amax[r]). */
int orc_split(int fmt, int row_scaled, const uint16_t *src, int64_t total_rows, int64_t cols,
              const int64_t *split_rows, int n, float g, int layout, uint8_t *payload,
              uint8_t *scales, float *row_amax);
/* NVFP4 encode scale from an amax (a tensor's or a row's): 1 for amax 0,
 * else fp32(2688 / amax), capped at FLT_MAX * 2^-9 (every block multiplier
 * g / s_q then stays finite). */
float orc_nvfp4_encode_scale(float amax);
/* max |x| over a bf16 [rows, cols] tensor with row stride ld. */
float orc_tensor_amax(const uint16_t *src, int64_t rows, int64_t cols, int64_t ld);

/* Residual add + RMSNorm: residual_out = bf16(x + res);
 * norm_out = bf16(r * gamma / sqrt(mean(r^2) + eps)), computed in double. */
int orc_add_rmsnorm(const uint16_t *x, const uint16_t *res, const uint16_t *gamma,
                    float eps, int64_t T, int64_t H, uint16_t *residual_out,
                    uint16_t *norm_out);

/* Linear [rows, sf_cols] scale bytes -> swizzled 128x4 layout, zero padded. */
int orc_scale_swizzle(const uint8_t *linear, int64_t rows, int64_t sf_cols, uint8_t *swizzled);

/* Vector helpers for exhaustive checks (apply the scalar rule elementwise). */
void orc_e4m3_encode_f32(const float *v, int64_t n, uint8_t *out);
void orc_e2m1_encode_f32(const float *v, int64_t n, uint8_t *out);
void orc_mxfp8_scale_code_bf16(const uint16_t *amax_bits, int64_t n, uint8_t *out);
void orc_mxfp8_elements(const uint16_t *x, int64_t n, uint8_t code, uint8_t *out);

#ifdef __cplusplus
}
#endif
#endif
