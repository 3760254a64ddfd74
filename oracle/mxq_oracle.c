/*
 * mxq_oracle.c -- plain CPU reference for MXFP8 / NVFP4 block quantization.
 *
 * TEST INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline).  No
 * code here is shared with, or called by, the GPU library.
 *
 * Every rule is written as its definition, step by step, in the order the
 * rules are stated.  Rounding to a format is "the nearest value of the
 * format, ties to the even significand" (the pages call the quantizers
 * deterministic: [TE-3800, Changes]); values are held in double, where every
 * bf16, E4M3, E2M1 and power-of-two product used here is exact.  Where a rule
 * fixes an fp32 operation (the NVFP4 scale arithmetic) it is a C float
 * operation, which on the x86-64 SSE target is IEEE binary32 with round to
 * nearest even; the build disables contraction and fast-math.
 */
#include "mxq_oracle.h"

#include <assert.h>
#include <float.h>
#include <math.h>
#include <string.h>

/* ----------------------------------------------------------------------- */
/* Rounding onto the grid of a small binary floating-point format.          */
/* ----------------------------------------------------------------------- */

/* Nearest value to a >= 0 on the grid of a binary format with `mbits`
 * explicit significand bits and smallest normal exponent `emin`.  Inside the
 * binade [2^e, 2^(e+1)) the spacing is 2^(e - mbits); below 2^emin the spacing
 * stays 2^(emin - mbits) (the subnormals).  A tie goes to the even multiple of
 * the spacing, which is the even significand.  The result may be 2^(e+1)
 * (carry into the next binade).  No upper limit is applied here. */
static double round_to_grid(double a, int emin, int mbits)
{
    int e;
    double spacing;
    assert(a >= 0.0 && isfinite(a));
    if (a == 0.0)
        return 0.0;
    (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1): a lies in [2^(e-1), 2^e) */
    e -= 1;
    if (e < emin)
        e = emin;
    spacing = ldexp(1.0, e - mbits);
    return nearbyint(a / spacing) * spacing; /* a/spacing is exact; ties to even */
}

/* Exponent e with v in [2^e, 2^(e+1)), for v > 0. */
static int binade(double v)
{
    int e;
    (void)frexp(v, &e);
    return e - 1;
}

/* ----------------------------------------------------------------------- */
/* bf16: 1 sign, 8 exponent bits (bias 127), 7 mantissa bits.               */
/* ----------------------------------------------------------------------- */

double orc_bf16_value(uint16_t bits)
{
    int s = bits >> 15, e = (bits >> 7) & 0xFF, m = bits & 0x7F;
    double v;
    if (e == 0xFF)
        v = m ? NAN : INFINITY;
    else if (e == 0)
        v = ldexp((double)m, -133); /* subnormal: m/128 * 2^-126 */
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return s ? -v : v;
}

uint16_t orc_bf16_round(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v), r;
    assert(!isnan(v));
    if (isinf(a))
        return sign | 0x7F80;
    r = round_to_grid(a, -126, 7);
    if (r >= ldexp(1.0, 128))
        return sign | 0x7F80; /* rounds past the largest finite value */
    if (r < ldexp(1.0, -126))
        return sign | (uint16_t)(r / ldexp(1.0, -133)); /* subnormal (or zero) */
    {
        int e = binade(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 128.0);
        return sign | (uint16_t)(((e + 127) << 7) | m);
    }
}

/* ----------------------------------------------------------------------- */
/* E4M3 (OCP OFP8 E4M3, no infinities): 1 sign, 4 exponent bits (bias 7),    */
/* 3 mantissa bits; S.1111.111 is NaN; the largest finite value is 448.     */
/* ----------------------------------------------------------------------- */

double orc_e4m3_value(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

uint8_t orc_e4m3_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00; /* the sign of zero is kept */
    double a = fabs(v), r;
    assert(!isnan(v));
    if (a >= 448.0)
        return sign | 0x7E; /* saturate, never NaN */
    r = round_to_grid(a, -6, 3);
    if (r > 448.0)
        r = 448.0;
    if (r < ldexp(1.0, -6))
        return sign | (uint8_t)(r / ldexp(1.0, -9)); /* subnormal m * 2^-9 */
    {
        int e = binade(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
        return sign | (uint8_t)(((e + 7) << 3) | m);
    }
}

/* ----------------------------------------------------------------------- */
/* E2M1 (OCP MX FP4): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.      */
/* Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; no NaN or infinity.               */
/* ----------------------------------------------------------------------- */

double orc_e2m1_value(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

uint8_t orc_e2m1_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs(v), r;
    assert(!isnan(v));
    if (a >= 6.0)
        return sign | 0x7; /* saturate */
    r = round_to_grid(a, 0, 1);
    if (r > 6.0)
        r = 6.0;
    if (r < 1.0)
        return sign | (uint8_t)(r / 0.5); /* 0 or 0.5 */
    {
        int e = binade(r);
        int m = (int)((r / ldexp(1.0, e) - 1.0) * 2.0);
        return sign | (uint8_t)(((e + 1) << 1) | m);
    }
}

/* E8M0 (OCP MX scale): 2^(code - 127), code 0xFF is NaN. */
double orc_e8m0_value(uint8_t code)
{
    return code == 0xFF ? NAN : ldexp(1.0, (int)code - 127);
}

/* ----------------------------------------------------------------------- */
/* MXFP8 block: 32 contiguous row elements, E8M0 scale, E4M3 elements.       */
/* [RL-3804, Self-review > Verified clean]: per-block, row-independent, with  */
/* a zero-scale clamp.  [TRT-17453, Triton func commit]: flush-to-zero on the */
/* reciprocal of the block scale.                                           */
/* ----------------------------------------------------------------------- */

/* Scale code c: the smallest c in [0, 254] whose scale 2^(c-127) brings the
 * block maximum into E4M3 range, amax <= 448 * 2^(c-127).  (Exponent rounded
 * up, so the largest element never saturates.)  amax = 0 gives c = 0. */
uint8_t orc_mxfp8_scale_code(double amax)
{
    int c;
    assert(amax >= 0.0 && !isnan(amax));
    for (c = 0; c <= 254; ++c)
        if (amax <= 448.0 * ldexp(1.0, c - 127))
            return (uint8_t)c;
    return 254;
}

/* Element multiplier m = 1 / 2^(c-127), taken flush-to-zero: when the scale
 * is not a normal fp32 number (c = 0 gives 2^-127) or its reciprocal is not a
 * normal fp32 number (c = 254), m = 0 and the block's elements encode as
 * signed zeros. */
double orc_mxfp8_multiplier(uint8_t code)
{
    double scale = ldexp(1.0, (int)code - 127);
    double m;
    if (scale < FLT_MIN)
        return 0.0;
    m = 1.0 / scale; /* exact: a power of two */
    if (m < FLT_MIN)
        return 0.0;
    return m;
}

void orc_mxfp8_block(const uint16_t *x, int n, uint8_t *payload, uint8_t *scale)
{
    double amax = 0.0, m;
    uint8_t c;
    int i;
    for (i = 0; i < n; ++i) {
        double v = orc_bf16_value(x[i]);
        assert(isfinite(v));
        if (fabs(v) > amax)
            amax = fabs(v);
    }
    c = orc_mxfp8_scale_code(amax);
    m = orc_mxfp8_multiplier(c);
    for (i = 0; i < n; ++i)
        payload[i] = orc_e4m3_encode(orc_bf16_value(x[i]) * m); /* product exact */
    *scale = c;
}

/* ----------------------------------------------------------------------- */
/* NVFP4 block: 16 contiguous row elements, E4M3 block scale under an fp32   */
/* second-level encode scale g, E2M1 elements packed two per byte.          */
/* [TRT-17452, exactness-test commit]: the quantize takes the scale as an     */
/* argument.  [MO-2750, review]: one fp32 second-level scale per expert,     */
/* shared by the fused gate/up.                                             */
/* Reading fixed here: s = fp32(fp32(amax / 6) * g); the block scale code is  */
/* E4M3(s); the element multiplier is fp32(g / decode(code)), zero when the  */
/* decoded scale is zero or the multiplier is not a normal fp32 number       */
/* (subnormal, or infinite after overflow: the flush-to-zero of the block-   */
/* scale reciprocal, [TRT-17453, Triton func commit], applied to any result  */
/* outside the normal range); each element is E2M1(fp32(x * m)); element 2j  */
/* goes to the low nibble of byte j.  g is any positive finite fp32 number.  */
/* ----------------------------------------------------------------------- */

void orc_nvfp4_block(const uint16_t *x, int n, float g, uint8_t *payload, uint8_t *scale)
{
    double amax = 0.0;
    float a, t, s, sq, m;
    uint8_t k;
    int i;
    for (i = 0; i < n; ++i) {
        double v = orc_bf16_value(x[i]);
        assert(isfinite(v));
        if (fabs(v) > amax)
            amax = fabs(v);
    }
    a = (float)amax; /* exact: a bf16 value */
    t = a / 6.0f;    /* fp32 division, correctly rounded */
    s = t * g;       /* fp32 product, correctly rounded */
    k = orc_e4m3_encode((double)s);
    sq = (float)orc_e4m3_value(k);
    assert(g > 0.0f && g <= FLT_MAX);
    m = 0.0f;
    if (sq != 0.0f) {
        m = g / sq; /* fp32 division, correctly rounded (may overflow to inf) */
        if (!(m >= FLT_MIN && m <= FLT_MAX))
            m = 0.0f; /* not a normal number: flushed */
    }
    for (i = 0; i < n; i += 2)
        payload[i / 2] = 0;
    for (i = 0; i < n; ++i) {
        float xf = (float)orc_bf16_value(x[i]); /* exact */
        float y = xf * m;                       /* fp32 product, correctly rounded */
        uint8_t q = orc_e2m1_encode((double)y);
        payload[i / 2] |= (uint8_t)(q << (4 * (i & 1)));
    }
    *scale = k;
}

/* ----------------------------------------------------------------------- */
/* Scale-factor layouts.                                                     */
/* LINEAR [TRT-17452, layout commit]: byte (r, c) at r * C + c, no padding.  */
/* SWIZZLED 128x4 [TRT-17452, layout commit; TRT-17453, AllReduce epilogue   */
/* commit]: rows padded to a multiple of 128 and columns to a multiple of 4; */
/* each 128-row x 4-column tile is 512 contiguous bytes, tiles ordered by    */
/* row tile then column tile; inside a tile, row r and column c sit at       */
/* (r mod 32) * 16 + ((r mod 128) div 32) * 4 + (c mod 4).  Padding bytes    */
/* are zero.  (The in-tile permutation is the public block-scaled GEMM      */
/* scale layout; the pages name it but do not spell it out.)                */
/* ----------------------------------------------------------------------- */

static int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

int64_t orc_sf_cols(int64_t cols, int fmt) { return cols / (fmt == ORC_MXFP8 ? 32 : 16); }

int64_t orc_sf_bytes(int64_t rows, int64_t sf_cols, int layout)
{
    if (layout == ORC_LINEAR)
        return rows * sf_cols;
    return round_up(rows, 128) * round_up(sf_cols, 4);
}

int64_t orc_sf_offset(int64_t r, int64_t c, int64_t sf_cols, int layout)
{
    int64_t tiles_per_row_band;
    if (layout == ORC_LINEAR)
        return r * sf_cols + c;
    tiles_per_row_band = round_up(sf_cols, 4) / 4;
    return ((r / 128) * tiles_per_row_band + c / 4) * 512 + (r % 32) * 16 + ((r % 128) / 32) * 4
           + (c % 4);
}

/* ----------------------------------------------------------------------- */
/* Whole tensors.                                                            */
/* ----------------------------------------------------------------------- */

int orc_quantize(int fmt, int layout, const uint16_t *src, int64_t rows, int64_t cols, int64_t ld,
                 float g, uint8_t *payload, uint8_t *scales)
{
    int64_t bs = fmt == ORC_MXFP8 ? 32 : 16;
    int64_t C = orc_sf_cols(cols, fmt), r, c;
    int64_t payload_row = fmt == ORC_MXFP8 ? cols : cols / 2;
    if ((fmt != ORC_MXFP8 && fmt != ORC_NVFP4) || (layout != ORC_LINEAR && layout != ORC_SWIZZLED))
        return -1;
    if (rows < 0 || cols <= 0 || cols % bs != 0 || ld < cols)
        return -1;
    if (fmt == ORC_NVFP4 && !(g > 0.0f && g <= FLT_MAX))
        return -1; /* the encode scale is a positive finite number */
    memset(scales, 0, (size_t)orc_sf_bytes(rows, C, layout)); /* padding is zero */
    for (r = 0; r < rows; ++r) {
        for (c = 0; c < C; ++c) {
            const uint16_t *x = src + r * ld + c * bs;
            uint8_t sc;
            if (fmt == ORC_MXFP8)
                orc_mxfp8_block(x, 32, payload + r * payload_row + c * 32, &sc);
            else
                orc_nvfp4_block(x, 16, g, payload + r * payload_row + c * 8, &sc);
            scales[orc_sf_offset(r, c, C, layout)] = sc;
        }
    }
    return 0;
}

/* Split [TE-3800, Description; Changes; Summary diagram]: the concatenated
 * activation is quantized once and its payload, row amax and scales are
 * partitioned per expert; each expert's scales are padded on their own
 * (an expert with no rows owns no scale storage).  Expert i owns global rows
 * [o_i, o_i + m_i) of the payload, and its scales start at the sum of the
 * scale-region sizes of experts 0..i-1.  row_amax[r] = max_j |x[r, j]|. */
int64_t orc_split_scale_offset(const int64_t *split_rows, int n, int i, int64_t cols, int fmt,
                               int layout)
{
    int64_t off = 0, C = orc_sf_cols(cols, fmt);
    int j;
    for (j = 0; j < i && j < n; ++j)
        off += orc_sf_bytes(split_rows[j], C, layout);
    return off;
}

/* NVFP4 encode scale from an amax a, for a whole tensor [MO-2750, review: a
 * per-expert second-level scale, one for the fused gate/up pair since they
 * share one amax] or for one row of a row-scaled activation [TE-3800,
 * Description: the second-level scale is per row, from the row amax].  The
 * pages print no formula; the convention that maps the amax onto the largest
 * E4M3 block scale (448) times the largest E2M1 element (6) gives
 * g = fp32(2688 / a), a correctly rounded fp32 division.  An all-zero input
 * takes g = 1 (any value quantizes it to zeros).
 *
 * Range.  Every block multiplier is g / s_q with s_q an E4M3 value in
 * [2^-9, 448].  From above, g is capped at FLT_MAX * 2^-9, the largest g for
 * which g / 2^-9 is finite; only a < 2688 * 2^9 / FLT_MAX (about 2^-107.6)
 * reaches the cap, and for a < 2688 / FLT_MAX the quotient itself overflows.
 * No lower bound is needed: a <= FLT_MAX gives g >= 2688 / FLT_MAX (about
 * 2^-116.6), so g / 448 stays above the smallest normal fp32 number. */
float orc_nvfp4_encode_scale(float amax)
{
    const float g_max = FLT_MAX / 512.0f; /* exact: FLT_MAX * 2^-9 */
    float g;
    assert(amax >= 0.0f && isfinite(amax));
    if (amax == 0.0f)
        return 1.0f;
    g = 2688.0f / amax; /* fp32 division, correctly rounded (may overflow to inf) */
    if (g > g_max)
        g = g_max;
    return g;
}

float orc_tensor_amax(const uint16_t *src, int64_t rows, int64_t cols, int64_t ld)
{
    double amax = 0.0;
    int64_t r, j;
    for (r = 0; r < rows; ++r)
        for (j = 0; j < cols; ++j) {
            double v = fabs(orc_bf16_value(src[r * ld + j]));
            assert(isfinite(v));
            if (v > amax)
                amax = v;
        }
    return (float)amax; /* exact: a bf16 value */
}

static float row_amax_of(const uint16_t *x, int64_t cols)
{
    double amax = 0.0;
    int64_t j;
    for (j = 0; j < cols; ++j) {
        double v = fabs(orc_bf16_value(x[j]));
        assert(isfinite(v));
        if (v > amax)
            amax = v;
    }
    return (float)amax; /* exact: a bf16 value */
}

int orc_split(int fmt, int row_scaled, const uint16_t *src, int64_t total_rows, int64_t cols,
              const int64_t *split_rows, int n, float g, int layout, uint8_t *payload,
              uint8_t *scales, float *row_amax)
{
    int64_t o = 0, sum = 0, bs = fmt == ORC_MXFP8 ? 32 : 16, r;
    int64_t payload_row = fmt == ORC_MXFP8 ? cols : cols / 2;
    int64_t C;
    int i;
    if ((fmt != ORC_MXFP8 && fmt != ORC_NVFP4) || (row_scaled && fmt != ORC_NVFP4))
        return -1;
    if (layout != ORC_LINEAR && layout != ORC_SWIZZLED)
        return -1;
    for (i = 0; i < n; ++i) {
        if (split_rows[i] < 0)
            return -1;
        sum += split_rows[i];
    }
    if (sum != total_rows || cols <= 0 || cols % bs != 0)
        return -1;
    if (fmt == ORC_NVFP4 && !row_scaled && !(g > 0.0f && g <= FLT_MAX))
        return -1; /* the encode scale is a positive finite number */
    C = orc_sf_cols(cols, fmt);
    for (i = 0; i < n; ++i) {
        int64_t m = split_rows[i];
        int64_t base = orc_split_scale_offset(split_rows, n, i, cols, fmt, layout);
        if (m > 0 && !row_scaled) {
            /* the expert's rows form one tensor with its own scale matrix */
            if (orc_quantize(fmt, layout, src + o * cols, m, cols, cols, g,
                             payload + o * payload_row, scales + base) != 0)
                return -1;
        } else if (m > 0) {
            /* each row under its own encode scale; local row index r - o */
            memset(scales + base, 0, (size_t)orc_sf_bytes(m, C, layout));
            for (r = 0; r < m; ++r) {
                const uint16_t *x = src + (o + r) * cols;
                float gr = orc_nvfp4_encode_scale(row_amax_of(x, cols));
                int64_t c;
                for (c = 0; c < C; ++c) {
                    uint8_t sc;
                    orc_nvfp4_block(x + c * 16, 16, gr, payload + (o + r) * payload_row + c * 8, &sc);
                    scales[base + orc_sf_offset(r, c, C, layout)] = sc;
                }
            }
        }
        o += m;
    }
    for (r = 0; r < total_rows; ++r)
        row_amax[r] = row_amax_of(src + r * cols, cols);
    return 0;
}

int orc_nvfp4_split(const uint16_t *src, int64_t total_rows, int64_t cols, const int64_t *split_rows,
                    int n, float g, int layout, uint8_t *payload, uint8_t *scales, float *row_amax)
{
    return orc_split(ORC_NVFP4, 0, src, total_rows, cols, split_rows, n, g, layout, payload,
                     scales, row_amax);
}

/* Residual add + RMSNorm [TRT-17452, fold commit; TRT-17453, AllReduce
 * epilogue commit]: the epilogue writes the bf16 residual sum and the bf16
 * norm, and the quantized form is the quantization of that bf16 norm.
 * r_j = bf16(x_j + res_j); n_j = bf16(r_j * gamma_j / sqrt(mean_j(r_j^2) + eps)),
 * with one rounding to bf16 at the end (double-precision intermediate). */
int orc_add_rmsnorm(const uint16_t *x, const uint16_t *res, const uint16_t *gamma, float eps,
                    int64_t T, int64_t H, uint16_t *residual_out, uint16_t *norm_out)
{
    int64_t t, j;
    if (T < 0 || H <= 0 || !(eps > 0.0f))
        return -1;
    for (t = 0; t < T; ++t) {
        double ss = 0.0, den;
        for (j = 0; j < H; ++j) {
            double r;
            uint16_t rb = orc_bf16_round(orc_bf16_value(x[t * H + j]) + orc_bf16_value(res[t * H + j]));
            residual_out[t * H + j] = rb;
            r = orc_bf16_value(rb);
            ss += r * r;
        }
        den = sqrt(ss / (double)H + (double)eps);
        for (j = 0; j < H; ++j) {
            double r = orc_bf16_value(residual_out[t * H + j]);
            norm_out[t * H + j] = orc_bf16_round(r * orc_bf16_value(gamma[j]) / den);
        }
    }
    return 0;
}

int orc_scale_swizzle(const uint8_t *linear, int64_t rows, int64_t sf_cols, uint8_t *swizzled)
{
    int64_t r, c;
    if (rows < 0 || sf_cols <= 0)
        return -1;
    memset(swizzled, 0, (size_t)orc_sf_bytes(rows, sf_cols, ORC_SWIZZLED));
    for (r = 0; r < rows; ++r)
        for (c = 0; c < sf_cols; ++c)
            swizzled[orc_sf_offset(r, c, sf_cols, ORC_SWIZZLED)] = linear[r * sf_cols + c];
    return 0;
}

/* ----------------------------------------------------------------------- */
/* Elementwise forms of the scalar rules, for exhaustive checks.            */
/* ----------------------------------------------------------------------- */

void orc_e4m3_encode_f32(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode((double)v[i]);
}

void orc_e2m1_encode_f32(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e2m1_encode((double)v[i]);
}

void orc_mxfp8_scale_code_bf16(const uint16_t *amax_bits, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_mxfp8_scale_code(fabs(orc_bf16_value(amax_bits[i])));
}

void orc_mxfp8_elements(const uint16_t *x, int64_t n, uint8_t code, uint8_t *out)
{
    double m = orc_mxfp8_multiplier(code);
    int64_t i;
    for (i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(orc_bf16_value(x[i]) * m);
}
