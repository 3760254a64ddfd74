// mxq_device.h -- device-side building blocks for gfx950 (CDNA4, wave64):
// bf16 unpacking, block-amax reductions across lanes with DPP, and the
// MXFP8 / NVFP4 scale and element encoders.
//
// The encoders implement the exact rules of the formats (OCP OFP8 E4M3 with
// largest finite 448; OCP MX E8M0 and E2M1; the NVFP4 16-element block with an
// E4M3 scale under an fp32 encode scale): round to nearest even, sign of zero
// kept, saturation where a value can exceed the format.  Element rounding uses
// gfx950's scaled conversion instructions in the forms shown (by exhaustive
// comparison with the rules) to reproduce them bit for bit.  See
// include/mxq.h for the block rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mxq.h"

namespace mxq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---- bf16 ------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---- block amax --------------------------------------------------------------
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    u16x2 x = __builtin_bit_cast(u16x2, a);
    u16x2 y = __builtin_bit_cast(u16x2, b);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(x, y));
}

// Largest |x| over the 8 bf16 values in v, as 15-bit magnitude bits.  For
// finite bf16 the magnitude order equals the unsigned order of bits & 0x7FFF.
__device__ __forceinline__ uint32_t amax_bits8(u32x4 v) {
    uint32_t m = pk_max_u16(pk_max_u16(v.x & 0x7FFF7FFFu, v.y & 0x7FFF7FFFu),
                            pk_max_u16(v.z & 0x7FFF7FFFu, v.w & 0x7FFF7FFFu));
    return max(m & 0xFFFFu, m >> 16);
}

// DPP quad_perm lane exchanges inside groups of four lanes.
template <int kQuadPerm>
__device__ __forceinline__ uint32_t dpp_quad(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kQuadPerm, 0xF, 0xF, false);
}
constexpr int kQuadXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // [2,3,0,1]

// Max across the lanes that share one block: 4 lanes (32 elements, MXFP8) or
// 2 lanes (16 elements, NVFP4).  Every lane of the group gets the result.
__device__ __forceinline__ uint32_t block_max4(uint32_t v) {
    v = max(v, dpp_quad<kQuadXor1>(v));
    return max(v, dpp_quad<kQuadXor2>(v));
}
__device__ __forceinline__ uint32_t block_max2(uint32_t v) { return max(v, dpp_quad<kQuadXor1>(v)); }

// Max across the whole wave (row amax); all lanes get the result.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    for (int o = 1; o < kWave; o <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 1; o < kWave; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

// ---- E4M3 --------------------------------------------------------------------
// Decode a non-negative, non-NaN E4M3 code.
__device__ __forceinline__ float e4m3_decode_pos(uint32_t k) {
    uint32_t e = k >> 3, m = k & 7u;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---- MXFP8 block rule --------------------------------------------------------
// Scale code: the smallest c with amax <= 448 * 2^(c-127).  On the bf16
// fields (exponent E, mantissa M) that is E - 8, plus one when M > 0x60
// (amax above 1.75 * 2^(E-127)); zero and subnormal amax give 0.
__device__ __forceinline__ uint32_t mx_scale_code(uint32_t amax_bits) {
    int E = (int)(amax_bits >> 7);
    int c = E - 8 + ((amax_bits & 0x7Fu) > 0x60u ? 1 : 0);
    return E == 0 ? 0u : (uint32_t)max(c, 0);
}

typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Quantize 8 bf16 values (one lane's share of a 32-element block) under
// scale code c; returns 8 E4M3 bytes, element k in byte k.
//
// gfx950's v_cvt_scalef32_pk_fp8_bf16 takes the scale as an fp32 whose
// exponent field e divides the input by 2^(e-127) before rounding to E4M3
// (nearest even, sign kept), so e = c gives x * 2^(127-c) exactly.  Its result
// equals the E4M3 rule for every bf16 input and every code with
// |x| * 2^(127-c) <= 448, i.e. every input a block with code c can hold (the
// GPU parity tests enumerate all of them).  Code 0 stands for a scale of
// 2^-127, whose reciprocal is flushed to zero: there every element must
// encode as a signed zero, which e = 254 (divide by 2^127) yields because
// such blocks hold only magnitudes <= 448 * 2^-127.
__device__ __forceinline__ u32x2 mx_encode8(u32x4 v, uint32_t c) {
    const float sc = __uint_as_float((c == 0 ? 254u : c) << 23);
    // The pairs are built from one whole-vector cast: this compiler folds a
    // bit_cast of each ext-vector element (v.y, v.z, ...) to element 0.
    const v8bf e = __builtin_bit_cast(v8bf, v);
    v2s lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, v2bf{e[0], e[1]}, sc, false);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(lo, v2bf{e[2], e[3]}, sc, true);
    v2s hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(v2s{0, 0}, v2bf{e[4], e[5]}, sc, false);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(hi, v2bf{e[6], e[7]}, sc, true);
    return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// ---- NVFP4 block rule --------------------------------------------------------
struct Nv4Scale {
    uint32_t code;  // E4M3 block scale byte
    float mult;     // element multiplier fp32(g / s_q), 0 when flushed
};

// fp32(a / 6), correctly rounded, for a non-negative bf16 value a: one
// product with fp32(1/6) and one fused correction step.  Checked exactly
// against the rounded quotient for every finite non-negative bf16 value.
__device__ __forceinline__ float div6(float a) {
    const float r6 = 0.16666667163372040f;  // fp32(1/6)
    const float q = a * r6;
    const float r = __builtin_fmaf(-q, 6.0f, a);
    return __builtin_fmaf(r, r6, q);
}

// Element multiplier m = fp32(g / s_q), flushed to 0 when it is not a
// normal fp32 number (subnormal, or infinite after overflow), for any
// positive finite encode scale g.
//
// Quotient table (g >= 2^-117, every scale the library derives from an amax
// and nearly every caller's): every positive E4M3 value is s_q = d * 2^-k
// with d in 1..15 (d = 8 + mantissa for exponent field e >= 1, k = 10 - e;
// d = mantissa, k = 9 for subnormals), and rounding commutes with scaling by
// 2^k while the values stay normal, so fp32(g / s_q) = fp32(g / d) * 2^k.
// For g >= 2^-117, g / 15 and g / 448 are normal, so that holds for every
// code, and no multiplier is subnormal; a quotient that overflows does so in
// both forms at the same threshold (round to 24 bits, then compare with
// 2^128), so the ldexp gives inf exactly when the division does.  Each wave
// computes the quotients once, lane d of every 16 holding fp32(g / d) (IEEE
// division) and lane 0 holding 0 for code 0; a block fetches its quotient
// with a cross-lane read, so every lane of the wave must take part.
//
// Below 2^-117 (a caller's scale; subnormal g included) the products can
// leave the normal range, where that identity fails: each block then divides
// (IEEE) and flushes a subnormal result.  g is uniform over the wave in
// every kernel, so the two paths are a uniform branch.
struct NvG {
    float g;
    float quot;  // table path: lane d of each 16 holds fp32(g / d), lane 0 holds 0
    bool table;  // g >= 2^-117
};

__device__ __forceinline__ NvG nv_prepare(float g) {
    const int d = threadIdx.x & 15;
    NvG r;
    r.g = g;
    r.table = g >= 0x1p-117f;
    r.quot = d == 0 ? 0.0f : g / (float)d;
    return r;
}

// s = fp32(fp32(amax / 6) * g); code = E4M3(s), saturating at 448; multiplier
// as above (0 for code 0, where s_q = 0).  All lanes of the wave must be
// active.
__device__ __forceinline__ Nv4Scale nv_scale(uint32_t amax_bits, const NvG &G) {
    const float s = div6(__uint_as_float(amax_bits << 16)) * G.g;
    Nv4Scale r;
    // v_cvt_scalef32_pk_fp8_f32 (scale 1.0) rounds to nearest even and keeps
    // values up to 448 exact to the rule; larger values are clamped first.
    const v2s k = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, __builtin_fminf(s, 448.0f),
                                                           0.0f, 1.0f, false);
    r.code = __builtin_bit_cast(uint32_t, k) & 0xFFu;
    float m;
    if (G.table) {
        const uint32_t e = r.code >> 3, mant = r.code & 7u;
        const int d = e == 0 ? (int)mant : (int)(8 + mant);
        const int sh = e == 0 ? 9 : 10 - (int)e;
        m = __builtin_ldexpf(__shfl(G.quot, d, 16), sh);
    } else {
        m = G.g / e4m3_decode_pos(r.code);  // code 0: g / 0 = inf, flushed below
        m = m >= 0x1p-126f ? m : 0.0f;
    }
    r.mult = m <= 0x1.fffffep+127f ? m : 0.0f;
    return r;
}

// NVFP4 encode scale from an amax a (a tensor's, a scale slot's or a row's):
// 1 when a = 0, else fp32(2688 / a) (IEEE division; 2688 = 448 * 6 maps the
// amax onto the largest block scale times the largest element), capped at
// FLT_MAX * 2^-9, the largest g for which g / 2^-9, the largest multiplier,
// is finite.  No lower bound is needed: any finite a gives g >= 2688 /
// FLT_MAX (about 2^-116.6), inside the quotient-table range.
__device__ __forceinline__ float nv_encode_scale(float a) {
    if (a == 0.0f) return 1.0f;
    return __builtin_fminf(2688.0f / a, 0x1.fffffep+118f);
}

// Quantize 8 bf16 values with multiplier m; returns 4 bytes of packed E2M1
// (element 2j in the low nibble of byte j).  fp32(x * m) is formed first;
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 then rounds each fp32 to E2M1
// exactly as the rule does (nearest, ties to the even code, saturation at 6,
// sign kept), first operand in the low nibble.
__device__ __forceinline__ uint32_t nv_encode8(u32x4 v, float m) {
    uint32_t out = 0;
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, bf16_lo(v.x) * m, bf16_hi(v.x) * m, 1.0f, 0);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, bf16_lo(v.y) * m, bf16_hi(v.y) * m, 1.0f, 1);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, bf16_lo(v.z) * m, bf16_hi(v.z) * m, 1.0f, 2);
    out = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(out, bf16_lo(v.w) * m, bf16_hi(v.w) * m, 1.0f, 3);
    return out;
}

// ---- shared per-lane quantization step ----------------------------------------
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
// and NVFP4 fetches its multiplier quotient across the wave (NvG), so every
// lane of the wave must call it (lanes past the tensor pass zeros
// and discard the result).  Returns the block's scale byte (every lane of the
// block holds it) and the lane's payload: 8 bytes (MXFP8) or 4 bytes in pay.x
// (NVFP4).
template <int FMT>
__device__ __forceinline__ uint32_t quant8(u32x4 v, const NvG &G, u32x2 &pay) {
    uint32_t a = amax_bits8(v);
    if constexpr (FMT == MXQ_MXFP8) {
        a = block_max4(a);
        const uint32_t c = mx_scale_code(a);
        pay = mx_encode8(v, c);
        return c;
    } else {
        a = block_max2(a);
        const Nv4Scale s = nv_scale(a, G);
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

}  // namespace mxq
