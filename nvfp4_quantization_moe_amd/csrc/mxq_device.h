// mxq_device.h -- device-side building blocks for gfx950 (CDNA4, wave64):
// bf16 unpacking, block-amax reductions across lanes with DPP, and the
// MXFP8 / NVFP4 scale and element encoders.
//
// The encoders implement, in fp32/integer arithmetic, the exact rules of the
// formats (OCP OFP8 E4M3 with largest finite 448; OCP MX E8M0 and E2M1; the
// NVFP4 16-element block with an E4M3 scale under an fp32 encode scale):
// round to nearest even, sign of zero kept, saturation where a value can
// exceed the format.  See include/mxq.h for the block rules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
// Encode fp32 y with |y| <= 448 (or any y when kSaturate): round to nearest
// even on the E4M3 grid, subnormals below 2^-6 on a 2^-9 grid, sign kept.
template <bool kSaturate>
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    uint32_t u = __float_as_uint(y);
    uint32_t s = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (kSaturate) a = min(a, 0x43E00000u);  // 448; also catches +inf
    // normal range: keep 3 mantissa bits, RNE at bit 20, rebias 127 -> 7
    uint32_t rn = a + 0x7FFFFu + ((a >> 20) & 1u);
    uint32_t cn = (rn >> 20) - (120u << 3);
    // below 2^-6: adding 2^14 (ulp 2^-9) rounds |y| to the subnormal grid
    uint32_t cs = __float_as_uint(__uint_as_float(a) + 16384.0f) - 0x46800000u;
    return (a < 0x3C800000u ? cs : cn) | s;
}

// Decode a non-negative, non-NaN E4M3 code.
__device__ __forceinline__ float e4m3_decode_pos(uint32_t k) {
    uint32_t e = k >> 3, m = k & 7u;
    return e == 0 ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---- E2M1 --------------------------------------------------------------------
// Encode fp32 y: nearest of {0,.5,1,1.5,2,3,4,6}, ties to the even code,
// saturating at 6, sign in bit 3.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    uint32_t u = __float_as_uint(y);
    uint32_t s = (u >> 28) & 0x8u;
    uint32_t a = u & 0x7FFFFFFFu;
    uint32_t rn = a + 0x1FFFFFu + ((a >> 22) & 1u);         // keep 1 mantissa bit
    uint32_t cn = min((rn >> 22) - ((127u - 1u) << 1), 7u);  // rebias 127 -> 1
    uint32_t cs = __float_as_uint(__uint_as_float(a) + 4194304.0f) - 0x4A800000u;  // 0.5 grid
    return (a < 0x3F800000u ? cs : cn) | s;
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

// Element multiplier 2^(127-c); code 0 (scale 2^-127, not a normal fp32)
// flushes the reciprocal to zero.  Codes above 253 cannot occur for bf16.
__device__ __forceinline__ float mx_multiplier(uint32_t c) {
    return c == 0 ? 0.0f : __uint_as_float((254u - c) << 23);
}

// Quantize 8 bf16 values (one lane's share of a 32-element block) with the
// multiplier m; returns 8 E4M3 bytes.  x*m is exact (power of two) except
// below 2^-126, where the code is a signed zero either way.
__device__ __forceinline__ u32x2 mx_encode8(u32x4 v, float m) {
    u32x2 out;
    uint32_t b[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        b[2 * j] = e4m3_encode<false>(bf16_lo(v[j]) * m);
        b[2 * j + 1] = e4m3_encode<false>(bf16_hi(v[j]) * m);
    }
    out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    return out;
}

// ---- NVFP4 block rule --------------------------------------------------------
struct Nv4Scale {
    uint32_t code;  // E4M3 block scale byte
    float mult;     // element multiplier fp32(g / s_q), 0 when flushed
};

// s = fp32(fp32(amax / 6) * g); code = E4M3(s) saturating; multiplier
// fp32(g / decode(code)), zero when the decoded scale is zero or the
// multiplier is not a normal fp32 number.  Divisions are IEEE (the build
// keeps fp32 division correctly rounded and denormals enabled).
__device__ __forceinline__ Nv4Scale nv_scale(uint32_t amax_bits, float g) {
    float a = __uint_as_float(amax_bits << 16);
    float t = a / 6.0f;
    float s = t * g;
    Nv4Scale r;
    r.code = e4m3_encode<true>(s);
    float sq = e4m3_decode_pos(r.code);
    float m = g / sq;
    r.mult = (sq == 0.0f || !(m >= 0x1p-126f)) ? 0.0f : m;
    return r;
}

// Quantize 8 bf16 values with multiplier m; returns 4 bytes of packed E2M1
// (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t nv_encode8(u32x4 v, float m) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        uint32_t lo = e2m1_encode(bf16_lo(v[j]) * m);
        uint32_t hi = e2m1_encode(bf16_hi(v[j]) * m);
        out |= (lo | (hi << 4)) << (8 * j);
    }
    return out;
}

// ---- swizzled 128x4 scale layout ----------------------------------------------
// Work units are 32 rows.  With the swizzled layout a unit takes the rows
// band*128 + 32*q + 8*g + i (q = wave 0..3, i = 0..7) of one 128-row band, so
// in every 512-byte tile it fills exactly one 128-byte line (line g).  The
// unit stages those lines in LDS: tile t's line at stage[t*128 + i*16 + q*4 + c%4].
__device__ __forceinline__ int stage_index_swz(int q, int i, int c) {
    return (c >> 2) * 128 + i * 16 + q * 4 + (c & 3);
}

}  // namespace mxq
