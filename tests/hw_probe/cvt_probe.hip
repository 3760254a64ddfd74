// cvt_probe.hip -- test-only probe of the two gfx950 conversions the NVFP4
// path relies on, over every non-negative fp32 bit pattern (zero, every
// subnormal, every normal, +inf).  Not part of the library: the parity tests
// compare what it records with the oracle's encoders.
//
//   E2M1: v_cvt_scalef32_pk_fp4_f32 with scale 1.0 (the element step: each
//         fp32 product x * m is rounded to E2M1); both operand slots.
//   E4M3: v_cvt_scalef32_pk_fp8_f32 with scale 1.0 on min(s, 448) (the block
//         scale step).
//
// Rounding to a format is a non-decreasing step function of a non-negative
// input, and the bit patterns of non-negative fp32 values are in value order,
// so the conversion is fully described by the patterns at which its code
// changes.  Each kernel records every pattern p whose code differs from the
// code of p - 1, and counts the patterns where the negative input does not
// give the same code with the sign bit set.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef short v2s __attribute__((ext_vector_type(2)));

constexpr uint32_t kLast = 0x7F800000u;  // +inf: patterns 0 .. kLast

__device__ __forceinline__ uint32_t fp4_lo(float y) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, 0.0f, 1.0f, 0) & 0xFu;
}
__device__ __forceinline__ uint32_t fp4_hi(float y) {
    return (__builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, 0.0f, y, 1.0f, 0) >> 4) & 0xFu;
}
__device__ __forceinline__ uint32_t fp8_code(float s) {
    const v2s k = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2s{0, 0}, __builtin_fminf(s, 448.0f),
                                                           0.0f, 1.0f, false);
    return __builtin_bit_cast(uint32_t, k) & 0xFFu;
}

// out[0]: steps found; out[1]: sign mismatches; out[2]: operand-slot
// mismatches; out[4 + 2k], out[5 + 2k]: pattern and (code | previous << 8) of
// step k, for k < cap.
__device__ __forceinline__ void record(uint32_t *out, int cap, uint32_t p, uint32_t c,
                                       uint32_t prev) {
    const uint32_t k = atomicAdd(&out[0], 1u);
    if (k < (uint32_t)cap) {
        out[4 + 2 * k] = p;
        out[5 + 2 * k] = c | (prev << 8);
    }
}

template <bool FP4>
__global__ __launch_bounds__(256) void k_steps(uint32_t *out, int cap) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i <= kLast; i += stride) {
        const uint32_t p = (uint32_t)i;
        const float y = __uint_as_float(p);
        uint32_t c, cn, prev;
        if constexpr (FP4) {
            c = fp4_lo(y);
            cn = fp4_lo(-y);
            if (fp4_hi(y) != c || fp4_hi(-y) != cn) atomicAdd(&out[2], 1u);
            prev = p == 0 ? c : fp4_lo(__uint_as_float(p - 1));
            if (cn != (c | 0x8u)) atomicAdd(&out[1], 1u);
        } else {
            c = fp8_code(y);
            prev = p == 0 ? c : fp8_code(__uint_as_float(p - 1));
        }
        if (c != prev) record(out, cap, p, c, prev);
    }
}

}  // namespace

extern "C" {

// out: device uint32 [4 + 2 * cap], zeroed by the caller.  Returns 0 or the
// launch error.
int probe_fp4_steps(uint32_t *out, int cap, void *stream) {
    hipLaunchKernelGGL((k_steps<true>), dim3(8192), dim3(256), 0, (hipStream_t)stream, out, cap);
    return (int)hipGetLastError();
}

int probe_fp8_steps(uint32_t *out, int cap, void *stream) {
    hipLaunchKernelGGL((k_steps<false>), dim3(8192), dim3(256), 0, (hipStream_t)stream, out, cap);
    return (int)hipGetLastError();
}

}  // extern "C"
