// varq_quant_math.h - the scalar arithmetic of VAR-Q's quantizer and dequantizer,
// shared by the gfx950 kernels and by the host-side exhaustive self-test.
//
// Quantizer (project page summary and "Next-block prediction": one scale per
// feature channel within each generation block; symmetric, no zero point):
//   s = fp32(absmax / qmax),  q = rint(fp32(x / s)) with ties to even, q = 0 if s = 0.
// Dequantizer (project page "Quantization, bit packing, and retrieval":
// values are dequantized to BF16 before attention): bf16_rne(fp32(q) * s).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace varq {

// Below this scale the division-free quotient below may differ from IEEE
// division (it can only fail when the residual underflows; an exhaustive host
// check over all bf16 (x, absmax) pairs finds failures only for absmax < 6e-36).
// Channels with such tiny scales take the IEEE division instead.
constexpr float kFastScaleMin = 0x1p-100f;

// 1.5 * 2^23: adding it to |v| < 2^22 rounds v to an integer with ties to even
// and leaves that integer, offset by 2^22, in the low mantissa bits.
constexpr float kRoundMagic = 12582912.0f;
constexpr uint32_t kRoundMagicBits = 0x4B400000u;

__host__ __device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Correctly rounded reciprocal used by the division-free quotient; 0 when s = 0
// (every element of such a group is 0, and the code formula then yields 0).
__host__ __device__ inline float recip_for_codes(float s) { return s == 0.0f ? 0.0f : 1.0f / s; }

// True when code_fast() is exact for this scale.
__host__ __device__ inline bool fast_scale_ok(float s) { return s == 0.0f || s >= kFastScaleMin; }

// rint(fl32(x / s)) as a two's complement integer, for |x| <= qmax * s.
// r = x*y is within an ulp of x/s; the residual e = x - r*s is exact under a
// fused multiply-add, and r + e*y rounds to the correctly rounded quotient
// (Markstein's correction step with a correctly rounded reciprocal y).
// The _bits forms return the rounded float's bit pattern, whose low 22 bits
// hold the code in two's complement (the magic constant has none there):
// packing, which keeps only a code's low BITS bits, needs no more.
__host__ __device__ inline uint32_t code_fast_bits(float x, float s, float y) {
    float r = x * y;
    float e = __builtin_fmaf(-r, s, x);
    float qf = __builtin_fmaf(e, y, r);
    return f2u(qf + kRoundMagic);
}
__host__ __device__ inline int32_t code_fast(float x, float s, float y) {
    return (int32_t)(code_fast_bits(x, s, y) - kRoundMagicBits);
}

// The same code by IEEE division (used for scales below kFastScaleMin).
__host__ __device__ inline uint32_t code_exact_bits(float x, float s) {
    if (s == 0.0f) return kRoundMagicBits;
    return f2u(x / s + kRoundMagic);
}
__host__ __device__ inline int32_t code_exact(float x, float s) {
    return (int32_t)(code_exact_bits(x, s) - kRoundMagicBits);
}

// bf16 bit pattern of the fp32 value v, round to nearest even (finite v).
__host__ __device__ inline uint32_t bf16_bits_rne(float v) {
    uint32_t u = f2u(v);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Dequantized bf16 bit pattern of code q with scale s.
__host__ __device__ inline uint32_t dequant_bits(int32_t q, float s) {
    return bf16_bits_rne((float)q * s);
}

}  // namespace varq
