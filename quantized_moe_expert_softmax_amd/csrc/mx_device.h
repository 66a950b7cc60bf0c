// mx_device.h -- device-side MX (OCP microscaling) and BF16 conversions.
//
// They implement the 1x32-block rule with which the pages turn BF16
// activations into MX codes, one E8M0 scale per 32 elements (FlyDSL #972
// Technical Details): block exponent X = floor(log2(amax)) - emax of the
// element type, clamped to [-127, 127]; each element v / 2^X rounded to
// nearest even on the element grid and saturated; the sign of zero kept.  The
// element rounding is gfx950's scaled conversion instructions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Element type parameters: explicit mantissa bits, exponent of the smallest
// normal, emax, largest finite magnitude code, code width.
struct E4M3 {  // OCP E4M3FN (max 448 = 0x7E; 0x7F is NaN and never produced)
  static constexpr int kMbits = 3, kEmin = -6, kEmax = 8, kBits = 8;
  static constexpr uint32_t kMaxCode = 0x7E;
};
struct E2M1 {  // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
  static constexpr int kMbits = 1, kEmin = 0, kEmax = 2, kBits = 4;
  static constexpr uint32_t kMaxCode = 0x7;
};

// floor(log2(|v|)) of a finite, non-zero |v| given as fp32 bits.
__device__ __forceinline__ int ilog2_bits(uint32_t a) {
  const int e = (int)(a >> 23);
  return e ? e - 127 : (31 - __builtin_clz(a & 0x7fffffu)) - 149;
}

// Shared block exponent from the largest |v| (fp32 bits, sign cleared).
template <class F>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  const int X = ilog2_bits(amax_bits | 1u) - F::kEmax;  // (| 1: no clz of 0; amax 0 is handled below)
  return amax_bits == 0 ? -127 : (X < -127 ? -127 : (X > 127 ? 127 : X));
}

// The codes of two values a, b of one 1x32 block with block exponent X, by
// gfx950's scaled conversions (a / 2^X and b / 2^X rounded to nearest even
// on the element grid, subnormal codes included, the sign of zero kept).
// E4M3 values are first clamped to the largest magnitude times 2^X, since
// the rule saturates where the instruction would give NaN; E2M1's conversion
// saturates by itself.  On an MI355X these codes equalled those of a
// branch-free FP32 implementation of the rule (exact power-of-two scaling,
// then nearest-even rounding by adding and subtracting a power of two) on
// every code value, every midpoint and its neighbours, and 200 000 random
// values, for every block exponent from -127 to 119 (every finite block:
// X = floor(log2(amax)) - emax), both formats and both halves of a pair;
// the quantiser built on them matches the oracle on every finite BF16
// pattern.
template <class F>
__device__ __forceinline__ void encode_pair(float a, float b, int X, uint32_t &ca, uint32_t &cb) {
  const float sc = ldexpf(1.0f, X);
  if (F::kBits == 4) {
    const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, sc, 0);
    ca = r & 0xFu;
    cb = (r >> 4) & 0xFu;
  } else {
    typedef short short2v __attribute__((ext_vector_type(2)));
    const float mx = ldexpf(448.0f, X);
    const short2v r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(
        (short2v){0, 0}, __builtin_amdgcn_fmed3f(a, -mx, mx), __builtin_amdgcn_fmed3f(b, -mx, mx),
        sc, false);
    const uint32_t w = (uint32_t)(uint16_t)r[0];
    ca = w & 0xFFu;
    cb = w >> 8;
  }
}

__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }

// Round a finite fp32 to bf16, nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace moe
