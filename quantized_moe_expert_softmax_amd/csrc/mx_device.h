// mx_device.h -- device-side MX (OCP microscaling) and BF16 conversions.
//
// All conversions work on IEEE bit patterns with integer arithmetic, so the
// results do not depend on the floating-point mode of the kernel.  They
// implement the 1x32-block rule the pages quantise with ("quantize BF16
// activations to MXFP4 with per-1x32 E8M0 scales", FlyDSL #972 Technical
// Details): block exponent X = floor(log2(amax)) - emax of the element type,
// clamped to [-127, 127]; each element rounded to nearest even on the
// element grid and saturated; the sign of zero kept.
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
  uint32_t e = a >> 23;
  if (e) return (int)e - 127;
  return (31 - __builtin_clz(a & 0x7fffffu)) - 149;
}

// Shared block exponent from the largest |v| (fp32 bits, sign cleared).
template <class F>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  if (amax_bits == 0) return -127;
  int X = ilog2_bits(amax_bits) - F::kEmax;
  return X < -127 ? -127 : (X > 127 ? 127 : X);
}

// Code of v * 2^-X (v as fp32 bits, finite) in element type F.
template <class F>
__device__ __forceinline__ uint32_t encode_element(uint32_t v, int X) {
  const uint32_t sign = (v >> 31) << (F::kBits - 1);
  const uint32_t a = v & 0x7fffffffu;
  if (a == 0) return sign;
  // |v| = M * 2^E with M a 24-bit integer significand
  uint32_t e = a >> 23;
  uint32_t M = a & 0x7fffffu;
  int E;
  if (e) { M |= 0x800000u; E = (int)e - 150; } else { E = -149; }
  const int lg = (31 - __builtin_clz(M)) + E - X;  // floor(log2(|v| * 2^-X))
  const int ex = lg < F::kEmin ? F::kEmin : lg;    // binade (subnormals share emin's spacing)
  const int sh = (ex - F::kMbits) - (E - X);       // right shift giving multiples of the ulp
  uint32_t r;
  if (sh <= 0) {
    r = M << (-sh);  // exact; r < 2^(kMbits+1) so no overflow
  } else if (sh >= 25) {
    r = 0;           // below half an ulp
  } else {
    r = M >> sh;
    const uint32_t rem = M & ((1u << sh) - 1u);
    const uint32_t half = 1u << (sh - 1);
    if (rem > half || (rem == half && (r & 1u))) r += 1u;
  }
  // In the binade of exponent ex the code is (ex - emin) * 2^mbits + r; a
  // rounding carry (r == 2^(mbits+1)) lands on the next binade's first code.
  uint32_t code = ((uint32_t)(ex - F::kEmin) << F::kMbits) + r;
  if (code > F::kMaxCode) code = F::kMaxCode;
  return sign | code;
}

__device__ __forceinline__ uint32_t f32_bits(float f) { return __float_as_uint(f); }

// Round a finite fp32 to bf16, nearest even.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace moe
