// mx_device.h -- device-side MX (OCP microscaling) and BF16 conversions.
//
// Conversions take IEEE bit patterns; element rounding uses exact fp32 adds
// under the default round-to-nearest-even mode.  They implement the 1x32-block
// rule with which the pages turn BF16 activations into MX codes, one E8M0 scale
// per 32 elements (FlyDSL #972 Technical Details):
// block exponent X = floor(log2(amax)) - emax of the element type,
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

// 2^k as an fp32 for -126 <= k <= 127.
__device__ __forceinline__ float exp2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

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

// Code of v * 2^-X (v as fp32 bits, finite, |v| <= 2^(X + emax + 1)) in
// element type F, without branches.
//   y = |v| * 2^-X is exact whenever it is an fp32 normal (a power-of-two
//   scaling; X <= 127 - emax keeps 2^-X a normal); a y below 2^-126 lies far
//   under half the smallest element step and gives code 0 however it rounds.
//   The grid step at y is u = 2^(max(floor(log2 y), emin) - mbits); adding and
//   subtracting c = 2^23 * u rounds y to a multiple of u, ties to even (c is
//   an even multiple of u, and y + c stays in c's binade).
//   The code of a grid point r >= 2^emin is its biased binade and top mbits
//   of fraction; below 2^emin it is r / 2^(emin - mbits); past the largest
//   finite element it saturates.
template <class F>
__device__ __forceinline__ uint32_t encode_element(uint32_t v, int X) {
  const uint32_t sign = (v >> 31) << (F::kBits - 1);
  const float y = __uint_as_float(v & 0x7fffffffu) * exp2i(-X);
  const int ey = (int)(__float_as_uint(y) >> 23) - 127;
  const int eb = ey > F::kEmin ? ey : F::kEmin;
  const float c = exp2i(eb + 23 - F::kMbits);
  const float t = y + c;
  const float r = t - c;
  const uint32_t rb = __float_as_uint(r);
  const int er = (int)(rb >> 23) - 127;
  const uint32_t normal = ((uint32_t)(er - F::kEmin + 1) << F::kMbits) |
                          ((rb >> (23 - F::kMbits)) & ((1u << F::kMbits) - 1u));
  const uint32_t sub = (uint32_t)(r * exp2i(F::kMbits - F::kEmin));
  uint32_t code = er >= F::kEmin ? normal : sub;
  code = code < F::kMaxCode ? code : F::kMaxCode;
  return sign | code;
}

// The codes of two values a, b of one 1x32 block with block exponent X, by
// gfx950's scaled conversions (a / 2^X and b / 2^X rounded to nearest even
// in the element format): the same codes as encode_element for every finite
// value and every block exponent up to 119, which covers every finite block
// (X = floor(log2(amax)) - emax).  E4M3 values are first clamped to the
// largest magnitude times 2^X, since the rule saturates where the
// instruction would give NaN; E2M1's conversion saturates by itself.  One
// instruction per pair instead of the branch-free rounding sequence per
// element (checked against encode_element on every code, every midpoint and
// its neighbours, and 200 000 random values across the exponent range).
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
