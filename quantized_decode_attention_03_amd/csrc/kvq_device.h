// Device-side helpers shared by the kvq kernels (gfx950).
//
// The group arithmetic follows "KV Cache Quantization — 8-bit and 4-bit",
// section "Integer quantization in one screen": scale = (x_max - x_min) /
// (q_max - q_min), zero_point = q_min - round(x_min / scale), q = round(x /
// scale) + zero_point, x_hat = scale * (q - zero_point). Every step is an IEEE
// fp32 operation with round-to-nearest-even; the fp16 scale is rounded toward
// +inf so the reconstruction error stays within scale/2. Divisions are true
// divisions (the library is built with correctly rounded fp32 division).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_internal.h"

namespace kvq {

__device__ __forceinline__ float h2f(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ uint16_t f2h_rne(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
// Smallest fp16 >= f for finite f >= 0.
__device__ __forceinline__ uint16_t f2h_up(float f) {
  uint16_t b = f2h_rne(f);
  if (h2f(b) < f) b += 1;
  return b;
}

__host__ __device__ constexpr int qmin_of(int bits) { return -(1 << (bits - 1)); }
__host__ __device__ constexpr int qmax_of(int bits) { return (1 << (bits - 1)) - 1; }

struct GroupQ {
  float s;      // scale as fp32 (exactly the stored fp16)
  float r;      // its reciprocal, to within 1 ulp (for div_rint)
  float z;      // zero-point as fp32 (an integer in [-2048, 2048])
  uint32_t meta;  // fp16 scale bits | fp16 zero bits << 16
};

// rint(x / s) with x / s the correctly rounded fp32 quotient, given r =
// 1/s to within 1 ulp, for |x / s| < 2^12 (every caller: a group's codes lie
// within 2^11 + 2^8 steps of zero). y = x * r is within 2^-22 |x/s| < 2^-10 of
// that quotient, so when y is more than 2^-9 from the nearest half-integer both
// round to the same integer; otherwise the true division decides. That case
// is rare (about one element in 256), so the division sits behind a
// wave-uniform branch: the wavefront skips it unless one of its lanes needs it.
__device__ __forceinline__ float div_rint(float x, float s, float r) {
#pragma clang fp contract(off)
  const float y = x * r;
  float k = __builtin_rintf(y);
  const bool near_half = __builtin_fabsf(y - k) > 0.498046875f;  // 1/2 - 2^-9
  if (__builtin_amdgcn_ballot_w64(near_half)) {
    if (near_half) k = __builtin_rintf(x / s);
  }
  return k;
}

// Scale and zero-point of a group from its fp32 extremes.
__device__ __forceinline__ GroupQ group_params(float xmin, float xmax, int bits) {
#pragma clang fp contract(off)
  const float nlev = (float)(qmax_of(bits) - qmin_of(bits));
  uint16_t s16;
  if (xmax > xmin) {
    s16 = f2h_up((xmax - xmin) / nlev);
  } else {
    s16 = (xmin != 0.0f) ? f2h_rne(__builtin_fabsf(xmin)) : (uint16_t)0x3C00;
  }
  GroupQ g;
  g.s = h2f(s16);
  float r = __builtin_rintf(xmin / g.s);
  constexpr float kLim0 = 2048.0f;  // every integer up to 2048 is an exact fp16
  const float lim = kLim0 + (float)qmin_of(bits);
  if (__builtin_fabsf(r) > lim) {
    // a group far from zero compared with its spread: the zero point z, or
    // z - q_min in stored-code units, would not be an exact fp16 integer, so
    // the scale widens until |round(x_min / s)| <= 2048 + q_min (the codes
    // still span at most q_max - q_min steps, keeping the scale/2 bound)
    s16 = f2h_up(__builtin_fabsf(xmin) / lim);
    g.s = h2f(s16);
    r = __builtin_rintf(xmin / g.s);
  }
  const float z = (float)qmin_of(bits) - r;
  g.z = z;
  g.r = __builtin_amdgcn_rcpf(g.s);
  g.meta = (uint32_t)s16 | ((uint32_t)f2h_rne(z) << 16);
  return g;
}

// Stored unsigned code u = q - q_min of one element: rint(x / s) + (z - q_min)
// clamped to [0, q_max - q_min] (integers, exact in fp32).
__device__ __forceinline__ uint32_t quant_code(float x, const GroupQ& g, int bits) {
#pragma clang fp contract(off)
  const float u = div_rint(x, g.s, g.r) + (g.z - (float)qmin_of(bits));
  return (uint32_t)__builtin_amdgcn_fmed3f(u, 0.0f, (float)(qmax_of(bits) - qmin_of(bits)));
}

// Exact fp32 reconstruction s * (q - z) from a stored code and a meta word.
__device__ __forceinline__ float dequant(uint32_t u, uint32_t meta, int bits) {
#pragma clang fp contract(off)
  const float s = h2f((uint16_t)(meta & 0xFFFFu));
  const float z = h2f((uint16_t)(meta >> 16));
  return s * ((float)((int)u + qmin_of(bits)) - z);
}

// ---- fp8 E4M3 elements (OCP layout: sign bit 7, exponent bits 6..3 with
// bias 7, mantissa bits 2..0; exponent field 0 holds the subnormals m * 2^-9;
// S.1111.111 is NaN, so the largest finite magnitude is 448) ----------------

// Code of an fp32 value: the nearest E4M3 magnitude, ties to the even code,
// magnitudes at or above 448 saturated to 448, the sign kept (a negative value
// that rounds to zero gives 0x80). Finite inputs.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t ab = bits & 0x7FFFFFFFu;
  const float a = __builtin_bit_cast(float, ab);
  uint32_t c;
  if (a >= 448.0f) {
    c = 0x7Eu;
  } else if (a < 0.015625f) {
    // subnormal range (below 2^-6): steps of 2^-9; rint ties to even, and the
    // even integer is the even code (8 becomes the smallest normal, 2^-6)
    c = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // normal: keep 3 of the 23 fp32 mantissa bits, rounding to nearest even
    // on the integer bit pattern (a carry moves into the exponent), then
    // rebias the exponent from 127 to 7
    const uint32_t r = ab + 0x7FFFFu + ((ab >> 20) & 1u);
    c = (r >> 20) - ((127u - 7u) << 3);
  }
  return c | sign;
}

// Exact fp32 value of an E4M3 code (NaN for S.1111.111).
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float v;
  if (e == 0xFu && m == 7u) {
    v = __builtin_nanf("");
  } else if (e == 0) {
    v = (float)m * 0.001953125f;  // m * 2^-9
  } else {
    v = __builtin_bit_cast(float, ((e + 127u - 7u) << 23) | (m << 20));
  }
  return (c & 0x80u) ? -v : v;
}

// ---- symmetric blocks: x_hat = s * q, q in [-q_max, q_max] ----------------

// Block scale: the smallest fp16 >= max|x| / q_max, 1.0 for an all-zero block.
__device__ __forceinline__ uint16_t sym_scale16(float amax, int bits) {
#pragma clang fp contract(off)
  if (amax == 0.0f) return (uint16_t)0x3C00;
  return f2h_up(amax / (float)qmax_of(bits));
}

// Stored code u = q - q_min of one element of a block with scale s
// (r = 1/s to within 1 ulp).
__device__ __forceinline__ uint32_t sym_code(float x, float s, float r, int bits) {
#pragma clang fp contract(off)
  const float qm = (float)qmax_of(bits);
  const float q = __builtin_fminf(__builtin_fmaxf(div_rint(x, s, r), -qm), qm);
  return (uint32_t)((int)q - qmin_of(bits));
}

// b-bit field i of a little-endian packed byte array.
__device__ __forceinline__ uint32_t get_field(const uint8_t* p, int i, int bits) {
  const int bit = i * bits;
  return (p[bit >> 3] >> (bit & 7)) & ((1u << bits) - 1u);
}

}  // namespace kvq
