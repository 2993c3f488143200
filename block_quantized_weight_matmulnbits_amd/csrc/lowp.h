// lowp.h -- element formats of the low-precision scaled GEMM (rlx-cpu
// quant.rs: the FP8 / FP6 / FP4 scaled-GEMM reference lowp_scaled_matmul,
// lowp_quantize, lowp_compute_scales) for gfx950 kernels.
//
// Formats (the selector is also the matrix-core instruction's operand format):
//   0 E4M3 (OCP FP8): bias 7, 3 mantissa bits, S.1111.111 nan, max 448
//   1 E5M2 (OCP FP8): bias 15, 2 mantissa bits, exponent 31 inf / nan, max 57344
//   2 E2M3 (OCP MX FP6): bias 1, 3 mantissa bits, max 7.5
//   3 E3M2 (OCP MX FP6): bias 3, 2 mantissa bits, max 28
//   4 E2M1 (OCP MX FP4): bias 1, 1 mantissa bit, max 6
// Exponent field 0 is subnormal.  A code occupies the low bits of its byte
// (higher bits are ignored).
#pragma once

#include "qmm_device.h"

namespace qmm {

template <int F>
struct LowpFmt {
  static constexpr int EB = F == 0 ? 4 : F == 1 ? 5 : F == 2 ? 2 : F == 3 ? 3 : 2;
  static constexpr int MB = F == 0 ? 3 : F == 1 ? 2 : F == 2 ? 3 : F == 3 ? 2 : 1;
  static constexpr int BIAS = F == 0 ? 7 : F == 1 ? 15 : F == 2 ? 1 : F == 3 ? 3 : 1;
  static constexpr int BITS = 1 + EB + MB;
  static constexpr uint32_t MASK = (1u << BITS) - 1u;
  static constexpr float MAXF = F == 0 ? 448.0f : F == 1 ? 57344.0f : F == 2 ? 7.5f
                              : F == 3 ? 28.0f : 6.0f;
  // The code of the largest finite value (E4M3: S.1111.110; E5M2: S.11110.11).
  static constexpr uint32_t MAXC = F == 0 ? 0x7Eu : F == 1 ? 0x7Bu : (MASK >> 1);
};

// Exact binary32 value of a code.
template <int F>
__device__ __forceinline__ float lowp_decode(uint32_t code) {
  using L = LowpFmt<F>;
  const uint32_t c = code & L::MASK;
  const uint32_t sign = (c >> (L::BITS - 1)) << 31;
  const uint32_t e = (c >> L::MB) & ((1u << L::EB) - 1u);
  const uint32_t m = c & ((1u << L::MB) - 1u);
  uint32_t bits;
  if (F == 0 && e == 15 && m == 7) {
    bits = 0x7FC00000u;
  } else if (F == 1 && e == 31) {
    bits = m == 0 ? 0x7F800000u : 0x7FC00000u;
  } else if (e == 0) {
    // m * 2^(1 - bias - mb), exact.
    return __uint_as_float(sign | __float_as_uint((float)m * __uint_as_float((uint32_t)(127 + 1 - L::BIAS - L::MB) << 23)));
  } else {
    bits = ((e + 127u - (uint32_t)L::BIAS) << 23) | (m << (23 - L::MB));
  }
  return __uint_as_float(sign | bits);
}

// Code of v: the nearest finite value, ties to the even mantissa, saturating
// beyond the largest finite value; nan -> the format's nan (E4M3, E5M2: 0x7F)
// or 0; the sign of zero is kept.
template <int F>
__device__ __forceinline__ uint32_t lowp_encode(float v) {
  using L = LowpFmt<F>;
  if (v != v) return (F == 0 || F == 1) ? 0x7Fu : 0u;
  const uint32_t sign = (__float_as_uint(v) >> 31) << (L::BITS - 1);
  const float a = fabsf(v);
  if (a >= L::MAXF) return sign | L::MAXC;
  constexpr int EMIN = 1 - L::BIAS;                 // exponent of the smallest normal
  const int ea = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  uint32_t code;
  if (ea < EMIN) {
    // Subnormal range: q = a / 2^(EMIN - MB), exact; round to an integer
    // (ties to even).  q = 2^MB is the smallest normal's code.
    const float q = a * __uint_as_float((uint32_t)(127 - (EMIN - L::MB)) << 23);
    code = (uint32_t)rintf(q);
  } else {
    // a = 2^ea * (1 + f): q = f * 2^MB, exact; a carry moves to the next
    // exponent (the code as an integer is continuous across binades).
    const float frac = __uint_as_float((__float_as_uint(a) & 0x007FFFFFu) | 0x3F800000u) - 1.0f;
    const uint32_t q = (uint32_t)rintf(frac * (float)(1 << L::MB));
    code = ((uint32_t)(ea - EMIN + 1) << L::MB) + q;
  }
  if (code > L::MAXC) code = L::MAXC;
  return sign | code;
}

}  // namespace qmm
