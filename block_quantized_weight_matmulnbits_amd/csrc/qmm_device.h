// qmm_device.h -- device-side helpers shared by the gfx950 kernels of the
// block-quantized-weight matmul library: dtype traits, packed-code field
// extraction and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

enum : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Cache policy of buffer loads of data read once (the packed codes streamed by
// the M = 1 kernels): the non-temporal bit of gfx950's buffer-load cache
// policy.  A plain read of the decode layer's gate|up bytes ran at 5.9 TB/s
// with it and 5.6 without; the tiled GEMV's gate|up launch went from 16.6 to
// 15.1-15.5 us.  (The few-row matrix-core kernel, whose 8 waves read adjacent
// pieces of each column, measured 2-7 % slower with it and does not use it;
// nor do the scale and zero-point loads, which neighbouring waves share.)
constexpr int BUF_STREAM = 2;

// Storage type and exact widening / rounding narrowing of each float dtype.
template <int DT> struct dt;
template <> struct dt<DT_F32> {
  using T = float;
  static __device__ __forceinline__ float to_f32(T v) { return v; }
  static __device__ __forceinline__ T from_f32(float f) { return f; }
};
template <> struct dt<DT_F16> {
  using T = _Float16;
  static __device__ __forceinline__ float to_f32(T v) { return (float)v; }
  static __device__ __forceinline__ T from_f32(float f) { return (_Float16)f; }
};
template <> struct dt<DT_BF16> {
  using T = uint16_t;  // raw bfloat16 bits
  static __device__ __forceinline__ float to_f32(T v) {
    return __uint_as_float((uint32_t)v << 16);
  }
  // Round to nearest even (the hardware conversion on gfx950).
  static __device__ __forceinline__ T from_f32(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
};

// Widen the raw 16-bit pattern of an f16 or bf16 value to fp32 (exact).
template <int DT>
__device__ __forceinline__ float bits16_to_f32(uint16_t h) {
  if constexpr (DT == DT_BF16) return __uint_as_float((uint32_t)h << 16);
  else return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ half2_t as_half2(uint32_t u) {
  return __builtin_bit_cast(half2_t, u);
}
__device__ __forceinline__ uint32_t as_u32(half2_t h) {
  return __builtin_bit_cast(uint32_t, h);
}

// Two codes of a 32-bit word of packed codes as an fp16 pair.
// A word holds P = 32 / BITS codes e_0 .. e_{P-1}, element e_j at bits
// [j*BITS, (j+1)*BITS).  Field i of the word pairs e_i (low half) with
// e_{i + P/2} (high half): shifting by i*BITS and masking both 16-bit halves
// keeps exactly those two codes.  OR-ing 0x6400 (fp16 1024.0, whose ulp is 1)
// makes each half the fp16 number 1024 + code, exactly.
template <int BITS>
__device__ __forceinline__ uint32_t code_pair_1024(uint32_t w, int i) {
  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  constexpr uint32_t mask2 = m | (m << 16);
  return ((w >> (i * BITS)) & mask2) | 0x64006400u;
}

// fp16 pair holding -(1024 + z) twice: adding it to code_pair_1024 gives the
// exact small integers (code - z) (|code - z| <= 255 is exact in fp16).
__device__ __forceinline__ half2_t neg_zero_point_pair(uint32_t z) {
  uint32_t h = 0xE400u | z;  // fp16 bits of -(1024 + z), z < 1024
  return as_half2(h | (h << 16));
}

// Sum over the 64 lanes of a wave with DPP row operations; every lane gets
// the total.
__device__ __forceinline__ float wave_sum(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));  // row_mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));  // row_bcast:15
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_sum_i32(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
  return __builtin_amdgcn_readlane(v, 63);
}

// Zero point of block b from a packed zero-point row (LSB first); absent
// zero points are 2^(BITS-1).
template <int BITS, bool HAS_ZP>
__device__ __forceinline__ uint32_t load_zp(const uint8_t* __restrict__ zrow, int b) {
  if constexpr (!HAS_ZP) {
    return 1u << (BITS - 1);
  } else {
    constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
    const int bit = b * BITS;
    return ((uint32_t)zrow[bit >> 3] >> (bit & 7)) & m;
  }
}

// Block-scaled FP4 weight formats: MXFP4 (E8M0 scale per 32) and NVFP4
// (E4M3 scale per 16, with a global scale).
enum : int { FP4_MX = 0, FP4_NV = 1 };

// A decoded FP4 block scale, exact in fp32 (nan stays nan): E8M0 is
// 2^(e - 127) (255 = nan; 0 = 2^-127, an fp32 subnormal); E4M3 has bias 7,
// subnormals m/8 * 2^-6 and nan S.1111.111.
__device__ __forceinline__ float fp4_scale(uint32_t byte, int fmt) {
  byte &= 0xFFu;
  if (fmt == FP4_MX) {
    if (byte == 0xFFu) return __uint_as_float(0x7FC00000u);
    if (byte == 0u) return __uint_as_float(0x00400000u);
    return __uint_as_float(byte << 23);
  }
  const uint32_t e = (byte >> 3) & 15u, m = byte & 7u;
  float v;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  else if (e == 0u) v = (float)m * 0x1p-9f;
  else v = __uint_as_float(((e + 120u) << 23) | (m << 20));   // 2^(e-7) * (1 + m/8)
  return (byte & 0x80u) ? -v : v;
}

}  // namespace qmm
