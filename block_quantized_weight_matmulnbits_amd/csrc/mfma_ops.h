// mfma_ops.h -- helpers shared by the matrix-core kernels over 16-bit
// activations (gemm.hip, gemm_skinny.hip): the bf16 / f16 16x16x32 MFMA with
// its rounding of a dequantized weight to the activation dtype, and the
// unpacking of a 32-bit word of codes into fp32 values.
#pragma once

#include "qmm_device.h"

namespace qmm {

// Word 3 of a buffer resource descriptor for raw byte-addressed loads.
constexpr int BUF_WORD3 = 0x00020000;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int XDT> struct MfmaOp;
template <> struct MfmaOp<DT_BF16> {
  using V = bf16x8;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t round(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
  }
  // Two values rounded to nearest even and packed (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <> struct MfmaOp<DT_F16> {
  using V = f16x8;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t round(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    const half2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  }
};

// w & m through an instruction the compiler cannot look into, so that the
// byte conversions below stay v_cvt_f32_ubyte{0..3} of the masked word
// instead of becoming one bit-field extract per code.
__device__ __forceinline__ uint32_t opaque_and(uint32_t w, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %2, %1" : "=v"(r) : "v"(w), "s"(m));
  return r;
}

// Codes of one 32-bit word as fp32 values, in element order.
template <int BITS>
__device__ __forceinline__ void word_codes_f32(uint32_t w, float* q) {
  if constexpr (BITS == 8) {
    q[0] = (float)(w & 0xFF); q[1] = (float)((w >> 8) & 0xFF);
    q[2] = (float)((w >> 16) & 0xFF); q[3] = (float)(w >> 24);
  } else if constexpr (BITS == 4) {
    const uint32_t lo = opaque_and(w, 0x0F0F0F0Fu), hi = opaque_and(w >> 4, 0x0F0F0F0Fu);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      q[2 * j] = (float)((lo >> (8 * j)) & 0xFF);
      q[2 * j + 1] = (float)((hi >> (8 * j)) & 0xFF);
    }
  } else {
    const uint32_t f[4] = {opaque_and(w, 0x03030303u), opaque_and(w >> 2, 0x03030303u),
                           opaque_and(w >> 4, 0x03030303u), opaque_and(w >> 6, 0x03030303u)};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[4 * j + i] = (float)((f[i] >> (8 * j)) & 0xFF);
  }
}

}  // namespace qmm
