// codec.hip -- device-side codec of the MatMulNBits layout, exported for the
// bit-exact tests: per element, the code at bit (k % bs) * bits of block k / bs
// (least-significant bits first; 3-bit codes in the 2 + 1 bit-plane blob of
// MNN ConvInt8TiledExecutor.cpp's 3-bit reorder), the block's zero point
// (packed the same way, default 2^(bits-1)) and the dequantized fp32 weight
// (code - zp) * scale (onnx-runtime-ep-cpu matmul_nbits.rs:
// dequantize_nbits_value).
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

template <int SDT>
__global__ __launch_bounds__(256) void unpack_kernel(const uint8_t* __restrict__ B,
                                                     const typename dt<SDT>::T* __restrict__ scales,
                                                     const uint8_t* __restrict__ zp,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ zps,
                                                     float* __restrict__ w, int K, int N, int bs,
                                                     int bits, int kb, int blob, int zp_row_bytes) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)N * K) return;
  const int n = (int)(i / K), k = (int)(i % K);
  const int b = k / bs;
  const uint32_t mask = (bits == 8) ? 0xFFu : ((1u << bits) - 1u);
  const uint8_t* blk = B + ((int64_t)n * kb + b) * blob;
  uint32_t q;
  if (bits == 3) {
    // 2 + 1 bit planes: low two bits at bits 2 (i % 4) of byte i / 4, the
    // high bit at bit i % 8 of byte bs / 4 + i / 8.
    const int i = k % bs;
    q = (((uint32_t)blk[i / 4] >> (2 * (i % 4))) & 3u) |
        ((((uint32_t)blk[bs / 4 + i / 8] >> (i % 8)) & 1u) << 2);
  } else {
    const int bit = (k % bs) * bits;
    q = ((uint32_t)blk[bit >> 3] >> (bit & 7)) & mask;
  }
  uint32_t z = 1u << (bits - 1);
  if (zp) {
    // One LSB-first stream per row; a 3-bit value may cross a byte.
    const int zbit = b * bits;
    const uint8_t* zr = zp + (int64_t)n * zp_row_bytes;
    uint32_t v = (uint32_t)zr[zbit >> 3] >> (zbit & 7);
    if ((zbit & 7) + bits > 8) v |= (uint32_t)zr[(zbit >> 3) + 1] << (8 - (zbit & 7));
    z = v & mask;
  }
  if (codes) codes[i] = (uint8_t)q;
  if (zps && k % bs == 0) zps[(int64_t)n * kb + b] = (uint8_t)z;
  if (w) w[i] = (float)((int)q - (int)z) * dt<SDT>::to_f32(scales[(int64_t)n * kb + b]);
}

hipError_t launch_unpack(const MatArgs& a, uint8_t* codes, uint8_t* zps, float* w) {
  const int64_t total = a.N * a.K;
  const int grid = (int)((total + 255) / 256);
  switch (a.s_dtype) {
    case DT_F32:
      hipLaunchKernelGGL((unpack_kernel<DT_F32>), dim3(grid), dim3(256), 0, a.stream, a.B,
                         (const float*)a.scales, a.zp, codes, zps, w, (int)a.K, (int)a.N,
                         (int)a.block_size, a.bits, (int)a.kb, (int)a.blob, (int)a.zp_row_bytes);
      break;
    case DT_F16:
      hipLaunchKernelGGL((unpack_kernel<DT_F16>), dim3(grid), dim3(256), 0, a.stream, a.B,
                         (const _Float16*)a.scales, a.zp, codes, zps, w, (int)a.K, (int)a.N,
                         (int)a.block_size, a.bits, (int)a.kb, (int)a.blob, (int)a.zp_row_bytes);
      break;
    default:
      hipLaunchKernelGGL((unpack_kernel<DT_BF16>), dim3(grid), dim3(256), 0, a.stream, a.B,
                         (const uint16_t*)a.scales, a.zp, codes, zps, w, (int)a.K, (int)a.N,
                         (int)a.block_size, a.bits, (int)a.kb, (int)a.blob, (int)a.zp_row_bytes);
      break;
  }
  return hipGetLastError();
}

}  // namespace qmm
