// repack.hip -- one-time repack of MatMulNBits weights into the tiled layout
// of qmm_layout.h, and its inverse.
//
// The operator keeps each output column's codes as one row of kb * blob bytes
// (onnx-runtime-ep-cpu matmul_nbits.rs, module documentation).  Kernels that
// give each lane a different column then touch one cache line per lane; the
// tiled layout stores, for every group of 32 columns and every chunk of 64
// codes, the 32 columns' chunks back to back (one contiguous 1 KiB wave load
// for 4-bit codes), and stores scales and zero points block-major across the
// 32 columns.  It is a pure byte permutation (the CPU pages make the same
// one-time move when they repack weights at upload: the AMX path's VNNI tile
// order, ggml's repack at set_tensor).
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

namespace qmm {

// Codes: one thread per 4-byte word of the tiled code region.
__global__ __launch_bounds__(256) void repack_codes_kernel(const uint8_t* __restrict__ B,
                                                           uint8_t* __restrict__ T, int64_t words,
                                                           int N, int row_bytes, int chunks,
                                                           int chunk_bytes, bool inverse) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= words) return;
  const int wpc = chunk_bytes / 4;              // words per column chunk
  const int64_t col_chunk = t / wpc;            // (group, chunk, column) index
  const int w = (int)(t % wpc);
  const int i = (int)(col_chunk % TG);
  const int64_t gc = col_chunk / TG;
  const int c = (int)(gc % chunks);
  const int64_t g = gc / chunks;
  const int64_t n = g * TG + i;
  const int64_t off = (int64_t)c * chunk_bytes + 4 * w;   // byte offset in the row
  const bool inside = n < N && off < row_bytes;
  uint32_t* tw = reinterpret_cast<uint32_t*>(T) + t;
  if (!inverse) {
    *tw = inside ? *reinterpret_cast<const uint32_t*>(B + n * row_bytes + off) : 0u;
  } else if (inside) {
    *reinterpret_cast<uint32_t*>(const_cast<uint8_t*>(B) + n * row_bytes + off) = *tw;
  }
}

// Scales: one thread per (group, block, column), raw element copy.
template <typename ST>
__global__ __launch_bounds__(256) void repack_scales_kernel(const ST* __restrict__ S,
                                                            ST* __restrict__ T, int64_t total,
                                                            int N, int kb, bool inverse) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int i = (int)(t % TG);
  const int64_t gb = t / TG;
  const int b = (int)(gb % kb);
  const int64_t g = gb / kb;
  const int64_t n = g * TG + i;
  if (!inverse) {
    T[t] = n < N ? S[n * kb + b] : ST{};
  } else if (n < N) {
    const_cast<ST*>(S)[n * kb + b] = T[t];
  }
}

// Zero points, forward: one thread per byte of the tiled region (packed along
// the 32 columns of a (group, block)).
__global__ __launch_bounds__(256) void repack_zp_kernel(const uint8_t* __restrict__ Z,
                                                        uint8_t* __restrict__ T, int64_t total,
                                                        int N, int kb, int zp_row_bytes, int bits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int per = TG * bits / 8;                 // bytes per (group, block)
  const int j = (int)(t % per);
  const int64_t gb = t / per;
  const int b = (int)(gb % kb);
  const int64_t g = gb / kb;
  const uint32_t mask = (bits == 8) ? 0xFFu : ((1u << bits) - 1u);
  uint32_t out = 0;
  for (int e = 0; e < 8 / bits; ++e) {
    const int i = j * (8 / bits) + e;
    const int64_t n = g * TG + i;
    if (n < N) {
      const int bit = b * bits;
      const uint32_t z = ((uint32_t)Z[n * zp_row_bytes + (bit >> 3)] >> (bit & 7)) & mask;
      out |= z << (e * bits);
    }
  }
  T[t] = (uint8_t)out;
}

// Zero points, inverse: one thread per byte of the operator's zero-point
// rows; bits past the last block are written as zero.
__global__ __launch_bounds__(256) void unrepack_zp_kernel(uint8_t* __restrict__ Z,
                                                          const uint8_t* __restrict__ T,
                                                          int64_t total, int kb, int zp_row_bytes,
                                                          int bits) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int64_t n = t / zp_row_bytes;
  const int j = (int)(t % zp_row_bytes);
  const int64_t g = n / TG;
  const int i = (int)(n % TG);
  const int per = TG * bits / 8;
  const uint32_t mask = (bits == 8) ? 0xFFu : ((1u << bits) - 1u);
  uint32_t out = 0;
  for (int e = 0; e < 8 / bits; ++e) {
    const int b = j * (8 / bits) + e;
    if (b < kb) {
      const int ib = i * bits;
      const uint32_t z = ((uint32_t)T[(g * kb + b) * per + (ib >> 3)] >> (ib & 7)) & mask;
      out |= z << (e * bits);
    }
  }
  Z[t] = (uint8_t)out;
}

// Zero fill of the alignment gaps between and after the regions, so that the
// repacked buffer is fully determined by its inputs.
__global__ __launch_bounds__(256) void zero_gap_kernel(uint8_t* __restrict__ p, int64_t n) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < n) p[t] = 0;
}

hipError_t launch_repack(const MatArgs& a, uint8_t* tiled, bool inverse, uint8_t* B_out,
                         void* scales_out, uint8_t* zp_out) {
  const int ssz = a.s_dtype == DT_F32 ? 4 : 2;
  const TiledGeom g = tiled_geom(a.K, a.N, a.block_size, a.bits, ssz, a.zp != nullptr || zp_out);
  const int row_bytes = (int)(a.kb * a.blob);
  auto grid = [](int64_t n) { return dim3((unsigned)((n + 255) / 256)); };
  if (!inverse) {
    const int64_t gaps[3][2] = {{g.codes_off + g.codes_bytes, g.scales_off},
                                {g.scales_off + g.scales_bytes, g.zps_off},
                                {g.zps_off + g.zps_bytes, g.total}};
    for (const auto& gp : gaps) {
      if (gp[1] <= gp[0]) continue;
      hipLaunchKernelGGL(zero_gap_kernel, grid(gp[1] - gp[0]), dim3(256), 0, a.stream,
                         tiled + gp[0], gp[1] - gp[0]);
    }
  }
  // Codes.
  const int64_t words = g.codes_bytes / 4;
  hipLaunchKernelGGL(repack_codes_kernel, grid(words), dim3(256), 0, a.stream,
                     inverse ? B_out : a.B, tiled + g.codes_off, words, (int)a.N, row_bytes,
                     (int)g.chunks, (int)g.chunk_bytes, inverse);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Scales.
  const int64_t ns = g.groups * g.kb * TG;
  if (ssz == 4)
    hipLaunchKernelGGL((repack_scales_kernel<uint32_t>), grid(ns), dim3(256), 0, a.stream,
                       (const uint32_t*)(inverse ? scales_out : a.scales),
                       (uint32_t*)(tiled + g.scales_off), ns, (int)a.N, (int)a.kb, inverse);
  else
    hipLaunchKernelGGL((repack_scales_kernel<uint16_t>), grid(ns), dim3(256), 0, a.stream,
                       (const uint16_t*)(inverse ? scales_out : a.scales),
                       (uint16_t*)(tiled + g.scales_off), ns, (int)a.N, (int)a.kb, inverse);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Zero points.
  if (!inverse && a.zp) {
    hipLaunchKernelGGL(repack_zp_kernel, grid(g.zps_bytes), dim3(256), 0, a.stream, a.zp,
                       tiled + g.zps_off, g.zps_bytes, (int)a.N, (int)a.kb, (int)a.zp_row_bytes,
                       a.bits);
  } else if (inverse && zp_out) {
    const int64_t nz = a.N * a.zp_row_bytes;
    hipLaunchKernelGGL(unrepack_zp_kernel, grid(nz), dim3(256), 0, a.stream, zp_out,
                       tiled + g.zps_off, nz, (int)a.kb, (int)a.zp_row_bytes, a.bits);
  }
  return hipGetLastError();
}

}  // namespace qmm
