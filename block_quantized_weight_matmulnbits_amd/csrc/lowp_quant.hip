// lowp_quant.hip -- the producers of the low-precision scaled GEMM's
// operands for gfx950 (rlx-cpu quant.rs: lowp_compute_scales with
// lowp_snap_scale and the stored scale forms of ScaledQuantScale, then
// lowp_quantize): for x [rows, cols],
//   scale   per tensor: amax(|x|) / max_finite (1 where amax is 0), one f32;
//           per block of bs along cols (MX 32, NVFP4 16): the same over the
//           block, snapped to what the layout stores (E8M0: the binary32
//           exponent field; NVFP4: the nearest E4M3), stored as that byte;
//   code    encode(x / s) with the binary32 quotient (0 where s is 0): the
//           nearest finite value of the format, ties to even, saturating.
// Maxima skip nan (as fmaxf does).  The divisions are IEEE binary32 (the
// library is built with correctly rounded division), so every code and
// scale byte equals the definition's bit for bit.
//
// Blocks: bs / 4 adjacent lanes own one block, 4 elements each, and combine
// their maxima with cross-lane shuffles; a row is padded to whole blocks of
// lanes so that a block never straddles a wave.  Per tensor: a zero-fill
// kernel, an amax kernel (wave maxima combined with an atomic maximum on
// the binary32 bits, which order like the values for non-negative floats),
// the quantize kernel, and a one-thread kernel that replaces the stored
// amax by the scale.
#include <algorithm>

#include "lowp.h"
#include "mfma_ops.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int QTPB = 256;

template <int XDT>
__device__ __forceinline__ float load_x(const void* x, int64_t i) {
  if constexpr (XDT == DT_F32) return reinterpret_cast<const float*>(x)[i];
  else return bits16_to_f32<XDT>(reinterpret_cast<const uint16_t*>(x)[i]);
}

// E8M0 byte of a binary32 scale: its exponent field.
__device__ __forceinline__ uint32_t e8m0_of(float s) { return (__float_as_uint(s) >> 23) & 0xFFu; }
__device__ __forceinline__ float e8m0_value(uint32_t e) {
  // 2^(e - 127): e = 0 is the binary32 subnormal 2^-127, 255 nan.
  if (e == 0) return __uint_as_float(0x00400000u);
  return __uint_as_float(e == 255 ? 0x7FC00000u : e << 23);
}

template <int F, int XDT, int LAYOUT>
__global__ __launch_bounds__(QTPB) void lowp_quant_kernel(const void* __restrict__ x,
                                                          uint8_t* __restrict__ codes,
                                                          void* __restrict__ scales, int rows,
                                                          int cols, int lanes_per_row) {
  constexpr int BS = LAYOUT == 1 ? 32 : 16;
  constexpr int LPB = LAYOUT == 0 ? 1 : BS / 4;       // lanes per block
  const int64_t t = (int64_t)blockIdx.x * QTPB + threadIdx.x;
  const int row = (int)(t / lanes_per_row);
  const int c0 = (int)(t % lanes_per_row) * 4;
  const bool live = row < rows;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    v[j] = (live && c0 + j < cols) ? load_x<XDT>(x, (int64_t)row * cols + c0 + j) : 0.0f;
  float s;
  if constexpr (LAYOUT == 0) {
    // The stored value is still amax here (see the host sequence).
    const float amax = reinterpret_cast<const float*>(scales)[0];
    s = amax > 0.0f ? amax / LowpFmt<F>::MAXF : 1.0f;
  } else {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fabsf(v[j]));
#pragma unroll
    for (int o = 1; o < LPB; o *= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
    const float raw = amax > 0.0f ? amax / LowpFmt<F>::MAXF : 1.0f;
    uint32_t byte;
    if constexpr (LAYOUT == 1) {
      byte = e8m0_of(raw);
      s = e8m0_value(byte);
    } else {
      byte = lowp_encode<0>(raw);
      s = lowp_decode<0>(byte);
    }
    if (live && (threadIdx.x % LPB) == 0 && c0 < cols)
      reinterpret_cast<uint8_t*>(scales)[(int64_t)row * ((cols + BS - 1) / BS) + c0 / BS] = (uint8_t)byte;
  }
  if (!live) return;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (c0 + j < cols)
      codes[(int64_t)row * cols + c0 + j] = (uint8_t)lowp_encode<F>(s != 0.0f ? v[j] / s : 0.0f);
}

__global__ void lowp_zero_kernel(uint32_t* p) { p[0] = 0u; }

template <int XDT>
__global__ __launch_bounds__(QTPB) void lowp_amax_kernel(const void* __restrict__ x, int64_t total,
                                                         uint32_t* __restrict__ amax_bits) {
  float amax = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * QTPB + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * QTPB)
    amax = fmaxf(amax, fabsf(load_x<XDT>(x, i)));
#pragma unroll
  for (int o = 1; o < 64; o *= 2) amax = fmaxf(amax, __shfl_xor(amax, o));
  if ((threadIdx.x & 63) == 0) atomicMax(amax_bits, __float_as_uint(amax));
}

template <int F>
__global__ void lowp_amax_to_scale_kernel(float* scale) {
  const float amax = scale[0];
  scale[0] = amax > 0.0f ? amax / LowpFmt<F>::MAXF : 1.0f;
}

template <int F, int XDT>
hipError_t quant_t(const LowpQuantArgs& a) {
  const int bs = a.layout == 1 ? 32 : 16;
  const int64_t lanes_per_row = a.layout == 0 ? (a.cols + 3) / 4 : (a.cols + bs - 1) / bs * (bs / 4);
  const int64_t threads = lanes_per_row * a.rows;
  const dim3 grid((unsigned)((threads + QTPB - 1) / QTPB)), block(QTPB);
  if (a.layout == 0) {
    uint32_t* amax = reinterpret_cast<uint32_t*>(a.scales);
    hipLaunchKernelGGL(lowp_zero_kernel, dim3(1), dim3(1), 0, a.stream, amax);
    const int64_t total = a.rows * a.cols;
    const unsigned g = (unsigned)std::min<int64_t>(2048, (total + QTPB - 1) / QTPB);
    hipLaunchKernelGGL(lowp_amax_kernel<XDT>, dim3(g), block, 0, a.stream, a.x, total, amax);
    hipLaunchKernelGGL((lowp_quant_kernel<F, XDT, 0>), grid, block, 0, a.stream, a.x, a.codes,
                       a.scales, (int)a.rows, (int)a.cols, (int)lanes_per_row);
    hipLaunchKernelGGL(lowp_amax_to_scale_kernel<F>, dim3(1), dim3(1), 0, a.stream,
                       reinterpret_cast<float*>(a.scales));
  } else if (a.layout == 1) {
    hipLaunchKernelGGL((lowp_quant_kernel<F, XDT, 1>), grid, block, 0, a.stream, a.x, a.codes,
                       a.scales, (int)a.rows, (int)a.cols, (int)lanes_per_row);
  } else {
    hipLaunchKernelGGL((lowp_quant_kernel<F, XDT, 2>), grid, block, 0, a.stream, a.x, a.codes,
                       a.scales, (int)a.rows, (int)a.cols, (int)lanes_per_row);
  }
  return hipGetLastError();
}

template <int F>
hipError_t quant_f(const LowpQuantArgs& a) {
  switch (a.x_dtype) {
    case DT_F32: return quant_t<F, DT_F32>(a);
    case DT_F16: return quant_t<F, DT_F16>(a);
    default: return quant_t<F, DT_BF16>(a);
  }
}

}  // namespace

hipError_t launch_lowp_quantize(const LowpQuantArgs& a) {
  switch (a.fmt) {
    case 0: return quant_f<0>(a);
    case 1: return quant_f<1>(a);
    case 2: return quant_f<2>(a);
    case 3: return quant_f<3>(a);
    default: return quant_f<4>(a);
  }
}

}  // namespace qmm
