// conv.hip -- int8 convolution with requantization for gfx950, as an implicit
// GEMM on the int8 matrix cores (no im2col buffer).
//
// Definition (MNN ConvInt8TiledExecutor.cpp: the im2col of the input is padded
// with the input zero point, the post-treatment clamps to [clamp_min,
// clamp_max]; rlx-cpu quant.rs exec_q_mat_mul: the int32 accumulator starts
// at the bias, then requantizes as round(acc * mult) + out_zp):
//   acc[p, oc] = bias[oc] + sum_{kh,kw,c} (x - in_zp) * w[oc, kh, kw, c]
//   y = clamp(rne(float(acc) * mult[oc]) + out_zp),
//   mult[oc] = (in_scale * w_scale[oc]) / out_scale        (binary32)
//
// GEMM view: rows are output pixels p, columns output channels oc, and the
// reduction index k = (kh * KW + kw) * C + c, which is contiguous in both the
// NHWC input (per tap) and the OHWI weight rows.  A wave computes 16 pixels x
// 16*NT channels with v_mfma_i32_16x16x64_i8: each lane holds 16 int8 of its
// pixel (A) and of its channel (B) for the same 16 reduction indices, so the
// products pair correctly whatever order the instruction uses inside a lane.
// A tap outside the image contributes x = in_zp; the sum is taken over raw x
// and corrected by in_zp * sum(w), which an extra MFMA against an all-ones
// operand yields exactly.  Everything up to the requantization is int32.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int CONV_NT = 4;   // 16-channel tiles per wave (64 channels)

__global__ __launch_bounds__(64) void conv_int8_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ Wt, const int32_t* __restrict__ bias,
    const float* __restrict__ w_scale, float in_scale, float out_scale, int in_zp, int out_zp,
    int clamp_min, int clamp_max, int H, int W, int C, int Co, int KH, int KW, int sh, int sw,
    int ph, int pw, int OH, int OW, int P, int8_t* __restrict__ Y) {
  const int lane = threadIdx.x;
  const int p0 = blockIdx.x * 16;
  const int oc0 = blockIdx.y * (16 * CONV_NT);
  const int K = KH * KW * C;
  const int g = lane >> 4;          // which 16 reduction indices of the 64
  const int li = lane & 15;         // pixel (A) / channel (B) within the tile

  // This lane's pixel.
  const int p = p0 + li;
  const bool p_ok = p < P;
  const int pp = p_ok ? p : 0;
  const int nb = pp / (OH * OW);
  const int ohw = pp % (OH * OW);
  const int oh = ohw / OW, ow = ohw % OW;
  const uint32_t zp4 = ((uint32_t)(uint8_t)(int8_t)in_zp) * 0x01010101u;

  i32x4 acc[CONV_NT], wsum[CONV_NT];
#pragma unroll
  for (int t = 0; t < CONV_NT; ++t) {
    acc[t] = i32x4{0, 0, 0, 0};
    wsum[t] = i32x4{0, 0, 0, 0};
  }
  const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

  for (int k0 = 0; k0 < K; k0 += 64) {
    // A: 4 groups of 4 channels (C % 4 == 0, so a group stays in one tap).
    int av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + g * 16 + j * 4;
      uint32_t v = 0;                          // k >= K: zero (weights are zero too)
      if (k < K) {
        const int tap = k / C, c = k % C;
        const int kh = tap / KW, kw = tap % KW;
        const int ih = oh * sh - ph + kh, iw = ow * sw - pw + kw;
        v = zp4;                               // outside the image: the input zero point
        if (p_ok && ih >= 0 && ih < H && iw >= 0 && iw < W)
          v = *reinterpret_cast<const uint32_t*>(X + (((int64_t)nb * H + ih) * W + iw) * C + c);
      }
      av[j] = (int)v;
    }
    const i32x4 a = {av[0], av[1], av[2], av[3]};
#pragma unroll
    for (int t = 0; t < CONV_NT; ++t) {
      const int oc = oc0 + t * 16 + li;
      int bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + g * 16 + j * 4;
        bv[j] = (oc < Co && k < K) ? *reinterpret_cast<const int*>(Wt + (int64_t)oc * K + k) : 0;
      }
      const i32x4 b = {bv[0], bv[1], bv[2], bv[3]};
      acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
      wsum[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, wsum[t], 0, 0, 0);
    }
  }

  // Epilogue: lane l holds pixels 4 * (l / 16) + [0, 4) of channel l % 16.
#pragma unroll
  for (int t = 0; t < CONV_NT; ++t) {
    const int oc = oc0 + t * 16 + li;
    if (oc >= Co) continue;
    const float mult = (in_scale * w_scale[oc]) / out_scale;   // binary32, IEEE division
    const int b0 = bias ? bias[oc] : 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pe = p0 + g * 4 + e;
      if (pe >= P) continue;
      const int a = b0 + acc[t][e] - in_zp * wsum[t][e];
      const float r = rintf((float)a * mult);
      float v = r + (float)out_zp;
      v = fminf(fmaxf(v, (float)clamp_min), (float)clamp_max);
      Y[(int64_t)pe * Co + oc] = (int8_t)(int)v;
    }
  }
}

hipError_t launch_conv_int8(const ConvArgs& c) {
  const int OH = (c.H + 2 * c.pad_h - c.KH) / c.stride_h + 1;
  const int OW = (c.W + 2 * c.pad_w - c.KW) / c.stride_w + 1;
  const int P = c.Nb * OH * OW;
  dim3 grid((P + 15) / 16, (c.Co + 16 * CONV_NT - 1) / (16 * CONV_NT));
  hipLaunchKernelGGL(conv_int8_kernel, grid, dim3(64), 0, c.stream, c.X, c.Wt, c.bias, c.w_scale,
                     c.in_scale, c.out_scale, c.in_zp, c.out_zp, c.clamp_min, c.clamp_max, c.H,
                     c.W, c.C, c.Co, c.KH, c.KW, c.stride_h, c.stride_w, c.pad_h, c.pad_w, OH, OW,
                     P, c.Y);
  return hipGetLastError();
}

}  // namespace qmm
