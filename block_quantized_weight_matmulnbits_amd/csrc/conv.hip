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
// NHWC input (per tap) and the OHWI weight rows.  A workgroup computes 16
// pixels x 16*NT channels with v_mfma_i32_16x16x64_i8: each lane holds 16 int8
// of its pixel (A) and of its channel (B) for the same 16 reduction indices, so
// the products pair correctly whatever order the instruction uses inside a
// lane.
// A tap outside the image contributes x = in_zp; the sum is taken over raw x
// and corrected by in_zp * sum(w), which an extra MFMA against an all-ones
// operand yields exactly.  Everything up to the requantization is int32.
#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int CONV_NT = 4;      // 16-channel tiles per workgroup (64 channels)
constexpr int CONV_WAVES = 4;   // waves splitting the reduction
constexpr int CONV_BATCH = 3;   // 64-wide reduction steps whose loads are issued together

// q = n / d and r = n % d for 0 <= n < 2^24 from a float reciprocal, fixed up
// by one correction step (the float quotient is within one of the true one).
__device__ __forceinline__ void divmod_small(int n, int d, float inv_d, int& q, int& r) {
  q = (int)((float)n * inv_d);
  r = n - q * d;
  if (r < 0) { q -= 1; r += d; }
  else if (r >= d) { q += 1; r -= d; }
}

// A workgroup computes 16 output pixels x 64 output channels; its 4 waves
// take contiguous shares of the 64-wide reduction steps and add their exact
// int32 partial sums through LDS (integer addition: the order does not
// matter).  A wave issues the loads of up to CONV_BATCH steps before using
// any of them, from addresses that are always valid (out-of-image taps and
// the tail past K read element 0 and are replaced afterwards), so the loads
// stay free of branches and their latency is paid once per batch.
// VEC = 16: C % 16 == 0 and 16-byte aligned tensors, so a lane's 16
// reduction indices of a step lie in one tap and are 16 contiguous bytes of
// both the input pixel and the weight row: one 16-byte load each.
// VEC = 4: C % 4 == 0 and 4-byte aligned tensors: four 4-byte loads, each
// group of 4 channels inside one tap.
// VEC = 1: any C: every byte is gathered on its own (its own tap), and the
// zero-point / zero replacement is applied per byte as it is loaded.
template <int VEC>
__global__ __launch_bounds__(64 * CONV_WAVES) void conv_int8_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ Wt, const int32_t* __restrict__ bias,
    const float* __restrict__ w_scale, float in_scale, float out_scale, int in_zp, int out_zp,
    int clamp_min, int clamp_max, int H, int W, int C, int Co, int KH, int KW, int sh, int sw,
    int ph, int pw, int OH, int OW, int P, float inv_c, float inv_kw, int8_t* __restrict__ Y) {
  __shared__ i32x4 red[CONV_WAVES - 1][2 * CONV_NT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p0 = blockIdx.x * 16;
  const int oc0 = blockIdx.y * (16 * CONV_NT);
  const int K = KH * KW * C;
  const int KS = (K + 63) / 64;
  const int ksw = (KS + CONV_WAVES - 1) / CONV_WAVES;
  const int ks_lo = wave * ksw, ks_hi = min(KS, ks_lo + ksw);
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

  // The epilogue's per-channel bias and requantization multiplier, loaded
  // before the reduction so their latency hides under it.
  int bias_t[CONV_NT];
  float mult_t[CONV_NT];
#pragma unroll
  for (int t = 0; t < CONV_NT; ++t) {
    const int oc = oc0 + t * 16 + li;
    const int occ = oc < Co ? oc : 0;
    bias_t[t] = bias ? bias[occ] : 0;
    mult_t[t] = (in_scale * w_scale[occ]) / out_scale;   // binary32, IEEE division
  }

  for (int ks0 = ks_lo; ks0 < ks_hi; ks0 += CONV_BATCH) {
    uint32_t av[CONV_BATCH][4], bv[CONV_BATCH][CONV_NT][4];
    uint32_t ain = 0, kin = 0;       // bit 4 s + j: inside the image / k < K
#pragma unroll
    for (int s = 0; s < CONV_BATCH; ++s) {
      if constexpr (VEC == 16) {
        // The lane's 16 indices: one tap, channels c .. c + 15 (K % 16 == 0,
        // so the group is all in or all out).
        const int k = (ks0 + s) * 64 + g * 16;
        const bool k_ok = k < K;
        int tap, c, kh, kw;
        divmod_small(k_ok ? k : 0, C, inv_c, tap, c);
        divmod_small(tap, KW, inv_kw, kh, kw);
        const int ih = oh * sh - ph + kh, iw = ow * sw - pw + kw;
        const bool inside = p_ok && k_ok && ih >= 0 && ih < H && iw >= 0 && iw < W;
        const int64_t xoff = inside ? (((int64_t)nb * H + ih) * W + iw) * C + c : 0;
        const u32x4 xa = *reinterpret_cast<const u32x4*>(X + xoff);
        av[s][0] = xa.x; av[s][1] = xa.y; av[s][2] = xa.z; av[s][3] = xa.w;
        ain |= (inside ? 0xFu : 0u) << (4 * s);
        kin |= (k_ok ? 0xFu : 0u) << (4 * s);
#pragma unroll
        for (int t = 0; t < CONV_NT; ++t) {
          const int oc = oc0 + t * 16 + li;
          const bool w_ok = oc < Co && k_ok;
          const u32x4 wb = *reinterpret_cast<const u32x4*>(Wt + (w_ok ? (int64_t)oc * K + k : 0));
          bv[s][t][0] = wb.x; bv[s][t][1] = wb.y; bv[s][t][2] = wb.z; bv[s][t][3] = wb.w;
        }
        continue;
      }
      if constexpr (VEC == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t xw = 0, ww[CONV_NT];
#pragma unroll
          for (int t = 0; t < CONV_NT; ++t) ww[t] = 0;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k = (ks0 + s) * 64 + g * 16 + j * 4 + e;
            const bool k_ok = k < K;
            int tap, c, kh, kw;
            divmod_small(k_ok ? k : 0, C, inv_c, tap, c);
            divmod_small(tap, KW, inv_kw, kh, kw);
            const int ih = oh * sh - ph + kh, iw = ow * sw - pw + kw;
            const bool inside = p_ok && k_ok && ih >= 0 && ih < H && iw >= 0 && iw < W;
            const int64_t xoff = inside ? (((int64_t)nb * H + ih) * W + iw) * C + c : 0;
            const uint32_t xb = (uint8_t)X[xoff];
            xw |= (inside ? xb : (zp4 & 0xFFu)) << (8 * e);
#pragma unroll
            for (int t = 0; t < CONV_NT; ++t) {
              const int oc = oc0 + t * 16 + li;
              const bool w_ok = oc < Co && k_ok;
              const uint32_t wb = (uint8_t)Wt[w_ok ? (int64_t)oc * K + k : 0];
              ww[t] |= (w_ok ? wb : 0u) << (8 * e);
            }
          }
          // Already replaced byte by byte: mark the group as taken as is.
          av[s][j] = xw;
          ain |= 1u << (4 * s + j);
          kin |= 1u << (4 * s + j);
#pragma unroll
          for (int t = 0; t < CONV_NT; ++t) bv[s][t][j] = ww[t];
        }
        continue;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // A group of 4 channels (C % 4 == 0, so a group stays in one tap).
        const int k = (ks0 + s) * 64 + g * 16 + j * 4;
        const bool k_ok = k < K;
        int tap, c, kh, kw;
        divmod_small(k_ok ? k : 0, C, inv_c, tap, c);
        divmod_small(tap, KW, inv_kw, kh, kw);
        const int ih = oh * sh - ph + kh, iw = ow * sw - pw + kw;
        const bool inside = p_ok && k_ok && ih >= 0 && ih < H && iw >= 0 && iw < W;
        const int64_t xoff = inside ? (((int64_t)nb * H + ih) * W + iw) * C + c : 0;
        av[s][j] = *reinterpret_cast<const uint32_t*>(X + xoff);
        ain |= (uint32_t)inside << (4 * s + j);
        kin |= (uint32_t)k_ok << (4 * s + j);
#pragma unroll
        for (int t = 0; t < CONV_NT; ++t) {
          const int oc = oc0 + t * 16 + li;
          const bool w_ok = oc < Co && k_ok;
          bv[s][t][j] = *reinterpret_cast<const uint32_t*>(Wt + (w_ok ? (int64_t)oc * K + k : 0));
        }
      }
    }
#pragma unroll
    for (int s = 0; s < CONV_BATCH; ++s) {
      if (ks0 + s >= ks_hi) break;
      int a4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        // Outside the image (or past K, where the weights are zero) the
        // activation is the input zero point.
        a4[j] = (int)(((ain >> (4 * s + j)) & 1u) ? av[s][j] : zp4);
      const i32x4 a = {a4[0], a4[1], a4[2], a4[3]};
#pragma unroll
      for (int t = 0; t < CONV_NT; ++t) {
        const int oc = oc0 + t * 16 + li;
        int b4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          b4[j] = (int)((oc < Co && ((kin >> (4 * s + j)) & 1u)) ? bv[s][t][j] : 0u);
        const i32x4 b = {b4[0], b4[1], b4[2], b4[3]};
        acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[t], 0, 0, 0);
        wsum[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ones, b, wsum[t], 0, 0, 0);
      }
    }
  }

  // The shares of waves 1..3 into LDS; wave 0 adds them and finishes.
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < CONV_NT; ++t) {
      red[wave - 1][2 * t][lane] = acc[t];
      red[wave - 1][2 * t + 1][lane] = wsum[t];
    }
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < CONV_WAVES - 1; ++w)
#pragma unroll
    for (int t = 0; t < CONV_NT; ++t) {
      acc[t] += red[w][2 * t][lane];
      wsum[t] += red[w][2 * t + 1][lane];
    }

  // Epilogue: lane l holds pixels 4 * (l / 16) + [0, 4) of channel l % 16.
#pragma unroll
  for (int t = 0; t < CONV_NT; ++t) {
    const int oc = oc0 + t * 16 + li;
    if (oc >= Co) continue;
    const float mult = mult_t[t];
    const int b0 = bias_t[t];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int pe = p0 + g * 4 + e;
      if (pe >= P) continue;
      // The true accumulator in 64 bits (the bias is any int32); the int32
      // partial sums are exact under the host's bound on the reduction.
      const int64_t a = (int64_t)b0 + acc[t][e] - (int64_t)in_zp * wsum[t][e];
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
  const uintptr_t align = (uintptr_t)c.X | (uintptr_t)c.Wt;
  auto kern = ((c.C % 16) == 0 && (align & 15) == 0) ? conv_int8_kernel<16>
              : ((c.C % 4) == 0 && (align & 3) == 0) ? conv_int8_kernel<4>
                                                      : conv_int8_kernel<1>;
  hipLaunchKernelGGL(kern, grid, dim3(64 * CONV_WAVES), 0, c.stream, c.X, c.Wt,
                     c.bias, c.w_scale, c.in_scale, c.out_scale, c.in_zp, c.out_zp, c.clamp_min,
                     c.clamp_max, c.H, c.W, c.C, c.Co, c.KH, c.KW, c.stride_h, c.stride_w,
                     c.pad_h, c.pad_w, OH, OW, P, 1.0f / (float)c.C, 1.0f / (float)c.KW, c.Y);
  return hipGetLastError();
}

}  // namespace qmm
