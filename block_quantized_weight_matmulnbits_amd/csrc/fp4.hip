// fp4.hip -- matmuls with block-scaled FP4 weights (MXFP4, NVFP4) for gfx950.
//
// Definition (rlx-cpu quant.rs: dequant_matmul_nvfp4, lowp_dequantize):
//   w(n, k) = e2m1(code(n, k)) * scale(n, k / bs) * global_scale
//   Y[m, n] = sum_k A[m, k] * w(n, k)  (+ bias[n])
// MXFP4: bs = 32, E8M0 scale bytes (2^(e-127), 255 = nan), global scale 1.
// NVFP4: bs = 16, E4M3 scale bytes, an f32 global scale.
// Weights [N, kb, bs/2] bytes, element k of a row in byte k/2, the low nibble
// for even k; scales [N, kb] bytes.
//
// E2M1 codes are turned into values by the gfx950 conversion
// v_cvt_scalef32_pk_{bf16,f16,f32}_fp4 with a unit scale: E2M1 values (at
// most 2 significant bits) are exact in every output type, and the two values
// of a byte come out low nibble first, i.e. in element order.  Products with
// 16-bit activations are exact (v_dot2_f32_bf16 / _f16 accumulate in fp32);
// each block's sum is multiplied once by its decoded scale in fp32, and the
// global scale multiplies the result.
//
// fp4_gemv_kernel (M = 1): a wave owns R rows (output columns) and walks
// each row in wave-wide 16-byte loads (1 KiB per load, contiguous); every
// load of a piece (R rows x 2 per lane) is issued first, then each lane reads
// its units' activations straight from memory (16-byte loads; the vector
// stays in the caches, so there is no staging and no barrier).
// A lane's 16 bytes are 32 codes: one MXFP4 block or two NVFP4 blocks.
// fp4_rows_kernel (M > 1 without the matrix cores, or f32 activations): fp32
// throughout, MT rows of A per pass.
#include <algorithm>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int F4_LPC = 2;          // 16-byte units per lane, row and piece
constexpr int F4_CHUNK = 64 * F4_LPC * 32;   // activations staged per piece (4096)

// d + the products of the two E2M1 values of byte B of word w (low nibble =
// the even element) with activations x (16-bit pair word xp, or fp32 words
// x0, x1).
template <int XDT, int B>
__device__ __forceinline__ float fp4_pair_dot(uint32_t w, const uint32_t* x, int e, float d) {
  if constexpr (XDT == DT_BF16) {
    const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
    return __builtin_amdgcn_fdot2_f32_bf16(c, __builtin_bit_cast(bf16x2_t, x[e]), d, false);
  } else if constexpr (XDT == DT_F16) {
    const half2_t c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
    return __builtin_amdgcn_fdot2(c, as_half2(x[e]), d, false);
  } else {
    const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
    d = fmaf(c.x, __uint_as_float(x[2 * e]), d);
    return fmaf(c.y, __uint_as_float(x[2 * e + 1]), d);
  }
}

// Sum over the 32 codes of 16 bytes (v) times 32 activations (x, natural
// order, 16-bit pairs or fp32) for the two 16-code halves: out[0] covers
// bytes 0-7, out[1] bytes 8-15.
template <int XDT>
__device__ __forceinline__ void fp4_dot32(const u32x4& v, const uint32_t* x, float (&out)[2]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    float d = 0.0f;
#pragma unroll
    for (int wi = 2 * h; wi < 2 * h + 2; ++wi) {
      d = fp4_pair_dot<XDT, 0>(w[wi], x, wi * 4 + 0, d);
      d = fp4_pair_dot<XDT, 1>(w[wi], x, wi * 4 + 1, d);
      d = fp4_pair_dot<XDT, 2>(w[wi], x, wi * 4 + 2, d);
      d = fp4_pair_dot<XDT, 3>(w[wi], x, wi * 4 + 3, d);
    }
    out[h] = d;
  }
}

// Rows (output columns) per wave: fewer rows, more waves in flight (measured
// on 4096 x 14336: MXFP4 8 -> 4 rows 11.0 -> 9.7 us, NVFP4 8 -> 2 rows
// 13.1 -> 10.8 us, with its two scale bytes per unit).
template <int FMT>
constexpr int f4_rows() { return FMT == FP4_MX ? 4 : 2; }

template <int XDT, int FMT>
__global__ __launch_bounds__(256) void fp4_gemv_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ W, const uint8_t* __restrict__ scales,
    float global_scale, const void* __restrict__ bias, void* __restrict__ y, int K, int N,
    int kb) {
  constexpr int BS = FMT == FP4_MX ? 32 : 16;
  constexpr int XW = XDT == DT_F32 ? 32 : 16;          // 32-bit words of x per 32 codes
  using XT = typename dt<XDT>::T;
  // 16-byte activation loads when every 32-code unit is wholly inside or
  // wholly past K and x is 16-byte aligned.
  const bool xvec = (K % 32) == 0 && (((uintptr_t)x) & 15) == 0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * 4 + wave) * f4_rows<FMT>();
  const int row_bytes = kb * BS / 2;                    // a multiple of 8
  const int row_units = (row_bytes + 15) / 16;          // 16-byte units (the last may be half)
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, 0, N * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, N * kb, 0x00020000);
  float acc[f4_rows<FMT>()];
#pragma unroll
  for (int r = 0; r < f4_rows<FMT>(); ++r) acc[r] = 0.0f;

  for (int u0 = 0; u0 < row_units; u0 += F4_CHUNK / 32) {
    // Every load of the piece in flight first (the wave's rows x F4_LPC units per
    // lane, unit u0 + lane + 64 j; they do not depend on the staged
    // activations), then the activations staged.  Units past the row are
    // not loaded (a uniform skip when the whole wave is past it) or read
    // zeros through an out-of-range offset, and are not consumed.
    u32x4 cv[f4_rows<FMT>()][F4_LPC];
    uint32_t sv[f4_rows<FMT>()][F4_LPC], sv2[f4_rows<FMT>()][F4_LPC];
#pragma unroll
    for (int j = 0; j < F4_LPC; ++j) {
      const int u = u0 + lane + 64 * j;
      const bool live = u < row_units;
#pragma unroll
      for (int r = 0; r < f4_rows<FMT>(); ++r) {
        cv[r][j] = u32x4{0u, 0u, 0u, 0u};
        sv[r][j] = sv2[r][j] = 0u;
      }
      if (u0 + 64 * j >= row_units) continue;
#pragma unroll
      for (int r = 0; r < f4_rows<FMT>(); ++r) {
        const int n = n0 + r;
        const bool ok = live && n < N;
        cv[r][j] = __builtin_amdgcn_raw_buffer_load_b128(
            rw, ok ? n * row_bytes + u * 16 : 0x7FFFFFF0, 0, BUF_STREAM);
        // MXFP4: one scale per unit; NVFP4: two (bytes 2u and 2u + 1).
        const int sb = n * kb + (FMT == FP4_MX ? u : 2 * u);
        sv[r][j] = __builtin_amdgcn_raw_buffer_load_b8(rsc, ok ? sb : 0x7FFFFFF0, 0, 0);
        if constexpr (FMT != FP4_MX)
          sv2[r][j] = __builtin_amdgcn_raw_buffer_load_b8(rsc, ok ? sb + 1 : 0x7FFFFFF0, 0, 0);
      }
    }
    // Each lane's activations for its units, read straight from memory (the
    // vector stays in the caches; zero past K): no staging, no barrier.
    uint32_t xv[F4_LPC][XW];
#pragma unroll
    for (int j = 0; j < F4_LPC; ++j) {
      const int u = u0 + lane + 64 * j;
      const int k0 = u * 32;
      if (xvec) {
        const bool in = k0 < K;
        const u32x4* xp = reinterpret_cast<const u32x4*>(reinterpret_cast<const XT*>(x) + (in ? k0 : 0));
#pragma unroll
        for (int v = 0; v < XW / 4; ++v) {
          const u32x4 t = xp[v];
          xv[j][4 * v + 0] = in ? t.x : 0u;
          xv[j][4 * v + 1] = in ? t.y : 0u;
          xv[j][4 * v + 2] = in ? t.z : 0u;
          xv[j][4 * v + 3] = in ? t.w : 0u;
        }
      } else {
#pragma unroll
        for (int t = 0; t < XW; ++t) {
          uint32_t v = 0;
          if constexpr (XDT == DT_F32) {
            const int k = k0 + t;
            if (k < K) v = __float_as_uint(reinterpret_cast<const float*>(x)[k]);
          } else {
            const int k = k0 + 2 * t;
            const XT* xp = reinterpret_cast<const XT*>(x);
            const uint32_t lo = k < K ? __builtin_bit_cast(uint16_t, xp[k]) : 0u;
            const uint32_t hi = k + 1 < K ? __builtin_bit_cast(uint16_t, xp[k + 1]) : 0u;
            v = lo | (hi << 16);
          }
          xv[j][t] = v;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < F4_LPC; ++j) {
      const int u = u0 + lane + 64 * j;
      if (u >= row_units) break;
      const uint32_t* xl = xv[j];
#pragma unroll
      for (int r = 0; r < f4_rows<FMT>(); ++r) {
        float d[2];
        fp4_dot32<XDT>(cv[r][j], xl, d);
        if (FMT == FP4_MX) {
          acc[r] = fmaf(d[0] + d[1], fp4_scale(sv[r][j], FMT), acc[r]);
        } else {
          // The second half of the last unit of a row with an odd number of
          // blocks is past the row (its activations are zero; no scale).
          acc[r] = fmaf(d[0], fp4_scale(sv[r][j], FMT), acc[r]);
          if (2 * u + 1 < kb) acc[r] = fmaf(d[1], fp4_scale(sv2[r][j], FMT), acc[r]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < f4_rows<FMT>(); ++r) {
    const float v = wave_sum(acc[r]);
    const int n = n0 + r;
    if (lane == 0 && n < N) {
      float o = v * global_scale;
      if (bias) o += dt<XDT>::to_f32(reinterpret_cast<const XT*>(bias)[n]);
      reinterpret_cast<XT*>(y)[n] = dt<XDT>::from_f32(o);
    }
  }
}

// fp32 rows: MT rows of A per pass, a wave per R output columns, lanes
// striding over the row's bytes (two codes each).
template <int XDT, int FMT, int MT>
__global__ __launch_bounds__(256) void fp4_rows_kernel(
    const void* __restrict__ A, const uint8_t* __restrict__ W, const uint8_t* __restrict__ scales,
    float global_scale, const void* __restrict__ bias, void* __restrict__ Y, int Mp, int K, int N,
    int kb) {
  constexpr int BS = FMT == FP4_MX ? 32 : 16;
  constexpr int CH = 1024;
  using XT = typename dt<XDT>::T;
  __shared__ float xs[MT][CH];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * 4 + wave) * 2;
  const int row_bytes = kb * BS / 2;
  float acc[2][MT];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += CH) {
    __syncthreads();
    for (int t = threadIdx.x; t < CH; t += 256) {
      const int k = k0 + t;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xs[m][t] = (k < K && m < Mp)
                       ? dt<XDT>::to_f32(reinterpret_cast<const XT*>(A)[(int64_t)m * K + k])
                       : 0.0f;
    }
    __syncthreads();
    for (int e = lane; 2 * e < min(CH, K - k0); e += 64) {
      const int k = k0 + 2 * e;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int n = n0 + r;
        if (n >= N) continue;
        const uint32_t byte = W[(int64_t)n * row_bytes + k / 2];
        const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(byte, 1.0f, 0);
        const float s = fp4_scale(scales[(int64_t)n * kb + k / BS], FMT);
        const float w0 = c.x * s, w1 = c.y * s;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          acc[r][m] = fmaf(xs[m][2 * e], w0, acc[r][m]);
          acc[r][m] = fmaf(xs[m][2 * e + 1], w1, acc[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      const int n = n0 + r;
      if (lane == 0 && n < N && m < Mp) {
        float o = v * global_scale;
        if (bias) o += dt<XDT>::to_f32(reinterpret_cast<const XT*>(bias)[n]);
        reinterpret_cast<XT*>(Y)[(int64_t)m * N + n] = dt<XDT>::from_f32(o);
      }
    }
}

template <int XDT, int FMT>
hipError_t launch_fp4_t(const Fp4Args& a) {
  using XT = typename dt<XDT>::T;
  if (a.M == 1) {
    const int grid = (int)((a.N + 4 * f4_rows<FMT>() - 1) / (4 * f4_rows<FMT>()));
    hipLaunchKernelGGL((fp4_gemv_kernel<XDT, FMT>), dim3(grid), dim3(256), 0, a.stream, a.A, a.W,
                       a.scales, a.global_scale, a.bias, a.Y, (int)a.K, (int)a.N, (int)a.kb);
    return hipGetLastError();
  }
  if (gemm_skinny_fp4_supported(a)) return launch_gemm_skinny_fp4(a);
  if (gemm_mfma_fp4_supported(a)) return launch_gemm_mfma_fp4(a);
  constexpr int MT = 8;
  const int grid = (int)((a.N + 7) / 8);
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    hipLaunchKernelGGL((fp4_rows_kernel<XDT, FMT, MT>), dim3(grid), dim3(256), 0, a.stream,
                       (const XT*)a.A + m0 * a.K, a.W, a.scales, a.global_scale, a.bias,
                       (XT*)a.Y + m0 * a.N, Mp, (int)a.K, (int)a.N, (int)a.kb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int XDT>
hipError_t launch_fp4_x(const Fp4Args& a) {
  return a.format == FP4_MX ? launch_fp4_t<XDT, FP4_MX>(a)
                                : launch_fp4_t<XDT, FP4_NV>(a);
}

}  // namespace

hipError_t launch_fp4(const Fp4Args& a) {
  switch (a.a_dtype) {
    case DT_F32: return launch_fp4_x<DT_F32>(a);
    case DT_F16: return launch_fp4_x<DT_F16>(a);
    default: return launch_fp4_x<DT_BF16>(a);
  }
}

}  // namespace qmm
