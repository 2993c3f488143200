// gidx.hip -- MatMulNBits with group indices (g_idx, act-order) on the
// operator's layout, for gfx950.
//
// Definition (onnx-runtime-ep-cpu matmul_nbits.rs, the group-index branch of
// dequantize_weight): element k keeps its code from block k / bs of its row,
// but its scale and zero point are those of group g = g_idx[k]:
//   w(n, k) = (code(n, k) - zp(n, g)) * scale[n, g],  Y[m, n] = sum_k A[m, k] w(n, k).
// The scale changes from element to element in an arbitrary pattern, so the
// per-block factoring of the other kernels does not apply: every code is
// dequantized on its own, in fp32 ((code - zp) * scale is exact in fp32 for
// 16-bit scales), and multiplied into fp32 accumulators.
//
// gidx_rows_kernel: a workgroup of 4 waves owns 4 * R output columns; for
// each chunk of CH elements of K it stages MT rows of A (as fp32) and the
// chunk's group indices (clamped into 0..kb-1, so that an out-of-range entry
// reads in bounds) in LDS; the lanes of a wave walk the chunk's 32-bit words
// of codes of each of its columns (adjacent lanes, adjacent words), look up
// each code's scale and zero point in the column's rows (cached reads) and
// accumulate.  Used for every M with f32 activations and for M <= 16
// otherwise; larger M with 16-bit activations runs the matrix-core GEMM
// with the same lookups (gemm.hip).
#include <algorithm>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int GI_CH = 1024;   // K elements per LDS chunk

template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, int MT>
__global__ __launch_bounds__(256) void gidx_rows_kernel(
    const typename dt<XDT>::T* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ g_idx, const typename dt<XDT>::T* __restrict__ bias,
    typename dt<XDT>::T* __restrict__ Y, int Mp, int K, int N, int kb, int row_bytes,
    int zp_row_bytes) {
  constexpr int P = 32 / BITS;                           // codes per word
  constexpr uint32_t cm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  __shared__ float xs[MT][GI_CH];
  __shared__ int gs[GI_CH];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col0 = (blockIdx.x * 4 + wave) * R;
  const int ncols = max(0, min(R, N - col0));
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  // Words of a row that hold codes below K.
  const int kwords = (K + P - 1) / P;
  for (int k0 = 0; k0 < K; k0 += GI_CH) {
    __syncthreads();
    for (int t = threadIdx.x; t < GI_CH; t += 256) {
      const int k = k0 + t;
      const bool in = k < K;
      gs[t] = in ? min(max(g_idx[k], 0), kb - 1) : 0;
#pragma unroll
      for (int m = 0; m < MT; ++m)
        xs[m][t] = (in && m < Mp) ? dt<XDT>::to_f32(A[(int64_t)m * K + k]) : 0.0f;
    }
    __syncthreads();
    const int w0 = k0 / P, w1 = min(kwords, (k0 + GI_CH) / P);
    for (int w = w0 + lane; w < w1; w += 64) {
      const int e0 = w * P - k0;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= ncols) continue;
        const int64_t n = col0 + r;
        const uint32_t cwd = reinterpret_cast<const uint32_t*>(B + n * row_bytes)[w];
        const typename dt<SDT>::T* srow = scales + n * kb;
        const uint8_t* zrow = zp + n * zp_row_bytes;
#pragma unroll
        for (int j = 0; j < P; ++j) {
          // Codes past K (the tail of the last block) meet zero activations.
          const int g = gs[e0 + j];
          const float s = dt<SDT>::to_f32(srow[g]);
          const int z = (int)load_zp<BITS, HAS_ZP>(zrow, g);
          const float wv = (float)((int)((cwd >> (j * BITS)) & cm) - z) * s;
#pragma unroll
          for (int m = 0; m < MT; ++m) acc[r][m] = fmaf(xs[m][e0 + j], wv, acc[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0 && r < ncols && m < Mp) {
        float o = v;
        if (bias) o += dt<XDT>::to_f32(bias[col0 + r]);
        Y[(int64_t)m * N + col0 + r] = dt<XDT>::from_f32(o);
      }
    }
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t launch_rows_t(const MatArgs& a) {
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  constexpr int R = 2;
  const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
  // One row per pass for M = 1 (no idle accumulators), else 8.
  if (a.M == 1) {
    hipLaunchKernelGGL((gidx_rows_kernel<BITS, XDT, SDT, HAS_ZP, R, 1>), dim3(grid), dim3(256),
                       0, a.stream, (const XT*)a.A, a.B, (const ST*)a.scales, a.zp, a.g_idx,
                       (const XT*)a.bias, (XT*)a.Y, 1, (int)a.K, (int)a.N, (int)a.kb,
                       (int)(a.kb * a.blob), (int)a.zp_row_bytes);
    return hipGetLastError();
  }
  constexpr int MT = 8;
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    hipLaunchKernelGGL((gidx_rows_kernel<BITS, XDT, SDT, HAS_ZP, R, MT>), dim3(grid), dim3(256),
                       0, a.stream, (const XT*)a.A + m0 * a.K, a.B, (const ST*)a.scales, a.zp,
                       a.g_idx, (const XT*)a.bias, (XT*)a.Y + m0 * a.N, Mp, (int)a.K, (int)a.N,
                       (int)a.kb, (int)(a.kb * a.blob), (int)a.zp_row_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int XDT, int SDT>
hipError_t launch_rows_z(const MatArgs& a) {
  return a.zp ? launch_rows_t<BITS, XDT, SDT, true>(a) : launch_rows_t<BITS, XDT, SDT, false>(a);
}

template <int BITS, int XDT>
hipError_t launch_rows_s(const MatArgs& a) {
  switch (a.s_dtype) {
    case DT_F32: return launch_rows_z<BITS, XDT, DT_F32>(a);
    case DT_F16: return launch_rows_z<BITS, XDT, DT_F16>(a);
    default: return launch_rows_z<BITS, XDT, DT_BF16>(a);
  }
}

template <int BITS>
hipError_t launch_rows_x(const MatArgs& a) {
  switch (a.a_dtype) {
    case DT_F32: return launch_rows_s<BITS, DT_F32>(a);
    case DT_F16: return launch_rows_s<BITS, DT_F16>(a);
    default: return launch_rows_s<BITS, DT_BF16>(a);
  }
}

}  // namespace

hipError_t launch_gidx(const MatArgs& a) {
  if (gemm_mfma_gidx_supported(a)) return launch_gemm_mfma_gidx(a);
  switch (a.bits) {
    case 2: return launch_rows_x<2>(a);
    case 4: return launch_rows_x<4>(a);
    default: return launch_rows_x<8>(a);
  }
}

}  // namespace qmm
