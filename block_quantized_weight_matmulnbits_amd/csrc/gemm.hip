// gemm.hip -- batched / prefill matmul over block-quantized weights for gfx950:
// the routing of qmm_gemm, the 256-row matrix-core kernel's 224- and
// 256-column instances (template in gemm_mfma.h; 64- and 128-column ones in
// gemm_narrow.hip), its group-index and FP4 variants, and the fp32 row
// kernel.
//
// Y[M, N] = A[M, K] * W^T with W[n, k] = (code - zp) * scale (onnx-runtime-ep-cpu
// matmul_nbits.rs: the batched route dequantizes then multiplies; here the
// weight is dequantized tile by tile inside the kernels and never written to
// memory).
//
// Routes (launch_gemm): group indices -> gidx.hip; 16-bit activations with
// K % 8 == 0 -> the few-row kernel (gemm_skinny.hip) when M <= 16 or its
// grid has at most 1024 workgroups, else gemm_mfma_kernel with the narrowest
// column tile whose grid still fits one round of the compute units (64 / 128
// columns) or 224 / 256 columns; otherwise (f32 activations, K % 8 != 0,
// offsets past 2^31) gemm_rows_kernel, fp32 throughout -- each wave owns R
// output columns, stages MT rows of A in LDS as fp32 and accumulates exact
// (code - zp) * x products per block in fp32 before scaling (3-bit weights:
// the generic kernel).
#include <algorithm>
#include <type_traits>

#include "gemm_mfma.h"

namespace qmm {

// ---------------------------------------------------------------------------
// Fallback: fp32 multi-row kernel.  MT rows of A per launch pass (the host
// offsets A and Y), R output columns per wave, lanes stride over 32-bit words
// of codes.  Exact (code - zp) times fp32 activations, fp32 accumulation per
// block, then the block scale.
// ---------------------------------------------------------------------------
constexpr int ROWS_CHUNK = 2048;   // activations per LDS chunk and row

template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, int MT, bool TL>
__global__ __launch_bounds__(256) void gemm_rows_kernel(
    const typename dt<XDT>::T* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const typename dt<XDT>::T* __restrict__ bias, typename dt<XDT>::T* __restrict__ Y, int Mp,
    int K, int N, int kb, int log2_blob, int zp_row_bytes, int chunks) {
  constexpr int P = 32 / BITS;
  __shared__ float xs[MT * ROWS_CHUNK];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int nrows = max(0, min(R, N - row0));
  const int64_t row_bytes = (int64_t)kb << log2_blob;
  const int row_words = (int)(row_bytes >> 2);
  const int blob_words_log2 = log2_blob - 2;
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  constexpr int CW = ROWS_CHUNK / P;   // code words per chunk
  for (int w0 = 0; w0 < row_words; w0 += CW) {
    const int w1 = min(row_words, w0 + CW);
    __syncthreads();
    for (int t = threadIdx.x; t < MT * ROWS_CHUNK; t += 256) {
      const int m = t / ROWS_CHUNK, e = t % ROWS_CHUNK;
      const int k = w0 * P + e;
      xs[t] = (m < Mp && k < K) ? dt<XDT>::to_f32(A[(int64_t)m * K + k]) : 0.0f;
    }
    __syncthreads();
    for (int w = w0 + lane; w < w1; w += 64) {
      const int blk = w >> blob_words_log2;
      const int e0 = (w - w0) * P;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (r >= nrows) continue;
        const int n = row0 + r;
        uint32_t cwd;
        float s;
        int z = 1 << (BITS - 1);
        if constexpr (TL) {
          // Tiled layout (qmm_layout.h): word w of the row lies in chunk
          // w / chunk_words of group n / 32, column n % 32.
          constexpr int CW = TKC * BITS / 32;     // words per column chunk
          const int64_t g = n / TG, i = n % TG;
          cwd = reinterpret_cast<const uint32_t*>(B)[((g * chunks + w / CW) * TG + i) * CW + w % CW];
          const int64_t si = (g * kb + blk) * TG + i;
          s = dt<SDT>::to_f32(scales[si]);
          if constexpr (HAS_ZP) {
            constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
            const int64_t bit = si * BITS;
            z = (int)(((uint32_t)zp[bit >> 3] >> (bit & 7)) & zm);
          }
        } else {
          cwd = reinterpret_cast<const uint32_t*>(B + (int64_t)n * row_bytes)[w];
          s = dt<SDT>::to_f32(scales[(int64_t)n * kb + blk]);
          z = (int)load_zp<BITS, HAS_ZP>(zp + (int64_t)n * zp_row_bytes, blk);
        }
        float qz[P];
#pragma unroll
        for (int j = 0; j < P; ++j) {
          constexpr uint32_t cm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
          qz[j] = (float)((int)((cwd >> (j * BITS)) & cm) - z);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          float d = 0.0f;
#pragma unroll
          for (int j = 0; j < P; ++j) d = fmaf(xs[m * ROWS_CHUNK + e0 + j], qz[j], d);
          acc[r][m] = fmaf(d, s, acc[r][m]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      if (lane == 0 && r < nrows && m < Mp) {
        float o = v;
        if (bias) o += dt<XDT>::to_f32(bias[row0 + r]);
        Y[(int64_t)m * N + row0 + r] = dt<XDT>::from_f32(o);
      }
    }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_rows(const MatArgs& a) {
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  constexpr int MT = 8, R = 2;
  const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    auto kern = a.tiled ? gemm_rows_kernel<BITS, XDT, SDT, HAS_ZP, R, MT, true>
                        : gemm_rows_kernel<BITS, XDT, SDT, HAS_ZP, R, MT, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, a.stream, (const XT*)a.A + m0 * a.K, a.B,
                       (const ST*)a.scales, a.zp, (const XT*)a.bias, (XT*)a.Y + m0 * a.N, Mp,
                       (int)a.K, (int)a.N, (int)a.kb, ilog2i(a.blob), (int)a.zp_row_bytes,
                       (int)a.chunks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Every buffer offset of the MFMA kernel must fit in 31 bits.
// Shapes the 256-row kernel takes: 16-bit activations, K % 8 == 0, A 16-byte
// aligned, every byte offset below 2^31 (with a column tile's slack past N).
static bool mfma_shape_fits(const MatArgs& a) {
  const int64_t sz = a.s_dtype == DT_F32 ? 4 : 2;
  return a.a_dtype != DT_F32 && (a.K % 8) == 0 && ((uintptr_t)a.A & 15) == 0 &&
         a.M * a.K * 2 < 0x7FFFFF00LL && (a.N + 32) * a.kb * a.blob + 256 < 0x7FFFFF00LL &&
         (a.N + 32) * (a.chunks + 2) * 64 * a.bits / 8 < 0x7FFFFF00LL &&
         (a.N + 256) * a.kb * sz < 0x7FFFFF00LL && (a.N + 256) * a.zp_row_bytes < 0x7FFFFF00LL &&
         a.K * 4 < 0x7FFFFF00LL;
}

static bool mfma_fits(const MatArgs& a) { return a.M > 16 && mfma_shape_fits(a); }

template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_gemm_t(const MatArgs& a) {
  if constexpr (XDT != DT_F32) {
    if (mfma_fits(a)) {
      // Column tiles: the narrowest of 64 and 128 columns whose workgroups
      // still fit in one round over the compute units (each workgroup walks
      // all of K, so a short grid leaves units idle), else 224 columns when
      // they divide N evenly (no partial tiles), else 256.
      const int tiles_m = (int)((a.M + GBM - 1) / GBM);
      const auto groups = [&](int bn) { return tiles_m * ((a.N + bn - 1) / bn); };
      if (groups(64) <= GEMM_FULL_ROUND) return launch_gemm_narrow(a, tiles_m, 2);
      if (groups(128) <= GEMM_FULL_ROUND) return launch_gemm_narrow(a, tiles_m, 4);
      if ((a.N % 224) == 0) return launch_mfma_tn<BITS, XDT, SDT, HAS_ZP, 7>(a, tiles_m);
      return launch_mfma_tn<BITS, XDT, SDT, HAS_ZP, 8>(a, tiles_m);
    }
  }
  if constexpr (BITS == 3) return launch_generic_float(a);
  else return launch_rows<BITS, XDT, SDT, HAS_ZP>(a);
}

template <int BITS, int XDT, int SDT>
static hipError_t launch_gemm_z(const MatArgs& a) {
  return a.zp ? launch_gemm_t<BITS, XDT, SDT, true>(a) : launch_gemm_t<BITS, XDT, SDT, false>(a);
}

template <int BITS, int XDT>
static hipError_t launch_gemm_s(const MatArgs& a) {
  switch (a.s_dtype) {
    case DT_F32: return launch_gemm_z<BITS, XDT, DT_F32>(a);
    case DT_F16: return launch_gemm_z<BITS, XDT, DT_F16>(a);
    default: return launch_gemm_z<BITS, XDT, DT_BF16>(a);
  }
}

template <int BITS>
static hipError_t launch_gemm_x(const MatArgs& a) {
  switch (a.a_dtype) {
    case DT_F32: return launch_gemm_s<BITS, DT_F32>(a);
    case DT_F16: return launch_gemm_s<BITS, DT_F16>(a);
    default: return launch_gemm_s<BITS, DT_BF16>(a);
  }
}

// Group indices on the matrix cores: 256-column tiles, operator layout.
template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_gidx_t(const MatArgs& a) {
  using ST = typename dt<SDT>::T;
  const int tiles_m = (int)((a.M + GBM - 1) / GBM), tiles_n = (int)((a.N + GBN - 1) / GBN);
  constexpr size_t lds = mfma_lds_bytes<GBN>();
  auto kern = gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, 8, false, 1>;
  const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(GEMM_TPB), lds, a.stream,
                     (const uint16_t*)a.A, a.B, (const ST*)a.scales, a.zp,
                     (const uint16_t*)a.bias, (uint16_t*)a.Y, (int)a.M, (int)a.K, (int)a.N,
                     (int)a.kb, ilog2i(a.block_size), ilog2i(a.blob), (int)a.zp_row_bytes,
                     tiles_m, (int)a.chunks, a.g_idx, 1.0f);
  return hipGetLastError();
}

template <int BITS, int XDT>
static hipError_t launch_gidx_s(const MatArgs& a) {
  auto z = [&](auto sdt) {
    constexpr int SDT = decltype(sdt)::value;
    return a.zp ? launch_gidx_t<BITS, XDT, SDT, true>(a) : launch_gidx_t<BITS, XDT, SDT, false>(a);
  };
  switch (a.s_dtype) {
    case DT_F32: return z(std::integral_constant<int, DT_F32>{});
    case DT_F16: return z(std::integral_constant<int, DT_F16>{});
    default: return z(std::integral_constant<int, DT_BF16>{});
  }
}

template <int BITS>
static hipError_t launch_gidx_x(const MatArgs& a) {
  return a.a_dtype == DT_F16 ? launch_gidx_s<BITS, DT_F16>(a) : launch_gidx_s<BITS, DT_BF16>(a);
}

// Group indices: the tabled kernel (gidx_mfma.hip) for M >= 2 when its
// table fits in LDS beside the 64-column tiles, else, for M > 16, the
// 256-column kernel with lookups in memory.
// (Its group indices are read 16 bytes at a time: 16-byte aligned.)
static bool gidx_table_fits(const MatArgs& a, int bn) {
  return ((uintptr_t)a.g_idx & 15) == 0 &&
         (bn == 64 ? mfma_lds_bytes<64>() : mfma_lds_bytes<128>()) + gidx_table_bytes(a, bn) <= LDS_MAX;
}

bool gemm_mfma_gidx_supported(const MatArgs& a) {
  return !a.tiled && a.M >= 2 && mfma_shape_fits(a) && (a.M > 16 || gidx_table_fits(a, 64));
}

// FP4 weights on the matrix cores: the 4-bit operator-layout geometry with
// blocks of 32 (MXFP4) or 16 (NVFP4) and one scale byte per block.
static MatArgs fp4_as_mat(const Fp4Args& f) {
  MatArgs a;
  a.A = f.A; a.B = f.W; a.scales = f.scales; a.bias = f.bias; a.Y = f.Y;
  a.M = f.M; a.K = f.K; a.N = f.N; a.kb = f.kb;
  a.block_size = f.format == FP4_MX ? 32 : 16;
  a.blob = a.block_size / 2;
  a.bits = 4; a.a_dtype = f.a_dtype; a.s_dtype = DT_F32;   // 4-byte bound in mfma_fits
  a.stream = f.stream;
  return a;
}

bool gemm_mfma_fp4_supported(const Fp4Args& f) { return mfma_fits(fp4_as_mat(f)); }

template <int XDT, int WF>
static hipError_t launch_fp4_mfma_t(const Fp4Args& f) {
  const MatArgs a = fp4_as_mat(f);
  const int tiles_m = (int)((a.M + GBM - 1) / GBM), tiles_n = (int)((a.N + GBN - 1) / GBN);
  constexpr size_t lds = mfma_lds_bytes<GBN>();
  auto kern = gemm_mfma_kernel<4, XDT, DT_BF16, false, 8, false, 0, WF>;
  const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(GEMM_TPB), lds, a.stream,
                     (const uint16_t*)a.A, a.B, (const uint16_t*)a.scales, (const uint8_t*)nullptr,
                     (const uint16_t*)a.bias, (uint16_t*)a.Y, (int)a.M, (int)a.K, (int)a.N,
                     (int)a.kb, ilog2i(a.block_size), ilog2i(a.blob), 0, tiles_m, 0,
                     (const int32_t*)nullptr, f.global_scale);
  return hipGetLastError();
}

hipError_t launch_gemm_mfma_fp4(const Fp4Args& f) {
  const bool f16 = f.a_dtype == DT_F16;
  if (f.format == FP4_MX)
    return f16 ? launch_fp4_mfma_t<DT_F16, 1 + FP4_MX>(f) : launch_fp4_mfma_t<DT_BF16, 1 + FP4_MX>(f);
  return f16 ? launch_fp4_mfma_t<DT_F16, 1 + FP4_NV>(f) : launch_fp4_mfma_t<DT_BF16, 1 + FP4_NV>(f);
}

hipError_t launch_gemm_mfma_gidx(const MatArgs& a) {
  const int tiles_m = (int)((a.M + GBM - 1) / GBM);
  // 128-column tiles when their table fits and their grid still fills the
  // compute units, else 64.
  if (gidx_table_fits(a, 128) && tiles_m * ((a.N + 127) / 128) >= GEMM_FULL_ROUND)
    return launch_gidx_staged(a, tiles_m, 4);
  if (gidx_table_fits(a, 64)) return launch_gidx_staged(a, tiles_m, 2);
  switch (a.bits) {
    case 2: return launch_gidx_x<2>(a);
    case 4: return launch_gidx_x<4>(a);
    default: return launch_gidx_x<8>(a);
  }
}

hipError_t launch_gemm(const MatArgs& a) {
  if (a.g_idx) return launch_gidx(a);
  if (gemm_skinny_supported(a)) return launch_gemm_skinny(a);
  switch (a.bits) {
    case 2: return launch_gemm_x<2>(a);
    case 3: return launch_gemm_x<3>(a);
    case 4: return launch_gemm_x<4>(a);
    default: return launch_gemm_x<8>(a);
  }
}

}  // namespace qmm
