// gemm.hip -- batched / prefill matmul over block-quantized weights for gfx950.
//
// Y[M, N] = A[M, K] * W^T with W[n, k] = (code - zp) * scale (onnx-runtime-ep-cpu
// matmul_nbits.rs: the batched route dequantizes then multiplies; here the
// weight is dequantized tile by tile inside the kernel and never written to
// memory).
//
// gemm_mfma_kernel (bf16 / f16 activations): a workgroup of 4 waves computes a
// BM x BN = 256 x 256 tile of Y, each wave 128 x 128 as 8 x 8
// v_mfma_f32_16x16x32_{bf16,f16} tiles accumulated in fp32.  Per K-step of
// BK = 32: the A tile is copied to LDS, the B tile is dequantized once for
// the whole workgroup (each thread one output column: unpack codes, subtract
// the zero point, multiply by the block scale in fp32, round to the activation
// dtype) and stored to LDS; then every wave reads its operand fragments from
// LDS.  LDS rows are padded by 16 bytes so the fragment reads of 16 rows fall
// in distinct banks.  Loads of A and of the codes go through buffer
// descriptors whose extents end at M, K and N, so ragged edges read zeros.
//
// gemm_rows_kernel (fallback: f32 activations, small M, unaligned operands):
// fp32 throughout -- each wave owns R output columns, stages MT rows of A in
// LDS as fp32 and accumulates exact (code - zp) * x products per block in fp32
// before scaling.
#include <algorithm>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int GEMM_THREADS = 256;
constexpr int GBM = 256, GBN = 256, GBK = 32;
constexpr int LDS_ROW = GBK + 8;             // padded row, in 16-bit elements
constexpr int BUF_WORD3 = 0x00020000;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int XDT> struct MfmaOp;
template <> struct MfmaOp<DT_BF16> {
  using V = bf16x8;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint16_t round(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
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
};

// ---------------------------------------------------------------------------
// MFMA kernel.  Requirements checked by the launcher: K % 8 == 0 and A 16-byte
// aligned (A rows are read as 16-byte chunks of 8 activations).
// ---------------------------------------------------------------------------
template <int BITS, int XDT, int SDT, bool HAS_ZP>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int K, int N, int kb,
    int log2_bs, int log2_blob, int zp_row_bytes, int tiles_n) {
  using Op = MfmaOp<XDT>;
  using ST = typename dt<SDT>::T;
  constexpr int P = 32 / BITS;                 // codes per 32-bit word
  constexpr int WPS = GBK / P;                 // code words per column per K-step
  __shared__ __attribute__((aligned(16))) uint16_t As[GBM * LDS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[GBN * LDS_ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int m0 = tile_m * GBM, n0 = tile_n * GBN;
  const int wm = (wave >> 1) * 128, wn = (wave & 1) * 128;

  // Whole-matrix descriptors; rows past M read zeros through the extent.
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, 0, (int)std::min<int64_t>((int64_t)M * K * 2, 0x7FFFFFFF), BUF_WORD3);
  const int64_t row_bytes = (int64_t)kb << log2_blob;
  // This thread's dequantization column.
  const int ncol = n0 + tid;
  const bool ncol_ok = ncol < N;
  const int nc = ncol_ok ? ncol : N - 1;
  const __amdgpu_buffer_rsrc_t rbc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (int64_t)nc * row_bytes), 0, ncol_ok ? (int)row_bytes : 0, BUF_WORD3);

  f32x4 acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += GBK) {
    // ---- A tile: 256 rows x 32 activations = 1024 chunks of 8; 4 per thread.
    u32x4 av[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * GEMM_THREADS;
      const int r = c >> 2, kc = (c & 3) * 8;
      const int row = m0 + r, k = k0 + kc;
      const bool ok = row < M && k < K;      // K % 8 == 0: a chunk is all in or all out
      const int off = ok ? (row * K + k) * 2 : 0x7FFFFFF0;
      av[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 0);
    }
    // ---- B codes of this thread's column for k in [k0, k0 + 32).
    uint32_t cw[WPS];
    const int byte0 = (k0 * BITS) >> 3;
#pragma unroll
    for (int w = 0; w < WPS; ++w) cw[w] = __builtin_amdgcn_raw_buffer_load_b32(rbc, byte0 + 4 * w, 0, 0);

    __syncthreads();   // previous K-step's fragment reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * GEMM_THREADS;
      const int r = c >> 2, kc = (c & 3) * 8;
      *reinterpret_cast<u32x4*>(&As[r * LDS_ROW + kc]) = av[i];
    }
    // Dequantize: each word lies inside one block.
    uint16_t wq[GBK];
#pragma unroll
    for (int w = 0; w < WPS; ++w) {
      const int kw = k0 + w * P;
      const int blk = min(kw >> log2_bs, kb - 1);
      float s = 0.0f;
      uint32_t z = 1u << (BITS - 1);
      if (ncol_ok) {
        s = dt<SDT>::to_f32(scales[(int64_t)ncol * kb + blk]);
        if constexpr (HAS_ZP) {
          constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
          const int zbit = blk * BITS;
          z = ((uint32_t)zp[(int64_t)ncol * zp_row_bytes + (zbit >> 3)] >> (zbit & 7)) & zm;
        }
      }
      const float zs = (float)z * s;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        constexpr uint32_t cm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
        const float q = (float)((cw[w] >> (j * BITS)) & cm);
        // (q - z) * s as q * s - z * s: both products exact, one rounding.
        wq[w * P + j] = Op::round(fmaf(q, s, -zs));
      }
    }
#pragma unroll
    for (int j = 0; j < GBK / 8; ++j) {
      u32x4 t;
      t.x = wq[8 * j + 0] | ((uint32_t)wq[8 * j + 1] << 16);
      t.y = wq[8 * j + 2] | ((uint32_t)wq[8 * j + 3] << 16);
      t.z = wq[8 * j + 4] | ((uint32_t)wq[8 * j + 5] << 16);
      t.w = wq[8 * j + 6] | ((uint32_t)wq[8 * j + 7] << 16);
      *reinterpret_cast<u32x4*>(&Bs[tid * LDS_ROW + 8 * j]) = t;
    }
    __syncthreads();

    // ---- MFMA: lane l takes row/column (l % 16) and activations
    // [8 * (l / 16), +8) of the 32-wide K-step.
    const int fr = lane & 15, fk = (lane >> 4) * 8;
    typename Op::V bf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      bf[j] = __builtin_bit_cast(typename Op::V,
                                 *reinterpret_cast<const u32x4*>(&Bs[(wn + j * 16 + fr) * LDS_ROW + fk]));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const typename Op::V af = __builtin_bit_cast(
          typename Op::V, *reinterpret_cast<const u32x4*>(&As[(wm + i * 16 + fr) * LDS_ROW + fk]));
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = Op::run(af, bf[j], acc[i][j]);
    }
  }

  // ---- Epilogue: lane l holds rows 4 * (l / 16) + [0, 4) of column l % 16 of
  // each 16 x 16 tile.
  const int cc = lane & 15, rr = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int n = n0 + wn + j * 16 + cc;
    if (n >= N) continue;
    const float bv = bias ? bits16_to_f32<XDT>(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm + i * 16 + rr + e;
        if (m < M) Y[(int64_t)m * N + n] = Op::round(acc[i][j][e] + bv);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fallback: fp32 multi-row kernel.  MT rows of A per launch pass (the host
// offsets A and Y), R output columns per wave, lanes stride over 32-bit words
// of codes.  Exact (code - zp) times fp32 activations, fp32 accumulation per
// block, then the block scale.
// ---------------------------------------------------------------------------
constexpr int ROWS_CHUNK = 2048;   // activations per LDS chunk and row

template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, int MT>
__global__ __launch_bounds__(256) void gemm_rows_kernel(
    const typename dt<XDT>::T* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const typename dt<XDT>::T* __restrict__ bias, typename dt<XDT>::T* __restrict__ Y, int Mp,
    int K, int N, int kb, int log2_blob, int zp_row_bytes) {
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
        const uint32_t cwd = reinterpret_cast<const uint32_t*>(B + (int64_t)n * row_bytes)[w];
        const float s = dt<SDT>::to_f32(scales[(int64_t)n * kb + blk]);
        const int z = (int)load_zp<BITS, HAS_ZP>(zp + (int64_t)n * zp_row_bytes, blk);
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
static int ilog2i(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_rows(const MatArgs& a) {
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  constexpr int MT = 8, R = 2;
  const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    hipLaunchKernelGGL((gemm_rows_kernel<BITS, XDT, SDT, HAS_ZP, R, MT>), dim3(grid), dim3(256),
                       0, a.stream, (const XT*)a.A + m0 * a.K, a.B, (const ST*)a.scales, a.zp,
                       (const XT*)a.bias, (XT*)a.Y + m0 * a.N, Mp, (int)a.K, (int)a.N,
                       (int)a.kb, ilog2i(a.blob), (int)a.zp_row_bytes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_gemm_t(const MatArgs& a) {
  using ST = typename dt<SDT>::T;
  const bool mfma_ok = XDT != DT_F32 && a.M > 16 && (a.K % 8) == 0 &&
                       ((uintptr_t)a.A & 15) == 0 && a.M * a.K * 2 < 0x7FFFFFF0LL;
  if constexpr (XDT != DT_F32) {
    if (mfma_ok) {
      const int tiles_m = (int)((a.M + GBM - 1) / GBM), tiles_n = (int)((a.N + GBN - 1) / GBN);
      hipLaunchKernelGGL((gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP>), dim3(tiles_m * tiles_n),
                         dim3(GEMM_THREADS), 0, a.stream, (const uint16_t*)a.A, a.B,
                         (const ST*)a.scales, a.zp, (const uint16_t*)a.bias, (uint16_t*)a.Y,
                         (int)a.M, (int)a.K, (int)a.N, (int)a.kb, ilog2i(a.block_size),
                         ilog2i(a.blob), (int)a.zp_row_bytes, tiles_n);
      return hipGetLastError();
    }
  }
  return launch_rows<BITS, XDT, SDT, HAS_ZP>(a);
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

hipError_t launch_gemm(const MatArgs& a) {
  switch (a.bits) {
    case 2: return launch_gemm_x<2>(a);
    case 4: return launch_gemm_x<4>(a);
    default: return launch_gemm_x<8>(a);
  }
}

}  // namespace qmm
