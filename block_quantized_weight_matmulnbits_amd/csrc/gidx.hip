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
// accumulate.  Used past gidx_gemv_kernel's rows with f32 activations, and
// for M <= 16 otherwise when the matrix-core GEMM's table does not fit; larger M with
// 16-bit activations runs the matrix-core GEMM with the same lookups
// (gemm.hip, gidx_mfma.hip).
//
// gidx_gemv_kernel (M <= 4 or 16, any activation dtype; MT rows per launch,
// every code dequantized once for them): a workgroup of W waves
// owns CW = 16 R output columns and cuts K into 4 W slices; lane l of wave w
// takes columns (l % 16) + 16 r and slice 4 w + l / 16.  A row of codes is
// read in 16-byte units (128 / BITS codes each): chunk ch holds 64 codes of
// every slice, slice s taking units s, s + 4 W, ... of the chunk (each load
// of a wave covers 64 contiguous bytes of 16 columns, through one buffer
// resource for the workgroup's rows).  Before the K loop the workgroup
// builds in LDS the table of its columns' {scale, zp * scale} in fp32 for
// every group (entry (g, c) at g (CW + 1) + c); per chunk each wave stages
// its own slices' activations (fp32) and group indices (clamped into
// 0..kb-1, stored as byte offsets of table rows) in a double buffer, loaded
// one chunk ahead like the codes, so the chunk loop has no workgroup
// barrier.  The 16 lanes of a quarter wave work on the same code
// position, so they read one table row's adjacent entries.  Per code: one
// address add, one 8-byte table read per column, fma(q, scale, -zp * scale)
// (the exact dequantized value for 16-bit scales) and the fma into the
// column's accumulator; the slices are summed at the end in a fixed order.
#include <algorithm>

#include "mfma_ops.h"
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

constexpr int GV_SLICE = 64;                // codes of a row per slice and chunk
constexpr int64_t GV_LDS_MAX = 96 * 1024;

// LDS of gidx_gemv_kernel: two staging buffers of a chunk (MT activations
// and a table offset per position), then the table.
int64_t gidx_gemv_lds(int64_t kb, int R, int W, int MT) {
  return (int64_t)2 * (4 * W * GV_SLICE) * (4 * MT + 4) + (kb + 1) * (16 * R + 1) * 8;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, int W, int PF, int MT>
__global__ __launch_bounds__(64 * W) void gidx_gemv_kernel(
    const typename dt<XDT>::T* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const int32_t* __restrict__ g_idx, const typename dt<XDT>::T* __restrict__ bias,
    typename dt<XDT>::T* __restrict__ Y, int Mp, int K, int N, int kb, int row_bytes,
    int zp_row_bytes, int chunks) {
  constexpr int CW = 16 * R, TS = CW + 1;
  constexpr int T = 64 * W;                     // threads
  constexpr int CH = 4 * W * GV_SLICE;          // codes of a row per chunk
  constexpr int P = 128 / BITS;                 // codes per 16-byte unit
  constexpr int UPC = GV_SLICE / P;             // units per slice per chunk
  constexpr int WPU = 32 / BITS;                // codes per 32-bit word
  constexpr int WCH = CH / W;                   // positions a wave stages per chunk
  static_assert(CH == 4 * T, "each thread stages 4 positions of a chunk");
  extern __shared__ __align__(16) unsigned char gv_smem[];
  float* xs = reinterpret_cast<float*>(gv_smem);                     // [2][MT][CH]
  int* gs = reinterpret_cast<int*>(gv_smem + 2 * MT * CH * 4);       // [2][CH]
  f32x2* tab = reinterpret_cast<f32x2*>(gv_smem + 2 * (MT + 1) * CH * 4);  // [kb + 1][TS]
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = lane & 15, s = wave * 4 + (lane >> 4);
  const int col0 = blockIdx.x * CW;

  // One resource for the workgroup's rows (a buffer resource must be the
  // same in every lane); a lane's column is a byte offset into it.
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + (int64_t)col0 * row_bytes), 0, min(CW, N - col0) * row_bytes, BUF_WORD3);
  // Codes of chunks ch .. ch + PF (slot 0: the chunk being computed).
  u32x4 cd[PF + 1][R][UPC];
  auto load_codes = [&](int ch, u32x4 (&dst)[R][UPC]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < UPC; ++i)
        dst[r][i] = __builtin_amdgcn_raw_buffer_load_b128(
            rb, (c + 16 * r) * row_bytes + ((ch * UPC + i) * 4 * W + s) * 16, 0, BUF_STREAM);
  };
  float xv[MT][4];
  int gv[4];
  // Each wave stages the positions of its own 4 slices (entry (i, q, e) of
  // its region: unit i of slice 4 w + q, code e), so that only the wave
  // reads what it wrote and the chunk loop needs no workgroup barrier.
  // Lane l stages entries 4 l .. 4 l + 3 (one unit, consecutive codes).
  const int sidx = lane * 4, si = sidx / (4 * P), sq = (sidx / P) % 4, se = sidx % P;
  const int skl = (si * 4 * W + wave * 4 + sq) * P + se;   // its chunk offset
  // Loads are unconditional (of an element in bounds) and selected after,
  // so that they are issued together; positions past K stage zeros.
  auto stage_load = [&](int ch) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = ch * CH + skl + j;
      const int kk = min(k, K - 1);
      const int g = min(max(g_idx[kk], 0), kb - 1);
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        // Rows past Mp read row Mp - 1 and stage zeros.
        const float x = dt<XDT>::to_f32(A[(int64_t)min(m, Mp - 1) * K + kk]);
        xv[m][j] = (k < K && m < Mp) ? x : 0.0f;
      }
      gv[j] = k < K ? g * (TS * 8) : 0;
    }
  };
  auto stage_store = [&](int buf) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
      *reinterpret_cast<f32x4*>(xs + (buf * MT + m) * CH + wave * WCH + sidx) =
          f32x4{xv[m][0], xv[m][1], xv[m][2], xv[m][3]};
    *reinterpret_cast<i32x4*>(gs + buf * CH + wave * WCH + sidx) = i32x4{gv[0], gv[1], gv[2], gv[3]};
  };

#pragma unroll
  for (int p = 0; p < PF; ++p) load_codes(p, cd[p]);
  stage_load(0);   // in flight with the table's loads
  // The table: lanes take adjacent groups of one column (adjacent scales);
  // groups past kb go to the spare row kb, which no lookup reads.
  for (int g0 = 0; g0 < kb; g0 += T) {
    const int g = min(g0 + t, kb - 1);
    float sv[CW], zv[CW];
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) {
      const int64_t n = min(col0 + cc, N - 1);
      sv[cc] = dt<SDT>::to_f32(scales[n * kb + g]);
      zv[cc] = (float)load_zp<BITS, HAS_ZP>(zp + n * zp_row_bytes, g);
    }
    const int row = g0 + t < kb ? g : kb;
#pragma unroll
    for (int cc = 0; cc < CW; ++cc) tab[row * TS + cc] = f32x2{sv[cc], zv[cc] * sv[cc]};
  }
  stage_store(0);
  __syncthreads();

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;
  const unsigned char* tbytes = reinterpret_cast<const unsigned char*>(tab) + c * 8;
  for (int ch = 0; ch < chunks; ++ch) {
    // Chunk ch + PF's codes and chunk ch + 1's staging values (past the
    // row: zeros from the buffer loads' range check and from stage_load),
    // loaded without a branch so that the loop body stays one block.
    load_codes(ch + PF, cd[PF]);
    stage_load(ch + 1);
    const int buf = ch & 1;
    const float* xb = xs + buf * MT * CH;
    const int* gb = gs + buf * CH;
#pragma unroll
    for (int i = 0; i < UPC; ++i) {
      const int kl = wave * WCH + (i * 4 + (lane >> 4)) * P;   // this lane's unit, staged
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        float q[R][WPU];
#pragma unroll
        for (int r = 0; r < R; ++r) word_codes_f32<BITS>(cd[0][r][i][wd], q[r]);
#pragma unroll
        for (int j4 = 0; j4 < WPU; j4 += 4) {
          const int k4 = kl + wd * WPU + j4;
          f32x4 a4[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) a4[m] = *reinterpret_cast<const f32x4*>(xb + m * CH + k4);
          const i32x4 g4 = *reinterpret_cast<const i32x4*>(gb + k4);
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const unsigned char* e = tbytes + g4[jj];
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const f32x2 sz = *reinterpret_cast<const f32x2*>(e + 128 * r);
              const float w = fmaf(q[r][j4 + jj], sz.x, -sz.y);
#pragma unroll
              for (int m = 0; m < MT; ++m) acc[r][m] = fmaf(a4[m][jj], w, acc[r][m]);
            }
          }
        }
        // One word's LDS reads at a time: hoisting every read of the chunk
        // would take the whole register file.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    stage_store(buf ^ 1);
    // The wave's own LDS writes and reads run in order: a compiler fence is
    // all the double buffer needs.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int p = 0; p < PF; ++p)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < UPC; ++i) cd[p][r][i] = cd[p + 1][r][i];
  }
  // Slices of a wave (lanes c, c + 16, c + 32, c + 48), then the waves in
  // order.
  __syncthreads();   // every wave done with its staging before red reuses it
  float* red = xs;   // [W][MT][CW]
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      float v = acc[r][m];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (lane < 16) red[(wave * MT + m) * CW + c + 16 * r] = v;
    }
  __syncthreads();
  static_assert(MT * CW <= T, "one thread per output");
  const int m = t / CW, cc = t % CW;
  if (m < Mp && m < MT && col0 + cc < N) {
    float o = red[m * CW + cc];
#pragma unroll
    for (int w = 1; w < W; ++w) o += red[(w * MT + m) * CW + cc];
    if (bias) o += dt<XDT>::to_f32(bias[col0 + cc]);
    Y[(int64_t)m * N + col0 + cc] = dt<XDT>::from_f32(o);
  }
}

// One launch per MT rows of A (each reads every code once for its rows).
template <int BITS, int XDT, int SDT, bool HAS_ZP, int W, int MT>
hipError_t launch_gemv_r(const MatArgs& a) {
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  const auto kern = gidx_gemv_kernel<BITS, XDT, SDT, HAS_ZP, 1, W, 1, MT>;
  const int64_t lds = gidx_gemv_lds(a.kb, 1, W, MT);
  if (lds > 64 * 1024) {
    const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)GV_LDS_MAX);
    if (e != hipSuccess) return e;
  }
  const int grid = (int)((a.N + 15) / 16);
  const int row_bytes = (int)(a.kb * a.blob);
  const int64_t ch = 4 * W * GV_SLICE;
  const int chunks = (int)((a.kb * a.block_size + ch - 1) / ch);
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(64 * W), (size_t)lds, a.stream,
                       (const XT*)a.A + m0 * a.K, a.B, (const ST*)a.scales, a.zp, a.g_idx,
                       (const XT*)a.bias, (XT*)a.Y + m0 * a.N, Mp, (int)a.K, (int)a.N, (int)a.kb,
                       row_bytes, (int)a.zp_row_bytes, chunks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The route for M <= 4, and M <= 16 when the matrix-core GEMM's grid of
// 64-column tiles would cover under half the compute units (measured,
// K 4096 N 14336: M = 1 / 2 / 4 20 / 28 / 37 us here against 59-60 us on
// the matrix cores for M >= 2, M = 8 75 us against 60; K 14336 N 4096:
// M = 1 / 2 / 4 / 8 / 16 19 / 22 / 40 / 64 / 127 us against 170-176 us):
// one column per lane (two measured no faster), codes one chunk ahead (two
// or three chunks ahead measured slower), MT = 1, 2, 4 or 8 rows per launch;
// 8 waves (32 slices) when the grid has fewer than 512 workgroups or for two
// rows (31 against 40 us with 4 waves at N 14336; one row: 25 against 20),
// if their LDS fits, else 4 waves; 0 when neither fits (another kernel then).
int gidx_gemv_rows(int64_t M) { return M == 1 ? 1 : M == 2 ? 2 : M <= 4 ? 4 : 8; }

int gidx_gemv_waves(const MatArgs& a) {
  const bool few = a.M <= 4 || (a.M <= 16 && (a.N + 63) / 64 < 128);
  if (!few || 16 * a.kb * a.blob >= ((int64_t)1 << 31)) return 0;
  const int mt = gidx_gemv_rows(a.M);
  if (((a.N + 15) / 16 < 512 || mt == 2) && gidx_gemv_lds(a.kb, 1, 8, mt) <= GV_LDS_MAX) return 8;
  return gidx_gemv_lds(a.kb, 1, 4, mt) <= GV_LDS_MAX ? 4 : 0;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int W>
hipError_t launch_gemv_w(const MatArgs& a) {
  switch (gidx_gemv_rows(a.M)) {
    case 1: return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, W, 1>(a);
    case 2: return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, W, 2>(a);
    case 4: return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, W, 4>(a);
    default: return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, W, 8>(a);
  }
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t launch_gemv_t(const MatArgs& a) {
  return gidx_gemv_waves(a) == 8 ? launch_gemv_w<BITS, XDT, SDT, HAS_ZP, 8>(a)
                                 : launch_gemv_w<BITS, XDT, SDT, HAS_ZP, 4>(a);
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t launch_rows_t(const MatArgs& a) {
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  constexpr int R = 2;
  const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
  if (gidx_gemv_waves(a) != 0) return launch_gemv_t<BITS, XDT, SDT, HAS_ZP>(a);
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
  if (gidx_gemv_waves(a) == 0 && gemm_mfma_gidx_supported(a)) return launch_gemm_mfma_gidx(a);
  switch (a.bits) {
    case 2: return launch_rows_x<2>(a);
    case 4: return launch_rows_x<4>(a);
    default: return launch_rows_x<8>(a);
  }
}

}  // namespace qmm
