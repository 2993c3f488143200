// compint8_tiled.hip -- CompInt8 (accuracy_level 4) with the int8 matrix
// cores of gfx950, on the tiled weight layout (qmm_layout.h) and, for M >= 2,
// on the operator's layout (there also 3-bit weights: their two bit planes
// are merged into the 2-bit codes' plane order).
//
// Definition (onnx-runtime-ep-cpu matmul_nbits.rs: quantize_activation_signed,
// int4_dot_row_scalar, int8_row): with qa / sa the int8 activations and their
// per-block scales written by quantize_a_kernel,
//   dot[m, n, b] = sum_{k in b} qa[m, k] * (code(n, k) - zp(n, b))   (int32)
//   y[m, n]      = sum_b float(dot) * (sa[m, b] * scale[n, b]) (+ bias[n]).
//
// One v_mfma_i32_16x16x64_i8 multiplies 16 activation rows (M padded with
// zero rows) by 16 weight columns over one 64-code chunk: lane l holds 16
// int8 of row / column l % 16 for reduction indices 16 * (l / 16) + [0, 16).
// The codes enter raw (0 <= code < 2^bits; 8-bit codes as code - 128) and the
// zero point is applied per block through the identity
//   sum qa * (code - zp) = sum qa * code' - (zp - off) * sum qa,
// off = 0 (2/4-bit) or 128 (8-bit, code' = code - 128), with sum qa taken by a
// second MFMA against an all-ones operand; all of it is exact int32.  The
// codes' unpacking leaves them in a fixed order inside each lane's 16 bytes
// (nibble or crumb planes); the activation bytes are permuted the same way
// with v_perm_b32, so products pair correctly.
//
// Work split: a wave owns a slice of 16 columns (half a 32-column group) and
// a share of the blocks of K; a workgroup holds CS slices x S shares and adds
// the shares through LDS.  Each chunk costs the wave one load of its codes
// (tiled: the 16 columns' bytes of a chunk are 8 * BITS * 16 contiguous
// bytes; operator layout (OPL): 8 * BITS bytes of each column's row) and one
// 16-byte load of activations per lane (rows past M read zeros from past the
// buffer's extent), then two MFMAs.  On the operator layout the scales and
// zero points are read with loads of their own width (rows of kb scales and
// of whole zero-point bytes need not fill 32-bit words: a buffer load zeroes
// a dword not wholly inside the extent).
#include "compint8_tiled.h"

namespace qmm {

namespace {

using namespace ct;

template <int BITS, int SDT, int YDT, bool HAS_ZP, bool DOTS, bool STAGE>
hipError_t launch_t(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  const int chunks = (int)tg.chunks;             // kb * bs / 64 on either layout
  const bool hb = a.block_size == 32;
  const int log2_cpb = hb ? 0 : __builtin_ctz((unsigned)(a.block_size / TKC));
  const int n_slices = (int)tg.groups * 2;
  const int Kp = (int)(a.kb * a.block_size);
  // Two slices (one group) per workgroup, shares of K until a workgroup has
  // 8 waves; staged above 4 rows, four slices sharing the rows and shares
  // until 16 waves.  Both keep at least two blocks per share.
  const bool wide = STAGE && a.M > 4;
  const int CS = wide ? 4 : 2;
  const int maxw = wide ? 16 : 8;
  int S = 1;
  const int64_t units = hb ? (a.kb + 1) / 2 : a.kb;
  while (CS * S < maxw && (units + 2 * S - 1) / (2 * S) >= 2) S *= 2;
  const int rows = (int)std::min<int64_t>(16, a.M);
  const size_t lds = ct_lds(a.kb, Kp, CS, S, STAGE, rows);
  decltype(&compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, true, false>) kern;
  if constexpr (BITS == 3)
    kern = hb ? compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, true, true>
              : compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, true, false>;
  else if (a.tiled)
    kern = hb ? compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, false, true>
              : compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, false, false>;
  else
    kern = hb ? compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, true, true>
              : compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, STAGE, true, false>;
  if (lds > 64 * 1024) {
    const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)CT_STAGE_LDS_MAX);
    if (e != hipSuccess) return e;
  }
  const int grid = (n_slices + CS - 1) / CS;
  using YT = typename dt<YDT>::T;
  for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
    const int Mp = (int)std::min<int64_t>(16, a.M - m0);
    hipLaunchKernelGGL(kern, dim3(grid),
                       dim3(CS * S * 64), lds, a.stream, qa + m0 * Kp, sa + m0 * a.kb,
                       a.B + (a.tiled ? tg.codes_off : 0), (const uint8_t*)a.scales, a.zp,
                       (const YT*)a.bias, DOTS ? nullptr : (YT*)a.Y + m0 * a.N,
                       DOTS ? dots + m0 * a.N * a.kb : nullptr, Mp, (int)a.N, (int)a.kb, Kp,
                       chunks, log2_cpb, n_slices, CS, S,
                       (int)(BITS == 3 ? a.kb * (3 * a.block_size / 8) : a.kb * a.blob),
                       (int)a.zp_row_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int SDT, int YDT, bool DOTS>
hipError_t launch_z(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  // Staged rows when they fit (the block-dot export keeps the plain form).
  // Above 4 rows four slices share them (unstaged, every wave re-read its
  // 16 rows from L2 with each chunk: 59 MB per call at M = 16, K = 4096,
  // N = 14336); at up to 4 rows two slices do, which keeps 448 workgroups
  // for N = 14336 (four would leave 32 compute units idle).
  const int64_t Kp = a.kb * a.block_size;
  const bool stage = !DOTS && ct_lds(a.kb, Kp, 4, 4, true, 16) <= CT_STAGE_LDS_MAX;
  if constexpr (!DOTS) {
    if (stage)
      return a.zp ? launch_t<BITS, SDT, YDT, true, false, true>(a, qa, sa, dots)
                  : launch_t<BITS, SDT, YDT, false, false, true>(a, qa, sa, dots);
  }
  return a.zp ? launch_t<BITS, SDT, YDT, true, DOTS, false>(a, qa, sa, dots)
              : launch_t<BITS, SDT, YDT, false, DOTS, false>(a, qa, sa, dots);
}

template <int BITS, int SDT, bool DOTS>
hipError_t launch_y(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.a_dtype) {
    case DT_F32: return launch_z<BITS, SDT, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_z<BITS, SDT, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_z<BITS, SDT, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

template <int BITS, bool DOTS>
hipError_t launch_s(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.s_dtype) {
    case DT_F32: return launch_y<BITS, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_y<BITS, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_y<BITS, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

template <bool DOTS>
hipError_t launch_b(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.bits) {
    case 2: return launch_s<2, DOTS>(a, qa, sa, dots);
    case 3: return launch_s<3, DOTS>(a, qa, sa, dots);
    case 4: return launch_s<4, DOTS>(a, qa, sa, dots);
    default: return launch_s<8, DOTS>(a, qa, sa, dots);
  }
}

}  // namespace

bool compint8_tiled_supported(const MatArgs& a) {
  // Whole blocks of 64-code chunks; LDS for the activation scales; 32-bit
  // offsets (operator layout: the code rows, the scale rows and the
  // zero-point rows of N + 32 columns, the slices' padding).
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  const int64_t row_bytes = a.bits == 3 ? a.kb * (3 * a.block_size / 8) : a.kb * a.blob;
  if (a.bits == 3 && a.tiled) return false;      // 3-bit weights: operator layout only
  const bool fits = a.tiled ? tg.total < 0x7FFFFF00LL
                            : (a.N + 32) * row_bytes < 0x7FFFFF00LL &&
                                  (a.N + 32) * a.kb * 4 < 0x7FFFFF00LL &&
                                  (a.N + 32) * a.zp_row_bytes * 8 < 0x7FFFFF00LL;
  return a.block_size >= 32 && (a.kb * 16 + 8 * 256) * 4 <= 64 * 1024 && fits &&
         16 * a.kb * a.block_size < 0x7FFFFF00LL;
}

bool compint8_tiled_preferred(const MatArgs& a) {
  // On the operator's layout the other kernels win at few rows where this one
  // reads more per code: blocks of 32 (two blocks per chunk: twice the MFMAs
  // and scale loads) and 3-bit weights (two planes) -- measured at K 4096,
  // N 14336: 4-bit bs 32, M = 4 / 8: 36.8 / 37.4 us here against 22.3 / 63.4
  // on compint8_kernel; 3-bit: 53.9 / 54.4 against 40.4 / 78.2 on the
  // generic kernel.
  if (a.M < 2 || !compint8_tiled_supported(a)) return false;
  return a.M >= 8 || (a.block_size >= TKC && a.bits != 3);
}

hipError_t launch_compint8_tiled(const MatArgs& a, const int8_t* qa, const float* sa) {
  return launch_b<false>(a, qa, sa, nullptr);
}

hipError_t launch_compint8_tiled_dots(const MatArgs& a, const int8_t* qa, const float* sa,
                                      int32_t* dots) {
  return launch_b<true>(a, qa, sa, dots);
}

}  // namespace qmm
