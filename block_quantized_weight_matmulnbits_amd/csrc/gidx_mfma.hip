// gidx_mfma.hip -- MatMulNBits with group indices (act-order) on the matrix
// cores: the 256-row kernel of gemm_mfma.h with a per-workgroup table of its
// columns' scales and zero points in LDS (GI = 2), 64- or 128-column tiles.
//
// Element k of column n takes the scale and zero point of group g_idx[k]
// (onnx-runtime-ep-cpu matmul_nbits.rs, the group-index branch of
// dequantize_weight).  The workgroup first builds the table entry
// {scale, zp * scale} in fp32 for every group of each of its columns, then
// every K-step each of its 512 threads dequantizes 8 (64 columns) or 16 (128
// columns) codes of one column, one table read per code, so the lookups cost
// LDS reads instead of the cached memory reads of the untabled variant, and
// the vector work is spread over all four SIMDs.
#include "gemm_mfma.h"

namespace qmm {

namespace {

template <int BITS, int XDT, int SDT, bool HAS_ZP, int TN>
hipError_t staged_t(const MatArgs& a, int tiles_m) {
  using ST = typename dt<SDT>::T;
  constexpr int BN = 32 * TN;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  const size_t lds = mfma_lds_bytes<BN>() + gidx_table_bytes(a, BN);
  if (lds > LDS_MAX) return hipErrorInvalidValue;
  auto kern = gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, TN, false, 2>;
  const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)LDS_MAX);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(GEMM_TPB), lds, a.stream,
                     (const uint16_t*)a.A, a.B, (const ST*)a.scales, a.zp,
                     (const uint16_t*)a.bias, (uint16_t*)a.Y, (int)a.M, (int)a.K, (int)a.N,
                     (int)a.kb, ilog2i(a.block_size), ilog2i(a.blob), (int)a.zp_row_bytes,
                     tiles_m, (int)a.chunks, a.g_idx, 1.0f);
  return hipGetLastError();
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t staged_tn(const MatArgs& a, int tiles_m, int tn) {
  return tn == 2 ? staged_t<BITS, XDT, SDT, HAS_ZP, 2>(a, tiles_m)
                 : staged_t<BITS, XDT, SDT, HAS_ZP, 4>(a, tiles_m);
}

template <int BITS, int XDT>
hipError_t staged_s(const MatArgs& a, int tiles_m, int tn) {
  switch (a.s_dtype) {
    case DT_F32: return a.zp ? staged_tn<BITS, XDT, DT_F32, true>(a, tiles_m, tn) : staged_tn<BITS, XDT, DT_F32, false>(a, tiles_m, tn);
    case DT_F16: return a.zp ? staged_tn<BITS, XDT, DT_F16, true>(a, tiles_m, tn) : staged_tn<BITS, XDT, DT_F16, false>(a, tiles_m, tn);
    default: return a.zp ? staged_tn<BITS, XDT, DT_BF16, true>(a, tiles_m, tn) : staged_tn<BITS, XDT, DT_BF16, false>(a, tiles_m, tn);
  }
}

template <int BITS>
hipError_t staged_x(const MatArgs& a, int tiles_m, int tn) {
  return a.a_dtype == DT_F16 ? staged_s<BITS, DT_F16>(a, tiles_m, tn) : staged_s<BITS, DT_BF16>(a, tiles_m, tn);
}

}  // namespace

hipError_t launch_gidx_staged(const MatArgs& a, int tiles_m, int tn) {
  switch (a.bits) {
    case 2: return staged_x<2>(a, tiles_m, tn);
    case 4: return staged_x<4>(a, tiles_m, tn);
    default: return staged_x<8>(a, tiles_m, tn);
  }
}

}  // namespace qmm
