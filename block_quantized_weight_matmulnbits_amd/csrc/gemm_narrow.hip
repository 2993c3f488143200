// gemm_narrow.hip -- the 256-row matrix-core kernel (gemm_mfma.h) with 64- and
// 128-column tiles, for products whose 224/256-column grid would leave compute
// units idle: each workgroup walks all of K, so a grid shorter than one
// workgroup per compute unit is bound by a single workgroup's time.
#include "gemm_mfma.h"

namespace qmm {

template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t narrow_tn(const MatArgs& a, int tiles_m, int tn) {
  return tn == 2 ? launch_mfma_tn<BITS, XDT, SDT, HAS_ZP, 2>(a, tiles_m)
                 : launch_mfma_tn<BITS, XDT, SDT, HAS_ZP, 4>(a, tiles_m);
}

template <int BITS, int XDT>
static hipError_t narrow_s(const MatArgs& a, int tiles_m, int tn) {
  switch (a.s_dtype) {
    case DT_F32: return a.zp ? narrow_tn<BITS, XDT, DT_F32, true>(a, tiles_m, tn) : narrow_tn<BITS, XDT, DT_F32, false>(a, tiles_m, tn);
    case DT_F16: return a.zp ? narrow_tn<BITS, XDT, DT_F16, true>(a, tiles_m, tn) : narrow_tn<BITS, XDT, DT_F16, false>(a, tiles_m, tn);
    default: return a.zp ? narrow_tn<BITS, XDT, DT_BF16, true>(a, tiles_m, tn) : narrow_tn<BITS, XDT, DT_BF16, false>(a, tiles_m, tn);
  }
}

template <int BITS>
static hipError_t narrow_x(const MatArgs& a, int tiles_m, int tn) {
  return a.a_dtype == DT_F16 ? narrow_s<BITS, DT_F16>(a, tiles_m, tn) : narrow_s<BITS, DT_BF16>(a, tiles_m, tn);
}

hipError_t launch_gemm_narrow(const MatArgs& a, int tiles_m, int tn) {
  switch (a.bits) {
    case 2: return narrow_x<2>(a, tiles_m, tn);
    case 3: return narrow_x<3>(a, tiles_m, tn);
    case 4: return narrow_x<4>(a, tiles_m, tn);
    default: return narrow_x<8>(a, tiles_m, tn);
  }
}

}  // namespace qmm
