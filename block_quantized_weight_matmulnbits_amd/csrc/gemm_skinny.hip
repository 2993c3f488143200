// gemm_skinny.hip -- routing of the few-row matrix-core kernel
// (gemm_skinny.h) and its 4-bit and FP4 instances; the 2-, 3- and 8-bit ones
// are in gemm_skinny_w.hip.
#include "gemm_skinny.h"

namespace qmm {

bool gemm_skinny_supported(const MatArgs& a) {
  const int64_t sz = a.s_dtype == DT_F32 ? 4 : 2;
  // Past the limit the 256-row kernel, whose workgroups each cover many
  // rows, is faster: every workgroup here dequantizes its columns afresh.
  const bool few = a.M <= 16 || ((a.M + 31) / 32) * ((a.N + 31) / 32) <= SKINNY_MAX_GROUPS;
  constexpr int64_t LIM = 0x7FFFE000LL;       // every buffer extent (OOB_A in the kernel)
  return a.a_dtype != DT_F32 && !(a.bits == 3 && a.tiled) && !a.g_idx && a.M >= 2 && few &&
         (a.K % 8) == 0 && ((uintptr_t)a.A & 15) == 0 && a.M * a.K * 2 <= LIM &&
         (a.N + 32) * a.kb * a.blob + 256 <= LIM &&
         (a.N + 32) * (a.chunks + 2) * 64 * a.bits / 8 <= LIM &&
         (a.N + 32) * a.kb * sz <= LIM && (a.N + 32) * (a.zp_row_bytes + 4) <= LIM;
}

// FP4 weights: the operator-layout 4-bit geometry with blocks of 32 (MXFP4)
// or 16 (NVFP4), one scale byte per block, no zero points.
template <int XDT, int WF, int TN, int MT>
static hipError_t launch_skinny_fp4_t(const Fp4Args& f) {
  const int64_t bs = (WF - 1) == FP4_MX ? 32 : 16;
  const dim3 grid((unsigned)((f.N + 16 * TN - 1) / (16 * TN)), (unsigned)((f.M + 16 * MT - 1) / (16 * MT)));
  const int64_t lds = (16 * TN * f.kb + 15 + 15) / 16 * 16;
  const bool slab = lds <= SK_SLAB_MAX;
  auto kern = slab ? gemm_skinny_kernel<4, XDT, DT_BF16, false, TN, MT, false, true, WF>
                   : gemm_skinny_kernel<4, XDT, DT_BF16, false, TN, MT, false, false, WF>;
  if (slab) {
    const hipError_t e = ensure_dynamic_lds((const void*)kern, SK_SLAB_MAX);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(SK_TPB), slab ? (size_t)lds : 0, f.stream, (const uint16_t*)f.A,
                     f.W, (const uint16_t*)f.scales, (const uint8_t*)nullptr, (const uint16_t*)f.bias,
                     (uint16_t*)f.Y, (int)f.M, (int)f.K, (int)f.N, (int)f.kb, sk_log2(bs),
                     (int)(f.kb * bs / 2), 0, 0, f.global_scale);
  return hipGetLastError();
}

template <int XDT, int WF>
static hipError_t launch_skinny_fp4_m(const Fp4Args& f) {
  const int64_t row_tiles = f.M <= 16 ? 1 : (f.M + 31) / 32;
  const bool narrow = row_tiles * ((f.N + 31) / 32) < SK_FULL_ROUND;
  if (f.M <= 16) return narrow ? launch_skinny_fp4_t<XDT, WF, 1, 1>(f) : launch_skinny_fp4_t<XDT, WF, 2, 1>(f);
  return narrow ? launch_skinny_fp4_t<XDT, WF, 1, 2>(f) : launch_skinny_fp4_t<XDT, WF, 2, 2>(f);
}

bool gemm_skinny_fp4_supported(const Fp4Args& f) {
  const int64_t bs = f.format == FP4_MX ? 32 : 16;
  const bool few = f.M <= 16 || ((f.M + 31) / 32) * ((f.N + 31) / 32) <= SKINNY_MAX_GROUPS;
  constexpr int64_t LIM = 0x7FFFE000LL;
  return f.a_dtype != DT_F32 && f.M >= 2 && few && (f.K % 8) == 0 && ((uintptr_t)f.A & 15) == 0 &&
         f.M * f.K * 2 <= LIM && (f.N + 32) * f.kb * (bs / 2) + 256 <= LIM && (f.N + 32) * f.kb <= LIM;
}

hipError_t launch_gemm_skinny_fp4(const Fp4Args& f) {
  const bool f16 = f.a_dtype == DT_F16;
  if (f.format == FP4_MX)
    return f16 ? launch_skinny_fp4_m<DT_F16, 1 + FP4_MX>(f) : launch_skinny_fp4_m<DT_BF16, 1 + FP4_MX>(f);
  return f16 ? launch_skinny_fp4_m<DT_F16, 1 + FP4_NV>(f) : launch_skinny_fp4_m<DT_BF16, 1 + FP4_NV>(f);
}

hipError_t launch_gemm_skinny(const MatArgs& a) {
  return a.bits == 4 ? launch_skinny_x<4>(a) : launch_gemm_skinny_w(a);
}

}  // namespace qmm
