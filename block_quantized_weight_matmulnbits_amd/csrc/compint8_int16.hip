// compint8_int16.hip -- int16 activations on the int8 matrix cores of gfx950
// (the int16 route of onnx-runtime-ep-cpu matmul_nbits.rs, execute: 8-bit
// weights with int16 activations, offered for every width): the CompInt8
// kernel of compint8_tiled.h with its activations split into two int8
// planes (AB = 2), operator layout, from M = 8.
#include "compint8_tiled.h"

namespace qmm {

namespace {

using namespace ct;

// int16 activations (AB = 2): operator layout, unstaged.
template <int BITS, int SDT, int YDT, bool HAS_ZP, bool DOTS>
hipError_t launch_i16_t(const MatArgs& a, const int16_t* qa, const float* sa, int32_t* dots) {
  const bool hb = a.block_size == 32;
  const int log2_cpb = hb ? 0 : __builtin_ctz((unsigned)(a.block_size / TKC));
  const int chunks = (int)((a.kb * a.block_size + TKC - 1) / TKC);
  const int n_slices = (int)((a.N + TG - 1) / TG) * 2;
  const int Kp = (int)(a.kb * a.block_size);
  const int CS = 2;
  const int64_t units = hb ? (a.kb + 1) / 2 : a.kb;
  int S = 1;
  while (CS * S < 8 && (units + 2 * S - 1) / (2 * S) >= 2) S *= 2;
  const size_t lds = ct_lds(a.kb, Kp, CS, S, false, 0);
  auto kern = hb ? compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, false, true, true, 2>
                 : compint8_tiled_kernel<BITS, SDT, YDT, HAS_ZP, DOTS, false, true, false, 2>;
  const int grid = (n_slices + CS - 1) / CS;
  using YT = typename dt<YDT>::T;
  const int row_bytes = (int)(BITS == 3 ? a.kb * (3 * a.block_size / 8) : a.kb * a.blob);
  for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
    const int Mp = (int)std::min<int64_t>(16, a.M - m0);
    hipLaunchKernelGGL(kern, dim3(grid), dim3(CS * S * 64), lds, a.stream,
                       (const int8_t*)(qa + m0 * Kp), sa + m0 * a.kb, a.B,
                       (const uint8_t*)a.scales, a.zp, (const YT*)a.bias,
                       DOTS ? nullptr : (YT*)a.Y + m0 * a.N,
                       DOTS ? dots + m0 * a.N * a.kb : nullptr, Mp, (int)a.N, (int)a.kb, Kp,
                       chunks, log2_cpb, n_slices, CS, S, row_bytes, (int)a.zp_row_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int BITS, int SDT, bool DOTS>
hipError_t launch_i16_s(const MatArgs& a, const int16_t* qa, const float* sa, int32_t* dots) {
  auto y = [&](auto ydt) {
    constexpr int YDT = decltype(ydt)::value;
    return a.zp ? launch_i16_t<BITS, SDT, YDT, true, DOTS>(a, qa, sa, dots)
                : launch_i16_t<BITS, SDT, YDT, false, DOTS>(a, qa, sa, dots);
  };
  switch (a.a_dtype) {
    case DT_F32: return y(std::integral_constant<int, DT_F32>{});
    case DT_F16: return y(std::integral_constant<int, DT_F16>{});
    default: return y(std::integral_constant<int, DT_BF16>{});
  }
}

template <int BITS, bool DOTS>
hipError_t launch_i16_b(const MatArgs& a, const int16_t* qa, const float* sa, int32_t* dots) {
  switch (a.s_dtype) {
    case DT_F32: return launch_i16_s<BITS, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_i16_s<BITS, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_i16_s<BITS, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

template <bool DOTS>
hipError_t launch_i16(const MatArgs& a, const int16_t* qa, const float* sa, int32_t* dots) {
  switch (a.bits) {
    case 2: return launch_i16_b<2, DOTS>(a, qa, sa, dots);
    case 3: return launch_i16_b<3, DOTS>(a, qa, sa, dots);
    case 4: return launch_i16_b<4, DOTS>(a, qa, sa, dots);
    default: return launch_i16_b<8, DOTS>(a, qa, sa, dots);
  }
}

}  // namespace

bool int16_tiled_preferred(const MatArgs& a) {
  // From M = 8 on the operator's layout, blocks of at most 128 codes (the
  // int32 block dot of int16 activations).
  return !a.tiled && a.M >= 8 && a.block_size <= 128 && compint8_tiled_supported(a) &&
         32 * a.kb * a.block_size < 0x7FFFFF00LL;
}

hipError_t launch_int16_tiled(const MatArgs& a, const int16_t* qa, const float* sa,
                              int32_t* dots) {
  return dots ? launch_i16<true>(a, qa, sa, dots) : launch_i16<false>(a, qa, sa, nullptr);
}

}  // namespace qmm
