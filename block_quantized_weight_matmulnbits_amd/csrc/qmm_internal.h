// qmm_internal.h -- host-side interface between the validated C ABI
// (qmm_api.cpp) and the kernel launchers (*.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace qmm {

// A validated MatMulNBits problem.  Pointers are device pointers.
struct MatArgs {
  const void* A = nullptr;        // [M, K] a_dtype
  const uint8_t* B = nullptr;     // [N, kb, blob]
  const void* scales = nullptr;   // [N, kb] s_dtype
  const uint8_t* zp = nullptr;    // [N, zp_row_bytes] or null
  const int32_t* g_idx = nullptr; // [K] group of each K element, or null (block k / bs)
  const void* bias = nullptr;     // [N] a_dtype or null
  void* Y = nullptr;              // [M, N] a_dtype
  int64_t M = 1, K = 0, N = 0;
  int64_t block_size = 0, kb = 0, blob = 0, zp_row_bytes = 0;
  int bits = 4;
  int a_dtype = 0, s_dtype = 0;
  // 0: operator layout; 1: tiled (qmm_layout.h), B / scales / zp then point
  // at the regions of the repacked buffer.
  int tiled = 0;
  int64_t chunks = 0;     // tiled: 64-code chunks per column
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  hipStream_t stream = nullptr;
};
using GemvArgs = MatArgs;

hipError_t launch_gemv(const MatArgs& a);
// Group indices on the operator's layout (gidx.hip): the fp32 row kernel,
// or the matrix-core GEMM for 16-bit activations and M > 16.
hipError_t launch_gidx(const MatArgs& a);
// The matrix-core GEMM with per-code group lookups (gemm.hip).
bool gemm_mfma_gidx_supported(const MatArgs& a);
// A few rows of 16-bit activations on the matrix cores, K split over the
// waves of a workgroup (gemm_skinny.hip): M <= 16, or a grid of at most
// SKINNY_MAX_GROUPS workgroups of 32 rows x 32 columns.
constexpr int64_t SKINNY_MAX_GROUPS = 1024;
bool gemm_skinny_supported(const MatArgs& a);
hipError_t launch_gemm_skinny(const MatArgs& a);
hipError_t launch_gemm_mfma_gidx(const MatArgs& a);
// M = 1 on the tiled layout (gemv_tiled.hip).
bool gemv_tiled_supported(const MatArgs& a);
hipError_t launch_gemv_tiled(const MatArgs& a);

// Batched / prefill matmul (M > 1): bf16/f16 MFMA kernel, or the fp32
// multi-row fallback.
hipError_t launch_gemm(const MatArgs& a);

// CompInt8: quantize A into qa [M, kb*bs] int8 and sa [M, kb] float, then
// the int8 block-dot matmul (or, for the test export, the exact int32 block
// dots [M, N, kb] accumulated into a zeroed buffer).
hipError_t launch_quantize_a(const MatArgs& a, int8_t* qa, float* sa);
hipError_t launch_compint8(const MatArgs& a, const int8_t* qa, const float* sa);
hipError_t launch_compint8_dots(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots);
// CompInt8 for M = 1 on the tiled layout, quantization fused
// (compint8_small.hip); it needs no workspace.
bool compint8_small_supported(const MatArgs& a);
hipError_t launch_compint8_small(const MatArgs& a);
// The same kernel, writing its exact int32 block dots [M, N, kb] and the
// activations it quantized in LDS (qa [M, kb*bs], sa [M, kb]) instead of Y.
hipError_t launch_compint8_small_dots(const MatArgs& a, int8_t* qa, float* sa, int32_t* dots);
// CompInt8 on the tiled layout with int8 MFMA (compint8_tiled.hip).
bool compint8_tiled_supported(const MatArgs& a);
// Whether M >= 2 on the operator's layout takes compint8_tiled (faster there).
bool compint8_tiled_preferred(const MatArgs& a);
// int16 activations on the int8 matrix cores (two activation planes).
bool int16_tiled_preferred(const MatArgs& a);
hipError_t launch_int16_tiled(const MatArgs& a, const int16_t* qa, const float* sa, int32_t* dots);
hipError_t launch_compint8_tiled(const MatArgs& a, const int8_t* qa, const float* sa);
hipError_t launch_compint8_tiled_dots(const MatArgs& a, const int8_t* qa, const float* sa,
                                      int32_t* dots);

// Block-scaled FP4 weights (fp4.hip): a validated problem.
struct Fp4Args {
  const void* A = nullptr;        // [M, K] a_dtype
  const uint8_t* W = nullptr;     // [N, kb, bs/2] E2M1 codes
  const uint8_t* scales = nullptr;  // [N, kb] E8M0 (MXFP4) or E4M3 (NVFP4) bytes
  float global_scale = 1.0f;
  const void* bias = nullptr;     // [N] a_dtype or null
  void* Y = nullptr;              // [M, N] a_dtype
  int64_t M = 1, K = 0, N = 0, kb = 0;
  int format = 0;                 // 0 = MXFP4, 1 = NVFP4
  int a_dtype = 0;
  hipStream_t stream = nullptr;
};
hipError_t launch_fp4(const Fp4Args& a);
// The matrix-core GEMM on FP4 weights (gemm.hip): 16-bit activations, M > 16.
bool gemm_mfma_fp4_supported(const Fp4Args& a);
hipError_t launch_gemm_mfma_fp4(const Fp4Args& a);
// FP4 weights on the few-row kernel (gemm_skinny.hip), the same routing rule.
bool gemm_skinny_fp4_supported(const Fp4Args& a);
hipError_t launch_gemm_skinny_fp4(const Fp4Args& a);

// Low-precision scaled GEMM (validated problem; lowp.hip).
struct LowpArgs {
  const uint8_t* lhs = nullptr;   // [m, k] codes, one per byte
  const uint8_t* rhs = nullptr;   // [n, k] codes
  const void* lsc = nullptr;      // per tensor: one f32; MX / NVFP4: [m, nblk] bytes
  const void* rsc = nullptr;      // per tensor: one f32; MX / NVFP4: [n, nblk] bytes
  const float* bias = nullptr;    // [n] or null
  float* out = nullptr;           // [m, n]
  int64_t m = 0, n = 0, k = 0;
  int layout = 0;                 // 0 per tensor, 1 MX (E8M0 / 32), 2 NVFP4 (E4M3 / 16)
  int lfmt = 0, rfmt = 0;         // 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1
  hipStream_t stream = nullptr;
};
hipError_t launch_lowp_matmul(const LowpArgs& a);
struct LowpQuantArgs {
  const void* x = nullptr;        // [rows, cols] x_dtype
  uint8_t* codes = nullptr;       // [rows, cols]
  void* scales = nullptr;         // per tensor: one f32; else [rows, nblk] bytes
  int64_t rows = 0, cols = 0;
  int x_dtype = 0, fmt = 0, layout = 0;
  hipStream_t stream = nullptr;
};
hipError_t launch_lowp_quantize(const LowpQuantArgs& a);

// int8 convolution (validated NHWC / OHWI problem).
struct ConvArgs {
  const int8_t* X = nullptr;
  const int8_t* Wt = nullptr;
  const int32_t* bias = nullptr;
  const float* w_scale = nullptr;
  float in_scale = 1.f, out_scale = 1.f;
  int in_zp = 0, out_zp = 0, clamp_min = -128, clamp_max = 127;
  int Nb = 0, H = 0, W = 0, C = 0, Co = 0, KH = 0, KW = 0;
  int stride_h = 1, stride_w = 1, pad_h = 0, pad_w = 0;
  int8_t* Y = nullptr;
  hipStream_t stream = nullptr;
};
hipError_t launch_conv_int8(const ConvArgs& c);

// Repack into / out of the tiled layout (qmm_layout.h).
hipError_t launch_repack(const MatArgs& a, uint8_t* tiled, bool inverse, uint8_t* B_out,
                         void* scales_out, uint8_t* zp_out);

// Codec export: codes [N, K], zero points [N, kb], dequantized weight [N, K].
hipError_t launch_unpack(const MatArgs& a, uint8_t* codes, uint8_t* zps, float* w);

// Workspace layout of CompInt8: qa [M, kb*bs] int8, then sa [M, kb] float,
// each region 256-byte aligned.
inline size_t ws_align(size_t v) { return (v + 255) / 256 * 256; }
inline size_t ws_qa_bytes(int64_t M, int64_t kb, int64_t bs) { return ws_align((size_t)(M * kb * bs)); }
inline size_t ws_total_bytes(int64_t M, int64_t kb, int64_t bs) {
  return ws_qa_bytes(M, kb, bs) + ws_align((size_t)(M * kb * 4));
}

// The generic operator-layout kernel (generic.hip): 3-bit codes, and int8
// / int16 activations quantized per block (qa, sa) for any code width; with
// dots non-null the exact int32 block dots [M, N, kb] are written instead of
// Y.  Blocks of at most GENERIC_MAX_BS codes.
constexpr int64_t GENERIC_MAX_BS = 8192;
hipError_t launch_generic_float(const MatArgs& a);
hipError_t launch_generic_int(const MatArgs& a, const void* qa, int act_bytes, const float* sa,
                              int32_t* dots);
// int16 activations: qa16 [M, kb*bs] int16 and sa [M, kb] f32 (compint8.hip).
hipError_t launch_quantize_a16(const MatArgs& a, int16_t* qa, float* sa);
inline size_t ws16_qa_bytes(int64_t M, int64_t kb, int64_t bs) { return ws_align((size_t)(M * kb * bs * 2)); }
inline size_t ws16_total_bytes(int64_t M, int64_t kb, int64_t bs) {
  return ws16_qa_bytes(M, kb, bs) + ws_align((size_t)(M * kb * 4));
}

// The body of qmm_gemm_compint8 (validation, route choice, launches), shared
// with the entry point that takes no workspace: fn names the entry point in
// messages; when resolve_workspace is non-null it is called after the
// arguments have been validated (and only if there is work) to obtain the
// workspace, which then holds workspace_bytes.
int gemm_compint8_impl(const char* fn, const void* A, int a_dtype, const uint8_t* B,
                       int b_layout, const void* scales, int s_dtype, const uint8_t* zero_points,
                       const int32_t* g_idx, int64_t g_idx_len, const void* bias, void* Y,
                       int64_t M, int64_t K, int64_t N, int block_size, int bits,
                       int accuracy_level, void* workspace, size_t workspace_bytes,
                       hipError_t (*resolve_workspace)(void**), void* stream);
// Allow `kernel` up to `bytes` of dynamic LDS on the current device
// (hipFuncSetAttribute once per device and kernel; thread-safe).
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);

// Record a message for qmm_last_error and return code.
int set_error(int code, const char* message);


}  // namespace qmm
