// qmm_api.cpp -- the extern "C" entry points declared in include/qmm.h:
// argument validation (mirroring MatMulNBitsFactory::create and execute of
// onnx-runtime-ep-cpu matmul_nbits.rs, with errors that say what, why and how
// to fix), then dispatch to the kernel launchers.  Nothing here allocates
// device memory or synchronizes.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "../../include/qmm.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

using qmm::MatArgs;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* fn) {
  if (e == hipSuccess) return QMM_OK;
  return fail(QMM_ERR_HIP, "%s: the HIP runtime reported '%s' while enqueueing the kernel. "
              "Why: the launch or an earlier asynchronous operation on this device failed. "
              "How to fix: check the device state and earlier errors on the stream.",
              fn, hipGetErrorString(e));
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int dtype_size(int dt) {
  switch (dt) {
    case QMM_F32: return 4;
    case QMM_F16: return 2;
    case QMM_BF16: return 2;
    default: return 0;
  }
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

enum class Route { Float, CompInt8 };

// Validation shared by qmm_gemv, qmm_gemm and qmm_gemm_compint8.
int validate_matmul(const char* fn, Route route, const void* A, int a_dtype, const uint8_t* B,
                    int b_layout, const void* scales, int s_dtype, const uint8_t* zp,
                    const void* bias, void* Y, int64_t M, int64_t K, int64_t N, int block_size,
                    int bits, int accuracy_level, MatArgs* out) {
  if (bits != 2 && bits != 3 && bits != 4 && bits != 8)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: bits must be 2, 3, 4 or 8, got bits=%d. Why: other packed widths have no "
                "validated unpacking path. How to fix: export the weight with bits=2, 3, 4 or 8.",
                fn, bits);
  if (block_size < 16 || !is_pow2(block_size))
    return fail(QMM_ERR_INVALID_ARG,
                "%s: block_size must be a power of two and at least 16, got %d. Why: the "
                "operator defines blocks of block_size codes that fill whole bytes. How to fix: "
                "re-quantize with block_size 16, 32, 64, 128, ...",
                fn, block_size);
  if (K <= 0 || N <= 0)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: K and N must be positive, got K=%lld N=%lld. Why: they are required "
                "positive attributes of the operator. How to fix: pass the weight's K and N.",
                fn, (long long)K, (long long)N);
  if (M < 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: M must be >= 0, got %lld. How to fix: pass the "
                "product of A's leading dimensions.", fn, (long long)M);
  if (K > INT32_MAX / 2 || N > INT32_MAX / 2 || M > INT32_MAX / 2)
    return fail(QMM_ERR_UNSUPPORTED,
                "%s: M, K and N must each be below 2^30 (got M=%lld K=%lld N=%lld). Why: kernel "
                "indices are 32-bit. How to fix: split the matmul along M or N.",
                fn, (long long)M, (long long)K, (long long)N);
  if (dtype_size(a_dtype) == 0 || dtype_size(s_dtype) == 0)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: a_dtype=%d / s_dtype=%d is not a qmm_dtype. Why: A, scales, bias and Y must "
                "be a float compute dtype. How to fix: pass QMM_F32, QMM_F16 or QMM_BF16.",
                fn, a_dtype, s_dtype);
  if (b_layout != QMM_LAYOUT_ORT && b_layout != QMM_LAYOUT_TILED &&
      b_layout != QMM_LAYOUT_TILED_ZP)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: b_layout=%d is not a qmm_layout. How to fix: pass QMM_LAYOUT_ORT for the "
                "operator's [N, kb, block_size*bits/8] bytes, or QMM_LAYOUT_TILED[_ZP] for a "
                "buffer written by qmm_repack.", fn, b_layout);
  const bool tiled = b_layout != QMM_LAYOUT_ORT;
  if (bits == 3 && (tiled || block_size > qmm::GENERIC_MAX_BS))
    return fail(QMM_ERR_UNSUPPORTED,
                "%s: 3-bit weights run on the operator's layout with block_size <= %lld (got "
                "layout %d, block_size %d). Why: the tiled layout and the repack are defined for "
                "2, 4 and 8 bits. How to fix: pass the operator's B (QMM_LAYOUT_ORT).", fn,
                (long long)qmm::GENERIC_MAX_BS, b_layout, block_size);
  if (tiled && (scales != nullptr || zp != nullptr))
    return fail(QMM_ERR_INVALID_ARG,
                "%s: with a tiled layout the scales and zero_points arguments must be NULL. "
                "Why: the repacked buffer carries them. How to fix: pass NULL and the layout "
                "that matches how the buffer was repacked (QMM_LAYOUT_TILED_ZP if it was "
                "repacked with zero points).", fn);
  if (tiled && ((uintptr_t)B & 255) != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: a repacked buffer must be 256-byte aligned. How to "
                "fix: pass the start of the buffer given to qmm_repack.", fn);
  if (tiled) scales = B;   // placeholder for the null check below; replaced at the end
  if (route == Route::Float && accuracy_level == 4)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: accuracy_level=4 requests int8 activations (CompInt8). Why: this entry "
                "point computes with float activations and takes no workspace for the int8 "
                "activations. How to fix: call qmm_gemm_compint8 with a workspace of "
                "qmm_compint8_workspace_size(M, K, block_size) bytes.", fn);
  if (route == Route::CompInt8 && accuracy_level != 4)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: accuracy_level must be 4 here, got %d. Why: this entry point implements "
                "the int8-activation (CompInt8) computation only. How to fix: use qmm_gemm for "
                "accuracy levels 0-3.", fn, accuracy_level);
  if (accuracy_level < 0 || accuracy_level > 4)
    return fail(QMM_ERR_INVALID_ARG,
                "%s: accuracy_level must be in 0..4, got %d. Why: 0 = default, 1 = fp32, "
                "2 = fp16, 3 = bf16, 4 = int8. How to fix: pass one of these.", fn,
                accuracy_level);
  if (B == nullptr || scales == nullptr || (M > 0 && (A == nullptr || Y == nullptr)))
    return fail(QMM_ERR_INVALID_ARG,
                "%s: A, B, scales and Y must be non-null device pointers. Why: they are the "
                "required inputs and output. How to fix: pass allocated device buffers.", fn);
  if (!aligned(B, 16))
    return fail(QMM_ERR_INVALID_ARG,
                "%s: B must be 16-byte aligned. Why: the kernels read packed codes with "
                "128-bit loads. How to fix: pass a contiguous, freshly allocated tensor.", fn);
  const int asz = dtype_size(a_dtype);
  if (!aligned(A, asz) || !aligned(Y, asz) || !aligned(bias, asz) ||
      !aligned(scales, dtype_size(s_dtype)))
    return fail(QMM_ERR_INVALID_ARG,
                "%s: A, Y, bias and scales must be aligned to their element size. How to fix: "
                "pass contiguous tensors.", fn);
  out->A = A;
  out->B = B;
  out->scales = scales;
  out->zp = zp;
  out->bias = bias;
  out->Y = Y;
  out->M = M;
  out->K = K;
  out->N = N;
  out->block_size = block_size;
  out->kb = (K + block_size - 1) / block_size;
  out->blob = (int64_t)block_size * bits / 8;
  out->zp_row_bytes = (out->kb * bits + 7) / 8;
  out->bits = bits;
  out->a_dtype = a_dtype;
  out->s_dtype = s_dtype;
  if (tiled) {
    const qmm::TiledGeom g = qmm::tiled_geom(K, N, block_size, bits, dtype_size(s_dtype),
                                             b_layout == QMM_LAYOUT_TILED_ZP);
    out->tiled = 1;
    out->chunks = g.chunks;
    out->scales = B + g.scales_off;
    out->zp = b_layout == QMM_LAYOUT_TILED_ZP ? B + g.zps_off : nullptr;
  }
  return QMM_OK;
}

int check_workspace(const char* fn, const MatArgs& a, void* workspace, size_t bytes) {
  const size_t need = qmm::ws_total_bytes(a.M, a.kb, a.block_size);
  if (workspace == nullptr || bytes < need)
    return fail(QMM_ERR_WORKSPACE,
                "%s: the workspace holds %zu bytes at %p, %zu are needed. Why: CompInt8 stores the "
                "int8 activations and their per-block scales there (the library never allocates). "
                "How to fix: pass qmm_compint8_workspace_size(M, K, block_size) bytes of device "
                "memory.", fn, bytes, workspace, need);
  if (((uintptr_t)workspace & 255) != 0)
    return fail(QMM_ERR_WORKSPACE, "%s: the workspace must be 256-byte aligned. How to fix: "
                "pass the start of a fresh allocation.", fn);
  return QMM_OK;
}

// Group indices (MatMulNBits input 4; matmul_nbits.rs execute: int32 of
// shape [K] or [kb * block_size]).  The range of the entries is the caller's
// to check on the host (qmm_check_g_idx): the kernels clamp each entry into
// 0..kb-1 so that an out-of-range one reads in bounds.
int validate_g_idx(const char* fn, MatArgs* a, const int32_t* g_idx, int64_t g_idx_len) {
  if (g_idx == nullptr) {
    if (g_idx_len != 0)
      return fail(QMM_ERR_INVALID_ARG, "%s: g_idx is NULL but g_idx_len=%lld. How to fix: pass "
                  "g_idx_len = 0 without group indices.", fn, (long long)g_idx_len);
    return QMM_OK;
  }
  const int64_t padded = a->kb * a->block_size;
  if (g_idx_len != a->K && g_idx_len != padded)
    return fail(QMM_ERR_INVALID_ARG, "%s: g_idx must have shape [%lld] or [%lld], got [%lld]. "
                "Why: the operator gives one group index per K element (optionally padded to "
                "whole blocks). How to fix: pass the g_idx tensor's length.", fn,
                (long long)a->K, (long long)padded, (long long)g_idx_len);
  if (((uintptr_t)g_idx & 3) != 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: g_idx must be 4-byte aligned (int32).", fn);
  if (a->tiled)
    return fail(QMM_ERR_UNSUPPORTED, "%s: group indices are supported on the operator's layout "
                "only. Why: the tiled buffer is laid out for block-contiguous groups. How to "
                "fix: pass the operator's B, scales and zero points (QMM_LAYOUT_ORT).", fn);
  if (a->bits == 3)
    return fail(QMM_ERR_UNSUPPORTED, "%s: group indices are not supported with 3-bit weights. "
                "Why: the group-index kernels read codes as one bit stream per row, the 3-bit "
                "blob holds two bit planes per block.", fn);
  a->g_idx = g_idx;
  return QMM_OK;
}

}  // namespace

namespace qmm {

int set_error(int code, const char* message) { return fail(code, "%s", message); }

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::tuple<int, const void*, int>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, kernel, bytes);
  if (done.count(key)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert(key);
  return e;
}

int gemm_compint8_impl(const char* fn, const void* A, int a_dtype, const uint8_t* B,
                       int b_layout, const void* scales, int s_dtype, const uint8_t* zero_points,
                       const int32_t* g_idx, int64_t g_idx_len, const void* bias, void* Y,
                       int64_t M, int64_t K, int64_t N, int block_size, int bits,
                       int accuracy_level, void* workspace, size_t workspace_bytes,
                       hipError_t (*resolve_workspace)(void**), void* stream) {
  MatArgs a;
  int st = validate_matmul(fn, Route::CompInt8, A, a_dtype, B, b_layout, scales, s_dtype,
                           zero_points, bias, Y, M, K, N, block_size, bits, accuracy_level, &a);
  if (st != QMM_OK) return st;
  st = validate_g_idx(fn, &a, g_idx, g_idx_len);
  if (st != QMM_OK) return st;
  if (a.g_idx != nullptr) {
    // As the operator routes it: with group indices the weight scale varies
    // inside an activation block, so there is no per-block integer dot; the
    // product is computed with float activations (the workspace is unused).
    if (M == 0) return QMM_OK;
    a.stream = (hipStream_t)stream;
    return hip_status(M == 1 ? launch_gemv(a) : launch_gemm(a), fn);
  }
  const bool small = M > 0 && compint8_small_supported(a);
  if (a.tiled && !small && !compint8_tiled_supported(a))
    return fail(QMM_ERR_UNSUPPORTED, "%s: on the tiled layout CompInt8 needs "
                "block_size >= 32 (64-code chunks holding one block, or two of 32) and at most 896 "
                "blocks per "
                "row, or M = 1 with a block of at least one 16-byte unit of codes and at most "
                "1024 codes (got M=%lld, block_size=%d, %lld blocks). How to fix: pass the "
                "operator's layout (QMM_LAYOUT_ORT) for this weight.", fn, (long long)M,
                block_size, (long long)a.kb);
  if (M == 0) return QMM_OK;
  if (resolve_workspace != nullptr) {
    const hipError_t e = resolve_workspace(&workspace);
    if (e != hipSuccess) return hip_status(e, fn);
  }
  st = check_workspace(fn, a, workspace, workspace_bytes);
  if (st != QMM_OK) return st;
  a.stream = (hipStream_t)stream;
  // M = 1 on the tiled layout: one launch that quantizes the activations in
  // LDS (the workspace is not touched).
  if (small) return hip_status(launch_compint8_small(a), fn);
  int8_t* qa = (int8_t*)workspace;
  float* sa = (float*)((char*)workspace + ws_qa_bytes(a.M, a.kb, a.block_size));
  hipError_t e = launch_quantize_a(a, qa, sa);
  if (e == hipSuccess) {
    // The int8 matrix cores where they are faster (compint8_tiled_preferred);
    // else 3-bit weights on the generic kernel, the rest on compint8_kernel.
    if (a.tiled || compint8_tiled_preferred(a)) e = launch_compint8_tiled(a, qa, sa);
    else if (a.bits == 3) e = launch_generic_int(a, qa, 1, sa, nullptr);
    else e = launch_compint8(a, qa, sa);
  }
  return hip_status(e, fn);
}

}  // namespace qmm

extern "C" {

const char* qmm_last_error(void) { return g_last_error.c_str(); }

int qmm_gemv(const void* A, int a_dtype, const uint8_t* B, int b_layout, const void* scales,
             int s_dtype, const uint8_t* zero_points, const int32_t* g_idx, int64_t g_idx_len,
             const void* bias, void* Y, int64_t K, int64_t N, int block_size, int bits,
             int accuracy_level, void* stream) {
  MatArgs a;
  int st = validate_matmul("qmm_gemv", Route::Float, A, a_dtype, B, b_layout, scales, s_dtype,
                           zero_points, bias, Y, 1, K, N, block_size, bits, accuracy_level, &a);
  if (st != QMM_OK) return st;
  st = validate_g_idx("qmm_gemv", &a, g_idx, g_idx_len);
  if (st != QMM_OK) return st;
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_gemv(a), "qmm_gemv");
}

int qmm_gemm(const void* A, int a_dtype, const uint8_t* B, int b_layout, const void* scales,
             int s_dtype, const uint8_t* zero_points, const int32_t* g_idx, int64_t g_idx_len,
             const void* bias, void* Y, int64_t M, int64_t K, int64_t N, int block_size,
             int bits, int accuracy_level, void* stream) {
  MatArgs a;
  int st = validate_matmul("qmm_gemm", Route::Float, A, a_dtype, B, b_layout, scales, s_dtype,
                           zero_points, bias, Y, M, K, N, block_size, bits, accuracy_level, &a);
  if (st != QMM_OK) return st;
  st = validate_g_idx("qmm_gemm", &a, g_idx, g_idx_len);
  if (st != QMM_OK) return st;
  a.stream = (hipStream_t)stream;
  if (M == 0) return QMM_OK;
  if (M == 1) return hip_status(qmm::launch_gemv(a), "qmm_gemm");
  return hip_status(qmm::launch_gemm(a), "qmm_gemm");
}

size_t qmm_compint8_workspace_size(int64_t M, int64_t K, int block_size) {
  if (M < 0 || K <= 0 || block_size <= 0) return 0;
  const int64_t kb = (K + block_size - 1) / block_size;
  return qmm::ws_total_bytes(M, kb, block_size);
}


int qmm_gemm_compint8(const void* A, int a_dtype, const uint8_t* B, int b_layout,
                      const void* scales, int s_dtype, const uint8_t* zero_points,
                      const int32_t* g_idx, int64_t g_idx_len, const void* bias, void* Y,
                      int64_t M, int64_t K, int64_t N, int block_size, int bits,
                      int accuracy_level, void* workspace, size_t workspace_bytes, void* stream) {
  return qmm::gemm_compint8_impl("qmm_gemm_compint8", A, a_dtype, B, b_layout, scales, s_dtype,
                                 zero_points, g_idx, g_idx_len, bias, Y, M, K, N, block_size, bits,
                                 accuracy_level, workspace, workspace_bytes, nullptr, stream);
}

int qmm_check_g_idx(const int32_t* g_idx, int64_t g_idx_len, int64_t K, int block_size) {
  const char* fn = "qmm_check_g_idx";
  if (g_idx == nullptr || K <= 0 || block_size < 16 || !is_pow2(block_size))
    return fail(QMM_ERR_INVALID_ARG, "%s: g_idx must be a non-null host array, K > 0 and "
                "block_size a power of two >= 16.", fn);
  const int64_t kb = (K + block_size - 1) / block_size;
  if (g_idx_len != K && g_idx_len != kb * block_size)
    return fail(QMM_ERR_INVALID_ARG, "%s: g_idx must have shape [%lld] or [%lld], got [%lld].",
                fn, (long long)K, (long long)(kb * block_size), (long long)g_idx_len);
  for (int64_t i = 0; i < g_idx_len; ++i)
    if (g_idx[i] < 0 || (int64_t)g_idx[i] >= kb)
      return fail(QMM_ERR_INVALID_ARG, "%s: g_idx[%lld]=%d is outside 0..%lld. Why: every "
                  "group index selects one of the kb = ceil(K / block_size) scales of a row. "
                  "How to fix: re-export the weight's group indices.", fn, (long long)i,
                  (int)g_idx[i], (long long)kb);
  return QMM_OK;
}

size_t qmm_int16_workspace_size(int64_t M, int64_t K, int block_size) {
  if (M < 0 || K <= 0 || block_size <= 0) return 0;
  const int64_t kb = (K + block_size - 1) / block_size;
  return qmm::ws16_total_bytes(M, kb, block_size);
}

// Shared by qmm_gemm_int16 and its block-dot export: validation, workspace,
// quantization, then the generic kernel (dots non-null: the export).
static int int16_impl(const char* fn, const void* A, int a_dtype, const uint8_t* B,
                      int b_layout, const void* scales, int s_dtype, const uint8_t* zero_points,
                      const void* bias, void* Y, int64_t M, int64_t K, int64_t N, int block_size,
                      int bits, void* workspace, size_t workspace_bytes, int32_t* dots,
                      void* stream) {
  MatArgs a;
  int st = validate_matmul(fn, Route::Float, A, a_dtype, B, b_layout, scales, s_dtype,
                           zero_points, bias, dots ? (void*)dots : Y, M, K, N, block_size, bits,
                           0, &a);
  if (st != QMM_OK) return st;
  if (a.tiled || block_size > 128)
    return fail(QMM_ERR_UNSUPPORTED, "%s: int16 activations run on the operator's layout with "
                "block_size <= 128 (got layout %d, block_size %d). Why: a block's dot of int16 "
                "activations and codes is exact in int32 up to 128 codes. How to fix: use "
                "qmm_gemm, or a smaller block.", fn, b_layout, block_size);
  if (M == 0) return QMM_OK;
  const size_t need = qmm::ws16_total_bytes(a.M, a.kb, a.block_size);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0)
    return fail(QMM_ERR_WORKSPACE, "%s: the workspace holds %zu bytes at %p, %zu are needed "
                "(256-byte aligned). Why: the int16 activations and their block scales are "
                "stored there. How to fix: pass qmm_int16_workspace_size(M, K, block_size) "
                "bytes.", fn, workspace_bytes, workspace, need);
  a.stream = (hipStream_t)stream;
  int16_t* qa = (int16_t*)workspace;
  float* sa = (float*)((char*)workspace + qmm::ws16_qa_bytes(a.M, a.kb, a.block_size));
  hipError_t e = hipSuccess;
  if (dots) e = hipMemsetAsync(dots, 0, (size_t)(a.M * a.N * a.kb) * sizeof(int32_t), a.stream);
  if (e == hipSuccess) e = qmm::launch_quantize_a16(a, qa, sa);
  if (e == hipSuccess) {
    // From M = 8 the int8 matrix cores with the activations split into two
    // int8 planes; else the generic kernel.
    e = qmm::int16_tiled_preferred(a) ? qmm::launch_int16_tiled(a, qa, sa, dots)
                                      : qmm::launch_generic_int(a, qa, 2, sa, dots);
  }
  return hip_status(e, fn);
}

int qmm_gemm_int16(const void* A, int a_dtype, const uint8_t* B, int b_layout,
                   const void* scales, int s_dtype, const uint8_t* zero_points, const void* bias,
                   void* Y, int64_t M, int64_t K, int64_t N, int block_size, int bits,
                   void* workspace, size_t workspace_bytes, void* stream) {
  return int16_impl("qmm_gemm_int16", A, a_dtype, B, b_layout, scales, s_dtype, zero_points,
                    bias, Y, M, K, N, block_size, bits, workspace, workspace_bytes, nullptr,
                    stream);
}

int qmm_debug_int16_block_dots(const void* A, int a_dtype, const uint8_t* B,
                               const uint8_t* zero_points, int64_t M, int64_t K, int64_t N,
                               int block_size, int bits, int32_t* dots, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (dots == nullptr)
    return fail(QMM_ERR_INVALID_ARG, "qmm_debug_int16_block_dots: dots must be non-null.");
  // Scales are not read by the block dots; B stands in for the pointer.
  return int16_impl("qmm_debug_int16_block_dots", A, a_dtype, B, QMM_LAYOUT_ORT, B, QMM_F32,
                    zero_points, nullptr, nullptr, M, K, N, block_size, bits, workspace,
                    workspace_bytes, dots, stream);
}

int qmm_gemm_fp4(const void* A, int a_dtype, const uint8_t* W, const uint8_t* scales,
                 int format, float global_scale, const void* bias, void* Y, int64_t M,
                 int64_t K, int64_t N, void* stream) {
  const char* fn = "qmm_gemm_fp4";
  if (format != QMM_MXFP4 && format != QMM_NVFP4)
    return fail(QMM_ERR_INVALID_ARG, "%s: format=%d is not a qmm_fp4_format. How to fix: pass "
                "QMM_MXFP4 (E8M0 scales per 32) or QMM_NVFP4 (E4M3 scales per 16).", fn, format);
  if (K <= 0 || N <= 0 || M < 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: K and N must be positive and M >= 0 (got M=%lld "
                "K=%lld N=%lld).", fn, (long long)M, (long long)K, (long long)N);
  if (dtype_size(a_dtype) == 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: a_dtype=%d is not a qmm_dtype. How to fix: pass "
                "QMM_F32, QMM_F16 or QMM_BF16.", fn, a_dtype);
  if (W == nullptr || scales == nullptr || (M > 0 && (A == nullptr || Y == nullptr)))
    return fail(QMM_ERR_INVALID_ARG, "%s: A, W, scales and Y must be non-null device "
                "pointers (bias may be NULL).", fn);
  if (!aligned(W, 16))
    return fail(QMM_ERR_INVALID_ARG, "%s: W must be 16-byte aligned. Why: the kernels read "
                "codes with 128-bit loads. How to fix: pass a freshly allocated tensor.", fn);
  const int asz = dtype_size(a_dtype);
  if (!aligned(A, asz) || !aligned(Y, asz) || !aligned(bias, asz))
    return fail(QMM_ERR_INVALID_ARG, "%s: A, Y and bias must be aligned to their element size.",
                fn);
  const int64_t bs = format == QMM_MXFP4 ? 32 : 16;
  const int64_t kb = (K + bs - 1) / bs;
  if (N * kb * bs / 2 + 64 > INT32_MAX / 2 || M * K > INT32_MAX / 2 || K > INT32_MAX / 4)
    return fail(QMM_ERR_UNSUPPORTED, "%s: the weight or activations are too large for 32-bit "
                "offsets. How to fix: split the matmul along N or M.", fn);
  if (M == 0) return QMM_OK;
  qmm::Fp4Args a;
  a.A = A; a.W = W; a.scales = scales; a.global_scale = global_scale; a.bias = bias; a.Y = Y;
  a.M = M; a.K = K; a.N = N; a.kb = kb; a.format = format; a.a_dtype = a_dtype;
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_fp4(a), fn);
}

int qmm_lowp_matmul(const uint8_t* lhs, const uint8_t* rhs, const void* lhs_scales,
                    const void* rhs_scales, const float* bias, float* out, int64_t m, int64_t n,
                    int64_t k, int layout, int lhs_format, int rhs_format, void* stream) {
  const char* fn = "qmm_lowp_matmul";
  if (layout < QMM_LOWP_PER_TENSOR || layout > QMM_LOWP_NVFP4)
    return fail(QMM_ERR_INVALID_ARG, "%s: layout=%d is not a qmm_lowp_layout. How to fix: pass "
                "QMM_LOWP_PER_TENSOR, QMM_LOWP_MX (E8M0 per 32) or QMM_LOWP_NVFP4 (E4M3 per 16).",
                fn, layout);
  for (int f : {lhs_format, rhs_format})
    if (f < QMM_LOWP_E4M3 || f > QMM_LOWP_E2M1)
      return fail(QMM_ERR_INVALID_ARG, "%s: format=%d is not a qmm_lowp_format. How to fix: pass "
                  "QMM_LOWP_E4M3, _E5M2, _E2M3, _E3M2 or _E2M1.", fn, f);
  if (n <= 0 || k <= 0 || m < 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: n and k must be positive and m >= 0 (got m=%lld "
                "n=%lld k=%lld).", fn, (long long)m, (long long)n, (long long)k);
  if (rhs == nullptr || lhs_scales == nullptr || rhs_scales == nullptr ||
      (m > 0 && (lhs == nullptr || out == nullptr)))
    return fail(QMM_ERR_INVALID_ARG, "%s: lhs, rhs, both scale tensors and out must be non-null "
                "device pointers (bias may be NULL).", fn);
  if (!aligned(out, 4) || !aligned(bias, 4) || (layout == QMM_LOWP_PER_TENSOR &&
      (!aligned(lhs_scales, 4) || !aligned(rhs_scales, 4))))
    return fail(QMM_ERR_INVALID_ARG, "%s: out, bias and f32 scales must be 4-byte aligned.", fn);
  if (m * k + 64 > INT32_MAX || n * k + 64 > INT32_MAX)
    return fail(QMM_ERR_UNSUPPORTED, "%s: m * k or n * k (%lld, %lld) reaches 2^31, past the "
                "kernels' 32-bit offsets. How to fix: split the matmul along m or n.", fn,
                (long long)(m * k), (long long)(n * k));
  if (m == 0) return QMM_OK;
  qmm::LowpArgs a;
  a.lhs = lhs; a.rhs = rhs; a.lsc = lhs_scales; a.rsc = rhs_scales; a.bias = bias; a.out = out;
  a.m = m; a.n = n; a.k = k; a.layout = layout; a.lfmt = lhs_format; a.rfmt = rhs_format;
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_lowp_matmul(a), fn);
}

int qmm_lowp_quantize(const void* x, int x_dtype, int64_t rows, int64_t cols, int format,
                      int layout, uint8_t* codes, void* scales, void* stream) {
  const char* fn = "qmm_lowp_quantize";
  if (layout < QMM_LOWP_PER_TENSOR || layout > QMM_LOWP_NVFP4)
    return fail(QMM_ERR_INVALID_ARG, "%s: layout=%d is not a qmm_lowp_layout. How to fix: pass "
                "QMM_LOWP_PER_TENSOR, QMM_LOWP_MX or QMM_LOWP_NVFP4.", fn, layout);
  if (format < QMM_LOWP_E4M3 || format > QMM_LOWP_E2M1)
    return fail(QMM_ERR_INVALID_ARG, "%s: format=%d is not a qmm_lowp_format. How to fix: pass "
                "QMM_LOWP_E4M3, _E5M2, _E2M3, _E3M2 or _E2M1.", fn, format);
  if (dtype_size(x_dtype) == 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: x_dtype=%d is not a qmm_dtype. How to fix: pass "
                "QMM_F32, QMM_F16 or QMM_BF16.", fn, x_dtype);
  if (cols <= 0 || rows < 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: cols must be positive and rows >= 0 (got rows=%lld "
                "cols=%lld).", fn, (long long)rows, (long long)cols);
  if (rows > 0 && (x == nullptr || codes == nullptr || scales == nullptr))
    return fail(QMM_ERR_INVALID_ARG, "%s: x, codes and scales must be non-null device "
                "pointers.", fn);
  if (!aligned(x, dtype_size(x_dtype)) || (layout == QMM_LOWP_PER_TENSOR && !aligned(scales, 4)))
    return fail(QMM_ERR_INVALID_ARG, "%s: x must be aligned to its element size and a per-tensor "
                "scale to 4 bytes.", fn);
  if (rows * cols + 64 > INT32_MAX)
    return fail(QMM_ERR_UNSUPPORTED, "%s: rows * cols (%lld) reaches 2^31. How to fix: quantize "
                "in row slices.", fn, (long long)(rows * cols));
  if (rows == 0) return QMM_OK;
  qmm::LowpQuantArgs a;
  a.x = x; a.codes = codes; a.scales = scales; a.rows = rows; a.cols = cols;
  a.x_dtype = x_dtype; a.fmt = format; a.layout = layout; a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_lowp_quantize(a), fn);
}

int qconv_int8(const int8_t* X, const int8_t* Wt, const int32_t* bias, const float* w_scale,
               float in_scale, float out_scale, int in_zp, int out_zp, int clamp_min,
               int clamp_max, int Nb, int H, int W, int C, int Co, int KH, int KW, int stride_h,
               int stride_w, int pad_h, int pad_w, int8_t* Y, void* stream) {
  const char* fn = "qconv_int8";
  if (X == nullptr || Wt == nullptr || w_scale == nullptr || Y == nullptr)
    return fail(QMM_ERR_INVALID_ARG, "%s: X, Wt, w_scale and Y must be non-null device "
                "pointers (bias may be NULL).", fn);
  if (Nb < 1 || H < 1 || W < 1 || C < 1 || Co < 1 || KH < 1 || KW < 1 || stride_h < 1 ||
      stride_w < 1 || pad_h < 0 || pad_w < 0)
    return fail(QMM_ERR_INVALID_ARG, "%s: sizes, kernel and strides must be >= 1 and pads >= 0 "
                "(got Nb=%d H=%d W=%d C=%d Co=%d KH=%d KW=%d stride=%d,%d pad=%d,%d).", fn, Nb, H,
                W, C, Co, KH, KW, stride_h, stride_w, pad_h, pad_w);
  if (H + 2 * pad_h < KH || W + 2 * pad_w < KW)
    return fail(QMM_ERR_INVALID_ARG, "%s: the padded input (%dx%d) is smaller than the kernel "
                "(%dx%d), so there is no output pixel.", fn, H + 2 * pad_h, W + 2 * pad_w, KH, KW);
  if (in_zp < -128 || in_zp > 127 || clamp_min < -128 || clamp_max > 127 || clamp_min > clamp_max)
    return fail(QMM_ERR_INVALID_ARG, "%s: in_zp must be an int8 value and -128 <= clamp_min <= "
                "clamp_max <= 127 (got in_zp=%d clamp=[%d,%d]). Why: the output is int8; a ReLU "
                "is clamp_min = out_zp.", fn, in_zp, clamp_min, clamp_max);
  if (!(out_scale != 0.0f) || !(in_scale == in_scale))
    return fail(QMM_ERR_INVALID_ARG, "%s: out_scale must be nonzero and the scales must not be "
                "NaN. Why: the requantization multiplier is (in_scale * w_scale) / out_scale.", fn);
  const int64_t K = (int64_t)KH * KW * C;
  const int64_t OH = (H + 2 * pad_h - KH) / stride_h + 1, OW = (W + 2 * pad_w - KW) / stride_w + 1;
  if (K * 128 * 128 >= (int64_t)1 << 31 || (int64_t)Nb * OH * OW * Co >= (int64_t)1 << 31 ||
      (int64_t)Nb * H * W * C >= (int64_t)1 << 31)
    return fail(QMM_ERR_UNSUPPORTED, "%s: the reduction (KH*KW*C = %lld) or a tensor is too large "
                "for the exact int32 accumulator / 32-bit indices. How to fix: split the "
                "convolution.", fn, (long long)K);
  qmm::ConvArgs c;
  c.X = X; c.Wt = Wt; c.bias = bias; c.w_scale = w_scale;
  c.in_scale = in_scale; c.out_scale = out_scale; c.in_zp = in_zp; c.out_zp = out_zp;
  c.clamp_min = clamp_min; c.clamp_max = clamp_max;
  c.Nb = Nb; c.H = H; c.W = W; c.C = C; c.Co = Co; c.KH = KH; c.KW = KW;
  c.stride_h = stride_h; c.stride_w = stride_w; c.pad_h = pad_h; c.pad_w = pad_w;
  c.Y = Y;
  c.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_conv_int8(c), fn);
}

size_t qmm_repacked_bytes(int64_t K, int64_t N, int block_size, int bits, int s_dtype,
                          int has_zero_points) {
  if (K <= 0 || N <= 0 || block_size < 16 || !is_pow2(block_size) ||
      (bits != 2 && bits != 4 && bits != 8) || dtype_size(s_dtype) == 0)
    return 0;
  return (size_t)qmm::tiled_geom(K, N, block_size, bits, dtype_size(s_dtype),
                                 has_zero_points != 0).total;
}

int qmm_repack(const uint8_t* B, const void* scales, int s_dtype, const uint8_t* zero_points,
               int64_t K, int64_t N, int block_size, int bits, void* out, size_t out_bytes,
               void* stream) {
  MatArgs a;
  int st = validate_matmul("qmm_repack", Route::Float, B, QMM_BF16, B, QMM_LAYOUT_ORT, scales,
                           s_dtype, zero_points, nullptr, (void*)B, 0, K, N, block_size, bits, 0,
                           &a);
  if (st != QMM_OK) return st;
  if (bits == 3)
    return fail(QMM_ERR_UNSUPPORTED, "qmm_repack: 3-bit weights have no tiled layout. How to "
                "fix: pass the operator's layout to the matmuls.");
  const size_t need = qmm_repacked_bytes(K, N, block_size, bits, s_dtype, zero_points != nullptr);
  if (out == nullptr || out_bytes < need || ((uintptr_t)out & 255) != 0)
    return fail(QMM_ERR_INVALID_ARG, "qmm_repack: out must be a 256-byte aligned device buffer "
                "of at least %zu bytes (got %zu at %p). How to fix: allocate "
                "qmm_repacked_bytes(K, N, block_size, bits, s_dtype, has_zero_points) bytes.",
                need, out_bytes, out);
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_repack(a, (uint8_t*)out, false, nullptr, nullptr, nullptr),
                    "qmm_repack");
}

int qmm_unrepack(const void* tiled, int has_zero_points, int64_t K, int64_t N, int block_size,
                 int bits, int s_dtype, uint8_t* B, void* scales, uint8_t* zero_points,
                 void* stream) {
  MatArgs a;
  int st = validate_matmul("qmm_unrepack", Route::Float, B, QMM_BF16, B, QMM_LAYOUT_ORT, scales,
                           s_dtype, nullptr, nullptr, (void*)B, 0, K, N, block_size, bits, 0, &a);
  if (st != QMM_OK) return st;
  if (bits == 3)
    return fail(QMM_ERR_UNSUPPORTED, "qmm_unrepack: 3-bit weights have no tiled layout.");
  if (tiled == nullptr || ((uintptr_t)tiled & 255) != 0 || (has_zero_points && !zero_points))
    return fail(QMM_ERR_INVALID_ARG, "qmm_unrepack: tiled must be a 256-byte aligned repacked "
                "buffer, and zero_points non-NULL when it holds zero points.");
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_repack(a, (uint8_t*)tiled, true, B, scales,
                                       has_zero_points ? zero_points : nullptr),
                    "qmm_unrepack");
}

int qmm_debug_unpack(const uint8_t* B, int b_layout, const void* scales, int s_dtype,
                     const uint8_t* zero_points, int64_t K, int64_t N, int block_size, int bits,
                     uint8_t* codes, uint8_t* zps, float* w, void* stream) {
  MatArgs a;
  if (b_layout != QMM_LAYOUT_ORT)
    return fail(QMM_ERR_UNSUPPORTED, "qmm_debug_unpack: only the operator's layout is decoded "
                "here. How to fix: qmm_unrepack the buffer first.");
  // Validate as a matmul with a dummy activation/output (never touched).
  const void* dummy = B;
  if (w != nullptr && scales == nullptr)
    return fail(QMM_ERR_INVALID_ARG, "qmm_debug_unpack: scales are required to write w.");
  int st = validate_matmul("qmm_debug_unpack", Route::Float, dummy, QMM_BF16, B, b_layout,
                           scales ? scales : dummy, scales ? s_dtype : QMM_BF16, zero_points,
                           nullptr, (void*)dummy, 0, K, N, block_size, bits, 0, &a);
  if (st != QMM_OK) return st;
  a.scales = scales;
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_unpack(a, codes, zps, w), "qmm_debug_unpack");
}

int qmm_debug_quantize_a(const void* A, int a_dtype, int64_t M, int64_t K, int block_size,
                         int8_t* qa, float* sa, void* stream) {
  if (qa == nullptr || sa == nullptr)
    return fail(QMM_ERR_INVALID_ARG, "qmm_debug_quantize_a: qa and sa must be non-null.");
  MatArgs a;
  static const uint8_t* const kAligned = reinterpret_cast<const uint8_t*>(256);
  int st = validate_matmul("qmm_debug_quantize_a", Route::CompInt8, A, a_dtype, kAligned, 0,
                           kAligned, QMM_F32, nullptr, nullptr, (void*)qa, M, K, 1, block_size,
                           4, 4, &a);
  if (st != QMM_OK) return st;
  if (M == 0) return QMM_OK;
  a.stream = (hipStream_t)stream;
  return hip_status(qmm::launch_quantize_a(a, qa, sa), "qmm_debug_quantize_a");
}

int qmm_debug_compint8_block_dots(const void* A, int a_dtype, const uint8_t* B, int b_layout,
                                  int s_dtype, const uint8_t* zero_points, int64_t M, int64_t K,
                                  int64_t N, int block_size, int bits, int32_t* dots,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  if (dots == nullptr)
    return fail(QMM_ERR_INVALID_ARG, "qmm_debug_compint8_block_dots: dots must be non-null.");
  MatArgs a;
  const bool tiled = b_layout == QMM_LAYOUT_TILED || b_layout == QMM_LAYOUT_TILED_ZP;
  int st = validate_matmul("qmm_debug_compint8_block_dots", Route::CompInt8, A, a_dtype, B,
                           b_layout, tiled ? nullptr : B, tiled ? s_dtype : QMM_F32, zero_points,
                           nullptr, (void*)dots, M, K, N, block_size, bits, 4, &a);
  if (st != QMM_OK) return st;
  // The route qmm_gemm_compint8 takes for the same arguments.
  const bool small = M > 0 && qmm::compint8_small_supported(a);
  if (a.tiled && !small && !qmm::compint8_tiled_supported(a))
    return fail(QMM_ERR_UNSUPPORTED, "qmm_debug_compint8_block_dots: on the tiled layout "
                "CompInt8 needs block_size >= 32, or M = 1 with a block of at least one 16-byte "
                "unit of codes. How to fix: pass the operator's layout.");
  if (M == 0) return QMM_OK;
  st = check_workspace("qmm_debug_compint8_block_dots", a, workspace, workspace_bytes);
  if (st != QMM_OK) return st;
  if (!a.tiled) a.scales = nullptr;   // the block dots need no scales
  a.Y = nullptr;
  a.stream = (hipStream_t)stream;
  int8_t* qa = (int8_t*)workspace;
  float* sa = (float*)((char*)workspace + qmm::ws_qa_bytes(a.M, a.kb, a.block_size));
  hipError_t e = hipMemsetAsync(dots, 0, (size_t)(a.M * a.N * a.kb) * sizeof(int32_t), a.stream);
  if (small) {
    // One launch: the kernel quantizes in LDS and writes its qa / sa to the
    // workspace beside the dots.
    if (e == hipSuccess) e = qmm::launch_compint8_small_dots(a, qa, sa, dots);
    return hip_status(e, "qmm_debug_compint8_block_dots");
  }
  if (e == hipSuccess) e = qmm::launch_quantize_a(a, qa, sa);
  if (e == hipSuccess) {
    if (a.tiled || qmm::compint8_tiled_preferred(a))
      e = qmm::launch_compint8_tiled_dots(a, qa, sa, dots);
    else if (a.bits == 3) e = qmm::launch_generic_int(a, qa, 1, sa, dots);
    else e = qmm::launch_compint8_dots(a, qa, sa, dots);
  }
  return hip_status(e, "qmm_debug_compint8_block_dots");
}

}  // extern "C"
