// compint8_noalloc.hip -- qmm_gemm_compint8_noalloc: the CompInt8 matmul
// with its workspace (the int8 activations and their per-block scales that
// pass between the quantization launch and the block-dot launch) in a fixed
// device array of the library instead of caller memory, for callers that
// cannot allocate device memory.  The kernels, routes and results are those
// of qmm_gemm_compint8.
//
// The array is a module global, so every device the library runs on holds
// its own copy (QMM_NOALLOC_SCRATCH_BYTES) from module load until the process
// ends.  In host code the array's name is only a host-side handle: its
// device address is looked up once per device, with that device current,
// and that address is what the kernels receive.  All calls on one device
// share the array and it keeps the last call's contents; every byte a call
// reads was written earlier in the same call, so nothing needs clearing.
// Calls that overlap on one device (other streams, other host threads
// without ordering) race on it.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <mutex>

#include "../../include/qmm.h"
#include "qmm_internal.h"

namespace {

static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of scratch, per device

// The current device's address of scratch, looked up on the device's first
// call (hipGetSymbolAddress with the device current) and kept.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int qmm_gemm_compint8_noalloc(const void* A, int a_dtype, const uint8_t* B,
                                         int b_layout, const void* scales, int s_dtype,
                                         const uint8_t* zero_points, const int32_t* g_idx,
                                         int64_t g_idx_len, const void* bias, void* Y, int64_t M,
                                         int64_t K, int64_t N, int block_size, int bits,
                                         int accuracy_level, void* stream) {
  const size_t need = qmm_compint8_workspace_size(M, K, block_size);
  if (need > (size_t)QMM_NOALLOC_SCRATCH_BYTES) {
    char msg[512];
    snprintf(msg, sizeof(msg),
             "qmm_gemm_compint8_noalloc: M=%lld, K=%lld, block_size=%d need %zu bytes of "
             "workspace, more than the library's fixed %d-byte device array. Why: this entry "
             "point allocates nothing and has only that array. How to fix: split A into row "
             "batches that fit, or call qmm_gemm_compint8 with a workspace of "
             "qmm_compint8_workspace_size(M, K, block_size) bytes.",
             (long long)M, (long long)K, block_size, need, (int)QMM_NOALLOC_SCRATCH_BYTES);
    return qmm::set_error(QMM_ERR_WORKSPACE, msg);
  }
  return qmm::gemm_compint8_impl("qmm_gemm_compint8_noalloc", A, a_dtype, B, b_layout, scales,
                                 s_dtype, zero_points, g_idx, g_idx_len, bias, Y, M, K, N,
                                 block_size, bits, accuracy_level, nullptr,
                                 (size_t)QMM_NOALLOC_SCRATCH_BYTES, scratch_address, stream);
}
