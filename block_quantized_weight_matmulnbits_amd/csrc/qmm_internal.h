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
  const void* bias = nullptr;     // [N] a_dtype or null
  void* Y = nullptr;              // [M, N] a_dtype
  int64_t M = 1, K = 0, N = 0;
  int64_t block_size = 0, kb = 0, blob = 0, zp_row_bytes = 0;
  int bits = 4;
  int a_dtype = 0, s_dtype = 0;
  void* workspace = nullptr;
  size_t workspace_bytes = 0;
  hipStream_t stream = nullptr;
};
using GemvArgs = MatArgs;

hipError_t launch_gemv(const MatArgs& a);

}  // namespace qmm
