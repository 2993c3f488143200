// step.cpp -- a fixed sequence of matmul calls (for example the projections
// of one decode step) recorded once and replayed as one HIP graph.
//
// The pages' end-to-end decode measurements put the time lost outside the
// kernels: per-operator fork/join and dispatch, not the matmul itself, made
// decode 2.3x slower than it needed to be, and a persistent pool raised it
// from 6 to 28 tok/s (onnx-runtime-ep-cpu matmul_nbits.rs, module notes on
// the decode step and the persistent decode pool).  On a GPU the same cost is
// the host's work per launch: each qmm_gemv call validates its arguments and
// enqueues one kernel, microseconds that a small projection's kernel does
// not cover.  A step pays it once: qmm_step_finalize validates every
// recorded call and captures their launches into a graph; qmm_step_launch is
// one hipGraphLaunch.  The replayed kernels and their arguments (pointers
// included) are exactly those of the direct calls; callers change inputs in
// place between launches.  The calls contain no memory-set operations.
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <functional>
#include <string>
#include <vector>

#include "../../include/qmm.h"
#include "qmm_internal.h"

struct qmm_step {
  // Each recorded call enqueues itself on the given stream and returns a
  // qmm_status (validation included).
  std::vector<std::function<int(void*)>> calls;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int device = -1;
};

namespace {

int step_error(int code, const char* fmt, long long v) {
  char msg[512];
  snprintf(msg, sizeof(msg), fmt, v);
  return qmm::set_error(code, msg);
}

int add_call(qmm_step* step, std::function<int(void*)> call) {
  if (step == nullptr) return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step: step is NULL.");
  if (step->exec != nullptr)
    return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step_add_*: the step was already "
                          "finalized. How to fix: record every call before qmm_step_finalize.");
  step->calls.push_back(std::move(call));
  return QMM_OK;
}

}  // namespace

extern "C" {

int qmm_step_create(qmm_step** step) {
  if (step == nullptr) return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step_create: step is NULL.");
  *step = new qmm_step();
  return QMM_OK;
}

int qmm_step_add_gemv(qmm_step* step, const void* A, int a_dtype, const uint8_t* B,
                      int b_layout, const void* scales, int s_dtype, const uint8_t* zero_points,
                      const int32_t* g_idx, int64_t g_idx_len, const void* bias, void* Y,
                      int64_t K, int64_t N, int block_size, int bits, int accuracy_level) {
  return add_call(step, [=](void* s) {
    return qmm_gemv(A, a_dtype, B, b_layout, scales, s_dtype, zero_points, g_idx, g_idx_len,
                    bias, Y, K, N, block_size, bits, accuracy_level, s);
  });
}

int qmm_step_add_gemm(qmm_step* step, const void* A, int a_dtype, const uint8_t* B,
                      int b_layout, const void* scales, int s_dtype, const uint8_t* zero_points,
                      const int32_t* g_idx, int64_t g_idx_len, const void* bias, void* Y,
                      int64_t M, int64_t K, int64_t N, int block_size, int bits,
                      int accuracy_level) {
  return add_call(step, [=](void* s) {
    return qmm_gemm(A, a_dtype, B, b_layout, scales, s_dtype, zero_points, g_idx, g_idx_len,
                    bias, Y, M, K, N, block_size, bits, accuracy_level, s);
  });
}

int qmm_step_add_gemm_compint8(qmm_step* step, const void* A, int a_dtype, const uint8_t* B,
                               int b_layout, const void* scales, int s_dtype,
                               const uint8_t* zero_points, const int32_t* g_idx,
                               int64_t g_idx_len, const void* bias, void* Y, int64_t M,
                               int64_t K, int64_t N, int block_size, int bits,
                               int accuracy_level, void* workspace, size_t workspace_bytes) {
  return add_call(step, [=](void* s) {
    return qmm_gemm_compint8(A, a_dtype, B, b_layout, scales, s_dtype, zero_points, g_idx,
                             g_idx_len, bias, Y, M, K, N, block_size, bits, accuracy_level,
                             workspace, workspace_bytes, s);
  });
}

int qmm_step_finalize(qmm_step* step) {
  if (step == nullptr) return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step_finalize: step is NULL.");
  if (step->exec != nullptr) return QMM_OK;
  if (step->calls.empty())
    return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step_finalize: no call was recorded.");
  hipError_t e = hipGetDevice(&step->device);
  hipStream_t cs = nullptr;
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
  if (e != hipSuccess) {
    if (cs) (void)hipStreamDestroy(cs);
    return step_error(QMM_ERR_HIP, "qmm_step_finalize: could not start a graph capture (HIP "
                      "error %lld).", (long long)e);
  }
  int st = QMM_OK;
  size_t failed = 0;
  for (size_t i = 0; i < step->calls.size() && st == QMM_OK; ++i) {
    st = step->calls[i](cs);
    failed = i;
  }
  hipGraph_t graph = nullptr;
  const hipError_t ec = hipStreamEndCapture(cs, &graph);
  (void)hipStreamDestroy(cs);
  if (st != QMM_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    // Keep the failing call's message, prefixed with its position.
    std::string msg = "qmm_step_finalize: recorded call " + std::to_string(failed) + " failed: " +
                      qmm_last_error();
    return qmm::set_error(st, msg.c_str());
  }
  if (ec != hipSuccess || graph == nullptr)
    return step_error(QMM_ERR_HIP, "qmm_step_finalize: the graph capture failed (HIP error "
                      "%lld).", (long long)ec);
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(graph);
    return step_error(QMM_ERR_HIP, "qmm_step_finalize: hipGraphInstantiate failed (HIP error "
                      "%lld).", (long long)e);
  }
  step->graph = graph;
  step->exec = exec;
  return QMM_OK;
}

int qmm_step_launch(const qmm_step* step, void* stream) {
  if (step == nullptr || step->exec == nullptr)
    return qmm::set_error(QMM_ERR_INVALID_ARG, "qmm_step_launch: the step is NULL or not "
                          "finalized. How to fix: call qmm_step_finalize first.");
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess && dev != step->device)
    return step_error(QMM_ERR_INVALID_ARG, "qmm_step_launch: the step was finalized on device "
                      "%lld, another device is current.", (long long)step->device);
  const hipError_t e = hipGraphLaunch(step->exec, (hipStream_t)stream);
  if (e != hipSuccess)
    return step_error(QMM_ERR_HIP, "qmm_step_launch: hipGraphLaunch failed (HIP error %lld).",
                      (long long)e);
  return QMM_OK;
}

int qmm_step_size(const qmm_step* step) {
  return step == nullptr ? 0 : (int)step->calls.size();
}

void qmm_step_destroy(qmm_step* step) {
  if (step == nullptr) return;
  if (step->exec) (void)hipGraphExecDestroy(step->exec);
  if (step->graph) (void)hipGraphDestroy(step->graph);
  delete step;
}

}  // extern "C"
