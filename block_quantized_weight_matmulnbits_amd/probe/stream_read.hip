// stream_read.hip -- a plain streaming read of device memory, the reference
// the benchmark times beside a memory-bound kernel: the time one launch
// needs just to read the same number of bytes on this GPU.
//
// Every thread reads 16-byte words with non-temporal loads, two per
// iteration of a grid-stride loop, xors them together and writes one word,
// so nothing is optimized away.  Built into its own library (libqmm_probe.so);
// the matmul library does not contain it.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read_kernel(const probe_u32x4* __restrict__ src,
                                                          int64_t n16,
                                                          uint32_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nth = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = tid; i < n16; i += 2 * nth) {
    const probe_u32x4 a = __builtin_nontemporal_load(src + i);
    const probe_u32x4 b = i + nth < n16 ? __builtin_nontemporal_load(src + i + nth)
                                        : probe_u32x4{0, 0, 0, 0};
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
  }
  out[tid] = acc;
}

// Reads nbytes (a multiple of 16) from src; out holds grid * 256 words.
// Returns 0 or the HIP error code.
extern "C" int qmm_probe_stream_read(const void* src, int64_t nbytes, void* out, int grid,
                                     void* stream) {
  if (src == nullptr || out == nullptr || nbytes < 0 || nbytes % 16 != 0 || grid <= 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     (const probe_u32x4*)src, nbytes / 16, (uint32_t*)out);
  return (int)hipGetLastError();
}
