// stream_read.hip -- a plain streaming read of device memory: the reference
// the benchmark times beside its memory-bound kernels, to measure what one
// launch of a given size can read on this GPU.  Measurement code only; the
// matmul library does not contain it.
//
// Every thread reads 16-byte words, U loads issued back to back before any
// is consumed (U words in flight per lane), xors them together and writes
// one word per thread so nothing is optimized away.  Two access orders:
//   stride: a grid-stride loop (iteration i of thread t reads words
//           t + (i * U + u) * threads);
//   slab:   each workgroup owns one contiguous slab of ceil(words / grid)
//           words and its threads walk it in block-wide steps (the order of
//           a GEMV whose waves own contiguous shares of the weight).
// Loads are either non-temporal or plain.  Every load is guarded by the
// word count, so any grid and block size stay in bounds.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t probe_u32x4 __attribute__((ext_vector_type(4)));

template <bool NT>
__device__ __forceinline__ probe_u32x4 probe_load(const probe_u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int U, bool NT, bool SLAB>
__global__ __launch_bounds__(1024) void stream_read_kernel(const probe_u32x4* __restrict__ src,
                                                           int64_t n16,
                                                           uint32_t* __restrict__ out) {
  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t lo, hi, step, first;
  if constexpr (SLAB) {
    const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
    lo = (int64_t)blockIdx.x * per;
    hi = lo + per < n16 ? lo + per : n16;
    step = blockDim.x;
    first = lo + threadIdx.x;
  } else {
    lo = 0;
    hi = n16;
    step = (int64_t)gridDim.x * blockDim.x;
    first = tid;
  }
  uint32_t acc = 0;
  for (int64_t i = first; i < hi; i += step * U) {
    probe_u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = i + (int64_t)u * step;
      v[u] = j < hi ? probe_load<NT>(src + j) : probe_u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[tid] = acc;
}

template <int U, bool NT>
static hipError_t launch_u(bool slab, const probe_u32x4* src, int64_t n16, uint32_t* out,
                           int grid, int block, hipStream_t s) {
  if (slab)
    hipLaunchKernelGGL((stream_read_kernel<U, NT, true>), dim3(grid), dim3(block), 0, s, src,
                       n16, out);
  else
    hipLaunchKernelGGL((stream_read_kernel<U, NT, false>), dim3(grid), dim3(block), 0, s, src,
                       n16, out);
  return hipGetLastError();
}

template <bool NT>
static hipError_t launch_nt(int unroll, bool slab, const probe_u32x4* src, int64_t n16,
                            uint32_t* out, int grid, int block, hipStream_t s) {
  switch (unroll) {
    case 1: return launch_u<1, NT>(slab, src, n16, out, grid, block, s);
    case 2: return launch_u<2, NT>(slab, src, n16, out, grid, block, s);
    case 4: return launch_u<4, NT>(slab, src, n16, out, grid, block, s);
    case 8: return launch_u<8, NT>(slab, src, n16, out, grid, block, s);
    default: return launch_u<16, NT>(slab, src, n16, out, grid, block, s);
  }
}

// Reads nbytes (a multiple of 16) from src with grid workgroups of block
// threads; out must hold grid * block 32-bit words (out_words).  unroll in
// {1, 2, 4, 8, 16}; block a multiple of 64 in [64, 1024].  Returns 0 or a
// HIP error code (invalid arguments: hipErrorInvalidValue, nothing launched).
extern "C" int qmm_probe_stream_read(const void* src, int64_t nbytes, void* out,
                                     int64_t out_words, int grid, int block, int unroll,
                                     int nontemporal, int slab, void* stream) {
  if (src == nullptr || out == nullptr || nbytes < 0 || nbytes % 16 != 0 || grid <= 0 ||
      block < 64 || block > 1024 || block % 64 != 0 ||
      (int64_t)grid * block > out_words ||
      (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8 && unroll != 16))
    return (int)hipErrorInvalidValue;
  const hipStream_t s = (hipStream_t)stream;
  const probe_u32x4* p = (const probe_u32x4*)src;
  uint32_t* o = (uint32_t*)out;
  return (int)(nontemporal ? launch_nt<true>(unroll, slab != 0, p, nbytes / 16, o, grid, block, s)
                           : launch_nt<false>(unroll, slab != 0, p, nbytes / 16, o, grid, block, s));
}
