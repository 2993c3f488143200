// generic.hip -- one operator-layout kernel for the code widths and
// activation types the specialized kernels do not take: 3-bit weights
// (float, int8 and int16 activations) and int16 activations (any width).
//
// Definitions:
//  * Float activations (onnx-runtime-ep-cpu matmul_nbits.rs: module
//    documentation, dequantize_nbits_value): y = sum_b s[n,b] *
//    sum_{k in b} x[k] * (code - zp), fp32.
//  * int8 (CompInt8) or int16 activations, quantized per block beforehand
//    (quantize_a_kernel): dot[m,n,b] = sum_{k in b} qa * (code - zp), exact
//    int32, y = sum_b float(dot) * (sa[m,b] * s[n,b]).  The int16 route is the
//    8-bit route of execute on that page (activations quantized to int16 per
//    K-block, an integer dot against the codes); with |qa| <= 32767 and
//    |code - zp| <= 255 the dot of a block of at most 128 codes is exact in
//    int32.
//  * 3-bit codes (MNN ConvInt8TiledExecutor.cpp, the 3-bit weight reorder):
//    a block's blob is bs/4 bytes of the low two bits of each code (LSB
//    first) then bs/8 bytes of the high bits; zero points are one LSB-first
//    3-bit stream per row; default zero point 4.
//
// Work split: a workgroup of 4 waves owns 4 * R output columns; a wave walks
// the blocks of its R columns with one lane per block (lanes stride over the
// row's blocks), so each block's sum is formed in one lane and scaled once.
// The activations of MT rows (MT = 1 for a single row) are staged in LDS per
// chunk of up to 64 whole blocks (fp32 values, or the int8 / int16 codes
// widened to int32), each block followed by one pad word: lane l reads block
// l of the chunk at a stride of bs + 1 words, an odd stride, so the 64 lanes
// of a read hit 64 different banks.
#include <algorithm>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

enum : int { ACT_F = 0, ACT_I8 = 1, ACT_I16 = 2 };
constexpr int GN_R = 4;          // output columns per wave

// 16 codes of a block, starting at code i0 (a multiple of 16) of the block
// whose blob starts at `blk` (bs codes).
template <int BITS>
__device__ __forceinline__ void codes16(const uint8_t* __restrict__ blk, int bs, int i0,
                                        int (&c)[16]) {
  if constexpr (BITS == 3) {
    // A blob of 3 bs / 8 bytes is even-sized, so both planes are 2-aligned.
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(blk + i0 / 4);  // 2 bits per code
    const uint32_t l = (uint32_t)lo[0] | ((uint32_t)lo[1] << 16);
    const uint32_t h = *reinterpret_cast<const uint16_t*>(blk + bs / 4 + i0 / 8);  // 1 bit
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = (int)(((l >> (2 * j)) & 3u) | (((h >> j) & 1u) << 2));
  } else {
    constexpr int P = 32 / BITS;
    constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
    const uint32_t* w = reinterpret_cast<const uint32_t*>(blk + i0 * BITS / 8);
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = (int)((w[j / P] >> ((j % P) * BITS)) & m);
  }
}

// The raw 32-bit words of 16 codes (starting at code i0, a multiple of 16)
// of the block whose blob starts at blk: 3-bit: the 2-bit plane's word and
// the 1-bit plane's 16 bits; otherwise 16 * BITS / 32 code words.
template <int BITS>
struct Raw16 {
  static constexpr int W = BITS == 3 ? 2 : 16 * BITS / 32;
};
template <int BITS>
__device__ __forceinline__ void load_raw16(const uint8_t* __restrict__ blk, int bs, int i0,
                                           uint32_t (&w)[Raw16<BITS>::W]) {
  // Codes are read once: non-temporal loads.
  if constexpr (BITS == 3) {
    const uint16_t* lo = reinterpret_cast<const uint16_t*>(blk + i0 / 4);
    w[0] = (uint32_t)__builtin_nontemporal_load(lo) | ((uint32_t)__builtin_nontemporal_load(lo + 1) << 16);
    w[1] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(blk + bs / 4 + i0 / 8));
  } else {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(blk + i0 * BITS / 8);
#pragma unroll
    for (int i = 0; i < Raw16<BITS>::W; ++i) w[i] = __builtin_nontemporal_load(p + i);
  }
}
template <int BITS>
__device__ __forceinline__ void decode16(const uint32_t (&w)[Raw16<BITS>::W], int (&c)[16]) {
  if constexpr (BITS == 3) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      c[j] = (int)(((w[0] >> (2 * j)) & 3u) | (((w[1] >> j) & 1u) << 2));
  } else {
    constexpr int P = 32 / BITS;
    constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
#pragma unroll
    for (int j = 0; j < 16; ++j) c[j] = (int)((w[j / P] >> ((j % P) * BITS)) & m);
  }
}

// (code - zp) of 16 codes as eight int16 pairs (codes 2v, 2v + 1 in the low
// and high halves of pair v), for v_dot2_i32_i16 against int16 activation
// pairs.  8-bit and 4-bit codes are moved into 16-bit lanes with byte
// permutes; the other widths are decoded first.  |code - zp| <= 255.
typedef short short2_t __attribute__((ext_vector_type(2)));
template <int BITS>
__device__ __forceinline__ void code_pairs16(const uint32_t (&w)[Raw16<BITS>::W], int z,
                                             uint32_t (&pr)[8]) {
  if constexpr (BITS == 8) {
#pragma unroll
    for (int v = 0; v < 8; ++v)
      pr[v] = __builtin_amdgcn_perm(0u, w[v / 2], (v & 1) ? 0x0C030C02u : 0x0C010C00u);
  } else if constexpr (BITS == 4) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int b = 0; b < 4; ++b)
        pr[4 * i + b] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | ((4u + b) << 16) | (uint32_t)b);
    }
  } else {
    int c[16];
    decode16<BITS>(w, c);
#pragma unroll
    for (int v = 0; v < 8; ++v) pr[v] = (uint32_t)c[2 * v] | ((uint32_t)c[2 * v + 1] << 16);
  }
  const short2_t zz = {(short)z, (short)z};
#pragma unroll
  for (int v = 0; v < 8; ++v)
    pr[v] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(short2_t, pr[v]) - zz);
}

// Zero point of block b of a packed zero-point row of row_bytes bytes,
// without a branch: both bytes a 3-bit value can touch are read (the second
// clamped into the row).
template <int BITS, bool HAS_ZP>
__device__ __forceinline__ int zero_point2(const uint8_t* __restrict__ zrow, int b, int row_bytes) {
  if constexpr (!HAS_ZP) {
    return 1 << (BITS - 1);
  } else {
    constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
    const int bit = b * BITS, i = bit >> 3;
    const uint32_t v = (uint32_t)zrow[i] | ((uint32_t)zrow[min(i + 1, row_bytes - 1)] << 8);
    return (int)((v >> (bit & 7)) & m);
  }
}

// Zero point of block b from a packed zero-point row (LSB-first stream; a
// 3-bit value may continue into the next byte).
template <int BITS, bool HAS_ZP>
__device__ __forceinline__ int zero_point(const uint8_t* __restrict__ zrow, int b) {
  if constexpr (!HAS_ZP) {
    return 1 << (BITS - 1);
  } else {
    constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
    const int bit = b * BITS;
    uint32_t v = (uint32_t)zrow[bit >> 3] >> (bit & 7);
    if ((bit & 7) + BITS > 8) v |= (uint32_t)zrow[(bit >> 3) + 1] << (8 - (bit & 7));
    return (int)(v & m);
  }
}

template <int ACT, int BITS, int XDT, int SDT, bool HAS_ZP, int MT, bool DOTS>
__global__ __launch_bounds__(256) void generic_rows_kernel(
    const void* __restrict__ A, const void* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ B, const typename dt<SDT>::T* __restrict__ scales,
    const uint8_t* __restrict__ zp, const void* __restrict__ bias, void* __restrict__ Y,
    int32_t* __restrict__ dots, int Mp, int M, int K, int N, int bs, int kb, int blob,
    int zp_row_bytes, int chunk_blocks) {
  extern __shared__ float gn_lds[];
  float* xs = gn_lds;                                        // [MT][chunk_p] fp32 (ACT_F)
  int* qs = reinterpret_cast<int*>(gn_lds);                  // [MT][chunk_p] int32 (ACT_I*)
  using XT = typename dt<XDT>::T;
  const int chunk = chunk_blocks * bs;
  const int chunk_p = chunk_blocks * (bs + 1);               // one pad word per block
  const int bs_log2 = __builtin_ctz(bs);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * 4 + wave) * GN_R;
  const int64_t padded = (int64_t)kb * bs;
  float acc[GN_R][MT];
#pragma unroll
  for (int r = 0; r < GN_R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  for (int b0 = 0; b0 < kb; b0 += chunk_blocks) {
    const int k0 = b0 * bs;
    __syncthreads();
    for (int t = threadIdx.x; t < MT * chunk; t += 256) {
      const int m = t / chunk, e = t % chunk, k = k0 + e;
      const int at = m * chunk_p + e + (e >> bs_log2);
      if constexpr (ACT == ACT_F) {
        xs[at] = (m < Mp && k < K) ? dt<XDT>::to_f32(reinterpret_cast<const XT*>(A)[(int64_t)m * K + k])
                                   : 0.0f;
      } else if constexpr (ACT == ACT_I8) {
        qs[at] = (m < Mp && k < padded) ? (int)reinterpret_cast<const int8_t*>(qa)[m * padded + k] : 0;
      } else {
        qs[at] = (m < Mp && k < padded) ? (int)reinterpret_cast<const int16_t*>(qa)[m * padded + k] : 0;
      }
    }
    __syncthreads();
    const int b1 = min(kb, b0 + chunk_blocks);
    for (int b = b0 + lane; b < b1; b += 64) {
#pragma unroll
      for (int r = 0; r < GN_R; ++r) {
        const int n = n0 + r;
        if (n >= N) continue;
        const uint8_t* blk = B + ((int64_t)n * kb + b) * blob;
        const int z = zero_point<BITS, HAS_ZP>(zp + (int64_t)n * zp_row_bytes, b);
        const float s = dt<SDT>::to_f32(scales[(int64_t)n * kb + b]);
        float df[MT];
        int di[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          df[m] = 0.0f;
          di[m] = 0;
        }
        const int e0 = (b - b0) * (bs + 1);
        for (int i0 = 0; i0 < bs; i0 += 16) {
          int c[16];
          codes16<BITS>(blk, bs, i0, c);
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int w = c[j] - z;
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if constexpr (ACT == ACT_F) df[m] = fmaf(xs[m * chunk_p + e0 + i0 + j], (float)w, df[m]);
              else di[m] += qs[m * chunk_p + e0 + i0 + j] * w;
            }
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if constexpr (ACT == ACT_F) {
            acc[r][m] = fmaf(df[m], s, acc[r][m]);
          } else {
            if constexpr (DOTS) {
              if (m < Mp) dots[((int64_t)m * N + n) * kb + b] = di[m];
            }
            const float sab = m < Mp ? sa[(int64_t)m * kb + b] : 0.0f;
            acc[r][m] = fmaf((float)di[m], sab * s, acc[r][m]);
          }
        }
      }
    }
  }
  if constexpr (DOTS) return;
#pragma unroll
  for (int r = 0; r < GN_R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      const int n = n0 + r;
      if (lane == 0 && n < N && m < Mp) {
        float o = v;
        if (bias) o += dt<XDT>::to_f32(reinterpret_cast<const XT*>(bias)[n]);
        reinterpret_cast<XT*>(Y)[(int64_t)m * N + n] = dt<XDT>::from_f32(o);
      }
    }
}

// ---------------------------------------------------------------------------
// Unit form (blocks of at most 512 codes): lane l of a wave takes unit
// (16 codes) u0 + l of each of the wave's GU_R columns, so a wave covers 1024
// codes of a column per pass and every lane is busy whatever the block size.
// Each lane reads its unit's activations of MT rows straight from memory
// (16-byte loads; the vector stays in the caches): no staging, no barrier.
// Per code: (code - zp) as an integer, then an fp32 FMA with the activation
// (float) or an integer multiply-add (int8); int16 activations meet packed
// int16 (code - zp) pairs in v_dot2_i32_i16.
// Float: each unit's sum is scaled by its block's scale.  Integer: the
// block's UB = bs / 16 lanes (aligned, adjacent) add their exact int32 sums
// by XOR shuffles, and the first lane scales the block dot once.
// ---------------------------------------------------------------------------
constexpr int GU_R = 2;            // columns per wave
constexpr int GU_MAX_BS = 512;     // a block spans at most 32 lanes

template <int ACT, int BITS, int XDT, int SDT, bool HAS_ZP, int MT, bool DOTS>
__global__ __launch_bounds__(256) void generic_unit_kernel(
    const void* __restrict__ A, const void* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ B, const typename dt<SDT>::T* __restrict__ scales,
    const uint8_t* __restrict__ zp, const void* __restrict__ bias, void* __restrict__ Y,
    int32_t* __restrict__ dots, int Mp, int K, int N, int bs, int kb, int blob,
    int zp_row_bytes) {
  using XT = typename dt<XDT>::T;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = (blockIdx.x * 4 + wave) * GU_R;
  const int ub_log2 = __builtin_ctz(bs) - 4;           // units per block, log2
  const int units = kb << ub_log2;                      // units per column
  const int64_t padded = (int64_t)kb * bs;
  // 16-byte activation loads: float rows whose units are wholly inside or
  // wholly past K and 16-byte aligned; the quantized rows always are (padded
  // to whole blocks, 256-byte aligned).
  const bool vec = ACT != ACT_F || ((K % 16) == 0 && (((uintptr_t)A) & 15) == 0);
  float acc[GU_R][MT];
#pragma unroll
  for (int r = 0; r < GU_R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  // Units start at multiples of 64 per pass, so the lanes of one block are
  // aligned and adjacent.
  for (int ub = 0; ub < units; ub += 64) {
    {
      const int u = ub + lane;
      const bool live = u < units;
      const int uc = live ? u : 0;                      // in-bounds stand-in
      const int b = uc >> ub_log2, ui = uc & ((1 << ub_log2) - 1);
      const int64_t k0 = (int64_t)uc * 16;
      // This unit's activations of the MT rows (rows past Mp read row 0 and
      // are discarded), read straight from memory: the vector is small and
      // stays in the caches, so there is no staging and no barrier.
      float xf[MT][16];
      int xi[MT][16];
      uint32_t xw[MT][8];          // int16: the raw activation pairs
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int64_t mr = m < Mp ? m : 0;
        if constexpr (ACT == ACT_F) {
          if (vec) {
            const bool in = k0 < K;
            const XT* xr = reinterpret_cast<const XT*>(A) + mr * K + (in ? k0 : 0);
            if constexpr (sizeof(XT) == 4) {
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const u32x4 w = reinterpret_cast<const u32x4*>(xr)[v];
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) xf[m][4 * v + j] = in ? __uint_as_float(ww[j]) : 0.0f;
              }
            } else {
#pragma unroll
              for (int v = 0; v < 2; ++v) {
                const u32x4 w = reinterpret_cast<const u32x4*>(xr)[v];
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 8; ++j)
                  xf[m][8 * v + j] = in ? dt<XDT>::to_f32(__builtin_bit_cast(
                                              XT, (uint16_t)(ww[j / 2] >> (16 * (j & 1)))))
                                        : 0.0f;
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              const int64_t k = k0 + j;
              xf[m][j] = k < K ? dt<XDT>::to_f32(reinterpret_cast<const XT*>(A)[mr * K + k]) : 0.0f;
            }
          }
        } else if constexpr (ACT == ACT_I8) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(
              reinterpret_cast<const int8_t*>(qa) + mr * padded + k0);
          const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 16; ++j) xi[m][j] = (int)(int8_t)(ww[j / 4] >> (8 * (j & 3)));
        } else {
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const u32x4 w = reinterpret_cast<const u32x4*>(
                reinterpret_cast<const int16_t*>(qa) + mr * padded + k0)[v];
            xw[m][4 * v + 0] = w.x;
            xw[m][4 * v + 1] = w.y;
            xw[m][4 * v + 2] = w.z;
            xw[m][4 * v + 3] = w.w;
          }
        }
      }
      // Every column's loads first (a column past N reads column N - 1 and
      // is discarded), so that they are in flight together.
      uint32_t raw[GU_R][Raw16<BITS>::W];
      int zr[GU_R];
      float sr[GU_R];
#pragma unroll
      for (int r = 0; r < GU_R; ++r) {
        const int64_t nc = min(n0 + r, N - 1);
        load_raw16<BITS>(B + (nc * kb + b) * blob, bs, ui * 16, raw[r]);
        zr[r] = zero_point2<BITS, HAS_ZP>(zp + nc * zp_row_bytes, b, zp_row_bytes);
        sr[r] = dt<SDT>::to_f32(scales[nc * kb + b]);
      }
#pragma unroll
      for (int r = 0; r < GU_R; ++r) {
        const int n = n0 + r;
        if (n >= N) continue;                           // wave-uniform
        int c[16];
        uint32_t pr[8];
        if constexpr (ACT == ACT_I16) code_pairs16<BITS>(raw[r], zr[r], pr);
        else decode16<BITS>(raw[r], c);
        const int z = zr[r];
        const float s = sr[r];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          if constexpr (ACT == ACT_F) {
            float d = 0.0f;
#pragma unroll
            for (int j = 0; j < 16; ++j) d = fmaf(xf[m][j], (float)(c[j] - z), d);
            acc[r][m] = fmaf(live ? d : 0.0f, s, acc[r][m]);
          } else {
            int d = 0;
            if constexpr (ACT == ACT_I16) {
              // Exact: |pair dot| < 2^24, block sums < 2^31 (bs <= 128).
#pragma unroll
              for (int v = 0; v < 8; ++v)
                d = __builtin_amdgcn_sdot2(__builtin_bit_cast(short2_t, pr[v]),
                                           __builtin_bit_cast(short2_t, xw[m][v]), d, false);
            } else {
#pragma unroll
              for (int j = 0; j < 16; ++j) d += xi[m][j] * (c[j] - z);
            }
            d = live ? d : 0;
            for (int o = 1; o < (1 << ub_log2); o <<= 1) d += __shfl_xor(d, o);
            if (live && ui == 0) {
              if constexpr (DOTS) {
                if (m < Mp) dots[((int64_t)m * N + n) * kb + b] = d;
              }
              const float sab = m < Mp ? sa[(int64_t)m * kb + b] : 0.0f;
              acc[r][m] = fmaf((float)d, sab * s, acc[r][m]);
            }
          }
        }
      }
    }
  }
  if constexpr (DOTS) return;
#pragma unroll
  for (int r = 0; r < GU_R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      const float v = wave_sum(acc[r][m]);
      const int n = n0 + r;
      if (lane == 0 && n < N && m < Mp) {
        float o = v;
        if (bias) o += dt<XDT>::to_f32(reinterpret_cast<const XT*>(bias)[n]);
        reinterpret_cast<XT*>(Y)[(int64_t)m * N + n] = dt<XDT>::from_f32(o);
      }
    }
}

int dtype_bytes(int dt) { return dt == DT_F32 ? 4 : 2; }

template <int ACT, int BITS, int XDT, int SDT, bool HAS_ZP, bool DOTS, int MT>
hipError_t launch_gu_m(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  using ST = typename dt<SDT>::T;
  const int grid = (int)((a.N + 4 * GU_R - 1) / (4 * GU_R));
  const int64_t padded = a.kb * a.block_size;
  const int qb = ACT == ACT_I16 ? 2 : 1;
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    hipLaunchKernelGGL((generic_unit_kernel<ACT, BITS, XDT, SDT, HAS_ZP, MT, DOTS>), dim3(grid),
                       dim3(256), 0, a.stream,
                       ACT == ACT_F ? (const void*)((const char*)a.A + m0 * a.K * dtype_bytes(a.a_dtype))
                                    : a.A,
                       qa ? (const void*)((const char*)qa + m0 * padded * qb) : nullptr,
                       sa ? sa + m0 * a.kb : nullptr, a.B, (const ST*)a.scales, a.zp, a.bias,
                       DOTS ? nullptr : (void*)((char*)a.Y + m0 * a.N * dtype_bytes(a.a_dtype)),
                       DOTS ? dots + m0 * a.N * a.kb : nullptr, Mp, (int)a.K, (int)a.N,
                       (int)a.block_size, (int)a.kb, (int)a.blob, (int)a.zp_row_bytes);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int ACT, int BITS, int XDT, int SDT, bool HAS_ZP, bool DOTS, int MT>
hipError_t launch_gn_m(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  using ST = typename dt<SDT>::T;
  // Whole blocks per staged chunk: one per lane (64) where that fits in about
  // 40 KiB of LDS, else fewer, at least one.
  const int64_t per_block = (int64_t)MT * (a.block_size + 1) * 4;
  const int chunk_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(64, 40960 / per_block));
  const size_t lds = (size_t)(chunk_blocks * per_block);
  auto kern = generic_rows_kernel<ACT, BITS, XDT, SDT, HAS_ZP, MT, DOTS>;
  if (lds > 64 * 1024) {
    const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
    if (e != hipSuccess) return e;
  }
  const int grid = (int)((a.N + 4 * GN_R - 1) / (4 * GN_R));
  const int64_t padded = a.kb * a.block_size;
  for (int64_t m0 = 0; m0 < a.M; m0 += MT) {
    const int Mp = (int)std::min<int64_t>(MT, a.M - m0);
    const int qb = ACT == ACT_I16 ? 2 : 1;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(256), lds, a.stream,
                       ACT == ACT_F ? (const void*)((const char*)a.A + m0 * a.K * dtype_bytes(a.a_dtype))
                                    : a.A,
                       qa ? (const void*)((const char*)qa + m0 * padded * qb) : nullptr,
                       sa ? sa + m0 * a.kb : nullptr, a.B, (const ST*)a.scales, a.zp, a.bias,
                       DOTS ? nullptr : (void*)((char*)a.Y + m0 * a.N * dtype_bytes(a.a_dtype)),
                       DOTS ? dots + m0 * a.N * a.kb : nullptr, Mp, (int)a.M, (int)a.K, (int)a.N,
                       (int)a.block_size, (int)a.kb, (int)a.blob, (int)a.zp_row_bytes,
                       chunk_blocks);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int ACT, int BITS, int XDT, int SDT, bool HAS_ZP, bool DOTS>
hipError_t launch_gn_t(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  if (ACT == ACT_I16 || a.block_size <= GU_MAX_BS)   // int16: block_size <= 128
    return a.M == 1 ? launch_gu_m<ACT, BITS, XDT, SDT, HAS_ZP, DOTS, 1>(a, qa, sa, dots)
                    : launch_gu_m<ACT, BITS, XDT, SDT, HAS_ZP, DOTS, 4>(a, qa, sa, dots);
  if constexpr (ACT != ACT_I16)
    return a.M == 1 ? launch_gn_m<ACT, BITS, XDT, SDT, HAS_ZP, DOTS, 1>(a, qa, sa, dots)
                    : launch_gn_m<ACT, BITS, XDT, SDT, HAS_ZP, DOTS, 4>(a, qa, sa, dots);
  return hipErrorInvalidValue;
}

template <int ACT, int BITS, int XDT, bool DOTS>
hipError_t launch_gn_s(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  auto z = [&](auto sdt) {
    constexpr int SDT = decltype(sdt)::value;
    return a.zp ? launch_gn_t<ACT, BITS, XDT, SDT, true, DOTS>(a, qa, sa, dots)
                : launch_gn_t<ACT, BITS, XDT, SDT, false, DOTS>(a, qa, sa, dots);
  };
  switch (a.s_dtype) {
    case DT_F32: return z(std::integral_constant<int, DT_F32>{});
    case DT_F16: return z(std::integral_constant<int, DT_F16>{});
    default: return z(std::integral_constant<int, DT_BF16>{});
  }
}

template <int ACT, int BITS, bool DOTS>
hipError_t launch_gn_x(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  switch (a.a_dtype) {
    case DT_F32: return launch_gn_s<ACT, BITS, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_gn_s<ACT, BITS, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_gn_s<ACT, BITS, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

// Float and int8 activations reach these kernels with 3-bit weights only
// (the other widths have their own kernels); int16 activations with any.
template <int ACT, bool DOTS>
hipError_t launch_gn_b(const MatArgs& a, const void* qa, const float* sa, int32_t* dots) {
  if constexpr (ACT != ACT_I16) {
    return a.bits == 3 ? launch_gn_x<ACT, 3, DOTS>(a, qa, sa, dots) : hipErrorInvalidValue;
  } else {
    switch (a.bits) {
      case 2: return launch_gn_x<ACT, 2, DOTS>(a, qa, sa, dots);
      case 3: return launch_gn_x<ACT, 3, DOTS>(a, qa, sa, dots);
      case 4: return launch_gn_x<ACT, 4, DOTS>(a, qa, sa, dots);
      default: return launch_gn_x<ACT, 8, DOTS>(a, qa, sa, dots);
    }
  }
}

}  // namespace

hipError_t launch_generic_float(const MatArgs& a) {
  return launch_gn_b<ACT_F, false>(a, nullptr, nullptr, nullptr);
}

hipError_t launch_generic_int(const MatArgs& a, const void* qa, int act_bytes, const float* sa,
                              int32_t* dots) {
  if (act_bytes == 1)
    return dots ? launch_gn_b<ACT_I8, true>(a, qa, sa, dots)
                : launch_gn_b<ACT_I8, false>(a, qa, sa, nullptr);
  return dots ? launch_gn_b<ACT_I16, true>(a, qa, sa, dots)
              : launch_gn_b<ACT_I16, false>(a, qa, sa, nullptr);
}

}  // namespace qmm
