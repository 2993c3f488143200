// compint8.hip -- CompInt8 (accuracy_level 4) for gfx950: activations
// quantized to int8 per K-block, exact int32 block dot products against the
// packed weight codes, then fp32 scaling (onnx-runtime-ep-cpu matmul_nbits.rs:
// quantize_activation_signed, prepack_int8_weight, int4_dot_row_scalar,
// int8_row).
//
// Step 1, quantize_a_kernel: per row m and block b of block_size activations,
//   sa = max|x| / 127 (IEEE binary32 division), qa = clamp(rne(x / sa),
//   -127, 127), zero past K and for a block whose sa is 0.  Written to the
//   caller's workspace in natural order: qa [M, kb*bs] int8, sa [M, kb] f32.
// Step 2, compint8_kernel: dot[m,n,b] = sum qa * (code - zp) in int32 and
//   y[m,n] = sum_b float(dot) * (sa[m,b] * scale[n,b]) (+ bias) in fp32.
//
// The int32 arithmetic of step 2 is exact: for 2- and 4-bit weights each code
// byte is turned into the int8 (code - zp) with one SWAR add/xor, and
// v_dot4_i32_i8 multiplies it with four activations; for 8-bit weights
// (code - zp can reach +-255) the codes enter as (code - 128) and the block
// dot is corrected by (zp - 128) * sum(qa), the identity
// sum qa*(q - z) = sum qa*(q - 128) - (z - 128) * sum qa.
// The work split follows the GEMV: a wave owns R output columns and walks
// (chunk, row) jobs of one 16-byte unit of codes per lane, loaded through
// buffer descriptors; the unit's activations for all M rows come from LDS.
#include <algorithm>

#include "qmm_device.h"
#include "qmm_internal.h"

namespace qmm {

constexpr int CI8_THREADS = 256;
constexpr int BUFFER_WORD3 = 0x00020000;  // raw byte-addressed buffer descriptor
// LDS budget for the staged int8 activations of one K-chunk (all M rows).
constexpr int CI8_LDS_BYTES = 64 * 1024;

// ---------------------------------------------------------------------------
// Step 1: activation quantization, one wave per (m, block).
// ---------------------------------------------------------------------------
// QT = int8_t: sa = max|x| / 127 (CompInt8); QT = int16_t: sa = max|x| / 32767
// (the int16-activation route), codes clamped to +-QMAX.
template <int XDT, typename QT = int8_t>
__global__ __launch_bounds__(256) void quantize_a_kernel(const typename dt<XDT>::T* __restrict__ A,
                                                         QT* __restrict__ qa,
                                                         float* __restrict__ sa, int M, int K,
                                                         int bs, int kb) {
  constexpr float QMAX = sizeof(QT) == 1 ? 127.0f : 32767.0f;
  // Blocks of up to QA_REG * 64 activations are read once and kept in
  // registers between the maximum and the quantization (one global round
  // trip); longer blocks read their activations a second time.
  constexpr int QA_REG = 4;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= M * kb) return;
  const int m = gw / kb, b = gw % kb;
  const int k0 = b * bs;
  const int64_t padded = (int64_t)kb * bs;
  const bool in_regs = bs <= QA_REG * 64;
  float xv[QA_REG];
#pragma unroll
  for (int i = 0; i < QA_REG; ++i) {
    const int k = k0 + lane + 64 * i;
    xv[i] = (lane + 64 * i < bs && k < K) ? dt<XDT>::to_f32(A[(int64_t)m * K + k]) : 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < QA_REG; ++i) amax = fmaxf(amax, fabsf(xv[i]));
  for (int e = lane + 64 * QA_REG; e < bs; e += 64) {
    const int k = k0 + e;
    if (k < K) amax = fmaxf(amax, fabsf(dt<XDT>::to_f32(A[(int64_t)m * K + k])));
  }
  // Wave max (exact: max is order independent).
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
  const float scale = amax / QMAX;     // IEEE binary32 division
  if (lane == 0) sa[(int64_t)m * kb + b] = scale;
  auto quant = [&](float x) {
    float r = rintf(x / scale);        // IEEE division, ties to even
    r = fminf(fmaxf(r, -QMAX), QMAX);
    return (QT)r;
  };
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < QA_REG; ++i) {
      const int e = lane + 64 * i;
      // Positions past K (the padding of the last block) are zero; so is
      // every position of a block whose scale is 0.
      if (e < bs) qa[(int64_t)m * padded + k0 + e] = (k0 + e < K && scale != 0.0f) ? quant(xv[i]) : (QT)0;
    }
  } else {
    for (int e = lane; e < bs; e += 64) {
      const int k = k0 + e;
      QT v = 0;
      if (k < K && scale != 0.0f) v = quant(dt<XDT>::to_f32(A[(int64_t)m * K + k]));
      qa[(int64_t)m * padded + k] = v;
    }
  }
}

// Signed-byte form of the codes of one 32-bit word, ordered to match the
// activation permutation of stage_qa.  For 2/4-bit codes each byte is
// (code - z) (|code - z| < 16 fits int8); for 8-bit codes it is (code - 128).
// Output: NB dwords of four int8 each.
template <int BITS>
struct CodeBytes {
  static constexpr int NB = (BITS == 8) ? 1 : (BITS == 4 ? 2 : 4);
};

template <int BITS>
__device__ __forceinline__ void code_bytes(uint32_t w, uint32_t z, uint32_t* out) {
  if constexpr (BITS == 8) {
    out[0] = w ^ 0x80808080u;
  } else {
    constexpr uint32_t m = (BITS == 4) ? 0x0F0F0F0Fu : 0x03030303u;
    const uint32_t zz = z * 0x01010101u;
#pragma unroll
    for (int i = 0; i < CodeBytes<BITS>::NB; ++i) {
      const uint32_t f = (w >> (i * BITS)) & m;
      // (f | 0x80) - z stays in [0x80 - 15, 0x8F] per byte (no borrow), and
      // xor 0x80 turns it into the two's-complement byte (code - z).
      out[i] = ((f | 0x80808080u) - zz) ^ 0x80808080u;
    }
  }
}

// Position, inside a word of P codes, of the activation that pairs with byte j
// of code_bytes dword i: dword i holds field i of each byte, i.e. codes
// (i, i + NB, i + 2 NB, i + 3 NB) for 2/4-bit (NB fields per byte), and the
// natural order for 8-bit.
template <int BITS>
__device__ __forceinline__ int pair_pos(int i, int j) {
  constexpr int NB = CodeBytes<BITS>::NB;
  return (BITS == 8) ? j : (j * NB + i);
}

// ---------------------------------------------------------------------------
// Stage qa for rows [0, M) and K-chunk elements [k0, k0 + len) into LDS in the
// pairing order: for each word of codes (P elements), the NB activation dwords
// that match code_bytes.  Layout: xs[m][word][i] (uint32).
// ---------------------------------------------------------------------------
template <int BITS>
__device__ void stage_qa(const int8_t* __restrict__ qa, int64_t padded, int M, int k0,
                         int len_words, uint32_t* __restrict__ xs) {
  constexpr int P = 32 / BITS;
  constexpr int NB = CodeBytes<BITS>::NB;
  const int total = M * len_words;
  for (int t = threadIdx.x; t < total; t += CI8_THREADS) {
    const int m = t / len_words, w = t % len_words;
    const int8_t* src = qa + (int64_t)m * padded + k0 + w * P;
    int8_t v[P];
    if constexpr (P == 4) {
      const uint32_t u = *reinterpret_cast<const uint32_t*>(src);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = (int8_t)(u >> (8 * j));
    } else if constexpr (P == 8) {
      const u32x2 u = *reinterpret_cast<const u32x2*>(src);
#pragma unroll
      for (int j = 0; j < 4; ++j) { v[j] = (int8_t)(u.x >> (8 * j)); v[4 + j] = (int8_t)(u.y >> (8 * j)); }
    } else {
      const u32x4 u = *reinterpret_cast<const u32x4*>(src);
      const uint32_t uw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (int8_t)(uw[j / 4] >> (8 * (j % 4)));
    }
    uint32_t* dst = xs + ((int64_t)m * len_words + w) * NB;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      uint32_t d = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) d |= (uint32_t)(uint8_t)v[pair_pos<BITS>(i, j)] << (8 * j);
      dst[i] = d;
    }
  }
}

// ---------------------------------------------------------------------------
// Step 2.  One launch handles Mp <= MT rows of A (the host offsets qa, sa, y
// and dots per pass); acc[R][MT] per lane.  DOTS: also add each lane's exact
// int32 partial block dot into dots[m,n,b] (integer atomics: the sum is
// order independent) and write no y.
// Dynamic LDS: staged qa, Mp * chunk_words * NB dwords (Mp * chunk bytes).
// ---------------------------------------------------------------------------
template <int BITS, int SDT, int YDT, bool HAS_ZP, int R, int MT, bool DOTS>
__global__ __launch_bounds__(CI8_THREADS) void compint8_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const typename dt<YDT>::T* __restrict__ bias, typename dt<YDT>::T* __restrict__ y,
    int32_t* __restrict__ dots, int Mp, int N, int kb, int log2_blob, int zp_row_bytes,
    int chunk_words) {
  constexpr int P = 32 / BITS;
  constexpr int NB = CodeBytes<BITS>::NB;
  using ST = typename dt<SDT>::T;
  extern __shared__ u32x4 smem_c[];
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_c);

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int nrows = max(0, min(R, N - row0));
  const int64_t row_bytes = (int64_t)kb << log2_blob;
  const int row_words = (int)(row_bytes >> 2);
  constexpr int LOG2_EPB = (BITS == 2) ? 2 : (BITS == 4 ? 1 : 0);  // log2(codes per byte)
  const int64_t padded = ((int64_t)kb << log2_blob) << LOG2_EPB;    // kb * block_size
  const int blob_words_log2 = log2_blob - 2;
  // 16-byte units per lane when blocks are at least 16 bytes, else words.
  const bool vec = (log2_blob >= 4);
  const int UW = vec ? 4 : 1;
  const int total_units = row_words / UW;
  const int chunk_units = chunk_words / UW;

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[r][m] = 0.0f;

  __amdgpu_buffer_rsrc_t rb[R], rs[R], rz[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const bool live = r < nrows;
    const int row = min(row0 + r, N - 1);
    rb[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)row * row_bytes), 0,
                                              live ? (int)row_bytes : 0, BUFFER_WORD3);
    // The block-dot export passes no scales: an empty descriptor reads zeros.
    rs[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + (int64_t)row * kb), 0,
                                              (live && scales) ? kb * (int)sizeof(ST) : 0,
                                              BUFFER_WORD3);
    if constexpr (HAS_ZP)
      rz[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(zp + (int64_t)row * zp_row_bytes), 0,
                                                live ? zp_row_bytes : 0, BUFFER_WORD3);
  }

  for (int c0 = 0; c0 < total_units; c0 += chunk_units) {
    const int c1 = min(total_units, c0 + chunk_units);
    const int cw0 = c0 * UW, cwn = (c1 - c0) * UW;   // chunk start / length in words
    __syncthreads();
    stage_qa<BITS>(qa, padded, Mp, cw0 * P, cwn, xs);
    __syncthreads();
    for (int ub = c0; ub < c1; ub += 64) {           // wave-uniform unit base
      const int u = ub + lane;
      const bool ok = u < c1;
      const int uc = min(u, c1 - 1);
      const int blk = (uc * UW) >> blob_words_log2;
      // Codes, scale and zero point of this unit for the R rows.
      uint32_t cw[R][4];
      float sc[R];
      uint32_t zb[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (vec) {
          const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rb[r], uc * 16, 0, BUF_STREAM);
          cw[r][0] = t.x; cw[r][1] = t.y; cw[r][2] = t.z; cw[r][3] = t.w;
        } else {
          cw[r][0] = __builtin_amdgcn_raw_buffer_load_b32(rb[r], uc * 4, 0, BUF_STREAM);
          cw[r][1] = cw[r][2] = cw[r][3] = 0;
        }
        if constexpr (sizeof(ST) == 4)
          sc[r] = dt<SDT>::to_f32(__builtin_bit_cast(
              ST, __builtin_amdgcn_raw_buffer_load_b32(rs[r], blk * 4, 0, 0)));
        else
          sc[r] = dt<SDT>::to_f32(__builtin_bit_cast(
              ST, __builtin_amdgcn_raw_buffer_load_b16(rs[r], blk * 2, 0, 0)));
        zb[r] = HAS_ZP ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz[r], (blk * BITS) >> 3, 0, 0)
                       : 0u;
      }
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        if (mi < Mp) {   // wave-uniform; keeps the loop unrollable
        const float s_a = sa[(int64_t)mi * kb + blk];
        // Activations of this unit for row mi (UW words x NB dwords).
        uint32_t xa[4][NB];
        const uint32_t* xsrc = xs + ((int64_t)mi * cwn + (uc - c0) * UW) * NB;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int i = 0; i < NB; ++i) xa[j][i] = (j < UW) ? xsrc[j * NB + i] : 0u;
        int qsum = 0;
        if constexpr (BITS == 8) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            qsum = __builtin_amdgcn_sdot4((int)xa[j][0], 0x01010101, qsum, false);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t z = 1u << (BITS - 1);
          if constexpr (HAS_ZP) {
            constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
            z = (zb[r] >> ((blk * BITS) & 7)) & zm;
          }
          int p = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t cb[NB];
            code_bytes<BITS>(cw[r][j], z, cb);
#pragma unroll
            for (int i = 0; i < NB; ++i)
              p = __builtin_amdgcn_sdot4((int)cb[i], (int)xa[j][i], p, false);
          }
          // Words past UW hold zero activations, so they add nothing; for
          // 8-bit codes the offset correction uses the same activations.
          if constexpr (BITS == 8) p -= ((int)z - 128) * qsum;
          if (ok && r < nrows) {
            acc[r][mi] = fmaf((float)p, s_a * sc[r], acc[r][mi]);
            if constexpr (DOTS) atomicAdd(&dots[((int64_t)mi * N + row0 + r) * kb + blk], p);
          }
        }
        }
      }
    }
  }

  if constexpr (!DOTS) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int mi = 0; mi < MT; ++mi) {
        const float v = wave_sum(acc[r][mi]);
        if (lane == 0 && r < nrows && mi < Mp) {
          float o = v;
          if (bias) o += dt<YDT>::to_f32(bias[row0 + r]);
          y[(int64_t)mi * N + row0 + r] = dt<YDT>::from_f32(o);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

template <typename QT>
static hipError_t launch_quantize_t(const MatArgs& a, QT* qa, float* sa) {
  const int blocks = (int)(a.M * a.kb);
  const int grid = (blocks + 3) / 4;
  if (blocks == 0) return hipSuccess;
  switch (a.a_dtype) {
    case DT_F32:
      hipLaunchKernelGGL((quantize_a_kernel<DT_F32, QT>), dim3(grid), dim3(256), 0, a.stream,
                         (const float*)a.A, qa, sa, (int)a.M, (int)a.K, (int)a.block_size, (int)a.kb);
      break;
    case DT_F16:
      hipLaunchKernelGGL((quantize_a_kernel<DT_F16, QT>), dim3(grid), dim3(256), 0, a.stream,
                         (const _Float16*)a.A, qa, sa, (int)a.M, (int)a.K, (int)a.block_size, (int)a.kb);
      break;
    default:
      hipLaunchKernelGGL((quantize_a_kernel<DT_BF16, QT>), dim3(grid), dim3(256), 0, a.stream,
                         (const uint16_t*)a.A, qa, sa, (int)a.M, (int)a.K, (int)a.block_size, (int)a.kb);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_quantize_a(const MatArgs& a, int8_t* qa, float* sa) {
  return launch_quantize_t<int8_t>(a, qa, sa);
}

hipError_t launch_quantize_a16(const MatArgs& a, int16_t* qa, float* sa) {
  return launch_quantize_t<int16_t>(a, qa, sa);
}

template <int BITS, int SDT, int YDT, bool HAS_ZP, bool DOTS>
static hipError_t launch_ci8_t(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  constexpr int NB = CodeBytes<BITS>::NB;
  constexpr int P = 32 / BITS;
  const int log2_blob = ilog2(a.blob);
  const int64_t row_words = a.kb * a.blob / 4;
  const int uw = (a.blob >= 16) ? 4 : 1;
  const int64_t padded = a.kb * a.block_size;
  using ST = typename dt<SDT>::T;
  using YT = typename dt<YDT>::T;
  for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
    const int Mp = (int)std::min<int64_t>(16, a.M - m0);
    // Chunk: as many whole units as fit the LDS budget for Mp rows.
    int64_t cw = CI8_LDS_BYTES / (Mp * NB * 4);
    cw = std::min<int64_t>(row_words, cw / uw * uw);
    const size_t lds = (size_t)Mp * cw * NB * 4;
    const int8_t* q = qa + m0 * padded;
    const float* s = sa + m0 * a.kb;
    YT* y = DOTS ? nullptr : (YT*)a.Y + m0 * a.N;
    int32_t* d = DOTS ? dots + m0 * a.N * a.kb : nullptr;
    if (Mp <= 1) {
      constexpr int R = 4;
      const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
      hipLaunchKernelGGL((compint8_kernel<BITS, SDT, YDT, HAS_ZP, R, 1, DOTS>), dim3(grid),
                         dim3(CI8_THREADS), lds, a.stream, q, s, a.B, (const ST*)a.scales, a.zp,
                         (const YT*)a.bias, y, d, Mp, (int)a.N, (int)a.kb, log2_blob,
                         (int)a.zp_row_bytes, (int)cw);
    } else if (Mp <= 4) {
      constexpr int R = 2;
      const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
      hipLaunchKernelGGL((compint8_kernel<BITS, SDT, YDT, HAS_ZP, R, 4, DOTS>), dim3(grid),
                         dim3(CI8_THREADS), lds, a.stream, q, s, a.B, (const ST*)a.scales, a.zp,
                         (const YT*)a.bias, y, d, Mp, (int)a.N, (int)a.kb, log2_blob,
                         (int)a.zp_row_bytes, (int)cw);
    } else {
      constexpr int R = 1;
      const int grid = (int)((a.N + 4 * R - 1) / (4 * R));
      hipLaunchKernelGGL((compint8_kernel<BITS, SDT, YDT, HAS_ZP, R, 16, DOTS>), dim3(grid),
                         dim3(CI8_THREADS), lds, a.stream, q, s, a.B, (const ST*)a.scales, a.zp,
                         (const YT*)a.bias, y, d, Mp, (int)a.N, (int)a.kb, log2_blob,
                         (int)a.zp_row_bytes, (int)cw);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    (void)P;
  }
  return hipSuccess;
}

template <int BITS, int SDT, int YDT, bool DOTS>
static hipError_t launch_ci8_z(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  return a.zp ? launch_ci8_t<BITS, SDT, YDT, true, DOTS>(a, qa, sa, dots)
              : launch_ci8_t<BITS, SDT, YDT, false, DOTS>(a, qa, sa, dots);
}

template <int BITS, int SDT, bool DOTS>
static hipError_t launch_ci8_y(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.a_dtype) {
    case DT_F32: return launch_ci8_z<BITS, SDT, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_ci8_z<BITS, SDT, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_ci8_z<BITS, SDT, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

template <int BITS, bool DOTS>
static hipError_t launch_ci8_s(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.s_dtype) {
    case DT_F32: return launch_ci8_y<BITS, DT_F32, DOTS>(a, qa, sa, dots);
    case DT_F16: return launch_ci8_y<BITS, DT_F16, DOTS>(a, qa, sa, dots);
    default: return launch_ci8_y<BITS, DT_BF16, DOTS>(a, qa, sa, dots);
  }
}

template <bool DOTS>
static hipError_t launch_ci8(const MatArgs& a, const int8_t* qa, const float* sa, int32_t* dots) {
  switch (a.bits) {
    case 2: return launch_ci8_s<2, DOTS>(a, qa, sa, dots);
    case 4: return launch_ci8_s<4, DOTS>(a, qa, sa, dots);
    default: return launch_ci8_s<8, DOTS>(a, qa, sa, dots);
  }
}

hipError_t launch_compint8(const MatArgs& a, const int8_t* qa, const float* sa) {
  return launch_ci8<false>(a, qa, sa, nullptr);
}

hipError_t launch_compint8_dots(const MatArgs& a, const int8_t* qa, const float* sa,
                                int32_t* dots) {
  return launch_ci8<true>(a, qa, sa, dots);
}

}  // namespace qmm
