// gemm_skinny.h -- the matmul over block-quantized weights for a few rows of
// 16-bit activations (batched decode, short prompts: M <= 16, or up to 1024
// workgroups of 32 x 32 outputs) on the gfx950 matrix cores.
//
// Y[M, N] = A[M, K] * W^T, W[n, k] = (code - zp) * scale (onnx-runtime-ep-cpu
// matmul_nbits.rs: the batched route dequantizes then multiplies).  With few
// rows the work is the weight stream, as in the M = 1 GEMV: every code is read
// once from memory and dequantized once, for all rows together, and the
// products run on v_mfma_f32_16x16x32_{bf16,f16}.
//
// Work split: a workgroup of 8 waves owns 16 * TN consecutive columns and
// 16 * MT rows; its waves take turns over K in steps of 256 (wave w steps w,
// w + 8, ...), so the 8 waves read adjacent 128-byte pieces of each column at
// once, and sum their partial tiles through LDS at the end.
// Within a step, lane l = 16 g + c (c = l % 16, g = l / 16) holds the 64
// consecutive codes k0 .. k0 + 63, k0 = 256 step + 64 g, of column c of each
// of the TN 16-column tiles (one 16-byte load per 32 codes of 4 bits), and
// for its MFMA operand of sub-step s (0..7) the 8 codes k0 + 8 s .. + 7.  Its
// activation operand, row c of each 16-row tile, covers the same 8 k, so each
// v_mfma_f32_16x16x32 of the step sums 32 distinct k of the step: the order
// of k inside a product is free, only the pairing of A and B has to agree.
// Dequantization matches the 256-row kernel: fp32 (code * s - z * s) (exact
// for 16-bit scales), rounded once to the activation dtype, accumulated in
// fp32.
#pragma once

#include <algorithm>
#include <type_traits>

#include "mfma_ops.h"
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

namespace qmm {

constexpr int SK_WAVES = 8;
constexpr int SK_TPB = 64 * SK_WAVES;
constexpr int SK_KSTEP = 256;               // K per wave step (4 lane groups x 64 codes)
constexpr int SK_FULL_ROUND = 256;          // workgroups that give every compute unit one
// Scales and zero points of a workgroup's 32 columns are staged in LDS when
// both fit in this many bytes (each range is copied from a 16-byte aligned
// start, hence the slack); otherwise every lane loads its own.
constexpr int SK_SLAB_MAX = 64 * 1024;

// Eight codes k0 + 8 s .. + 7 of a lane's 64 (cw holds them LSB first) as
// fp32 values.
template <int BITS>
__device__ __forceinline__ void step_codes(const uint32_t* cw, int s, float* q) {
  if constexpr (BITS == 3) {
    // cw[0..3]: the 64 codes' 2-bit plane fields in code order, cw[4..5]:
    // their 1-bit plane bits (see load_codes); code i of sub-step s is
    // field 8 s + i plus 4 times bit 8 s + i.
    const uint32_t lo = cw[s >> 1] >> (16 * (s & 1));
    const uint32_t hi = cw[4 + (s >> 2)] >> (8 * (s & 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = (float)(((lo >> (2 * i)) & 3u) | (((hi >> i) & 1u) << 2));
  } else if constexpr (BITS == 8) {
    word_codes_f32<8>(cw[2 * s], q);
    word_codes_f32<8>(cw[2 * s + 1], q + 4);
  } else if constexpr (BITS == 4) {
    word_codes_f32<4>(cw[s], q);
  } else {
    // 16 codes per word: the low or high byte pair of word s / 2.
    const uint32_t w = cw[s >> 1] >> (16 * (s & 1));
    const uint32_t f[4] = {opaque_and(w, 0x0303u), opaque_and(w >> 2, 0x0303u),
                           opaque_and(w >> 4, 0x0303u), opaque_and(w >> 6, 0x0303u)};
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) q[4 * j + i] = (float)((f[i] >> (8 * j)) & 0xFF);
  }
}

// Requirements checked by the launcher: K % 8 == 0, A 16-byte aligned, every
// buffer byte offset below 2^31.  Rows past M and k past K read zeros through
// the buffer descriptors' extents; codes past a column's last block belong to
// the next column (or lie past the matrix and read as zero) and meet zero
// activations.
//
// Scales and zero points: a workgroup's columns lie in one contiguous byte
// range of each tensor on both layouts -- operator layout: its 16 TN rows of
// kb scales and of zp_row_bytes zero-point bytes; tiled: the 32 columns of
// its group (kb x 32 scales, 4 kb bits bytes of zero points).  With SLAB the
// workgroup copies both ranges into LDS once (16-byte loads) and every lookup
// reads LDS.
//
// WF: block-scaled FP4 weights (1 + FP4_MX or 1 + FP4_NV; operator layout,
// BITS = 4, no zero points): codes are E2M1 values, scales one E8M0 / E4M3
// byte per block, and the sums are multiplied by gscale.  Each weight,
// e2m1 * scale, has at most 6 significant bits, so its rounding to the
// activation dtype is exact.
template <int BITS, int XDT, int SDT, bool HAS_ZP, int TN, int MT, bool TL, bool SLAB, int WF = 0>
__global__ __launch_bounds__(SK_TPB, 2) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int K, int N, int kb,
    int log2_bs, int row_bytes, int zp_row_bytes, int chunks, float gscale) {
  static_assert(TN == 1 || TN == 2, "16 or 32 columns: within one group of the tiled layout");
  static_assert(BITS != 3 || !TL, "3-bit weights: operator layout");
  static_assert(!WF || (BITS == 4 && !TL && !HAS_ZP), "FP4 weights: operator layout");
  using Op = MfmaOp<XDT>;
  using ST = typename dt<SDT>::T;
  constexpr int LW = 2 * BITS;                 // code words per lane and tile (64 codes)
  constexpr int CHUNK_BYTES = TKC * BITS / 8;  // tiled layout: one column's 64 codes
  constexpr int OOB = 0x7FFFFFF0;
  // Past every extent (the launcher keeps them at most this) with room for
  // the constant offsets added to it below 2^31.
  constexpr int OOB_A = 0x7FFFE000;
  constexpr uint32_t ZM = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  constexpr int SZ = WF ? 1 : (int)sizeof(typename dt<SDT>::T);   // bytes per scale
  __shared__ float red[SK_WAVES / 2][MT * TN * 4][64];
  extern __shared__ __attribute__((aligned(16))) uint8_t slab_lds[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * TN, m0 = blockIdx.y * 16 * MT;
  const int kpad = kb << log2_bs;
  const int steps = (kpad + SK_KSTEP - 1) / SK_KSTEP;
  const int qsh = min(log2_bs - 4, 2);        // quarter j (16 codes) lies in block b0 + (j >> qsh)
  const int nbl = 4 >> qsh;                   // distinct blocks among a lane's 64 codes

  const int ngroups = (N + TG - 1) / TG;
  const int code_extent = TL ? ngroups * chunks * TG * CHUNK_BYTES : N * row_bytes;
  const int sc_extent = (TL ? ngroups * kb * TG : N * kb) * SZ;
  const int zp_extent = TL ? ngroups * kb * TG * BITS / 8 : N * zp_row_bytes;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, M * K * 2, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rbc = __builtin_amdgcn_make_buffer_rsrc((void*)B, 0, code_extent, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc((void*)scales, 0, sc_extent, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rzp =
      __builtin_amdgcn_make_buffer_rsrc((void*)zp, 0, HAS_ZP ? zp_extent : 0, BUF_WORD3);

  // The workgroup's ranges: columns from col0 (tiled: its group's first),
  // scales from byte s_lo, zero points from z_lo.
  const int cols = TL ? TG : 16 * TN;
  const int col0 = TL ? n0 / TG * TG : n0;
  const int zrow = TL ? kb * 4 * BITS : cols * zp_row_bytes;
  const int s_lo = col0 * kb * SZ, z_lo = TL ? n0 / TG * zrow : n0 * zp_row_bytes;
  const int s_al = s_lo & ~15, z_al = z_lo & ~15;
  const int s_cnt = (s_lo - s_al + cols * kb * SZ + 15) & ~15;   // bytes copied
  // 3-bit: a block's 4-byte zero-point window may reach 3 bytes past a row.
  const int z_cnt = HAS_ZP ? (z_lo - z_al + zrow + (BITS == 3 ? 4 : 0) + 15) & ~15 : 0;

  // Per tile: the byte offset of this lane's codes at k0 = 0 (and per 64-code
  // chunk), the index of its first scale and bit of its first zero point
  // (and their strides per block), relative to the workgroup's ranges.
  int code0[TN], sc0[TN], zb0[TN];
  bool col_ok[TN];
  const int code_chunk = TL ? TG * CHUNK_BYTES : CHUNK_BYTES;
  const int sc_stride = TL ? TG : 1;
  const int zb_stride = TL ? TG * BITS : BITS;
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + c, ci = n - col0;         // ci: column within the range
    col_ok[t] = n < N;
    code0[t] = TL ? ((n / TG) * chunks * TG + ci) * CHUNK_BYTES : n * row_bytes;
    sc0[t] = TL ? ci : ci * kb;
    zb0[t] = TL ? ci * BITS : ci * zp_row_bytes * 8;
  }

  // Scale (as fp32) and zero point of block b of tile t.
  auto scale_at = [&](int t, int b, bool ok) -> float {
    const int e = sc0[t] + b * sc_stride;
    if constexpr (WF) {
      const uint32_t byte = SLAB ? (uint32_t)slab_lds[(s_lo - s_al) + e]
                                 : __builtin_amdgcn_raw_buffer_load_b8(rsc, ok ? s_lo + e : OOB, 0, 0);
      return fp4_scale(byte, WF - 1);
    }
    ST v;
    if constexpr (SLAB) {
      v = *reinterpret_cast<const ST*>(slab_lds + (s_lo - s_al) + e * SZ);
    } else {
      const int so = ok ? s_lo + e * SZ : OOB;
      if constexpr (SZ == 4) v = __builtin_bit_cast(ST, __builtin_amdgcn_raw_buffer_load_b32(rsc, so, 0, 0));
      else v = __builtin_bit_cast(ST, __builtin_amdgcn_raw_buffer_load_b16(rsc, so, 0, 0));
    }
    return dt<SDT>::to_f32(v);
  };
  auto zp_byte = [&](int byte, bool ok) -> uint32_t {      // byte offset within the range
    if constexpr (SLAB) return slab_lds[s_cnt + (z_lo - z_al) + byte];
    else return __builtin_amdgcn_raw_buffer_load_b8(rzp, ok ? z_lo + byte : OOB, 0, 0);
  };

  f32x4 acc[MT][TN];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[i][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint32_t cw[TN][LW];          // codes of the lane's 64 k, per tile
  u32x4 ar[MT][8];              // activations as loaded

  // Codes of step st (a step past the last reads zeros).
  auto load_codes = [&](int st) {
    const int k0 = st * SK_KSTEP + 64 * g;
    const int chunk = k0 >> 6;
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const bool ok = k0 < kpad && col_ok[t];
      if constexpr (BITS == 3) {
        // Operator layout, blob of 3 bs / 8 bytes: the 2-bit plane (bs / 4
        // bytes) then the 1-bit plane (bs / 8 bytes).  The lane's 64 codes
        // go to cw[0..3] (2-bit fields) and cw[4..5] (bits), in code order.
        const int bsz = 1 << log2_bs;
        if (bsz >= 64) {
          // One block: 16 bytes of the first plane, 8 of the second.
          const int base = code0[t] + (k0 >> log2_bs) * (3 * bsz / 8);
          const int i0 = k0 & (bsz - 1);
          const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rbc, ok ? base + i0 / 4 : OOB_A, 0, 0);
          const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(rbc, ok ? base + bsz / 4 + i0 / 8 : OOB_A, 0, 0);
          cw[t][0] = lo.x; cw[t][1] = lo.y; cw[t][2] = lo.z; cw[t][3] = lo.w;
          cw[t][4] = hi.x; cw[t][5] = hi.y;
        } else {
          // 2 (bs 32) or 4 (bs 16) whole blocks: 24 contiguous bytes.
          const int base = ok ? code0[t] + 3 * (k0 / 8) : OOB_A;
          if (bsz == 32) {
            // [plane 2: 8][plane 1: 4] twice, 4-byte aligned.
            const u32x2 a0 = __builtin_amdgcn_raw_buffer_load_b64(rbc, base, 0, 0);
            const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b32(rbc, base + 8, 0, 0);
            const u32x2 a1 = __builtin_amdgcn_raw_buffer_load_b64(rbc, base + 12, 0, 0);
            const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b32(rbc, base + 20, 0, 0);
            cw[t][0] = a0.x; cw[t][1] = a0.y; cw[t][2] = a1.x; cw[t][3] = a1.y;
            cw[t][4] = b0; cw[t][5] = b1;
          } else {
            // [plane 2: 4][plane 1: 2] four times, 2-byte aligned.
            uint32_t h[12];
#pragma unroll
            for (int i = 0; i < 12; ++i) h[i] = __builtin_amdgcn_raw_buffer_load_b16(rbc, base + 2 * i, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; ++j) cw[t][j] = h[3 * j] | (h[3 * j + 1] << 16);
            cw[t][4] = h[2] | (h[5] << 16);
            cw[t][5] = h[8] | (h[11] << 16);
          }
        }
      } else {
        const int off = ok ? code0[t] + chunk * code_chunk : OOB_A;
#pragma unroll
        for (int v = 0; v < LW; v += 4) {
          const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rbc, off + 4 * v, 0, 0);
          cw[t][v] = x.x; cw[t][v + 1] = x.y; cw[t][v + 2] = x.z; cw[t][v + 3] = x.w;
        }
      }
    }
  };
  // Activations of step st: sub-load s of lane (r, g) holds the 8 values
  // k = 256 st + 32 s + 8 g .. + 7 of row r, so each load reads 64
  // contiguous bytes of 16 rows.
  auto load_a = [&](int st) {
    const bool whole = (st + 1) * SK_KSTEP <= K;   // every k of the step inside K
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = m0 + 16 * i + c;
      const int base = row < M ? (row * K + st * SK_KSTEP + 8 * g) * 2 : OOB_A;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        // K % 8 == 0: 8 activations are all in or all out.
        const bool ok = whole || st * SK_KSTEP + 32 * s + 8 * g < K;
        ar[i][s] = __builtin_amdgcn_raw_buffer_load_b128(ra, ok ? base + 64 * s : OOB_A, 0, 0);
      }
    }
  };
  // Dequantize step st and multiply.
  auto compute = [&](int st) {
    const int k0 = st * SK_KSTEP + 64 * g;
    const bool live = k0 < kpad;
    const int b0 = k0 >> log2_bs;
    // Per quarter j (16 codes) of the lane's 64: scale and z * scale.  The
    // lane's distinct blocks are b0 + d, d < nbl; on the operator layout
    // b0 * bits is a multiple of 8 whenever nbl > 1, so their zero points
    // share bytes and one byte serves 8 / bits of them.
    float sfq[TN][4], zsq[TN][4];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const bool ok = live && col_ok[t];
      float sd[4] = {0.f, 0.f, 0.f, 0.f};
      uint32_t zb = 0;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        if (d > 0 && d >= nbl) break;
        const int bd = min(b0 + d, kb - 1);
        sd[d] = scale_at(t, bd, ok);
        if constexpr (HAS_ZP && BITS == 3) {
          // 3-bit zero points may straddle bytes: the 4 bytes from the
          // first block's hold every block's (at most 7 + 4 * 3 bits).
          if (d == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) zb |= zp_byte((zb0[t] >> 3) + ((b0 * 3) >> 3) + i, ok) << (8 * i);
          }
        } else if constexpr (HAS_ZP) {
          if (TL) {
            const int bit = zb0[t] + bd * zb_stride;
            zb |= ((zp_byte(bit >> 3, ok) >> (bit & 7)) & ZM) << (8 * d);
          } else if (((d * BITS) & 7) == 0) {
            zb |= zp_byte((zb0[t] >> 3) + ((b0 * BITS) >> 3) + ((d * BITS) >> 3), ok)
                  << (8 * ((d * BITS) >> 3));
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = j >> qsh;                 // 0 .. nbl - 1
        float sv = sd[0];
        if (d == 1) sv = sd[1];
        else if (d == 2) sv = sd[2];
        else if (d == 3) sv = sd[3];
        uint32_t z = WF ? 0u : 1u << (BITS - 1);
        if constexpr (HAS_ZP) {
          if (TL && BITS != 3) z = (zb >> (8 * d)) & ZM;
          else z = (zb >> (((b0 * BITS) & 7) + d * BITS)) & ZM;
        }
        sfq[t][j] = sv;
        zsq[t][j] = (float)z * sv;
      }
    }
    // The lane's operand of sub-step s' must cover k = 256 st + 64 g + 8 s',
    // like its codes: for h = s' / 4, sub-loads 2 u + h (u = 0..3) of the
    // four lane groups form a 4 x 4 matrix [lane group][u] whose transpose is
    // exactly those operands (lane group g, register j = s' % 4); each dword
    // is transposed with two rounds of lane swaps.
    typename Op::V af[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        u32x4 x[4] = {ar[i][h], ar[i][2 + h], ar[i][4 + h], ar[i][6 + h]};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto p02 = __builtin_amdgcn_permlane32_swap(x[0][e], x[2][e], false, false);
          const auto p13 = __builtin_amdgcn_permlane32_swap(x[1][e], x[3][e], false, false);
          const auto q01 = __builtin_amdgcn_permlane16_swap(p02[0], p13[0], false, false);
          const auto q23 = __builtin_amdgcn_permlane16_swap(p02[1], p13[1], false, false);
          x[0][e] = q01[0]; x[1][e] = q01[1]; x[2][e] = q23[0]; x[3][e] = q23[1];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) af[i][4 * h + j] = __builtin_bit_cast(typename Op::V, x[j]);
      }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        float q[8];
        if constexpr (WF) {
          // Byte j of the word: E2M1 values of codes 2j (low nibble), 2j + 1.
          typedef float f2 __attribute__((ext_vector_type(2)));
          const f2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t][s], 1.0f, 0);
          const f2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t][s], 1.0f, 1);
          const f2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t][s], 1.0f, 2);
          const f2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[t][s], 1.0f, 3);
          q[0] = c0.x; q[1] = c0.y; q[2] = c1.x; q[3] = c1.y;
          q[4] = c2.x; q[5] = c2.y; q[6] = c3.x; q[7] = c3.y;
        } else {
          step_codes<BITS>(cw[t], s, q);
        }
        const float sv = sfq[t][s >> 1], zv = zsq[t][s >> 1];
        u32x4 pk;
        pk.x = Op::pack(fmaf(q[0], sv, -zv), fmaf(q[1], sv, -zv));
        pk.y = Op::pack(fmaf(q[2], sv, -zv), fmaf(q[3], sv, -zv));
        pk.z = Op::pack(fmaf(q[4], sv, -zv), fmaf(q[5], sv, -zv));
        pk.w = Op::pack(fmaf(q[6], sv, -zv), fmaf(q[7], sv, -zv));
        const typename Op::V bf = __builtin_bit_cast(typename Op::V, pk);
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i][t] = Op::run(af[i][s], bf, acc[i][t]);
      }
    }
  };

  // The first step's loads go out before the staging copy and its barrier.
  load_codes(wave);
  load_a(wave);
  if constexpr (SLAB) {
    // A buffer load reads zero for every dword not wholly inside the extent,
    // so the 16 bytes that hold a tensor's last byte are read byte by byte.
    auto copy = [&](__amdgpu_buffer_rsrc_t r, int extent, int from, int count, uint8_t* to) {
      for (int o = threadIdx.x * 16; o < count; o += SK_TPB * 16) {
        if (from + o + 16 <= extent) {
          *reinterpret_cast<u32x4*>(to + o) = __builtin_amdgcn_raw_buffer_load_b128(r, from + o, 0, 0);
        } else if (from + o >= extent) {
          *reinterpret_cast<u32x4*>(to + o) = u32x4{0u, 0u, 0u, 0u};
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) to[o + j] = (uint8_t)__builtin_amdgcn_raw_buffer_load_b8(r, from + o + j, 0, 0);
        }
      }
    };
    copy(rsc, sc_extent, s_al, s_cnt, slab_lds);
    if constexpr (HAS_ZP) copy(rzp, zp_extent, z_al, z_cnt, slab_lds + s_cnt);
    __syncthreads();
  }
  for (int st = wave; st < steps; st += SK_WAVES) {
    if (st != wave) {
      load_codes(st);
      load_a(st);
    }
    compute(st);
  }

  // Partial tiles of the 8 waves summed through LDS in a fixed tree (waves
  // w + h into w for h = 4, 2, 1); wave 0 writes the result.
#pragma unroll
  for (int h = SK_WAVES / 2; h >= 1; h /= 2) {
    if (wave >= h && wave < 2 * h) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) red[wave - h][(i * TN + t) * 4 + e][lane] = acc[i][t][e];
    }
    __syncthreads();
    if (wave < h) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][t][e] += red[wave][(i * TN + t) * 4 + e][lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;
  // Lane l holds rows 4 (l / 16) + e of column l % 16 of each 16 x 16 tile.
#pragma unroll
  for (int t = 0; t < TN; ++t) {
    const int n = n0 + 16 * t + c;
    if (n >= N) continue;
    const float bv = bias ? bits16_to_f32<XDT>(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + 16 * i + 4 * g + e;
        if (m < M) Y[(int64_t)m * N + n] = Op::round((WF ? acc[i][t][e] * gscale : acc[i][t][e]) + bv);
      }
  }
}

// ---------------------------------------------------------------------------
// Launchers.
// ---------------------------------------------------------------------------
static int sk_log2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int TN, int MT>
static hipError_t launch_skinny_t(const MatArgs& a) {
  using ST = typename dt<SDT>::T;
  constexpr int64_t SZ = sizeof(ST);
  const dim3 grid((unsigned)((a.N + 16 * TN - 1) / (16 * TN)), (unsigned)((a.M + 16 * MT - 1) / (16 * MT)));
  // Bytes of a workgroup's zero-point range; LDS for both ranges (with the
  // slack of their 16-byte aligned copies).
  const int64_t cols = a.tiled ? TG : 16 * TN;
  const int64_t zrow = a.tiled ? a.kb * 4 * BITS : cols * a.zp_row_bytes;
  const int64_t zslack = BITS == 3 ? 4 : 0;
  const int64_t lds = (cols * a.kb * SZ + 15 + 15) / 16 * 16 + (HAS_ZP ? (zrow + zslack + 15 + 15) / 16 * 16 : 0);
  const bool slab = lds <= SK_SLAB_MAX;
  decltype(&gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, false, false>) kern;
  if constexpr (BITS == 3) {      // operator layout only
    kern = slab ? gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, false, true>
                : gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, false, false>;
  } else if (slab) {
    kern = a.tiled ? gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, true, true>
                   : gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, false, true>;
  } else {
    kern = a.tiled ? gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, true, false>
                   : gemm_skinny_kernel<BITS, XDT, SDT, HAS_ZP, TN, MT, false, false>;
  }
  if (slab) {
    const hipError_t e = ensure_dynamic_lds((const void*)kern, SK_SLAB_MAX);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, grid, dim3(SK_TPB), slab ? (size_t)lds : 0, a.stream, (const uint16_t*)a.A,
                     a.B, (const ST*)a.scales, a.zp, (const uint16_t*)a.bias, (uint16_t*)a.Y, (int)a.M,
                     (int)a.K, (int)a.N, (int)a.kb, sk_log2(a.block_size), (int)(a.kb * a.blob),
                     (int)a.zp_row_bytes, (int)a.chunks, 1.0f);
  return hipGetLastError();
}

// M <= 16: one 16-row tile per workgroup; more rows: 32-row tiles (grid y).
// 32 columns per workgroup, or 16 when 32 would leave compute units idle.
template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_skinny_m(const MatArgs& a) {
  const int64_t row_tiles = a.M <= 16 ? 1 : (a.M + 31) / 32;
  const bool narrow = row_tiles * ((a.N + 31) / 32) < SK_FULL_ROUND;
  if (a.M <= 16) return narrow ? launch_skinny_t<BITS, XDT, SDT, HAS_ZP, 1, 1>(a)
                               : launch_skinny_t<BITS, XDT, SDT, HAS_ZP, 2, 1>(a);
  return narrow ? launch_skinny_t<BITS, XDT, SDT, HAS_ZP, 1, 2>(a)
                : launch_skinny_t<BITS, XDT, SDT, HAS_ZP, 2, 2>(a);
}

template <int BITS, int XDT>
static hipError_t launch_skinny_s(const MatArgs& a) {
  switch (a.s_dtype) {
    case DT_F32: return a.zp ? launch_skinny_m<BITS, XDT, DT_F32, true>(a) : launch_skinny_m<BITS, XDT, DT_F32, false>(a);
    case DT_F16: return a.zp ? launch_skinny_m<BITS, XDT, DT_F16, true>(a) : launch_skinny_m<BITS, XDT, DT_F16, false>(a);
    default: return a.zp ? launch_skinny_m<BITS, XDT, DT_BF16, true>(a) : launch_skinny_m<BITS, XDT, DT_BF16, false>(a);
  }
}

template <int BITS>
static hipError_t launch_skinny_x(const MatArgs& a) {
  return a.a_dtype == DT_F16 ? launch_skinny_s<BITS, DT_F16>(a) : launch_skinny_s<BITS, DT_BF16>(a);
}

// 2-, 3- and 8-bit weights (gemm_skinny_w.hip; 4-bit and FP4 in
// gemm_skinny.hip), so that the two halves compile in parallel.
hipError_t launch_gemm_skinny_w(const MatArgs& a);

}  // namespace qmm
