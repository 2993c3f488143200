// compint8_tiled.h -- the CompInt8 int8 matrix-core kernel template (see
// compint8_tiled.hip for the definition it computes), shared by
// compint8_tiled.hip (int8 activations) and compint8_int16.hip (int16
// activations as two int8 planes) so the two instance sets compile in
// parallel.
#pragma once

#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

#include <algorithm>
#include <type_traits>

namespace qmm {

namespace ct {

constexpr int RSRC3 = 0x00020000;
constexpr int CT_D = 4;            // chunks in flight per wave
constexpr int CT_MAXW = 16;

template <int BITS>
struct CtGeom {
  static constexpr int CB = TKC * BITS / 8;     // bytes per column chunk
  static constexpr int LB = CB / 4;             // code bytes per lane per chunk (16 codes)
};
// 3-bit codes (operator layout only): a block of bs codes is bs / 4 bytes of
// the 2-bit plane then bs / 8 of the 1-bit plane (blocks of 64 codes or
// more: a chunk lies inside one block).

// The lane's 16 codes as four words of int8, in plane order (see unpack).
template <int BITS>
__device__ __forceinline__ i32x4 unpack_codes(const u32x4& raw) {
  if constexpr (BITS == 4) {
    // 8 bytes, code 2j in the low nibble of byte j: planes of even and odd
    // codes of each 4-byte word.
    const uint32_t w0 = raw.x, w1 = raw.y;
    return i32x4{(int)(w0 & 0x0F0F0F0Fu), (int)((w0 >> 4) & 0x0F0F0F0Fu),
                 (int)(w1 & 0x0F0F0F0Fu), (int)((w1 >> 4) & 0x0F0F0F0Fu)};
  } else if constexpr (BITS == 2) {
    // 4 bytes, code 4j + i at bits 2i of byte j: plane i holds codes i, 4 + i,
    // 8 + i, 12 + i.
    const uint32_t w = raw.x;
    return i32x4{(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u),
                 (int)((w >> 4) & 0x03030303u), (int)((w >> 6) & 0x03030303u)};
  } else if constexpr (BITS == 3) {
    // Operator layout's two planes: raw.x = the 2-bit plane of the lane's 16
    // codes (code j at bits 2j), raw.y = the 1-bit plane (bit j).  Planes as
    // for 2-bit codes; bit 4j + i of the 1-bit plane goes to bit 2 of byte j
    // of plane i.
    const uint32_t w = raw.x, h = raw.y;
    auto hi = [&](int i) {
      const uint32_t t = h >> i;
      return ((t & 1u) << 2) | ((t & 0x10u) << 6) | ((t & 0x100u) << 10) | ((t & 0x1000u) << 14);
    };
    return i32x4{(int)((w & 0x03030303u) | hi(0)), (int)(((w >> 2) & 0x03030303u) | hi(1)),
                 (int)(((w >> 4) & 0x03030303u) | hi(2)), (int)(((w >> 6) & 0x03030303u) | hi(3))};
  } else {
    // 16 bytes in order, as code - 128.
    return i32x4{(int)(raw.x ^ 0x80808080u), (int)(raw.y ^ 0x80808080u),
                 (int)(raw.z ^ 0x80808080u), (int)(raw.w ^ 0x80808080u)};
  }
}

// The lane's 16 activation bytes (natural order) permuted into the codes'
// plane order.  __builtin_amdgcn_perm(hi, lo, sel): selector byte values 0-3
// pick bytes of lo, 4-7 bytes of hi.
template <int BITS>
__device__ __forceinline__ i32x4 permute_acts(const u32x4& a) {
  if constexpr (BITS == 3) {
    return permute_acts<2>(a);
  } else if constexpr (BITS == 4) {
    return i32x4{(int)__builtin_amdgcn_perm(a.y, a.x, 0x06040200u),
                 (int)__builtin_amdgcn_perm(a.y, a.x, 0x07050301u),
                 (int)__builtin_amdgcn_perm(a.w, a.z, 0x06040200u),
                 (int)__builtin_amdgcn_perm(a.w, a.z, 0x07050301u)};
  } else if constexpr (BITS == 2) {
    // Plane i = bytes (i, 4 + i, 8 + i, 12 + i): byte i of each word.
    const uint32_t p01[2] = {__builtin_amdgcn_perm(a.y, a.x, 0x05010400u),   // x0 y0 x1 y1
                             __builtin_amdgcn_perm(a.y, a.x, 0x07030602u)};  // x2 y2 x3 y3
    const uint32_t p23[2] = {__builtin_amdgcn_perm(a.w, a.z, 0x05010400u),
                             __builtin_amdgcn_perm(a.w, a.z, 0x07030602u)};
    return i32x4{(int)__builtin_amdgcn_perm(p23[0], p01[0], 0x05040100u),   // x0 y0 z0 w0
                 (int)__builtin_amdgcn_perm(p23[0], p01[0], 0x07060302u),   // x1 y1 z1 w1
                 (int)__builtin_amdgcn_perm(p23[1], p01[1], 0x05040100u),
                 (int)__builtin_amdgcn_perm(p23[1], p01[1], 0x07060302u)};
  } else {
    return i32x4{(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  }
}

// One chunk in flight: the lane's code bytes (LB of them used), its 16
// activation bytes, and the aligned 32-bit words holding the scale and zero
// point of the chunk's block (loaded with every chunk so that no load sits
// inside the block-end branch).
struct CtSlot {
  u32x4 code;
  u32x4 act;
  uint32_t sw, zw;
  uint32_t sw2, zw2;   // HB: the chunk's second block
  u32x4 act2;          // AB = 2: the lane's activations 8..15
};

// STAGE: the workgroup first copies its Mp activation rows into LDS, padded
// by 16 bytes per row so that the rows of a fragment read fall in distinct
// banks, and its waves read them there (rows past Mp as zeros, by a select);
// otherwise every wave loads its rows from memory with each chunk.  The CS
// column slices of the workgroup share the staged rows.
// HB: blocks of 32 codes, two per 64-code chunk: each chunk runs its MFMAs
// twice, once with the activations of the second block zeroed (lane groups
// 2 and 3) and once with those of the first (groups 0 and 1), and closes both
// blocks; shares of K are whole pairs of blocks.
// AB = 2: int16 activations (the int16 route, operator layout, unstaged):
// a = 256 ah + (al - 128) + 128 with ah = a >> 8 and al - 128 = (a & 255) ^
// 128 both int8, so sum a (c - zp) = 256 sum ah (c - zp) + sum (al - 128)
// (c - zp) + 128 sum (c - zp): two activation planes through the MFMAs, and
// the codes' sum per block by one more MFMA against all-ones activations.
template <int BITS, int SDT, int YDT, bool HAS_ZP, bool DOTS, bool STAGE, bool OPL, bool HB,
          int AB = 1>
__global__ __launch_bounds__(CT_MAXW * 64) void compint8_tiled_kernel(
    const int8_t* __restrict__ qa, const float* __restrict__ sa, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zps,
    const typename dt<YDT>::T* __restrict__ bias, typename dt<YDT>::T* __restrict__ Y,
    int32_t* __restrict__ dots, int Mp, int N, int kb, int Kp, int chunks, int log2_cpb,
    int n_slices, int CS, int S, int row_bytes, int zp_row_bytes) {
  using G = CtGeom<BITS>;
  using ST = typename dt<SDT>::T;
  constexpr int CB = G::CB, LB = G::LB;
  constexpr int SZ = (int)sizeof(ST);
  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  constexpr int OFF = (BITS == 8) ? 128 : 0;

  extern __shared__ float smem_ct[];
  float* saT = smem_ct;                         // [kb][16]: sa of row r, block b (0 past Mp)
  float* red = smem_ct + kb * 16;               // [W][16 x 16] partial sums
  const int qrow = Kp + 16;                     // STAGE: bytes per staged row
  int8_t* qs = reinterpret_cast<int8_t*>(red + CS * S * 256);   // STAGE: [16][qrow]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int W = CS * S;
  const int cs = wave % CS, s = wave / CS;
  const int slice = blockIdx.x * CS + cs;
  const bool has_slice = slice < n_slices;
  const int grp = slice >> 1;
  const int col = (slice & 1) * 16 + (lane & 15);   // column within the group
  const int n = grp * TG + col;
  const int g = lane >> 4;                          // 16 reduction indices of the 64
  const int rowA = lane & 15;                       // activation row of this lane (A)

  for (int i = threadIdx.x; i < kb * 16; i += blockDim.x) {
    const int b = i >> 4, r = i & 15;
    saT[i] = r < Mp ? sa[r * kb + b] : 0.0f;
  }

  const int groups = (N + TG - 1) / TG;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)codes, 0, OPL ? N * row_bytes : groups * chunks * TG * CB, RSRC3);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)qa, 0, Mp * Kp * AB, RSRC3);
  // No scales (the block-dot export on the operator layout): every scale
  // load is out of range and reads zero.
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, scales ? (OPL ? N * kb : groups * kb * TG) * SZ : 0, RSRC3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)zps, 0, HAS_ZP ? (OPL ? N * zp_row_bytes : groups * kb * TG * BITS / 8) : 0, RSRC3);
  // Blocks of this wave's share (whole blocks, so no block is split).
  // HB: units are pairs of blocks (one chunk each).
  const int units = HB ? (kb + 1) / 2 : kb;
  const int bps = (units + S - 1) / S;
  const int b_lo = s * bps;
  const int b_hi = has_slice ? min(units, b_lo + bps) : b_lo;
  const int cpb = HB ? 1 : 1 << log2_cpb;           // chunks per unit
  const int c_lo = b_lo * cpb;
  const int nch = max(0, (b_hi - b_lo) * cpb);

  // Codes of chunk c: lane_code + c * code_step.  Columns past N read zeros
  // (tiled: the group's padding; operator layout: past the extent).
  const int lane_code = OPL ? n * row_bytes + g * LB : (grp * chunks * TG + col) * CB + g * LB;
  const int code_step = OPL ? CB : TG * CB;
  // Scale entry of block b: sc_base + b * sc_step; zero-point bit: zb_base +
  // b * zb_step.
  const int sc_base = OPL ? n * kb : grp * kb * TG + col, sc_step = OPL ? 1 : TG;
  const int zb_base = OPL ? n * zp_row_bytes * 8 : (grp * kb * TG + col) * BITS;
  const int zb_step = OPL ? BITS : TG * BITS;
  const int lane_act = (rowA * Kp + g * 16) * AB;
  auto issue = [&](CtSlot& sl, int j) {
    const int c = c_lo + j;
    if constexpr (BITS == 3) {
      // The lane's 16 codes: 4 bytes of the 2-bit plane and 2 of the 1-bit
      // plane of its block (columns past N: past the extent, zeros).
      const int bs = HB ? 32 : TKC << log2_cpb;
      const int base = n * row_bytes + (HB ? 2 * c + (g >> 1) : c >> log2_cpb) * (3 * bs / 8);
      const int i0 = HB ? 16 * (g & 1) : (c & (cpb - 1)) * TKC + 16 * g;
      sl.code = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rc, base + i0 / 4, 0, BUF_STREAM),
                      (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rc, base + bs / 4 + i0 / 8, 0,
                                                                      BUF_STREAM),
                      0u, 0u};
    } else if constexpr (LB == 16)
      sl.code = __builtin_amdgcn_raw_buffer_load_b128(rc, lane_code + c * code_step, 0, BUF_STREAM);
    else if constexpr (LB == 8) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rc, lane_code + c * code_step, 0, BUF_STREAM);
      sl.code = u32x4{v.x, v.y, 0u, 0u};
    } else {
      sl.code = u32x4{__builtin_amdgcn_raw_buffer_load_b32(rc, lane_code + c * code_step, 0, BUF_STREAM),
                      0u, 0u, 0u};
    }
    if constexpr (!STAGE) sl.act = __builtin_amdgcn_raw_buffer_load_b128(ra, lane_act + c * TKC * AB, 0, 0);
    if constexpr (AB == 2) sl.act2 = __builtin_amdgcn_raw_buffer_load_b128(ra, lane_act + c * TKC * 2 + 16, 0, 0);
    const int b = HB ? 2 * c : c >> log2_cpb;
    const int si = sc_base + b * sc_step;
    const int zbit = zb_base + b * zb_step;
    if constexpr (HB) {
      // The second block's scale and zero point (read, and used, only as a
      // value at bit 0: a load of its own width at its own offset).
      const int si2 = si + sc_step, zbit2 = zbit + zb_step;
      if constexpr (SZ == 4) sl.sw2 = __builtin_amdgcn_raw_buffer_load_b32(rs, si2 * 4, 0, 0);
      else sl.sw2 = __builtin_amdgcn_raw_buffer_load_b16(rs, si2 * 2, 0, 0);
      if constexpr (HAS_ZP) {
        sl.zw2 = __builtin_amdgcn_raw_buffer_load_b8(rz, zbit2 >> 3, 0, 0);
        if constexpr (BITS == 3) sl.zw2 |= __builtin_amdgcn_raw_buffer_load_b8(rz, (zbit2 >> 3) + 1, 0, 0) << 8;
      }
      // The first block's, the same way.
      if constexpr (SZ == 4) sl.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, si * 4, 0, 0);
      else sl.sw = __builtin_amdgcn_raw_buffer_load_b16(rs, si * 2, 0, 0);
      if constexpr (HAS_ZP) {
        sl.zw = __builtin_amdgcn_raw_buffer_load_b8(rz, zbit >> 3, 0, 0);
        if constexpr (BITS == 3) sl.zw |= __builtin_amdgcn_raw_buffer_load_b8(rz, (zbit >> 3) + 1, 0, 0) << 8;
      }
    } else if constexpr (OPL) {
      // The value itself (shifted back to bit 0 of the word on use).
      if constexpr (SZ == 4) sl.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, si * 4, 0, 0);
      else sl.sw = __builtin_amdgcn_raw_buffer_load_b16(rs, si * 2, 0, 0);
      if constexpr (HAS_ZP) {
        sl.zw = __builtin_amdgcn_raw_buffer_load_b8(rz, zbit >> 3, 0, 0);
        // A 3-bit zero point may continue into the next byte (past the
        // zero-point rows: zero).
        if constexpr (BITS == 3) sl.zw |= __builtin_amdgcn_raw_buffer_load_b8(rz, (zbit >> 3) + 1, 0, 0) << 8;
      }
    } else {
      sl.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, (si * SZ) & ~3, 0, 0);
      if constexpr (HAS_ZP) sl.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, ((zbit) >> 5) * 4, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  CtSlot sl[CT_D];
#pragma unroll
  for (int q = 0; q < CT_D; ++q) issue(sl[q], q);
  if constexpr (STAGE) {
    // 16-byte pieces of the 16 rows (rows past Mp read zeros).
    const int ppr = Kp / 16;
    for (int i = threadIdx.x; i < Mp * ppr; i += blockDim.x) {
      const int r = i / ppr, c16 = i - r * ppr;
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ra, r * Kp + c16 * 16, 0, 0);
      *reinterpret_cast<u32x4*>(qs + r * qrow + c16 * 16) = v;
    }
  }
  __syncthreads();   // saT (and the activation rows) staged

  const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  f32x4 y = {0.0f, 0.0f, 0.0f, 0.0f};
  i32x4 acc = {0, 0, 0, 0}, asum = {0, 0, 0, 0};
  i32x4 acc2 = {0, 0, 0, 0}, asum2 = {0, 0, 0, 0}, csum = {0, 0, 0, 0};   // AB = 2
  // Chunk j: two MFMAs; at the block's last chunk the epilogue scales it.
  auto consume = [&](const CtSlot& sl, int j) {
    const i32x4 bv = unpack_codes<BITS>(sl.code);
    u32x4 raw_act;
    if constexpr (STAGE) {
      // (HB, odd kb: the last chunk's second half lies past the staged rows;
      // its block is not closed, zeros stand in.)
      const int koff = (c_lo + j) * TKC + g * 16;
      const bool kok = !HB || koff < Kp;
      const u32x4 v = *reinterpret_cast<const u32x4*>(qs + min(rowA, Mp - 1) * qrow +
                                                      (kok ? koff : 0));
      raw_act = (rowA < Mp && kok) ? v : u32x4{0u, 0u, 0u, 0u};
    } else

      raw_act = sl.act;
    if constexpr (AB == 2) {
      // The two int8 planes of the lane's 16 int16 activations (natural
      // order), then the codes' plane order.
      const uint32_t d[8] = {sl.act.x, sl.act.y, sl.act.z, sl.act.w,
                             sl.act2.x, sl.act2.y, sl.act2.z, sl.act2.w};
      u32x4 hi, lo;
      hi.x = __builtin_amdgcn_perm(d[1], d[0], 0x07050301u); lo.x = __builtin_amdgcn_perm(d[1], d[0], 0x06040200u);
      hi.y = __builtin_amdgcn_perm(d[3], d[2], 0x07050301u); lo.y = __builtin_amdgcn_perm(d[3], d[2], 0x06040200u);
      hi.z = __builtin_amdgcn_perm(d[5], d[4], 0x07050301u); lo.z = __builtin_amdgcn_perm(d[5], d[4], 0x06040200u);
      hi.w = __builtin_amdgcn_perm(d[7], d[6], 0x07050301u); lo.w = __builtin_amdgcn_perm(d[7], d[6], 0x06040200u);
      lo ^= 0x80808080u;
      const i32x4 ah = permute_acts<BITS>(hi), al = permute_acts<BITS>(lo);
      const i32x4 zero = {0, 0, 0, 0};
      // Per half (HB: the chunk's two blocks; else one pass over the chunk).
#pragma unroll
      for (int h = 0; h < (HB ? 2 : 1); ++h) {
        const bool live = !HB || (h == 0 ? g < 2 : g >= 2);
        const i32x4 ahh = live ? ah : zero, alh = live ? al : zero, onh = live ? ones : zero;
        i32x4 t_h = HB ? zero : acc, s_h = HB ? zero : asum;
        i32x4 t_l = HB ? zero : acc2, s_l = HB ? zero : asum2, cs = HB ? zero : csum;
        t_h = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahh, bv, t_h, 0, 0, 0);
        s_h = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahh, ones, s_h, 0, 0, 0);
        t_l = __builtin_amdgcn_mfma_i32_16x16x64_i8(alh, bv, t_l, 0, 0, 0);
        s_l = __builtin_amdgcn_mfma_i32_16x16x64_i8(alh, ones, s_l, 0, 0, 0);
        cs = __builtin_amdgcn_mfma_i32_16x16x64_i8(onh, bv, cs, 0, 0, 0);
        const bool close = HB || ((j + 1) & (cpb - 1)) == 0;
        if (!HB && !close) {
          acc = t_h; asum = s_h; acc2 = t_l; asum2 = s_l; csum = cs;
          continue;
        }
        const int b = HB ? 2 * (c_lo + j) + h : b_lo + (j >> log2_cpb);
        if (b >= kb) break;
        const uint32_t sw = (HB && h) ? sl.sw2 : sl.sw, zw = (HB && h) ? sl.zw2 : sl.zw;
        const int si = sc_base + b * sc_step;
        const int zbit = zb_base + b * zb_step;
        float sc;
        if constexpr (SZ == 4) sc = __uint_as_float(sw);
        else sc = bits16_to_f32<SDT>((uint16_t)(OPL || HB ? sw : sw >> ((si & 1) * 16)));
        int z = 1 << (BITS - 1);
        if constexpr (HAS_ZP) z = (int)((zw >> (zbit & (OPL || HB ? 7 : 31))) & m);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(saT + b * 16 + 4 * g);
        const int zo = z - OFF;
        const int kcount = HB ? 32 : TKC * cpb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // Modular int32 arithmetic; the exact block dot fits (|dot| <
          // 2^31 for blocks of at most 128 codes).
          const int d = 256 * (t_h[e] - zo * s_h[e]) + (t_l[e] - zo * s_l[e]) +
                        128 * (cs[e] - zo * kcount);
          if constexpr (DOTS) {
            const int r = 4 * g + e;
            if (r < Mp && n < N) dots[((int64_t)r * N + n) * kb + b] = d;
          }
          y[e] = fmaf((float)d, s4[e] * sc, y[e]);
        }
        if constexpr (!HB) {
          acc = zero; asum = zero; acc2 = zero; asum2 = zero; csum = zero;
        }
      }
      return;
    }
    const i32x4 av = permute_acts<BITS>(raw_act);
    if constexpr (HB) {
      // Both blocks of the chunk, each closed at once.
      const i32x4 zero = {0, 0, 0, 0};
      const i32x4 av0 = g < 2 ? av : zero, av1 = g < 2 ? zero : av;
      const i32x4 d0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av0, bv, zero, 0, 0, 0);
      const i32x4 s0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av0, ones, zero, 0, 0, 0);
      const i32x4 d1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av1, bv, zero, 0, 0, 0);
      const i32x4 s1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(av1, ones, zero, 0, 0, 0);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int b = 2 * (c_lo + j) + h;
        if (b >= kb) break;
        const uint32_t sw = h ? sl.sw2 : sl.sw, zw = h ? sl.zw2 : sl.zw;
        float sc;
        if constexpr (SZ == 4) sc = __uint_as_float(sw);
        else sc = bits16_to_f32<SDT>((uint16_t)sw);
        int z = 1 << (BITS - 1);
        if constexpr (HAS_ZP) z = (int)((zw >> ((zb_base + b * zb_step) & 7)) & m);
        const f32x4 s4 = *reinterpret_cast<const f32x4*>(saT + b * 16 + 4 * g);
        const int zo = z - OFF;
        const i32x4 dd = h ? d1 : d0, ss = h ? s1 : s0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = dd[e] - zo * ss[e];
          if constexpr (DOTS) {
            const int r = 4 * g + e;
            if (r < Mp && n < N) dots[((int64_t)r * N + n) * kb + b] = d;
          }
          y[e] = fmaf((float)d, s4[e] * sc, y[e]);
        }
      }
      return;
    }
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, acc, 0, 0, 0);
    asum = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, ones, asum, 0, 0, 0);
    if (((j + 1) & (cpb - 1)) == 0) {
      const int b = b_lo + (j >> log2_cpb);
      const int si = sc_base + b * sc_step;
      const int zbit = zb_base + b * zb_step;
      float sc;
      if constexpr (SZ == 4) sc = __uint_as_float(sl.sw);
      else sc = bits16_to_f32<SDT>((uint16_t)(OPL ? sl.sw : sl.sw >> ((si & 1) * 16)));
      int z = 1 << (BITS - 1);
      if constexpr (HAS_ZP) z = (int)((sl.zw >> (zbit & (OPL ? 7 : 31))) & m);
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(saT + b * 16 + 4 * g);
      const int zo = z - OFF;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int d = acc[e] - zo * asum[e];
        if constexpr (DOTS) {
          const int r = 4 * g + e;
          if (r < Mp && n < N) dots[((int64_t)r * N + n) * kb + b] = d;
        }
        y[e] = fmaf((float)d, s4[e] * sc, y[e]);
      }
      acc = i32x4{0, 0, 0, 0};
      asum = i32x4{0, 0, 0, 0};
    }
  };
  int j0 = 0;
  for (; j0 + CT_D < nch; j0 += CT_D) {
#pragma unroll
    for (int q = 0; q < CT_D; ++q) {
      consume(sl[q], j0 + q);
      issue(sl[q], j0 + q + CT_D);
    }
  }
#pragma unroll
  for (int q = 0; q < CT_D; ++q)
    if (j0 + q < nch) consume(sl[q], j0 + q);

  if constexpr (!DOTS) {
    // Lane l holds rows 4 * (l / 16) + e of column l % 16.
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wave * 256 + (4 * g + e) * 16 + (lane & 15)] = y[e];
    __syncthreads();
    if (s == 0 && has_slice) {
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float o = red[cs * 256 + r * 16 + (lane & 15)];
        for (int t = 1; t < S; ++t) o += red[(t * CS + cs) * 256 + r * 16 + (lane & 15)];
        if (r < Mp && n < N) {
          if (bias) o += dt<YDT>::to_f32(bias[n]);
          Y[(int64_t)r * N + n] = dt<YDT>::from_f32(o);
        }
      }
    }
  }
  (void)W;
}

// LDS bytes of a launch: sa [kb][16], the share sums [CS * S][256], and for
// STAGE the rows padded activation rows.
inline size_t ct_lds(int64_t kb, int64_t Kp, int CS, int S, bool stage, int rows) {
  return (size_t)(kb * 16 + CS * S * 256) * 4 + (stage ? (size_t)rows * (Kp + 16) : 0);
}
constexpr size_t CT_STAGE_LDS_MAX = 128 * 1024;

}  // namespace ct

}  // namespace qmm
