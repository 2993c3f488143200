// gemm_mfma.h -- the 256-row matrix-core kernel over block-quantized weights
// (bf16 / f16 activations) and its launch for one column-tile width; shared
// by gemm.hip (224- and 256-column tiles, group indices, FP4) and
// gemm_narrow.hip (64- and 128-column tiles), so that the two instantiation
// sets compile in parallel.
//
// A workgroup of 8 waves computes a 256 x BN tile of Y, each wave 64 x BN/2
// as 4 x BN/32 v_mfma_f32_16x16x32_{bf16,f16} tiles accumulated in fp32.
// Per K-step of 64: the A tile goes from memory straight into LDS, the B
// tile is dequantized once for the whole workgroup (each thread 32 codes of
// one column: unpack, subtract the zero point, multiply by the block scale in
// fp32, round to the activation dtype) and stored to LDS; then every wave
// reads its operand fragments from LDS.  LDS rows are 128 bytes with their
// 16-byte pieces XOR-permuted by the row (lds_at), so the 16 rows of a
// fragment read fall in distinct bank groups.  Loads of A and of the codes
// go through buffer descriptors whose extents end at M, K and N, so ragged
// edges read zeros.
#pragma once

#include <algorithm>
#include <type_traits>

#include "mfma_ops.h"
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

namespace qmm {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int LDS_ROW = GBK;                 // LDS row (128 bytes), in 16-bit elements
constexpr int STAGE = GBM * LDS_ROW;         // one operand tile, in 16-bit elements

// Element offset of 16-byte piece p (8 elements) of row r of an LDS tile.
// The 8 pieces of a row are permuted by an XOR with a function of the row's
// low four bits, so that the 16 rows of a fragment read (same piece) fall in
// distinct 16-byte bank groups whether a pass serves 8 lanes from 32 banks
// or 16 lanes from 64 banks; so do the 8 pieces of one row written by 8
// adjacent lanes.
__device__ __forceinline__ int lds_at(int r, int p) {
  const int f = ((r >> 1) & 7) ^ ((r & 1) << 2);
  return r * LDS_ROW + ((p ^ f) << 3);
}
// ---------------------------------------------------------------------------
// MFMA kernel.  Requirements checked by the launcher: K % 8 == 0, A 16-byte
// aligned (A rows are read as 16-byte chunks of 8 activations), and every
// buffer byte offset below 2^31.
//
// Tile GBM x BN with BN = 32 * TN (TN = 8: 256 columns, TN = 7: 224 columns,
// which splits N = 14336 into whole tiles and 2048 x 14336 into exactly two
// rounds of 256 workgroups; TN = 4 and 2, 128 and 64 columns, when wider
// tiles would leave compute units idle).  8 waves, two per SIMD so one wave's waits hide
// under the other's MFMAs, arranged 4 (M) x 2 (N); each wave owns 64 x 16*TN
// outputs as 4 x TN v_mfma_f32_16x16x32 tiles.
// Per K-step of GBK = 64: thread t dequantizes 32 codes of column t >> 1
// (half t & 1 of the step); threads t >= 2 * BN only copy A.
// Pipeline: A tiles are loaded into LDS one step ahead, the codes,
// scales and zero points two steps ahead (register stage = step parity, fixed
// at compile time by unrolling the loop by two); the next step is written to
// the other LDS buffer, after this step's MFMAs by waves 0-3 and (its B tile)
// before them by waves 4-7, so that the two waves of a SIMD alternate matrix
// and vector work; one barrier per step.  The
// loop body has no branch around its loads (loads past the last step use
// out-of-range offsets or harmless in-range addresses), so the compiler's
// waits on the load counter stay exact.
// ---------------------------------------------------------------------------
// LDS bytes of the kernel's double-buffered A (256 rows) and B (BN rows)
// tiles.
template <int BN>
constexpr size_t mfma_lds_bytes() {
  return (size_t)(2 * STAGE + 2 * BN * LDS_ROW) * sizeof(uint16_t);
}

constexpr int GEMM_WAVES = 8;
constexpr int GEMM_TPB = 64 * GEMM_WAVES;

// GI: group indices (operator layout only): code k of a column takes the
// scale and zero point of group g_idx[k] (clamped into 0..kb-1) instead of
// its block's, looked up per code during the dequantization -- GI = 1 from
// memory; GI = 2 from a table of the tile's columns built in LDS after the
// operand tiles (mfma_lds_bytes), with the step's group indices loaded with
// its codes.
// WF: block-scaled FP4 weights (1 + FP4_MX or 1 + FP4_NV; operator layout,
// BITS = 4, no zero points): codes are E2M1 values (v_cvt_scalef32_pk_f32_fp4
// with a unit scale), scales are one E8M0 / E4M3 byte per block, and the
// result is multiplied by gscale.  Each weight, e2m1 * scale, has at most 6
// significant bits, so its rounding to the activation dtype is exact.
template <int BITS, int XDT, int SDT, bool HAS_ZP, int TN, bool TL, int GI = 0, int WF = 0>
__global__ __launch_bounds__(GEMM_TPB) void gemm_mfma_kernel(
    const uint16_t* __restrict__ A, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ Y, int M, int K, int N, int kb,
    int log2_bs, int log2_blob, int zp_row_bytes, int tiles_m, int chunks,
    const int32_t* __restrict__ g_idx, float gscale) {
  static_assert(!(GI && TL), "group indices run on the operator layout");
  static_assert(!WF || (BITS == 4 && !TL && !GI && !HAS_ZP), "FP4 weights: operator layout");
  using Op = MfmaOp<XDT>;
  using ST = typename dt<SDT>::T;
  constexpr int BN = 32 * TN;
  static_assert(BITS != 3 || (!TL && !GI && !WF), "3-bit weights: operator layout");
  constexpr int P = BITS == 3 ? 8 : 32 / BITS; // codes per 32-bit word (3-bit: unused)
  constexpr int HK = GBK / 2;                  // codes per thread per K-step
  // Code words per thread per K-step; 3-bit: the 32 codes' 2-bit plane (two
  // words) and 1-bit plane (one word).
  constexpr int WPT = BITS == 3 ? 3 : HK / P;
  constexpr int TM = 4;                        // MFMA row tiles per wave
  constexpr int BSTRIDE = BN * LDS_ROW;        // one B tile, in 16-bit elements
  extern __shared__ __attribute__((aligned(16))) uint16_t lds_g[];
  uint16_t* As = lds_g;                        // [2][GBM][LDS_ROW], pieces per lds_at
  uint16_t* Bs = lds_g + 2 * STAGE;            // [2][BN][LDS_ROW], pieces per lds_at
  // GI = 2: the table of the BN columns' scales and zero points.
  uint8_t* gslab = reinterpret_cast<uint8_t*>(lds_g + 2 * STAGE + 2 * BSTRIDE);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Consecutive workgroups take consecutive M tiles of one N tile: with the
  // round-robin dispatch over the 8 XCDs, each XCD keeps re-using the same A
  // rows in its L2 while the B columns stream.
  const int tile_m = blockIdx.x % tiles_m, tile_n = blockIdx.x / tiles_m;
  const int m0 = tile_m * GBM, n0 = tile_n * BN;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * (16 * TN);

  constexpr int OOB = 0x7FFFFFF0;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void*)A, 0, M * K * 2, BUF_WORD3);
  // Whole-matrix descriptors (wave-uniform: a lane-varying descriptor would
  // make the compiler loop over the lanes for every load).  This thread's
  // column is addressed by offset; a column past N (or a thread with no
  // column) gets an offset past the extent, which reads zeros.
  // Thread t dequantizes half t & 1 (32 codes) of column t >> 1 of the tile,
  // so adjacent lanes read adjacent 16-byte pieces.
  //   operator layout: codes at n * row_bytes + k * bits / 8; scale (n, b) at
  //     n * kb + b; zero point (n, b) at bit n * zp_row_bytes * 8 + b * bits.
  //   tiled layout (qmm_layout.h): codes at ((g * chunks + c) * 32 + i) *
  //     chunk_bytes + half; scale at (g * kb + b) * 32 + i; zero point at bit
  //     ((g * kb + b) * 32 + i) * bits, with n = 32 g + i and c = k / 64.
  // Row length of the operator layout (3-bit blobs, 3 bs / 8 bytes, are not
  // powers of two).
  const int row_bytes = BITS == 3 ? kb * (3 << log2_bs) / 8 : kb << log2_blob;
  constexpr int CHUNK_BYTES = TKC * BITS / 8;
  const bool dq = tid < 2 * BN;                // this thread dequantizes
  const int bcol = tid >> 1;
  const int ncol = n0 + bcol;
  const int khalf = (tid & 1) * HK;            // which half of the K-step
  const bool ncol_ok = dq && ncol < N;
  const int ngroups = (N + TG - 1) / TG;
  const int code_extent = TL ? ngroups * chunks * TG * CHUNK_BYTES : N * row_bytes;
  const int sc_extent = TL ? ngroups * kb * TG : N * kb;
  const int zp_extent = TL ? ngroups * kb * TG * BITS / 8 : N * zp_row_bytes;
  const __amdgpu_buffer_rsrc_t rbc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)B, 0, code_extent, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, sc_extent * (WF ? 1 : (int)sizeof(ST)), BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rzp = __builtin_amdgcn_make_buffer_rsrc(
      (void*)zp, 0, HAS_ZP ? zp_extent : 0, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rgi = __builtin_amdgcn_make_buffer_rsrc(
      (void*)g_idx, 0, GI ? K * 4 : 0, BUF_WORD3);
  const int cg = ncol / TG, ci = ncol % TG;
  // Byte offset of this thread's codes for the K-step starting at k0 = 64 s:
  // col_code0 + s * code_step.
  const int col_code0 = !ncol_ok ? OOB
                        : TL ? (cg * chunks * TG + ci) * CHUNK_BYTES + (khalf * BITS) / 8
                             : ncol * row_bytes + (khalf * BITS) / 8;
  const int code_step = TL ? TG * CHUNK_BYTES : CHUNK_BYTES;
  // Scale index of block b: col_sc0 + b * sc_stride.
  const int col_sc0 = !ncol_ok ? OOB / 4 : TL ? cg * kb * TG + ci : ncol * kb;
  const int sc_stride = TL ? TG : 1;
  // Zero-point bit of block b: col_zb0 + b * zb_stride.
  const int col_zb0 = TL ? (cg * kb * TG + ci) * BITS : ncol * zp_row_bytes * 8;
  const int zb_stride = TL ? TG * BITS : BITS;

  // Register stages.
  uint32_t cw[2][WPT];               // codes, two steps
  ST scr[2][2];                      // scales of the (at most 2) blocks of 32 codes
  uint32_t sc8[2][2];                // WF: their scale bytes
  uint32_t zbr[2][2];                // zero-point bytes of those blocks
  // GI = 2: every thread dequantizes: TPC threads per column, HKG codes
  // each (8 for 64-column tiles, 16 for 128), with their group indices.
  constexpr int TPC = GEMM_TPB / BN, HKG = GBK / TPC;
  constexpr int WG2 = (HKG * BITS + 31) / 32;    // code words (2-bit, 8 codes: a half word)
  constexpr int TSTRIDE = BN + 1;                // table row, in entries (see the prologue)
  const int gcol = tid / TPC, gk = (tid % TPC) * HKG;
  const bool gok = n0 + gcol < N;
  const int gcode0 = gok ? (n0 + gcol) * row_bytes + gk * BITS / 8 : 0;
  uint32_t cg2[GI == 2 ? 2 : 1][GI == 2 ? WG2 : 1];
  int gir[GI == 2 ? 2 : 1][GI == 2 ? HKG : 1];

  // The A tile goes from memory straight into LDS buffer buf (buffer loads
  // with the LDS flag, no registers, no LDS write instructions): load i of
  // wave w fills the 1 KiB of LDS rows 8 q .. 8 q + 7, q = 8 i + w, one
  // 16-byte piece per lane at offset 16 * lane.  The slot a lane fills is
  // fixed, so the lane fetches the piece lds_at places there: piece
  // (lane & 7) ^ f of row 8 q + lane / 8, where f, that row's XOR, depends only
  // on the wave's parity and the lane.
  const int a_rw = 8 * wave + (lane >> 3);
  const int a_k = ((lane & 7) ^ (((a_rw >> 1) & 7) ^ ((a_rw & 1) << 2))) * 8;
  auto load_a = [&](int k0, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 64 * i + a_rw, k = k0 + a_k;
      const bool ok = row < M && k < K;    // K % 8 == 0: a piece is all in or all out
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(As + buf * STAGE + (8 * i + wave) * 512),
          16, ok ? (row * K + k) * 2 : OOB, 0, 0, 0);
    }
  };
  // Codes past the row's last block (k0 + 64 > kb * bs) come from the next
  // row (or read zeros past the matrix); they meet zero activations
  // (k >= K), so they add nothing.
  auto load_b = [&](int k0, int st) {
    const int kt = k0 + khalf;
    const int byte0 = col_code0 + (k0 >> 6) * code_step;
    if constexpr (BITS == 3) {
      // Operator layout, blob of 3 bs / 8 bytes per block: the 2-bit plane
      // (bs / 4 bytes) then the 1-bit plane (bs / 8 bytes).  bs >= 32: this
      // thread's 32 codes are 8 bytes of the first plane and 4 of the second
      // of one block (4-aligned: blobs of 12 bytes or more); bs = 16: two
      // whole blocks, 12 contiguous bytes.  Past the row's last block the
      // bytes belong to the next row or lie past the matrix (zeros); they
      // meet zero activations.
      const int bsz = 1 << log2_bs;
      const int rb = ncol_ok ? ncol * row_bytes : 0;
      const int base = rb + (kt >> log2_bs) * (3 * bsz / 8);
      if (bsz >= 32) {
        const int i0 = kt & (bsz - 1);
        const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(rbc, ncol_ok ? base + i0 / 4 : OOB, 0, 0);
        cw[st][0] = lo.x;
        cw[st][1] = lo.y;
        cw[st][2] = __builtin_amdgcn_raw_buffer_load_b32(rbc, ncol_ok ? base + bsz / 4 + i0 / 8 : OOB,
                                                         0, 0);
      } else {
        // [lo0 4 B][hi0 2 B][lo1 4 B][hi1 2 B], 2-aligned only (rows of
        // 6 kb bytes): six 16-bit loads.
        uint32_t h[6];
#pragma unroll
        for (int i = 0; i < 6; ++i)
          h[i] = __builtin_amdgcn_raw_buffer_load_b16(rbc, ncol_ok ? base + 2 * i : OOB, 0, 0);
        cw[st][0] = h[0] | (h[1] << 16);
        cw[st][1] = h[3] | (h[4] << 16);
        cw[st][2] = h[2] | (h[5] << 16);
      }
    } else if constexpr (GI == 2) {
      // This thread's HKG codes and their group indices (the codes of a
      // column are contiguous, so adjacent threads read adjacent bytes).
      const int kg = k0 + gk;
#pragma unroll
      for (int i = 0; i < HKG; i += 4) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rgi, (kg + i) * 4, 0, 0);
        gir[st][i] = (int)t.x; gir[st][i + 1] = (int)t.y; gir[st][i + 2] = (int)t.z; gir[st][i + 3] = (int)t.w;
      }
      const int cb = gok ? gcode0 + (k0 >> 6) * CHUNK_BYTES : OOB;
      if constexpr (HKG * BITS == 16) {
        cg2[st][0] = __builtin_amdgcn_raw_buffer_load_b16(rbc, cb, 0, 0);
      } else if constexpr (HKG * BITS == 32) {
        cg2[st][0] = __builtin_amdgcn_raw_buffer_load_b32(rbc, cb, 0, 0);
      } else if constexpr (HKG * BITS == 64) {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rbc, cb, 0, 0);
        cg2[st][0] = t.x; cg2[st][1] = t.y;
      } else {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rbc, cb, 0, 0);
        cg2[st][0] = t.x; cg2[st][1] = t.y; cg2[st][2] = t.z; cg2[st][3] = t.w;
      }
      return;
    } else if constexpr (GI) {
      // Codes only; the scales and zero points are looked up per code when
      // the step is dequantized.
      if constexpr (WPT >= 4) {
#pragma unroll
        for (int w = 0; w < WPT; w += 4) {
          const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rbc, byte0 + 4 * w, 0, 0);
          cw[st][w] = t.x; cw[st][w + 1] = t.y; cw[st][w + 2] = t.z; cw[st][w + 3] = t.w;
        }
      } else {
        const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rbc, byte0, 0, 0);
        cw[st][0] = t.x; cw[st][1] = t.y;
      }
      return;
    } else if constexpr (WPT >= 4) {
#pragma unroll
      for (int w = 0; w < WPT; w += 4) {
        const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rbc, byte0 + 4 * w, 0, 0);
        cw[st][w] = t.x; cw[st][w + 1] = t.y; cw[st][w + 2] = t.z; cw[st][w + 3] = t.w;
      }
    } else {
      const u32x2 t = __builtin_amdgcn_raw_buffer_load_b64(rbc, byte0, 0, 0);
      cw[st][0] = t.x; cw[st][1] = t.y;
    }
    const int blk0 = kt >> log2_bs;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int b = min(blk0 + i, kb - 1);
      const int si = col_sc0 + b * sc_stride;
      if constexpr (WF)
        sc8[st][i] = __builtin_amdgcn_raw_buffer_load_b8(rsc, si, 0, 0);
      else if constexpr (sizeof(ST) == 4)
        scr[st][i] = __builtin_bit_cast(ST, __builtin_amdgcn_raw_buffer_load_b32(rsc, si * 4, 0, 0));
      else
        scr[st][i] = __builtin_bit_cast(ST, __builtin_amdgcn_raw_buffer_load_b16(rsc, si * 2, 0, 0));
      if constexpr (HAS_ZP) {
        const int zo = ncol_ok ? (col_zb0 + b * zb_stride) >> 3 : OOB;
        zbr[st][i] = __builtin_amdgcn_raw_buffer_load_b8(rzp, zo, 0, 0);
        // A 3-bit zero point may continue into the next byte (read past the
        // zero-point rows as zero).
        if constexpr (BITS == 3)
          zbr[st][i] |= __builtin_amdgcn_raw_buffer_load_b8(rzp, ncol_ok ? zo + 1 : OOB, 0, 0) << 8;
      }
    }
  };
  // Dequantize register stage `st` (step starting at k0) into LDS buffer buf.
  auto store_b = [&](int k0, int st, int buf) {
    uint16_t* bs = Bs + buf * BSTRIDE;
    if constexpr (GI == 2) {
      // Per code: its group (past K: group 0, meeting zero activations),
      // then this column's table entry {s, z * s} of that group.
      constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
      constexpr int PW = 32 / BITS;
      const f32x2* tab = reinterpret_cast<const f32x2*>(gslab) + gcol;
      uint32_t pk[HKG / 2];
#pragma unroll
      for (int j = 0; j < HKG; j += 2) {
        float w2[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int i = j + t;
          const f32x2 e = tab[min(max(gir[st][i], 0), kb - 1) * TSTRIDE];
          const float q = (float)((cg2[st][i / PW] >> ((i % PW) * BITS)) & zm);
          w2[t] = fmaf(q, e.x, -e.y);
        }
        pk[j / 2] = Op::pack(w2[0], w2[1]);
      }
#pragma unroll
      for (int j = 0; j < HKG / 8; ++j)
        *reinterpret_cast<u32x4*>(&bs[lds_at(gcol, (gk >> 3) + j)]) =
            u32x4{pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
      return;
    }
    if (!dq) return;
    const int kt = k0 + khalf;
    if constexpr (GI) {
      // Per code k = kt + i: g = g_idx[k] (zero past K, where the activations
      // are zero), then that group's scale and zero point of this column.
      // Eight codes at a time, fenced, so the lookups of one group are in
      // flight together without holding every group's registers.
      constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
      uint32_t pk[HK / 2];
#pragma unroll
      for (int c8 = 0; c8 < HK; c8 += 8) {
        float s[8], zsv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int g = min(max((int)__builtin_amdgcn_raw_buffer_load_b32(
                                    rgi, (kt + c8 + j) * 4, 0, 0), 0), kb - 1);
          const int si = col_sc0 + g;
          float sv;
          if constexpr (sizeof(ST) == 4)
            sv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsc, si * 4, 0, 0));
          else
            sv = dt<SDT>::to_f32(__builtin_bit_cast(
                ST, __builtin_amdgcn_raw_buffer_load_b16(rsc, si * 2, 0, 0)));
          uint32_t z = 1u << (BITS - 1);
          if constexpr (HAS_ZP) {
            const int bit = col_zb0 + g * BITS;
            z = (__builtin_amdgcn_raw_buffer_load_b8(rzp, ncol_ok ? bit >> 3 : OOB, 0, 0) >>
                 (bit & 7)) & zm;
          }
          s[j] = sv;
          zsv[j] = (float)z * sv;
        }
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int i0 = c8 + j, i1 = c8 + j + 1;
          const float q0 = (float)((cw[st][i0 / P] >> ((i0 % P) * BITS)) & zm);
          const float q1 = (float)((cw[st][i1 / P] >> ((i1 % P) * BITS)) & zm);
          pk[i0 / 2] = Op::pack(fmaf(q0, s[j], -zsv[j]), fmaf(q1, s[j + 1], -zsv[j + 1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int j = 0; j < HK / 8; ++j)
        *reinterpret_cast<u32x4*>(&bs[lds_at(bcol, (khalf >> 3) + j)]) =
            u32x4{pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
      return;
    }
    const int blk0 = min(kt >> log2_bs, kb - 1);
    float sf[2], zs[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (WF) {
        sf[i] = fp4_scale(sc8[st][i], WF - 1);
        zs[i] = 0.0f;
        continue;
      }
      sf[i] = dt<SDT>::to_f32(scr[st][i]);
      uint32_t z = 1u << (BITS - 1);
      if constexpr (HAS_ZP) {
        constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
        const int b = min(blk0 + i, kb - 1);
        z = (zbr[st][i] >> ((col_zb0 + b * zb_stride) & 7)) & zm;
      }
      zs[i] = (float)z * sf[i];
    }
    uint32_t pk[HK / 2];
    if constexpr (BITS == 3) {
      // Code j = 2-bit plane bits 2 (j % 16) of word j / 16, plus bit j of the
      // 1-bit plane times 4; codes 16..31 lie in the second block when bs = 16.
      const bool two = (1 << log2_bs) < HK;
#pragma unroll
      for (int j = 0; j < HK; j += 2) {
        const int bi = (two && j >= 16) ? 1 : 0;
        const float s = bi ? sf[1] : sf[0], z = bi ? zs[1] : zs[0];
        float q[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int jj = j + t;
          q[t] = (float)(((cw[st][jj / 16] >> (2 * (jj % 16))) & 3u) | (((cw[st][2] >> jj) & 1u) << 2));
        }
        pk[j / 2] = Op::pack(fmaf(q[0], s, -z), fmaf(q[1], s, -z));
      }
#pragma unroll
      for (int j = 0; j < HK / 8; ++j)
        *reinterpret_cast<u32x4*>(&bs[lds_at(bcol, (khalf >> 3) + j)]) =
            u32x4{pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
      return;
    }
    // (q - z) * s = q * s - z * s: for 16-bit scales both products are
    // exact and so is the difference; one rounding to the activation dtype.
    auto dequant_word = [&](int w, float s, float z) {
      float q[P];
      if constexpr (WF) {
        // Byte j of the word: E2M1 values of codes 2j (low nibble), 2j + 1.
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 c0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[st][w], 1.0f, 0);
        const f2 c1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[st][w], 1.0f, 1);
        const f2 c2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[st][w], 1.0f, 2);
        const f2 c3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[st][w], 1.0f, 3);
        q[0] = c0.x; q[1] = c0.y; q[2] = c1.x; q[3] = c1.y;
        q[4] = c2.x; q[5] = c2.y; q[6] = c3.x; q[7] = c3.y;
      } else {
        word_codes_f32<BITS>(cw[st][w], q);
      }
#pragma unroll
      for (int j = 0; j < P; j += 2) pk[(w * P + j) / 2] = Op::pack(fmaf(q[j], s, -z), fmaf(q[j + 1], s, -z));
    };
    // The thread's HK codes start on a block boundary (kt is a multiple of
    // HK, and bs >= 16 divides it or is a multiple of it).
    if ((1 << log2_bs) >= HK) {
      // All in one block.
#pragma unroll
      for (int w = 0; w < WPT; ++w) dequant_word(w, sf[0], zs[0]);
    } else {
      // bs = 16: word w lies in the second block when w * P >= bs.
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        const bool second = w * P >= (1 << log2_bs);
        dequant_word(w, second ? sf[1] : sf[0], second ? zs[1] : zs[0]);
      }
    }
#pragma unroll
    for (int j = 0; j < HK / 8; ++j)
      *reinterpret_cast<u32x4*>(&bs[lds_at(bcol, (khalf >> 3) + j)]) =
          u32x4{pk[4 * j], pk[4 * j + 1], pk[4 * j + 2], pk[4 * j + 3]};
  };

  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int fr = lane & 15, fk = (lane >> 4) * 8;
  auto mfma_step = [&](int buf) {
    const uint16_t* as = As + buf * STAGE;
    const uint16_t* bs = Bs + buf * BSTRIDE;
#pragma unroll
    for (int kk = 0; kk < GBK; kk += 32) {
      typename Op::V af[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = __builtin_bit_cast(typename Op::V,
                                   *reinterpret_cast<const u32x4*>(&as[lds_at(wm + i * 16 + fr, (kk + fk) >> 3)]));
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const typename Op::V bf = __builtin_bit_cast(
            typename Op::V, *reinterpret_cast<const u32x4*>(&bs[lds_at(wn + j * 16 + fr, (kk + fk) >> 3)]));
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = Op::run(af[i], bf, acc[i][j]);
      }
    }
  };
  // One pipelined step s (register stage and LDS buffer = s & 1 = ST).
  // Waves are placed on the four SIMDs round robin, so waves w and w + 4
  // share one.  The first four run a step's MFMAs before the next step's
  // dequantization, the other four after it, so on each SIMD one wave's
  // vector work overlaps the other's matrix work (measured: 0.298 -> 0.280 ms
  // on the tiled layout; pairing odd with even waves instead gives 0.286).
  // The next A tile is loaded into the other LDS buffer at the start of the
  // step; the barrier at its end waits for those loads.
  auto step = [&](int s, auto st_tag, auto deq_first) {
    constexpr int ST_ = decltype(st_tag)::value;
    load_a((s + 1) * GBK, ST_ ^ 1);
    load_b((s + 2) * GBK, ST_);
    if constexpr (decltype(deq_first)::value) {
      store_b((s + 1) * GBK, ST_ ^ 1, ST_ ^ 1);
      mfma_step(ST_);
    } else {
      mfma_step(ST_);
      store_b((s + 1) * GBK, ST_ ^ 1, ST_ ^ 1);
    }
    __syncthreads();
  };

  const int nsteps = (K + GBK - 1) / GBK;
  load_a(0, 0);
  load_b(0, 0);
  load_b(GBK, 1);
  if constexpr (GI == 2) {
    // Table of the tile's BN columns, entry (g, c) at g * (BN + 1) + c: the
    // scale of group g of column n0 + c and its product with the zero point,
    // both in fp32 (the product rounded as the other paths round it).  Lanes
    // take adjacent columns, so the table is written without bank conflicts;
    // a wave reads it at BN / TPC adjacent columns times TPC groups, which
    // the odd row length spreads over the banks.  Past N the loads read
    // zeros.
    constexpr int GPP = GEMM_TPB / BN;         // groups per pass
    constexpr uint32_t zm = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
    const int c = tid % BN;
    const int sc0 = (n0 + c) * kb, zr0 = (n0 + c) * zp_row_bytes;
    f32x2* tab = reinterpret_cast<f32x2*>(gslab);
    for (int gb = tid / BN; gb < kb; gb += 8 * GPP) {
      uint32_t sv[8], zv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int g = gb + u * GPP;
        const bool ok = g < kb;
        if constexpr (sizeof(ST) == 4)
          sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rsc, ok ? (sc0 + g) * 4 : OOB, 0, 0);
        else
          sv[u] = __builtin_amdgcn_raw_buffer_load_b16(rsc, ok ? (sc0 + g) * 2 : OOB, 0, 0);
        zv[u] = HAS_ZP ? __builtin_amdgcn_raw_buffer_load_b8(rzp, ok ? zr0 + ((g * BITS) >> 3) : OOB, 0, 0)
                       : 0u;
      }
      // Unconditional stores (groups past kb go to the spare row kb), so
      // that the loads above stay ahead of every use instead of being sunk
      // into a branch per group.
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int g = gb + u * GPP;
        float sf;
        if constexpr (sizeof(ST) == 4) sf = __builtin_bit_cast(float, sv[u]);
        else sf = dt<SDT>::to_f32(__builtin_bit_cast(ST, (uint16_t)sv[u]));
        const uint32_t z = HAS_ZP ? (zv[u] >> ((g * BITS) & 7)) & zm : 1u << (BITS - 1);
        tab[min(g, kb) * TSTRIDE + c] = f32x2{sf, (float)z * sf};
      }
    }
    __syncthreads();
  }
  store_b(0, 0, 0);
  __syncthreads();
  // The two orders are two copies of the loop (one wave-uniform branch
  // outside it), so each loop body stays one straight block.
  if (wave >= 4) {
    for (int s = 0; s < nsteps; s += 2) {
      step(s, std::integral_constant<int, 0>{}, std::true_type{});
      if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{}, std::true_type{});
    }
  } else {
    for (int s = 0; s < nsteps; s += 2) {
      step(s, std::integral_constant<int, 0>{}, std::false_type{});
      if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
  }

  // Epilogue: lane l holds rows 4 * (l / 16) + [0, 4) of column l % 16 of
  // each 16 x 16 tile.
  const int cc = lane & 15, rr = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int n = n0 + wn + j * 16 + cc;
    if (n >= N) continue;
    const float bv = bias ? bits16_to_f32<XDT>(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm + i * 16 + rr + e;
        if (m < M) Y[(int64_t)m * N + n] = Op::round((WF ? acc[i][j][e] * gscale : acc[i][j][e]) + bv);
      }
    }
  }
}

inline int ilog2i(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

// Group indices with a staged table (GI = 2): LDS bytes of the table of a
// BN-column workgroup, 8 bytes per group and column (rows of BN + 1; one
// spare row).
inline size_t gidx_table_bytes(const MatArgs& a, int bn) { return (size_t)(a.kb + 1) * (bn + 1) * 8; }

// The staged group-index kernel (GI = 2) with 64-column (tn = 2) or
// 128-column (tn = 4) tiles (gidx_mfma.hip).
hipError_t launch_gidx_staged(const MatArgs& a, int tiles_m, int tn);

// LDS available to one workgroup.
constexpr size_t LDS_MAX = 160 * 1024;

// Workgroups that fill the chip once (one per compute unit).
constexpr int GEMM_FULL_ROUND = 256;

// The kernel with 64-column (tn = 2) or 128-column (tn = 4) tiles, M tiles
// tiles_m (gemm_narrow.hip).
hipError_t launch_gemm_narrow(const MatArgs& a, int tiles_m, int tn);

template <int BITS, int XDT, int SDT, bool HAS_ZP, int TN>
hipError_t launch_mfma_tn(const MatArgs& a, int tiles_m) {
  using ST = typename dt<SDT>::T;
  constexpr int BN = 32 * TN;
  const int tiles_n = (int)((a.N + BN - 1) / BN);
  constexpr size_t lds = mfma_lds_bytes<BN>();   // double-buffered A and B
  decltype(&gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, TN, false>) kern;
  if constexpr (BITS == 3) kern = gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, TN, false>;
  else kern = a.tiled ? gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, TN, true>
                      : gemm_mfma_kernel<BITS, XDT, SDT, HAS_ZP, TN, false>;
  const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(GEMM_TPB), lds, a.stream,
                     (const uint16_t*)a.A, a.B, (const ST*)a.scales, a.zp,
                     (const uint16_t*)a.bias, (uint16_t*)a.Y, (int)a.M, (int)a.K, (int)a.N,
                     (int)a.kb, ilog2i(a.block_size), ilog2i(a.blob), (int)a.zp_row_bytes,
                     tiles_m, (int)a.chunks, (const int32_t*)nullptr, 1.0f);
  return hipGetLastError();
}

}  // namespace qmm
