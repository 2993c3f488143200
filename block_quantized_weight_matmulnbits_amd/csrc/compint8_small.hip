// compint8_small.hip -- CompInt8 (accuracy_level 4) for one activation row
// (M = 1, decode) on the tiled weight layout (qmm_layout.h), for gfx950.  The
// kernel is written for MR <= 4 rows; it is used for M = 1 only, since from
// two rows on the int8 matrix-core kernel (compint8_tiled.hip) after a
// separate quantization launch is faster (measured at K = 4096, N = 14336,
// M = 4: 17.5 vs 14.2 us for 4-bit weights).
//
// Definition (onnx-runtime-ep-cpu matmul_nbits.rs: quantize_activation_signed,
// int4_dot_row_scalar, int8_row): per row m and block b of block_size
// activations, sa = max|x| / 127 and qa = clamp(rne(x / sa), -127, 127)
// (0 past K, and for a block whose max is 0); then
//   dot[m, n, b] = sum_{k in b} qa[m, k] * (code(n, k) - zp(n, b))   (int32)
//   y[m, n]      = sum_b float(dot) * (sa[m, b] * scale[n, b]) (+ bias[n]).
//
// One launch does both steps.  Each workgroup quantizes all M rows of the
// activations into LDS (the same binary32 division and round-half-even as
// quantize_a_kernel; a block's maximum is combined across the lanes that
// hold it), then streams its weight columns as the tiled GEMV does: a wave
// owns an octet of 8 columns and a share of K, each lane loads 16 bytes of
// one column's codes per wave load (a unit of E = 128 / bits codes, inside
// one block since block_size >= E), four loads in flight.
//
// The block dots are exact int32: the codes of a 32-bit word are split into
// byte planes (4-bit: even / odd codes, 2-bit: four crumb planes, 8-bit:
// code - 128 by xor), the activations were stored in LDS permuted into the
// same plane order, v_dot4_i32_i8 multiplies four pairs at a time, and the
// zero point is removed per unit with the unit's sum of activations:
//   sum qa * (code - zp) = sum qa * code' - (zp - off) * sum qa
// (off = 128 for 8-bit codes, else 0).  The units of one block are added in
// int32 before any scaling, so the block dot of the definition exists as an
// exact integer: a load holds 8 units of each column (lane bits for the unit
// within the chunk and for the chunk), the units of a block are combined by
// integer lane exchanges over those bits, and a block wider than one load
// (8 units) carries its int32 sum from load to load.  The block's leading
// lane then adds float(dot) * (sa * scale) once.  A share of K per wave is a
// whole number of blocks, so no block is split between waves.  The DOTS
// variant writes the int32 block dots and, from workgroup 0, the quantized
// activations and scales it computed in LDS.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

#include <algorithm>

namespace qmm {

namespace {

constexpr int CS_OCT = 8;          // columns per wave
constexpr int CS_D = 4;            // wave loads in flight
constexpr int CS_MAXW = 16;
constexpr int CS_RSRC3 = 0x00020000;
constexpr int CS_OOB = 0x7FFFFFF0;
constexpr int CS_LDS_MAX = 64 * 1024;

template <int BITS>
struct CsGeom {
  static constexpr int P = 32 / BITS;          // codes per 32-bit word
  static constexpr int E = 4 * P;              // codes per 16-byte unit
  static constexpr int CB = TKC * BITS / 8;    // bytes per column chunk
  static constexpr int UPC = CB / 16;          // units per column chunk
  static constexpr int LPC = CS_OCT * UPC;     // lanes per chunk in a wave load
  static constexpr int CPL = 64 / LPC;         // chunks per wave load
  static constexpr int PPU = E / 16;           // 16-activation pieces per unit
  static_assert(CPL * TG * CB == 4096, "a wave load steps 4096 bytes through the codes");
};

// LDS regions, in bytes: qa [MR][RS] int8 (permuted pieces), the unit sums
// [MR][RS / E] int32, sa [MR][kb] f32, the share partial sums [W][8][MR].
// RS = Kc + 64 * CPL: reads of masked loads past the last chunk stay inside.
struct CsLds {
  int rs, qa_bytes, sq_off, sa_off, red_off, total;
};
template <int BITS>
__host__ __device__ inline CsLds cs_lds(int Kc, int kb, int MR, int W) {
  using G = CsGeom<BITS>;
  CsLds L;
  L.rs = Kc + 64 * G::CPL;
  L.qa_bytes = MR * L.rs;
  L.sq_off = (L.qa_bytes + 15) / 16 * 16;
  L.sa_off = L.sq_off + MR * (L.rs / G::E) * 4;
  L.red_off = L.sa_off + MR * kb * 4;
  L.total = L.red_off + W * CS_OCT * MR * 4;
  return L;
}

// Activation x[r, k] widened to fp32 (k < K), else 0.
template <int XDT>
__device__ __forceinline__ float cs_x(const void* x, int r, int K, int k) {
  if (k >= K) return 0.0f;
  return dt<XDT>::to_f32(reinterpret_cast<const typename dt<XDT>::T*>(x)[(int64_t)r * K + k]);
}

// Sixteen activations of row r from k0 (a multiple of 16) as fp32, zero past
// K.  vec: 16-bit activations, K % 8 == 0 and a 16-byte aligned base, so each
// 8-value half is wholly inside or wholly past the row.
template <int XDT>
__device__ __forceinline__ void cs_load16(const void* x, __amdgpu_buffer_rsrc_t rx, bool vec,
                                          int r, int K, int k0, float (&v)[16]) {
  if constexpr (XDT != DT_F32) {
    if (vec) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = k0 + 8 * h;
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            rx, k < K ? (r * K + k) * 2 : CS_OOB, 0, 0);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * h + 2 * i] = bits16_to_f32<XDT>((uint16_t)(ws[i] & 0xFFFFu));
          v[8 * h + 2 * i + 1] = bits16_to_f32<XDT>((uint16_t)(ws[i] >> 16));
        }
      }
      return;
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) v[j] = cs_x<XDT>(x, r, K, k0 + j);
}

// The 16 quantized activations of a piece (natural order) as four dwords in
// the byte-plane order of the codes they meet (see cs_planes).
template <int BITS>
__device__ __forceinline__ u32x4 cs_permute(const int (&q)[16]) {
  auto b = [&](int j) { return (uint32_t)(q[j] & 0xFF); };
  auto dw = [&](int a0, int a1, int a2, int a3) {
    return b(a0) | (b(a1) << 8) | (b(a2) << 16) | (b(a3) << 24);
  };
  if constexpr (BITS == 4) {
    // Two code words of 8 codes: plane 0 = codes 0, 2, 4, 6; plane 1 = 1, 3, 5, 7.
    return u32x4{dw(0, 2, 4, 6), dw(1, 3, 5, 7), dw(8, 10, 12, 14), dw(9, 11, 13, 15)};
  } else if constexpr (BITS == 2) {
    // One code word of 16 codes: plane i = codes i, 4 + i, 8 + i, 12 + i.
    return u32x4{dw(0, 4, 8, 12), dw(1, 5, 9, 13), dw(2, 6, 10, 14), dw(3, 7, 11, 15)};
  } else {
    return u32x4{dw(0, 1, 2, 3), dw(4, 5, 6, 7), dw(8, 9, 10, 11), dw(12, 13, 14, 15)};
  }
}

// The signed-byte planes of code word w, in the order of cs_permute:
// 4-bit: [even codes, odd codes]; 2-bit: the four crumb planes; 8-bit: code - 128.
template <int BITS>
__device__ __forceinline__ void cs_planes(uint32_t w, int* out) {
  if constexpr (BITS == 4) {
    out[0] = (int)(w & 0x0F0F0F0Fu);
    out[1] = (int)((w >> 4) & 0x0F0F0F0Fu);
  } else if constexpr (BITS == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = (int)((w >> (2 * i)) & 0x03030303u);
  } else {
    out[0] = (int)(w ^ 0x80808080u);
  }
}

// v from the lane whose index differs from this lane's in bit mask MASK (an
// integer exchange: DPP within a quad, a swizzle within 32 lanes, a
// permute across the halves of the wave).
template <int MASK>
__device__ __forceinline__ int cs_xor(int v) {
  if constexpr (MASK == 1) return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);
  else if constexpr (MASK == 2) return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);
  else if constexpr (MASK < 32) return __builtin_amdgcn_ds_swizzle(v, 0x1F | (MASK << 10));
  else return __shfl_xor(v, MASK);
}

// Lane-index bit that holds bit i of a lane's unit index q = chunk * UPC + u
// within its column's 8 units of a load: the unit bits are the lowest lane
// bits, the chunk bits sit above the 8 columns' lanes.
template <int LOG_UPC>
constexpr int cs_unit_bit_mask(int i) { return i < LOG_UPC ? (1 << i) : (1 << (i + 3)); }

template <int BITS, bool HAS_ZP, int MR, int XDT, bool DOTS>
__global__ __launch_bounds__(CS_MAXW * 64) void compint8_small_kernel(
    const void* __restrict__ x, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zps,
    const void* __restrict__ bias, void* __restrict__ Y, int Mp, int K, int N, int kb,
    int chunks, int log2_bs, int n_oct, int O, int S, int s_dtype,
    int32_t* __restrict__ dots, int8_t* __restrict__ qa_out, float* __restrict__ sa_out) {
  using G = CsGeom<BITS>;
  constexpr int P = G::P, E = G::E, CB = G::CB, UPC = G::UPC, LPC = G::LPC, CPL = G::CPL,
                PPU = G::PPU;
  constexpr int LOG_UPC = UPC == 1 ? 0 : (UPC == 2 ? 1 : 2);
  static_assert(CPL * UPC == 8, "a wave load holds 8 units of each of its 8 columns");
  constexpr uint32_t zmask = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  constexpr int OFF = (BITS == 8) ? 128 : 0;
  constexpr int NPL = (BITS == 4) ? 2 : (BITS == 2 ? 4 : 1);   // planes per code word

  extern __shared__ u32x4 smem_cs[];
  const int W = O * S;
  const int Kc = chunks * TKC;
  const CsLds L = cs_lds<BITS>(Kc, kb, MR, W);
  uint8_t* lds = reinterpret_cast<uint8_t*>(smem_cs);
  int8_t* qa = reinterpret_cast<int8_t*>(lds);
  int* sq = reinterpret_cast<int*>(lds + L.sq_off);
  float* sa = reinterpret_cast<float*>(lds + L.sa_off);
  float* red = reinterpret_cast<float*>(lds + L.red_off);
  const int su = L.rs / E;                           // unit sums per row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ol = wave % O, s = wave / O;
  const int oct = blockIdx.x * O + ol;
  const bool has_oct = oct < n_oct;
  const int g = oct >> 2;
  const int cl = lane / LPC;
  const int rem = lane % LPC;
  const int col = rem / UPC;
  const int u = rem % UPC;
  const int gcol = (oct & 3) * CS_OCT + col;
  const int n = g * TG + gcol;
  const int SZ = s_dtype == DT_F32 ? 4 : 2;

  const int groups = (N + TG - 1) / TG;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)codes, 0, groups * chunks * TG * CB, CS_RSRC3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, groups * kb * TG * SZ, CS_RSRC3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)zps, 0, HAS_ZP ? groups * kb * TG * BITS / 8 : 0, CS_RSRC3);
  constexpr int XB = (XDT == DT_F32) ? 4 : 2;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, Mp * K * XB, CS_RSRC3);
  const bool x_vec = XDT != DT_F32 && (K % 8) == 0 && (((uintptr_t)x) & 15) == 0;

  // Units of a block in one load (log2, at most 8 units = 3) and whether a
  // block spans several loads.
  const int log2_ub = log2_bs - __builtin_ctz(E);   // block_size >= E
  const int log2_rb = min(log2_ub, 3);
  const bool multi_load = log2_ub > 3;
  // This wave's share of the chunks: whole wave loads and whole blocks.
  const int share_step = max(CPL, (1 << log2_bs) / TKC);
  const int cs = (chunks + S * share_step - 1) / (S * share_step) * share_step;
  const int c_lo = s * cs;
  const int c_hi = has_oct ? min(chunks, c_lo + cs) : c_lo;
  const int nloads = c_hi > c_lo ? (c_hi - c_lo + CPL - 1) / CPL : 0;
  const int lane_code = ((g * chunks + c_lo + cl) * TG + gcol) * CB + u * 16;
  const int lane_k = (c_lo + cl) * TKC + u * E;       // first code of the lane's unit, load 0

  struct Slot { u32x4 cw; uint32_t sw, zw; };
  auto issue = [&](Slot& sl, int j) {
    sl.cw = __builtin_amdgcn_raw_buffer_load_b128(rc, lane_code + 4096 * j, 0, BUF_STREAM);
    const int b = min((lane_k + j * CPL * TKC) >> log2_bs, kb - 1);
    const int si = (g * kb + b) * TG + gcol;
    sl.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, (si * SZ) & ~3, 0, 0);
    if constexpr (HAS_ZP)
      sl.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, ((si * BITS) >> 5) * 4, 0, 0);
    else
      sl.zw = 0;
    __builtin_amdgcn_sched_barrier(0);
  };
  Slot sl[CS_D];
#pragma unroll
  for (int q = 0; q < CS_D; ++q) issue(sl[q], q);

  // Quantize the activations into LDS: one 16-activation piece per thread and
  // pass; the bs / 16 pieces of a block sit in consecutive, aligned lanes.
  {
    const int ppr = Kc / 16;                        // pieces per row
    const int total = Mp * ppr;
    const int bsp = (1 << log2_bs) / 16;            // pieces per block (<= 64)
    const int nthreads = W * 64;
    for (int p0 = 0; p0 < total; p0 += nthreads) {
      const int p = p0 + (int)threadIdx.x;
      const bool valid = p < total;
      const int r = valid ? p / ppr : 0;
      const int k0 = valid ? (p % ppr) * 16 : 0;
      float v[16];
      if (valid) cs_load16<XDT>(x, rx, x_vec, r, K, k0, v);
      else
#pragma unroll
        for (int j = 0; j < 16; ++j) v[j] = 0.0f;
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
      // Maximum over the block's pieces (exact: max is order independent);
      // every lane takes part, so the shuffles read defined values.
      for (int o = 1; o < bsp; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      const float scale = amax / 127.0f;            // IEEE binary32 division
      int q[16];
      int qs = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        int t = 0;
        if (scale != 0.0f) {
          float rr = rintf(v[j] / scale);           // IEEE division, ties to even
          rr = fminf(fmaxf(rr, -127.0f), 127.0f);
          t = (int)rr;
        }
        q[j] = t;
        qs += t;
      }
      // Sum over the unit's pieces (consecutive, aligned lanes).
      for (int o = 1; o < PPU; o <<= 1) qs += __shfl_xor(qs, o);
      if (valid) {
        *reinterpret_cast<u32x4*>(qa + r * L.rs + k0) = cs_permute<BITS>(q);
        if ((p % PPU) == 0) sq[r * su + k0 / E] = qs;
        // Pieces past the last block (the chunk padding of short blocks)
        // hold zeros and no scale.
        if ((p % bsp) == 0 && (k0 >> log2_bs) < kb) sa[r * kb + (k0 >> log2_bs)] = scale;
        if constexpr (DOTS) {
          // Workgroup 0 exports the quantization in natural order:
          // qa_out [Mp, kb * bs], sa_out [Mp, kb].
          const int kbbs = kb << log2_bs;
          if (blockIdx.x == 0 && k0 < kbbs) {
            *reinterpret_cast<u32x4*>(qa_out + r * kbbs + k0) = cs_permute<8>(q);
            if ((p % bsp) == 0) sa_out[r * kb + (k0 >> log2_bs)] = scale;
          }
        }
      }
    }
  }
  __syncthreads();

  float acc[MR];
  int dsum[MR];                  // int32 sum of the current block (multi-load blocks)
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    acc[r] = 0.0f;
    dsum[r] = 0;
  }
  // The lane that adds its block's scaled dot: unit 0 of the block in a load.
  const int q_unit = cl * UPC + u;
  const bool leader = (q_unit & ((1 << log2_rb) - 1)) == 0;

  // Load j: the lane's unit starts at k = lane_k + j * CPL * 64.
  auto compute = [&](const Slot& sl, int j, bool masked) {
    const int k = lane_k + j * CPL * TKC;
    const int b = min(k >> log2_bs, kb - 1);
    const int si = (g * kb + b) * TG + gcol;
    float sc;
    if (SZ == 4) sc = __uint_as_float(sl.sw);
    else {
      const uint16_t h = (uint16_t)(sl.sw >> ((si & 1) * 16));
      sc = s_dtype == DT_F16 ? bits16_to_f32<DT_F16>(h) : bits16_to_f32<DT_BF16>(h);
    }
    int z = 1 << (BITS - 1);
    if constexpr (HAS_ZP) z = (int)((sl.zw >> ((si * BITS) & 31)) & zmask);
    const int zo = z - OFF;
    int pl[4][NPL];
    const uint32_t cw[4] = {sl.cw.x, sl.cw.y, sl.cw.z, sl.cw.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) cs_planes<BITS>(cw[w], pl[w]);
    const int c = c_lo + j * CPL + cl;
    const bool live = !masked || (c < c_hi && (k >> log2_bs) < kb);
    // A multi-load block ends after this load at the next block boundary or
    // at the share's last load; other blocks end within the load.
    const bool flush = !multi_load || j == nloads - 1 ||
                       ((k + CPL * TKC) >> log2_bs) != (k >> log2_bs);
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      if (r >= Mp) break;
      // The unit's E activations: E / 16 pieces of four plane dwords.
      const u32x4* qv = reinterpret_cast<const u32x4*>(qa + r * L.rs + k);
      int d = 0;
#pragma unroll
      for (int pc = 0; pc < PPU; ++pc) {
        const u32x4 a4 = qv[pc];
        const int av[4] = {(int)a4.x, (int)a4.y, (int)a4.z, (int)a4.w};
        // Piece pc holds 16 / P code words' planes: word pc * 16 / P + i.
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int wd = (pc * 16 + t * 4) / P;     // code word of activation dword t
          const int pln = (BITS == 4) ? (t & 1) : (BITS == 2 ? t : 0);
          d = __builtin_amdgcn_sdot4(av[t], pl[wd][pln], d, false);
        }
      }
      d -= zo * sq[r * su + k / E];
      d = live ? d : 0;
      // Integer sum over the block's units of this load (the reduction
      // conditions are uniform across the wave).
      if (log2_rb > 0) d += cs_xor<cs_unit_bit_mask<LOG_UPC>(0)>(d);
      if (log2_rb > 1) d += cs_xor<cs_unit_bit_mask<LOG_UPC>(1)>(d);
      if (log2_rb > 2) d += cs_xor<cs_unit_bit_mask<LOG_UPC>(2)>(d);
      dsum[r] += d;
      if (flush) {
        const bool add = leader && live;
        const float t = fmaf((float)dsum[r], sa[r * kb + b] * sc, acc[r]);
        acc[r] = add ? t : acc[r];
        if constexpr (DOTS) {
          if (add && has_oct && n < N) dots[((int64_t)r * N + n) * kb + (k >> log2_bs)] = dsum[r];
        }
        dsum[r] = 0;
      }
    }
  };

  int j0 = 0;
  for (; j0 + CS_D < nloads; j0 += CS_D) {
#pragma unroll
    for (int q = 0; q < CS_D; ++q) {
      compute(sl[q], j0 + q, false);
      issue(sl[q], j0 + q + CS_D);
    }
  }
#pragma unroll
  for (int q = 0; q < CS_D; ++q)
    if (j0 + q < nloads) compute(sl[q], j0 + q, true);

  // Lanes of one column: the UPC units of a chunk, then the CPL chunks.
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    if constexpr (UPC >= 2) acc[r] += __shfl_xor(acc[r], 1);
    if constexpr (UPC >= 4) acc[r] += __shfl_xor(acc[r], 2);
#pragma unroll
    for (int st = LPC; st < 64; st *= 2) acc[r] += __shfl_xor(acc[r], st);
  }
  if constexpr (DOTS) return;
  const bool writer = lane < LPC && u == 0;
  if (writer)
#pragma unroll
    for (int r = 0; r < MR; ++r) red[(wave * CS_OCT + col) * MR + r] = acc[r];
  __syncthreads();
  if (s == 0 && writer && has_oct && n < N) {
    for (int r = 0; r < Mp; ++r) {
      float o = red[(ol * CS_OCT + col) * MR + r];
      for (int t = 1; t < S; ++t) o += red[((t * O + ol) * CS_OCT + col) * MR + r];
      using YT = typename dt<XDT>::T;
      if (bias) o += dt<XDT>::to_f32(reinterpret_cast<const YT*>(bias)[n]);
      reinterpret_cast<YT*>(Y)[(int64_t)r * N + n] = dt<XDT>::from_f32(o);
    }
  }
}

template <int BITS>
bool cs_fits(const MatArgs& a, int* O_out, int* S_out, size_t* lds_out) {
  using G = CsGeom<BITS>;
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  const int chunks = (int)tg.chunks;
  const int n_oct = (int)tg.groups * (TG / CS_OCT);
  // Octets per workgroup: one workgroup per compute unit where there are
  // enough octets; then shares of K until a workgroup has 8 waves.
  const int O = std::min(CS_MAXW, std::max(1, (n_oct + 255) / 256));
  int S = 1;
  while (O * S * 2 <= CS_MAXW && O * S < 8 && chunks >= 2 * (2 * S) * G::CPL) S *= 2;
  const int MR = 1;
  const CsLds L = cs_lds<BITS>(chunks * TKC, (int)a.kb, MR, O * S);
  if (O_out) *O_out = O;
  if (S_out) *S_out = S;
  if (lds_out) *lds_out = (size_t)L.total;
  // 32-bit buffer offsets: shares rounded up to whole blocks may start past
  // the last chunk (by at most 8 shares of 16 chunks), and loads run 4 ahead.
  return L.total <= CS_LDS_MAX && tg.total + (1 << 20) < 0x7FFFFF00LL;
}

template <int BITS, bool HAS_ZP, int MR, int XDT, bool DOTS>
hipError_t cs_launch(const MatArgs& a, int32_t* dots, int8_t* qa_out, float* sa_out) {
  int O = 1, S = 1;
  size_t lds = 0;
  cs_fits<BITS>(a, &O, &S, &lds);
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  const int n_oct = (int)tg.groups * (TG / CS_OCT);
  const int grid = (n_oct + O - 1) / O;
  hipLaunchKernelGGL((compint8_small_kernel<BITS, HAS_ZP, MR, XDT, DOTS>), dim3(grid),
                     dim3(O * S * 64), lds, a.stream, a.A, a.B + tg.codes_off,
                     (const uint8_t*)a.scales, a.zp, a.bias, a.Y, (int)a.M, (int)a.K, (int)a.N,
                     (int)a.kb, (int)tg.chunks, __builtin_ctz((unsigned)a.block_size), n_oct, O,
                     S, a.s_dtype, dots, qa_out, sa_out);
  return hipGetLastError();
}

template <int BITS, bool HAS_ZP, int MR, bool DOTS>
hipError_t cs_launch_x(const MatArgs& a, int32_t* dots, int8_t* qa_out, float* sa_out) {
  switch (a.a_dtype) {
    case DT_F32: return cs_launch<BITS, HAS_ZP, MR, DT_F32, DOTS>(a, dots, qa_out, sa_out);
    case DT_F16: return cs_launch<BITS, HAS_ZP, MR, DT_F16, DOTS>(a, dots, qa_out, sa_out);
    default: return cs_launch<BITS, HAS_ZP, MR, DT_BF16, DOTS>(a, dots, qa_out, sa_out);
  }
}

template <int BITS, bool DOTS>
hipError_t cs_launch_z(const MatArgs& a, int32_t* dots, int8_t* qa_out, float* sa_out) {
  return a.zp ? cs_launch_x<BITS, true, 1, DOTS>(a, dots, qa_out, sa_out)
              : cs_launch_x<BITS, false, 1, DOTS>(a, dots, qa_out, sa_out);
}

template <bool DOTS>
hipError_t cs_launch_b(const MatArgs& a, int32_t* dots, int8_t* qa_out, float* sa_out) {
  switch (a.bits) {
    case 2: return cs_launch_z<2, DOTS>(a, dots, qa_out, sa_out);
    case 4: return cs_launch_z<4, DOTS>(a, dots, qa_out, sa_out);
    default: return cs_launch_z<8, DOTS>(a, dots, qa_out, sa_out);
  }
}

}  // namespace

bool compint8_small_supported(const MatArgs& a) {
  // One row; a 16-byte unit of codes inside one block, and a block's pieces
  // within one wave (block_size <= 1024); LDS for the quantized row.
  const int E = 128 / a.bits;
  if (!a.tiled || a.M != 1 || a.block_size < E || a.block_size > 1024) return false;
  switch (a.bits) {
    case 2: return cs_fits<2>(a, nullptr, nullptr, nullptr);
    case 4: return cs_fits<4>(a, nullptr, nullptr, nullptr);
    default: return cs_fits<8>(a, nullptr, nullptr, nullptr);
  }
}

hipError_t launch_compint8_small(const MatArgs& a) {
  return cs_launch_b<false>(a, nullptr, nullptr, nullptr);
}

hipError_t launch_compint8_small_dots(const MatArgs& a, int8_t* qa, float* sa, int32_t* dots) {
  return cs_launch_b<true>(a, dots, qa, sa);
}

}  // namespace qmm
