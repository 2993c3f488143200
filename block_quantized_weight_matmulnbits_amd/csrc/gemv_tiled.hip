// gemv_tiled.hip -- M = 1 decode GEMV on the tiled weight layout (qmm_layout.h)
// for gfx950.
//
// Computes y[n] = sum_k x[k] * (code(n,k) - zp(n, k/bs)) * scale[n, k/bs]
// (+ bias[n]) (onnx-runtime-ep-cpu matmul_nbits.rs: module documentation and
// dequantize_nbits_value) from the buffer written by qmm_repack.
//
// Work split.  A wave owns an octet of 8 columns of one 32-column group and
// a contiguous share of K; a workgroup holds O octets times S shares of K
// (O * S waves), sized so that the grid covers the 256 compute units about
// once.  In the tiled layout the 8 columns' bytes of one 64-code chunk are
// contiguous (8 * 8 * BITS bytes), so one 16-byte-per-lane wave load reads
// 64 / (8 * BITS / 2) consecutive chunks in runs of 256 (4-bit) bytes; the
// byte offset of load j is a per-lane base plus 4096 * j.  Lane l keeps one
// column and one fp32 partial sum; lanes of a column are combined with
// cross-lane shuffles and the S shares of K through LDS.
//
// Activations are staged once per workgroup into LDS (pieces of at most
// 16384): as they are for f16 x; for bf16 x re-encoded exactly as fp16
// after a power-of-two shift per 16-byte unit of codes (the largest
// magnitude lands in [2^14, 2^15), so every value within 2^28 of it keeps
// all of its 8 significant bits).  A piece with inf/nan, bf16 subnormals or
// a wider dynamic range takes an exact fp32 path instead.
//
// Arithmetic.  A 16-bit half of a code word holds 16 / BITS codes at bit
// offsets 0, BITS, ...; the codes at offsets p <= 8 - BITS of the word and
// of the word shifted right by 8 are masked in place and OR-ed with fp16
// 1024.0 (one v_and_or_b32 per pair), giving 1024 + 2^p * code exactly.
// Adding the fp16 pair -(1024 + 2^p * zp) leaves 2^p * (code - zp) exactly,
// and v_dot2_f32_f16 multiplies that by two activations (exact products)
// and accumulates in fp32, one accumulator per p, scaled back by 2^-p at the
// end of each 16-byte unit.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

#include <algorithm>

namespace qmm {

namespace {

constexpr int OCT = 8;            // columns per wave
constexpr int PIECE_CHUNKS = 256; // 64-code chunks staged at once (16384 activations)
constexpr int RSRC_WORD3 = 0x00020000;
constexpr int MAX_WAVES = 16;

// Geometry of one code width.
template <int BITS>
struct TGeom {
  static constexpr int P = 32 / BITS;          // codes per 32-bit word
  static constexpr int E = 4 * P;              // codes per 16-byte unit
  static constexpr int CB = TKC * BITS / 8;    // bytes per column chunk
  static constexpr int UPC = CB / 16;          // units per column chunk
  static constexpr int LPC = OCT * UPC;        // lanes per chunk in a load
  static constexpr int CPL = 64 / LPC;         // chunks per wave load
  static constexpr int NPOS = 8 / BITS;        // bit offsets p per half word
  static constexpr int LPU = E / 16;           // staging lanes per unit
  static_assert(CPL * TG * CB == 4096, "a wave load steps 4096 bytes through the codes");
};

// One in-flight load of a wave: the lane's 16 bytes of codes and the aligned
// 32-bit words holding its scale and zero point.  Everything is loaded as
// whole 32-bit words so that no narrow value is carried around the pipeline
// loop (the compiler would widen it at the loop head, waiting for the load).
struct TSlot {
  u32x4 cw;
  uint32_t sw;
  uint32_t zw;
};

// 16 activations x[k, k + 16) as raw 16-bit values; positions past K read
// zero (buffer range checking).  vec: K % 8 == 0 and x 16-byte aligned, so a
// 16-byte load is wholly inside or wholly past the end.
__device__ __forceinline__ void load_x16(__amdgpu_buffer_rsrc_t rx, int k, bool vec,
                                         u32x4 (&raw)[2]) {
  if (vec) {
    raw[0] = __builtin_amdgcn_raw_buffer_load_b128(rx, k * 2, 0, 0);
    raw[1] = __builtin_amdgcn_raw_buffer_load_b128(rx, k * 2 + 16, 0, 0);
  } else {
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rx, (k + 2 * j) * 2, 0, 0);
      const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rx, (k + 2 * j + 1) * 2, 0, 0);
      w[j] = lo | (hi << 16);
    }
    raw[0] = u32x4{w[0], w[1], w[2], w[3]};
    raw[1] = u32x4{w[4], w[5], w[6], w[7]};
  }
}

// Staging of 16 activations (starting at a multiple of 16) into fp16 pairs:
// pair word w*P/2 + i of code word w holds activations (wP + i, wP + i + P/2).
// pw[unit] undoes the unit's shift.  Returns whether a unit is not exact.
// The LPU lanes of a unit are adjacent and all take part (whole units).
//
// bf16: the magnitude bits of a bf16 value order like the value, so the
// largest magnitude of the unit (packed 16-bit max) gives the largest
// exponent, and the smallest nonzero one (packed 16-bit min after
// subtracting 1, which sends zeros to 0xFFFF) the smallest.  Every value is
// then scaled by 2^sh (exact) and packed to fp16 with round-toward-zero,
// which is exact as well because the scaled values are fp16 normals with at
// most 8 significant bits.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

template <int BITS, int XDT>
__device__ __forceinline__ bool stage16(const u32x4 (&raw)[2], int a, uint32_t* __restrict__ xs,
                                        float* __restrict__ pw) {
  constexpr int P = 32 / BITS, E = 4 * P, LPU = E / 16;
  const uint32_t w[8] = {raw[0].x, raw[0].y, raw[0].z, raw[0].w,
                         raw[1].x, raw[1].y, raw[1].z, raw[1].w};
  bool bad = false;
  int sh = 0;
  uint32_t pairs[8];
  if constexpr (XDT == DT_BF16) {
    u16x2 mx = {0, 0}, mn = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const u16x2 m = __builtin_bit_cast(u16x2, w[j] & 0x7FFF7FFFu);
      mx = __builtin_elementwise_max(mx, m);
      mn = __builtin_elementwise_min(mn, m - u16x2{1, 1});
    }
    uint32_t umax = max((uint32_t)mx.x, (uint32_t)mx.y);
    uint32_t umin = min((uint32_t)mn.x, (uint32_t)mn.y);
    if constexpr (LPU >= 2) {
      umax = max(umax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)umax, 0xB1, 0xF, 0xF, false));
      umin = min(umin, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)umin, 0xB1, 0xF, 0xF, false));
    }
    if constexpr (LPU >= 4) {
      umax = max(umax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)umax, 0x4E, 0xF, 0xF, false));
      umin = min(umin, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)umin, 0x4E, 0xF, 0xF, false));
    }
    if (umax != 0) {
      const int emax = (int)(umax >> 7);          // 255: inf or nan
      const int emin = (int)((umin + 1) >> 7);    // 0: a subnormal
      bad = (emax == 255) || (emin == 0) || (emin < emax - 28);
      sh = 141 - emax;   // 14 - (emax - 127)
    }
    // Value j of the unit's 16 as fp32 (bf16 is the upper half of fp32).
    auto val = [&](int j) {
      const uint32_t u = w[j >> 1];
      return __uint_as_float((j & 1) ? (u & 0xFFFF0000u) : (u << 16));
    };
#pragma unroll
    for (int c = 0; c < 16 / P; ++c) {
#pragma unroll
      for (int i = 0; i < P / 2; ++i) {
        const float lo = ldexpf(val(c * P + i), sh);
        const float hi = ldexpf(val(c * P + i + P / 2), sh);
        pairs[c * (P / 2) + i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
      }
    }
  } else {
    // fp16 activations are used as they are; only inf / nan are not exact.
    // Pairs are regrouped with byte permutes.
#pragma unroll
    for (int j = 0; j < 8; ++j) bad |= ((w[j] & 0x7C00u) == 0x7C00u) || ((w[j] & 0x7C000000u) == 0x7C000000u);
    auto half_of = [&](int j) { return (w[j >> 1] >> ((j & 1) * 16)) & 0xFFFFu; };
#pragma unroll
    for (int c = 0; c < 16 / P; ++c)
#pragma unroll
      for (int i = 0; i < P / 2; ++i)
        pairs[c * (P / 2) + i] = half_of(c * P + i) | (half_of(c * P + i + P / 2) << 16);
  }
  u32x4* dst = reinterpret_cast<u32x4*>(xs + a / 2);
  dst[0] = u32x4{pairs[0], pairs[1], pairs[2], pairs[3]};
  dst[1] = u32x4{pairs[4], pairs[5], pairs[6], pairs[7]};
  if ((threadIdx.x % LPU) == 0) pw[a / E] = ldexpf(1.0f, -sh);
  return bad;
}

// a.lo * b.lo + a.hi * b.hi + 0 in fp32, as __builtin_amdgcn_fdot2(a, b, 0.0f,
// false); written as the three-operand form with an inline zero so that a
// chain's first product needs no register cleared beforehand.
__device__ __forceinline__ float dot2_first(half2_t a, half2_t b) {
  float d;
  asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// LDS layout, in 32-bit words, for a piece of pc chunks and S shares of D
// loads in flight: the fp16 pairs, the unit factors, then the S-share
// partial sums.  The first pc + CPL chunks are staged; the pairs and factors
// extend (S + D) * CPL chunks past pc so that every activation read of a
// load past the end of its share (whose result is discarded) stays inside
// the allocation: such reads reach at most chunk pn + (S + D) * CPL - 1.
template <int BITS>
struct TLds {
  int xs_words, pw_words, total;
  __host__ __device__ TLds(int pc, int O, int S, int D) {
    constexpr int CPL = TGeom<BITS>::CPL, E = TGeom<BITS>::E;
    const int span = pc + (S + D) * CPL;
    xs_words = span * 32;
    pw_words = (span * 64 / E + 3) / 4 * 4;
    total = xs_words + pw_words + O * S * OCT;
  }
};

// LINB: blocks no longer than one wave load (bs <= 64 * CPL), so the scale
// and zero-point offsets of load j are a per-lane base plus j times a step.
template <int BITS, int XDT, int SDT, bool HAS_ZP, int D, bool LINB>
__global__ __launch_bounds__(MAX_WAVES * 64) void gemv_tiled_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const uint8_t* __restrict__ scales, const uint8_t* __restrict__ zps,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int K, int N, int kb,
    int chunks, int log2_bs, int n_oct, int O, int S, int pc) {
  using G = TGeom<BITS>;
  using ST = typename dt<SDT>::T;
  constexpr int P = G::P, E = G::E, CB = G::CB, UPC = G::UPC, LPC = G::LPC, CPL = G::CPL;
  constexpr int SZ = (int)sizeof(ST);
  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);

  extern __shared__ u32x4 smem_tv[];
  const int W = O * S;
  const TLds<BITS> L(pc, O, S, D);
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_tv);
  float* pw = reinterpret_cast<float*>(xs + L.xs_words);
  float* red = pw + L.pw_words;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ol = wave % O, s = wave / O;             // octet in the workgroup, share of K
  const int oct = blockIdx.x * O + ol;
  const bool has_oct = oct < n_oct;
  const int g = oct >> 2;                            // group
  const int cl = lane / LPC;                         // chunk within a wave load
  const int rem = lane % LPC;
  const int col = rem / UPC;                         // column within the octet
  const int u = rem % UPC;                           // unit within the column chunk
  const int gcol = (oct & 3) * OCT + col;            // column within the group
  const int ue = cl * TKC + u * E;                   // unit start within a wave load

  const int groups = (N + TG - 1) / TG;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)codes, 0, groups * chunks * TG * CB, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, groups * kb * TG * SZ, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)zps, 0, HAS_ZP ? groups * kb * TG * BITS / 8 : 0, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, K * 2, RSRC_WORD3);
  const bool x_vec = (K % 8) == 0 && (((uintptr_t)x) & 15) == 0;

  // Block of a unit: chunk bases are multiples of CPL, so when a block spans
  // at most one wave load (bs <= 64 * CPL) the block is the base's block plus
  // a per-lane part, and otherwise the base's block alone.
  const int lane_db = (TKC * CPL >= (1 << log2_bs)) ? (ue >> log2_bs) : 0;
  const int lane_si = lane_db * TG + gcol;           // scale index minus the uniform part
  const int lane_soff = (lane_si * SZ) & ~3;
  const int lane_shalf = (SZ == 2) ? (lane_si & 1) * 16 : 0;
  const int lane_zoff = ((lane_si * BITS) >> 3) & ~3;
  const int lane_zbit = (lane_si * BITS) & 31;
  // fp16 1024.0 twice, held in a register the compiler cannot see through:
  // (code & mask) | magic then selects one v_and_or_b32 with the mask in a
  // scalar register (gfx9 VOP3 takes no literal constants, so with both
  // constants literal it would emit an AND and an OR).
  uint32_t magic;
  asm("v_mov_b32 %0, 0x64006400" : "=v"(magic));

  float acc = 0.0f;
  const int nthreads = W * 64;

  for (int P0 = 0; P0 < chunks; P0 += pc) {
    const int pn = min(pc, chunks - P0);
    // This wave's share of the piece: whole wave loads.
    const int cs = (pn + S * CPL - 1) / (S * CPL) * CPL;
    const int c_lo = P0 + s * cs;
    const int c_hi = has_oct ? min(P0 + pn, c_lo + cs) : c_lo;
    const int nloads = c_hi > c_lo ? (c_hi - c_lo + CPL - 1) / CPL : 0;
    const int lane_code = ((g * chunks + c_lo + cl) * TG + gcol) * CB + u * 16;
    const int lane_kr = (c_lo - P0) * TKC + ue;      // unit start within the staged piece

    // x of the first two staging passes, loaded before the weights: loads
    // return in order, so x loaded after them would wait for them.
    const int n_act = (pn + CPL) * TKC;              // with CPL chunks of padding
    const int a0 = threadIdx.x * 16, a1 = a0 + nthreads * 16;
    u32x4 xr0[2], xr1[2];
    load_x16(rx, P0 * TKC + a0, x_vec, xr0);
    load_x16(rx, P0 * TKC + a1, x_vec, xr1);

    // Uniform scale-index base of load 0 and, for LINB, the step per load.
    const int ub0 = (g * kb + ((c_lo * TKC) >> log2_bs)) * TG;
    const int ubs = ((CPL * TKC) >> log2_bs) * TG;
    auto issue = [&](TSlot& sl, int j) {
      sl.cw = __builtin_amdgcn_raw_buffer_load_b128(rc, lane_code + 4096 * j, 0, BUF_STREAM);
      const int ub = LINB ? ub0 + j * ubs
                          : (g * kb + (((c_lo + j * CPL) * TKC) >> log2_bs)) * TG;
      sl.sw = __builtin_amdgcn_raw_buffer_load_b32(rs, ub * SZ + lane_soff, 0, 0);
      if constexpr (HAS_ZP)
        sl.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, ub * BITS / 8 + lane_zoff, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    };
    TSlot sl[D];
#pragma unroll
    for (int q = 0; q < D; ++q) issue(sl[q], q);

    // Stage the piece (all waves), then agree on the path.
    bool bad = false;
    if (a0 < n_act) bad |= stage16<BITS, XDT>(xr0, a0, xs, pw);
    if (a1 < n_act) bad |= stage16<BITS, XDT>(xr1, a1, xs, pw);
    for (int a = a1 + nthreads * 16; a < n_act; a += nthreads * 16) {
      u32x4 raw[2];
      load_x16(rx, P0 * TKC + a, x_vec, raw);
      bad |= stage16<BITS, XDT>(raw, a, xs, pw);
    }
    const bool exact = __syncthreads_or(bad) != 0;

    if (!exact) {
      // The activations of load j (read from LDS one load ahead of their use,
      // so that the LDS latency hides behind the previous load's arithmetic).
      // Loads past the share read the padding past the staged piece.
      struct XV { uint32_t w[E / 2]; float f; };
      // This lane's unit in the staged piece (lane_kr is a multiple of E);
      // load j reads CPL chunks further on.
      const u32x4* x_lane = reinterpret_cast<const u32x4*>(xs) + lane_kr / 8;
      const float* pw_lane = pw + lane_kr / E;
      auto fetch = [&](XV& xv, int j) {
        const u32x4* p = x_lane + j * (CPL * TKC / 8);
#pragma unroll
        for (int t = 0; t < E / 8; ++t) {
          const u32x4 v = p[t];
          xv.w[4 * t + 0] = v.x; xv.w[4 * t + 1] = v.y; xv.w[4 * t + 2] = v.z; xv.w[4 * t + 3] = v.w;
        }
        xv.f = pw_lane[j * (CPL * TKC / E)];
      };
      // acc += scale * (codes . activations) for load j from slot sl.
      // masked: the load may hold lanes past the share or past the blocks.
      auto compute = [&](const TSlot& sl, const XV& xv, int j, bool masked) {
        uint32_t z = 1u << (BITS - 1);
        if constexpr (HAS_ZP) z = (sl.zw >> lane_zbit) & m;
        float sc;
        if constexpr (SZ == 4) sc = __uint_as_float(sl.sw);
        else sc = bits16_to_f32<SDT>((uint16_t)(sl.sw >> lane_shalf));
        float dp[G::NPOS];
        half2_t nz[G::NPOS];
#pragma unroll
        for (int pi = 0; pi < G::NPOS; ++pi) {
          const uint32_t h = 0xE400u | (z << (pi * BITS));   // -(1024 + 2^p z)
          nz[pi] = as_half2(h | (h << 16));
        }
        const uint32_t cw[4] = {sl.cw.x, sl.cw.y, sl.cw.z, sl.cw.w};
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const uint32_t src = hf ? (cw[wi] >> 8) : cw[wi];
#pragma unroll
            for (int pi = 0; pi < G::NPOS; ++pi) {
              const int p = pi * BITS;
              const uint32_t mask = (m << p) | (m << (p + 16));
              const half2_t cv = as_half2((src & mask) | magic) + nz[pi];
              const int ci = (hf * 8 + p) / BITS;            // code index in the word
              const half2_t xh = as_half2(xv.w[wi * (P / 2) + ci]);
              if (wi == 0 && hf == 0)
                dp[pi] = dot2_first(cv, xh);
              else
                dp[pi] = __builtin_amdgcn_fdot2(cv, xh, dp[pi], false);
            }
          }
        }
        float d = dp[0];
#pragma unroll
        for (int pi = 1; pi < G::NPOS; ++pi) d = fmaf(dp[pi], ldexpf(1.0f, -pi * BITS), d);
        const float t = fmaf(d, xv.f * sc, acc);
        if (masked) {
          const int c = c_lo + j * CPL + cl;
          const int b = (((c_lo + j * CPL) * TKC) >> log2_bs) + lane_db;
          acc = (c < c_hi && b < kb) ? t : acc;
        } else {
          acc = t;
        }
      };
      // Steady state: each consumed slot is refilled with the load D ahead.
      // Only the last load of a share can hold dead lanes, and it is always
      // among the last D, which are consumed masked and without refills (a
      // dead load would still cost an address-unit pass).
      // 2-bit units hold 64 activations: without the look-ahead, to stay
      // within 128 registers.
      constexpr bool AHEAD = BITS != 2;
      // The look-ahead alternates two activation buffers by the parity of q,
      // which restarts at every D loads: D must be even.
      static_assert(!AHEAD || D % 2 == 0, "the activation look-ahead needs an even D");
      XV xa, xb;
      if constexpr (AHEAD) fetch(xa, 0);
      int j0 = 0;
      for (; j0 + D < nloads; j0 += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
          XV& cur = (q & 1) ? xb : xa;
          XV& nxt = (q & 1) ? xa : xb;
          if constexpr (AHEAD) fetch(nxt, j0 + q + 1);
          else fetch(cur, j0 + q);
          compute(sl[q], cur, j0 + q, false);
          issue(sl[q], j0 + q + D);
        }
      }
#pragma unroll
      for (int q = 0; q < D; ++q) {
        XV& cur = (q & 1) ? xb : xa;
        XV& nxt = (q & 1) ? xa : xb;
        if constexpr (AHEAD) {
          if (q + 1 < D) fetch(nxt, j0 + q + 1);
        } else {
          fetch(cur, j0 + q);
        }
        compute(sl[q], cur, j0 + q, true);
      }
    } else {
      // Exact fp32 path: every code times the activation read from memory.
      for (int j = 0; j < nloads; ++j) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, lane_code + 4096 * j, 0, BUF_STREAM);
        const int ub = (g * kb + (((c_lo + j * CPL) * TKC) >> log2_bs)) * TG;
        const uint32_t sw = __builtin_amdgcn_raw_buffer_load_b32(rs, ub * SZ + lane_soff, 0, 0);
        float sc;
        if constexpr (SZ == 4) sc = __uint_as_float(sw);
        else sc = bits16_to_f32<SDT>((uint16_t)(sw >> lane_shalf));
        int z = 1 << (BITS - 1);
        if constexpr (HAS_ZP)
          z = (int)((__builtin_amdgcn_raw_buffer_load_b32(rz, ub * BITS / 8 + lane_zoff, 0, 0) >>
                     lane_zbit) & m);
        const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
        const int c = c_lo + j * CPL + cl;
        const int k0 = c * TKC + u * E;
        float d = 0.0f;
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
          for (int e = 0; e < P; ++e) {
            const int k = k0 + wi * P + e;
            const int q = (int)((cw[wi] >> (e * BITS)) & m);
            const float xk = (k < K) ? bits16_to_f32<XDT>(x[k]) : 0.0f;
            d = fmaf(xk, (float)(q - z), d);
          }
        }
        const int b = (((c_lo + j * CPL) * TKC) >> log2_bs) + lane_db;
        const float t = fmaf(d, sc, acc);
        acc = (c < c_hi && b < kb) ? t : acc;
      }
    }
    // The next piece overwrites the staged activations.
    if (P0 + pc < chunks) __syncthreads();
  }

  // Lanes of one column: the UPC units of a chunk, then the CPL chunks.
  if constexpr (UPC >= 2) acc += __shfl_xor(acc, 1);
  if constexpr (UPC >= 4) acc += __shfl_xor(acc, 2);
#pragma unroll
  for (int st = LPC; st < 64; st *= 2) acc += __shfl_xor(acc, st);
  const bool writer = lane < LPC && u == 0;
  const int n = g * TG + gcol;
  if (S == 1) {
    if (writer && has_oct && n < N) {
      float o = acc;
      if (bias) o += bits16_to_f32<XDT>(bias[n]);
      y[n] = __builtin_bit_cast(uint16_t, dt<XDT>::from_f32(o));
    }
  } else {
    if (writer) red[wave * OCT + col] = acc;
    __syncthreads();
    if (s == 0 && writer && has_oct && n < N) {
      float o = red[ol * OCT + col];
      for (int t = 1; t < S; ++t) o += red[(t * O + ol) * OCT + col];
      if (bias) o += bits16_to_f32<XDT>(bias[n]);
      y[n] = __builtin_bit_cast(uint16_t, dt<XDT>::from_f32(o));
    }
  }
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t launch_z(const MatArgs& a, const TiledGeom& tg) {
  using G = TGeom<BITS>;
  // Loads in flight per wave (2-bit units hold 64 activations: fewer slots
  // keep the kernel within 128 registers).
  constexpr int D = (BITS == 2) ? 2 : 4;
  const int chunks = (int)tg.chunks;
  const int n_oct = (int)tg.groups * (TG / OCT);
  // Octets per workgroup: one workgroup per compute unit where there are
  // enough octets; then, for one or two octets, shares of K up to 4 waves,
  // keeping at least two wave loads per share (measured at K = 4096: N = 4096
  // 5.0 µs with two shares against 6.4 with one; N = 6144, three octets,
  // 6.1 µs with one share against 6.6 with two).
  const int O = std::min(MAX_WAVES, std::max(1, (n_oct + 255) / 256));
  int S = 1;
  while (O * S * 2 <= 4 && chunks >= 2 * (2 * S) * G::CPL) S *= 2;
  // More shares while the workgroup's threads cannot stage the activations
  // in their two first passes (every further pass is a dependent load).
  const int pc = std::min(chunks, PIECE_CHUNKS);
  while (O * S * 2 <= MAX_WAVES && O * S * 64 * 32 < (pc + G::CPL) * TKC) S *= 2;
  const TLds<BITS> L(pc, O, S, D);
  const size_t lds = (size_t)L.total * 4;
  const int grid = (n_oct + O - 1) / O;
  const bool linb = a.block_size <= TKC * G::CPL;
  auto kern = linb ? gemv_tiled_kernel<BITS, XDT, SDT, HAS_ZP, D, true>
                   : gemv_tiled_kernel<BITS, XDT, SDT, HAS_ZP, D, false>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(O * S * 64), lds, a.stream, (const uint16_t*)a.A,
                     a.B + tg.codes_off, (const uint8_t*)a.scales, a.zp, (const uint16_t*)a.bias,
                     (uint16_t*)a.Y, (int)a.K, (int)a.N, (int)a.kb, chunks,
                     __builtin_ctz((unsigned)a.block_size), n_oct, O, S, pc);
  return hipGetLastError();
}

template <int BITS, int XDT, int SDT>
hipError_t launch_s(const MatArgs& a, const TiledGeom& tg) {
  return a.zp ? launch_z<BITS, XDT, SDT, true>(a, tg) : launch_z<BITS, XDT, SDT, false>(a, tg);
}

template <int BITS, int XDT>
hipError_t launch_x(const MatArgs& a, const TiledGeom& tg) {
  switch (a.s_dtype) {
    case DT_F32: return launch_s<BITS, XDT, DT_F32>(a, tg);
    case DT_F16: return launch_s<BITS, XDT, DT_F16>(a, tg);
    default: return launch_s<BITS, XDT, DT_BF16>(a, tg);
  }
}

template <int BITS>
hipError_t launch_b(const MatArgs& a, const TiledGeom& tg) {
  return a.a_dtype == DT_F16 ? launch_x<BITS, DT_F16>(a, tg) : launch_x<BITS, DT_BF16>(a, tg);
}

}  // namespace

bool gemv_tiled_supported(const MatArgs& a) {
  // 16-bit activations, and blocks no shorter than a 16-byte unit of codes
  // (one scale per unit); 32-bit offsets with room for a few wave loads past
  // the end.
  const int E = 128 / a.bits;
  if (a.a_dtype == DT_F32 || a.block_size < E) return false;
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  return tg.total + 16 * 4096 < 0x7FFFFF00LL && a.K < (1 << 28);
}

hipError_t launch_gemv_tiled(const MatArgs& a) {
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  switch (a.bits) {
    case 2: return launch_b<2>(a, tg);
    case 4: return launch_b<4>(a, tg);
    default: return launch_b<8>(a, tg);
  }
}

}  // namespace qmm
