// gemv_tiled.hip -- M = 1 decode GEMV on the tiled weight layout (qmm_layout.h)
// for gfx950: split-K over the waves of a workgroup, one coalesced 1 KiB load
// of packed codes per wave instruction, a DPP / LDS reduction at the end.
//
// Computes y[n] = sum_k x[k] * (code(n,k) - zp(n, k/bs)) * scale[n, k/bs]
// (+ bias[n]) (onnx-runtime-ep-cpu matmul_nbits.rs: module documentation and
// dequantize_nbits_value) from the buffer written by qmm_repack.
//
// Work split.  A workgroup owns CW columns of one 32-column group (CW = 32, 16
// or 8) over the whole of K; its 4 waves split K into 4 contiguous ranges of
// 64-code chunks.  In the tiled layout the CW columns' bytes of one chunk are
// contiguous (CW * 8 * BITS bytes), so a wave-wide 16-byte-per-lane load reads
// 1 KiB covering 64 / (CW * BITS / 2) consecutive chunks.  Lane l keeps one
// column for the whole kernel and one fp32 partial sum; lanes of a column are
// combined with cross-lane shuffles, and the 4 waves through LDS.
//
// Activations.  Each wave stages its own K range of x into LDS (no workgroup
// barrier): as fp16 for f16 x; for bf16 x re-encoded exactly as fp16 after a
// power-of-two shift per 16-byte unit of codes (the largest magnitude lands
// in [2^14, 2^15), so every value within 2^28 of it keeps all of its 8
// significant bits).  A range with inf/nan, bf16 subnormals or a wider
// dynamic range takes an exact fp32 path instead.
//
// Arithmetic.  A 16-bit half of a code word holds 16 / BITS codes at bit
// offsets 0, BITS, ...; the codes at offsets p <= 8 - BITS of the word and of
// the word shifted right by 8 are masked in place and OR-ed with fp16 1024.0,
// giving 1024 + 2^p * code exactly.  Adding the fp16 pair -(1024 + 2^p * zp)
// leaves 2^p * (code - zp) exactly, and v_dot2_f32_f16 multiplies that by two
// activations (exact products) and accumulates in fp32, one accumulator per p,
// scaled back by 2^-p at the end of the unit.
#include "qmm_device.h"
#include "qmm_internal.h"
#include "qmm_layout.h"

#include <algorithm>

namespace qmm {

namespace {

constexpr int TGV_THREADS = 256;
constexpr int TGV_WAVES = 4;
// Chunks of 64 codes staged at once per wave (4096 activations, 8 KiB).
constexpr int TGV_PIECE = 64;
constexpr int RSRC_WORD3 = 0x00020000;
// Byte offset used for lanes without work: past every extent, reads zeros.
constexpr int OFF_NONE = 0x7FFFFFF0;

// Geometry of one (BITS, CW) variant.
template <int BITS, int CW>
struct TGeom {
  static constexpr int P = 32 / BITS;          // codes per 32-bit word
  static constexpr int E = 4 * P;              // codes per 16-byte unit
  static constexpr int CB = TKC * BITS / 8;    // bytes per column chunk
  static constexpr int UPC = CB / 16;          // units per column chunk
  static constexpr int LPC = CW * UPC;         // lanes per chunk in a load
  static constexpr int CPL = 64 / LPC;         // chunks per wave load
  static constexpr int NPOS = 8 / BITS;        // bit offsets p per half word
  static constexpr int LPU = E / 16;           // staging lanes per unit
  static_assert(LPC <= 64 && 64 % LPC == 0, "a chunk's columns must fit one wave load");
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

// Staging of 16 activations per lane into fp16 pairs (pair word w*P/2 + i of
// a code word w holds activations (wP + i, wP + i + P/2)), the per-unit
// factor pw undoing the shift, and whether every unit was exact.
template <int BITS, int XDT>
__device__ __forceinline__ bool stage16(const u32x4 (&raw)[2], int a, uint32_t* __restrict__ xs,
                                        float* __restrict__ pw) {
  constexpr int P = 32 / BITS, E = 4 * P, LPU = E / 16;
  float v[16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bits16_to_f32<XDT>((uint16_t)(w[j] & 0xFFFFu));
      v[8 * q + 2 * j + 1] = bits16_to_f32<XDT>((uint16_t)(w[j] >> 16));
    }
  }
  bool bad = false;
  int sh = 0;
  if constexpr (XDT == DT_BF16) {
    int emax = 0, emin = 255;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t u = __float_as_uint(v[j]) & 0x7FFFFFFFu;
      const int e = (int)(u >> 23);
      emax = (u != 0) ? max(emax, e) : emax;
      emin = (u != 0) ? min(emin, e) : emin;
    }
    if constexpr (LPU >= 2) {
      emax = max(emax, __builtin_amdgcn_update_dpp(0, emax, 0xB1, 0xF, 0xF, false));
      emin = min(emin, __builtin_amdgcn_update_dpp(0, emin, 0xB1, 0xF, 0xF, false));
    }
    if constexpr (LPU >= 4) {
      emax = max(emax, __builtin_amdgcn_update_dpp(0, emax, 0x4E, 0xF, 0xF, false));
      emin = min(emin, __builtin_amdgcn_update_dpp(0, emin, 0x4E, 0xF, 0xF, false));
    }
    if (emax != 0) {
      bad = (emax == 255) || (emin == 0) || (emin < emax - 28);
      sh = 141 - emax;   // 14 - (emax - 127)
    }
  } else {
    // fp16 activations are used as they are; only inf / nan are not exact.
#pragma unroll
    for (int j = 0; j < 16; ++j) bad |= !__builtin_isfinite(v[j]);
  }
  uint32_t pairs[8];
#pragma unroll
  for (int w = 0; w < 16 / P; ++w) {
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
      const _Float16 lo = (_Float16)ldexpf(v[w * P + i], sh);
      const _Float16 hi = (_Float16)ldexpf(v[w * P + i + P / 2], sh);
      half2_t h = {lo, hi};
      pairs[w * (P / 2) + i] = as_u32(h);
    }
  }
  // 16 activations of a 2-bit word span a whole word (P = 16) but only when
  // the lane holds the full word; a lane always holds 16 consecutive
  // activations starting at a multiple of 16, which is a whole number of
  // code words for BITS >= 4 and one full word for BITS = 2.
  u32x4* dst = reinterpret_cast<u32x4*>(xs + a / 2);
  dst[0] = u32x4{pairs[0], pairs[1], pairs[2], pairs[3]};
  dst[1] = u32x4{pairs[4], pairs[5], pairs[6], pairs[7]};
  if ((threadIdx.x % LPU) == 0) pw[a / E] = ldexpf(1.0f, -sh);
  return bad;
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int CW, int D>
__global__ __launch_bounds__(TGV_THREADS) void gemv_tiled_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zps,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int K, int N, int kb,
    int chunks, int log2_bs, int per_wave, int pc) {
  using G = TGeom<BITS, CW>;
  using ST = typename dt<SDT>::T;
  constexpr int P = G::P, E = G::E, CB = G::CB, UPC = G::UPC, LPC = G::LPC, CPL = G::CPL;
  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);

  extern __shared__ u32x4 smem_tv[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Per-wave LDS region: pc * 32 pair words, then pc * 64 / E unit factors,
  // rounded up to 16 bytes.
  const int region = pc * 32 + (pc * (64 / E) + 3) / 4 * 4;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_tv) + wave * region;
  float* pw = reinterpret_cast<float*>(xs + pc * 32);
  float* red = reinterpret_cast<float*>(smem_tv) + TGV_WAVES * region;

  const int slices = 32 / CW;
  const int g = blockIdx.x / slices;
  const int col0 = (blockIdx.x % slices) * CW;     // first column within the group
  const int cl = lane / LPC;                        // chunk within a wave load
  const int rem = lane % LPC;
  const int col = rem / UPC;                        // column within the slice
  const int u = rem % UPC;                          // unit within the column chunk
  const int gcol = col0 + col;                      // column within the group

  const int groups = (N + TG - 1) / TG;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)codes, 0, groups * chunks * TG * CB, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)scales, 0, groups * kb * TG * (int)sizeof(ST), RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
      (void*)zps, 0, HAS_ZP ? groups * kb * TG * BITS / 8 : 0, RSRC_WORD3);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, 0, K * 2, RSRC_WORD3);
  const bool x_vec = (K % 8) == 0 && (((uintptr_t)x) & 15) == 0;

  const int w_lo = wave * per_wave;
  const int w_hi = min(chunks, w_lo + per_wave);
  float acc = 0.0f;

  for (int p_lo = w_lo; p_lo < w_hi; p_lo += pc) {
    const int p_hi = min(w_hi, p_lo + pc);
    const int nloads = (p_hi - p_lo + CPL - 1) / CPL;

    // Load j of the piece: chunk p_lo + j*CPL + cl; lanes past the piece
    // read zeros from past the extents.
    auto chunk_of = [&](int j) { return p_lo + j * CPL + cl; };
    // A lane is live when its chunk is in the piece and its unit starts
    // inside the blocks (chunk padding past kb * bs has no scale).
    auto live_of = [&](int c) { return c < p_hi && ((c * TKC + u * E) >> log2_bs) < kb; };
    auto issue = [&](TSlot& s, int j) {
      const int c = chunk_of(j);
      const bool live = live_of(c);
      const int off = live ? ((g * chunks + c) * TG + gcol) * CB + u * 16 : OFF_NONE;
      s.cw = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
      const int b = (c * TKC + u * E) >> log2_bs;
      const int si = (g * kb + b) * TG + gcol;
      // Region sizes are multiples of 4 bytes, so aligned words are wholly
      // inside or wholly past them.
      s.sw = __builtin_amdgcn_raw_buffer_load_b32(
          rs, live ? (si * (int)sizeof(ST)) & ~3 : OFF_NONE, 0, 0);
      if constexpr (HAS_ZP)
        s.zw = __builtin_amdgcn_raw_buffer_load_b32(rz, live ? ((si * BITS) >> 3) & ~3 : OFF_NONE,
                                                    0, 0);
      __builtin_amdgcn_sched_barrier(0);
    };

    TSlot sl[D];
#pragma unroll
    for (int q = 0; q < D; ++q) issue(sl[q], q);

    // Stage this piece's activations (wave-local: the same wave reads them).
    const int n_act = (p_hi - p_lo) * TKC;
    bool bad = false;
    for (int a = lane * 16; a < n_act; a += 64 * 16) {
      const int k = p_lo * TKC + a;
      u32x4 raw[2];
      if (x_vec) {
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
      bad |= stage16<BITS, XDT>(raw, a, xs, pw);
    }
    // Make the staged values visible to the other lanes of this wave.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const bool exact = __builtin_amdgcn_ballot_w64(bad) != 0;

    if (!exact) {
      for (int j0 = 0; j0 < nloads; j0 += D) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
          const int j = j0 + q;
          TSlot& s = sl[q];
          const int c = chunk_of(j);
          const bool live = live_of(c);
          // Unit start relative to the piece; dead lanes read a staged spot.
          const int kr = live ? (c - p_lo) * TKC + u * E : 0;
          const u32x4* xv = reinterpret_cast<const u32x4*>(xs + kr / 2);
          uint32_t xw[E / 2];
#pragma unroll
          for (int t = 0; t < E / 8; ++t) {
            const u32x4 v = xv[t];
            xw[4 * t + 0] = v.x; xw[4 * t + 1] = v.y; xw[4 * t + 2] = v.z; xw[4 * t + 3] = v.w;
          }
          const float f = pw[kr / E];
          const int b = (c * TKC + u * E) >> log2_bs;
          const int si = (g * kb + b) * TG + gcol;
          uint32_t z = 1u << (BITS - 1);
          if constexpr (HAS_ZP) z = (s.zw >> ((si * BITS) & 31)) & m;
          float sc;
          if constexpr (sizeof(ST) == 4) sc = __uint_as_float(s.sw);
          else sc = bits16_to_f32<SDT>((uint16_t)(s.sw >> ((si & 1) * 16)));
          float dp[G::NPOS];
          half2_t nz[G::NPOS];
#pragma unroll
          for (int pi = 0; pi < G::NPOS; ++pi) {
            dp[pi] = 0.0f;
            const uint32_t h = 0xE400u | (z << (pi * BITS));   // -(1024 + 2^p z)
            nz[pi] = as_half2(h | (h << 16));
          }
          const uint32_t cw[4] = {s.cw.x, s.cw.y, s.cw.z, s.cw.w};
#pragma unroll
          for (int wi = 0; wi < 4; ++wi) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const uint32_t src = hf ? (cw[wi] >> 8) : cw[wi];
#pragma unroll
              for (int pi = 0; pi < G::NPOS; ++pi) {
                const int p = pi * BITS;
                const uint32_t mask = (m << p) | (m << (p + 16));
                const half2_t cv = as_half2((src & mask) | 0x64006400u) + nz[pi];
                const int ci = (hf * 8 + p) / BITS;            // code index in the word
                dp[pi] = __builtin_amdgcn_fdot2(cv, as_half2(xw[wi * (P / 2) + ci]), dp[pi],
                                                false);
              }
            }
          }
          float d = dp[0];
#pragma unroll
          for (int pi = 1; pi < G::NPOS; ++pi) d = fmaf(dp[pi], ldexpf(1.0f, -pi * BITS), d);
          const float t = fmaf(d, f * sc, acc);
          acc = live ? t : acc;
          issue(s, j + D);
        }
      }
    } else {
      // Exact fp32 path: every code times the activation read from memory.
      for (int j = 0; j < nloads; ++j) {
        const int c = chunk_of(j);
        const bool live = live_of(c);
        const int off = live ? ((g * chunks + c) * TG + gcol) * CB + u * 16 : OFF_NONE;
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, off, 0, 0);
        const int b = (c * TKC + u * E) >> log2_bs;
        const int si = (g * kb + b) * TG + gcol;
        const int soff = live ? si * (int)sizeof(ST) : OFF_NONE;
        float s;
        if constexpr (sizeof(ST) == 4)
          s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, soff, 0, 0));
        else
          s = bits16_to_f32<SDT>(__builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0));
        int z = 1 << (BITS - 1);
        if constexpr (HAS_ZP)
          z = (int)((__builtin_amdgcn_raw_buffer_load_b8(rz, live ? (si * BITS) >> 3 : OFF_NONE,
                                                         0, 0) >> ((si * BITS) & 7)) & m);
        const uint32_t cw[4] = {v.x, v.y, v.z, v.w};
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
        const float t = fmaf(d, s, acc);
        acc = live ? t : acc;
      }
    }
  }

  // Lanes of one column: the UPC units of a chunk, then the CPL chunks.
  if constexpr (UPC >= 2) acc += __shfl_xor(acc, 1);
  if constexpr (UPC >= 4) acc += __shfl_xor(acc, 2);
#pragma unroll
  for (int st = LPC; st < 64; st *= 2) acc += __shfl_xor(acc, st);
  if (lane < LPC && u == 0) red[wave * CW + col] = acc;
  __syncthreads();
  if (threadIdx.x < CW) {
    const int n = g * TG + col0 + threadIdx.x;
    if (n < N) {
      float o = red[threadIdx.x];
#pragma unroll
      for (int w = 1; w < TGV_WAVES; ++w) o += red[w * CW + threadIdx.x];
      if (bias) o += bits16_to_f32<XDT>(bias[n]);
      y[n] = __builtin_bit_cast(uint16_t, dt<XDT>::from_f32(o));
    }
  }
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int CW>
hipError_t launch_cw(const MatArgs& a, const TiledGeom& tg) {
  using G = TGeom<BITS, CW>;
  constexpr int D = (BITS == 8) ? 8 : 8;
  const int chunks = (int)tg.chunks;
  // Chunks per wave: a whole number of wave loads.
  const int per_wave = (chunks + TGV_WAVES * G::CPL - 1) / (TGV_WAVES * G::CPL) * G::CPL;
  const int pc = std::min(per_wave, TGV_PIECE);
  const int region = pc * 32 + (pc * (64 / G::E) + 3) / 4 * 4;
  const size_t lds = (size_t)(TGV_WAVES * region + TGV_WAVES * CW) * 4;
  const int grid = (int)tg.groups * (32 / CW);
  const uint8_t* codes = a.B + tg.codes_off;
  hipLaunchKernelGGL((gemv_tiled_kernel<BITS, XDT, SDT, HAS_ZP, CW, D>), dim3(grid),
                     dim3(TGV_THREADS), lds, a.stream, (const uint16_t*)a.A, codes,
                     (const typename dt<SDT>::T*)a.scales, a.zp, (const uint16_t*)a.bias,
                     (uint16_t*)a.Y, (int)a.K, (int)a.N, (int)a.kb, chunks,
                     __builtin_ctz((unsigned)a.block_size), per_wave, pc);
  return hipGetLastError();
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
hipError_t launch_z(const MatArgs& a, const TiledGeom& tg) {
  // Columns per workgroup: enough workgroups to cover the 256 compute units
  // about twice.
  const int64_t groups = tg.groups;
  if constexpr (BITS != 8)
    if (groups >= 256) return launch_cw<BITS, XDT, SDT, HAS_ZP, 32>(a, tg);
  if (groups >= 128) return launch_cw<BITS, XDT, SDT, HAS_ZP, 16>(a, tg);
  return launch_cw<BITS, XDT, SDT, HAS_ZP, 8>(a, tg);
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
  // (one scale per unit); 32-bit offsets.
  const int E = 128 / a.bits;
  if (a.a_dtype == DT_F32 || a.block_size < E) return false;
  const TiledGeom tg = tiled_geom(a.K, a.N, a.block_size, a.bits, a.s_dtype == DT_F32 ? 4 : 2,
                                  a.zp != nullptr);
  return tg.total < 0x7FFFFF00LL && a.K < (1 << 28);
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
