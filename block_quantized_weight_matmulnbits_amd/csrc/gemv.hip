// gemv.hip -- M = 1 decode GEMV over block-quantized weights for gfx950.
//
// Computes y[n] = sum_k x[k] * (code(n,k) - zp(n, k/bs)) * scale[n, k/bs]
// (+ bias[n]) from the MatMulNBits layout B[N, kb, bs*bits/8], codes packed
// least-significant bits first (onnx-runtime-ep-cpu matmul_nbits.rs: module
// documentation and dequantize_nbits_value).  The kernel is bound by HBM
// traffic on the packed weight bytes, so it never writes a dequantized weight.
//
// Work split: a workgroup of 4 waves owns 4*R consecutive output rows, R per
// wave.  The activation vector is staged once per workgroup into LDS; lanes
// then stride over 16-byte units of a row (lane l takes units l, l+64, ...),
// so one wave-wide load reads 1 KiB of contiguous codes per row.  Each lane
// keeps R partial sums that a DPP reduction combines at the end.
//
// Arithmetic for f16/bf16 activations: codes become fp16 (1024 + code) with one
// AND/OR, the zero point is removed with an exact packed fp16 add, and
// v_dot2_f32_f16 multiplies by fp16 activations and accumulates in fp32.
// bf16 activations are re-encoded exactly as fp16 after a per-unit power-of-two
// shift (bf16 has 8 significant bits, fp16 11); a unit whose dynamic range does
// not fit fp16 normals, or that holds inf/nan, makes its chunk take an exact
// fp32 path instead.  Products are therefore exact and accumulation is fp32.
// f32 activations always take the fp32 path.
#include "qmm_device.h"
#include "qmm_internal.h"

#include <algorithm>

namespace qmm {

// Word 3 of a gfx9 buffer resource descriptor for raw byte-addressed loads
// (32-bit data format; no swizzle, no index stride).
constexpr int BUFFER_RSRC_WORD3 = 0x00020000;

// Activation elements staged per LDS chunk (fp16 path: 2 bytes each).
constexpr int GEMV_CHUNK = 16384;
constexpr int GEMV_THREADS = 256;

// ---------------------------------------------------------------------------
// Staging of x for the fp16 path.
// Thread t converts TE consecutive activations per pass (whole 32-bit words
// of codes).  The LDS pair layout matches code_pair_1024: for the word of
// codes holding elements [wP, wP+P), LDS word (w*P/2 + i) holds
// (x[wP+i], x[wP+i+P/2]).  pw[g] is the power of two that undoes the shift of
// 16-byte unit g (E = 4P elements).  *inexact is raised when a unit cannot be
// carried exactly (range beyond fp16 normals, inf/nan, bf16 subnormals).
// ---------------------------------------------------------------------------
template <int BITS>
struct StageGeom {
  static constexpr int P = 32 / BITS;          // codes per 32-bit word
  static constexpr int TE = (P > 8) ? P : 8;   // activations per thread and pass
  static constexpr int E = 4 * P;              // activations per 16-byte unit
  static constexpr int TPU = E / TE;           // threads per unit (2 or 4)
  static constexpr int PASS = GEMV_THREADS * TE;
};

// Raw 16-bit activations of one thread-pass, kept as the loaded 128-bit
// vectors so that loading does not wait for the data.  `live` is false when
// the pass lies past K; its values are then replaced by zeros on use.
template <int BITS>
struct XRaw {
  u32x4 v[StageGeom<BITS>::TE / 8];
  bool live;
};

// vec_ok (wave-uniform): x is 16-byte aligned and K is a multiple of TE, so
// every pass is either wholly inside [0, K) or wholly past it and can be read
// with plain vector loads from a clamped, in-bounds address, with no
// lane-divergent branch (which would make the compiler wait for all loads).
template <int BITS, int XDT>
__device__ __forceinline__ void load_x_raw(const uint16_t* __restrict__ x, int kg, int K,
                                           bool vec_ok, XRaw<BITS>& r) {
  constexpr int TE = StageGeom<BITS>::TE;
  if (vec_ok) {
    r.live = kg < K;
    const int kc = min(kg, K - TE);
#pragma unroll
    for (int v = 0; v < TE / 8; ++v) r.v[v] = *reinterpret_cast<const u32x4*>(x + kc + 8 * v);
  } else {
    r.live = true;
#pragma unroll
    for (int v = 0; v < TE / 8; ++v) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = kg + 8 * v + 2 * j;
        const uint32_t lo = (k < K) ? x[k] : 0u;
        const uint32_t hi = (k + 1 < K) ? x[k + 1] : 0u;
        w[j] = lo | (hi << 16);
      }
      r.v[v] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

template <int XDT>
__device__ __forceinline__ float raw_to_f32(uint16_t h) {
  if constexpr (XDT == DT_BF16) return __uint_as_float((uint32_t)h << 16);
  else return (float)__builtin_bit_cast(_Float16, h);
}

// 16-byte piece slot of logical piece j of unit u when units hold NP pieces
// (NP = 0: no swizzle).  The pieces of a unit are XOR-permuted by a function
// of the unit so that the 8 lanes of an LDS read pass (consecutive units,
// the same logical piece, units 8 NP words apart) fall in distinct banks of
// the 32 that these accesses see: without it, units 64 bytes apart (4-bit)
// put lanes 2 apart in one bank.
template <int NP>
__device__ __forceinline__ int x_piece(int u, int j) {
  if constexpr (NP == 0) return u * 0 + j;
  else return u * NP + (j ^ ((u / (8 / NP)) % NP));
}

template <int BITS, int XDT, int NP>
__device__ __forceinline__ void stage_pass(const XRaw<BITS>& r, int base,
                                           uint32_t* __restrict__ xs, float* __restrict__ pw,
                                           int* inexact) {
  using G = StageGeom<BITS>;
  constexpr int P = G::P, TE = G::TE, E = G::E, TPU = G::TPU;
  float v[TE];
#pragma unroll
  for (int q = 0; q < TE / 8; ++q) {
    const uint32_t w[4] = {r.live ? r.v[q].x : 0u, r.live ? r.v[q].y : 0u,
                           r.live ? r.v[q].z : 0u, r.live ? r.v[q].w : 0u};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = raw_to_f32<XDT>((uint16_t)(w[j] & 0xFFFFu));
      v[8 * q + 2 * j + 1] = raw_to_f32<XDT>((uint16_t)(w[j] >> 16));
    }
  }
  // Biased exponent range of the nonzero values (bf16 shares fp32's exponent
  // field; f16 values widen to fp32 normals).
  int emax = 0, emin = 255;
#pragma unroll
  for (int j = 0; j < TE; ++j) {
    const uint32_t u = __float_as_uint(v[j]) & 0x7FFFFFFFu;
    const int e = (int)(u >> 23);
    emax = (u != 0) ? max(emax, e) : emax;
    emin = (u != 0) ? min(emin, e) : emin;
  }
  // Combine over the TPU adjacent lanes of one unit (quad_perm DPP).
  emax = max(emax, __builtin_amdgcn_update_dpp(0, emax, 0xB1, 0xF, 0xF, false));
  emin = min(emin, __builtin_amdgcn_update_dpp(0, emin, 0xB1, 0xF, 0xF, false));
  if constexpr (TPU == 4) {
    emax = max(emax, __builtin_amdgcn_update_dpp(0, emax, 0x4E, 0xF, 0xF, false));
    emin = min(emin, __builtin_amdgcn_update_dpp(0, emin, 0x4E, 0xF, 0xF, false));
  }
  // Shift so the largest magnitude lands in [2^14, 2^15): fp16 normals then
  // hold every value down to 2^-14 with 11 significant bits, which covers
  // every activation within 2^28 of the unit's largest.
  bool bad = false;
  int sh = 0;
  if (emax != 0) {
    bad = (emax == 255) || (emin == 0) || (emin < emax - 28);
    sh = 141 - emax;  // 14 - (emax - 127)
  }
  if (bad) atomicOr(inexact, 1);
  uint32_t pairs[TE / 2];
#pragma unroll
  for (int w = 0; w < TE / P; ++w) {
#pragma unroll
    for (int i = 0; i < P / 2; ++i) {
      const _Float16 lo = (_Float16)ldexpf(v[w * P + i], sh);
      const _Float16 hi = (_Float16)ldexpf(v[w * P + i + P / 2], sh);
      half2_t h = {lo, hi};
      pairs[w * (P / 2) + i] = as_u32(h);
    }
  }
  u32x4* dst = reinterpret_cast<u32x4*>(xs);
#pragma unroll
  for (int j = 0; j < TE / 8; ++j) {
    u32x4 t = {pairs[4 * j], pairs[4 * j + 1], pairs[4 * j + 2], pairs[4 * j + 3]};
    const int pg = base / 8 + j;   // piece of the chunk
    dst[NP ? x_piece<NP>(pg / (NP ? NP : 1), pg % (NP ? NP : 1)) : pg] = t;
  }
  if ((threadIdx.x % TPU) == 0) pw[base / E] = ldexpf(1.0f, -sh);
}

// Exact fp32 contribution of one 32-bit word of codes with activations read
// from global memory (fp32 activations, and the fallback of the fp16 path).
template <int BITS, int XDT>
__device__ __forceinline__ float word_dot_exact(uint32_t w, const typename dt<XDT>::T* __restrict__ x,
                                                int k, int K, int z) {
  constexpr int P = 32 / BITS;
  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < P; ++j) {
    const int q = (int)((w >> (j * BITS)) & m);
    const float xv = (k + j < K) ? dt<XDT>::to_f32(x[k + j]) : 0.0f;
    acc = fmaf(xv, (float)(q - z), acc);
  }
  return acc;
}

// One in-flight job of a wave: the codes of one unit per lane of one row,
// with that unit's scale and zero point.
// Loaded values are kept raw (scale bits, zero-point byte) and decoded only
// when the job is consumed, so issuing a job never waits for memory.
template <int UW, typename ST>
struct Slot {
  uint32_t cw[UW];
  ST sc;
  uint32_t zb;   // zero-point byte (HAS_ZP)
  int blk;       // block index of the unit
};

// ---------------------------------------------------------------------------
// The GEMV kernel.
// A workgroup owns 4*R consecutive rows, R per wave.  A wave walks a queue of
// jobs (row r, 64-unit chunk c): lane l handles unit c*64 + l of row r, so
// each job is one coalesced 64 x 16-byte load.  D jobs are kept in flight in
// registers (a software pipeline); the first D are issued before x is staged,
// so staging overlaps the first HBM round trip.
// VEC: 16-byte units inside one block (blob >= 16); otherwise 4-byte units.
// FAST: fp16 dot path for f16/bf16 activations; otherwise exact fp32 only.
// Dynamic LDS: x pairs (staged/2 words), pw (staged/E floats), two flags,
// staged = chunk_units*UE rounded up to whole 16-byte units.
// ---------------------------------------------------------------------------
template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, bool VEC, bool FAST, int D,
          bool ONE_CHUNK>
__global__ __launch_bounds__(GEMV_THREADS) void gemv_kernel(
    const typename dt<XDT>::T* __restrict__ x, const uint8_t* __restrict__ B,
    const typename dt<SDT>::T* __restrict__ scales, const uint8_t* __restrict__ zp,
    const typename dt<XDT>::T* __restrict__ bias, typename dt<XDT>::T* __restrict__ y,
    int K, int N, int kb, int log2_blob, int zp_row_bytes, int chunk_units) {
  using G = StageGeom<BITS>;
  constexpr int P = G::P;
  constexpr int E = G::E;
  constexpr int UW = VEC ? 4 : 1;   // 32-bit words per unit
  constexpr int UE = UW * P;        // activations per unit
  // 16-byte pieces per unit whose LDS slots are swizzled (16-byte units:
  // 2, 4 or 8 pieces; 4-byte units are read a word at a time, unswizzled).
  constexpr int XNP = VEC ? UE / 8 : 0;
  extern __shared__ u32x4 smem_v[];
  // Staged activations per chunk, rounded up to whole 16-byte units of codes.
  const int staged = (chunk_units * UE + E - 1) / E * E;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_v);
  float* pw = reinterpret_cast<float*>(xs + staged / 2);
  // One flag per chunk parity: a wave may still read chunk c's flag after
  // another has reset chunk c+1's; chunk c's is reset again only after every
  // wave has passed chunk c+1's first barrier.
  int* inexact = reinterpret_cast<int*>(pw + staged / E);

  const int lane = threadIdx.x & 63;
  // Wave index as a scalar: everything derived from it stays wave-uniform, so
  // the job-queue branches are scalar branches.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row0 = (blockIdx.x * 4 + wave) * R;
  const int nrows = max(0, min(R, N - row0));
  const int64_t row_bytes = (int64_t)kb << log2_blob;
  const int blob_words_log2 = log2_blob - 2;
  const int total_units = (int)(row_bytes / (4 * UW));
  const bool x_vec = ((uintptr_t)x & 15) == 0 && (K % StageGeom<BITS>::TE) == 0;

  using ST_ = typename dt<SDT>::T;
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;

  // ONE_CHUNK (the row fits one LDS chunk): no loop around the pipeline, so
  // the compiler sees no load still pending from an earlier chunk.
  const int n_chunks = ONE_CHUNK ? 1 : (total_units + chunk_units - 1) / chunk_units;
  for (int ci = 0; ci < n_chunks; ++ci) {
    const int c0 = ci * chunk_units;
    const int c1 = ONE_CHUNK ? total_units : min(total_units, c0 + chunk_units);
    bool exact = !FAST;
    if constexpr (FAST) {
      const int cpr = (c1 - c0 + 63) >> 6;   // 64-unit chunks in this K-chunk
      const int len = (c1 - c0) * UE;        // activations in this K-chunk
      const int len_units = (len + E - 1) / E * E;

      // x of the first two staging passes: loaded before the weights so that
      // waiting for it does not wait for the weight loads.
      XRaw<BITS> xr0, xr1;
      const int b0 = threadIdx.x * G::TE, b1 = b0 + G::PASS;
      load_x_raw<BITS, XDT>((const uint16_t*)x, c0 * UE + b0, K, x_vec, xr0);
      load_x_raw<BITS, XDT>((const uint16_t*)x, c0 * UE + b1, K, x_vec, xr1);

      // Jobs run chunk-major: job j is (chunk j / R, row j % R), so a chunk's
      // activations are read from LDS once and reused for the R rows, and a
      // pipeline slot s always serves row s % R.  D / R chunks are in flight.
      // Loads go through per-row buffer descriptors; rows past N get
      // num_records = 0, and so do chunks past the last (by a zero extent),
      // so every issue is branch-free (a branch around the loads, even a
      // wave-uniform one, makes the compiler wait for all of them) and
      // out-of-range loads return zeros without touching memory.  Lanes past
      // the K-chunk's last unit read past num_records and are masked on use.
      constexpr int CIF = D / R;              // chunks in flight
      __amdgpu_buffer_rsrc_t rb[R], rs[R], rz[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const bool live = r < nrows;
        const int row = min(row0 + r, N - 1);
        rb[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)row * row_bytes), 0,
                                                  live ? c1 * (4 * UW) : 0, BUFFER_RSRC_WORD3);
        rs[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(scales + (int64_t)row * kb), 0,
                                                  live ? kb * (int)sizeof(ST_) : 0,
                                                  BUFFER_RSRC_WORD3);
        if constexpr (HAS_ZP)
          rz[r] = __builtin_amdgcn_make_buffer_rsrc((void*)(zp + (int64_t)row * zp_row_bytes), 0,
                                                    live ? zp_row_bytes : 0, BUFFER_RSRC_WORD3);
      }
      // Chunk c of the wave reads unit c0 + c*64 + lane; chunks >= cpr are
      // pushed past every row's end.
      auto unit_of = [&](int c) { return (c < cpr) ? c0 + c * 64 + lane : (1 << 30) / 16; };
      Slot<UW, ST_> sl[D];
      auto issue = [&](Slot<UW, ST_>& q, int r, int u) {
        if constexpr (VEC) {
          const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rb[r], u * 16, 0, BUF_STREAM);
          q.cw[0] = t.x; q.cw[1] = t.y; q.cw[2] = t.z; q.cw[3] = t.w;
        } else {
          q.cw[0] = __builtin_amdgcn_raw_buffer_load_b32(rb[r], u * 4, 0, BUF_STREAM);
        }
        const int blk = (u * UW) >> blob_words_log2;
        q.blk = blk;
        if constexpr (sizeof(ST_) == 4)
          q.sc = __builtin_bit_cast(ST_, __builtin_amdgcn_raw_buffer_load_b32(rs[r], blk * 4, 0, 0));
        else
          q.sc = __builtin_bit_cast(ST_, __builtin_amdgcn_raw_buffer_load_b16(rs[r], blk * 2, 0, 0));
        if constexpr (HAS_ZP) q.zb = __builtin_amdgcn_raw_buffer_load_b8(rz[r], (blk * BITS) >> 3, 0, 0);
        // Keep each job's loads together and in issue order: the scheduler
        // would otherwise hoist every code load above the scale loads, and
        // consuming the first job would then wait for all of them.
        __builtin_amdgcn_sched_barrier(0);
      };
#pragma unroll
      for (int q = 0; q < D; ++q) issue(sl[q], q % R, unit_of(q / R));

      // Stage x into LDS.
      if (threadIdx.x == 0) inexact[ci & 1] = 0;
      __syncthreads();
      if (b0 < len_units) stage_pass<BITS, XDT, XNP>(xr0, b0, xs, pw, &inexact[ci & 1]);
      if (b1 < len_units) stage_pass<BITS, XDT, XNP>(xr1, b1, xs, pw, &inexact[ci & 1]);
      for (int b = b1 + G::PASS; b < len_units; b += G::PASS) {
        XRaw<BITS> xr;
        load_x_raw<BITS, XDT>((const uint16_t*)x, c0 * UE + b, K, x_vec, xr);
        stage_pass<BITS, XDT, XNP>(xr, b, xs, pw, &inexact[ci & 1]);
      }
      __syncthreads();
      exact = inexact[ci & 1] != 0;

      if (!exact) {
        // ---------------- fp16 dot path, pipelined ----------------
        for (int cb = 0; cb < cpr; cb += CIF) {
#pragma unroll
          for (int q0 = 0; q0 < D; q0 += R) {
            const int c = cb + q0 / R;
            if (c < cpr) {
              // This chunk's activations, read once for all R rows.  Masked
              // lanes read a clamped, staged position.
              const int lu_raw = c * 64 + lane;
              const bool ok = lu_raw < c1 - c0;
              const int lu = min(lu_raw, c1 - c0 - 1);
              uint32_t xw[UE / 2];
              if constexpr (VEC) {
                const u32x4* xv = reinterpret_cast<const u32x4*>(xs);
#pragma unroll
                for (int j = 0; j < UE / 8; ++j) {
                  const u32x4 t = xv[x_piece<XNP>(lu, j)];
                  xw[4 * j + 0] = t.x; xw[4 * j + 1] = t.y;
                  xw[4 * j + 2] = t.z; xw[4 * j + 3] = t.w;
                }
              } else {
#pragma unroll
                for (int j = 0; j < UE / 2; ++j) xw[j] = xs[lu * (UE / 2) + j];
              }
              const float p = pw[(lu * UE) / E];
#pragma unroll
              for (int r = 0; r < R; ++r) {
                Slot<UW, ST_>& q = sl[q0 + r];
                uint32_t z = 1u << (BITS - 1);
                if constexpr (HAS_ZP) {
                  constexpr uint32_t m = (BITS == 8) ? 0xFFu : ((1u << BITS) - 1u);
                  z = (q.zb >> ((q.blk * BITS) & 7)) & m;
                }
                const half2_t nz = neg_zero_point_pair(z);
                float d = 0.0f;
#pragma unroll
                for (int j = 0; j < UW; ++j) {
#pragma unroll
                  for (int i = 0; i < P / 2; ++i) {
                    const half2_t cv = as_half2(code_pair_1024<BITS>(q.cw[j], i)) + nz;
                    d = __builtin_amdgcn_fdot2(cv, as_half2(xw[j * (P / 2) + i]), d, false);
                  }
                }
                const float t = fmaf(d, p * dt<SDT>::to_f32(q.sc), acc[r]);
                acc[r] = ok ? t : acc[r];
              }
            }
            // Refill these R slots with chunk c + CIF.
#pragma unroll
            for (int r = 0; r < R; ++r) issue(sl[q0 + r], r, unit_of(c + CIF));
          }
        }
      }
    }
    if (exact) {
      // ---------------- exact fp32 path ----------------
      for (int r = 0; r < nrows; ++r) {
        const int row = row0 + r;
        const uint8_t* rowp = B + (int64_t)row * row_bytes;
        float cur = 0.0f;
        for (int u = c0 + lane; u < c1; u += 64) {
          const int blk = (u * UW) >> blob_words_log2;
          const float s = dt<SDT>::to_f32(scales[(int64_t)row * kb + blk]);
          const int z = (int)load_zp<BITS, HAS_ZP>(zp + (int64_t)row * zp_row_bytes, blk);
          float d = 0.0f;
#pragma unroll
          for (int j = 0; j < UW; ++j) {
            const uint32_t w = reinterpret_cast<const uint32_t*>(rowp)[u * UW + j];
            d += word_dot_exact<BITS, XDT>(w, x, (u * UW + j) * P, K, z);
          }
          cur = fmaf(d, s, cur);
        }
#pragma unroll
        for (int q = 0; q < R; ++q) acc[q] += (q == r) ? cur : 0.0f;
      }
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float v = wave_sum(acc[r]);
    const int row = row0 + r;
    if (lane == 0 && r < nrows) {
      float o = v;
      if (bias) o += dt<XDT>::to_f32(bias[row]);
      y[row] = dt<XDT>::from_f32(o);
    }
  }
}

template <int BITS, int XDT, int SDT, bool HAS_ZP, int R, bool VEC>
static hipError_t launch_gemv_r(const GemvArgs& a) {
  constexpr bool FAST = XDT != DT_F32;
  // Jobs in flight per wave (a multiple of R); on the 4096 x 14336 shape,
  // D = 4 measured faster than 8 or 16 at every R (fewer VGPRs, more waves).
  constexpr int D = (R > 4) ? R : 4;
  constexpr int P = 32 / BITS;
  constexpr int UE = (VEC ? 4 : 1) * P;
  constexpr int E = 4 * P;
  const int rows_per_block = 4 * R;
  const int grid = (int)((a.N + rows_per_block - 1) / rows_per_block);
  int log2_blob = 0;
  while ((1 << log2_blob) < a.blob) ++log2_blob;
  const int64_t total_units = a.kb * a.blob / (4 * (VEC ? 4 : 1));
  const int chunk_units = (int)std::min<int64_t>(total_units, GEMV_CHUNK / UE);
  // x pairs + unit factors + flags (the kernel lays them out the same way).
  const int staged = (chunk_units * UE + E - 1) / E * E;
  const size_t lds = FAST ? (size_t)staged * 2 + (size_t)(staged / E) * 4 + 16 : 16;
  using XT = typename dt<XDT>::T;
  using ST = typename dt<SDT>::T;
  if (total_units <= chunk_units)
    hipLaunchKernelGGL((gemv_kernel<BITS, XDT, SDT, HAS_ZP, R, VEC, FAST, D, true>), dim3(grid),
                       dim3(GEMV_THREADS), lds, a.stream, (const XT*)a.A, a.B,
                       (const ST*)a.scales, a.zp, (const XT*)a.bias, (XT*)a.Y, (int)a.K,
                       (int)a.N, (int)a.kb, log2_blob, (int)a.zp_row_bytes, chunk_units);
  else
    hipLaunchKernelGGL((gemv_kernel<BITS, XDT, SDT, HAS_ZP, R, VEC, FAST, D, false>), dim3(grid),
                       dim3(GEMV_THREADS), lds, a.stream, (const XT*)a.A, a.B,
                       (const ST*)a.scales, a.zp, (const XT*)a.bias, (XT*)a.Y, (int)a.K,
                       (int)a.N, (int)a.kb, log2_blob, (int)a.zp_row_bytes, chunk_units);
  return hipGetLastError();
}

template <int BITS, int XDT, int SDT, bool HAS_ZP>
static hipError_t launch_gemv_t(const GemvArgs& a) {
  const bool vec = a.blob >= 16;
  // Rows per wave: enough workgroups to cover 256 CUs several times.
  const int64_t n = a.N;
  if (vec) {
    if (n >= 8192) return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, 4, true>(a);
    if (n >= 2048) return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, 2, true>(a);
    return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, 1, true>(a);
  }
  if (n >= 8192) return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, 4, false>(a);
  return launch_gemv_r<BITS, XDT, SDT, HAS_ZP, 1, false>(a);
}

template <int BITS, int XDT, int SDT>
static hipError_t launch_gemv_z(const GemvArgs& a) {
  return a.zp ? launch_gemv_t<BITS, XDT, SDT, true>(a) : launch_gemv_t<BITS, XDT, SDT, false>(a);
}

template <int BITS, int XDT>
static hipError_t launch_gemv_s(const GemvArgs& a) {
  switch (a.s_dtype) {
    case DT_F32: return launch_gemv_z<BITS, XDT, DT_F32>(a);
    case DT_F16: return launch_gemv_z<BITS, XDT, DT_F16>(a);
    default: return launch_gemv_z<BITS, XDT, DT_BF16>(a);
  }
}

template <int BITS>
static hipError_t launch_gemv_x(const GemvArgs& a) {
  switch (a.a_dtype) {
    case DT_F32: return launch_gemv_s<BITS, DT_F32>(a);
    case DT_F16: return launch_gemv_s<BITS, DT_F16>(a);
    default: return launch_gemv_s<BITS, DT_BF16>(a);
  }
}

hipError_t launch_gemv(const GemvArgs& a) {
  if (a.g_idx) return launch_gidx(a);
  if (a.bits == 3) return launch_generic_float(a);
  // The tiled layout: its own split-K kernel, or for f32 activations and
  // blocks shorter than a 16-byte unit of codes, the row kernel of the GEMM.
  if (a.tiled) return gemv_tiled_supported(a) ? launch_gemv_tiled(a) : launch_gemm(a);
  switch (a.bits) {
    case 2: return launch_gemv_x<2>(a);
    case 4: return launch_gemv_x<4>(a);
    default: return launch_gemv_x<8>(a);
  }
}

}  // namespace qmm
