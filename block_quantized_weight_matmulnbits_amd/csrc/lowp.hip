// lowp.hip -- the low-precision scaled GEMM for gfx950 (rlx-cpu quant.rs:
// lowp_scaled_matmul with its scale layouts, lowp_read_scales):
//
//   out[i, j] = sum_p a(i, p) * b(j, p)  (+ bias[j])
//   a(i, p) = decode(lhs[i, p]) * ls(i, p),  b(j, p) = decode(rhs[j, p]) * rs(j, p)
//
// with lhs [m, k] and rhs [n, k] one code per byte (rows K-last, TN), the
// scale of (row, p) per layout: per tensor one f32 per operand; MX one E8M0
// byte per 32 elements along K; NVFP4 one E4M3 byte per 16.
//
// Per tensor and MX run on gfx950's block-scaled matrix-core instruction
// v_mfma_scale_f32_16x16x128_f8f6f4: lane group b (lanes 16 b .. 16 b + 15,
// one per row) passes the E8M0 byte of K block b of its row, so the MX
// scales are applied inside the instruction (per tensor: unit scales, the
// product of the two f32 scales applied to the result).  NVFP4's E4M3 scales
// per 16 are not powers of two, which that instruction cannot take: there
// each element is decoded and multiplied by its scale into bf16 -- exact,
// since an element has at most 4 significant bits and an E4M3 scale 4 -- and
// the bf16 matrix-core instruction accumulates in fp32.
//
// Tiles: a workgroup of 4 or 8 waves (2 x 2 or 4 x 2) owns 128 x 128 or
// 256 x 128 outputs, each wave 64 x 64 as 4 x 4 MFMA tiles; per K-step of
// 128 every thread loads 16-byte pieces of each operand (16 codes of one
// row), packs them to the instruction's operand width (8, 6 or 4 bits per
// code; bf16 values for NVFP4) and stores them to LDS in fragment order:
// fragment (row tile t, K-group g, row r) -- the 32 elements lane 16 g + r of
// a wave reads -- so a wave's fragment read is one contiguous run.  LDS is
// double-buffered and the pieces are loaded into registers two steps ahead.
// Measured (m 2048, k 4096, n 14336): the MFMAs are not the bound (removing
// them changes the time by under 15 %); the byte-per-code operand loads and
// the pack-and-store into LDS are, behind one barrier per step.
#include <type_traits>

#include "lowp.h"
#include "mfma_ops.h"
#include "qmm_internal.h"

namespace qmm {

namespace {

constexpr int LT = 128;      // tile rows and columns
constexpr int LK = 128;      // K per step
constexpr int LTPB = 256;    // 4 waves
constexpr int LOWP_OOB = 0x7FFFFFF0;

// Output tile of workgroup b.  Workgroups are dispatched round robin over the
// 8 XCDs (b % 8), each with its own L2.  With the plain order (consecutive
// workgroups take consecutive M tiles of one N tile) every XCD keeps its
// rows of lhs in L2 but reads all of rhs through the fabric; when the grid
// splits evenly, XCD x instead owns M tiles of group x % 4 (a quarter of
// lhs) and N tiles of half x / 4 (half of rhs), walking its M tiles fastest,
// so its lhs rows stay in L2 and each rhs tile crosses the fabric to only 4
// XCDs: half the fabric traffic of the plain order.
__device__ __forceinline__ void lowp_tile(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  if ((tiles_m & 3) == 0 && (tiles_n & 1) == 0) {
    const int x = b & 7, q = b >> 3;
    const int gm = tiles_m >> 2;                   // M tiles per group
    tm = (x & 3) * gm + q % gm;
    tn = (x >> 2) * (tiles_n >> 1) + q / gm;
  } else {
    tm = b % tiles_m;
    tn = b / tiles_m;
  }
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// LDS bytes of one 32-element fragment: 32 (FP8; FP6 too, 24 used), 16 (FP4).
template <int F>
constexpr int slot_bytes() { return LowpFmt<F>::BITS == 4 ? 16 : 32; }

// 16 codes (one per byte) packed to the instruction's operand form: element
// j at bits [j * BITS, (j + 1) * BITS).
template <int F>
__device__ __forceinline__ void pack16(const u32x4 c, uint32_t* o) {
  constexpr int B = LowpFmt<F>::BITS;
  if constexpr (B == 8) {
    o[0] = c.x; o[1] = c.y; o[2] = c.z; o[3] = c.w;
  } else if constexpr (B == 4) {
    // (w & 0x0F0F0F0F) | (... >> 4): bytes 0 and 2 hold code pairs.
    auto pairs = [](uint32_t w) { w &= 0x0F0F0F0Fu; return w | (w >> 4); };
    o[0] = __builtin_amdgcn_perm(pairs(c.y), pairs(c.x), 0x06040200u);
    o[1] = __builtin_amdgcn_perm(pairs(c.w), pairs(c.z), 0x06040200u);
  } else {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = (w[j >> 2] >> (8 * (j & 3))) & 63u;
    o[0] = v[0] | (v[1] << 6) | (v[2] << 12) | (v[3] << 18) | (v[4] << 24) | (v[5] << 30);
    o[1] = (v[5] >> 2) | (v[6] << 4) | (v[7] << 10) | (v[8] << 16) | (v[9] << 22) | (v[10] << 28);
    o[2] = (v[10] >> 4) | (v[11] << 2) | (v[12] << 8) | (v[13] << 14) | (v[14] << 20) |
           (v[15] << 26);
  }
}

// 16 codes of row `row` at K offset kk (a multiple of 16); zeros past the
// row (k) or the matrix (rows).  VEC: k % 16 == 0 and a 16-byte aligned
// matrix, so a piece is wholly inside or wholly past a row; otherwise bytes.
template <bool VEC>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int row, int rows, int kk,
                                        int k) {
  if (row >= rows || kk >= k) return u32x4{0u, 0u, 0u, 0u};
  const int off = row * k + kk;
  if (VEC) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (kk + j < k) w[j >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, off + j, 0, 0) << (8 * (j & 3));
  return u32x4{w[0], w[1], w[2], w[3]};
}

// ---------------------------------------------------------------------------
// Per tensor (LAYOUT 0) and MX (LAYOUT 1): the block-scaled instruction.
// WM waves along M (2: 128-row tiles, 256 threads; 4: 256-row tiles, 512
// threads), 2 along N; each wave 64 x 64.  SS (MX with k % 128 == 0 and
// 4-byte aligned scales): a step's scale bytes -- 4 blocks of each tile row,
// one 32-bit word -- are loaded by one thread per row with the codes and
// staged in LDS beside them; otherwise each lane loads its bytes.
// ---------------------------------------------------------------------------
template <int LF, int RF, int LAYOUT, bool VEC, int WM, bool SS>
__global__ __launch_bounds__(128 * WM) void lowp_mfma_kernel(
    const uint8_t* __restrict__ lhs, const uint8_t* __restrict__ rhs,
    const void* __restrict__ lsc, const void* __restrict__ rsc, const float* __restrict__ bias,
    float* __restrict__ out, int m, int n, int k, int tiles_m) {
  constexpr int TPB = 128 * WM, LTM = 64 * WM;
  constexpr int RPP = TPB / 8;                      // tile rows per load pass
  constexpr int PA = LTM / RPP, PB = LT / RPP;      // passes: A, B
  constexpr int LS = slot_bytes<LF>(), RS = slot_bytes<RF>();
  constexpr int LST = LTM * LK / 32 * LS, RST = LT * LK / 32 * RS;   // stage bytes
  constexpr int SROWS = LTM + LT;                   // staged scale words per step
  constexpr int SW = (SROWS + TPB - 1) / TPB;       // scale words per thread
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_l[];
  uint8_t* As = lds_l;                              // [2][LST]
  uint8_t* Bs = lds_l + 2 * LST;                    // [2][RST]
  uint32_t* Ss = reinterpret_cast<uint32_t*>(lds_l + 2 * LST + 2 * RST);   // [2][SROWS]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tile_m, tile_n;
  lowp_tile(blockIdx.x, tiles_m, (int)gridDim.x / tiles_m, tile_m, tile_n);
  const int m0 = tile_m * LTM, n0 = tile_n * LT;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nblk = (k + 31) / 32;

  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)lhs, 0, m * k, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)rhs, 0, n * k, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rls = __builtin_amdgcn_make_buffer_rsrc(
      (void*)lsc, 0, LAYOUT == 1 ? m * nblk : 0, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)rsc, 0, LAYOUT == 1 ? n * nblk : 0, BUF_WORD3);

  // Thread t loads, in pass p, 16 codes of tile row RPP p + t / 8 at K
  // offset 16 c, c = t % 8.  The instruction's lane groups g = 0..3 hold, for
  // FP6 and FP4 operands, K 32 g .. 32 g + 31 (piece c: group c / 2, half
  // c % 2), and for FP8 operands K 16 g .. 16 g + 15 in their first four
  // registers and 64 + 16 g .. 64 + 16 g + 15 in the other four (piece c:
  // group c % 4, half c / 4).  Either way the block scale of K 32 b ..
  // 32 b + 31 is the one lane group b passes (measured on gfx950 with
  // one-hot operands).
  const int lrow = tid >> 3, lkk = (tid & 7) * 16;
  auto piece_slot = [&](int bits, int& g, int& half) {
    const int c = tid & 7;
    g = bits == 8 ? (c & 3) : (c >> 1);
    half = bits == 8 ? (c >> 2) : (c & 1);
  };
  // Two register stages (stage = step parity): the codes of step s + 2 are
  // loaded while step s multiplies and step s + 1 is packed into LDS.
  u32x4 pa[2][PA], pb[2][PB];
  uint32_t sw[2][SW];
  auto load = [&](int k0, int st) {
#pragma unroll
    for (int p = 0; p < PA; ++p) pa[st][p] = load16<VEC>(rl, m0 + RPP * p + lrow, m, k0 + lkk, k);
#pragma unroll
    for (int p = 0; p < PB; ++p) pb[st][p] = load16<VEC>(rh, n0 + RPP * p + lrow, n, k0 + lkk, k);
    if constexpr (SS) {
#pragma unroll
      for (int i = 0; i < SW; ++i) {
        const int r = tid + i * TPB;
        const bool isa = r < LTM;
        const int row = isa ? m0 + r : n0 + r - LTM;
        const bool ok = r < SROWS && row < (isa ? m : n);
        const int off = ok ? row * nblk + k0 / 32 : LOWP_OOB;
        sw[st][i] = isa ? __builtin_amdgcn_raw_buffer_load_b32(rls, off, 0, 0)
                        : __builtin_amdgcn_raw_buffer_load_b32(rrs, off, 0, 0);
      }
    }
  };
  // LDS fragment slots, swizzled against bank conflicts (these accesses see
  // 32 banks of 4 bytes, as measured): the entry of (row r of a 16-row tile,
  // lane group g) is 16 g + (r ^ swz(g)), swz(g) = 2 g for 16-byte slots and
  // g for 32-byte ones, so that the four groups of one row (stored by
  // adjacent threads) land in different banks; a 32-byte slot of a row with bit 3 set holds its
  // two 16-byte halves swapped, so that the two reads of a fragment (16 bytes
  // at a 32-byte stride) spread lanes l and l + 8 over different banks.  The
  // reads see each 16-lane group's entries permuted within their 256 or 512
  // bytes.
  auto put = [&](uint8_t* base, int slot, int bits, int row, int g, int half, const uint32_t* o) {
    const int r = row & 15;
    const int swz = slot == 16 ? 2 * g : g;
    const int e = ((row >> 4) * 4 + g) * 16 + (r ^ swz);
    uint32_t* d = reinterpret_cast<uint32_t*>(base + e * slot);
    const int hs = (slot == 32 && (r & 8)) ? 4 : 0;
    if (bits == 8) {
      // A whole 16-byte half: one store.
      *reinterpret_cast<u32x4*>(d + ((4 * half) ^ hs)) = u32x4{o[0], o[1], o[2], o[3]};
    } else if (bits == 4) {
      *reinterpret_cast<u32x2*>(d + 2 * half) = u32x2{o[0], o[1]};
    } else {
#pragma unroll
      for (int j = 0; j < 3; ++j) d[(half * 3 + j) ^ hs] = o[j];
    }
  };
  auto store = [&](int buf, int st) {
    int g, half;
#pragma unroll
    for (int p = 0; p < PA; ++p) {
      const int row = RPP * p + lrow;
      piece_slot(LowpFmt<LF>::BITS, g, half);
      uint32_t o[4];
      pack16<LF>(pa[st][p], o);
      put(As + buf * LST, LS, LowpFmt<LF>::BITS, row, g, half, o);
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int row = RPP * p + lrow;
      piece_slot(LowpFmt<RF>::BITS, g, half);
      uint32_t o[4];
      pack16<RF>(pb[st][p], o);
      put(Bs + buf * RST, RS, LowpFmt<RF>::BITS, row, g, half, o);
    }
    if constexpr (SS) {
#pragma unroll
      for (int i = 0; i < SW; ++i)
        if (tid + i * TPB < SROWS) Ss[buf * SROWS + tid + i * TPB] = sw[st][i];
    }
  };
  // Without staging: the E8M0 byte of this lane's block for row tile i of
  // the wave (127, a unit scale, per tensor and past the last block).
  uint32_t sa[2][4], sb[2][4];
  auto load_scales = [&](int k0, int st) {
    const int blk = k0 / 32 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (LAYOUT == 1 && !SS) {
        const int ra = m0 + wm + 16 * i + (lane & 15), rb = n0 + wn + 16 * i + (lane & 15);
        sa[st][i] = blk < nblk ? __builtin_amdgcn_raw_buffer_load_b8(rls, ra < m ? ra * nblk + blk : LOWP_OOB, 0, 0)
                               : 127u;
        sb[st][i] = blk < nblk ? __builtin_amdgcn_raw_buffer_load_b8(rrs, rb < n ? rb * nblk + blk : LOWP_OOB, 0, 0)
                               : 127u;
      } else {
        sa[st][i] = 127u;
        sb[st][i] = 127u;
      }
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto frag = [&](const uint8_t* base, int slot, int tile) {
    // Fragment (tile, lane): 16, 24 or 32 bytes of the lane's swizzled entry
    // (see put).
    const int g = lane >> 4, r = lane & 15;
    const int e = tile * 64 + g * 16 + (r ^ (slot == 16 ? 2 * g : g));
    const uint8_t* p = base + e * slot;
    const int hs = (slot == 32 && (r & 8)) ? 16 : 0;
    v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
    const u32x4 lo = *reinterpret_cast<const u32x4*>(p + hs);
    v[0] = (int)lo.x; v[1] = (int)lo.y; v[2] = (int)lo.z; v[3] = (int)lo.w;
    if (slot == 32) {
      const u32x4 hi = *reinterpret_cast<const u32x4*>(p + (16 - hs));
      v[4] = (int)hi.x; v[5] = (int)hi.y; v[6] = (int)hi.z; v[7] = (int)hi.w;
    }
    return v;
  };

  const int nsteps = (k + LK - 1) / LK;
  // Step s (register stage and LDS buffer s & 1 = ST): load step s + 2 into
  // stage ST, multiply buffer ST, pack stage ST ^ 1 (step s + 1) into buffer
  // ST ^ 1.  Loads past the last step read nothing (zero pieces).
  auto step = [&](int s, auto st_tag) {
    constexpr int ST = decltype(st_tag)::value;
    uint32_t csa[4], csb[4];
    if constexpr (SS) {
      const int sh = 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        csa[i] = Ss[ST * SROWS + wm + 16 * i + (lane & 15)] >> sh;
        csb[i] = Ss[ST * SROWS + LTM + wn + 16 * i + (lane & 15)] >> sh;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) { csa[i] = sa[ST][i]; csb[i] = sb[ST][i]; }
    }
    if (s + 2 < nsteps) {
      load((s + 2) * LK, ST);
      load_scales((s + 2) * LK, ST);
    }
    v8i b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = frag(Bs + ST * RST, RS, (wn >> 4) + j);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const v8i a = frag(As + ST * LST, LS, (wm >> 4) + i);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            a, b[j], acc[i][j], LF, RF, 0, (int)csa[i], 0, (int)csb[j]);
    }
    if (s + 1 < nsteps) store(ST ^ 1, ST ^ 1);
    __syncthreads();
  };
  load(0, 0);
  load_scales(0, 0);
  if (nsteps > 1) {
    load(LK, 1);
    load_scales(LK, 1);
  }
  store(0, 0);
  __syncthreads();
  for (int s = 0; s < nsteps; s += 2) {
    step(s, std::integral_constant<int, 0>{});
    if (s + 1 < nsteps) step(s + 1, std::integral_constant<int, 1>{});
  }

  // Per tensor: the product of the two f32 scales.
  float ps = 1.0f;
  if constexpr (LAYOUT == 0) ps = reinterpret_cast<const float*>(lsc)[0] * reinterpret_cast<const float*>(rsc)[0];
  const int cc = lane & 15, rr = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn + 16 * j + cc;
    if (col >= n) continue;
    const float bv = bias ? bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + 16 * i + rr + e;
        if (row < m) out[(int64_t)row * n + col] = (LAYOUT == 0 ? acc[i][j][e] * ps : acc[i][j][e]) + bv;
      }
  }
}

// ---------------------------------------------------------------------------
// NVFP4 (LAYOUT 2): elements times their E4M3 scales into bf16 (exact), then
// v_mfma_f32_16x16x32_bf16.  LDS fragment (K-sub-step ks of 32, row tile t,
// group g of 8, row r): 16 bytes at (((ks * 8 + t) * 4 + g) * 16 + r) * 16.
// ---------------------------------------------------------------------------
template <int LF, int RF, bool VEC>
__global__ __launch_bounds__(LTPB) void lowp_nvfp4_kernel(
    const uint8_t* __restrict__ lhs, const uint8_t* __restrict__ rhs,
    const uint8_t* __restrict__ lsc, const uint8_t* __restrict__ rsc,
    const float* __restrict__ bias, float* __restrict__ out, int m, int n, int k, int tiles_m) {
  constexpr int ST = LT * LK * 2;         // one operand stage (bf16)
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_n[];
  uint8_t* As = lds_n;
  uint8_t* Bs = lds_n + 2 * ST;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tile_m, tile_n;
  lowp_tile(blockIdx.x, tiles_m, (int)gridDim.x / tiles_m, tile_m, tile_n);
  const int m0 = tile_m * LT, n0 = tile_n * LT;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
  const int nblk = (k + 15) / 16;

  const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc((void*)lhs, 0, m * k, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc((void*)rhs, 0, n * k, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rls = __builtin_amdgcn_make_buffer_rsrc((void*)lsc, 0, m * nblk, BUF_WORD3);
  const __amdgpu_buffer_rsrc_t rrs = __builtin_amdgcn_make_buffer_rsrc((void*)rsc, 0, n * nblk, BUF_WORD3);

  const int lrow = tid >> 3, lkk = (tid & 7) * 16;
  // This lane's swizzled fragment entry in K sub-step ks (see put).
  auto lsw = [&](int ks) { return (lane & 48) | ((lane & 15) ^ (2 * ks + ((lane >> 5) & 1))); };
  u32x4 pa[4], pb[4];
  uint32_t qa[4], qb[4];                  // the pieces' E4M3 scale bytes
  auto load = [&](int k0) {
    const int blk = (k0 + lkk) / 16;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int ra = m0 + 32 * p + lrow, rb = n0 + 32 * p + lrow;
      pa[p] = load16<VEC>(rl, ra, m, k0 + lkk, k);
      pb[p] = load16<VEC>(rh, rb, n, k0 + lkk, k);
      // Past the last block: 0x38 (1.0), meeting zero codes.
      qa[p] = blk < nblk ? __builtin_amdgcn_raw_buffer_load_b8(rls, ra < m ? ra * nblk + blk : LOWP_OOB, 0, 0) : 0x38u;
      qb[p] = blk < nblk ? __builtin_amdgcn_raw_buffer_load_b8(rrs, rb < n ? rb * nblk + blk : LOWP_OOB, 0, 0) : 0x38u;
    }
  };
  auto put = [&](uint8_t* st, u32x4 c, uint32_t q, int row, auto fmt_tag) {
    constexpr int F = decltype(fmt_tag)::value;
    const float s = lowp_decode<0>(q);
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t pk[8];
    // Exact products: the upper halves of their binary32 values are bf16.
    auto two = [&](int j, f32x2 v) {
      pk[j / 2] = (__float_as_uint(v.x * s) >> 16) | (__float_as_uint(v.y * s) & 0xFFFF0000u);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // Codes 4 i .. 4 i + 3 as exact binary32 values: gfx950's conversions
      // with a unit scale (FP8: two bytes of the word per instruction; FP4:
      // the code pairs first packed into bytes 0 and 2), else bit decoding.
      if constexpr (F == 0 || F == 1) {
        const uint32_t x = w[i];
        two(4 * i, F == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, false)
                          : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(x, 1.0f, false));
        two(4 * i + 2, F == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(x, 1.0f, true)
                              : __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(x, 1.0f, true));
      } else if constexpr (F == 4) {
        uint32_t x = w[i] & 0x0F0F0F0Fu;
        x |= x >> 4;
        two(4 * i, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 0));
        two(4 * i + 2, __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(x, 1.0f, 2));
      } else {
#pragma unroll
        for (int j = 0; j < 4; j += 2)
          two(4 * i + j, f32x2{lowp_decode<F>(w[i] >> (8 * j)), lowp_decode<F>(w[i] >> (8 * (j + 1)))});
      }
    }
    // Fragment entry (row r, lane group g) of K sub-step ks at
    // 16 g + (r ^ (2 ks + g / 2)): the eight pieces of a row, stored by
    // adjacent threads, then fall in eight different banks of the 32 these
    // accesses see (reads permute within a group's 256 bytes).
    const int ks = lkk / 32, g0 = (lkk & 31) / 8;
    const int t = row >> 4, r = (row & 15) ^ (2 * ks + g0 / 2);
    u32x4* d0 = reinterpret_cast<u32x4*>(st + ((((ks * 8 + t) * 4 + g0) * 16 + r) * 16));
    u32x4* d1 = reinterpret_cast<u32x4*>(st + ((((ks * 8 + t) * 4 + g0 + 1) * 16 + r) * 16));
    *d0 = u32x4{pk[0], pk[1], pk[2], pk[3]};
    *d1 = u32x4{pk[4], pk[5], pk[6], pk[7]};
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      put(As + buf * ST, pa[p], qa[p], 32 * p + lrow, std::integral_constant<int, LF>{});
      put(Bs + buf * ST, pb[p], qb[p], 32 * p + lrow, std::integral_constant<int, RF>{});
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = (k + LK - 1) / LK;
  load(0);
  store(0);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load((s + 1) * LK);
    const uint8_t* as = As + buf * ST;
    const uint8_t* bs = Bs + buf * ST;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8_t b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                bs + ((ks * 8 + (wn >> 4) + j) * 64 + lsw(ks)) * 16));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4*>(
                                                            as + ((ks * 8 + (wm >> 4) + i) * 64 + lsw(ks)) * 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[i][j], 0, 0, 0);
      }
    }
    if (s + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  const int cc = lane & 15, rr = (lane >> 4) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = n0 + wn + 16 * j + cc;
    if (col >= n) continue;
    const float bv = bias ? bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm + 16 * i + rr + e;
        if (row < m) out[(int64_t)row * n + col] = acc[i][j][e] + bv;
      }
  }
}

template <int LF, int RF>
hipError_t launch_pair(const LowpArgs& a) {
  const int tiles_m = (int)((a.m + LT - 1) / LT), tiles_n = (int)((a.n + LT - 1) / LT);
  const bool vec = (a.k % 16) == 0 && ((uintptr_t)a.lhs & 15) == 0 && ((uintptr_t)a.rhs & 15) == 0;
  const dim3 grid(tiles_m * tiles_n), block(LTPB);
  if (a.layout == 2) {
    const size_t lds = 4 * (size_t)LT * LK * 2;
    auto kern = vec ? lowp_nvfp4_kernel<LF, RF, true> : lowp_nvfp4_kernel<LF, RF, false>;
    const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, block, lds, a.stream, a.lhs, a.rhs, (const uint8_t*)a.lsc,
                       (const uint8_t*)a.rsc, a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, tiles_m);
    return hipGetLastError();
  }
  // 256-row tiles when their grid still fills the chip, else 128.
  const int tiles_m4 = (int)((a.m + 255) / 256);
  const bool wide = (int64_t)tiles_m4 * tiles_n >= 256;
  const bool ss = a.layout == 1 && (a.k % 128) == 0 && ((uintptr_t)a.lsc & 3) == 0 &&
                  ((uintptr_t)a.rsc & 3) == 0;
  auto go = [&](auto wm_tag, auto ss_tag) {
    constexpr int WM = decltype(wm_tag)::value;
    constexpr bool SS = decltype(ss_tag)::value;
    const int tm = WM == 4 ? tiles_m4 : tiles_m;
    const size_t lds = 2 * (size_t)LK / 32 * (64 * WM * slot_bytes<LF>() + LT * slot_bytes<RF>()) +
                       (SS ? 2 * (size_t)(64 * WM + LT) * 4 : 0);
    decltype(&lowp_mfma_kernel<LF, RF, 0, true, WM, SS>) kern;
    if constexpr (WM == 2 && !SS) {
      // The byte-load fallback (k % 16 != 0 or unaligned codes) only here.
      if (a.layout == 0) kern = vec ? lowp_mfma_kernel<LF, RF, 0, true, 2, false> : lowp_mfma_kernel<LF, RF, 0, false, 2, false>;
      else kern = vec ? lowp_mfma_kernel<LF, RF, 1, true, 2, false> : lowp_mfma_kernel<LF, RF, 1, false, 2, false>;
    } else {
      kern = a.layout == 0 ? lowp_mfma_kernel<LF, RF, 0, true, WM, SS> : lowp_mfma_kernel<LF, RF, 1, true, WM, SS>;
    }
    const hipError_t e = ensure_dynamic_lds((const void*)kern, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(tm * tiles_n), dim3(128 * WM), lds, a.stream, a.lhs, a.rhs, a.lsc,
                       a.rsc, a.bias, a.out, (int)a.m, (int)a.n, (int)a.k, tm);
    return hipGetLastError();
  };
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (!vec) return go(I2{}, std::false_type{});
  if (wide) return ss ? go(I4{}, std::true_type{}) : go(I4{}, std::false_type{});
  return ss ? go(I2{}, std::true_type{}) : go(I2{}, std::false_type{});
}

template <int LF>
hipError_t launch_lf(const LowpArgs& a) {
  switch (a.rfmt) {
    case 0: return launch_pair<LF, 0>(a);
    case 1: return launch_pair<LF, 1>(a);
    case 2: return launch_pair<LF, 2>(a);
    case 3: return launch_pair<LF, 3>(a);
    default: return launch_pair<LF, 4>(a);
  }
}

}  // namespace

hipError_t launch_lowp_matmul(const LowpArgs& a) {
  switch (a.lfmt) {
    case 0: return launch_lf<0>(a);
    case 1: return launch_lf<1>(a);
    case 2: return launch_lf<2>(a);
    case 3: return launch_lf<3>(a);
    default: return launch_lf<4>(a);
  }
}

}  // namespace qmm
