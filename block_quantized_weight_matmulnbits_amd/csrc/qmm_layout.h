// qmm_layout.h -- the tiled weight layout produced by qmm_repack (host and
// device).  A one-time byte permutation of the MatMulNBits tensors (codes
// B[N, kb, bs*bits/8], scales [N, kb], packed zero points) that makes every
// wave-wide load of the GEMV and the GEMM contiguous.
//
// Columns (output features n) form groups of TG = 32; K is cut into chunks of
// TKC = 64 codes (chunk c holds codes k in [64c, 64c + 64) of every column,
// zero codes past the row's last block).  Three regions, each starting on a
// 256-byte boundary:
//   codes  [group][chunk][column in group][64 * bits / 8 bytes]
//          (a column's 64 codes in k order, least-significant bits first,
//           exactly the bytes of the operator's row)
//   scales [group][block][column in group]           (scale dtype)
//   zps    [group][block][column in group]  packed LSB first, bits per entry
//          (present only for the zero-point variant of the layout)
// Columns past N (the last group's padding) hold zero codes, zero scales and
// zero zero points.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qmm {

constexpr int TG = 32;    // columns per group
constexpr int TKC = 64;   // codes per chunk

struct TiledGeom {
  int64_t groups = 0, chunks = 0, kb = 0;
  int64_t chunk_bytes = 0;        // bytes of one column's chunk: 64 * bits / 8
  int64_t codes_off = 0, codes_bytes = 0;
  int64_t scales_off = 0, scales_bytes = 0;
  int64_t zps_off = 0, zps_bytes = 0;
  int64_t total = 0;
};

inline int64_t tiled_align(int64_t v) { return (v + 255) / 256 * 256; }

inline TiledGeom tiled_geom(int64_t K, int64_t N, int64_t bs, int bits, int scale_bytes,
                            bool has_zp) {
  TiledGeom g;
  g.kb = (K + bs - 1) / bs;
  g.groups = (N + TG - 1) / TG;
  g.chunks = (g.kb * bs + TKC - 1) / TKC;
  g.chunk_bytes = (int64_t)TKC * bits / 8;
  g.codes_off = 0;
  g.codes_bytes = g.groups * g.chunks * TG * g.chunk_bytes;
  g.scales_off = tiled_align(g.codes_off + g.codes_bytes);
  g.scales_bytes = g.groups * g.kb * TG * scale_bytes;
  g.zps_off = tiled_align(g.scales_off + g.scales_bytes);
  g.zps_bytes = has_zp ? g.groups * g.kb * TG * bits / 8 : 0;
  g.total = tiled_align(g.zps_off + g.zps_bytes);
  return g;
}

}  // namespace qmm
