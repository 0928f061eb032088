// fa_varlen_bwd_tiling.h -- LDS byte addresses of the 256-key backward
// workgroup (bwd16w_kernel in fa_varlen_bwd.hip).
//
// Compiles as HIP device code and as plain host C++: tests/host/check_tiling.cpp
// checks every formula below against the element-index form it replaces, for
// every lane and loop index.
//
// Each address a kernel reads or writes in its main loop splits into three
// parts: a lane part (one register per access pattern, computed once), a
// 16-byte-chunk XOR that depends only on loop indices, and a byte offset
// that depends only on loop indices.  The XOR swizzles of these tiles act on
// the chunk index (bits 4-7 of a 256-byte row, 4-8 of a 512-byte row) as
// linear maps of row bits, and the loop indices and the lane supply disjoint
// bits of the row and the chunk, so
//     address = (lane part XOR chunk term) + row term,
// and a read costs one XOR (shared between tiles of one layout) plus an
// immediate offset, instead of re-deriving row, chunk and swizzle per read.
#pragma once

#include "fa_varlen_tiling.h"

namespace fa {
namespace bwdt {

// Layout of the Q, dO and K tiles of the backward pass: read both with
// 16-byte operand reads and with transposing reads.  The operand reads of a
// 16-lane group take one chunk of rows {0-3, 16-19, 4-7, 20-23} (+8): the
// chunk index is XORed with two low bits that differ across those four row
// sets (row bit 2, and row bits 3 and 4 combined).  A transposing read of a
// 32-lane half takes rows r..r+3 (r a multiple of 4) and a quad of four
// chunks, or, for K^T, rows r..r+3 and r+8..r+11 and a pair of chunks: the
// quad bits are XORed with row % 4 and the low bits flip between r and r+8,
// so either read touches 16 distinct 16-byte bank groups.  Rows of head_dim
// 64 keep the K-style layout.  Rows of head_dim 96 (12 chunks) sit in
// 128-element slots and take the head_dim-128 swizzle; the slots' last four
// chunk positions hold no data.
template <int D>
FA_HD int tq_swz(int row) {
  if constexpr (D == 128 || D == 96) return 4 * (row & 3) | ((row >> 2) & 1) | ((((row >> 3) ^ (row >> 4)) & 1) << 1);
  else return tiling::k_swz<D>(row);
}
template <int D>
FA_HD int tq_index(int row, int ch) {
  return row * tiling::k_stride<D>() + 8 * (ch ^ tq_swz<D>(row));
}

template <int D>
constexpr int row_bytes() { return 2 * tiling::k_stride<D>(); }

// --- 16-byte operand reads (S = Q K^T, dP = dO V^T): row `row` (the lane's),
// chunk 2 ks + g of the Q / dO tiles (tq layout) or of the V tile (K-style
// layout).  The lane part is the address at ks = 0.
template <int D>
FA_HD uint32_t op_lane_tq(int row, int g) { return (uint32_t)(2 * tq_index<D>(row, g)); }
template <int D>
FA_HD uint32_t op_lane_ks(int row, int g) { return (uint32_t)(2 * tiling::ks_index<D>(row, g)); }
FA_HD uint32_t op_xor(int ks) { return 32u * (uint32_t)ks; }

// --- transposing reads of dV^T += dO^T P and dK^T += Q^T dS: within each
// 16-lane group (lane i = li, group lg = lane / 16) lane i reads row
// r0 + i/4, columns c0 + 4(i%4) .. +3 with r0 = 16 (lg / 2) + 8 t + 4 h and
// c0 = 32 db + 16 (lg % 2) (h: the lower or upper four of the eight rows).
template <int D>
FA_HD uint32_t trq_orig(int li, int lg, int db, int t, int h) {
  const int row = 16 * (lg >> 1) + 8 * t + 4 * h + (li >> 2);
  const int col = 32 * db + 16 * (lg & 1) + 4 * (li & 3);
  return (uint32_t)(2 * (tq_index<D>(row, col >> 3) + (col & 7)));
}
template <int D>
FA_HD uint32_t trq_lane(int li, int lg) { return trq_orig<D>(li, lg, 0, 0, 0); }
template <int D>
FA_HD uint32_t trq_xor(int db, int t, int h) {
  // chunk bits 2-3 from db; the swizzle adds h (row bit 2) and, at 96 and
  // 128, t (row bit 3) in bit 1
  return 16u * (uint32_t)(4 * db ^ h ^ ((D == 64 ? 0 : 2) * t));
}
template <int D>
FA_HD uint32_t trq_add(int t, int h) { return (uint32_t)((8 * t + 4 * h) * row_bytes<D>()); }

// --- transposing reads of K^T for dQ: rows r0 + i/4 with r0 = 32 kk + 8 lg + 4 h,
// columns 16 ct + 4(i%4) .. +3 (ct: the wave's 16-column tile).
template <int D>
FA_HD uint32_t trk_orig(int li, int lg, int kk, int ct, int h) {
  const int row = 32 * kk + 8 * lg + 4 * h + (li >> 2);
  const int col = 16 * ct + 4 * (li & 3);
  return (uint32_t)(2 * (tq_index<D>(row, col >> 3) + (col & 7)));
}
template <int D>
FA_HD uint32_t trk_lane(int li, int lg) { return trk_orig<D>(li, lg, 0, 0, 0); }
FA_HD uint32_t trk_xor(int ct, int h) { return 16u * (uint32_t)(2 * ct ^ h); }
template <int D>
FA_HD uint32_t trk_add(int kk, int h) { return (uint32_t)((32 * kk + 4 * h) * row_bytes<D>()); }

// --- dS tile (row-major [32 rows][256 keys], K-style swizzle of 256-element
// rows).  dQ reads its A operand at row dq_row(rt, li) (row tile rt of 16
// rows: rows 8 rt .. +7 and 16 + 8 rt .. +7), chunk 4 kk + lg.
FA_HD int dq_row(int rt, int i) { return (i < 8 ? 0 : 8) + 8 * rt + i; }
FA_HD uint32_t dsa_orig(int li, int lg, int kk, int rt) {
  return (uint32_t)(2 * tiling::ks_index<256>(dq_row(rt, li), 4 * kk + lg));
}
FA_HD uint32_t dsa_lane(int li, int lg) { return dsa_orig(li, lg, 0, 0); }
FA_HD uint32_t dsa_xor(int kk) { return 64u * (uint32_t)kk; }
FA_HD uint32_t dsa_add(int rt) { return (uint32_t)(8 * rt * 512); }

// dS stores: lane half g, register r holds row 16 g + r of the lane's key `key`.
FA_HD uint32_t dss_orig(int key, int g, int r) {
  return (uint32_t)(2 * (tiling::ks_index<256>(16 * g + r, key >> 3) + (key & 7)));
}
FA_HD uint32_t dss_lane(int key, int g) { return dss_orig(key, g, 0); }
FA_HD uint32_t dss_xor(int r) { return 16u * (uint32_t)((r & 3) | (((r >> 2) & 1) << 3)); }
FA_HD uint32_t dss_add(int r) { return (uint32_t)(r * 512); }

}  // namespace bwdt
}  // namespace fa
