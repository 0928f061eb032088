// fa_varlen_tiling.h -- index arithmetic of the forward kernels' tiles.
//
// Compiles as HIP device code (used by fa_varlen_kernels.hip) and as plain
// host C++ (used by tests/host/check_tiling.cpp, which enumerates every
// thread's global offsets and LDS indices and checks them against the
// buffers they address).  No HIP headers are needed here.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define FA_HD __host__ __device__ __forceinline__
#else
#define FA_HD inline
#endif

namespace fa {
namespace tiling {

// Accumulator row R of the 32x32 MFMA layout lives in register 4*(R/8) + R%4
// of lane half (R/4)%2.  Feeding key pi(R) = 16*((R/4)%2) + 4*(R/8) + R%4 into
// A-operand row R makes register r of lane half g hold key 16g + r.
FA_HD int key_of_arow(int R) { return ((R >> 2) & 1) * 16 + (R >> 3) * 4 + (R & 3); }

// XOR swizzles of 16-byte chunks so that the MFMA operand reads from LDS hit
// distinct banks within each group of 8 and of 16 lanes.
//   K rows (D 16-bit elements per key row): the chunk index is XORed with bits of the row.
//   V^T rows (BN elements per dimension): the chunk index is XORed with bits of d.
//   A row of 256 elements spans the 64 banks twice, so its chunks fall on the
//   same bank groups as those of a 128-element row and it uses the same swizzle
//   (which only touches the low 4 bits of the chunk index).
template <int D>
FA_HD int k_swz(int row) {
  if constexpr (D == 128 || D == 256) return (row & 3) | ((row >> 2) & 4) | ((row << 1) & 8);
  else return ((row ^ (row >> 2)) & 1) | (row & 2) | ((row >> 2) & 4);
}
template <int BN>
FA_HD int v_swz(int d) {
  if constexpr (BN == 128) return d & 15;
  else if constexpr (BN == 32) return (d >> 2) & 3;
  else return ((d >> 1) & 3) | (((d ^ (d >> 3)) & 1) << 2);
}

// Elements per K row in LDS: head_dim 96 rows (12 chunks) are kept in slots of
// 128 elements so that they use the 16-chunk swizzle of head_dim 128 (the
// last 4 chunks of a slot stay unused).
template <int D>
constexpr int k_stride() { return D == 96 ? 128 : D; }

// LDS element index of K chunk `ch` of key row `row` (8 consecutive elements), and
// of key `key` of dimension `d` in V^T (keys 8*(key/8) .. +7 are contiguous).
template <int D>
FA_HD int ks_index(int row, int ch) {
  constexpr int KS = k_stride<D>();
  return row * KS + 8 * (ch ^ k_swz<KS>(row));
}
template <int BN>
FA_HD int vt_index(int d, int key) { return d * BN + 8 * ((key >> 3) ^ v_swz<BN>(d)) + (key & 7); }

// Row-major V tiles ([BN keys][k_stride<D>()], read by transposing LDS reads):
// a transposing read of a 16-lane group covers rows r0..r0+3 (r0 a multiple
// of 4) and two adjacent 16-byte chunks, and the two groups of a 32-lane half
// cover the next two chunks of the same rows (a quad of 4 chunks).  The
// swizzle puts those 4 rows x 4 chunks on 16 distinct 16-byte bank groups:
// rows of 16 or more chunks XOR the chunk index with 4 * (row % 4); rows of 8
// chunks (head_dim 64) share a bank cycle in pairs, so rows r and r+2 take
// opposite quads (XOR with 4 * ((row / 2) % 2)).
template <int D>
FA_HD int vrow_swz(int row) {
  if constexpr (D == 64) return 4 * ((row >> 1) & 1);
  else return 4 * (row & 3);
}
template <int D>
FA_HD int vr_index(int row, int ch) { return row * k_stride<D>() + 8 * (ch ^ vrow_swz<D>(row)); }

// Direct global -> LDS tile loads (16 bytes per lane, lane-consecutive in
// LDS): LDS 16-byte slot p of a [rows][k_stride<D>()] tile receives logical
// chunk `ch` of tile row `row` of the K-style (V_LAYOUT false: ks_index) or
// row-major V (V_LAYOUT true: vr_index) layout.  At head_dim 96 the last 4
// slots of a 128-element row hold no chunk; they are given a chunk of the same
// row (in range, never read).
template <int D, bool V_LAYOUT>
FA_HD void direct_slot_chunk(int p, int& row, int& ch) {
  constexpr int CPR = k_stride<D>() / 8;
  row = p / CPR;
  ch = (p % CPR) ^ (V_LAYOUT ? vrow_swz<D>(row) : k_swz<k_stride<D>()>(row));
  if (D == 96 && ch >= D / 8) ch -= 8;
}

// Element index, in a row-major V tile, of lane `lane`'s transposing read of
// tile rows r0 .. r0+3 (r0 a multiple of 4) for output dimension block db:
// within each 16-lane group, lane i reads row r0 + i/4, dimensions
// c0 + 4(i%4) .. +3 with c0 = 32 db + 16 ((lane/16) % 2), and receives
// dimension c0 + i (= 32 db + lane % 32) of rows r0 .. r0+3.
template <int D>
FA_HD int vr_tr_index(int lane, int r0, int db) {
  const int i = lane & 15;
  const int row = r0 + (i >> 2);
  const int ch = 4 * db + 2 * ((lane >> 4) & 1) + ((i >> 1) & 1);
  return row * k_stride<D>() + 8 * (ch ^ vrow_swz<D>(row)) + 4 * (i & 1);
}

// Byte extent, from the first element of one head's slice of a row, of that
// head's slices in `rows` consecutive token rows: the last byte is the end of
// the last row's slice, so nothing past the tensor is ever in range.
FA_HD uint32_t head_rows_bytes(int rows, int64_t row_stride, int head_dim, int esize) {
  return rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * row_stride + head_dim) * esize) : 0u;
}

// 16-bit (bf16 or fp16) tiles: K tile [BN keys][D], staged as 16-byte chunks (8 elements); V tile
// staged as units of 4 consecutive keys x 8 consecutive dims and written to
// LDS transposed (V^T, [D][BN]).
template <int D, int BN, int NW>
struct Geom16 {
  static constexpr int THREADS = NW * 64;
  static constexpr int K_CHUNKS = BN * D / 8;
  static constexpr int K_PER_THREAD = K_CHUNKS / THREADS;
  static constexpr int V_UNITS = (BN / 4) * (D / 8);
  static constexpr int V_PER_THREAD = (V_UNITS + THREADS - 1) / THREADS;
  static constexpr bool V_GUARD = (V_UNITS % THREADS) != 0;  // some threads own no unit
  static constexpr int LDS_K = BN * k_stride<D>();           // elements per K buffer
  static constexpr int LDS_V = D * BN;                       // elements per V^T buffer
  static_assert(K_CHUNKS % THREADS == 0, "K tile/threads mismatch");
  static_assert(!V_GUARD || V_PER_THREAD == 1, "V units must fill the threads evenly or cover a prefix");
  static_assert((D / 8) % 4 == 0, "V unit mapping needs D/8 divisible by 4");
  static_assert(BN % 32 == 0 && D % 32 == 0, "32x32 MFMA blocks");

  // K chunk c (c = tid + i*THREADS): key row in the tile, 16-byte chunk in the row
  static FA_HD int k_row(int c) { return c / (D / 8); }
  static FA_HD int k_chunk(int c) { return c % (D / 8); }
  // V unit w: keys 4*v_group .. +3, dims 8*v_dchunk .. +7.  Four consecutive
  // units share a key group and cover 64 contiguous bytes of a row.
  static FA_HD bool v_owned(int w) { return !V_GUARD || w < V_UNITS; }
  static FA_HD int v_group(int w) { return (w >> 2) % (BN / 4); }
  static FA_HD int v_dchunk(int w) { return ((w >> 2) / (BN / 4)) * 4 + (w & 3); }
  static FA_HD int ks_index(int row, int ch) { return tiling::ks_index<D>(row, ch); }
  static FA_HD int vt_index(int d, int key) { return tiling::vt_index<BN>(d, key); }
};

// fp32 tiles: K and V both [BN keys][D + 4] in LDS (padded rows), staged as
// float4 chunks.
template <int D, int NW>
struct F32Geom {
  static constexpr int BN = 32;
  static constexpr int THREADS = NW * 64;
  static constexpr int LD = D + 4;
  static constexpr int CHUNKS = BN * D / 4;
  static constexpr int PER_THREAD = CHUNKS / THREADS;
  static constexpr int LDS_ELEMS = BN * LD;
  static_assert(CHUNKS % THREADS == 0, "tile/threads mismatch");
  static FA_HD int row(int c) { return c / (D / 4); }
  static FA_HD int chunk(int c) { return c % (D / 4); }
  // accumulator register r of lane half g holds key 8*(r/4) + 4g + r%4
  static FA_HD int key_of_reg(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }
};

}  // namespace tiling
}  // namespace fa
