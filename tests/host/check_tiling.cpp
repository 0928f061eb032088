// check_tiling.cpp -- host-side bounds and consistency check of the forward
// kernels' index arithmetic (fa_varlen_tiling.h, and the backward's
// fa_varlen_bwd_tiling.h), built with g++ by
// tests/test_host_tiling.py.  For every thread of a workgroup it enumerates:
//   * the byte offsets of the K/V/Q buffer loads against the resource extents,
//     under a conservative model of the hardware range check (a load whose
//     offset is below the extent is taken to touch all of its 16 bytes): every
//     such access must lie inside a valid token row's slice of the current
//     head, and every valid element must be loaded exactly once;
//   * the LDS indices written by the K/V staging and read as MFMA operands:
//     inside the buffers, aligned, every tile element written exactly once,
//     and each operand read returning the keys/dimensions the MFMA expects;
//   * the output-store offsets of the epilogue.
// Prints a line per configuration and exits non-zero on any violation.
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "fa_varlen_tiling.h"
#include "fa_varlen_bwd_tiling.h"

using namespace fa::tiling;

static int g_fail = 0;
#define CHECK(cond, ...)                                 \
  do {                                                   \
    if (!(cond)) {                                       \
      if (g_fail < 30) {                                 \
        std::fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        std::fprintf(stderr, __VA_ARGS__);               \
        std::fprintf(stderr, "\n");                      \
      }                                                  \
      ++g_fail;                                          \
    }                                                    \
  } while (0)

// A packed tensor [T, H, D] of elements; a resource starting at the head-h
// slice of row `row0` with extent `bytes`; a 16-byte load at byte `off`.
struct Access {
  long T, H, D, h, row0, rows;  // rows: valid rows from row0
  unsigned bytes;
};

// Returns the first element index of the load if it may touch memory, or -1.
static long touch(const Access& a, unsigned off, int esize, int nbytes) {
  if (off >= a.bytes) return -1;  // out of range: the hardware returns zeros
  CHECK(off % esize == 0, "unaligned offset %u", off);
  const long rs = a.H * a.D;
  const long first = (a.row0 * rs + a.h * a.D) + off / esize;
  const long last = first + nbytes / esize - 1;
  const long row = first / rs, col = first % rs;
  CHECK(row == last / rs, "load crosses a row: first %ld last %ld", first, last);
  CHECK(row >= a.row0 && row < a.row0 + a.rows, "row %ld outside valid rows [%ld, %ld)", row, a.row0,
        a.row0 + a.rows);
  CHECK(row < a.T, "row %ld past tensor rows %ld", row, a.T);
  CHECK(col >= a.h * a.D && col + nbytes / esize <= (a.h + 1) * a.D, "cols [%ld,%ld) outside head %ld slice",
        col, col + nbytes / esize, a.h);
  return first;
}

template <int D, int BN, int NW>
static void check_bf16(long H) {
  using G = Geom16<D, BN, NW>;
  const long rs = H * D;
  // --- K/V tile loads: a sequence that ends at the very end of the tensor
  for (long h : {0L, H - 1}) {
    for (int Lk : {1, 5, 31, 63, 64, 65, 100, 128, 129, 200, 333}) {
      const long k_start = 7, T = k_start + Lk;
      for (int key0 = 0; key0 < Lk; key0 += BN) {
        const int rows = (Lk - key0) < BN ? (Lk - key0) : BN;
        Access a{T, H, D, h, k_start + key0, rows, head_rows_bytes(rows, rs, D, 2)};
        std::vector<int> kseen(BN * D, 0), vseen(BN * D, 0);
        for (int tid = 0; tid < G::THREADS; ++tid) {
          for (int i = 0; i < G::K_PER_THREAD; ++i) {
            const int c = tid + i * G::THREADS;
            const int row = G::k_row(c), ch = G::k_chunk(c);
            const bool inside = row < BN && ch * 8 + 8 <= D;
            CHECK(inside, "K chunk %d maps outside the tile", c);
            const long e = touch(a, (unsigned)((row * rs + ch * 8) * 2), 2, 16);
            if (e >= 0 && inside)
              for (int j = 0; j < 8; ++j) kseen[row * D + ch * 8 + j]++;
          }
          for (int i = 0; i < G::V_PER_THREAD; ++i) {
            const int w = tid + i * G::THREADS;
            if (!G::v_owned(w)) continue;
            const int u = G::v_group(w), dc = G::v_dchunk(w);
            const bool inside = 4 * u + 3 < BN && dc * 8 + 8 <= D;
            CHECK(inside, "V unit %d maps outside the tile", w);
            for (int r = 0; r < 4; ++r) {
              const long e = touch(a, (unsigned)(((4 * u + r) * rs + dc * 8) * 2), 2, 16);
              if (e >= 0 && inside)
                for (int j = 0; j < 8; ++j) vseen[(4 * u + r) * D + dc * 8 + j]++;
            }
          }
        }
        for (int r = 0; r < BN; ++r)
          for (int d = 0; d < D; ++d) {
            const int want = r < rows ? 1 : 0;
            CHECK(kseen[r * D + d] == want, "K element (%d,%d) loaded %d times", r, d, kseen[r * D + d]);
            CHECK(vseen[r * D + d] == want, "V element (%d,%d) loaded %d times", r, d, vseen[r * D + d]);
          }
      }
    }
  }
  // --- Q loads of one wave (32 rows), rows past the sequence end give zeros
  for (long h : {0L, H - 1})
    for (int qrows : {0, 1, 17, 31, 32}) {
      const long T = 3 + qrows;
      Access a{T, H, D, h, 3, qrows, head_rows_bytes(qrows, rs, D, 2)};
      int loaded = 0;
      for (int lane = 0; lane < 64; ++lane)
        for (int ks = 0; ks < D / 16; ++ks) {
          const int l32 = lane & 31, g = lane >> 5;
          if (touch(a, (unsigned)((l32 * rs + 16 * ks + 8 * g) * 2), 2, 16) >= 0) ++loaded;
        }
      CHECK(loaded == qrows * D / 8, "Q: %d chunks loaded for %d rows", loaded, qrows);
    }
  // --- LDS staging writes: exact cover, in range, aligned
  {
    std::vector<int> kcnt(G::LDS_K, 0), vcnt(G::LDS_V, 0);
    std::vector<long> kkey(G::LDS_K, -1), vkey(G::LDS_V, -1);
    for (int tid = 0; tid < G::THREADS; ++tid) {
      for (int i = 0; i < G::K_PER_THREAD; ++i) {
        const int c = tid + i * G::THREADS;
        const int idx = G::ks_index(G::k_row(c), G::k_chunk(c));
        CHECK(idx >= 0 && idx + 8 <= G::LDS_K && idx % 8 == 0, "K LDS index %d", idx);
        for (int j = 0; j < 8; ++j) {
          kcnt[idx + j]++;
          kkey[idx + j] = (long)G::k_row(c) * 100000 + G::k_chunk(c) * 8 + j;
        }
      }
      for (int i = 0; i < G::V_PER_THREAD; ++i) {
        const int w = tid + i * G::THREADS;
        if (!G::v_owned(w)) continue;
        const int u = G::v_group(w), dc = G::v_dchunk(w);
        for (int e = 0; e < 8; ++e) {
          const int d = dc * 8 + e, idx = G::vt_index(d, 4 * u);
          CHECK(idx >= 0 && idx + 4 <= G::LDS_V && idx % 4 == 0, "V LDS index %d", idx);
          for (int j = 0; j < 4; ++j) {
            CHECK(G::vt_index(d, 4 * u + j) == idx + j, "V keys of a unit not contiguous");
            vcnt[idx + j]++;
            vkey[idx + j] = (long)d * 100000 + 4 * u + j;
          }
        }
      }
    }
    // every K element once; a row slot wider than D (head_dim 96 in 128) leaves its tail unwritten
    long kwritten = 0;
    for (int i = 0; i < G::LDS_K; ++i) {
      CHECK(kcnt[i] <= 1, "K LDS element %d written %d times", i, kcnt[i]);
      kwritten += kcnt[i];
    }
    CHECK(kwritten == (long)BN * D, "K LDS: %ld elements written, want %d", kwritten, BN * D);
    for (int i = 0; i < G::LDS_V; ++i) CHECK(vcnt[i] == 1, "V LDS element %d written %d times", i, vcnt[i]);
    // --- MFMA operand reads: the elements each lane feeds
    std::set<int> perm;
    for (int R = 0; R < 32; ++R) perm.insert(key_of_arow(R));
    CHECK((int)perm.size() == 32 && *perm.begin() == 0 && *perm.rbegin() == 31, "key_of_arow not a permutation");
    for (int R = 0; R < 32; ++R) {  // accumulator row R: register 4*(R/8)+R%4 of half (R/4)%2 holds key 16g+r
      const int g = (R >> 2) & 1, r = 4 * (R >> 3) + (R & 3);
      CHECK(key_of_arow(R) == 16 * g + r, "A-row permutation breaks the register/key correspondence");
    }
    for (int lane = 0; lane < 64; ++lane) {
      const int l32 = lane & 31, g = lane >> 5;
      for (int kb = 0; kb < BN / 32; ++kb)
        for (int ks = 0; ks < D / 16; ++ks) {
          const int krow = kb * 32 + key_of_arow(l32), ch = 2 * ks + g;
          const int idx = ks_index<D>(krow, ch);
          CHECK(idx >= 0 && idx + 8 <= G::LDS_K && (idx * 2) % 16 == 0, "K operand read %d", idx);
          for (int e = 0; e < 8; ++e)
            CHECK(kkey[idx + e] == (long)krow * 100000 + ch * 8 + e, "K operand element (%d,%d) is wrong", krow,
                  ch * 8 + e);
        }
      for (int d0 = 0; d0 < D; d0 += 32)
        for (int kb = 0; kb < BN / 32; ++kb)
          for (int t = 0; t < 2; ++t) {
            const int d = d0 + l32, key = kb * 32 + 16 * g + 8 * t;
            const int idx = vt_index<BN>(d, key);
            CHECK(idx >= 0 && idx + 8 <= G::LDS_V && (idx * 2) % 16 == 0, "V operand read %d", idx);
            for (int e = 0; e < 8; ++e)
              CHECK(vkey[idx + e] == (long)d * 100000 + key + e, "V operand element (%d,%d) holds the wrong key", d,
                    key + e);
          }
    }
  }
  // --- bank behaviour of the operand reads (information): lanes of a 16-lane
  // group reading 16-byte chunks should cover 16 distinct 4-bank groups
  int kconf = 0, vconf = 0;
  for (int base = 0; base < 64; base += 16) {
    for (int kb = 0; kb < BN / 32; ++kb)
      for (int ks = 0; ks < D / 16; ++ks) {
        std::set<int> banks;
        for (int lane = base; lane < base + 16; ++lane) {
          const int l32 = lane & 31, g = lane >> 5;
          banks.insert((ks_index<D>(kb * 32 + key_of_arow(l32), 2 * ks + g) / 8) % 16);
        }
        kconf += 16 - (int)banks.size();
      }
    for (int kb = 0; kb < BN / 32; ++kb)
      for (int t = 0; t < 2; ++t) {
        std::set<int> banks;
        for (int lane = base; lane < base + 16; ++lane) {
          const int l32 = lane & 31, g = lane >> 5;
          banks.insert((vt_index<BN>(l32, kb * 32 + 16 * g + 8 * t) / 8) % 16);
        }
        vconf += 16 - (int)banks.size();
      }
  }
  // --- epilogue stores: lane (row l32, half g) writes dims db*32 + 8*s4 + 4g + c
  {
    std::vector<int> cnt(D, 0);
    for (int g = 0; g < 2; ++g)
      for (int db = 0; db < D / 32; ++db)
        for (int s4 = 0; s4 < 4; ++s4)
          for (int c = 0; c < 4; ++c) {
            const int d = db * 32 + 8 * s4 + 4 * g + c;
            CHECK(d >= 0 && d < D, "output dim %d", d);
            cnt[d]++;
          }
    for (int d = 0; d < D; ++d) CHECK(cnt[d] == 1, "output dim %d written %d times", d, cnt[d]);
  }
  std::printf("bf16 D=%d BN=%d NW=%d H=%ld: ok (operand-read bank overlaps: K %d, V %d)\n", D, BN, NW, H, kconf,
              vconf);
}

template <int D, int NW>
static void check_f32() {
  using G = F32Geom<D, NW>;
  std::vector<int> cnt(G::LDS_ELEMS, 0);
  for (int tid = 0; tid < G::THREADS; ++tid)
    for (int i = 0; i < G::PER_THREAD; ++i) {
      const int c = tid + i * G::THREADS;
      const int row = G::row(c), ch = G::chunk(c);
      CHECK(row < G::BN && 4 * ch + 4 <= D, "fp32 chunk %d outside the tile", c);
      const int idx = row * G::LD + 4 * ch;
      CHECK(idx % 4 == 0 && idx + 4 <= G::LDS_ELEMS, "fp32 LDS index %d", idx);
      for (int j = 0; j < 4; ++j) cnt[idx + j]++;
    }
  for (int r = 0; r < G::BN; ++r)
    for (int d = 0; d < G::LD; ++d) CHECK(cnt[r * G::LD + d] == (d < D ? 1 : 0), "fp32 LDS (%d,%d)", r, d);
  std::set<int> keys;
  for (int g = 0; g < 2; ++g)
    for (int r = 0; r < 16; ++r) keys.insert(G::key_of_reg(r, g));
  CHECK((int)keys.size() == 32 && *keys.rbegin() == 31, "fp32 register/key map not a permutation");
  for (int lane = 0; lane < 64; ++lane) {
    const int l32 = lane & 31, g = lane >> 5;
    for (int ks = 0; ks < D / 2; ++ks) CHECK(l32 * G::LD + 2 * ks + g < G::LDS_ELEMS, "fp32 K read");
    for (int u = 0; u < 16; ++u)
      for (int db = 0; db < D / 32; ++db)
        CHECK(G::key_of_reg(u, g) * G::LD + db * 32 + l32 < G::LDS_ELEMS, "fp32 V read");
  }
  std::printf("f32 D=%d NW=%d: ok\n", D, NW);
}

// Forward kernel: K and V tiles of BN keys loaded straight into LDS (16 bytes
// per lane at LDS slot p = 64 * load + lane; the NW wavefronts take 1024 / NW
// consecutive slots each), K in the ks_index layout, V row-major (vr_index)
// and read with transposing LDS reads for the PV product.
template <int D, int BN, bool V_LAYOUT>
static void check_direct(long H) {
  constexpr int KS = k_stride<D>(), CPR = KS / 8, SLOTS = BN * CPR;
  CHECK(SLOTS % 64 == 0, "D=%d BN=%d: %d slots are not whole wavefront loads", D, BN, SLOTS);
  const long h = H - 1;
  std::vector<int> placed(BN * KS, 0);
  for (int rows : {BN, 1, BN / 2 + 3, BN - 1}) {  // valid keys in the tile
    const Access a{rows + 5, H, D, h, 2, rows, head_rows_bytes(rows, H * D, D, 2)};
    std::vector<int> seen(BN * D, 0);
    for (int p = 0; p < SLOTS; ++p) {
      int row, ch;
      direct_slot_chunk<D, V_LAYOUT>(p, row, ch);
      CHECK(row >= 0 && row < BN && ch >= 0 && ch < D / 8, "D=%d slot %d -> (%d,%d)", D, p, row, ch);
      const unsigned off = (unsigned)((row * H * D + ch * 8) * 2);
      const long first = touch(a, off, 2, 16);
      const int idx = V_LAYOUT ? vr_index<D>(row, ch) : ks_index<D>(row, ch);
      if (idx == 8 * p) {  // the slot holds this chunk in the read layout
        if (rows == BN) placed[idx] += 1;
        if (first >= 0)
          for (int j = 0; j < 8; ++j) seen[row * D + ch * 8 + j]++;
      } else {
        CHECK(D == 96, "D=%d: slot %d holds (%d,%d) but the layout puts it at %d", D, p, row, ch, idx / 8);
      }
    }
    for (int r = 0; r < BN; ++r)
      for (int d = 0; d < D; ++d)
        CHECK(seen[r * D + d] == (r < rows ? 1 : 0), "D=%d rows=%d: element (%d,%d) loaded %d times", D, rows, r,
              d, seen[r * D + d]);
  }
  for (int r = 0; r < BN; ++r)
    for (int ch = 0; ch < D / 8; ++ch) {
      const int idx = V_LAYOUT ? vr_index<D>(r, ch) : ks_index<D>(r, ch);
      CHECK(placed[idx] == 1, "D=%d chunk (%d,%d) placed %d times", D, r, ch, placed[idx]);
    }
  if (V_LAYOUT) {
    // transposing reads of O^T += V^T P^T: step (kb, t) reads keys
    // kb*32 + 16g + 8t + 4h .. +3 of dimensions 32 db + lane%32
    for (int kb = 0; kb < BN / 32; ++kb)
      for (int t = 0; t < 2; ++t)
        for (int h2 = 0; h2 < 2; ++h2)
          for (int db = 0; db < D / 32; ++db) {
            std::vector<int> bank_use[2] = {std::vector<int>(16, 0), std::vector<int>(16, 0)};
            for (int grp = 0; grp < 4; ++grp) {
              const int g = grp / 2, r0 = kb * 32 + 16 * g + 8 * t + 4 * h2;
              std::vector<int> got(4 * 16, 0);  // rows r0..r0+3 x the group's 16 dims
              for (int i = 0; i < 16; ++i) {
                const int lane = 16 * grp + i;
                const int idx = vr_tr_index<D>(lane, r0, db);
                CHECK(idx >= 0 && idx % 4 == 0 && idx + 4 <= BN * KS, "D=%d tr read index %d", D, idx);
                // the 4 elements at idx are row r0 + i/4, dims c0 + 4(i%4) .. +3
                const int row = r0 + (i >> 2), c0 = 32 * db + 16 * (grp & 1), col = c0 + 4 * (i & 3);
                CHECK(idx == vr_index<D>(row, col >> 3) + (col & 7), "D=%d tr read lane %d at wrong element", D,
                      lane);
                for (int e = 0; e < 4; ++e) got[(i >> 2) * 16 + 4 * (i & 3) + e]++;
                // lane i receives dim c0 + i: must be the output dim of this lane
                CHECK(c0 + i == 32 * db + (lane & 31), "D=%d lane %d receives dim %d", D, lane, c0 + i);
                bank_use[g][(idx * 2 / 16) % 16]++;
              }
              for (int e = 0; e < 64; ++e) CHECK(got[e] == 1, "D=%d tr group %d element %d read %d times", D, grp, e,
                                                 got[e]);
            }
            for (int g = 0; g < 2; ++g)
              for (int b = 0; b < 16; ++b)  // two lanes read the two halves of each 16-byte chunk
                CHECK(bank_use[g][b] == 2, "D=%d tr read: bank group %d used by %d lanes of a 32-lane half", D, b,
                      bank_use[g][b]);
          }
  }
  std::printf("direct %s D=%d BN=%d H=%ld: ok\n", V_LAYOUT ? "V" : "K", D, BN, H);
}

// The software-pipelined forward kernel's other LDS accesses: the K operand
// reads of S^T = K Q^T from every 32-key slab of a tile, and the epilogue,
// where wavefront w stages its 32 normalised rows in rows 32w .. 32w+31 of the
// K buffers (ks_index layout, 4 columns per lane and write) and reads them
// back as 16-byte row pieces for the global stores.
template <int D, int BN, int NW>
static void check_pipe() {
  constexpr int KS = k_stride<D>(), TILE = BN * KS, NBUF = 4, CH = D / 8;
  CHECK(NW * 32 * KS <= NBUF * TILE, "D=%d: %d waves' staging rows exceed the K buffers", D, NW);
  for (int lane = 0; lane < 64; ++lane) {
    const int l32 = lane & 31, g = lane >> 5;
    for (int row0 = 0; row0 < BN; row0 += 32)
      for (int ks = 0; ks < D / 16; ++ks) {
        const int idx = ks_index<D>(row0 + key_of_arow(l32), 2 * ks + g);
        CHECK(idx >= 0 && idx % 8 == 0 && idx + 8 <= TILE, "D=%d K operand read %d", D, idx);
      }
  }
  for (int w = 0; w < NW; ++w) {
    const int base = w * 32 * KS;
    std::vector<int> wrote(32 * D, 0), read(32 * D, 0);
    std::vector<int> at(32 * KS, -1);  // element of the slice -> (row * D + col) written there
    for (int lane = 0; lane < 64; ++lane) {
      const int l32 = lane & 31, g = lane >> 5;
      for (int db = 0; db < D / 32; ++db)
        for (int s4 = 0; s4 < 4; ++s4)
          for (int c = 0; c < 4; ++c) {
            const int idx = ks_index<D>(l32, 4 * db + s4) + 4 * g + c;
            const int col = 32 * db + 8 * s4 + 4 * g + c;
            CHECK(idx >= 0 && idx < 32 * KS && base + idx < NBUF * TILE, "D=%d staging write %d", D, idx);
            CHECK(at[idx] < 0, "D=%d staging element %d written twice", D, idx);
            at[idx] = l32 * D + col;
            wrote[l32 * D + col]++;
          }
    }
    for (int it = 0; it < 32 * CH / 64; ++it)
      for (int lane = 0; lane < 64; ++lane) {
        const int c = it * 64 + lane, r = c / CH, ch = c % CH;
        for (int j = 0; j < 8; ++j) {
          const int idx = ks_index<D>(r, ch) + j;
          CHECK(idx >= 0 && idx < 32 * KS, "D=%d staging read %d", D, idx);
          CHECK(at[idx] == r * D + 8 * ch + j, "D=%d staging read (%d,%d)+%d finds element %d", D, r, ch, j, at[idx]);
          read[r * D + 8 * ch + j]++;
        }
      }
    for (int e = 0; e < 32 * D; ++e)
      CHECK(wrote[e] == 1 && read[e] == 1, "D=%d staging element %d written %d, read %d times", D, e, wrote[e],
            read[e]);
  }
  std::printf("pipe D=%d BN=%d NW=%d: ok\n", D, BN, NW);
}


// Backward (256-key workgroup, 32-row query blocks): every main-loop LDS
// address written as (lane part ^ chunk term) + offset must equal the
// element-index form, stay inside its tile and keep its alignment; the chunk
// terms must stay below bit 10, the alignment of the tiles' base addresses.
template <int D>
static void check_bwd_addr() {
  namespace B = fa::bwdt;
  constexpr int KS = k_stride<D>(), BM = 32, BN = 256, CT = D / 16;
  const unsigned qtile = 2u * BM * KS, ktile = 2u * BN * KS, dstile = 2u * BM * BN;
  for (int g = 0; g < 2; ++g)
    for (int ks = 0; ks < D / 16; ++ks) {
      CHECK(B::op_xor(ks) < 1024u, "op xor");
      for (int row = 0; row < BM; ++row) {
        const unsigned a = B::op_lane_tq<D>(row, g) ^ B::op_xor(ks);
        CHECK(a == 2u * (unsigned)B::tq_index<D>(row, 2 * ks + g), "D=%d Q/dO operand row %d ks %d g %d", D, row, ks, g);
        CHECK(a % 16 == 0 && a + 16 <= qtile, "D=%d Q/dO operand out of tile", D);
      }
      for (int row = 0; row < BN; ++row) {
        const unsigned a = B::op_lane_ks<D>(row, g) ^ B::op_xor(ks);
        CHECK(a == 2u * (unsigned)ks_index<D>(row, 2 * ks + g), "D=%d V operand row %d ks %d g %d", D, row, ks, g);
        CHECK(a % 16 == 0 && a + 16 <= ktile, "D=%d V operand out of tile", D);
      }
    }
  for (int li = 0; li < 16; ++li)
    for (int lg = 0; lg < 4; ++lg) {
      for (int db = 0; db < D / 32; ++db)
        for (int t = 0; t < 2; ++t)
          for (int h = 0; h < 2; ++h) {
            CHECK(B::trq_xor<D>(db, t, h) < 1024u, "trq xor");
            const unsigned a = (B::trq_lane<D>(li, lg) ^ B::trq_xor<D>(db, t, h)) + B::trq_add<D>(t, h);
            CHECK(a == B::trq_orig<D>(li, lg, db, t, h), "D=%d dV/dK read li %d lg %d db %d t %d h %d", D, li, lg, db,
                  t, h);
            CHECK(a % 8 == 0 && a + 8 <= qtile, "D=%d dV/dK read out of tile", D);
          }
      for (int kk = 0; kk < BN / 32; ++kk)
        for (int ct = 0; ct < CT; ++ct)
          for (int h = 0; h < 2; ++h) {
            CHECK(B::trk_xor(ct, h) < 1024u, "trk xor");
            const unsigned a = (B::trk_lane<D>(li, lg) ^ B::trk_xor(ct, h)) + B::trk_add<D>(kk, h);
            CHECK(a == B::trk_orig<D>(li, lg, kk, ct, h), "D=%d K^T read li %d lg %d kk %d ct %d h %d", D, li, lg, kk,
                  ct, h);
            CHECK(a % 8 == 0 && a + 8 <= ktile, "D=%d K^T read out of tile", D);
          }
      for (int kk = 0; kk < BN / 32; ++kk)
        for (int rt = 0; rt < 2; ++rt) {
          CHECK(B::dsa_xor(kk) < 1024u, "dsa xor");
          const unsigned a = (B::dsa_lane(li, lg) ^ B::dsa_xor(kk)) + B::dsa_add(rt);
          const unsigned b = (B::dsa_lane(li, lg) + B::dsa_add(rt)) ^ B::dsa_xor(kk);
          CHECK(a == B::dsa_orig(li, lg, kk, rt) && b == a, "dS read li %d lg %d kk %d rt %d", li, lg, kk, rt);
          CHECK(a % 16 == 0 && a + 16 <= dstile, "dS read out of tile");
        }
    }
  for (int key = 0; key < BN; ++key)
    for (int g = 0; g < 2; ++g)
      for (int r = 0; r < 16; ++r) {
        CHECK(B::dss_xor(r) < 1024u, "dss xor");
        const unsigned a = (B::dss_lane(key, g) ^ B::dss_xor(r)) + B::dss_add(r);
        CHECK(a == B::dss_orig(key, g, r), "dS store key %d g %d r %d", key, g, r);
        CHECK(a % 2 == 0 && a + 2 <= dstile, "dS store out of tile");
      }
  // the dS stores of one step (32 keys per wave x 8 waves, 32 rows) cover the tile once
  std::vector<int> hit(BM * BN, 0);
  for (int key = 0; key < BN; ++key)
    for (int g = 0; g < 2; ++g)
      for (int r = 0; r < 16; ++r) ++hit[B::dss_orig(key, g, r) / 2];
  for (int e = 0; e < BM * BN; ++e) CHECK(hit[e] == 1, "dS element %d stored %d times", e, hit[e]);
  std::printf("backward addresses D=%d: ok\n", D);
}

int main() {
  check_pipe<64, 128, 8>();
  check_pipe<64, 64, 4>();
  check_pipe<96, 64, 8>();
  check_pipe<128, 64, 8>();
  check_pipe<128, 32, 4>();
  check_pipe<256, 32, 4>();
  for (long H : {1L, 3L, 16L}) {
    check_direct<64, 128, false>(H);
    check_direct<64, 128, true>(H);
    check_direct<64, 64, false>(H);
    check_direct<64, 64, true>(H);
    check_direct<96, 64, false>(H);
    check_direct<96, 64, true>(H);
    check_direct<128, 64, false>(H);
    check_direct<128, 64, true>(H);
    check_direct<128, 32, false>(H);
    check_direct<128, 32, true>(H);
    check_direct<256, 32, false>(H);
    check_direct<256, 32, true>(H);
  }
  // configurations the library instantiates (and neighbours it may use)
  for (long H : {1L, 3L, 16L}) {
    check_bf16<128, 64, 8>(H);
    check_bf16<128, 64, 4>(H);
    check_bf16<96, 64, 4>(H);
    check_bf16<256, 32, 4>(H);
    // backward: query blocks of 64 rows (head_dim 128, 8 waves) and 32 rows
    // (head_dim 64, 4 waves), and the 128-key K and V blocks
    check_bf16<128, 128, 8>(H);
    check_bf16<128, 256, 8>(H);
    check_bf16<64, 256, 8>(H);
    check_bf16<128, 32, 8>(H);
    check_bf16<128, 32, 4>(H);
    check_bf16<64, 32, 4>(H);
    check_bf16<128, 128, 4>(H);
    check_bf16<64, 64, 4>(H);
    check_bf16<64, 64, 8>(H);
    check_bf16<64, 128, 4>(H);
  }
  check_bwd_addr<64>();
  check_bwd_addr<96>();
  check_bwd_addr<128>();
  check_f32<64, 4>();
  check_f32<96, 4>();
  check_f32<128, 4>();
  if (g_fail) {
    std::fprintf(stderr, "%d violations\n", g_fail);
    return 1;
  }
  std::printf("all tiling checks passed\n");
  return 0;
}
