// fa_varlen_decode.hip -- gfx950 kernels for exact attention of packed queries
// against a key/value cache: per-sequence key lengths that are not
// cumulative, an optional left padding, an optional paged cache layout, and
// the key range of each sequence split across workgroups (the decode-shaped
// case: few query rows per sequence, long cached key ranges).
//
// Pages: friki.work "Mecanismo cu_seqlens en FlashAttention", sections "Lógica
// de cálculo de longitud" and "Optimización de acceso a memoria" (with the
// non-cumulative key format a sequence's keys sit at its batch index times a
// batch stride and its usable key length is the given length minus the left
// padding) and "Integración con máscaras causales y caché paginada" (a paged
// key/value cache); slavadubrov.com "O que FlashAttention muda na
// inferência", section "A implementação e a carga de trabalho continuam a
// importar" (single-token decoding exposes different parallelism than
// prefill).
//
// Layouts:
//   q, out   [total_q, heads, D] packed by cu_seqlens_q (as the forward pass)
//   caches   [cache_blocks, cache_rows, kv_heads, D]; without a block table
//            block b is sequence b's slot; with one, position p of sequence b
//            is row p % cache_rows of block block_table[b * blocks_per_seq +
//            p / cache_rows]
//   sequence b's keys are cache positions leftpad_k[b] .. seqlens_k[b]-1
//
// Work: one workgroup per (sequence, key/value head, split).  Its rows are all
// query rows of the sequence for all query heads of the key/value head
// (G * Lq rows, G = heads / kv_heads), so the cache is read once per group;
// they are processed 16 at a time (16x16x32 MFMAs).  The split's 32-key tiles
// are dealt to the 4 wavefronts round-robin; each wavefront streams its tiles straight from
// global memory (K as the A operand of S^T = K Q^T, V through a wave-private
// LDS tile read back with transposing reads as the A operand of O^T = V^T P^T),
// keeps an online softmax per row; the four wavefronts' (max, sum, O) are
// merged in LDS into the split's partial, which goes to the workspace.
// decode_combine_kernel merges the partials of every row
// (partials with max m_p, sum l_p and output O_p give out = sum_p 2^(m_p-m)
// O_p / sum_p 2^(m_p-m) l_p with m = max_p m_p; the same rescaling identity
// as the online softmax).  fp32 caches take decode_f32_kernel: the same work
// split on the fp32 16x16x4 MFMA.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_varlen_device.h"
#include "fa_varlen_launch.h"
#include "fa_varlen_tiling.h"

namespace fa {
namespace {

constexpr int kDecWaves = 4;  // wavefronts per workgroup
constexpr int kDecTile = 32;  // keys per tile

typedef short dec_s16x4 __attribute__((ext_vector_type(4)));

// transposing read of 4 rows r0 .. r0+3 of column c0 + i (16-lane groups, see
// ds_read_b64_tr_b16) from a row-major swizzled [rows][D] tile
template <int D>
__device__ __forceinline__ dec_s16x4 dec_tr_read4(const uint16_t* tile, int r0, int c0, int i) {
  const int row = r0 + (i >> 2), col = c0 + 4 * (i & 3);
  const uint16_t* p = tile + tiling::ks_index<D>(row, col >> 3) + (col & 7);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) dec_s16x4*)p);
}
template <typename V8, int D>
__device__ __forceinline__ V8 dec_tr_read8(const uint16_t* tile, int r0, int c0, int i) {
  const dec_s16x4 lo = dec_tr_read4<D>(tile, r0, c0, i);
  const dec_s16x4 hi = dec_tr_read4<D>(tile, r0 + 4, c0, i);
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}

// Element offset of cache position p of sequence b, key/value head hk.
__device__ __forceinline__ int64_t cache_offset(const DecArgs& a, int b, int p, int hk, int D) {
  int64_t row;
  if (a.block_table) {
    const int blk = a.block_table[(int64_t)b * a.blocks_per_seq + p / a.cache_rows];
    row = (int64_t)blk * a.cache_rows + p % a.cache_rows;
  } else {
    row = (int64_t)b * a.cache_rows + p;
  }
  return row * a.kv_row_stride + (int64_t)hk * D;
}

// The four wavefronts' results for the 16 rows of a row tile are merged in
// LDS before anything is written (the rescaling identity of the combine:
// weights 2^(m_w - M), M the largest m_w), so each split writes one partial
// per (row, head).  On entry lane (i, G) of wave w holds o[dt][r] = O^T(dim
// 16dt + 4G + r, row i) and the row's m and l (equal on the four lane
// groups); `ob` is LDS room for 4 x 16 x D floats (the waves' V tiles, free
// once every wave has left its key loop) and `mlb` for 4 x 16 (m, l) pairs.
// Wave w then merges dims w D/4 .. (w+1) D/4 - 1 of the tile, lane (i, G)
// the D/16 of them from w D/4 + G D/16 on.  Ends with a barrier, so the next
// row tile may overwrite the V tiles.
template <int D>
__device__ __forceinline__ void dec_merge_store(const DecArgs& a, const f32x4 (&o)[D / 16], float m_run, float l,
                                                float* ob, float (*mlb)[16][2], int wave, int li, int lg,
                                                bool rvalid, int64_t pr) {
  constexpr int DT = D / 16, DW = D / 4, DL = D / 16;
  __syncthreads();  // every wave has left its key loop: the V tiles are free
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) *(f32x4*)(ob + (wave * 16 + li) * D + 16 * dt + 4 * lg) = o[dt];
  if (lg == 0) {
    mlb[wave][li][0] = m_run;
    mlb[wave][li][1] = l;
  }
  __syncthreads();
  float mw[kDecWaves], M = kNegInf;
#pragma unroll
  for (int v = 0; v < kDecWaves; ++v) {
    mw[v] = mlb[v][li][0];
    M = fmaxf(M, mw[v]);
  }
  float wgt[kDecWaves], L = 0.f;
#pragma unroll
  for (int v = 0; v < kDecWaves; ++v) {
    wgt[v] = mw[v] == kNegInf ? 0.f : fast_exp2(mw[v] - M);
    L += wgt[v] * mlb[v][li][1];  // a NaN sum stays NaN, even at weight 0
  }
  if (rvalid) {
    // a split that saw no key (M = -inf) writes only its (m, l): the combine skips its O
    if (M != kNegInf) {
      float* po = a.part_o + pr * D + wave * DW + lg * DL;
      const float* src = ob + li * D + wave * DW + lg * DL;
#pragma unroll
      for (int c = 0; c < DL; ++c) {
        float x = 0.f;
#pragma unroll
        for (int v = 0; v < kDecWaves; ++v) x += wgt[v] != 0.f ? wgt[v] * src[v * 16 * D + c] : 0.f;
        po[c] = x;
      }
    }
    if (wave == 0 && lg == 0) {
      a.part_ml[2 * pr] = M;
      a.part_ml[2 * pr + 1] = L;
    }
  }
  __syncthreads();  // the merge has read the V-tile room
}

// Two wavefronts per SIMD up to head_dim 128; at 256 the output and the
// tile's K and V registers need more than half a SIMD's registers, so one.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void decode16_kernel(DecArgs a) {
  // 16x16x32 MFMA layout (gfx950): lane l, group G = l/16, i = l%16:
  //   A operand: row i, k = 8G..8G+7;  B operand: column i, k = 8G..8G+7;
  //   accumulator register r: row 4G + r, column i.
  constexpr int KS = D / 32;           // k-steps over head_dim
  constexpr int DT = D / 16;           // 16-row tiles of O^T
  constexpr int KT = kDecTile / 16;    // 16-key tiles of S^T per key tile
  constexpr int KK = kDecTile / 32;    // k-steps over the keys of a tile
  constexpr int LOADS = kDecTile * D / 8 / 64;  // 16-byte loads per lane for one of K or V
  using E = Elem16<T>;
  typedef typename E::v8 v8;
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kDecWaves][kDecTile * tiling::k_stride<D>()];

  // item: (sequence b, key/value head hk, split s)
  const int item = blockIdx.x;
  const int s = item % a.num_splits;
  const int hk = (item / a.num_splits) % a.kv_heads;
  const int b = item / (a.num_splits * a.kv_heads);
  if (b >= a.batch) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int G = a.head_group;
  const int q_start = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q_start;
  const int lp = a.leftpad_k ? a.leftpad_k[b] : 0;
  const int Lk = a.seqlens_k[b] - lp;
  const int shift = Lk - Lq;
  const int rows = G * Lq;
  const int ntiles = (max(Lk, 0) + kDecTile - 1) / kDecTile;
  const int tps = (ntiles + a.num_splits - 1) / a.num_splits;  // tiles per split
  const int t_begin = s * tps, t_end = min(ntiles, t_begin + tps);
  const int npart = a.num_splits;  // one partial per (row, head, split)
  __shared__ float lds_ml[kDecWaves][16][2];
  uint16_t* vt = lds_v[wave];

  for (int rt = 0; rt * 16 < rows; ++rt) {
    // Q^T of the row tile as the B operand: lane column li <-> row rt*16 + li
    const int r = rt * 16 + li;
    const bool rvalid = r < rows;
    const int qi = rvalid ? r / G : 0, gi = rvalid ? r % G : 0;
    const int h = hk * G + gi;
    v8 qreg[KS];
    {
      const uint16_t* qp = (const uint16_t*)a.q + (int64_t)(q_start + qi) * a.row_stride + (int64_t)h * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (rvalid) x = *(const u32x4*)(qp + 32 * ks + 8 * lg);
        qreg[ks] = __builtin_bit_cast(v8, x);
      }
    }
    const int lim = CAUSAL ? min(Lk - 1, qi + shift) : Lk - 1;  // last visible key of the row
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    // Lane (li, lg) loads K rows 16*kt + li (A operand, dims 32ks + 8lg ..)
    // and V rows 16*kt + li (dims 32ks + 8lg ..) of each key tile.  Keys
    // past the sequence point at its first key and are zeroed after the load,
    // so every load is issued without a branch.  The loads of the wave's next
    // tile are issued as soon as the current tile's K and V registers are
    // consumed (V stored to LDS, S computed), so they are in flight during the
    // softmax and O += V^T P^T of the current tile; the offsets (block-table
    // reads) run one more tile ahead.
    int64_t off[KT];
    v8 ka[KT][KS];
    u32x4 vr[KT][KS];
    int t = t_begin + wave;
    if (t < t_end) {
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = t * kDecTile + 16 * kt + li;
        off[kt] = cache_offset(a, b, lp + (key < Lk ? key : 0), hk, D);
      }
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          ka[kt][ks] = __builtin_bit_cast(v8, *(const u32x4*)((const uint16_t*)a.k_cache + off[kt] + 32 * ks + 8 * lg));
          vr[kt][ks] = *(const u32x4*)((const uint16_t*)a.v_cache + off[kt] + 32 * ks + 8 * lg);
        }
      if (t + kDecWaves < t_end) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int key = t * kDecTile + kDecWaves * kDecTile + 16 * kt + li;
          off[kt] = cache_offset(a, b, lp + (key < Lk ? key : 0), hk, D);
        }
      }
    }
    for (; t < t_end; t += kDecWaves) {
      const int key0 = t * kDecTile;
      const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
        if (!(key0 + 16 * kt + li < Lk))
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            ka[kt][ks] = __builtin_bit_cast(v8, zero);
            vr[kt][ks] = zero;
          }
      // V tile into the wave's LDS buffer (row-major, swizzled; 16-byte chunk
      // 4ks + lg of key row 16kt + li)
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          *(u32x4*)(vt + tiling::ks_index<D>(16 * kt + li, 4 * ks + lg)) = vr[kt][ks];
      const bool more = t + kDecWaves < t_end;
      // the next tile's V: its registers are free once V is in LDS
      if (more) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            vr[kt][ks] = *(const u32x4*)((const uint16_t*)a.v_cache + off[kt] + 32 * ks + 8 * lg);
      }

      // S^T = K Q^T: register e of tile kt holds key key0 + 16kt + 4lg + e of row li
      f32x4 sc[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          sc[kt] = Mfma16<T>::run(ka[kt][ks], qreg[ks], sc[kt]);
      }
      // the next tile's K: into the registers the product above consumed
      if (more) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            ka[kt][ks] =
                __builtin_bit_cast(v8, *(const u32x4*)((const uint16_t*)a.k_cache + off[kt] + 32 * ks + 8 * lg));
        if (t + 2 * kDecWaves < t_end) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
            const int key = key0 + 2 * kDecWaves * kDecTile + 16 * kt + li;
            off[kt] = cache_offset(a, b, lp + (key < Lk ? key : 0), hk, D);
          }
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = key0 + 16 * kt + 4 * lg + e <= lim;
          sc[kt][e] = vis ? sc[kt][e] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, sc[kt][e]);
        }
      // the four 16-lane groups hold different keys of the same row
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      // P^T as the B operand: k-index 8lg + j of k-step kk <-> key 32kk + 16(j/4) + 4lg + j%4
      v8 p[KK];
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = fast_exp2(sc[kt][e] - m_use);
          lsum += pe;
          p[kt >> 1][4 * (kt & 1) + e] = (T)pe;
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;

      // O^T += V^T P^T: the A operand of row d = 16dt + li holds keys
      // 32kk + 4lg + 0..3 and 32kk + 16 + 4lg + 0..3 (two transposing reads)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const dec_s16x4 lo = dec_tr_read4<D>(vt, 32 * kk + 4 * lg, 16 * dt, li);
          const dec_s16x4 hi = dec_tr_read4<D>(vt, 32 * kk + 16 + 4 * lg, 16 * dt, li);
          const short __attribute__((ext_vector_type(8))) av = {lo[0], lo[1], lo[2], lo[3],
                                                                 hi[0], hi[1], hi[2], hi[3]};
          o[dt] = Mfma16<T>::run(__builtin_bit_cast(v8, av), p[kk], o[dt]);
        }
    }

    // this wave's (m, l, O) for the rows of the tile, l summed over the four
    // groups; merged with the other waves' into the split's partial
    float l = l_run + __shfl_xor(l_run, 16, 64);
    l = pair_sum(l);
    const int64_t pr = ((int64_t)(q_start + qi) * a.heads + h) * npart + s;
    dec_merge_store<D>(a, o, m_run, l, reinterpret_cast<float*>(&lds_v[0][0]), lds_ml, wave, li, lg, rvalid, pr);
  }
}

// fp32 caches: the same work split with the fp32 16x16x4 MFMA (lane l,
// G = l/16, i = l%16: A row i, k = G; B column i, k = G; accumulator register
// r: row 4G + r, column i), one element per lane and operand.
//   * S^T = K Q^T contracts over head_dim in D/4 k-steps; k-step s of lane
//     group G takes dimension G*D/4 + s, so each lane reads its K and Q
//     elements as contiguous float4s.
//   * The k-step s of O^T += V^T P^T over 16-key subtile kt takes keys
//     16kt + 4G + s: register s of the lane's S^T subtile is then exactly its
//     B operand (no shuffle).  V goes through a wave-private padded LDS tile
//     (rows of D + 4 floats) and is read one element per lane.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void decode_f32_kernel(DecArgs a) {
  constexpr int KQ = D / 4;                    // head dimensions per lane group in S^T = K Q^T
  constexpr int NV = KQ / 4;                   // float4s per lane and row
  constexpr int DT = D / 16;                   // 16-row tiles of O^T
  constexpr int KT = kDecTile / 16;            // 16-key subtiles per key tile
  constexpr int LD = D + 4;                    // LDS row of the V tile (floats)
  constexpr int VCH = kDecTile * D / 4 / 64;   // float4s of the V tile per lane
  static_assert((kDecTile * D / 4) % 64 == 0 && KQ % 4 == 0, "tile must split into whole float4 loads");
  __shared__ __attribute__((aligned(16))) float lds_v[kDecWaves][kDecTile * LD];

  const int item = blockIdx.x;
  const int s_split = item % a.num_splits;
  const int hk = (item / a.num_splits) % a.kv_heads;
  const int b = item / (a.num_splits * a.kv_heads);
  if (b >= a.batch) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int G = a.head_group;
  const int q_start = a.cu_q[b];
  const int Lq = a.cu_q[b + 1] - q_start;
  const int lp = a.leftpad_k ? a.leftpad_k[b] : 0;
  const int Lk = a.seqlens_k[b] - lp;
  const int shift = Lk - Lq;
  const int rows = G * Lq;
  const int ntiles = (max(Lk, 0) + kDecTile - 1) / kDecTile;
  const int tps = (ntiles + a.num_splits - 1) / a.num_splits;
  const int t_begin = s_split * tps, t_end = min(ntiles, t_begin + tps);
  const int npart = a.num_splits;
  __shared__ float lds_ml[kDecWaves][16][2];
  float* vt = lds_v[wave];

  for (int rt = 0; rt * 16 < rows; ++rt) {
    const int r = rt * 16 + li;
    const bool rvalid = r < rows;
    const int qi = rvalid ? r / G : 0, gi = rvalid ? r % G : 0;
    const int h = hk * G + gi;
    f32x4 qv[NV];
    {
      const float* qp = (const float*)a.q + (int64_t)(q_start + qi) * a.row_stride + (int64_t)h * D + lg * KQ;
#pragma unroll
      for (int n = 0; n < NV; ++n) qv[n] = rvalid ? *(const f32x4*)(qp + 4 * n) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int lim = CAUSAL ? min(Lk - 1, qi + shift) : Lk - 1;
    f32x4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = kNegInf, l_run = 0.f;

    for (int t = t_begin + wave; t < t_end; t += kDecWaves) {
      const int key0 = t * kDecTile;
      // V tile -> LDS (keys past the sequence as zeros)
#pragma unroll
      for (int j = 0; j < VCH; ++j) {
        const int c = lane + 64 * j;
        const int row = c / (D / 4), c4 = c % (D / 4);
        const int key = key0 + row;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (key < Lk) x = *(const f32x4*)((const float*)a.v_cache + cache_offset(a, b, lp + key, hk, D) + 4 * c4);
        *(f32x4*)(vt + row * LD + 4 * c4) = x;
      }
      // S^T = K Q^T: register e of subtile kt holds key key0 + 16kt + 4lg + e of row li
      f32x4 sc[KT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int key = key0 + 16 * kt + li;
        const bool kvalid = key < Lk;
        const float* kp =
            (const float*)a.k_cache + cache_offset(a, b, lp + (kvalid ? key : 0), hk, D) + lg * KQ;
        sc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < NV; ++n) {
          const f32x4 kv = kvalid ? *(const f32x4*)(kp + 4 * n) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int c = 0; c < 4; ++c) sc[kt] = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[c], qv[n][c], sc[kt], 0, 0, 0);
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool vis = key0 + 16 * kt + 4 * lg + e <= lim;
          sc[kt][e] = vis ? sc[kt][e] * a.scale_log2 : kNegInf;
          mx = fmaxf(mx, sc[kt][e]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      m_run = m_new;
      float lsum = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sc[kt][e] = fast_exp2(sc[kt][e] - m_use);
          lsum += sc[kt][e];
        }
      l_run = l_run * alpha + lsum;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[dt][e] *= alpha;
      // O^T += V^T P^T: k-step (kt, e) takes keys 16kt + 4G + e
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float* vrow = vt + (16 * kt + 4 * lg + e) * LD + li;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * dt], sc[kt][e], o[dt], 0, 0, 0);
        }
    }

    float l = l_run + __shfl_xor(l_run, 16, 64);
    l = pair_sum(l);
    const int64_t pr = ((int64_t)(q_start + qi) * a.heads + h) * npart + s_split;
    dec_merge_store<D>(a, o, m_run, l, &lds_v[0][0], lds_ml, wave, li, lg, rvalid, pr);
  }
}

// One wavefront per (row, head): merge its partials into out and lse.  Lane
// p % 64 weighs partials p; the partial outputs are then read without
// dependent branches (empty partials, whose O was never written, enter through
// a select with weight 0), so the loads of all partials are in flight together.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t rh = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // row * heads + head
  const int64_t nrows = a.cu_q[a.batch];
  if (rh >= nrows * a.heads) return;
  const int npart = a.num_splits;
  const float* ml = a.part_ml + rh * npart * 2;
  float m = kNegInf;
  for (int p = lane; p < npart; p += 64) m = fmaxf(m, ml[2 * p]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float m_use = m == kNegInf ? 0.f : m;
  // lane holds dimensions lane + 64 j (j < PER); the last group may be partial
  constexpr int PER = (D + 63) / 64;
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) acc[j] = 0.f;
  float lsum = 0.f;
  const float* po = a.part_o + rh * npart * D + lane;
  for (int p0 = 0; p0 < npart; p0 += 64) {
    // weight of partial p0 + lane (0 for empty partials and past the end)
    const int p = p0 + lane;
    const float mp = p < npart ? ml[2 * p] : kNegInf;
    const float wl = mp == kNegInf ? 0.f : fast_exp2(mp - m_use);
    lsum += p < npart ? wl * ml[2 * p + 1] : 0.f;
    const int n = min(64, npart - p0);
    int i = 0;
    for (; i + 4 <= n; i += 4) {
      float x[4][PER], wv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wv[u] = __shfl(wl, i + u, 64);
#pragma unroll
        for (int j = 0; j < PER; ++j) x[u][j] = 64 * j + lane < D ? po[(int64_t)(p0 + i + u) * D + 64 * j] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < PER; ++j) acc[j] += wv[u] != 0.f ? wv[u] * x[u][j] : 0.f;
    }
    for (; i < n; ++i) {
      const float wv = __shfl(wl, i, 64);
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const float x = 64 * j + lane < D ? po[(int64_t)(p0 + i) * D + 64 * j] : 0.f;
        acc[j] += wv != 0.f ? wv * x : 0.f;
      }
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
  // lsum is exactly 0 only for a row that saw no key; a NaN score gives a NaN
  // sum, which must reach out and lse rather than read as an empty row
  const float inv = lsum != 0.f ? 1.f / lsum : 0.f;
  T* op = (T*)a.out + rh * D;
#pragma unroll
  for (int j = 0; j < PER; ++j)
    if (64 * j + lane < D) op[64 * j + lane] = (T)(acc[j] * inv);
  if (lane == 0) {
    const int64_t row = rh / a.heads;
    const int h = (int)(rh % a.heads);
    a.lse[(int64_t)h * a.total_q + row] = lsum != 0.f ? (m + fast_log2(lsum)) * kLn2 : kNegInf;
  }
}

template <typename F>
hipError_t launch(F kernel, int64_t grid, hipStream_t stream, const DecArgs& a) {
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_t(int head_dim, bool causal, int64_t grid, int64_t grid_c, const DecArgs& a,
                           hipStream_t stream) {
  hipError_t e;
  switch (head_dim) {
    case 64: e = causal ? launch(decode16_kernel<T, 64, true>, grid, stream, a)
                        : launch(decode16_kernel<T, 64, false>, grid, stream, a); break;
    case 96: e = causal ? launch(decode16_kernel<T, 96, true>, grid, stream, a)
                        : launch(decode16_kernel<T, 96, false>, grid, stream, a); break;
    case 128: e = causal ? launch(decode16_kernel<T, 128, true>, grid, stream, a)
                         : launch(decode16_kernel<T, 128, false>, grid, stream, a); break;
    case 256: e = causal ? launch(decode16_kernel<T, 256, true>, grid, stream, a)
                         : launch(decode16_kernel<T, 256, false>, grid, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || grid_c == 0) return e;
  switch (head_dim) {
    case 64: return launch(decode_combine_kernel<T, 64>, grid_c, stream, a);
    case 96: return launch(decode_combine_kernel<T, 96>, grid_c, stream, a);
    case 128: return launch(decode_combine_kernel<T, 128>, grid_c, stream, a);
    default: return launch(decode_combine_kernel<T, 256>, grid_c, stream, a);
  }
}

hipError_t launch_decode_f32(int head_dim, bool causal, int64_t grid, int64_t grid_c, const DecArgs& a,
                             hipStream_t stream) {
  hipError_t e;
  switch (head_dim) {
    case 64: e = causal ? launch(decode_f32_kernel<64, true>, grid, stream, a)
                        : launch(decode_f32_kernel<64, false>, grid, stream, a); break;
    case 96: e = causal ? launch(decode_f32_kernel<96, true>, grid, stream, a)
                        : launch(decode_f32_kernel<96, false>, grid, stream, a); break;
    case 128: e = causal ? launch(decode_f32_kernel<128, true>, grid, stream, a)
                         : launch(decode_f32_kernel<128, false>, grid, stream, a); break;
    case 256: e = causal ? launch(decode_f32_kernel<256, true>, grid, stream, a)
                         : launch(decode_f32_kernel<256, false>, grid, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || grid_c == 0) return e;
  switch (head_dim) {
    case 64: return launch(decode_combine_kernel<float, 64>, grid_c, stream, a);
    case 96: return launch(decode_combine_kernel<float, 96>, grid_c, stream, a);
    case 128: return launch(decode_combine_kernel<float, 128>, grid_c, stream, a);
    default: return launch(decode_combine_kernel<float, 256>, grid_c, stream, a);
  }
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, bool causal, const DecArgs& a, hipStream_t stream) {
  const int64_t grid = (int64_t)a.batch * a.kv_heads * a.num_splits;
  const int64_t grid_c = ((int64_t)a.total_q * a.heads + 3) / 4;
  if (grid == 0) return hipSuccess;
  if (dtype == 0) return launch_decode_f32(head_dim, causal, grid, grid_c, a, stream);
  if (dtype == 1) return launch_decode_t<__bf16>(head_dim, causal, grid, grid_c, a, stream);
  if (dtype == 2) return launch_decode_t<_Float16>(head_dim, causal, grid, grid_c, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa
