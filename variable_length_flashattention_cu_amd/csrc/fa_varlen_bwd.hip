// fa_varlen_bwd.hip -- gfx950 kernels for the backward pass of exact attention
// over packed variable-length sequences (bf16/fp16 at head_dim 64, 96, 128 and
// 256; fp32 at 64, 96 and 128).
//
// Organisation (zepes.com "Comprendiendo Flash-Atención y Flash-Atención-2",
// section "FashAttention v1" (sic)): each workgroup owns a block of key columns
// of one sequence and one key/value head; it recomputes the attention
// probabilities of its block from the forward pass's log-sum-exp instead of
// reading a stored score matrix, accumulates dK and dV of its keys in
// registers, and adds its share of dQ to a float32 accumulator with atomic
// operations.  With several query heads per key/value head the workgroup walks
// all of them, so dK and dV of a key/value head are complete when it ends.
//
// Per (sequence, query head), with the forward definition S = scale Q K^T,
// P = softmax(S) over visible keys, O = P V, the chain rule gives
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   D_i = rowsum(dO_i * O_i),
//   dQ = scale dS K,   dK = scale dS^T Q,
// where P_ij = exp(S_ij - lse_i) is rebuilt from the forward's lse
// (D_i equals rowsum(P * dP) because O_i = sum_j P_ij v_j).
//
// Three launches:
//   bwd_prep_kernel  D_i for every (row, head) and a zeroed dQ accumulator;
//   bwd16w_kernel    one workgroup per (256-key block, key/value head): dK, dV
//                    of the block and atomic dQ contributions (16-bit inputs,
//                    head_dim up to 128), or bwd_gen_kernel (fp32 inputs on
//                    64-key blocks, 16-bit head_dim 256 on 128-key blocks);
//   bwd_dq_kernel    dq = accumulator (already scaled) in the input type.
//
// Workgroup layout (8 wavefronts; wave w owns the 32 keys of key group w of
// the 256-key block; one 32-row query block per step):
//   * K and V of the block are staged in LDS once per item and give the B
//     operands of S = Q K^T and dP = dO V^T (contraction over head_dim); Q and
//     dO rows are read from LDS in the permuted row order of the forward
//     kernels, so that register r of lane half g of the 32x32 accumulators
//     holds query row 16g + r, and lane l32 takes key 32w + pi(l32) (pi: the
//     same permutation, which keeps the swizzled K and V reads conflict-free).
//   * That is the B-operand layout of dV^T = dO^T P and dK^T = Q^T dS
//     (contraction over the 32 query rows), whose A operands Q^T and dO^T come
//     from the row-major tiles by transposing LDS reads.  dK^T and dV^T
//     accumulate in registers.
//   * dS goes to LDS row-major; dQ = dS K reads it with K^T (transposing
//     reads of the K block), contracted over all 256 keys of the block, and
//     adds it to the float32 accumulator.  These atomic additions (D per query
//     row and key block) limited 128-key blocks at head_dim 128: the L2
//     caches retire about one lane's atomic per channel and clock.
//   * Q, dO, lse and D of the next query block are loaded into registers
//     while the current one is computed and stored into LDS after the
//     mid-step barrier, when no read of the current block remains.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "fa_varlen_device.h"
#include "fa_varlen_launch.h"
#include "fa_varlen_tiling.h"
#include "fa_varlen_bwd_tiling.h"

namespace fa {
namespace {

constexpr float kLog2eF = 1.4426950408889634074f;
constexpr int kBwdBNWide = 256;  // keys per work item (8 key groups of 32)

template <typename T>
__device__ __forceinline__ float half_to_f32(uint32_t bits16);
template <>
__device__ __forceinline__ float half_to_f32<__bf16>(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
template <>
__device__ __forceinline__ float half_to_f32<_Float16>(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
template <typename T>
__device__ __forceinline__ uint16_t f32_to_bits(float x) {
  return __builtin_bit_cast(uint16_t, (T)x);
}

// ---------------------------------------------------------------------------
// D_i = rowsum(dout * out) and the zeroed dq accumulator
// ---------------------------------------------------------------------------
// Elements of T in 16 bytes, and lanes per (row, head) pair: the row's
// 16-byte chunks rounded up to a power of two (16-bit head_dim 96: 12 chunks
// on 16 lanes, the last 4 idle).
template <typename T>
constexpr int chunk_elems() { return 16 / (int)sizeof(T); }
template <typename T, int D>
constexpr int pair_lanes() {
  constexpr int CH = D / chunk_elems<T>();
  return CH <= 8 ? 8 : (CH <= 16 ? 16 : (CH <= 32 ? 32 : 64));
}

template <typename T>
__device__ __forceinline__ float chunk_dot(u32x4 o, u32x4 g) {
  float dot = 0.f;
  if constexpr (std::is_same<T, float>::value) {
#pragma unroll
    for (int e = 0; e < 4; ++e) dot += __uint_as_float(o[e]) * __uint_as_float(g[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dot += half_to_f32<T>(o[e] & 0xffffu) * half_to_f32<T>(g[e] & 0xffffu);
      dot += half_to_f32<T>(o[e] >> 16) * half_to_f32<T>(g[e] >> 16);
    }
  }
  return dot;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int EPC = chunk_elems<T>();
  constexpr int CH = D / EPC;              // 16-byte chunks per (row, head)
  constexpr int LP = pair_lanes<T, D>();   // lanes per pair
  constexpr int PAIRS = 256 / LP;          // (row, head) pairs per workgroup
  const int tid = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * PAIRS + tid / LP;  // row * heads + head
  const int c = tid % LP;
  const int64_t npairs = (int64_t)a.total_q * a.heads;
  float dot = 0.f;
  if (p < npairs && c < CH) {
    const T* op = (const T*)a.out + p * D + EPC * c;
    const T* gp = (const T*)a.dout + p * D + EPC * c;
    dot = chunk_dot<T>(*(const u32x4*)op, *(const u32x4*)gp);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < EPC; e += 4) *(f32x4*)(a.dq_acc + p * D + EPC * c + e) = z;
  }
#pragma unroll
  for (int off = LP / 2; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
  if (p < npairs && c == 0) {
    const int64_t row = p / a.heads;
    const int h = (int)(p % a.heads);
    a.drow[(int64_t)h * a.total_q + row] = dot;
  }
}

// ---------------------------------------------------------------------------
// dq = accumulator (the scale is applied when the atomics add) in the input type
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int EPC = chunk_elems<T>();
  constexpr int CH = D / EPC;
  constexpr int LP = pair_lanes<T, D>();
  constexpr int PAIRS = 256 / LP;
  const int tid = threadIdx.x;
  const int64_t p = (int64_t)blockIdx.x * PAIRS + tid / LP;
  const int c = tid % LP;
  const int64_t rows = a.cu_q[a.batch];  // rows past the last sequence are not written
  if (p < rows * a.heads && c < CH) {
    const float* src = a.dq_acc + p * D + EPC * c;
    if constexpr (std::is_same<T, float>::value) {
      *(f32x4*)((float*)a.dq + p * D + EPC * c) = *(const f32x4*)src;
    } else {
      const f32x4 x0 = *(const f32x4*)src;
      const f32x4 x1 = *(const f32x4*)(src + 4);
      u32x4 r;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        r[e] = (uint32_t)f32_to_bits<T>(x0[2 * e]) | ((uint32_t)f32_to_bits<T>(x0[2 * e + 1]) << 16);
        r[e + 2] = (uint32_t)f32_to_bits<T>(x1[2 * e]) | ((uint32_t)f32_to_bits<T>(x1[2 * e + 1]) << 16);
      }
      *(u32x4*)((uint16_t*)a.dq + p * D + EPC * c) = r;
    }
  }
}

// ---------------------------------------------------------------------------
// work items: (key block j of sequence b, key/value head hk)
// ---------------------------------------------------------------------------
struct ColItem {
  int b, j, hk;
  int q_start, Lq, k_start, Lk;
};

template <int BN>
__device__ __forceinline__ bool decode_col(const BwdArgs& a, ColItem& w) {
  // each XCD (workgroup i runs on XCD i % 8) takes a contiguous slice of items
  const uint32_t per_xcd = gridDim.x >> 3;
  const uint32_t work = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  if (work >= (uint32_t)a.n_work) return false;
  w.hk = (int)(work / (uint32_t)a.tmax);
  const int t = (int)(work % (uint32_t)a.tmax);
  int b, j;
  if (a.by_block) {
    // key block j of every sequence before block j + 1 of any: under a causal
    // mask the first key blocks see the most query rows, so the longest items
    // are dispatched first and the short ones fill in at the end
    j = t / a.batch;
    b = t - j * a.batch;
    if (j * BN >= a.cu_k[b + 1] - a.cu_k[b]) return false;
  } else {
    const int T = a.blk_start[a.batch];
    if (t >= T) return false;
    int lo = 0, hi = a.batch;  // invariant: blk_start[lo] <= t < blk_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.blk_start[mid] <= t) lo = mid; else hi = mid;
    }
    b = lo;
    j = t - a.blk_start[lo];
  }
  w.b = b;
  w.j = j;
  w.q_start = a.cu_q[b];
  w.Lq = a.cu_q[b + 1] - w.q_start;
  w.k_start = a.cu_k[b];
  w.Lk = a.cu_k[b + 1] - w.k_start;
  return true;
}

// ---------------------------------------------------------------------------
// the backward workgroup
// ---------------------------------------------------------------------------
// Layout of the Q, dO and K tiles (read both with 16-byte operand reads and
// with transposing reads; V keeps the K-style layout tiling::ks_index):
// bwdt::tq_index, with the reasoning in fa_varlen_bwd_tiling.h.
using bwdt::tq_index;
using bwdt::tq_swz;

// Register-staged tile -> LDS in the tq_index layout
template <int D, typename Tile>
__device__ __forceinline__ void store_tq(const Tile& t, uint16_t* dst, int tid) {
#pragma unroll
  for (int i = 0; i < Tile::K_PER_THREAD; ++i) {
    const int c = tid + i * Tile::THREADS;
    *(u32x4*)(dst + tq_index<D>(Tile::k_row(c), Tile::k_chunk(c))) = t.kreg[i];
  }
}

// Direct global -> LDS staging of a row-major tile of ROWS rows x D 16-bit
// elements in the swizzled K-style layout (tiling::ks_index<D>), or with TQ in
// the tq_index layout: each lane's 16 bytes land at LDS chunk position
// p = 64 * instruction + lane, so the lane loads the logical chunk that the
// swizzle stores there.  Rows at or past `valid` read as zeros (buffer range
// check); no registers hold the data.
template <int D, int ROWS, int NW, bool TQ>
__device__ __forceinline__ void lds_load_rows(uint16_t* dst, const uint16_t* base, int64_t row_stride, int valid,
                                              int wave, int lane) {
  constexpr int CPR = tiling::k_stride<D>() / 8;  // 16-byte slots per LDS row
  constexpr int PER_WAVE = ROWS * CPR / (64 * NW);  // instructions per wave
  static_assert(ROWS * CPR % (64 * NW) == 0, "tile must split into whole wave loads");
  const __amdgpu_buffer_rsrc_t r =
      buffer_rsrc(base, tiling::head_rows_bytes(max(0, min(ROWS, valid)), row_stride, D, 2));
#pragma unroll
  for (int i = 0; i < PER_WAVE; ++i) {
    const int seg = wave * PER_WAVE + i;
    const int p = seg * 64 + lane;
    const int row = p / CPR;
    int lc = (p % CPR) ^ (TQ ? tq_swz<D>(row) : tiling::k_swz<tiling::k_stride<D>()>(row));
    if (D == 96 && lc >= D / 8) lc -= 8;  // a padding slot: any chunk of the row (never read)
    const uint32_t off = ((uint32_t)row * (uint32_t)row_stride + (uint32_t)lc * 8u) * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + seg * 512), 16, off,
                                             0, 0, 0);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// The value, hidden from the optimiser (an empty asm that may modify it).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i reads 8 bytes at row r0 + i/4, columns c0 + 4(i%4) .. +3 of a
// row-major swizzled tile, and the hardware hands lane i the four elements
// X[r0 + e][c0 + i], e = 0..3 (column c0 + i, four consecutive rows).
template <int D>
__device__ __forceinline__ s16x4 tr_read4(const uint16_t* tile, int r0, int c0, int i) {
  const int row = r0 + (i >> 2), col = c0 + 4 * (i & 3);
  const uint16_t* p = tile + tq_index<D>(row, col >> 3) + (col & 7);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}

// LDS accesses at absolute LDS byte addresses (the 256-key workgroup's main
// loop, fa_varlen_bwd_tiling.h): a constant added to the address becomes the
// instruction's offset field.
template <typename V>
__device__ __forceinline__ V lds_rd(uint32_t addr) {
  return *(const __attribute__((address_space(3))) V*)(uintptr_t)addr;
}
__device__ __forceinline__ void lds_wr16(uint32_t addr, uint16_t v) {
  *(__attribute__((address_space(3))) uint16_t*)(uintptr_t)addr = v;
}
__device__ __forceinline__ s16x4 lds_rd_tr(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(uintptr_t)addr);
}
// two transposing reads (rows r0..r0+3 and r0+4..r0+7) as one MFMA operand
template <typename V8>
__device__ __forceinline__ V8 lds_rd_tr8(uint32_t lo_addr, uint32_t hi_addr) {
  const s16x4 lo = lds_rd_tr(lo_addr);
  const s16x4 hi = lds_rd_tr(hi_addr);
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}

// 8 consecutive rows r0 .. r0+7 of column c0 + i as one MFMA operand
template <typename V8, int D>
__device__ __forceinline__ V8 tr_read8(const uint16_t* tile, int r0, int c0, int i) {
  const s16x4 lo = tr_read4<D>(tile, r0, c0, i);
  const s16x4 hi = tr_read4<D>(tile, r0 + 4, c0, i);
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}

// Scheduling order of a block of NM MFMAs fed by NR LDS reads (NR a multiple
// of NM): the first AHEAD reads, then each MFMA followed by the reads of a
// later one, so that AHEAD reads are in flight ahead of their use.
template <int I, int NM, int NR, int AHEAD>
__device__ __forceinline__ void read_ahead_tail() {
  if constexpr (I < NM) {
    constexpr int PER = NR / NM;
    constexpr int LEFT = NR - AHEAD - I * PER;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if constexpr (LEFT > 0) __builtin_amdgcn_sched_group_barrier(0x100, LEFT < PER ? LEFT : PER, 0);
    read_ahead_tail<I + 1, NM, NR, AHEAD>();
  }
}
template <int NM, int NR, int AHEAD>
__device__ __forceinline__ void read_ahead_schedule() {
  static_assert(NR % NM == 0 && AHEAD <= NR, "reads per MFMA");
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // LDS reads
  read_ahead_tail<0, NM, NR, AHEAD>();
}

// Query block s of a work item (Q, dO, lse, D): loaded into registers while
// the previous block is computed, then stored into an LDS buffer.  Rows past
// the sequence read as zeros.  Step s covers query head
// kv_head * head_group + s / nblk and rows (i_begin + s % nblk) * BM ...
template <int D, int BM, int NW>
struct BlockStage {
  // NW staging wavefronts; with more threads in the workgroup, thread t
  // stages as thread t % (64 NW) (the same chunks twice, equal values)
  static constexpr int NT = 64 * NW;
  Tile16<D, BM, NW> tq, tdo;
  float lse_v = 0.f, dr_v = 0.f;

  __device__ __forceinline__ void load(const BwdArgs& a, const ColItem& w, int s, int nblk, int i_begin, int tid) {
    const int h = w.hk * a.head_group + s / nblk;
    const int r0 = (i_begin + s % nblk) * BM;
    const int64_t rs = a.row_stride;
    const uint16_t* qh = (const uint16_t*)a.q + (int64_t)w.q_start * rs + (int64_t)h * D;
    const uint16_t* doh = (const uint16_t*)a.dout + (int64_t)w.q_start * rs + (int64_t)h * D;
    tq.load_k(qh, rs, r0, w.Lq, tid % NT);
    tdo.load_k(doh, rs, r0, w.Lq, tid % NT);
    // lse and D of the block's rows: branch-free buffer loads whose range
    // check (the rows of the sequence) reads rows past its end as zero
    const int64_t at = (int64_t)h * a.total_q + w.q_start + r0;
    const uint32_t bytes = (uint32_t)max(0, min(BM, w.Lq - r0)) * 4u;
    // lane l takes row (l % 16) + 16 * ((l / 32) % 2): each 16-lane row of the
    // wave then holds the 16 rows that one lane half needs (see probs16)
    const uint32_t off = (uint32_t)((tid & 15) | ((tid & 32) >> 1)) * 4u;
    lse_v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.lse + at, bytes), (int)off, 0, 0));
    dr_v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.drow + at, bytes), (int)off, 0, 0));
  }
};

// ---------------------------------------------------------------------------
// the backward workgroup: 256-key work items
// ---------------------------------------------------------------------------
// 8 wavefronts, one per 32-key group of a 256-key block, on 32-row query
// blocks.  The dQ contribution of a query block is contracted over all 256
// keys before it is added, which halves the float32 atomic additions per
// (row, key) against 128-key items.  At head_dim 128, LDS holds the K and V
// blocks (64 KB each), dS (16 KB) and one Q/dO block (16 KB): 160 KB, all of
// it (88 KB at head_dim 64).  The next block's Q/dO are stored after the
// mid-step barrier (no Q/dO reads remain in the step), so one buffer
// suffices; lse and D of the step's rows stay in registers (lane l holds row
// l % 32) and reach the lanes that need them through ds_bpermute.
//
// dQ uses 16x16x32 MFMAs (gfx950 layout, lane l, i = l % 16, G = l / 16:
// A row i, k = 8G..8G+7; B column i, k = 8G..8G+7; accumulator register r:
// row 4G + r, column i), one 16x16 tile of dQ per (wave, tile) pair so that no
// two waves add to the same element.  Row tile t takes the query rows
// 8t..8t+7 and 16+8t..16+8t+7, whose swizzled dS rows sit in 16 distinct
// bank groups.
__device__ __forceinline__ int dq16_row(int t, int i) {  // block row of A-row i of 16-row tile t
  return (i < 8 ? 0 : 8) + 8 * t + i;
}

// P and dS / scale (dS without the softmax scale, which dK and dQ apply at
// the end) of the lane's 16 rows 16g + r.  lse (log2
// units) and D of row 16g + r come from lane r of the lane's 16-lane row (lane
// l holds row (l % 16) + 16 * ((l / 32) % 2)), by a DPP row broadcast: vector
// ALU work instead of two LDS permutes per row.
// With MASKED, element r counts only if lo <= r < hi (the lane's key visible
// to row 16g + r); blocks that lie wholly inside the visible region skip the test.
template <int R>
__device__ __forceinline__ float row_bcast(float x) {
  // DPP row_newbcast:n writes lane n of each 16-lane row to every lane of the
  // row, so no lane keeps an old value (none is materialised)
  constexpr int kRowNewBcast = 0x150;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), kRowNewBcast + R, 0xf, 0xf, true));
}

template <bool MASKED, typename T, int R>
__device__ __forceinline__ void probs16_row(const f32x16& sc, const f32x16& dp, float cur_lse, float cur_dr, int lo,
                                            int hi, float scale_log2, float scale, typename Elem16<T>::v8 (&p16)[2],
                                            typename Elem16<T>::v8 (&ds16)[2]) {
  const float lse2 = row_bcast<R>(cur_lse);
  const float drr = row_bcast<R>(cur_dr);
  float pr = fast_exp2(__builtin_fmaf(sc[R], scale_log2, -lse2));
  if constexpr (MASKED) pr = (R >= lo && R < hi) ? pr : 0.f;
  const float dsr = pr * (dp[R] - drr);  // the softmax scale is applied to dK and dQ
  p16[R >> 3][R & 7] = (T)pr;
  ds16[R >> 3][R & 7] = (T)dsr;
}

template <bool MASKED, typename T, int... R>
__device__ __forceinline__ void probs16_rows(const f32x16& sc, const f32x16& dp, float cur_lse, float cur_dr, int lo,
                                             int hi, float scale_log2, float scale, typename Elem16<T>::v8 (&p16)[2],
                                             typename Elem16<T>::v8 (&ds16)[2], std::integer_sequence<int, R...>) {
  (probs16_row<MASKED, T, R>(sc, dp, cur_lse, cur_dr, lo, hi, scale_log2, scale, p16, ds16), ...);
}

template <bool MASKED, typename T>
__device__ __forceinline__ void probs16(const f32x16& sc, const f32x16& dp, float cur_lse, float cur_dr, int /*g*/,
                                        int lo, int hi, float scale_log2, float scale,
                                        typename Elem16<T>::v8 (&p16)[2], typename Elem16<T>::v8 (&ds16)[2]) {
  probs16_rows<MASKED, T>(sc, dp, cur_lse, cur_dr, lo, hi, scale_log2, scale, p16, ds16,
                          std::make_integer_sequence<int, 16>{});
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(512, 2) void bwd16w_kernel(BwdArgs a) {
  constexpr int BN = kBwdBNWide, BM = 32, NW = 8;
  constexpr int KSTEPS = D / 16;    // k-steps over head_dim
  constexpr int DB = D / 32;        // 32-dim tiles
  constexpr int CT = D / 16;        // 16-column tiles of dQ
  // 16x16 dQ tiles per wave: at D=128 and 96 wave w < CT takes column tile w of
  // both row tiles (one K^T operand feeds two MFMAs; at 96 waves 6 and 7 have
  // none), at D=64 one tile per wave
  constexpr int TPW = D == 64 ? 1 : 2;
  constexpr int DQW = 2 * CT / TPW;  // wavefronts with dQ tiles
  constexpr int NWS = BM * D / 8 / 64 < NW ? BM * D / 8 / 64 : NW;  // staging wavefronts
  static_assert(D == 64 || D == 96 || D == 128, "backward head_dim");
  constexpr int KSB = tiling::k_stride<D>();  // LDS row pitch of the K, V, Q and dO tiles
  using E = Elem16<T>;
  typedef typename E::v8 v8;

  // 1024-byte alignment: the chunk XOR terms of the main loop's addresses
  // (bits 4-8) must not meet bits of a tile's base address
  __shared__ __attribute__((aligned(1024))) uint16_t lds_k[BN * KSB];   // K block, row-major
  __shared__ __attribute__((aligned(1024))) uint16_t lds_v[BN * KSB];   // V block, row-major
  __shared__ __attribute__((aligned(1024))) uint16_t lds_ds[BM * BN];   // dS, row-major
  __shared__ __attribute__((aligned(1024))) uint16_t lds_qdo[2][BM * KSB];  // query block: Q, then dO
  uint16_t* const lds_q = lds_qdo[0];
  uint16_t* const lds_do = lds_qdo[1];
  constexpr uint32_t kDoOff = 2 * BM * KSB;  // bytes from the Q tile to the dO tile

  ColItem w;
  if (!decode_col<BN>(a, w)) return;

  const int tid0 = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  int tid = tid0, lane = tid0 & 63;
  int l32 = lane & 31, g = lane >> 5;
  int li = lane & 15, lg = lane >> 4;
  const int key0 = w.j * BN;
  const int klane = 32 * wave + tiling::key_of_arow(l32);  // this lane's key in the block
  const int kcol = key0 + klane;                            // in the sequence
  const int shift = w.Lk - w.Lq;
  const int64_t rs = a.row_stride, rsk = a.kv_row_stride;
  const uint16_t* __restrict__ kbase = (const uint16_t*)a.k + (int64_t)w.k_start * rsk + (int64_t)w.hk * D;
  const uint16_t* __restrict__ vbase = (const uint16_t*)a.v + (int64_t)w.k_start * rsk + (int64_t)w.hk * D;
  lds_load_rows<D, BN, NW, true>(lds_k, kbase + (int64_t)key0 * rsk, rsk, w.Lk - key0, wave, lane);
  lds_load_rows<D, BN, NW, false>(lds_v, vbase + (int64_t)key0 * rsk, rsk, w.Lk - key0, wave, lane);

  const int i_begin = CAUSAL ? max(0, key0 - shift) / BM : 0;
  const int i_end = (w.Lq + BM - 1) / BM;
  const int nblk = max(0, i_end - i_begin);
  const int nsteps = a.head_group * nblk;

  BlockStage<D, BM, NWS> stage;
  float cur_lse = 0.f, cur_dr = 0.f;  // lse (log2 units) and D of row (l % 16) + 16 ((l / 32) % 2) of the step

  f32x16 dkt[DB], dvt[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dkt[db] = f32x16{};
    dvt[db] = f32x16{};
  }

  if (nsteps > 0) {
    stage.load(a, w, 0, nblk, i_begin, tid);
    store_tq<D>(stage.tq, lds_q, tid % (64 * NWS));
    store_tq<D>(stage.tdo, lds_do, tid % (64 * NWS));
    cur_lse = stage.lse_v * kLog2eF;
    cur_dr = stage.dr_v;
  }
  __syncthreads();
  // Every load issued so far (K, V blocks, the first query block) has
  // landed.  Without this wait the compiler keeps the pre-loop loads pending
  // at the loop head and places vmcnt waits inside the loop; those then also
  // wait, every step, for the previous step's dQ atomics, since vector memory
  // operations complete in order.
  __builtin_amdgcn_s_waitcnt(0);

  // the K operand of S = Q K^T is the same for every step: held in registers
  v8 kreg[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) kreg[ks] = *(const v8*)(lds_k + tq_index<D>(klane, 2 * ks + g));

  // Lane parts of the main loop's LDS addresses (fa_varlen_bwd_tiling.h):
  // every access there is (lane part ^ loop-index chunk term) + loop-index
  // offset.  They pass through an empty asm each step, so the compiler keeps
  // these six registers rather than one register per address.
  // The tiles' base addresses are included (their bits below 10 are zero).
  const uint32_t at_qdo = lds_address(lds_qdo), at_v = lds_address(lds_v), at_k = lds_address(lds_k),
                 at_ds = lds_address(lds_ds);
  const uint32_t a_op_q0 = at_qdo + bwdt::op_lane_tq<D>(tiling::key_of_arow(l32), g);  // Q, dO operand reads
  const uint32_t a_op_v0 = at_v + bwdt::op_lane_ks<D>(klane, g);                       // V operand reads
  const uint32_t a_trq0 = at_qdo + bwdt::trq_lane<D>(li, lg);                          // dO^T, Q^T reads
  const uint32_t a_trk0 = at_k + bwdt::trk_lane<D>(li, lg);                            // K^T reads (dQ)
  const uint32_t a_dsa0 = at_ds + bwdt::dsa_lane(li, lg);                              // dS reads (dQ)
  const uint32_t a_dss0 = at_ds + bwdt::dss_lane(klane, g);                            // dS stores
  for (int s = 0; s < nsteps; ++s) {
    tid = opaque(tid0);
    lane = tid & 63;
    g = lane >> 5;
    li = lane & 15;
    lg = lane >> 4;
    const uint32_t a_op_q = opaque(a_op_q0), a_op_v = opaque(a_op_v0), a_trq = opaque(a_trq0),
                   a_trk = opaque(a_trk0), a_dsa = opaque(a_dsa0), a_dss = opaque(a_dss0);
    const int h = w.hk * a.head_group + s / nblk;
    const int r0 = (i_begin + s % nblk) * BM;
    stage.load(a, w, min(s + 1, nsteps - 1), nblk, i_begin, tid);

    // S = Q K^T and dP = dO V^T (rows permuted: register r of half g = row 16g + r)
    f32x16 sc = f32x16{}, dp = f32x16{};
    {
      constexpr int PF = 2;
      v8 aq[PF + 1], ad[PF + 1], bv[PF + 1];
      auto fetch = [&](int ks) __attribute__((always_inline)) {
        const int i = ks % (PF + 1);
        aq[i] = lds_rd<v8>(a_op_q ^ bwdt::op_xor(ks));
        ad[i] = lds_rd<v8>((a_op_q ^ bwdt::op_xor(ks)) + kDoOff);
        bv[i] = lds_rd<v8>(a_op_v ^ bwdt::op_xor(ks));
      };
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) fetch(ks);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        if (ks + PF < KSTEPS) fetch(ks + PF);
        const int i = ks % (PF + 1);
        sc = E::mfma(aq[i], kreg[ks], sc);
        dp = E::mfma(ad[i], bv[i], dp);
      }
    }
    __builtin_amdgcn_sched_barrier(0);

    // P and dS.  Row q = r0 + 16g + r sees the lane's key iff q < Lq, the key
    // is in the sequence and (causal) key <= q + shift: lo <= r < hi below.
    v8 p16[2], ds16[2];
    const bool full = r0 + BM <= w.Lq && key0 + BN <= w.Lk && (!CAUSAL || key0 + BN - 1 <= r0 + shift);
    if (full) {
      probs16<false, T>(sc, dp, cur_lse, cur_dr, g, 0, 16, a.scale_log2, a.scale, p16, ds16);
    } else {
      const int qb = r0 + 16 * g;
      const int lo = CAUSAL ? kcol - shift - qb : -1;
      const int hi = kcol < w.Lk ? w.Lq - qb : lo;  // an empty range when the key is past the sequence
      probs16<true, T>(sc, dp, cur_lse, cur_dr, g, lo, hi, a.scale_log2, a.scale, p16, ds16);
    }

    // dV^T += dO^T P and dK^T += Q^T dS (contraction over the 32 rows)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint32_t lo = (a_trq ^ bwdt::trq_xor<D>(db, t, 0)) + bwdt::trq_add<D>(t, 0);
        const uint32_t hi = (a_trq ^ bwdt::trq_xor<D>(db, t, 1)) + bwdt::trq_add<D>(t, 1);
        const v8 adt = lds_rd_tr8<v8>(lo + kDoOff, hi + kDoOff);
        const v8 aqt = lds_rd_tr8<v8>(lo, hi);
        dvt[db] = E::mfma(adt, p16[t], dvt[db]);
        dkt[db] = E::mfma(aqt, ds16[t], dkt[db]);
      }
    read_ahead_schedule<4 * DB, 8 * DB, 8>();

    // dS -> LDS, row-major [row][key].  The 16-bit values are taken from the
    // packed operand registers as whole words (element-wise access to the
    // 16-bit vector was miscompiled into one element per half).
    {
      const u32x4 w0 = __builtin_bit_cast(u32x4, ds16[0]);
      const u32x4 w1 = __builtin_bit_cast(u32x4, ds16[1]);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t word = r < 8 ? w0[(r & 7) >> 1] : w1[(r & 7) >> 1];
        lds_wr16((a_dss ^ bwdt::dss_xor(r)) + bwdt::dss_add(r), (uint16_t)((r & 1) ? (word >> 16) : word));
      }
    }
    __syncthreads();

    // dQ rows r0..r0+31 over the 256 keys: 16x16 tiles (row tile rt, dims
    // 16*ct..+15); D=128 and 96: wave w < CT takes column tile w of both row
    // tiles (one K^T operand feeds two MFMAs), D=64: column tile w % 4 of row
    // tile w / 4
    {
      const bool has_dq = DQW >= NW || wave < DQW;  // wave-uniform
      const int ct = wave % CT;
      const int rt0 = TPW == 2 ? 0 : wave / CT;
      f32x4 acc[TPW];
#pragma unroll
      for (int u = 0; u < TPW; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (has_dq) {
        // K^T of column tile ct: the chunk terms of the two row halves are
        // wave-uniform, so each costs one XOR per step
        const uint32_t k_lo = a_trk ^ bwdt::trk_xor(ct, 0), k_hi = a_trk ^ bwdt::trk_xor(ct, 1);
        // at D=64 the row tile is wave-uniform but not a constant: fold its
        // offset (bit 12, clear of the chunk terms) into the lane part
        const uint32_t a_ds = TPW == 2 ? a_dsa : a_dsa + bwdt::dsa_add(rt0);
#pragma unroll
        for (int kk = 0; kk < BN / 32; ++kk) {
          const v8 bkt = lds_rd_tr8<v8>(k_lo + bwdt::trk_add<D>(kk, 0), k_hi + bwdt::trk_add<D>(kk, 1));
#pragma unroll
          for (int u = 0; u < TPW; ++u) {
            const uint32_t off = TPW == 2 ? (a_ds ^ bwdt::dsa_xor(kk)) + bwdt::dsa_add(u) : a_ds ^ bwdt::dsa_xor(kk);
            const v8 av = lds_rd<v8>(off);
            acc[u] = Mfma16<T>::run(av, bkt, acc[u]);
          }
        }
        read_ahead_schedule<TPW * (BN / 32), (TPW + 2) * (BN / 32), 8>();
      }
      // the next query block: no Q/dO reads remain in this step
      store_tq<D>(stage.tq, lds_q, tid % (64 * NWS));
      store_tq<D>(stage.tdo, lds_do, tid % (64 * NWS));
      cur_lse = stage.lse_v * kLog2eF;
      cur_dr = stage.dr_v;
      if (has_dq) {
        // register r of tile u: block row dq16_row(rt0 + u, 4 lg + r), column 16*ct + li
        const __amdgpu_buffer_rsrc_t racc =
            buffer_rsrc(a.dq_acc + (int64_t)(w.q_start + r0) * rs + (int64_t)h * D,
                        tiling::head_rows_bytes(min(BM, w.Lq - r0), rs, D, 4));
#pragma unroll
        for (int u = 0; u < TPW; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t off = ((uint32_t)dq16_row(rt0 + u, 4 * lg + r) * (uint32_t)rs + 16 * ct + li) * 4u;
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[u][r] * a.scale, racc, (int)off, 0, 0);
          }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: dK (times the softmax scale, left out of dS) and dV of this lane's key
  if (kcol < w.Lk) {
    T* dkp = (T*)a.dk + (int64_t)(w.k_start + kcol) * rsk + (int64_t)w.hk * D;
    T* dvp = (T*)a.dv + (int64_t)(w.k_start + kcol) * rsk + (int64_t)w.hk * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        typename E::v4 k4, v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          k4[c] = (T)(dkt[db][4 * s4 + c] * a.scale);
          v4[c] = (T)dvt[db][4 * s4 + c];
        }
        const int d0 = 32 * db + 8 * s4 + 4 * g;
        *(typename E::v4*)(dkp + d0) = k4;
        *(typename E::v4*)(dvp + d0) = v4;
      }
  }
}

// ---------------------------------------------------------------------------
// the backward workgroup for fp32 inputs (head_dim 64, 96, 128) and for
// 16-bit inputs at head_dim 256: 4 wavefronts, 64 KW-key work items
// ---------------------------------------------------------------------------
// 16x16 MFMAs throughout (gfx950 layouts, lane l, i = l % 16, G = l / 16;
// accumulator register r holds row 4G + r, column i): fp32 16x16x4 (A row i,
// k = G; B column i, k = G) or 16-bit 16x16x32 (A row i, k = 8G..8G+7; B
// column i, the same k).
//   * Wave w owns the KW 16-key subtiles KW w .. KW w + KW - 1 of the item.
//     Lane (i, G) holds V (and with KW = 1 also K) of key i of each subtile,
//     head dimensions G*D/4 .. G*D/4 + D/4 - 1, in registers for the whole
//     item: the B operand of S = Q K^T and dP = dO V^T when the contraction
//     index of lane group G runs over those dimensions (Q and dO rows read
//     from LDS the same way as the A operand).  With KW = 2 the K operand is
//     read from the item's K block in LDS instead, which the wave needs for
//     dQ anyway.
//   * Each step takes 32 query rows of one query head, as two 16-row tiles u:
//     register r of tile u holds row 16u + 4G + r and key i of the subtile.
//     Those are the A operand of dV = P^T dO and dK = dS^T Q (row i = key,
//     contraction over the 32 rows): fp32 takes k-step (u, r) with row
//     16u + 4G + r on lane group G; 16-bit takes one k-step whose 8 indices of
//     group G are rows 4G + 0..3 and 16 + 4G + 0..3, the B operand coming from
//     two transposing reads of the row-major dO (or Q) tile, shared by the
//     wave's subtiles.
//   * dS goes to LDS (16-bit: transposed, [key][row], each lane's 2 x 4 rows
//     as two 8-byte stores, read back by transposing reads); dQ = dS K
//     (contraction over the item's 64 KW keys) is split into 16x16 tiles,
//     2D/64 per wave, and added to the float32 accumulator with atomic
//     additions: D additions per query row and item, so larger items need
//     fewer (at head_dim 256 they bound the pass).
// P and dS are kept without the softmax scale, which dK and dQ apply at the
// end, as in the 256-key workgroup.  The 256-key workgroup serves the 16-bit
// head dims up to 128.
constexpr int kGenBM = 32;  // query rows per step
// 16-key subtiles per wavefront: 2 at 16-bit head_dim 256 (128-key items), 1
// for fp32 (64-key items)
template <typename T, int D>
constexpr int gen_kw() { return std::is_same<T, float>::value ? 1 : 2; }

template <typename T, int D>
struct GenGeom {
  static constexpr bool F32 = std::is_same<T, float>::value;
  static constexpr int KW = gen_kw<T, D>();
  static constexpr int BN = 64 * KW;                    // keys per work item
  static constexpr int EL = (int)sizeof(T);
  static constexpr int EPC = 16 / EL;                   // elements per 16-byte chunk
  static constexpr int QP = F32 ? D + 4 : D + 8;        // Q / dO LDS row pitch (elements)
  static constexpr int KP = F32 ? D + 16 : D + 8;       // K LDS row pitch
  // dS in LDS: fp32 row-major [rows][keys], 16-bit transposed [keys][rows]
  static constexpr int SP = F32 ? BN + 4 : kGenBM + 8;
  static constexpr int DL = D / 4;                      // head dims of one lane group
  static constexpr int NV = DL / EPC;                   // 16-byte chunks of K (or V) per lane
  static constexpr int QBYTES = kGenBM * QP * EL;
  static constexpr int KBYTES = BN * KP * EL;
  static constexpr int SBYTES = (F32 ? kGenBM : BN) * SP * EL;
  static_assert(DL % EPC == 0 && (QP * EL) % 16 == 0 && (KP * EL) % 16 == 0 && (SP * EL) % 16 == 0,
                "rows must hold whole 16-byte chunks");
  static_assert(!F32 || KW == 1, "fp32 keeps one subtile per wavefront");
};
template <typename T, int D>
constexpr int gen_block_n() { return GenGeom<T, D>::BN; }

// transposing read of rows r0 .. r0+3 of column c0 + i from a row-major tile
// of 16-bit elements with row pitch P (see tr_read4)
template <int P>
__device__ __forceinline__ s16x4 gen_tr4(const uint16_t* tile, int r0, int c0, int i) {
  const uint16_t* p = tile + (r0 + (i >> 2)) * P + c0 + 4 * (i & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
}
template <typename V8, int P>
__device__ __forceinline__ V8 gen_tr8(const uint16_t* tile, int ra, int rb, int c0, int i) {
  const s16x4 lo = gen_tr4<P>(tile, ra, c0, i);
  const s16x4 hi = gen_tr4<P>(tile, rb, c0, i);
  const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(V8, v);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(256, D > 128 ? 1 : 2) void bwd_gen_kernel(BwdArgs a) {
  using Geo = GenGeom<T, D>;
  constexpr bool F32 = Geo::F32;
  constexpr int KW = Geo::KW, BN = Geo::BN, BM = kGenBM, EPC = Geo::EPC, QP = Geo::QP, KP = Geo::KP,
                SP = Geo::SP;
  constexpr int DL = Geo::DL, NV = Geo::NV, DT = D / 16;
  constexpr int DQT = 2 * D / 64;  // 16x16 dQ tiles per wave (2 row tiles x D/16 column tiles over 4 waves)
  constexpr bool KREG = KW == 1;   // K of the lane's key in registers (else read from the LDS block)
  static_assert(F32 ? (D == 64 || D == 96 || D == 128) : D == 256, "generic backward shapes");

  __shared__ __attribute__((aligned(16))) char lds_kb[Geo::KBYTES];
  __shared__ __attribute__((aligned(16))) char lds_qb[Geo::QBYTES];
  __shared__ __attribute__((aligned(16))) char lds_dob[Geo::QBYTES];
  __shared__ __attribute__((aligned(16))) char lds_dsb[Geo::SBYTES];
  __shared__ __attribute__((aligned(16))) float lds_lse[BM];
  __shared__ __attribute__((aligned(16))) float lds_dr[BM];

  ColItem w;
  if (!decode_col<BN>(a, w)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int key0 = w.j * BN;
  int kr0[KW], kc[KW];  // key of the lane in the item's block / in the sequence, per subtile
#pragma unroll
  for (int kt = 0; kt < KW; ++kt) {
    kr0[kt] = 16 * (KW * wave + kt) + li;
    kc[kt] = key0 + kr0[kt];
  }
  const int shift = w.Lk - w.Lq;
  const int64_t rs = a.row_stride, rsk = a.kv_row_stride;
  const T* kbase = (const T*)a.k + (int64_t)w.k_start * rsk + (int64_t)w.hk * D;
  const T* vbase = (const T*)a.v + (int64_t)w.k_start * rsk + (int64_t)w.hk * D;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // V (and K) of the lane's keys: head dims lg*DL .. lg*DL + DL - 1
  u32x4 vr[KW][NV];
  u32x4 kr[KREG ? KW : 1][NV];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      vr[kt][n] = zero;
      if (kc[kt] < w.Lk) vr[kt][n] = *(const u32x4*)(vbase + (int64_t)kc[kt] * rsk + lg * DL + n * EPC);
      if constexpr (KREG) {
        kr[kt][n] = zero;
        if (kc[kt] < w.Lk) kr[kt][n] = *(const u32x4*)(kbase + (int64_t)kc[kt] * rsk + lg * DL + n * EPC);
      }
    }
  // the item's K block in LDS (row-major, keys past the sequence as zeros): B operand of dQ = dS K
  for (int c = tid; c < BN * D / EPC; c += 256) {
    const int row = c / (D / EPC), ch = c % (D / EPC);
    u32x4 x = zero;
    if (key0 + row < w.Lk) x = *(const u32x4*)(kbase + (int64_t)(key0 + row) * rsk + ch * EPC);
    *(u32x4*)(lds_kb + (row * KP + ch * EPC) * Geo::EL) = x;
  }

  f32x4 dk[KW][DT], dv[KW][DT];
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      dk[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[kt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int i_begin = CAUSAL ? max(0, key0 - shift) / BM : 0;
  const int i_end = (w.Lq + BM - 1) / BM;
  const int nblk = max(0, i_end - i_begin);
  const int nsteps = a.head_group * nblk;

  for (int st = 0; st < nsteps; ++st) {
    const int h = w.hk * a.head_group + st / nblk;
    const int r0 = (i_begin + st % nblk) * BM;
    // ---- stage Q, dO, lse (log2 units) and D of rows r0 .. r0+31 (rows past the sequence as zeros)
    {
      const T* qh = (const T*)a.q + (int64_t)(w.q_start + r0) * rs + (int64_t)h * D;
      const T* doh = (const T*)a.dout + (int64_t)(w.q_start + r0) * rs + (int64_t)h * D;
      for (int c = tid; c < BM * D / EPC; c += 256) {
        const int row = c / (D / EPC), ch = c % (D / EPC);
        u32x4 x = zero, y = zero;
        if (r0 + row < w.Lq) {
          x = *(const u32x4*)(qh + (int64_t)row * rs + ch * EPC);
          y = *(const u32x4*)(doh + (int64_t)row * rs + ch * EPC);
        }
        *(u32x4*)(lds_qb + (row * QP + ch * EPC) * Geo::EL) = x;
        *(u32x4*)(lds_dob + (row * QP + ch * EPC) * Geo::EL) = y;
      }
      if (tid < BM) {
        const bool ok = r0 + tid < w.Lq;
        const int64_t at = (int64_t)h * a.total_q + w.q_start + r0 + tid;
        lds_lse[tid] = ok ? a.lse[at] * kLog2eF : 0.f;
        lds_dr[tid] = ok ? a.drow[at] : 0.f;
      }
    }
    __syncthreads();

    // ---- S = Q K^T and dP = dO V^T: subtile kt, tile u, register r <-> row 16u + 4lg + r, key kc[kt]
    f32x4 s[KW][2], dp[KW][2];
#pragma unroll
    for (int kt = 0; kt < KW; ++kt)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[kt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[kt][u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* qrow = lds_qb + ((16 * u + li) * QP + lg * DL) * Geo::EL;
      const char* dorow = lds_dob + ((16 * u + li) * QP + lg * DL) * Geo::EL;
#pragma unroll
      for (int n = 0; n < NV; ++n) {
        if constexpr (F32) {
          const f32x4 q4 = *(const f32x4*)(qrow + 16 * n), o4 = *(const f32x4*)(dorow + 16 * n);
          const f32x4 k4 = __builtin_bit_cast(f32x4, kr[0][n]), v4 = __builtin_bit_cast(f32x4, vr[0][n]);
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            s[0][u] = mfma4(q4[c], k4[c], s[0][u]);
            dp[0][u] = mfma4(o4[c], v4[c], dp[0][u]);
          }
        } else {
          typedef typename Elem16<T>::v8 v8;
          const v8 qa = *(const v8*)(qrow + 16 * n), oa = *(const v8*)(dorow + 16 * n);
#pragma unroll
          for (int kt = 0; kt < KW; ++kt) {
            v8 kb;
            if constexpr (KREG) kb = __builtin_bit_cast(v8, kr[kt][n]);
            else kb = *(const v8*)(lds_kb + (kr0[kt] * KP + lg * DL + 8 * n) * Geo::EL);
            s[kt][u] = Mfma16<T>::run(qa, kb, s[kt][u]);
            dp[kt][u] = Mfma16<T>::run(oa, __builtin_bit_cast(v8, vr[kt][n]), dp[kt][u]);
          }
        }
      }
    }

    // ---- P = exp(S scale - lse) on visible pairs, dS / scale = P (dP - D)
    float p[KW][2][4], ds[KW][2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const f32x4 l4 = *(const f32x4*)(lds_lse + 16 * u + 4 * lg);
      const f32x4 d4 = *(const f32x4*)(lds_dr + 16 * u + 4 * lg);
#pragma unroll
      for (int kt = 0; kt < KW; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = r0 + 16 * u + 4 * lg + r;
          const bool vis = row < w.Lq && kc[kt] < w.Lk && (!CAUSAL || kc[kt] <= row + shift);
          const float pr = vis ? fast_exp2(__builtin_fmaf(s[kt][u][r], a.scale_log2, -l4[r])) : 0.f;
          p[kt][u][r] = pr;
          ds[kt][u][r] = pr * (dp[kt][u][r] - d4[r]);
        }
    }

    // ---- dV += P^T dO, dK += dS^T Q; dS to LDS
    if constexpr (F32) {
      const float* qt = (const float*)lds_qb;
      const float* dot = (const float*)lds_dob;
      float* dst = (float*)lds_dsb;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * u + 4 * lg + r;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            dv[0][dt] = mfma4(p[0][u][r], dot[row * QP + 16 * dt + li], dv[0][dt]);
            dk[0][dt] = mfma4(ds[0][u][r], qt[row * QP + 16 * dt + li], dk[0][dt]);
          }
          dst[row * SP + kr0[0]] = ds[0][u][r];
        }
    } else {
      typedef typename Elem16<T>::v8 v8;
      typedef typename Elem16<T>::v4 v4;
      const uint16_t* qt = (const uint16_t*)lds_qb;
      const uint16_t* dot = (const uint16_t*)lds_dob;
      uint16_t* dst = (uint16_t*)lds_dsb;
      v8 pa[KW], da[KW];
#pragma unroll
      for (int kt = 0; kt < KW; ++kt) {
        v4 p0, p1, d0, d1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p0[r] = (T)p[kt][0][r];
          p1[r] = (T)p[kt][1][r];
          d0[r] = (T)ds[kt][0][r];
          d1[r] = (T)ds[kt][1][r];
        }
        pa[kt] = __builtin_shufflevector(p0, p1, 0, 1, 2, 3, 4, 5, 6, 7);
        da[kt] = __builtin_shufflevector(d0, d1, 0, 1, 2, 3, 4, 5, 6, 7);
        // dS^T row kr0[kt] (this lane's key): rows 4lg .. 4lg+3 and 16+4lg .. 16+4lg+3
        // (whole-vector stores: scalar 16-bit LDS stores of these values were
        // miscompiled into stores of one element)
        *(v4*)(dst + kr0[kt] * SP + 4 * lg) = d0;
        *(v4*)(dst + kr0[kt] * SP + 16 + 4 * lg) = d1;
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const v8 bo = gen_tr8<v8, QP>(dot, 4 * lg, 16 + 4 * lg, 16 * dt, li);
        const v8 bq = gen_tr8<v8, QP>(qt, 4 * lg, 16 + 4 * lg, 16 * dt, li);
#pragma unroll
        for (int kt = 0; kt < KW; ++kt) {
          dv[kt][dt] = Mfma16<T>::run(pa[kt], bo, dv[kt][dt]);
          dk[kt][dt] = Mfma16<T>::run(da[kt], bq, dk[kt][dt]);
        }
      }
    }
    __syncthreads();

    // ---- dQ = scale * dS K: tile t = wave + 4n takes row tile t % 2, column tile t / 2
    const __amdgpu_buffer_rsrc_t racc =
        buffer_rsrc(a.dq_acc + (int64_t)(w.q_start + r0) * rs + (int64_t)h * D,
                    tiling::head_rows_bytes(min(BM, w.Lq - r0), rs, D, 4));
#pragma unroll
    for (int n = 0; n < DQT; ++n) {
      const int t = wave + 4 * n, ru = t & 1, ct = t >> 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (F32) {
        const float* dst = (const float*)lds_dsb;
        const float* ktile = (const float*)lds_kb;
#pragma unroll
        for (int s4 = 0; s4 < BN / 4; ++s4)
          acc = mfma4(dst[(16 * ru + li) * SP + 4 * s4 + lg], ktile[(4 * s4 + lg) * KP + 16 * ct + li], acc);
      } else {
        typedef typename Elem16<T>::v8 v8;
        const uint16_t* dst = (const uint16_t*)lds_dsb;
        const uint16_t* ktile = (const uint16_t*)lds_kb;
#pragma unroll
        for (int s32 = 0; s32 < BN / 32; ++s32) {
          // A: dS row 16ru + li, keys 32 s32 + 8lg .. +7 (transposing reads of dS^T)
          const v8 av = gen_tr8<v8, SP>(dst, 32 * s32 + 8 * lg, 32 * s32 + 8 * lg + 4, 16 * ru, li);
          acc = Mfma16<T>::run(av, gen_tr8<v8, KP>(ktile, 32 * s32 + 8 * lg, 32 * s32 + 8 * lg + 4, 16 * ct, li),
                               acc);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * ru + 4 * lg + r;
        if (r0 + row < w.Lq) {
          const uint32_t off = ((uint32_t)row * (uint32_t)rs + 16 * ct + li) * 4u;
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r] * a.scale, racc, (int)off, 0, 0);
        }
      }
    }
  }

  // ---- epilogue: dK (times the softmax scale) and dV of keys key0 + 16 (KW wave + kt) + 4 lg + r
#pragma unroll
  for (int kt = 0; kt < KW; ++kt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int kk = key0 + 16 * (KW * wave + kt) + 4 * lg + r;
      if (kk < w.Lk) {
        T* dkp = (T*)a.dk + (int64_t)(w.k_start + kk) * rsk + (int64_t)w.hk * D;
        T* dvp = (T*)a.dv + (int64_t)(w.k_start + kk) * rsk + (int64_t)w.hk * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dkp[16 * dt + li] = (T)(dk[kt][dt][r] * a.scale);
          dvp[16 * dt + li] = (T)dv[kt][dt][r];
        }
      }
    }
}

template <typename F>
hipError_t launch(F kernel, int grid, int threads, hipStream_t stream, const BwdArgs& a) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_wide(bool causal, int grid, const BwdArgs& a, hipStream_t stream) {
  return causal ? launch(bwd16w_kernel<T, D, true>, grid, 512, stream, a)
                : launch(bwd16w_kernel<T, D, false>, grid, 512, stream, a);
}
template <typename T, int D>
hipError_t launch_gen(bool causal, int grid, const BwdArgs& a, hipStream_t stream) {
  return causal ? launch(bwd_gen_kernel<T, D, true>, grid, 256, stream, a)
                : launch(bwd_gen_kernel<T, D, false>, grid, 256, stream, a);
}

template <typename T>
hipError_t launch_bwd16(int head_dim, bool causal, int grid, const BwdArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_wide<T, 64>(causal, grid, a, stream);
    case 96: return launch_wide<T, 96>(causal, grid, a, stream);
    case 128: return launch_wide<T, 128>(causal, grid, a, stream);
    case 256: return launch_gen<T, 256>(causal, grid, a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bwd32(int head_dim, bool causal, int grid, const BwdArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return launch_gen<float, 64>(causal, grid, a, stream);
    case 96: return launch_gen<float, 96>(causal, grid, a, stream);
    case 128: return launch_gen<float, 128>(causal, grid, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// (row, head) pairs per workgroup of the prep and dq kernels: 256 / pair_lanes
int64_t row_pairs_grid(const BwdArgs& a, int dtype, int head_dim) {
  const int64_t pairs = (int64_t)a.total_q * a.heads;
  const int chunks = head_dim / (dtype == 0 ? 4 : 8);
  const int lanes = chunks <= 8 ? 8 : (chunks <= 16 ? 16 : (chunks <= 32 ? 32 : 64));
  const int64_t per = 256 / lanes;
  return (pairs + per - 1) / per;
}

template <template <typename, int> class K, typename T>
hipError_t launch_rows(int head_dim, int grid, hipStream_t stream, const BwdArgs& a) {
  switch (head_dim) {
    case 64: return launch(K<T, 64>::fn, grid, 256, stream, a);
    case 96: return launch(K<T, 96>::fn, grid, 256, stream, a);
    case 128: return launch(K<T, 128>::fn, grid, 256, stream, a);
    case 256: return launch(K<T, 256>::fn, grid, 256, stream, a);
    default: return hipErrorInvalidValue;
  }
}
template <typename T, int D>
struct PrepK { static constexpr auto fn = bwd_prep_kernel<T, D>; };
template <typename T, int D>
struct DqK { static constexpr auto fn = bwd_dq_kernel<T, D>; };

template <template <typename, int> class K>
hipError_t launch_rows_dtype(int dtype, int head_dim, const BwdArgs& a, hipStream_t stream) {
  const int64_t grid = row_pairs_grid(a, dtype, head_dim);
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (dtype == 0) return launch_rows<K, float>(head_dim, (int)grid, stream, a);
  if (dtype == 1) return launch_rows<K, __bf16>(head_dim, (int)grid, stream, a);
  if (dtype == 2) return launch_rows<K, _Float16>(head_dim, (int)grid, stream, a);
  return hipErrorInvalidValue;
}

}  // namespace

int bwd_block_n(int dtype, int head_dim) {
  const bool half = dtype == 1 || dtype == 2;
  if (half && (head_dim == 64 || head_dim == 96 || head_dim == 128)) return kBwdBNWide;
  if (half && head_dim == 256) return gen_block_n<__bf16, 256>();
  if (dtype == 0 && (head_dim == 64 || head_dim == 96 || head_dim == 128)) return gen_block_n<float, 64>();
  return 0;
}

hipError_t launch_bwd_prep(int dtype, int head_dim, const BwdArgs& a, hipStream_t stream) {
  return launch_rows_dtype<PrepK>(dtype, head_dim, a, stream);
}

hipError_t launch_bwd(int dtype, int head_dim, bool causal, int grid, const BwdArgs& a, hipStream_t stream) {
  if (dtype == 0) return launch_bwd32(head_dim, causal, grid, a, stream);
  if (dtype == 1) return launch_bwd16<__bf16>(head_dim, causal, grid, a, stream);
  if (dtype == 2) return launch_bwd16<_Float16>(head_dim, causal, grid, a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(int dtype, int head_dim, const BwdArgs& a, hipStream_t stream) {
  return launch_rows_dtype<DqK>(dtype, head_dim, a, stream);
}

}  // namespace fa
