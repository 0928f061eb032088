// fa_varlen_kernels.hip -- gfx950 kernels for exact attention forward over
// packed variable-length sequences.
//
// Kernels:
//   * tile_map_kernel       -- the work-item map: exclusive scan of per-sequence
//                              query-block counts (the sequence-dimension split,
//                              iplexlaw.co.kr "FlashAttention-2 GPU work
//                              partitioning", section "Tres mejoras en la
//                              utilización de la GPU").
//   * fwd16_pipe_kernel     -- 16-bit (bf16 or fp16) in/out, head_dim 64, 96,
//                              128 and 256: software-pipelined wavefronts
//                              (each stage: the first product of the next
//                              slab, the softmax of this one, the second
//                              product of the previous one); 16-bit MFMA for
//                              the two contractions, fp32 online softmax.
//   * fwd_f32_kernel        -- fp32 in/out, fp32 MFMA, same online softmax.
//   * check_cu_kernel       -- optional device validation of the offsets.
//
// Several query heads may share one key/value head (multi-query and
// grouped-query attention, zepes.com "Comprendiendo Flash-Atención y
// Flash-Atención-2", section "FlashAttention-2"): query head h reads the K/V
// slices of head h / head_group, in tensors of kv_heads = heads / head_group
// heads per token row.
//
// Forward-kernel organisation (all dtypes)
// -----------------------------------------
// One workgroup owns one (sequence b, query block m, head h) work item: BM
// query rows split across NW wavefronts, 32 rows per wavefront (split-Q:
// the waves share the K/V tiles and never exchange partial results, as the
// pages describe for FlashAttention-2's forward pass, zepes.com "Comprendiendo
// Flash-Atención y Flash-Atención-2", section "FlashAttention-2").  K/V tiles
// of BN keys stream through LDS; the score tile never leaves
// registers (slavadubrov.com "O que FlashAttention muda na inferência",
// section "Separar o armazenamento do cálculo").
//
// Scores are computed transposed, S^T = K Q^T, with the 32x32 MFMA: in the
// 32x32 accumulator layout a lane owns one column, so every lane owns one query
// row and holds 16 of the 32 keys of a key block (the other 16 sit in lane
// l^32).  Consequences:
//   * row max / row sum need one cross-lane exchange (lane l <-> l^32);
//   * rescaling the output by the online-softmax factor is a per-lane scalar
//     multiply, because O is also accumulated transposed (O^T = V^T P^T) and
//     each lane again owns one query row;
//   * the probabilities P^T are already in the B-operand layout of the second
//     MFMA: no shuffle or LDS round trip between the two contractions.
// The second contraction needs V^T as its A operand (8 consecutive keys per
// lane): the 16-bit kernels keep V row-major in LDS and read it with the
// transposing LDS read; the fp32 kernel's operands are single elements.
//
// Online softmax per query row (iplexlaw.co.kr, section "Bloques pequeños,
// normalización global"): with t = scale*log2(e)*s,
//   m' = max(m, max_j t_j), alpha = 2^(m - m'), l' = alpha l + sum_j 2^(t_j - m'),
//   O' = alpha O + sum_j 2^(t_j - m') v_j;  out = O / l,  lse = (m + log2 l) ln 2.
// The reference m need not be the exact running max: any finite m close
// enough to it that 2^(t - m) neither overflows nor loses all precision gives
// the same out and lse, because l and O are accumulated against the same m.  The kernel therefore raises m (and pays
// the rescale of O) only when some row of the wavefront outgrows it by more
// than 2^8, which after the first tiles is rare.
// A row that has seen no visible key keeps m = -inf and is guarded so that no
// -inf - -inf appears; such rows end with out = 0, lse = -inf.
//
// Masks (reading: bottom-right causal alignment, key j visible to query i iff
// j <= i + Lk - Lq; ragged tails from the offsets, friki.work "Mecanismo
// cu_seqlens en FlashAttention", section "Lógica de cálculo de longitud") are
// applied only to key tiles that cross the diagonal or the end of the
// sequence; tiles entirely above the diagonal are never visited.
//
// Scheduling: workgroup ids are remapped so that each of the 8 XCDs receives
// a contiguous range of work (all query blocks of a head land on one XCD and
// share its L2 for K/V), and inside a head the items run last-first so that
// the longest causal rows start early.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "fa_varlen_device.h"
#include "fa_varlen_launch.h"
#include "fa_varlen_tiling.h"

namespace fa {
namespace {

// The running max used as the softmax reference is only raised when a row's
// new maximum exceeds it by more than this many log2 units (wave-uniform
// decision).  Probabilities are then at most 2^kRescaleSlack; l and O share
// the same stale reference, so the result is unchanged.
constexpr float kRescaleSlack = 8.0f;

// ---------------------------------------------------------------------------
// work decoding shared by both forward kernels
// ---------------------------------------------------------------------------
struct WorkItem {
  int b, m, h;
  int q_start, Lq, k_start, Lk;
};

// Without a map (a.blk_start null: at most kMaplessBatch sequences) every
// wavefront rebuilds the scan itself: lane b holds sequence b's block count
// ceil(Lq_b / BM), a wave-wide inclusive scan gives the map, and block t
// belongs to the first sequence whose inclusive count exceeds t.  The same
// (b, m) as the map path, without the map's allocation and launch.
template <int BM>
__device__ __forceinline__ void locate_block_mapless(const FwdArgs& a, int tr, int& T, int& b, int& m) {
  const int lane = threadIdx.x & 63;
  int cnt = 0;
  if (lane < a.batch) cnt = (a.cu_q[lane + 1] - a.cu_q[lane] + BM - 1) / BM;
  int inc = cnt;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(inc, d, 64);
    if (lane >= d) inc += y;
  }
  T = __shfl(inc, 63, 64);
  const int t = T - 1 - tr;
  const uint64_t past = __builtin_amdgcn_ballot_w64(inc > t);  // sequences ending after block t
  b = past ? __builtin_ctzll(past) : 0;
  m = t - __shfl(inc - cnt, b, 64);
}

template <int BM>
__device__ __forceinline__ bool decode_work(const FwdArgs& a, WorkItem& w) {
  // hardware dispatch sends workgroup i to XCD i % 8; give each XCD a
  // contiguous slice of work ids (gridDim.x is a multiple of 8).
  const uint32_t per_xcd = gridDim.x >> 3;
  const uint32_t work = (blockIdx.x & 7u) * per_xcd + (blockIdx.x >> 3);
  if (work >= (uint32_t)a.n_work) return false;
  w.h = (int)(work / (uint32_t)a.tmax);
  const int tr = (int)(work % (uint32_t)a.tmax);
  int lo = 0;
  if (a.blk_start == nullptr) {
    int T, m;
    locate_block_mapless<BM>(a, tr, T, lo, m);
    if (tr >= T) return false;
    w.m = m;
  } else {
    const int T = a.blk_start[a.batch];
    if (tr >= T) return false;
    const int t = T - 1 - tr;
    int hi = a.batch;  // invariant: blk_start[lo] <= t < blk_start[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.blk_start[mid] <= t) lo = mid; else hi = mid;
    }
    w.m = t - a.blk_start[lo];
  }
  w.b = lo;
  w.q_start = a.cu_q[lo];
  w.Lq = a.cu_q[lo + 1] - w.q_start;
  w.k_start = a.cu_k[lo];
  w.Lk = a.cu_k[lo + 1] - w.k_start;
  return true;
}

// Key-tile range of a work item.  Tiles [0, n_full) need no mask, tiles
// [n_full, n_end) need the causal and/or tail mask, tiles >= n_end are
// invisible to every row of the item.
template <int BM, int BN, bool CAUSAL>
__device__ __forceinline__ void key_tiles(const WorkItem& w, int& n_full, int& n_end) {
  const int q0 = w.m * BM;
  const int rows = min(BM, w.Lq - q0);
  int j_hi = w.Lk, j_full = w.Lk;
  if (CAUSAL) {
    const int shift = w.Lk - w.Lq;
    j_hi = min(w.Lk, q0 + rows + shift);   // keys < j_hi seen by the last row
    j_full = min(w.Lk, q0 + shift + 1);    // keys < j_full seen by every row
  }
  n_end = j_hi > 0 ? (j_hi + BN - 1) / BN : 0;
  n_full = j_full > 0 ? j_full / BN : 0;
}

// ---------------------------------------------------------------------------
// tile map
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void tile_map_kernel(const int32_t* __restrict__ cu_q, int batch,
                                                       int block_m, int32_t* __restrict__ blk_start) {
  __shared__ int wave_tot[4];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (tid == 0) { blk_start[0] = 0; carry_s = 0; }
  __syncthreads();
  for (int base = 0; base < batch; base += 256) {
    const int b = base + tid;
    int n = 0;
    if (b < batch) {
      const int L = cu_q[b + 1] - cu_q[b];
      n = L > 0 ? (L - 1) / block_m + 1 : 0;
    }
    int x = n;  // inclusive scan inside the wavefront
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) wave_tot[wid] = x;
    __syncthreads();
    int before = carry_s;
    for (int i = 0; i < wid; ++i) before += wave_tot[i];
    const int incl = before + x;
    if (b < batch) blk_start[b + 1] = incl;
    __syncthreads();
    if (tid == 255) carry_s = incl;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// cu_seqlens validation (optional, debugging aid)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void check_cu_kernel(const int32_t* __restrict__ cu_q,
                                                       const int32_t* __restrict__ cu_k, int batch,
                                                       int total_q, int total_k, int max_q, int max_k,
                                                       int32_t* __restrict__ flags) {
  __shared__ int acc;
  if (threadIdx.x == 0) acc = 0;
  __syncthreads();
  int f = 0;
  if (threadIdx.x == 0) {
    if (cu_q[0] != 0) f |= 1;
    if (cu_k[0] != 0) f |= 16;
    if (cu_q[batch] > total_q) f |= 4;
    if (cu_k[batch] > total_k) f |= 64;
  }
  for (int b = threadIdx.x; b < batch; b += 256) {
    const int lq = cu_q[b + 1] - cu_q[b], lk = cu_k[b + 1] - cu_k[b];
    if (lq < 0) f |= 2;
    if (lk < 0) f |= 32;
    if (lq > max_q) f |= 8;
    if (lk > max_k) f |= 128;
  }
  if (f) atomicOr(&acc, f);
  __syncthreads();
  if (threadIdx.x == 0) flags[0] = acc;
}

// ---------------------------------------------------------------------------
// 16-bit LDS layouts
// ---------------------------------------------------------------------------
// 16-byte chunks are XOR-swizzled so that the MFMA operand reads hit distinct
// banks within each group of 8 and of 16 lanes:
//   Ks[key][d]   key-major, one row of k_stride<D>() elements per key
//   Vr[key][d]   key-major like Ks (its own swizzle), read with transposing
//                LDS reads as the A operand of O^T = V^T P^T
// Both are loaded straight from global memory (direct loads).  Index
// arithmetic (swizzles, chunk mappings, LDS indices, byte extents) lives in
// fa_varlen_tiling.h, shared with the host-side bounds checker.

// Work items of one workgroup.  Under a causal mask, query block m of a
// sequence with M blocks reads about (m+1)/M of its keys, so blocks m and
// M-1-m together always carry one full pass.  When the host asks for it
// (a.pair_blocks: causal, and only a few workgroups per CU, where the last
// few long workgroups would otherwise decide the run time), the workgroup of
// block m < M/2 of a sequence with at least kPairMinBlocks blocks processes
// both and the workgroups of the upper half exit.  Shorter sequences keep one
// block per workgroup: their blocks are short and pairing would only halve
// the parallelism.
constexpr int kPairMinBlocks = 6;

template <int BM, bool CAUSAL, typename Item>
__device__ __forceinline__ void run_work(const FwdArgs& a, WorkItem& w, Item&& item) {
  const int M = (w.Lq + BM - 1) / BM;
  if (CAUSAL && a.pair_blocks && M >= kPairMinBlocks) {
    if (2 * w.m >= M) return;
    item(w);
    if (M - 1 - w.m != w.m) {
      __syncthreads();  // the second item reuses the LDS buffers
      w.m = M - 1 - w.m;
      item(w);
    }
  } else {
    item(w);
  }
}

// ---------------------------------------------------------------------------
// 16-bit forward, software-pipelined wavefronts
// ---------------------------------------------------------------------------
// The workgroup's 8 wavefronts (two per SIMD) each own 32 query rows and walk
// the key range in 32-key slabs.  Stage j of a wavefront issues three pieces
// of work that do not depend on each other:
//   QK(j+1)    S^T of slab j+1 = K Q^T       8 MFMAs (head_dim 128), K from LDS
//   softmax(j) the online softmax of slab j  vector ALU and exponentials
//   PV(j-1)    O^T += V^T P^T of slab j-1    8 MFMAs, V^T by transposing LDS reads
// so the matrix instructions of one wavefront run while its own vector
// instructions issue, and both wavefronts of a SIMD always have both kinds of
// work.  (A wavefront on its own issues vector instructions at about half the
// rate two wavefronts reach together, and one MFMA of 32 cycles leaves room for
// several vector instructions of the same wavefront.)  The softmax of slab j
// needs S(j), computed in stage j-1; PV(j-1) needs P(j-1), produced in stage
// j-1: each stage reads only results of the previous one.
//
// K and V tiles of BN keys go from global memory straight into LDS (direct
// loads), four buffers each, tile m in buffer m % 4.  Iteration n of the
// workgroup loop runs the stages of slabs of tile n; it reads K tiles n and
// n+1 and V tiles n-1 and n, and issues the loads of K(n+3) and V(n+2), whose
// buffers were last read in iteration n-1.  A load has two iterations to land;
// each wavefront waits for its own loads before the barrier that ends the
// iteration.
constexpr int kPipeBuffers = 4;
// K fragments of the next slab that each steady stage reads ahead (half of
// the slab's eight): their LDS latency then overlaps the end of the stage
// instead of stalling the first products of the next one.
constexpr int kPipeKPre = 4;
// At head_dim 256 a SIMD runs one wavefront, which has no partner to cover
// LDS latency: there the whole K slab (16 fragments) is read ahead, right
// after the barrier that makes it visible, and so are the V fragments of the
// first k-step of the next stage's second product (8), read at the end of the
// previous stage (the V tile of stage j+1 is resident during stage j).  12 or
// 16 V fragments were slower, as were 4.
template <int D>
constexpr int pipe_kpre() { return D == 256 ? 16 : kPipeKPre; }
template <int D>
constexpr int pipe_vpre() { return D == 256 ? D / 32 : 0; }

template <int D, int BN, int NW>
struct PipeGeom {
  static constexpr int KS = tiling::k_stride<D>();  // elements per LDS row
  static constexpr int CPR = KS / 8;                 // 16-byte slots per LDS row
  static constexpr int LOADS = BN * CPR / 64;        // wave-wide direct loads per tile
  static constexpr int PER_WAVE = LOADS / NW;        // per wavefront (NW share a tile)
  static constexpr int SPT = BN / 32;                // 32-key slabs per tile
  static constexpr int TILE = BN * KS;               // elements per tile buffer
  static_assert(LOADS % NW == 0 && PER_WAVE >= 1 && PER_WAVE <= 4, "tile must split into whole wave loads");
};

// Direct loads of keys key0 .. key0+BN-1 of the head slice at `base` into the
// LDS tile at dst, in the K-style (V_LAYOUT false) or row-major V layout; this
// wavefront's share: slots 64 * (wave * PER_WAVE + i) + lane.  Keys at or past
// Lk read as zeros (buffer range check).
template <int D, int BN, int NW, bool V_LAYOUT>
__device__ __forceinline__ void pipe_issue(uint16_t* dst, const uint16_t* __restrict__ base, int64_t row_stride,
                                           int key0, int Lk, int wave, int lane) {
  using G = PipeGeom<D, BN, NW>;
  // no clamp at zero: head_rows_bytes gives 0 bytes for rows <= 0 (and a
  // min/max pair would be fused into a vector-only med3)
  const int rows = min(BN, Lk - key0);
  const u32x4 r = buffer_rsrc_words(base + (int64_t)key0 * row_stride, head_rows_bytes(rows, row_stride, D, 2));
  const uint32_t lds = lds_address(dst);
#pragma unroll
  for (int i = 0; i < G::PER_WAVE; ++i) {
    const int seg = wave * G::PER_WAVE + i;
    int row, ch;
    tiling::direct_slot_chunk<D, V_LAYOUT>(seg * 64 + lane, row, ch);
    const uint32_t off = ((uint32_t)row * (uint32_t)row_stride + (uint32_t)ch * 8u) * 2u;
    lds_dma16(r, off, lds + (uint32_t)seg * 1024u);
  }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
  // s_waitcnt needs an immediate: the loads a wavefront may leave in flight
  // are 0, PER_WAVE (V only) or 2 * PER_WAVE (K and V) per iteration
  if (n >= 2 * N) wait_vmcnt<2 * N>();
  else if (n >= N) wait_vmcnt<N>();
  else wait_vmcnt<0>();
}

// Per-wavefront state and the three pieces of a stage.
template <typename T, int D>
struct PipeWave {
  typedef typename Elem16<T>::v8 v8;
  static constexpr int KSTEPS = D / 16;  // MFMA k-steps of Q K^T
  static constexpr int DB = D / 32;      // 32-dimension blocks of the output
  static constexpr int KS = tiling::k_stride<D>();

  v8 q[KSTEPS];  // Q^T as the B operand
  f32x16 o[DB];  // O^T accumulators (lane: query row, registers: dimensions)
  float m_run, l_run;

  // S^T of the slab whose first key row in the tile at Ks is `row0`.  A-row R
  // reads key row key_of_arow(R), so register r of lane half g holds key
  // 16 g + r of the slab.
  __device__ __forceinline__ f32x16 qk(const uint16_t* Ks, int row0, int arow, int g) const {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const v8 av = *(const v8*)(Ks + tiling::ks_index<D>(row0 + arow, 2 * ks + g));
      s = Elem16<T>::mfma(av, q[ks], s);
    }
    return s;
  }

  // The same product with its first NPRE K fragments already in registers
  // (read by k_pre a stage earlier, so that their LDS latency is hidden).
  template <int NPRE>
  __device__ __forceinline__ f32x16 qk_pre(const uint16_t* Ks, const v8 (&pre)[NPRE], int arow, int g) const {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const v8 av = ks < NPRE ? pre[ks < NPRE ? ks : 0]
                              : *(const v8*)(Ks + tiling::ks_index<D>(arow, 2 * ks + g));
      s = Elem16<T>::mfma(av, q[ks], s);
    }
    return s;
  }
  template <int NPRE>
  __device__ __forceinline__ static void k_pre(const uint16_t* Ks, v8 (&pre)[NPRE], int arow, int g) {
#pragma unroll
    for (int ks = 0; ks < NPRE; ++ks) pre[ks] = *(const v8*)(Ks + tiling::ks_index<D>(arow, 2 * ks + g));
  }

  // O^T += V^T P^T for the slab whose first key row in the tile at Vr is
  // `row0`.  The A operand of k-step t (keys 16 g + 8 t .. +7 of the slab for
  // lane half g, the keys of the probabilities in p[t]) comes from two
  // transposing reads of 4 rows each.
  __device__ __forceinline__ void pv(const uint16_t* Vr, int row0, const v8 (&p)[2], int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const int g = lane >> 5;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int r0 = row0 + 16 * g + 8 * t;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(Vr + tiling::vr_tr_index<D>(lane, r0, db)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(Vr + tiling::vr_tr_index<D>(lane, r0 + 4, db)));
        const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db] = Elem16<T>::mfma(__builtin_bit_cast(v8, v), p[t], o[db]);
      }
  }

  // V^T operand fragments of the product above, in its order (k-step t, then
  // dimension block db: fragment t * DB + db); pv_pre takes the first NV of
  // them already read by v_pre.
  __device__ __forceinline__ static v8 v_frag(const uint16_t* Vr, int row0, int f, int lane) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const int g = lane >> 5, t = f / DB, db = f % DB;
    const int r0 = row0 + 16 * g + 8 * t;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(Vr + tiling::vr_tr_index<D>(lane, r0, db)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(Vr + tiling::vr_tr_index<D>(lane, r0 + 4, db)));
    return __builtin_bit_cast(v8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  template <int NV>
  __device__ __forceinline__ static void v_pre(const uint16_t* Vr, v8 (&pre)[NV], int lane) {
#pragma unroll
    for (int f = 0; f < NV; ++f) pre[f] = v_frag(Vr, 0, f, lane);
  }
  template <int NV>
  __device__ __forceinline__ void pv_pre(const uint16_t* Vr, const v8 (&p)[2], const v8 (&pre)[NV], int lane) {
#pragma unroll
    for (int f = 0; f < 2 * DB; ++f) {
      const v8 av = f < NV ? pre[f < NV ? f : 0] : v_frag(Vr, 0, f, lane);
      o[f % DB] = Elem16<T>::mfma(av, p[f / DB], o[f % DB]);
    }
  }

  // -inf for keys past the end of the sequence or (causal) above the diagonal;
  // `key0` is the slab's first key, `row` this lane's query row.
  template <bool CAUSAL>
  __device__ __forceinline__ static void mask(f32x16& s, int key0, int row, int g, int Lk, int shift) {
    const int lim = CAUSAL ? min(Lk - 1, row + shift) : (Lk - 1);  // last visible key
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + 16 * g + r > lim) s[r] = kNegInf;
  }

  // Online softmax of one slab: probabilities in the PV B-operand layout and
  // the running statistics; returns whether some row of the wavefront raised
  // its reference (then O must be scaled by alpha after the PV of the
  // previous slab).  The reference is raised only when a row's maximum passes
  // it by more than kRescaleSlack, which after the first slabs is rare.
  __device__ __forceinline__ bool softmax(const f32x16& s, v8 (&p)[2], float& alpha, float scale_log2) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    const float m_tile = pair_max(mx) * scale_log2;
    const bool need = wave_any(m_tile > m_run + kRescaleSlack);
    const float m_new = need ? fmaxf(m_run, m_tile) : m_run;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    alpha = fast_exp2(m_run - m_use);  // 1 when the reference is kept
    m_run = m_new;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(s[8 * t + e], scale_log2, -m_use));
        part[e & 3] += pe;
        p[t][e] = (T)pe;
      }
    const float lsum = (part[0] + part[1]) + (part[2] + part[3]);
    l_run = l_run * alpha + lsum;
    // The flag is formed from the row sums (never negative), so the rarely
    // taken rescale branch cannot be placed ahead of the exponentials: they
    // stay in one basic block with the MFMAs of the stage.
    return wave_any(need && !(lsum < 0.f));
  }

  // Softmax of an unmasked slab against the current references, without the
  // row maxima.  Used once every row of the wavefront has seen visible keys:
  // each row's reference m_run is then an earlier maximum of its own scores.
  // Any finite reference gives the same out = O / l and lse = m + log2(l):
  // float32 and the 16-bit types keep their relative precision at any
  // magnitude, and l and O share the reference.  The hazard is overflow when
  // scores outgrow the reference: the probabilities are rounded to T before
  // the second product, and fp16 ends at 65504.  The slab is accepted when
  // every row's sum over it -- a bound on each of its probabilities -- stays
  // at or below 2^15 (a NaN fails the test too); otherwise the caller redoes
  // it with softmax() above, which raises the reference.  On acceptance l_run
  // is updated and the probabilities are in p.
  static constexpr float kFastSlabLimit = 32768.f;  // 2^15
  __device__ __forceinline__ bool softmax_fast(const f32x16& s, v8 (&p)[2], float scale_log2) {
    float part[4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = fast_exp2(__builtin_fmaf(s[8 * t + e], scale_log2, -m_run));
        part[e & 3] = (t == 0 && e < 4) ? pe : part[e & 3] + pe;
        p[t][e] = (T)pe;
      }
    const float lsum = (part[0] + part[1]) + (part[2] + part[3]);
    const bool ok = !wave_any(!(lsum <= kFastSlabLimit));
    if (ok) l_run += lsum;
    return ok;
  }

  __device__ __forceinline__ void rescale(float alpha) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
  }
};

template <typename T, int D, int BN, int NW, bool CAUSAL>
__device__ __forceinline__ void fwd16_pipe_item(const FwdArgs& a, const WorkItem& wi,
                                                uint16_t (&lds_k)[kPipeBuffers][BN * tiling::k_stride<D>()],
                                                uint16_t (&lds_v)[kPipeBuffers][BN * tiling::k_stride<D>()]) {
  // the item's fields are workgroup-uniform: keep them in scalar registers so
  // that the per-iteration load set-up runs on the scalar unit
  WorkItem w;
  w.b = __builtin_amdgcn_readfirstlane(wi.b);
  w.m = __builtin_amdgcn_readfirstlane(wi.m);
  w.h = __builtin_amdgcn_readfirstlane(wi.h);
  w.q_start = __builtin_amdgcn_readfirstlane(wi.q_start);
  w.Lq = __builtin_amdgcn_readfirstlane(wi.Lq);
  w.k_start = __builtin_amdgcn_readfirstlane(wi.k_start);
  w.Lk = __builtin_amdgcn_readfirstlane(wi.Lk);
  using G = PipeGeom<D, BN, NW>;
  using Wave = PipeWave<T, D>;
  constexpr int BM = 32 * NW;
  typedef typename Wave::v8 v8;
  constexpr int SPT = G::SPT;
  constexpr int NB = kPipeBuffers;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int q0 = w.m * BM;                // first query row of the item (in its sequence)
  const int wrow0 = q0 + wave * 32;       // first query row of this wavefront
  const int shift = w.Lk - w.Lq;
  const int64_t rs = a.row_stride, rsk = a.kv_row_stride;
  const int hk = w.h / a.head_group;
  const uint16_t* __restrict__ kbase = (const uint16_t*)a.k + (int64_t)w.k_start * rsk + (int64_t)hk * D;
  const uint16_t* __restrict__ vbase = (const uint16_t*)a.v + (int64_t)w.k_start * rsk + (int64_t)hk * D;

  // Slabs of this wavefront: j_end slabs hold a key some row sees, the first
  // j_full slabs need no mask.  The workgroup walks the slabs of its last
  // wavefront with rows (the most, under a causal mask).
  int j_end = 0, j_full = 0;
  if (wrow0 < w.Lq) {
    const int hi = CAUSAL ? min(w.Lk, wrow0 + 32 + shift) : w.Lk;
    const int full = CAUSAL ? min(w.Lk, wrow0 + 1 + shift) : w.Lk;
    j_end = hi > 0 ? (hi + 31) / 32 : 0;
    j_full = full > 0 ? full / 32 : 0;
  }
  int J = 0;
  {
    const int last_row = min(w.Lq, q0 + BM) - 1;
    const int wlast = q0 + ((last_row - q0) & ~31);
    const int hi = CAUSAL ? min(w.Lk, wlast + 32 + shift) : w.Lk;
    J = hi > 0 ? (hi + 31) / 32 : 0;
  }
  const int NT = (J + SPT - 1) / SPT;  // K/V tiles the workgroup loads
  const int NIT = J > 0 ? J / SPT + 1 : 0;  // iterations: stage J is in iteration J / SPT

  // first tiles, then Q; one wait covers them all
  if (NT > 0) {
    pipe_issue<D, BN, NW, false>(lds_k[0], kbase, rsk, 0, w.Lk, wave, lane);
    pipe_issue<D, BN, NW, true>(lds_v[0], vbase, rsk, 0, w.Lk, wave, lane);
    if (NT > 1) pipe_issue<D, BN, NW, false>(lds_k[1], kbase, rsk, BN, w.Lk, wave, lane);
  }
  Wave wv;
  {  // Q rows past the end of the sequence load as zeros
    const int qrows = max(0, min(32, w.Lq - wrow0));
    const __amdgpu_buffer_rsrc_t rq =
        buffer_rsrc((const uint16_t*)a.q + (int64_t)(w.q_start + wrow0) * rs + (int64_t)w.h * D,
                    head_rows_bytes(qrows, rs, D, 2));
#pragma unroll
    for (int ks = 0; ks < Wave::KSTEPS; ++ks) {
      const uint32_t off = ((uint32_t)l32 * (uint32_t)rs + 16 * ks + 8 * g) * 2u;
      wv.q[ks] = __builtin_bit_cast(v8, buffer_load16(rq, off));
    }
  }
  wv.m_run = kNegInf;
  wv.l_run = 0.f;
#pragma unroll
  for (int db = 0; db < Wave::DB; ++db) wv.o[db] = f32x16{};
  wait_vmcnt<0>();
  __syncthreads();

  const int arow = key_of_arow(l32);
  const int row = wrow0 + l32;  // this lane's query row (in sequence)
  f32x16 s_cur = {};
  v8 p_prev[2] = {};
  if (j_end > 0) s_cur = wv.qk(lds_k[0], 0, arow, g);  // S(0)

  // K slab j+1 is in tile (j+1)/SPT, V slab j-1 in tile (j-1)/SPT
  auto kslab = [&](int j) { return (const uint16_t*)lds_k[((j + 1) / SPT) % NB] + ((j + 1) % SPT) * 32 * Wave::KS; };
  auto vslab = [&](int j) { return (const uint16_t*)lds_v[((j - 1) / SPT) % NB] + ((j - 1) % SPT) * 32 * Wave::KS; };
  // loads of later tiles: issued at the start of iteration n, they fly
  // during its work; returns the loads this wavefront may leave in flight
  // at the end of the iteration
  auto issue = [&](int n) {
    int in_flight = 0;
    if (n == 0) {
      if (2 < NT) pipe_issue<D, BN, NW, false>(lds_k[2], kbase, rsk, 2 * BN, w.Lk, wave, lane);
      if (1 < NT) pipe_issue<D, BN, NW, true>(lds_v[1], vbase, rsk, BN, w.Lk, wave, lane);
    }
    if (n + 3 < NT) {
      pipe_issue<D, BN, NW, false>(lds_k[(n + 3) % NB], kbase, rsk, (n + 3) * BN, w.Lk, wave, lane);
      in_flight += G::PER_WAVE;
    }
    if (n + 2 < NT) {
      pipe_issue<D, BN, NW, true>(lds_v[(n + 2) % NB], vbase, rsk, (n + 2) * BN, w.Lk, wave, lane);
      in_flight += G::PER_WAVE;
    }
    return in_flight;
  };
  // one iteration with every piece of every stage conditional (the first
  // iteration, slabs that need a mask, the last slabs, finished wavefronts)
  auto generic = [&](int n) {
    for (int st = 0; st < SPT; ++st) {
      const int j = n * SPT + st;
      if (j > j_end) break;
      v8 p_cur[2] = {};
      float alpha = 1.f;
      bool resc = false;
      f32x16 s_next = {};
      if (j + 1 < j_end) s_next = wv.qk(kslab(j), 0, arow, g);
      if (j < j_end) {
        if (j >= j_full) Wave::template mask<CAUSAL>(s_cur, 32 * j, row, g, w.Lk, shift);
        resc = wv.softmax(s_cur, p_cur, alpha, a.scale_log2);
      }
      if (j >= 1) wv.pv(vslab(j), 0, p_prev, lane);
      if (resc) wv.rescale(alpha);
      s_cur = s_next;
      p_prev[0] = p_cur[0];
      p_prev[1] = p_cur[1];
    }
  };
  // Iterations [1, n_steady) run only steady stages: QK, softmax and PV each
  // present, no mask.
  int n_steady = 1;
  {
    const int lim = min(j_end - 1, j_full);  // (n + 1) * SPT <= lim
    if (lim >= 2 * SPT) n_steady = lim / SPT;
  }
  if (NIT > 0) {
    const int fl = issue(0);
    generic(0);
    wait_vmcnt_dyn<G::PER_WAVE>(fl);
    __syncthreads();
  }
  int n = 1;
  v8 kpre[pipe_kpre<D>()];
  constexpr int NVP = pipe_vpre<D>();
  v8 vpre[NVP > 0 ? NVP : 1];
  if (NVP > 0 && n < n_steady) Wave::v_pre(vslab(n * SPT), vpre, lane);
  if (SPT > 1 && n < n_steady) Wave::k_pre(kslab(n * SPT), kpre, arow, g);
  const bool lead_first = wave >= 4;  // wavefronts 4-7 (the younger on each SIMD) lead the first stage
  constexpr bool kAlternate = NW == 8;  // two wavefronts of the workgroup share each SIMD
  for (; n < n_steady; ++n) {
    const int fl = issue(n);
    // one slab per tile: the first slab of an iteration was only waited for
    // at the barrier that began it
    if (SPT == 1) Wave::k_pre(kslab(n), kpre, arow, g);
#pragma unroll
    for (int st = 0; st < SPT; ++st) {
      // Issue priority alternates between the two wavefronts of a SIMD:
      // otherwise the older one always wins arbitration, finishes the
      // iteration early and idles at the barrier while the younger one runs
      // alone.
      if (kAlternate) {
        if (lead_first == ((st & 1) == 0)) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      const int j = n * SPT + st;
      v8 p_cur[2];
      const f32x16 s_next = wv.qk_pre(kslab(j), kpre, arow, g);
      const bool ok = wv.softmax_fast(s_cur, p_cur, a.scale_log2);
      if constexpr (NVP > 0) {
        wv.pv_pre(vslab(j), p_prev, vpre, lane);
        Wave::v_pre(vslab(j + 1), vpre, lane);  // V tile of the next stage: resident (issued two iterations ago)
      } else {
        wv.pv(vslab(j), 0, p_prev, lane);
      }
      // first K fragments of the next stage: with two or more slabs per tile
      // its slab is in K tile n + 1, which this iteration reads already
      if (SPT > 1) Wave::k_pre(kslab(j + 1), kpre, arow, g);
      if (__builtin_expect(!ok, 0)) {  // rare: redo the slab with raised references, O rescaled after PV(j-1)
        asm volatile("" ::: "memory");  // a real branch: the redo must not be executed speculatively
        float alpha;
        if (wv.softmax(s_cur, p_cur, alpha, a.scale_log2)) wv.rescale(alpha);
      }
      s_cur = s_next;
      p_prev[0] = p_cur[0];
      p_prev[1] = p_cur[1];
    }
    wait_vmcnt_dyn<G::PER_WAVE>(fl);
    __syncthreads();
  }
  __builtin_amdgcn_s_setprio(0);
  for (; n < NIT; ++n) {
    const int fl = issue(n);
    generic(n);
    wait_vmcnt_dyn<G::PER_WAVE>(fl);
    __syncthreads();
  }

  // ---- epilogue: normalise, write out (16-bit, round to nearest even) and lse.
  // The wavefront's rows go through its own 32-row slice of the K buffers
  // (free after the last barrier; every load has landed): registers hold 4
  // columns per row and lane, LDS hands them back as 16-byte row pieces, so
  // each global store writes whole rows instead of 8 bytes of 32 rows.
  T* __restrict__ op = (T*)a.out;
  // l is exactly 0 only for a row that saw no key; a NaN score gives a NaN
  // sum, which must reach out and lse rather than read as an empty row
  const float l = pair_sum(wv.l_run);
  const float inv = l != 0.f ? 1.f / l : 0.f;
  uint16_t* stage = &lds_k[0][0] + wave * 32 * Wave::KS;
#pragma unroll
  for (int db = 0; db < Wave::DB; ++db)
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      typename Elem16<T>::v4 v4;
#pragma unroll
      for (int c = 0; c < 4; ++c) v4[c] = (T)(wv.o[db][4 * s4 + c] * inv);
      *(typename Elem16<T>::v4*)(stage + tiling::ks_index<D>(l32, 4 * db + s4) + 4 * g) = v4;
    }
  constexpr int CH = D / 8;  // 16-byte pieces per row
  static_assert((32 * CH) % 64 == 0, "row pieces must fill whole wavefront passes");
#pragma unroll
  for (int it = 0; it < 32 * CH / 64; ++it) {
    const int c = it * 64 + lane;
    const int r = c / CH, ch = c % CH;
    const v8 val = *(const v8*)(stage + tiling::ks_index<D>(r, ch));
    if (wrow0 + r < w.Lq) *(v8*)(op + (int64_t)(w.q_start + wrow0 + r) * rs + (int64_t)w.h * D + 8 * ch) = val;
  }
  if (row < w.Lq && g == 0)
    a.lse[(int64_t)w.h * a.total_q + w.q_start + row] = l != 0.f ? (wv.m_run + fast_log2(l)) * kLn2 : kNegInf;
}

// NW wavefronts of 32 query rows: 8 (two per SIMD), or 4 (one per SIMD,
// which leaves a wavefront 512 registers: head_dim 256).
template <typename T, int D, int BN, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd16_pipe_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[kPipeBuffers][BN * tiling::k_stride<D>()];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[kPipeBuffers][BN * tiling::k_stride<D>()];
  WorkItem w;
  if (!decode_work<32 * NW>(a, w)) return;
  run_work<32 * NW, CAUSAL>(a, w, [&](const WorkItem& wi) { fwd16_pipe_item<T, D, BN, NW, CAUSAL>(a, wi, lds_k, lds_v); });
}

// ---------------------------------------------------------------------------
// fp32 forward (fp32 MFMA 32x32x2; no reduced precision anywhere)
// ---------------------------------------------------------------------------
// A/B operands of the fp32 MFMA are single elements per lane, so neither K
// nor V needs a transpose: rows are padded by 4 floats against bank conflicts.
// Register r of lane group g in the 32x32 accumulator holds key
// 8*(r/4) + 4g + r%4 of the 32-key block (natural key order in A).
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void fwd_f32_kernel(FwdArgs a) {
  constexpr int BN = 32;
  constexpr int BM = 32 * NW;
  constexpr int LD = D + 4;
  constexpr int DB = D / 32;
  constexpr int THREADS = NW * 64;
  constexpr int CHUNKS = BN * D / 4;  // float4 chunks per tile
  constexpr int PER_THREAD = CHUNKS / THREADS;
  static_assert(CHUNKS % THREADS == 0, "tile/threads mismatch");

  __shared__ __attribute__((aligned(16))) float lds_k[2][BN * LD];
  __shared__ __attribute__((aligned(16))) float lds_v[2][BN * LD];

  WorkItem w;
  if (!decode_work<BM>(a, w)) return;
  int n_full, n_end;
  key_tiles<BM, BN, CAUSAL>(w, n_full, n_end);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wrow0 = w.m * BM + wave * 32;
  const int shift = w.Lk - w.Lq;
  const int i = wrow0 + l32;

  // key/value head of this query head; K/V rows hold kv_heads * D elements
  const int hk = w.h / a.head_group;
  const float* __restrict__ kbase = (const float*)a.k + (int64_t)w.k_start * a.kv_row_stride + (int64_t)hk * D;
  const float* __restrict__ vbase = (const float*)a.v + (int64_t)w.k_start * a.kv_row_stride + (int64_t)hk * D;

  float qreg[D / 2];
  {
    const float* src = (const float*)a.q + (int64_t)(w.q_start + i) * a.row_stride + (int64_t)w.h * D;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qreg[ks] = (i < w.Lq) ? src[2 * ks + g] : 0.f;
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = kNegInf, l_run = 0.f;

  f32x4 kreg[PER_THREAD], vreg[PER_THREAD];
  auto load = [&](int key0) {
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it) {
      const int c = tid + it * THREADS;
      const int row = c / (D / 4), ch = c % (D / 4);
      f32x4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key0 + row < w.Lk) {
        kx = *(const f32x4*)(kbase + (int64_t)(key0 + row) * a.kv_row_stride + 4 * ch);
        vx = *(const f32x4*)(vbase + (int64_t)(key0 + row) * a.kv_row_stride + 4 * ch);
      }
      kreg[it] = kx;
      vreg[it] = vx;
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int it = 0; it < PER_THREAD; ++it) {
      const int c = tid + it * THREADS;
      const int row = c / (D / 4), ch = c % (D / 4);
      *(f32x4*)(&lds_k[buf][row * LD + 4 * ch]) = kreg[it];
      *(f32x4*)(&lds_v[buf][row * LD + 4 * ch]) = vreg[it];
    }
  };

  if (n_end > 0) { load(0); store(0); }
  __syncthreads();

  for (int n = 0; n < n_end; ++n) {
    const int buf = n & 1;
    const int key0 = n * BN;
    if (n + 1 < n_end) load(key0 + BN);
    const bool wave_active = (wrow0 < w.Lq) && (!CAUSAL || (key0 <= wrow0 + 31 + shift));
    if (wave_active) {
      const float* Ks = lds_k[buf];
      const float* Vs = lds_v[buf];
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 2; ++ks)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(Ks[l32 * LD + 2 * ks + g], qreg[ks], s, 0, 0, 0);
      if (n >= n_full) {
        const int lim = CAUSAL ? min(w.Lk - 1, i + shift) : (w.Lk - 1);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key > lim) s[r] = kNegInf;
        }
      }
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const float m_tile = pair_max(mx) * a.scale_log2;
      if (wave_any(m_tile > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, m_tile);
        const float alpha = fast_exp2(m_run - (m_new == kNegInf ? 0.f : m_new));
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      }
      const float m_use = m_run == kNegInf ? 0.f : m_run;
      float lsum = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, -m_use));
        lsum += s[r];
      }
      l_run += lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int key = 8 * (u >> 2) + 4 * g + (u & 3);
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * LD + db * 32 + l32], s[u], o[db], 0, 0, 0);
        }
      }
    }
    if (n + 1 < n_end) store(buf ^ 1);
    __syncthreads();
  }

  const float l = pair_sum(l_run);
  const float inv = l != 0.f ? 1.f / l : 0.f;  // NaN sums propagate (see the 16-bit kernel)
  if (i < w.Lq) {
    float* dst = (float*)a.out + (int64_t)(w.q_start + i) * a.row_stride + (int64_t)w.h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        f32x4 v4;
#pragma unroll
        for (int c = 0; c < 4; ++c) v4[c] = o[db][4 * s4 + c] * inv;
        *(f32x4*)(dst + db * 32 + 8 * s4 + 4 * g) = v4;
      }
    if (g == 0) a.lse[(int64_t)w.h * a.total_q + w.q_start + i] = l != 0.f ? (m_run + fast_log2(l)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// launch helpers
// ---------------------------------------------------------------------------
template <typename K>
hipError_t launch(K kernel, int grid, int block, hipStream_t stream, const FwdArgs& a) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Tile configuration per (dtype, head_dim): must agree with the kernels above.
TileConfig tile_config(int dtype, int head_dim) {
  TileConfig c{0, 0, 0};
  if (dtype == 1 || dtype == 2) {  // bf16, fp16
    if (head_dim == 128 || head_dim == 96) c = TileConfig{256, 64, 512};
    else if (head_dim == 256) c = TileConfig{128, 32, 256};
    else if (head_dim == 64) c = TileConfig{256, 128, 512};
  } else if (dtype == 0) {  // f32
    if (head_dim == 128 || head_dim == 96 || head_dim == 64) c = TileConfig{128, 32, 256};
  }
  return c;
}

TileConfig tile_config_short(int dtype, int head_dim) {
  if ((dtype == 1 || dtype == 2) && head_dim == 64) return TileConfig{128, 64, 256};
  if ((dtype == 1 || dtype == 2) && head_dim == 128) return TileConfig{128, 32, 256};
  return TileConfig{0, 0, 0};
}

hipError_t launch_tile_map(const int32_t* cu_q, int batch, int block_m, int32_t* blk_start, hipStream_t stream) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(256), 0, stream, cu_q, batch, block_m, blk_start);
  return hipGetLastError();
}

hipError_t launch_check_cu(const int32_t* cu_q, const int32_t* cu_k, int batch, int total_q, int total_k,
                           int max_q, int max_k, int32_t* flags, hipStream_t stream) {
  hipLaunchKernelGGL(check_cu_kernel, dim3(1), dim3(256), 0, stream, cu_q, cu_k, batch, total_q, total_k,
                     max_q, max_k, flags);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_fwd16(int head_dim, bool causal, bool short_items, int grid, const FwdArgs& a, hipStream_t stream) {
  if (short_items) {  // 128-row items of four wavefronts (tile_config_short)
    if (head_dim == 128)
      return causal ? launch(fwd16_pipe_kernel<T, 128, 32, 4, true>, grid, 256, stream, a)
                    : launch(fwd16_pipe_kernel<T, 128, 32, 4, false>, grid, 256, stream, a);
    if (head_dim == 64)
      return causal ? launch(fwd16_pipe_kernel<T, 64, 64, 4, true>, grid, 256, stream, a)
                    : launch(fwd16_pipe_kernel<T, 64, 64, 4, false>, grid, 256, stream, a);
    return hipErrorInvalidValue;
  }
  if (head_dim == 128)
    return causal ? launch(fwd16_pipe_kernel<T, 128, 64, 8, true>, grid, 512, stream, a)
                  : launch(fwd16_pipe_kernel<T, 128, 64, 8, false>, grid, 512, stream, a);
  if (head_dim == 96)
    return causal ? launch(fwd16_pipe_kernel<T, 96, 64, 8, true>, grid, 512, stream, a)
                  : launch(fwd16_pipe_kernel<T, 96, 64, 8, false>, grid, 512, stream, a);
  if (head_dim == 64)
    return causal ? launch(fwd16_pipe_kernel<T, 64, 128, 8, true>, grid, 512, stream, a)
                  : launch(fwd16_pipe_kernel<T, 64, 128, 8, false>, grid, 512, stream, a);
  if (head_dim == 256)
    return causal ? launch(fwd16_pipe_kernel<T, 256, 32, 4, true>, grid, 256, stream, a)
                  : launch(fwd16_pipe_kernel<T, 256, 32, 4, false>, grid, 256, stream, a);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(int dtype, int head_dim, bool causal, bool short_items, int grid, const FwdArgs& a,
                      hipStream_t stream) {
  if (dtype == 1) {
    return launch_fwd16<__bf16>(head_dim, causal, short_items, grid, a, stream);
  } else if (dtype == 2) {
    return launch_fwd16<_Float16>(head_dim, causal, short_items, grid, a, stream);
  } else if (dtype == 0) {
    if (short_items) return hipErrorInvalidValue;
    if (head_dim == 128)
      return causal ? launch(fwd_f32_kernel<128, 4, true>, grid, 256, stream, a)
                    : launch(fwd_f32_kernel<128, 4, false>, grid, 256, stream, a);
    if (head_dim == 96)
      return causal ? launch(fwd_f32_kernel<96, 4, true>, grid, 256, stream, a)
                    : launch(fwd_f32_kernel<96, 4, false>, grid, 256, stream, a);
    if (head_dim == 64)
      return causal ? launch(fwd_f32_kernel<64, 4, true>, grid, 256, stream, a)
                    : launch(fwd_f32_kernel<64, 4, false>, grid, 256, stream, a);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
