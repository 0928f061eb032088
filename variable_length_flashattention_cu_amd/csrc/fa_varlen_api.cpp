// fa_varlen_api.cpp -- the C ABI declared in include/fa_varlen.h: argument
// validation, launch sizing and the kernel launches of the forward and
// backward passes.  Every check runs on the host before any HIP call, so a
// validation error launches nothing.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>

#include "fa_varlen.h"
#include "fa_varlen_launch.h"

namespace {

constexpr double kLog2e = 1.4426950408889634074;
// Compute units of an MI355X; with at most kPairLimit workgroups per CU the
// causal forward pairs query blocks (see run_work in the kernels).
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kPairLimit = 8;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

struct Plan {
  fa::TileConfig tc;
  int64_t tmax;
  int64_t grid;
};

// Validation shared by fa_varlen_fwd and fa_varlen_fwd_mapped.
bool known_dtype(int32_t dtype) {
  return dtype == FA_DTYPE_F32 || dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16;
}

int validate(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
             int32_t max_q, int32_t max_k, float scale, int32_t causal, const void* out, const float* lse,
             int32_t batch, int32_t total_q, int32_t total_k, int32_t heads, int32_t heads_k, int32_t head_dim,
             int32_t dtype, Plan* plan) {
  if (!q || !k || !v || !cu_q || !cu_k || !out || !lse) return FA_ERR_NULL;
  if (!known_dtype(dtype)) return FA_ERR_DTYPE;
  const fa::TileConfig tc = fa::tile_config(dtype, head_dim);
  if (tc.block_m == 0) return FA_ERR_HEAD_DIM;
  if (batch < 0 || total_q < 0 || total_k < 0 || heads < 1 || max_q < 0 || max_k < 0) return FA_ERR_SHAPE;
  if (heads_k < 1 || heads % heads_k != 0) return FA_ERR_SHAPE;
  if (max_q > total_q || max_k > total_k) return FA_ERR_SHAPE;
  // In-tile byte offsets are 32-bit: bound the token row size.
  if ((int64_t)heads * head_dim > (int64_t{1} << 22)) return FA_ERR_TOO_LARGE;
  if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(cu_q, 4) || !aligned(cu_k, 4)) return FA_ERR_ALIGN;
  // Upper bound on the number of work items: sum_b ceil(Lq_b / BM) is at most
  // batch * ceil(max_seqlen_q / BM) and at most ceil(total_q / BM) + batch - 1.
  const int64_t bm = tc.block_m;
  const int64_t by_max = (int64_t)batch * ((max_q + bm - 1) / bm);
  const int64_t by_total = (total_q + bm - 1) / bm + (batch > 0 ? batch - 1 : 0);
  const int64_t tmax = by_max < by_total ? by_max : by_total;
  const int64_t work = tmax * heads;
  const int64_t grid = (work + 7) / 8 * 8;
  if (grid > INT32_MAX || tmax > INT32_MAX) return FA_ERR_TOO_LARGE;
  plan->tc = tc;
  plan->tmax = tmax;
  plan->grid = grid;
  return FA_OK;
}

fa::FwdArgs make_args(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                      float scale, int32_t causal, void* out, float* lse, int32_t batch, int32_t total_q,
                      int32_t heads, int32_t heads_k, int32_t head_dim, const int32_t* blk_start,
                      const Plan& plan) {
  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.blk_start = blk_start;
  a.row_stride = (int64_t)heads * head_dim;
  a.kv_row_stride = (int64_t)heads_k * head_dim;
  a.head_group = heads / heads_k;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.batch = batch;
  a.tmax = (int32_t)plan.tmax;
  a.n_work = (int32_t)(plan.tmax * heads);
  a.total_q = total_q;
  a.pair_blocks = (causal && plan.tmax * heads <= kPairLimit * kComputeUnits) ? 1 : 0;
  return a;
}

// Backward workspace: dq accumulator, row terms, key-block map (256-byte aligned parts).
struct BwdLayout {
  size_t dq_acc, drow, blk, total;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(int64_t batch, int64_t total_q, int64_t heads, int64_t head_dim) {
  BwdLayout l;
  l.dq_acc = 0;
  l.drow = round256((size_t)total_q * heads * head_dim * sizeof(float));
  l.blk = l.drow + round256((size_t)heads * total_q * sizeof(float));
  l.total = l.blk + round256(((size_t)batch + 1) * sizeof(int32_t));
  return l;
}

// Key/value-cache attention: split count and workspace.
constexpr int kMaxSplits = 64;

int64_t dec_parts(int32_t num_splits) { return (int64_t)(num_splits > 0 ? num_splits : kMaxSplits) * fa::decode_waves(); }

size_t dec_workspace(int64_t total_q, int64_t heads, int64_t head_dim, int32_t num_splits) {
  const int64_t rows = total_q * heads * dec_parts(num_splits);
  return round256((size_t)rows * head_dim * sizeof(float)) + round256((size_t)rows * 2 * sizeof(float));
}

// Splits when the caller leaves the choice: about eight workgroups per
// compute unit (the pass streams the cache from HBM and needs many loads in
// flight), at least one 64-key tile per wavefront of a split.
int32_t auto_splits(int64_t batch, int64_t kv_heads, int64_t max_k) {
  const int64_t items = batch * kv_heads;
  int64_t s = items > 0 ? (8 * kComputeUnits + items - 1) / items : 1;
  const int64_t by_keys = (max_k + 64 * 4 - 1) / (64 * 4);  // a 64-key tile per wavefront
  if (s > by_keys) s = by_keys;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int32_t)(s < 1 ? 1 : s);
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required pointer is NULL";
    case FA_ERR_DTYPE: return "unsupported dtype (expected FA_DTYPE_F32, FA_DTYPE_BF16 or FA_DTYPE_F16)";
    case FA_ERR_SHAPE:
      return "invalid sizes (negative, zero heads, key/value heads not dividing the query heads, or max_seqlen "
             "above the row count)";
    case FA_ERR_HEAD_DIM: return "unsupported head_dim (64, 96, 128; 256 with bf16/fp16)";
    case FA_ERR_ALIGN: return "misaligned pointer (tensors need 16 bytes, lse and offsets 4 bytes)";
    case FA_ERR_ARG: return "invalid argument (softmax_scale must be finite and > 0, causal 0 or 1, block_m 1..4096)";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_TOO_LARGE: return "problem too large for one launch";
    case FA_ERR_WORKSPACE: return "backward workspace missing or smaller than fa_varlen_bwd_workspace_size";
    default: return "unknown status";
  }
}

int fa_varlen_block_sizes(int32_t head_dim, int32_t dtype, int32_t* block_m, int32_t* block_n) {
  if (!block_m || !block_n) return FA_ERR_NULL;
  if (!known_dtype(dtype)) return FA_ERR_DTYPE;
  const fa::TileConfig tc = fa::tile_config(dtype, head_dim);
  if (tc.block_m == 0) return FA_ERR_HEAD_DIM;
  *block_m = tc.block_m;
  *block_n = tc.block_n;
  return FA_OK;
}

int fa_varlen_tile_map(const int32_t* cu_seqlens_q, int32_t batch, int32_t block_m, int32_t* blk_start,
                       void* stream) {
  if (!cu_seqlens_q || !blk_start) return FA_ERR_NULL;
  if (batch < 0) return FA_ERR_SHAPE;
  if (block_m < 1 || block_m > 4096) return FA_ERR_ARG;
  if (!aligned(cu_seqlens_q, 4) || !aligned(blk_start, 4)) return FA_ERR_ALIGN;
  if (fa::launch_tile_map(cu_seqlens_q, batch, block_m, blk_start, (hipStream_t)stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_fwd_mapped(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         float softmax_scale, int32_t causal, void* out, float* lse, int32_t batch,
                         int32_t total_q, int32_t total_k, int32_t num_heads, int32_t num_heads_k,
                         int32_t head_dim, int32_t dtype, const int32_t* blk_start, void* stream) {
  Plan plan;
  int st = validate(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                    out, lse, batch, total_q, total_k, num_heads, num_heads_k, head_dim, dtype, &plan);
  if (st != FA_OK) return st;
  if (!blk_start) return FA_ERR_NULL;
  if (!aligned(blk_start, 4)) return FA_ERR_ALIGN;
  if (plan.grid == 0) return FA_OK;  // no query rows: nothing to compute
  const fa::FwdArgs a = make_args(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, causal, out, lse, batch,
                                  total_q, num_heads, num_heads_k, head_dim, blk_start, plan);
  if (fa::launch_fwd(dtype, head_dim, causal != 0, (int)plan.grid, a, (hipStream_t)stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                  const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                  int32_t causal, void* out, float* lse, int32_t batch, int32_t total_q, int32_t total_k,
                  int32_t num_heads, int32_t num_heads_k, int32_t head_dim, int32_t dtype, void* stream) {
  Plan plan;
  int st = validate(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                    out, lse, batch, total_q, total_k, num_heads, num_heads_k, head_dim, dtype, &plan);
  if (st != FA_OK) return st;
  if (plan.grid == 0) return FA_OK;
  hipStream_t s = (hipStream_t)stream;
  int32_t* blk_start = nullptr;
  if (hipMallocAsync((void**)&blk_start, sizeof(int32_t) * ((size_t)batch + 1), s) != hipSuccess)
    return FA_ERR_HIP;
  int rc = FA_OK;
  if (fa::launch_tile_map(cu_seqlens_q, batch, plan.tc.block_m, blk_start, s) != hipSuccess) {
    rc = FA_ERR_HIP;
  } else {
    const fa::FwdArgs a = make_args(q, k, v, cu_seqlens_q, cu_seqlens_k, softmax_scale, causal, out, lse, batch,
                                    total_q, num_heads, num_heads_k, head_dim, blk_start, plan);
    if (fa::launch_fwd(dtype, head_dim, causal != 0, (int)plan.grid, a, s) != hipSuccess) rc = FA_ERR_HIP;
  }
  if (hipFreeAsync(blk_start, s) != hipSuccess) rc = FA_ERR_HIP;
  return rc;
}

int fa_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t num_heads, int32_t head_dim,
                                 size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  if (batch < 0 || total_q < 0 || num_heads < 1 || head_dim < 1) return FA_ERR_SHAPE;
  *bytes = bwd_layout(batch, total_q, num_heads, head_dim).total;
  return FA_OK;
}

int fa_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t max_seqlen_q,
                  int32_t max_seqlen_k, float softmax_scale, int32_t causal, void* dq, void* dk, void* dv,
                  int32_t batch, int32_t total_q, int32_t total_k, int32_t num_heads, int32_t num_heads_k,
                  int32_t head_dim, int32_t dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dout || !dq || !dk || !dv) return FA_ERR_NULL;
  Plan plan;  // the forward's checks cover q, k, v, offsets, out, lse, sizes, scale, causal
  int st = validate(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal, out,
                    lse, batch, total_q, total_k, num_heads, num_heads_k, head_dim, dtype, &plan);
  if (st != FA_OK) return st;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_DTYPE;
  const int bn = fa::bwd_block_n(dtype, head_dim);
  if (bn == 0) return FA_ERR_HEAD_DIM;
  if (!aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16)) return FA_ERR_ALIGN;
  const BwdLayout lay = bwd_layout(batch, total_q, num_heads, head_dim);
  if (!workspace || workspace_bytes < lay.total) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  // key blocks: sum_b ceil(Lk_b / bn) <= min(batch * ceil(max_k / bn), ceil(total_k / bn) + batch - 1)
  const int64_t by_max = (int64_t)batch * ((max_seqlen_k + bn - 1) / bn);
  const int64_t by_total = ((int64_t)total_k + bn - 1) / bn + (batch > 0 ? batch - 1 : 0);
  const int64_t compact = by_max < by_total ? by_max : by_total;
  // Under a causal mask a sequence's first key blocks carry the most work.
  // Block-major slots (block j of every sequence, then block j + 1) dispatch
  // them first; slots of sequences shorter than j stay empty, so this order
  // is used only while they are at most two thirds of the grid.
  const bool by_block = causal != 0 && 4 * by_max <= 5 * compact;
  const int64_t tmax = by_block ? by_max : compact;
  const int64_t grid = (tmax * num_heads_k + 7) / 8 * 8;
  if (grid > INT32_MAX) return FA_ERR_TOO_LARGE;

  char* ws = static_cast<char*>(workspace);
  int32_t* blk = reinterpret_cast<int32_t*>(ws + lay.blk);
  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.blk_start = blk;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dq_acc = reinterpret_cast<float*>(ws + lay.dq_acc);
  a.drow = reinterpret_cast<float*>(ws + lay.drow);
  a.row_stride = (int64_t)num_heads * head_dim;
  a.kv_row_stride = (int64_t)num_heads_k * head_dim;
  a.scale = softmax_scale;
  a.scale_log2 = (float)((double)softmax_scale * kLog2e);
  a.batch = batch;
  a.tmax = (int32_t)tmax;
  a.by_block = by_block ? 1 : 0;
  a.n_work = (int32_t)(tmax * num_heads_k);
  a.total_q = total_q;
  a.heads = num_heads;
  a.head_group = num_heads / num_heads_k;

  hipStream_t s = (hipStream_t)stream;
  if (fa::launch_bwd_prep(dtype, head_dim, a, s) != hipSuccess) return FA_ERR_HIP;
  if (grid > 0) {
    if (!by_block && fa::launch_tile_map(cu_seqlens_k, batch, bn, blk, s) != hipSuccess) return FA_ERR_HIP;
    if (fa::launch_bwd(dtype, head_dim, causal != 0, (int)grid, a, s) != hipSuccess) return FA_ERR_HIP;
  }
  if (fa::launch_bwd_dq(dtype, head_dim, a, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_kvcache_workspace_size(int32_t total_q, int32_t num_heads, int32_t head_dim, int32_t num_splits,
                                     size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  if (total_q < 0 || num_heads < 1 || head_dim < 1) return FA_ERR_SHAPE;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  *bytes = dec_workspace(total_q, num_heads, head_dim, num_splits);
  return FA_OK;
}

int fa_varlen_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache, const int32_t* cu_seqlens_q,
                          const int32_t* seqlens_k, const int32_t* leftpad_k, const int32_t* block_table,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                          void* out, float* lse, int32_t batch, int32_t total_q, int32_t cache_blocks,
                          int32_t cache_rows, int32_t blocks_per_seq, int32_t num_heads, int32_t num_heads_k,
                          int32_t head_dim, int32_t dtype, int32_t num_splits, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !seqlens_k || !out || !lse) return FA_ERR_NULL;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return FA_ERR_HEAD_DIM;
  if (batch < 0 || total_q < 0 || num_heads < 1 || max_seqlen_q < 0 || max_seqlen_k < 0) return FA_ERR_SHAPE;
  if (num_heads_k < 1 || num_heads % num_heads_k != 0) return FA_ERR_SHAPE;
  if (max_seqlen_q > total_q || cache_rows < 1 || cache_blocks < 0) return FA_ERR_SHAPE;
  if (block_table) {
    if (blocks_per_seq < 1 || (int64_t)max_seqlen_k > (int64_t)blocks_per_seq * cache_rows) return FA_ERR_SHAPE;
  } else {
    if (cache_blocks < batch || max_seqlen_k > cache_rows) return FA_ERR_SHAPE;
  }
  if ((int64_t)num_heads * head_dim > (int64_t{1} << 22)) return FA_ERR_TOO_LARGE;
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse, 4) || !aligned(cu_seqlens_q, 4) || !aligned(seqlens_k, 4)) return FA_ERR_ALIGN;
  if ((leftpad_k && !aligned(leftpad_k, 4)) || (block_table && !aligned(block_table, 4))) return FA_ERR_ALIGN;
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(batch, num_heads_k, max_seqlen_k);
  if (!workspace || workspace_bytes < dec_workspace(total_q, num_heads, head_dim, splits)) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  if ((int64_t)batch * num_heads_k * splits > INT32_MAX) return FA_ERR_TOO_LARGE;
  if (batch == 0 || total_q == 0) return FA_OK;  // no query rows

  const int64_t rows = (int64_t)total_q * num_heads * splits * fa::decode_waves();
  fa::DecArgs a;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.out = out;
  a.lse = lse;
  a.cu_q = cu_seqlens_q;
  a.seqlens_k = seqlens_k;
  a.leftpad_k = leftpad_k;
  a.block_table = block_table;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)rows * head_dim * 4));
  a.row_stride = (int64_t)num_heads * head_dim;
  a.kv_row_stride = (int64_t)num_heads_k * head_dim;
  a.scale_log2 = (float)((double)softmax_scale * kLog2e);
  a.batch = batch;
  a.total_q = total_q;
  a.heads = num_heads;
  a.kv_heads = num_heads_k;
  a.head_group = num_heads / num_heads_k;
  a.cache_rows = cache_rows;
  a.blocks_per_seq = block_table ? blocks_per_seq : 0;
  a.num_splits = splits;
  if (fa::launch_decode(dtype, head_dim, causal != 0, a, (hipStream_t)stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_check_cu_seqlens(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t batch,
                               int32_t total_q, int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t* flags, void* stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !flags) return FA_ERR_NULL;
  if (batch < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return FA_ERR_SHAPE;
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) || !aligned(flags, 4)) return FA_ERR_ALIGN;
  if (fa::launch_check_cu(cu_seqlens_q, cu_seqlens_k, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, flags,
                          (hipStream_t)stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

}  // extern "C"
