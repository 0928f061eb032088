// fa_varlen_api.cpp -- the C ABI declared in include/fa_varlen.h: descriptor
// validation, launch sizing and the kernel launches of the forward pass, the
// backward pass and attention against a key/value cache.  Every check runs on
// the host before any HIP call, so a validation error launches nothing.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "fa_varlen.h"
#include "fa_varlen_launch.h"

namespace {

constexpr double kLog2e = 1.4426950408889634074;
// With at most kPairLimit workgroups per compute unit the causal forward pass
// pairs query blocks (see run_work in the kernels).
constexpr int64_t kPairLimit = 8;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

// ---------------------------------------------------------------------------
// device properties
// ---------------------------------------------------------------------------
// Compute units of the current device, queried once per device and cached
// (the query is a runtime call; the value never changes).
int compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || n < 1)
    n = 256;  // MI355X; only sizes the schedule, never correctness
  if (dev >= 0) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// ---------------------------------------------------------------------------
// descriptors
// ---------------------------------------------------------------------------
int elem_code(int32_t dtype) {
  switch (dtype) {
    case FA_DTYPE_F32: return fa::kElemF32;
    case FA_DTYPE_BF16: return fa::kElemBF16;
    case FA_DTYPE_F16: return fa::kElemF16;
    default: return -1;
  }
}
int elem_size(int32_t dtype) { return dtype == FA_DTYPE_BF16 || dtype == FA_DTYPE_F16 ? 2 : 4; }

bool rank_ok(const fa_tensor& t, int ndim) {
  if (t.ndim != ndim) return false;
  for (int i = 0; i < ndim; ++i)
    if (t.shape[i] < 0) return false;
  return true;
}

int64_t numel(const fa_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}

// Row-major contiguity; the stride of a dimension of extent <= 1 is not used
// to address anything and is not looked at.
bool contiguous(const fa_tensor& t) {
  if (numel(t) == 0) return true;
  int64_t expect = 1;
  for (int i = t.ndim - 1; i >= 0; --i) {
    if (t.shape[i] > 1 && t.stride[i] != expect) return false;
    expect *= t.shape[i];
  }
  return true;
}

bool data_ok(const fa_tensor& t) { return t.data != nullptr || numel(t) == 0; }

bool same_shape(const fa_tensor& a, const fa_tensor& b) {
  if (a.ndim != b.ndim) return false;
  for (int i = 0; i < a.ndim; ++i)
    if (a.shape[i] != b.shape[i]) return false;
  return true;
}

// head_dim support per entry point
bool fwd_head_dim(int elem, int64_t d) {
  return d == 64 || d == 96 || d == 128 || (d == 256 && elem != fa::kElemF32);
}

// ---------------------------------------------------------------------------
// the attention problem shared by the forward and backward entry points
// ---------------------------------------------------------------------------
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t batch, total_q, total_k, heads, heads_k, head_dim, elem, dtype;
};

// q, k, v, offsets, out, lse, max_seqlen, scale and causal, in the documented
// order of status codes.  `extra` holds further tensors shaped and typed like
// q (first n_extra_q) or like k (the rest), checked with them.
int check_problem(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_q,
                  const fa_tensor* cu_k, const fa_tensor* out, const fa_tensor* lse, int32_t max_q, int32_t max_k,
                  float scale, int32_t causal, bool (*head_dim_ok)(int, int64_t), const fa_tensor* const* extra,
                  int n_extra, int n_extra_q, Problem* p) {
  if (!q || !k || !v || !cu_q || !cu_k || !out || !lse) return FA_ERR_NULL;
  for (int i = 0; i < n_extra; ++i)
    if (!extra[i]) return FA_ERR_NULL;
  // element types
  const int elem = elem_code(q->dtype);
  if (elem < 0 || k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype) return FA_ERR_DTYPE;
  for (int i = 0; i < n_extra; ++i)
    if (extra[i]->dtype != q->dtype) return FA_ERR_DTYPE;
  if (cu_q->dtype != FA_DTYPE_I32 || cu_k->dtype != FA_DTYPE_I32 || lse->dtype != FA_DTYPE_F32) return FA_ERR_DTYPE;
  // ranks, then head_dim, then the remaining shape relations
  if (!rank_ok(*q, 3) || !rank_ok(*k, 3) || !rank_ok(*v, 3) || !rank_ok(*out, 3) || !rank_ok(*cu_q, 1) ||
      !rank_ok(*cu_k, 1) || !rank_ok(*lse, 2))
    return FA_ERR_SHAPE;
  for (int i = 0; i < n_extra; ++i)
    if (!rank_ok(*extra[i], 3)) return FA_ERR_SHAPE;
  const int64_t D = q->shape[2];
  if (!head_dim_ok(elem, D)) return FA_ERR_HEAD_DIM;
  const int64_t Tq = q->shape[0], H = q->shape[1], Tk = k->shape[0], Hk = k->shape[1];
  if (H < 1 || Hk < 1 || H % Hk != 0 || k->shape[2] != D || !same_shape(*k, *v) || !same_shape(*q, *out))
    return FA_ERR_SHAPE;
  for (int i = 0; i < n_extra; ++i)
    if (!same_shape(*extra[i], i < n_extra_q ? *q : *k)) return FA_ERR_SHAPE;
  if (lse->shape[0] != H || lse->shape[1] != Tq) return FA_ERR_SHAPE;
  if (cu_q->shape[0] < 1 || cu_k->shape[0] != cu_q->shape[0]) return FA_ERR_SHAPE;
  if (max_q < 0 || max_k < 0 || max_q > Tq || max_k > Tk) return FA_ERR_SHAPE;
  // layout, then data pointers
  if (!contiguous(*q) || !contiguous(*k) || !contiguous(*v) || !contiguous(*out) || !contiguous(*lse) ||
      !contiguous(*cu_q) || !contiguous(*cu_k))
    return FA_ERR_LAYOUT;
  for (int i = 0; i < n_extra; ++i)
    if (!contiguous(*extra[i])) return FA_ERR_LAYOUT;
  if (!data_ok(*q) || !data_ok(*k) || !data_ok(*v) || !data_ok(*out) || !data_ok(*lse) || !cu_q->data ||
      !cu_k->data)
    return FA_ERR_NULL;
  for (int i = 0; i < n_extra; ++i)
    if (!data_ok(*extra[i])) return FA_ERR_NULL;
  // scalar arguments
  if (!(std::isfinite(scale) && scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  // alignment
  if (!aligned(q->data, 16) || !aligned(k->data, 16) || !aligned(v->data, 16) || !aligned(out->data, 16))
    return FA_ERR_ALIGN;
  for (int i = 0; i < n_extra; ++i)
    if (!aligned(extra[i]->data, 16)) return FA_ERR_ALIGN;
  if (!aligned(lse->data, 4) || !aligned(cu_q->data, 4) || !aligned(cu_k->data, 4)) return FA_ERR_ALIGN;
  // sizes one launch addresses: 32-bit row counts, 32-bit in-tile byte offsets
  if (Tq > INT32_MAX || Tk > INT32_MAX || H > INT32_MAX || cu_q->shape[0] - 1 > INT32_MAX) return FA_ERR_TOO_LARGE;
  if (H * D > (int64_t{1} << 22) || Hk * D > (int64_t{1} << 22)) return FA_ERR_TOO_LARGE;
  p->q = q->data;
  p->k = k->data;
  p->v = v->data;
  p->out = out->data;
  p->lse = static_cast<float*>(lse->data);
  p->cu_q = static_cast<const int32_t*>(cu_q->data);
  p->cu_k = static_cast<const int32_t*>(cu_k->data);
  p->batch = (int32_t)(cu_q->shape[0] - 1);
  p->total_q = (int32_t)Tq;
  p->total_k = (int32_t)Tk;
  p->heads = (int32_t)H;
  p->heads_k = (int32_t)Hk;
  p->head_dim = (int32_t)D;
  p->elem = elem;
  p->dtype = q->dtype;
  return FA_OK;
}

// An int32 vector [n] (offsets, lengths, maps, flags).
int check_i32_vector(const fa_tensor* t, int64_t n) {
  if (!t) return FA_ERR_NULL;
  if (t->dtype != FA_DTYPE_I32) return FA_ERR_DTYPE;
  if (!rank_ok(*t, 1) || t->shape[0] != n) return FA_ERR_SHAPE;
  if (!contiguous(*t)) return FA_ERR_LAYOUT;
  if (!data_ok(*t)) return FA_ERR_NULL;
  if (!aligned(t->data, 4)) return FA_ERR_ALIGN;
  return FA_OK;
}

// ---------------------------------------------------------------------------
// forward launch sizing
// ---------------------------------------------------------------------------
struct Plan {
  fa::TileConfig tc;
  bool short_items;  // the 128-row configuration of tile_config_short
  int64_t tmax;
  int64_t grid;
};

// Longest query sequence for which the entry points that build their own map
// take the 128-row items of tile_config_short: items of short sequences have
// few key tiles, and smaller items with two workgroups per compute unit
// overlap more of each item's start-up (at 2048 rows the larger items were
// faster again).
constexpr int32_t kShortMaxQ = 1024;

// own_map: the caller of the plan builds the map itself (or needs none), so
// it may take the short configuration; the mapped entry point keeps the BM of
// fa_varlen_block_sizes.
int plan_fwd(const Problem& p, int32_t max_q, bool own_map, Plan* plan) {
  const fa::TileConfig ts = fa::tile_config_short(p.elem, p.head_dim);
  const bool short_items = own_map && ts.block_m > 0 && max_q <= kShortMaxQ;
  const fa::TileConfig tc = short_items ? ts : fa::tile_config(p.elem, p.head_dim);
  // Upper bound on the number of work items: sum_b ceil(Lq_b / BM) is at most
  // batch * ceil(max_seqlen_q / BM) and at most ceil(total_q / BM) + batch - 1.
  const int64_t bm = tc.block_m;
  const int64_t by_max = (int64_t)p.batch * ((max_q + bm - 1) / bm);
  const int64_t by_total = (p.total_q + bm - 1) / bm + (p.batch > 0 ? p.batch - 1 : 0);
  const int64_t tmax = by_max < by_total ? by_max : by_total;
  const int64_t work = tmax * p.heads;
  const int64_t grid = (work + 7) / 8 * 8;
  if (grid > INT32_MAX || tmax > INT32_MAX) return FA_ERR_TOO_LARGE;
  plan->tc = tc;
  plan->short_items = short_items;
  plan->tmax = tmax;
  plan->grid = grid;
  return FA_OK;
}

fa::FwdArgs make_fwd_args(const Problem& p, float scale, int32_t causal, const int32_t* blk_start, const Plan& plan) {
  fa::FwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.lse = p.lse;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.blk_start = blk_start;
  a.row_stride = (int64_t)p.heads * p.head_dim;
  a.kv_row_stride = (int64_t)p.heads_k * p.head_dim;
  a.head_group = p.heads / p.heads_k;
  a.scale_log2 = (float)((double)scale * kLog2e);
  a.batch = p.batch;
  a.tmax = (int32_t)plan.tmax;
  a.n_work = (int32_t)(plan.tmax * p.heads);
  a.total_q = p.total_q;
  a.pair_blocks = (causal && plan.tmax * p.heads <= kPairLimit * compute_units()) ? 1 : 0;
  return a;
}

// The forward pass with the map in `blk_start` (built by the caller, or by
// fwd_with_map below).
int launch_fwd_mapped(const Problem& p, const Plan& plan, float scale, int32_t causal, const int32_t* blk_start,
                      hipStream_t s) {
  if (plan.grid == 0) return FA_OK;  // no query rows: nothing to compute
  const fa::FwdArgs a = make_fwd_args(p, scale, causal, blk_start, plan);
  if (fa::launch_fwd(p.elem, p.head_dim, causal != 0, plan.short_items, (int)plan.grid, a, s) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

// ---------------------------------------------------------------------------
// backward workspace
// ---------------------------------------------------------------------------
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

// ---------------------------------------------------------------------------
// key/value-cache attention: split count and workspace
// ---------------------------------------------------------------------------
constexpr int kMaxSplits = 64;

// One fp32 partial (O, max, sum) per (query row, head, split): the
// workgroup's wavefronts merge theirs before writing.
size_t dec_workspace(int64_t total_q, int64_t heads, int64_t head_dim, int32_t num_splits) {
  const int64_t rows = total_q * heads * (num_splits > 0 ? num_splits : kMaxSplits);
  return round256((size_t)rows * head_dim * sizeof(float)) + round256((size_t)rows * 2 * sizeof(float));
}

// Splits when the caller leaves the choice: about eight workgroups per
// compute unit (the pass streams the cache from HBM and needs many loads in
// flight), at least 64 keys (two 32-key tiles) per wavefront of a split.
int32_t auto_splits(int64_t batch, int64_t kv_heads, int64_t max_k) {
  const int64_t items = batch * kv_heads;
  int64_t s = items > 0 ? (8 * (int64_t)compute_units() + items - 1) / items : 1;
  const int64_t by_keys = (max_k + 64 * 4 - 1) / (64 * 4);  // 64 keys for each of the 4 wavefronts
  if (s > by_keys) s = by_keys;
  if (s > kMaxSplits) s = kMaxSplits;
  return (int32_t)(s < 1 ? 1 : s);
}

}  // namespace

extern "C" {

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "a required tensor descriptor or pointer is NULL";
    case FA_ERR_DTYPE: return "unsupported element type (attention tensors: FA_DTYPE_F32, FA_DTYPE_BF16 or "
                              "FA_DTYPE_F16 as the entry point allows; offsets int32; lse float32)";
    case FA_ERR_SHAPE:
      return "invalid shape (wrong rank, negative or inconsistent sizes, key/value heads not dividing the query "
             "heads, or max_seqlen above the row count)";
    case FA_ERR_HEAD_DIM: return "unsupported head_dim for this dtype and entry point";
    case FA_ERR_LAYOUT: return "tensor not contiguous in row-major order";
    case FA_ERR_ALIGN: return "misaligned data (attention tensors need 16 bytes, lse and int32 arrays 4 bytes)";
    case FA_ERR_ARG: return "invalid argument (softmax_scale must be finite and > 0, causal 0 or 1, num_splits "
                            "0..64)";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_TOO_LARGE: return "problem too large for one launch";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the size function reports";
    case FA_ERR_SCRATCH: return "batch larger than the static work-item map of fa_varlen_fwd_noalloc (65535 sequences)";
    default: return "unknown status";
  }
}

int fa_varlen_block_sizes(int32_t head_dim, int32_t dtype, int32_t* block_m, int32_t* block_n) {
  if (!block_m || !block_n) return FA_ERR_NULL;
  const int elem = elem_code(dtype);
  if (elem < 0) return FA_ERR_DTYPE;
  if (!fwd_head_dim(elem, head_dim)) return FA_ERR_HEAD_DIM;
  const fa::TileConfig tc = fa::tile_config(elem, head_dim);
  *block_m = tc.block_m;
  *block_n = tc.block_n;
  return FA_OK;
}

int fa_varlen_tile_map(const fa_tensor* cu_seqlens_q, int32_t max_seqlen_q, int32_t head_dim, int32_t dtype,
                       fa_tensor* blk_start_out, hipStream_t stream) {
  if (!cu_seqlens_q || !blk_start_out) return FA_ERR_NULL;
  const int elem = elem_code(dtype);
  if (elem < 0) return FA_ERR_DTYPE;
  if (!fwd_head_dim(elem, head_dim)) return FA_ERR_HEAD_DIM;
  if (cu_seqlens_q->dtype != FA_DTYPE_I32) return FA_ERR_DTYPE;
  if (!rank_ok(*cu_seqlens_q, 1) || cu_seqlens_q->shape[0] < 1) return FA_ERR_SHAPE;
  const int64_t batch = cu_seqlens_q->shape[0] - 1;
  if (max_seqlen_q < 0) return FA_ERR_SHAPE;
  int st = check_i32_vector(cu_seqlens_q, batch + 1);
  if (st != FA_OK) return st;
  st = check_i32_vector(blk_start_out, batch + 1);
  if (st != FA_OK) return st;
  if (batch > INT32_MAX - 1) return FA_ERR_TOO_LARGE;
  const fa::TileConfig tc = fa::tile_config(elem, head_dim);
  if (fa::launch_tile_map(static_cast<const int32_t*>(cu_seqlens_q->data), (int)batch, tc.block_m,
                          static_cast<int32_t*>(blk_start_out->data), stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_fwd_mapped(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_seqlens_q,
                         const fa_tensor* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                         float softmax_scale, int32_t causal, fa_tensor* out, fa_tensor* lse,
                         const fa_tensor* blk_start, hipStream_t stream) {
  Problem p;
  int st = check_problem(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, max_seqlen_q, max_seqlen_k, softmax_scale,
                         causal, fwd_head_dim, nullptr, 0, 0, &p);
  if (st != FA_OK) return st;
  st = check_i32_vector(blk_start, (int64_t)p.batch + 1);
  if (st != FA_OK) return st;
  Plan plan;
  st = plan_fwd(p, max_seqlen_q, false, &plan);
  if (st != FA_OK) return st;
  return launch_fwd_mapped(p, plan, softmax_scale, causal, static_cast<const int32_t*>(blk_start->data), stream);
}

int fa_varlen_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_seqlens_q,
                  const fa_tensor* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                  int32_t causal, fa_tensor* out, fa_tensor* lse, hipStream_t stream) {
  Problem p;
  int st = check_problem(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, max_seqlen_q, max_seqlen_k, softmax_scale,
                         causal, fwd_head_dim, nullptr, 0, 0, &p);
  if (st != FA_OK) return st;
  Plan plan;
  st = plan_fwd(p, max_seqlen_q, true, &plan);
  if (st != FA_OK) return st;
  if (plan.grid == 0) return FA_OK;
  // small batches: the kernel rebuilds the map itself (no allocation, one launch)
  if (p.batch <= fa::kMaplessBatch) return launch_fwd_mapped(p, plan, softmax_scale, causal, nullptr, stream);
  int32_t* blk_start = nullptr;
  if (hipMallocAsync((void**)&blk_start, sizeof(int32_t) * ((size_t)p.batch + 1), stream) != hipSuccess)
    return FA_ERR_HIP;
  int rc = FA_OK;
  if (fa::launch_tile_map(p.cu_q, p.batch, plan.tc.block_m, blk_start, stream) != hipSuccess)
    rc = FA_ERR_HIP;
  else
    rc = launch_fwd_mapped(p, plan, softmax_scale, causal, blk_start, stream);
  if (hipFreeAsync(blk_start, stream) != hipSuccess) rc = FA_ERR_HIP;
  return rc;
}

int fa_varlen_fwd_noalloc(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* cu_seqlens_q,
                          const fa_tensor* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          float softmax_scale, int32_t causal, fa_tensor* out, fa_tensor* lse, hipStream_t stream) {
  Problem p;
  int st = check_problem(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, max_seqlen_q, max_seqlen_k, softmax_scale,
                         causal, fwd_head_dim, nullptr, 0, 0, &p);
  if (st != FA_OK) return st;
  if (p.batch > fa::kNoAllocMaxBatch) return FA_ERR_SCRATCH;
  Plan plan;
  st = plan_fwd(p, max_seqlen_q, true, &plan);
  if (st != FA_OK) return st;
  if (plan.grid == 0) return FA_OK;
  // The map goes to this device's static array (written whole by the map
  // kernel before the attention kernel reads it, both on `stream`).
  int32_t* blk_start = nullptr;
  if (fa::noalloc_map_scratch(&blk_start) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_tile_map(p.cu_q, p.batch, plan.tc.block_m, blk_start, stream) != hipSuccess) return FA_ERR_HIP;
  return launch_fwd_mapped(p, plan, softmax_scale, causal, blk_start, stream);
}

int fa_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t num_heads, int32_t head_dim,
                                 size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  if (batch < 0 || total_q < 0 || num_heads < 1 || head_dim < 1) return FA_ERR_SHAPE;
  *bytes = bwd_layout(batch, total_q, num_heads, head_dim).total;
  return FA_OK;
}

int fa_varlen_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                  const fa_tensor* dout, const fa_tensor* lse, const fa_tensor* cu_seqlens_q,
                  const fa_tensor* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                  int32_t causal, fa_tensor* dq, fa_tensor* dk, fa_tensor* dv, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  // dout and dq are shaped like q, dk and dv like k
  const fa_tensor* extra[4] = {dout, dq, dk, dv};
  Problem p;
  int st = check_problem(q, k, v, cu_seqlens_q, cu_seqlens_k, out, lse, max_seqlen_q, max_seqlen_k, softmax_scale,
                         causal, fwd_head_dim, extra, 4, 2, &p);
  if (st != FA_OK) return st;
  const int bn = fa::bwd_block_n(p.elem, p.head_dim);
  if (bn == 0) return FA_ERR_HEAD_DIM;
  const BwdLayout lay = bwd_layout(p.batch, p.total_q, p.heads, p.head_dim);
  if (!workspace || workspace_bytes < lay.total) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  // key blocks: sum_b ceil(Lk_b / bn) <= min(batch * ceil(max_k / bn), ceil(total_k / bn) + batch - 1)
  const int64_t by_max = (int64_t)p.batch * ((max_seqlen_k + bn - 1) / bn);
  const int64_t by_total = ((int64_t)p.total_k + bn - 1) / bn + (p.batch > 0 ? p.batch - 1 : 0);
  const int64_t compact = by_max < by_total ? by_max : by_total;
  // Under a causal mask a sequence's first key blocks carry the most work.
  // Block-major slots (block j of every sequence, then block j + 1) dispatch
  // them first; slots of sequences shorter than j stay empty, so this order
  // is used only while the grid has at most 25% more slots than the compact
  // key-block map (4 * by_max <= 5 * compact).
  const bool by_block = causal != 0 && 4 * by_max <= 5 * compact;
  const int64_t tmax = by_block ? by_max : compact;
  const int64_t grid = (tmax * p.heads_k + 7) / 8 * 8;
  if (grid > INT32_MAX) return FA_ERR_TOO_LARGE;

  char* ws = static_cast<char*>(workspace);
  int32_t* blk = reinterpret_cast<int32_t*>(ws + lay.blk);
  fa::BwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.dout = dout->data;
  a.lse = p.lse;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.blk_start = blk;
  a.dq = dq->data;
  a.dk = dk->data;
  a.dv = dv->data;
  a.dq_acc = reinterpret_cast<float*>(ws + lay.dq_acc);
  a.drow = reinterpret_cast<float*>(ws + lay.drow);
  a.row_stride = (int64_t)p.heads * p.head_dim;
  a.kv_row_stride = (int64_t)p.heads_k * p.head_dim;
  a.scale = softmax_scale;
  a.scale_log2 = (float)((double)softmax_scale * kLog2e);
  a.batch = p.batch;
  a.tmax = (int32_t)tmax;
  a.by_block = by_block ? 1 : 0;
  a.n_work = (int32_t)(tmax * p.heads_k);
  a.total_q = p.total_q;
  a.heads = p.heads;
  a.head_group = p.heads / p.heads_k;

  if (fa::launch_bwd_prep(p.elem, p.head_dim, a, stream) != hipSuccess) return FA_ERR_HIP;
  if (grid > 0) {
    if (!by_block && fa::launch_tile_map(p.cu_k, p.batch, bn, blk, stream) != hipSuccess) return FA_ERR_HIP;
    if (fa::launch_bwd(p.elem, p.head_dim, causal != 0, (int)grid, a, stream) != hipSuccess) return FA_ERR_HIP;
  }
  if (fa::launch_bwd_dq(p.elem, p.head_dim, a, stream) != hipSuccess) return FA_ERR_HIP;
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

int fa_varlen_fwd_kvcache(const fa_tensor* q, const fa_tensor* k_cache, const fa_tensor* v_cache,
                          const fa_tensor* cu_seqlens_q, const fa_tensor* seqlens_k, const fa_tensor* leftpad_k,
                          const fa_tensor* block_table, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          float softmax_scale, int32_t causal, int32_t cache_rows, int32_t num_splits,
                          fa_tensor* out, fa_tensor* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !seqlens_k || !out || !lse) return FA_ERR_NULL;
  // element types
  const int elem = elem_code(q->dtype);
  if (elem < 0) return FA_ERR_DTYPE;
  if (k_cache->dtype != q->dtype || v_cache->dtype != q->dtype || out->dtype != q->dtype) return FA_ERR_DTYPE;
  if (lse->dtype != FA_DTYPE_F32 || cu_seqlens_q->dtype != FA_DTYPE_I32 || seqlens_k->dtype != FA_DTYPE_I32)
    return FA_ERR_DTYPE;
  if ((leftpad_k && leftpad_k->dtype != FA_DTYPE_I32) || (block_table && block_table->dtype != FA_DTYPE_I32))
    return FA_ERR_DTYPE;
  // shapes
  if (!rank_ok(*q, 3) || !rank_ok(*k_cache, 3) || !rank_ok(*out, 3) || !rank_ok(*lse, 2) ||
      !rank_ok(*cu_seqlens_q, 1) || !rank_ok(*seqlens_k, 1))
    return FA_ERR_SHAPE;
  const int64_t D = q->shape[2];
  if (D != 64 && D != 96 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  const int64_t Tq = q->shape[0], H = q->shape[1], Hk = k_cache->shape[1];
  const int64_t batch = cu_seqlens_q->shape[0] - 1;
  if (batch < 0 || H < 1 || Hk < 1 || H % Hk != 0 || k_cache->shape[2] != D || !same_shape(*k_cache, *v_cache) ||
      !same_shape(*q, *out) || lse->shape[0] != H || lse->shape[1] != Tq || seqlens_k->shape[0] != batch)
    return FA_ERR_SHAPE;
  if (leftpad_k && (!rank_ok(*leftpad_k, 1) || leftpad_k->shape[0] != batch)) return FA_ERR_SHAPE;
  if (cache_rows < 1 || k_cache->shape[0] % cache_rows != 0) return FA_ERR_SHAPE;
  const int64_t cache_blocks = k_cache->shape[0] / cache_rows;
  int64_t blocks_per_seq = 0;
  if (block_table) {
    if (!rank_ok(*block_table, 2) || block_table->shape[0] != batch || block_table->shape[1] < 1)
      return FA_ERR_SHAPE;
    blocks_per_seq = block_table->shape[1];
    if ((int64_t)max_seqlen_k > blocks_per_seq * cache_rows) return FA_ERR_SHAPE;
  } else {
    if (cache_blocks < batch || max_seqlen_k > cache_rows) return FA_ERR_SHAPE;
  }
  if (max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > Tq) return FA_ERR_SHAPE;
  // layout, data
  if (!contiguous(*q) || !contiguous(*k_cache) || !contiguous(*v_cache) || !contiguous(*out) ||
      !contiguous(*lse) || !contiguous(*cu_seqlens_q) || !contiguous(*seqlens_k) ||
      (leftpad_k && !contiguous(*leftpad_k)) || (block_table && !contiguous(*block_table)))
    return FA_ERR_LAYOUT;
  if (!data_ok(*q) || !data_ok(*k_cache) || !data_ok(*v_cache) || !data_ok(*out) || !data_ok(*lse) ||
      !cu_seqlens_q->data || !data_ok(*seqlens_k) || (leftpad_k && !data_ok(*leftpad_k)) ||
      (block_table && !data_ok(*block_table)))
    return FA_ERR_NULL;
  // scalars
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  if (num_splits < 0 || num_splits > kMaxSplits) return FA_ERR_ARG;
  // alignment
  if (!aligned(q->data, 16) || !aligned(k_cache->data, 16) || !aligned(v_cache->data, 16) ||
      !aligned(out->data, 16))
    return FA_ERR_ALIGN;
  if (!aligned(lse->data, 4) || !aligned(cu_seqlens_q->data, 4) || !aligned(seqlens_k->data, 4) ||
      (leftpad_k && !aligned(leftpad_k->data, 4)) || (block_table && !aligned(block_table->data, 4)))
    return FA_ERR_ALIGN;
  // sizes
  if (Tq > INT32_MAX || H * D > (int64_t{1} << 22) || Hk * D > (int64_t{1} << 22) || cache_blocks > INT32_MAX ||
      blocks_per_seq > INT32_MAX || batch > INT32_MAX)
    return FA_ERR_TOO_LARGE;
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(batch, Hk, max_seqlen_k);
  if (batch * Hk * splits > INT32_MAX) return FA_ERR_TOO_LARGE;
  if (!workspace || workspace_bytes < dec_workspace(Tq, H, D, splits)) return FA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return FA_ERR_ALIGN;
  if (batch == 0 || Tq == 0) return FA_OK;  // no query rows

  const int64_t rows = Tq * H * splits;
  fa::DecArgs a;
  a.q = q->data;
  a.k_cache = k_cache->data;
  a.v_cache = v_cache->data;
  a.out = out->data;
  a.lse = static_cast<float*>(lse->data);
  a.cu_q = static_cast<const int32_t*>(cu_seqlens_q->data);
  a.seqlens_k = static_cast<const int32_t*>(seqlens_k->data);
  a.leftpad_k = leftpad_k ? static_cast<const int32_t*>(leftpad_k->data) : nullptr;
  a.block_table = block_table ? static_cast<const int32_t*>(block_table->data) : nullptr;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)rows * D * 4));
  a.row_stride = H * D;
  a.kv_row_stride = Hk * D;
  a.scale_log2 = (float)((double)softmax_scale * kLog2e);
  a.batch = (int32_t)batch;
  a.total_q = (int32_t)Tq;
  a.heads = (int32_t)H;
  a.kv_heads = (int32_t)Hk;
  a.head_group = (int32_t)(H / Hk);
  a.cache_rows = cache_rows;
  a.blocks_per_seq = (int32_t)blocks_per_seq;
  a.num_splits = splits;
  if (fa::launch_decode(elem, (int)D, causal != 0, a, stream) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_varlen_check_cu_seqlens(const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k, int32_t total_q,
                               int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, fa_tensor* flags,
                               hipStream_t stream) {
  if (!cu_seqlens_q || !cu_seqlens_k || !flags) return FA_ERR_NULL;
  if (cu_seqlens_q->dtype != FA_DTYPE_I32) return FA_ERR_DTYPE;
  if (!rank_ok(*cu_seqlens_q, 1) || cu_seqlens_q->shape[0] < 1) return FA_ERR_SHAPE;
  const int64_t n = cu_seqlens_q->shape[0];
  if (total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return FA_ERR_SHAPE;
  int st = check_i32_vector(cu_seqlens_q, n);
  if (st == FA_OK) st = check_i32_vector(cu_seqlens_k, n);
  if (st == FA_OK) st = check_i32_vector(flags, 1);
  if (st != FA_OK) return st;
  if (n - 1 > INT32_MAX) return FA_ERR_TOO_LARGE;
  if (fa::launch_check_cu(static_cast<const int32_t*>(cu_seqlens_q->data),
                          static_cast<const int32_t*>(cu_seqlens_k->data), (int)(n - 1), total_q, total_k,
                          max_seqlen_q, max_seqlen_k, static_cast<int32_t*>(flags->data), stream) != hipSuccess)
    return FA_ERR_HIP;
  return FA_OK;
}

}  // extern "C"
