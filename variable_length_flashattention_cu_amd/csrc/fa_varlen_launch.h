// fa_varlen_launch.h -- internal interface between the C ABI (fa_varlen_api.cpp)
// and the kernels (fa_varlen_kernels.hip, fa_varlen_bwd.hip).  Not installed;
// callers use include/fa_varlen.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Element codes of the `dtype` arguments below (the C ABI maps its fa_dtype
// values onto these).
constexpr int kElemF32 = 0;
constexpr int kElemBF16 = 1;
constexpr int kElemF16 = 2;

// Kernel arguments of the forward pass (passed by value).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* blk_start;  // the work-item map, or null: rebuilt per wavefront (batch <= kMaplessBatch)
  int64_t row_stride;     // elements between consecutive tokens of q/out: heads * head_dim
  int64_t kv_row_stride;  // elements between consecutive tokens of k/v: kv_heads * head_dim
  float scale_log2;    // softmax_scale * log2(e)
  int32_t batch;
  int32_t tmax;        // upper bound on work items per head
  int32_t n_work;      // heads * tmax
  int32_t total_q;     // row count of q / columns of lse
  int32_t pair_blocks; // causal: one workgroup takes query blocks m and M-1-m
  int32_t head_group;  // query heads per key/value head (heads / kv_heads)
};

struct TileConfig {
  int block_m;  // query rows per work item
  int block_n;  // keys per streamed K/V tile
  int threads;  // workgroup size
};

// {0,0,0} for an unsupported (dtype, head_dim).
TileConfig tile_config(int dtype, int head_dim);
// Short sequences (16-bit inputs, head_dim 64 or 128): 128-row work items of
// four wavefronts on 64-key (head_dim 64) or 32-key (head_dim 128) tiles, 64 KB
// of LDS, so two workgroups share a compute unit.  Only the entry points that
// build their own map use it; {0,0,0} where there is none.
TileConfig tile_config_short(int dtype, int head_dim);

// Kernel arguments of the backward pass (passed by value).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;        // [heads, total_q], natural log
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* blk_start;  // key-block map: scan of ceil(Lk_b / block_n)
  void* dq;
  void* dk;
  void* dv;
  float* dq_acc;           // [total_q, heads, head_dim] float32 accumulator
  float* drow;             // [heads, total_q]: rowsum(dout * out)
  int64_t row_stride;      // heads * head_dim
  int64_t kv_row_stride;   // kv_heads * head_dim
  float scale;             // softmax_scale
  float scale_log2;        // softmax_scale * log2(e)
  int32_t batch;
  int32_t tmax;            // work slots per key/value head (see by_block below)
  int32_t n_work;          // kv_heads * tmax
  int32_t by_block;        // 1: slot t is key block t / batch of sequence t % batch (empty if
                           // the sequence is shorter), so every sequence's first blocks come
                           // first; 0: slot t is the t-th entry of the key-block map
  int32_t total_q;
  int32_t heads;
  int32_t head_group;      // query heads per key/value head
};

// Keys per work item of the backward pass for (dtype, head_dim); 0 if the
// backward pass does not support the pair.
int bwd_block_n(int dtype, int head_dim);

// rowsum(dout * out) per (head, row) and a zeroed dq accumulator
hipError_t launch_bwd_prep(int dtype, int head_dim, const BwdArgs& a, hipStream_t stream);
// dk, dv and the dq accumulator, one workgroup per (key block, key/value head)
hipError_t launch_bwd(int dtype, int head_dim, bool causal, int grid, const BwdArgs& a, hipStream_t stream);
// dq = softmax_scale * accumulator, in the input type
hipError_t launch_bwd_dq(int dtype, int head_dim, const BwdArgs& a, hipStream_t stream);

// Kernel arguments of attention against a key/value cache (passed by value).
struct DecArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  void* out;
  float* lse;
  const int32_t* cu_q;
  const int32_t* seqlens_k;    // [batch], not cumulative
  const int32_t* leftpad_k;    // [batch] or null
  const int32_t* block_table;  // [batch, blocks_per_seq] or null (one slot per sequence)
  float* part_o;               // [total_q, heads, num_splits * waves, head_dim] partial outputs
  float* part_ml;              // [total_q, heads, num_splits * waves, 2] partial max (log2) and sum
  int64_t row_stride;          // heads * head_dim
  int64_t kv_row_stride;       // kv_heads * head_dim (elements between cache rows)
  float scale_log2;
  int32_t batch;
  int32_t total_q;
  int32_t heads;
  int32_t kv_heads;
  int32_t head_group;
  int32_t cache_rows;          // rows per slot or per block
  int32_t blocks_per_seq;
  int32_t num_splits;
};

hipError_t launch_decode(int dtype, int head_dim, bool causal, const DecArgs& a, hipStream_t stream);

// fa_varlen_fwd_noalloc: the largest batch its static work-item map holds,
// and that map's device address on the current device (fa_varlen_scratch.hip).
constexpr int kNoAllocMaxBatch = 65535;
// Batches of at most this many sequences need no map: the forward kernels
// rebuild it per wavefront from cu_seqlens_q (one lane per sequence).
constexpr int kMaplessBatch = 64;
hipError_t noalloc_map_scratch(int32_t** ptr);

hipError_t launch_tile_map(const int32_t* cu_q, int batch, int block_m, int32_t* blk_start, hipStream_t stream);
hipError_t launch_fwd(int dtype, int head_dim, bool causal, bool short_items, int grid, const FwdArgs& a,
                      hipStream_t stream);
hipError_t launch_check_cu(const int32_t* cu_q, const int32_t* cu_k, int batch, int total_q, int total_k,
                           int max_q, int max_k, int32_t* flags, hipStream_t stream);

}  // namespace fa
