// fa_varlen_launch.h -- internal interface between the C ABI (fa_varlen_api.cpp)
// and the kernels (fa_varlen_kernels.hip).  Not installed; callers use
// include/fa_varlen.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Kernel arguments of the forward pass (passed by value).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* blk_start;
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

hipError_t launch_tile_map(const int32_t* cu_q, int batch, int block_m, int32_t* blk_start, hipStream_t stream);
hipError_t launch_fwd(int dtype, int head_dim, bool causal, int grid, const FwdArgs& a, hipStream_t stream);
hipError_t launch_check_cu(const int32_t* cu_q, const int32_t* cu_k, int batch, int total_q, int total_k,
                           int max_q, int max_k, int32_t* flags, hipStream_t stream);

}  // namespace fa
