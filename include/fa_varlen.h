/*
 * fa_varlen.h -- C ABI of libfa_varlen.so: exact attention over packed
 * variable-length sequences on AMD Instinct MI355X (gfx950), forward pass,
 * backward pass and attention against a key/value cache.
 *
 * The operation (FlashAttention pages):
 *   * Sequences are packed back to back with no padding and addressed by
 *     cumulative offsets of length batch+1; offsets [0,128,300] mean two
 *     sequences of 128 and 172 tokens (friki.work, "Mecanismo cu_seqlens en
 *     FlashAttention", sections "Estructuras de datos clave" and "Lógica de
 *     cálculo de longitud").  A sequence's first row is its offset times the
 *     row stride (same page, "Optimización de acceso a memoria").
 *   * For every sequence b and head h the result is the exact attention
 *     softmax(scale * Q K^T, optional causal mask) V; the tiled method never
 *     writes the score matrix to HBM and keeps a running (online) softmax
 *     whose statistics and partial outputs are rescaled block by block
 *     (iplexlaw.co.kr, "FlashAttention-2 GPU work partitioning", section
 *     "Bloques pequeños, normalización global"; slavadubrov.com, "O que
 *     FlashAttention muda na inferência", section "Separar o armazenamento
 *     do cálculo").
 *   * Work is split over (sequence, head, query block) so that long sequences
 *     in small batches still fill the GPU (iplexlaw.co.kr, section "Tres
 *     mejoras en la utilización de la GPU").
 *   * Causal masking may be combined with variable lengths (friki.work,
 *     section "Integración con máscaras causales y caché paginada").
 *   * Several query heads may share one key/value head (multi-query and
 *     grouped-query attention, zepes.com "Comprendiendo Flash-Atención y
 *     Flash-Atención-2", section "FlashAttention-2"); mixed precision
 *     (FP16/BF16) is the recommended input type (friki.work, section
 *     "Consejos de optimización").
 *   * The call takes whole tensors -- q, k, v and the two offset arrays, as
 *     in the page's PyTorch call (friki.work, section "Ejemplo de uso con
 *     PyTorch") -- and the kernels read the offsets through a parameter block
 *     that holds pointers to the two cumulative arrays (same page, section
 *     "Estructuras de datos clave").  Here a tensor is an fa_tensor
 *     descriptor: data pointer, element type, shape and element strides.
 *
 * Readings the pages leave open, fixed here:
 *   * causal alignment is bottom-right: query i of a sequence (0-based) sees
 *     key j iff j <= i + Lk - Lq;
 *   * a query row that sees no key gets out = 0 and lse = -inf;
 *   * lse is the natural log of sum_j exp(scale * q_i . k_j) over visible j;
 *   * with Hk key/value heads and H query heads, query head h attends with
 *     key/value head h / (H / Hk) (contiguous groups).
 *
 * Conventions shared by every entry point
 *   * Tensors are fa_tensor descriptors.  Device data lives on the current
 *     HIP device (hipSetDevice before the call).  Attention tensors must be
 *     contiguous in row-major order: stride[ndim-1] = 1 and stride[i] =
 *     stride[i+1] * shape[i+1] (the stride of a dimension of extent 1 is not
 *     looked at); any other layout gives FA_ERR_LAYOUT.  `data` may be NULL
 *     only for a tensor with no elements.
 *   * The caller owns every buffer; the library keeps no pointer after a
 *     call returns.
 *   * `stream` is a hipStream_t (NULL = the null stream).  All device work
 *     is enqueued on it; calls return before it runs.
 *   * Every function returns an fa_status.  On a validation error nothing is
 *     launched and no buffer is touched.  Faults raised by device work
 *     surface at the caller's next synchronisation on the stream.
 *   * cu_seqlens contents are a precondition, not checked on the device:
 *     cu[0] == 0, non-decreasing, cu[batch] <= total rows, and every length
 *     at most the max_seqlen passed.  fa_varlen_check_cu_seqlens validates
 *     them on the device for callers that want a check.
 *
 * Status codes are checked in this order: NULL descriptor, element type,
 * rank and shape (head_dim separately), layout, NULL data, scalar
 * arguments, alignment, size limits, workspace (or static scratch).
 */
#ifndef FA_VARLEN_H_
#define FA_VARLEN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle type (an opaque pointer); the same declaration as in
 * hip/hip_runtime_api.h, so both headers may be included together. */
typedef struct ihipStream_t* hipStream_t;

/* Element types. */
typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,   /* IEEE float32; attention arithmetic in float32 throughout */
  FA_DTYPE_BF16 = 1,  /* bfloat16 in and out; float32 accumulation */
  FA_DTYPE_I32 = 2,   /* int32: offsets, lengths, block tables, flags */
  FA_DTYPE_F16 = 3    /* IEEE float16 in and out; float32 accumulation */
} fa_dtype;

/* A tensor: `ndim` (1..3) dimensions of `shape`, `stride` in elements. */
typedef struct fa_tensor {
  void* data;
  int32_t dtype;       /* an fa_dtype */
  int32_t ndim;
  int64_t shape[3];
  int64_t stride[3];
} fa_tensor;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a required descriptor is NULL, or a non-empty tensor has NULL data */
  FA_ERR_DTYPE = 2,      /* element type not supported for this tensor or entry point */
  FA_ERR_SHAPE = 3,      /* wrong rank, negative or inconsistent sizes, key/value heads not
                            dividing the query heads, max_seqlen above the row count */
  FA_ERR_HEAD_DIM = 4,   /* head_dim not supported for this dtype and entry point */
  FA_ERR_LAYOUT = 5,     /* a tensor is not contiguous in row-major order */
  FA_ERR_ALIGN = 6,      /* data not aligned as documented */
  FA_ERR_ARG = 7,        /* softmax_scale not finite and > 0, causal not 0/1, num_splits out of range */
  FA_ERR_HIP = 8,        /* the HIP runtime reported an error (no device, launch failure) */
  FA_ERR_TOO_LARGE = 9,  /* sizes beyond what one launch addresses (grid above 2^31-1
                            workgroups, rows above 2^31-1, heads * head_dim above 2^22) */
  FA_ERR_WORKSPACE = 10, /* workspace NULL or smaller than the size function reports */
  FA_ERR_SCRATCH = 11    /* fa_varlen_fwd_noalloc: batch above its static map (65535 sequences) */
} fa_status;

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(int status);

/*
 * Query-block height BM and key-block height BN used by the forward pass
 * for a (head_dim, dtype) pair.  BM is the block height of the work-item map
 * (fa_varlen_tile_map): every work item covers at most BM query rows of one
 * sequence.  Host only; launches nothing.
 * Errors: FA_ERR_NULL (block_m or block_n NULL), FA_ERR_DTYPE (dtype not
 * F32/BF16/F16), FA_ERR_HEAD_DIM.
 */
int fa_varlen_block_sizes(int32_t head_dim, int32_t dtype, int32_t* block_m, int32_t* block_n);

/*
 * Work-item map of the ragged batch (the sequence-dimension split described
 * in iplexlaw.co.kr, "FlashAttention-2 GPU work partitioning", section "Tres
 * mejoras en la utilización de la GPU"; lengths per friki.work, section
 * "Lógica de cálculo de longitud"), with BM = the block height that
 * fa_varlen_block_sizes reports for (head_dim, dtype):
 *   blk_start[0] = 0,
 *   blk_start[b+1] = blk_start[b] + ceil((cu_seqlens_q[b+1] - cu_seqlens_q[b]) / BM).
 * Work item t belongs to the sequence b with blk_start[b] <= t < blk_start[b+1]
 * and covers its query rows (t - blk_start[b]) * BM ... + BM - 1, clipped to
 * the sequence, so no item straddles two sequences.
 *
 *   cu_seqlens_q   device int32 [batch + 1], batch >= 0
 *   max_seqlen_q   >= every query length (>= 0); sizes nothing here, checked
 *                  for sign only
 *   head_dim, dtype  select BM as above
 *   blk_start_out  device int32 [batch + 1], written
 * A negative length (precondition violation) counts as 0 blocks.
 * Alignment: 4 bytes for both arrays.
 */
int fa_varlen_tile_map(const fa_tensor* cu_seqlens_q, int32_t max_seqlen_q, int32_t head_dim, int32_t dtype,
                       fa_tensor* blk_start_out, hipStream_t stream);

/*
 * Exact attention forward over packed variable-length sequences.
 *
 *   q             [total_q, H, D], dtype BF16, F16 or F32
 *   k, v          [total_k, Hk, D], q's dtype; Hk >= 1 divides H (Hk == H is
 *                 multi-head attention, Hk == 1 multi-query attention)
 *   cu_seqlens_q  int32 [batch + 1] query offsets (batch >= 0)
 *   cu_seqlens_k  int32 [batch + 1] key/value offsets
 *   max_seqlen_q  >= every query length (sizes the launch; 0..total_q)
 *   max_seqlen_k  >= every key length (0..total_k)
 *   softmax_scale finite, > 0; multiplies q.k before the softmax
 *   causal        0 or 1 (bottom-right alignment, see above)
 *   out           [total_q, H, D], q's dtype; written for rows <
 *                 cu_seqlens_q[batch], other rows untouched
 *   lse           float32 [H, total_q], natural-log log-sum-exp per (head,
 *                 query row); same rows as out
 *
 * 16-bit inputs are multiplied on the matrix cores with float32
 * accumulation, the probabilities are rounded to the input type before the
 * second product and the output is rounded to nearest even; float32 inputs
 * use float32 arithmetic throughout.
 * D must be 64, 96 or 128, or 256 with BF16/F16 inputs (FA_ERR_HEAD_DIM).
 * Alignment: q, k, v and out data 16 bytes; lse and the offsets 4 bytes (the
 * offsets are best kept 32-byte aligned, as any hipMalloc'd buffer is).
 * Work items: with BF16/F16 inputs at D 64 or 128 and max_seqlen_q <= 1024
 * the pass takes 128-row work items (four wavefronts; two workgroups share a
 * compute unit) instead of the BM of fa_varlen_block_sizes; each query row
 * goes through the same steps either way, but which key slabs take the
 * full softmax (with row maxima) may differ, so its results can differ from
 * fa_varlen_fwd_mapped's in the last bits.
 * Scratch: up to 64 sequences none (the attention kernel rebuilds the
 * work-item map per wavefront from cu_seqlens_q and is the only launch);
 * above that a (batch+1)-entry int32 map is allocated and freed
 * stream-ordered (hipMallocAsync / hipFreeAsync) on `stream`.
 * Reentrant: concurrent calls on different streams do not interfere.
 */
int fa_varlen_fwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                  const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k,
                  int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                  fa_tensor* out, fa_tensor* lse, hipStream_t stream);

/*
 * The same forward pass with a work-item map the caller already built with
 * fa_varlen_tile_map for this head_dim and dtype, e.g. once per batch and
 * reused by every layer.  Launches only the attention kernel and allocates
 * nothing.  It always uses the BM of fa_varlen_block_sizes.
 *   blk_start     device int32 [batch + 1], 4-byte aligned, read only
 * Other arguments and errors as fa_varlen_fwd.  A map built for another
 * (head_dim, dtype) block height is a precondition violation (rows are then
 * skipped or repeated).
 */
int fa_varlen_fwd_mapped(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                         const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                         fa_tensor* out, fa_tensor* lse, const fa_tensor* blk_start, hipStream_t stream);

/*
 * The forward pass for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It computes exactly what fa_varlen_fwd computes (same kernels, same
 * results) but calls no hipMalloc, hipMallocAsync, hipFree or other
 * allocating routine: the (batch+1)-entry work-item map goes to a static
 * device array of 65536 int32 (256 KiB) that the library holds on every GPU
 * it runs on until the process ends.  The map kernel writes all batch+1
 * entries before the attention kernel reads them, so nothing needs clearing
 * between calls.
 *   Arguments and errors as fa_varlen_fwd, plus FA_ERR_SCRATCH when batch
 *   exceeds 65535.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (different streams, or different host threads, without ordering
 * between them) race on the map and may compute wrong rows.  Calls ordered on
 * one stream do not.
 */
int fa_varlen_fwd_noalloc(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v,
                          const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k,
                          int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                          fa_tensor* out, fa_tensor* lse, hipStream_t stream);

/*
 * Backward pass: gradients of the attention of fa_varlen_fwd with respect to
 * q, k and v, given the gradient dout of its output.
 *
 * What is computed (the derivative of the forward definition): per sequence
 * and query head, with P the attention probabilities,
 *   dv = P^T dout,  dP = dout v^T,  dS = P * (dP - rowsum(dout * out)),
 *   dq = softmax_scale * dS k,  dk = softmax_scale * dS^T q;
 * a key/value head shared by several query heads receives the sum of their
 * dk and dv.  How the pass is organised follows the pages (zepes.com,
 * "Comprendiendo Flash-Atención y Flash-Atención-2", section "FashAttention
 * v1" (sic)): workers own blocks of key columns, recompute P from the forward
 * pass's lse instead of storing it, and add their parts of dq with atomic
 * operations.
 *
 *   q, k, v, cu_seqlens_*, max_seqlen_*, softmax_scale, causal
 *                 exactly as passed to fa_varlen_fwd
 *   out, lse      the outputs of that fa_varlen_fwd call
 *   dout          [total_q, H, D], q's dtype
 *   dq            [total_q, H, D], q's dtype; written for rows <
 *                 cu_seqlens_q[batch] (rows that see no key get 0)
 *   dk, dv        [total_k, Hk, D], q's dtype; written for rows <
 *                 cu_seqlens_k[batch] (keys no query sees get 0)
 *   workspace     device scratch of at least workspace_bytes >=
 *                 fa_varlen_bwd_workspace_size(...) bytes, 16-byte aligned,
 *                 owned by the caller; its contents on entry do not matter
 *                 and are undefined afterwards.  Calls that run at the same
 *                 time need separate workspaces.
 * dtype and D as fa_varlen_fwd: BF16 or F16 with D 64, 96, 128 or 256, F32
 * with D 64, 96 or 128 (FA_ERR_DTYPE / FA_ERR_HEAD_DIM otherwise).  16-bit
 * products use the 16-bit MFMA with float32 accumulation, P and dS rounded
 * to dtype before they enter a product; F32 uses the float32 MFMA
 * throughout; dq is summed in float32.  Because dq is accumulated with atomic additions,
 * its low bits may differ from run to run.  Other checks as fa_varlen_fwd;
 * dout, dq, dk and dv need 16-byte alignment.  A workspace that is NULL or
 * too small gives FA_ERR_WORKSPACE.
 */
int fa_varlen_bwd(const fa_tensor* q, const fa_tensor* k, const fa_tensor* v, const fa_tensor* out,
                  const fa_tensor* dout, const fa_tensor* lse, const fa_tensor* cu_seqlens_q,
                  const fa_tensor* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                  int32_t causal, fa_tensor* dq, fa_tensor* dk, fa_tensor* dv, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of workspace fa_varlen_bwd needs for these sizes: a float32 dq
 * accumulator [total_q, num_heads, head_dim], the float32 row terms
 * rowsum(dout * out) [num_heads, total_q] and the key-block map
 * [batch + 1], each rounded up to 256 bytes.  Host only.
 * Errors: FA_ERR_NULL (bytes NULL), FA_ERR_SHAPE (negative sizes, no heads).
 */
int fa_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t num_heads, int32_t head_dim,
                                 size_t* bytes);

/*
 * Attention of packed queries against a key/value cache (the decode-shaped
 * case: few query rows per sequence, long cached key ranges).
 *
 * The operation is the forward pass above with each sequence's keys and
 * values taken from a cache (friki.work, "Mecanismo cu_seqlens en
 * FlashAttention", sections "Lógica de cálculo de longitud" and
 * "Optimización de acceso a memoria": per-sequence key lengths that are not
 * cumulative, a batch-strided cache slot, a left padding subtracted from the
 * length; section "Integración con máscaras causales y caché paginada": a
 * paged cache).  Readings fixed here: sequence b's keys are cache positions
 * leftpad_k[b] .. seqlens_k[b]-1 (key length seqlens_k[b] - leftpad_k[b]);
 * without a block table position p of sequence b is row p of cache block b;
 * with one it is row p % cache_rows of block block_table[b][p / cache_rows];
 * the causal mask is bottom-right as above, so one new query token sees
 * every cached key.
 *
 *   q, out        [total_q, H, D] packed by cu_seqlens_q (out written for
 *                 rows < cu_seqlens_q[batch]), BF16, F16 or F32
 *   k_cache, v_cache  [cache_blocks * cache_rows, Hk, D], q's dtype: cache
 *                 blocks of cache_rows token rows each, stored back to back
 *                 (a [cache_blocks, cache_rows, Hk, D] tensor viewed with its
 *                 first two dimensions merged)
 *   cu_seqlens_q  int32 [batch + 1], cumulative
 *   seqlens_k     int32 [batch], NOT cumulative
 *   leftpad_k     int32 [batch], or NULL (no left padding)
 *   block_table   int32 [batch, blocks_per_seq], or NULL (then cache_blocks
 *                 >= batch and block b is sequence b's slot)
 *   max_seqlen_q  >= every query length; max_seqlen_k >= every seqlens_k[b]
 *                 and at most the positions a sequence can hold (cache_rows,
 *                 or blocks_per_seq * cache_rows with a block table)
 *   cache_rows    token rows per cache block (>= 1)
 *   num_splits    0 (chosen from the sizes) or 1..64 workgroups per
 *                 (sequence, key/value head), each over a contiguous key range
 *   lse           float32 [H, total_q] as fa_varlen_fwd
 *   workspace     device scratch of >= fa_varlen_kvcache_workspace_size
 *                 bytes for this num_splits, 16-byte aligned, caller-owned
 * Preconditions (not checked on the device): 0 <= leftpad_k[b] <=
 * seqlens_k[b] <= max_seqlen_k and block table entries < cache_blocks.
 * D must be 64, 96, 128 or 256 for every dtype (FA_ERR_HEAD_DIM); other
 * checks and errors as
 * fa_varlen_fwd, plus FA_ERR_WORKSPACE and FA_ERR_ARG for num_splits out of
 * range.
 */
int fa_varlen_fwd_kvcache(const fa_tensor* q, const fa_tensor* k_cache, const fa_tensor* v_cache,
                          const fa_tensor* cu_seqlens_q, const fa_tensor* seqlens_k, const fa_tensor* leftpad_k,
                          const fa_tensor* block_table, int32_t max_seqlen_q, int32_t max_seqlen_k,
                          float softmax_scale, int32_t causal, int32_t cache_rows, int32_t num_splits,
                          fa_tensor* out, fa_tensor* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/*
 * Workspace bytes of fa_varlen_fwd_kvcache: float32 partial outputs and
 * (max, sum) pairs for every (query row, head, split); num_splits
 * 0 sizes for the largest automatic choice (64).  Host only.
 * Errors: FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_ARG (num_splits outside 0..64).
 */
int fa_varlen_kvcache_workspace_size(int32_t total_q, int32_t num_heads, int32_t head_dim, int32_t num_splits,
                                     size_t* bytes);

/*
 * Device-side check of the cu_seqlens preconditions (friki.work, section
 * "Estructuras de datos clave": batch+1 cumulative offsets).  Writes to
 * `flags` (int32 [1]) a bit mask, 0 when valid:
 *   1  cu[0] != 0            2  cu decreases somewhere
 *   4  cu[batch] > total     8  some length exceeds max_seqlen
 * for either array (q bits in 0..3, k bits shifted left by 4).
 *   cu_seqlens_q, cu_seqlens_k  int32 [batch + 1]
 *   total_q, total_k            row counts of q and k (>= 0)
 *   flags                       int32 [1], overwritten
 */
int fa_varlen_check_cu_seqlens(const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_k, int32_t total_q,
                               int32_t total_k, int32_t max_seqlen_q, int32_t max_seqlen_k, fa_tensor* flags,
                               hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_VARLEN_H_ */
