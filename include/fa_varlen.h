/*
 * fa_varlen.h -- C ABI of libfa_varlen.so: exact attention over packed
 * variable-length sequences on AMD Instinct MI355X (gfx950), forward pass
 * and backward pass.
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
 *
 * Readings the pages leave open, fixed here:
 *   * causal alignment is bottom-right: query i of a sequence (0-based) sees
 *     key j iff j <= i + Lk - Lq;
 *   * a query row that sees no key gets out = 0 and lse = -inf;
 *   * lse is the natural log of sum_j exp(scale * q_i . k_j) over visible j;
 *   * with num_heads_k key/value heads, query head h attends with key/value
 *     head h / (num_heads / num_heads_k) (contiguous groups).
 *
 * Conventions shared by every entry point
 *   * Device pointers live on the current HIP device (hipSetDevice before the
 *     call).  The caller owns every buffer; the library keeps no pointer
 *     after a call returns and holds no state across calls.
 *   * `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     All device work is enqueued on it; calls return before it runs.
 *   * Every function returns an fa_status.  On a validation error nothing is
 *     launched and no buffer is touched.  Faults raised by device work
 *     surface at the caller's next synchronisation on the stream.
 *   * cu_seqlens contents are a precondition, not checked on the device:
 *     cu[0] == 0, non-decreasing, cu[batch] <= total rows, and every length
 *     at most the max_seqlen passed.  fa_varlen_check_cu_seqlens validates
 *     them on the device for callers that want a check.
 */
#ifndef FA_VARLEN_H_
#define FA_VARLEN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and out. */
typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,   /* IEEE float32; arithmetic in float32 throughout */
  FA_DTYPE_BF16 = 1,  /* bfloat16 in and out; float32 accumulation */
  FA_DTYPE_F16 = 2    /* IEEE float16 in and out; float32 accumulation */
} fa_dtype;

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a required pointer is NULL */
  FA_ERR_DTYPE = 2,      /* dtype is not an fa_dtype */
  FA_ERR_SHAPE = 3,      /* negative size, zero heads, num_heads_k not dividing
                            num_heads, or max_seqlen > rows */
  FA_ERR_HEAD_DIM = 4,   /* head_dim not supported for this dtype (64, 96, 128; 256 for bf16/fp16) */
  FA_ERR_ALIGN = 5,      /* a pointer is not aligned as documented */
  FA_ERR_ARG = 6,        /* softmax_scale not finite and > 0, causal not 0/1, bad block_m */
  FA_ERR_HIP = 7,        /* the HIP runtime reported an error (no device, launch failure) */
  FA_ERR_TOO_LARGE = 8,  /* the launch grid would exceed 2^31 workgroups */
  FA_ERR_WORKSPACE = 9   /* backward workspace NULL or smaller than fa_varlen_bwd_workspace_size */
} fa_status;

/* Static, NUL-terminated description of a status code (never NULL). */
const char* fa_status_string(int status);

/*
 * Query-block height BM and key-block height BN used by fa_varlen_fwd for a
 * (head_dim, dtype) pair.  BM is the block height of the work-item map
 * (fa_varlen_tile_map): every work item covers at most BM query rows of one
 * sequence.
 * Returns FA_ERR_NULL, FA_ERR_DTYPE or FA_ERR_HEAD_DIM on bad arguments.
 * Host only; launches nothing.
 */
int fa_varlen_block_sizes(int32_t head_dim, int32_t dtype, int32_t* block_m, int32_t* block_n);

/*
 * Work-item map of the ragged batch (the sequence-dimension split described
 * in iplexlaw.co.kr, "FlashAttention-2 GPU work partitioning", section "Tres
 * mejoras en la utilización de la GPU"; lengths per friki.work, section
 * "Lógica de cálculo de longitud"):
 *   blk_start[0] = 0,
 *   blk_start[b+1] = blk_start[b] + ceil((cu_seqlens_q[b+1] - cu_seqlens_q[b]) / block_m).
 * Work item t belongs to the sequence b with blk_start[b] <= t < blk_start[b+1]
 * and covers its query rows (t - blk_start[b]) * block_m ... + block_m - 1,
 * clipped to the sequence, so no item straddles two sequences.
 *
 *   cu_seqlens_q  device, int32 [batch + 1], 4-byte aligned
 *   batch         >= 0
 *   block_m       1 .. 4096
 *   blk_start     device, int32 [batch + 1], written (4-byte aligned)
 * A negative length (precondition violation) counts as 0 blocks.
 */
int fa_varlen_tile_map(const int32_t* cu_seqlens_q, int32_t batch, int32_t block_m,
                       int32_t* blk_start, void* stream);

/*
 * Exact attention forward over packed variable-length sequences.
 *
 *   q             device [total_q, num_heads, head_dim], contiguous, dtype
 *   k, v          device [total_k, num_heads_k, head_dim], contiguous, dtype
 *   cu_seqlens_q  device int32 [batch + 1] query offsets
 *   cu_seqlens_k  device int32 [batch + 1] key/value offsets
 *   max_seqlen_q  >= every query length (sizes the launch; 0..total_q)
 *   max_seqlen_k  >= every key length (0..total_k)
 *   softmax_scale finite, > 0; multiplies q.k before the softmax
 *   causal        0 or 1 (bottom-right alignment, see above)
 *   out           device [total_q, num_heads, head_dim], dtype, written for
 *                 rows < cu_seqlens_q[batch]; other rows untouched
 *   lse           device float32 [num_heads, total_q], natural-log
 *                 log-sum-exp per (head, query row); same rows as out
 *   batch, total_q, total_k, num_heads, num_heads_k, head_dim, dtype
 *                 sizes and type; num_heads_k (>= 1) divides num_heads, query
 *                 head h reads key/value head h / (num_heads / num_heads_k);
 *                 num_heads_k == num_heads is ordinary multi-head attention,
 *                 num_heads_k == 1 multi-query attention
 *   stream        hipStream_t or NULL
 *
 * dtype is FA_DTYPE_BF16, FA_DTYPE_F16 or FA_DTYPE_F32 (FA_ERR_DTYPE
 * otherwise); 16-bit inputs are multiplied on the matrix cores with float32
 * accumulation, the probabilities are rounded to the input type before the
 * second product and the output is rounded to nearest even.
 * head_dim must be 64, 96 or 128, or 256 with bf16 or fp16 inputs
 * (FA_ERR_HEAD_DIM otherwise).  q, k, v and out must be 16-byte aligned,
 * lse and cu_seqlens 4-byte aligned (the offsets
 * are best kept 32-byte aligned, as any hipMalloc'd buffer is).
 * Scratch: a (batch+1)-entry int32 work-item map is allocated and freed
 * stream-ordered (hipMallocAsync / hipFreeAsync) on `stream`.
 * Reentrant: concurrent calls on different streams do not interfere.
 */
int fa_varlen_fwd(const void* q, const void* k, const void* v,
                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int32_t max_seqlen_q, int32_t max_seqlen_k,
                  float softmax_scale, int32_t causal,
                  void* out, float* lse,
                  int32_t batch, int32_t total_q, int32_t total_k,
                  int32_t num_heads, int32_t num_heads_k, int32_t head_dim, int32_t dtype,
                  void* stream);

/*
 * The same forward pass with a work-item map the caller already built with
 * fa_varlen_tile_map (block_m from fa_varlen_block_sizes for this head_dim
 * and dtype), e.g. once per batch and reused by every layer.  Launches only
 * the attention kernel and allocates nothing.
 *   blk_start     device int32 [batch + 1], 4-byte aligned, read only
 * Other arguments and errors as fa_varlen_fwd.  A map built with another
 * block_m is a precondition violation (rows are then skipped or repeated).
 */
int fa_varlen_fwd_mapped(const void* q, const void* k, const void* v,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         int32_t max_seqlen_q, int32_t max_seqlen_k,
                         float softmax_scale, int32_t causal,
                         void* out, float* lse,
                         int32_t batch, int32_t total_q, int32_t total_k,
                         int32_t num_heads, int32_t num_heads_k, int32_t head_dim, int32_t dtype,
                         const int32_t* blk_start, void* stream);

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
 *   q, k, v, cu_seqlens_*, max_seqlen_*, softmax_scale, causal, sizes
 *                 exactly as passed to fa_varlen_fwd
 *   out, lse      the outputs of that fa_varlen_fwd call (out [total_q,
 *                 num_heads, head_dim] dtype, lse float32 [num_heads,
 *                 total_q])
 *   dout          device [total_q, num_heads, head_dim], dtype
 *   dq            device [total_q, num_heads, head_dim], dtype; written for
 *                 rows < cu_seqlens_q[batch] (rows that see no key get 0)
 *   dk, dv        device [total_k, num_heads_k, head_dim], dtype; written
 *                 for rows < cu_seqlens_k[batch] (keys no query sees get 0)
 *   workspace     device scratch of at least workspace_bytes >=
 *                 fa_varlen_bwd_workspace_size(...) bytes, 16-byte aligned,
 *                 owned by the caller; its contents on entry do not matter
 *                 and are undefined afterwards.  Calls that run at the same
 *                 time need separate workspaces.
 * dtype must be FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_ERR_DTYPE otherwise) and
 * head_dim 64 or 128 (FA_ERR_HEAD_DIM otherwise); products use the 16-bit
 * MFMA with float32 accumulation, P and dS are rounded to dtype before they
 * enter a product, dq is summed in float32.  Because dq is accumulated with
 * atomic additions, its low bits may differ from run to run.
 * NULL, size, alignment and argument checks as for fa_varlen_fwd; dout, dq,
 * dk and dv need 16 bytes.  A workspace that is NULL or too small gives
 * FA_ERR_WORKSPACE.
 */
int fa_varlen_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                  const float* lse, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                  int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale, int32_t causal,
                  void* dq, void* dk, void* dv, int32_t batch, int32_t total_q, int32_t total_k,
                  int32_t num_heads, int32_t num_heads_k, int32_t head_dim, int32_t dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of workspace fa_varlen_bwd needs for these sizes: a float32 dq
 * accumulator [total_q, num_heads, head_dim], the float32 row terms
 * rowsum(dout * out) [num_heads, total_q] and the key-block map
 * [batch + 1], each rounded up to 256 bytes.  Host only.
 * Returns FA_ERR_NULL or FA_ERR_SHAPE on bad arguments.
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
 * with one it is row p % cache_rows of block block_table[b * blocks_per_seq
 * + p / cache_rows]; the causal mask is bottom-right as above, so one new
 * query token sees every cached key.
 *
 *   q, out        device [total_q, num_heads, head_dim] packed by
 *                 cu_seqlens_q (out written for rows < cu_seqlens_q[batch])
 *   k_cache, v_cache  device [cache_blocks, cache_rows, num_heads_k, head_dim]
 *   cu_seqlens_q  device int32 [batch + 1], cumulative
 *   seqlens_k     device int32 [batch], NOT cumulative
 *   leftpad_k     device int32 [batch] or NULL (no left padding)
 *   block_table   device int32 [batch, blocks_per_seq] or NULL (then
 *                 cache_blocks >= batch and block b is sequence b's slot)
 *   max_seqlen_q  >= every query length; max_seqlen_k >= every seqlens_k[b]
 *                 and at most the positions a sequence can hold (cache_rows,
 *                 or blocks_per_seq * cache_rows with a block table)
 *   lse           device float32 [num_heads, total_q] as fa_varlen_fwd
 *   num_splits    0 (chosen from the sizes) or 1..64 workgroups per
 *                 (sequence, key/value head), each over a contiguous key range
 *   workspace     device scratch of >= fa_varlen_kvcache_workspace_size
 *                 bytes for this num_splits, 16-byte aligned, caller-owned
 * Preconditions (not checked on the device): 0 <= leftpad_k[b] <=
 * seqlens_k[b] <= max_seqlen_k and block table entries < cache_blocks.
 * dtype FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_ERR_DTYPE), head_dim 64 or 128
 * (FA_ERR_HEAD_DIM); other checks and errors as fa_varlen_fwd, plus
 * FA_ERR_WORKSPACE and FA_ERR_ARG for num_splits out of range.
 */
int fa_varlen_fwd_kvcache(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                          const int32_t* leftpad_k, const int32_t* block_table,
                          int32_t max_seqlen_q, int32_t max_seqlen_k,
                          float softmax_scale, int32_t causal, void* out, float* lse,
                          int32_t batch, int32_t total_q, int32_t cache_blocks, int32_t cache_rows,
                          int32_t blocks_per_seq, int32_t num_heads, int32_t num_heads_k,
                          int32_t head_dim, int32_t dtype, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace bytes of fa_varlen_fwd_kvcache: float32 partial outputs and
 * (max, sum) pairs for every (query row, head, split, wavefront); num_splits
 * 0 sizes for the largest automatic choice (64).  Host only.
 */
int fa_varlen_kvcache_workspace_size(int32_t total_q, int32_t num_heads, int32_t head_dim,
                                     int32_t num_splits, size_t* bytes);

/*
 * Device-side check of the cu_seqlens preconditions (friki.work, section
 * "Estructuras de datos clave": batch+1 cumulative offsets).  Writes to
 * `flags` (device int32 [1]) a bit mask, 0 when valid:
 *   1  cu[0] != 0            2  cu decreases somewhere
 *   4  cu[batch] > total     8  some length exceeds max_seqlen
 * for either array (q bits in 0..3, k bits shifted left by 4).
 *   cu_seqlens_q, cu_seqlens_k  device int32 [batch + 1]
 *   flags                       device int32 [1], overwritten
 */
int fa_varlen_check_cu_seqlens(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t batch, int32_t total_q, int32_t total_k,
                               int32_t max_seqlen_q, int32_t max_seqlen_k,
                               int32_t* flags, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_VARLEN_H_ */
