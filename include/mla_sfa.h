/*
 * mla_sfa.h -- C ABI of the consumer of the MLA caches in libmla_prolog.so:
 * sparse flash attention in MLA-absorb mode for decode (one query per
 * batch), per the Ascend operator page aclnnSparseFlashAttention
 * ("Function" formula, parameter table, attentionMode 2).
 *
 * For each token t (its own batch) and head h, over the cache rows that
 * token's sparse indices select,
 *   s_j = scale * ([q^N | q^R][t, h] . [c^KV_j | k^R_j]),
 *   attention_out[t, h] = sum_j softmax(s)_j c^KV_j,
 *   softmax_max[t, h] = max_j s_j,  softmax_sum[t, h] = sum_j exp(s_j - max).
 * Index i selects the positions i*sparse_block_size .. +sparse_block_size-1
 * (sparse_block_size 1: token-wise); a negative index selects nothing, and
 * positions at or past the token's kv length are left out.  Position p
 * lives in slot block_table[t][p / block_size] * block_size + p % block_size
 * of the paged caches (PA_BSND); table entries outside [0, block_num) and
 * positions past max_blocks * block_size select nothing.  A token with no
 * selected row gets attention_out 0, softmax_max -inf and softmax_sum 0.
 * key = value = the kv cache (c^KV), keyRope = the kr cache (k^R), as the
 * MLA prolog writes them (separate, or concatenated rows of D + Dr).
 *
 * All tensors are caller-owned device pointers to contiguous row-major data,
 * 16-byte aligned; nothing is written but the outputs.  Runs are
 * stream-ordered on the caller's HIP stream and never block.  Status codes
 * are those of mla_prolog.h.
 */
#ifndef MLA_SFA_H
#define MLA_SFA_H

#include <stddef.h>
#include <stdint.h>

#include "mla_prolog.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * N heads (query heads; one kv head), D the latent width (c^KV, the value
 * width), Dr the rope width.  Supported: D a multiple of 32 up to 512, Dr a
 * multiple of 32 up to 64, N from 1 to 128 (MLA_ERR_UNSUPPORTED otherwise).
 * The caches are (block_num, block_size, 1, D) and (.., Dr), or one
 * (block_num, block_size, 1, D + Dr) cache with concat = 1.  block_table
 * rows hold max_blocks entries; sparse_indices rows hold sparse_size
 * entries.  max_tokens bounds T and sizes the handle's workspace (split
 * partial results).  scale is the page's scaleValue.
 */
typedef struct {
  int64_t N, D, Dr;
  int64_t block_num, block_size, max_blocks;
  int64_t sparse_size, sparse_block_size;
  int64_t max_tokens;
  double scale;
  int32_t concat;  /* 0 or 1 */
  int32_t device;  /* HIP device ordinal the handle and all tensors live on */
} mla_sfa_desc;

/*
 * One run's tensors (T tokens):
 *   query (T, N, D), query_rope (T, N, Dr)     bf16: q^N and q^R
 *   kv_cache, kr_cache                          bf16 (kr_cache NULL with concat)
 *   sparse_indices (T, sparse_size)             int32
 *   block_table (T, max_blocks)                 int32
 *   seq_lens_kv (T)                             int32 kv length of each token's batch
 *   attention_out (T, N, D)                     bf16
 *   softmax_max, softmax_sum (T, N)             fp32, optional (NULL = not written)
 */
typedef struct {
  const void* query;
  const void* query_rope;
  const void* kv_cache;
  const void* kr_cache;
  const int32_t* sparse_indices;
  const int32_t* block_table;
  const int32_t* seq_lens_kv;
  void* attention_out;
  float* softmax_max;
  float* softmax_sum;
} mla_sfa_tensors;

typedef struct mla_sfa* mla_sfa_t;

/* Checks a description and, when tensors is not NULL, one run's pointers
 * for T tokens; pure host: the parameter validation of the attention page's
 * first-phase call (aclnnSparseFlashAttentionGetWorkspaceSize, function
 * prototype), with the prolog page's return-code classes.  MLA_OK,
 * MLA_ERR_NULLPTR, MLA_ERR_PARAM_INVALID or MLA_ERR_UNSUPPORTED. */
mla_status mla_sfa_validate(const mla_sfa_desc* desc, const mla_sfa_tensors* tensors, int64_t T);

/* Creates a handle on desc->device with its workspace (the attention page's
 * first phase sizes a workspace the caller allocates; here the handle owns
 * it).  MLA_ERR_RUNTIME if the allocation fails.  *out is NULL on failure. */
mla_status mla_sfa_create(const mla_sfa_desc* desc, mla_sfa_t* out);

/* Enqueues one attention over T tokens on stream (a hipStream_t, NULL = the
 * default stream): the attention page's second-phase call
 * (aclnnSparseFlashAttention, function prototype).  T = 0 is a no-op.  One handle must not run on two
 * streams at once (its workspace is shared).  MLA_ERR_RUNTIME if a launch
 * fails.  The run only launches kernels, none of which waits on another
 * block, so it can be captured into a HIP graph: each replay computes the
 * attention of the tensors' contents at that time (replays share the
 * handle's workspace with its runs and must be ordered with them). */
mla_status mla_sfa_run(mla_sfa_t handle, const mla_sfa_tensors* tensors, int64_t T, void* stream);

/* Waits for the handle's device, frees the handle and its workspace (the
 * teardown after the page's sample call sequence). */
mla_status mla_sfa_destroy(mla_sfa_t handle);

#ifdef __cplusplus
}
#endif

#endif  /* MLA_SFA_H */
