/*
 * mla_prolog.h -- C ABI of the MI355X (gfx950) Multi-Head Latent Attention
 * prolog library, libmla_prolog.so.
 *
 * The operation is the MLA prolog of the Ascend operator page
 * aclnnMlaPrologV2WeightNz ("Function", formula block), per token t:
 *
 *   c^Q  = RmsNorm(x W^DQ)
 *   q^C  = c^Q W^UQ,  q^N = q^C W^UK         (per head)      -> queryOut
 *   q^R  = ROPE(c^Q W^QR)                    (per head)      -> queryRopeOut
 *   c^KV = RmsNorm(x W^DKV)                  -> kvCache[cacheIndex[t]]
 *   k^R  = ROPE(x W^KR)                      -> krCache[cacheIndex[t]]
 *   optional: dequantScaleQNope = RowMax(|q^N|)/127, q^N = round(q^N/scale)
 *
 * RmsNorm(v)_i = gamma_i v_i / sqrt(mean(v^2) + eps) ("RmsNorm formula").
 * ROPE is the rotate-half form (aclnnMlaPreprocess, constraints, rope mode):
 * for h = Dr/2 and i < h,
 *   out_i = v_i cos_i - v_{i+h} sin_i,  out_{i+h} = v_{i+h} cos_{i+h} + v_i sin_{i+h},
 * with cos/sin the caller's per-token table rows.
 *
 * Everything is stream-ordered on the caller's HIP stream; no call blocks on
 * the device.  All tensor arguments are caller-owned device pointers to
 * contiguous row-major data, 16-byte aligned.  The library never frees them.
 *
 * Status codes follow the operator page's return-code table ("Return Value").
 */
#ifndef MLA_PROLOG_H
#define MLA_PROLOG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_NULLPTR = 161001,       /* a required pointer is NULL */
  MLA_ERR_PARAM_INVALID = 161002, /* a shape, dtype, alignment or size is outside the domain */
  MLA_ERR_RUNTIME = 361001,       /* a HIP runtime call failed (allocation, launch) */
  MLA_ERR_UNSUPPORTED = 561002    /* legal on the page but no kernel tiling for it here */
} mla_status;

typedef enum { MLA_BF16 = 0, MLA_INT8 = 1, MLA_INT8_PARTIAL = 2, MLA_INT8_STATIC = 3, MLA_FP16 = 4 } mla_dtype;

/*
 * Problem description, fixed at create time (the page's "Shape format field
 * description"): He hidden size, Hcq q low-rank size, Hckv kv low-rank size,
 * N heads, D nope head dim, Dr rope dim, Nkv = 1.  Supported here: He, Hcq,
 * Hckv, D and Dr positive multiples of 8, Dr at most 64, D and Hckv at most
 * 512, N any positive count; in int8 mode He, Hcq, Hckv+Dr, D and Dr
 * multiples of 16.
 *
 * in_dtype MLA_BF16: the non-quantised scenario, every tensor bf16.
 * in_dtype MLA_INT8: the int8 full-quantisation scenario with a bf16 cache:
 *   tokenX, weightDq, weightUqQr, weightDkvKr int8 with fp32 dequantisation
 *   scales (per token for x, per output channel for the weights); weightUk,
 *   gammas, sin/cos and both caches bf16.  The RmsNorm output c^Q is
 *   quantised per token (scale RowMax(|c^Q|)/127) before the int8 W^UqQr
 *   product.
 * in_dtype MLA_INT8_PARTIAL: the partial-quantisation scenario with a bf16
 *   cache (same tables): weightUqQr int8 with its per-output-channel fp32
 *   scale, every other tensor bf16; c^Q is quantised per token as above.
 *   In both int8 scenarios the optional smoothScalesCq m (Hcq, fp32)
 *   multiplies c^Q element-wise before that quantisation (scale
 *   RowMax(|c^Q * m|)/127); the product is not divided back by m, so the
 *   int8 weightUqQr is expected to carry 1/m.  Only in_dtype takes this
 *   value (as it alone takes MLA_INT8_STATIC).
 * query_dtype MLA_INT8: queryOut is int8 with one fp32 dequantisation scale
 *   per (token, head), RowMax(|q^N|)/127 ("Dequant Scale Query Nope
 *   calculation formula"); MLA_BF16: queryOut is bf16.  As in the page's
 *   dtype table, an int8 queryOut needs in_dtype MLA_INT8 (otherwise
 *   MLA_ERR_PARAM_INVALID); int8 inputs with a bf16 queryOut are allowed.
 * cache_dtype MLA_INT8: quantised caches (the "kv_cache quantized" columns
 *   of the scenario and dtype tables), only with in_dtype MLA_INT8 or
 *   MLA_INT8_PARTIAL.  The kv cache holds int8 codes of c^KV with
 *   quant_scale_ckv; with partial quantisation the kr cache holds int8
 *   codes of k^R with quant_scale_ckr, while full quantisation keeps a bf16
 *   kr cache.  A code is the value times its channel's scale, rounded half
 *   to even and saturated to [-128, 127].  MLA_BF16: bf16 caches.
 * in_dtype MLA_INT8_STATIC: the static int8 scenario of the MLA preprocess
 *   page (aclnnMlaPreprocess, "Function" formulas and parameter table,
 *   quantMode 0: per-tensor static asymmetric quantisation).  tokenX is
 *   bf16 and the library quantises it by RmsNormQuant:
 *     code = saturate[-128, 127](round-half-even(f32(v) * quantScale) + quantOffset),
 *     v = gamma_x * x / sqrt(mean(x^2) + eps_x) + beta_x   (v = x when
 *     x_quant_only is 1, the page's doRmsNorm false),
 *   decided in fp32 with the one bf16 quant_scale_x and int8
 *   quant_offset_x.  weightDq, weightDkvKr and weightUqQr are int8; each
 *   int8 product is biased and dequantised per output channel,
 *   y = (acc + bias[n]) * deScale[n] (deScale0 = scale_w_dq | scale_w_dkv_kr,
 *   bias0 = bias_dqkv; deScale1 = scale_w_uq_qr, bias1 = bias_uq_qr).  c^Q
 *   is quantised the same way from gamma_cq * y_q / RMS + beta_cq with
 *   quant_scale_cq / quant_offset_cq; c^KV is RmsNorm(y_kv) with gamma_ckv
 *   (the page's gamma2).  weightUk and the caches are bf16; queryOut is
 *   bf16.  Same size rules as in_dtype MLA_INT8.  The scale multiplies, as
 *   the page's RmsNormQuant formula writes it; the offset is added to the
 *   rounded product.
 * concat 1: the preprocess page's cacheMode 0.  queryOut is (T, N, Hckv+Dr),
 *   each row q^N then q^R, and query_rope_out is NULL; kvCache is
 *   (block_num, block_size, 1, Hckv+Dr), each row c^KV then k^R, and
 *   kr_cache is NULL.  bf16 queryOut and caches only.  0: the separate
 *   outputs and caches of the prolog page (the preprocess page's cacheMode 1).
 * weights_nk 1: weightDq (Hcq, He), weightDkvKr (Hckv+Dr, He) and weightUqQr
 *   (N*(D+Dr), Hcq) come transposed, (n, k) row-major, as the preprocess
 *   page takes its weights (transposeWdq / transposeWuq); its fused
 *   (Hcq+Hckv+Dr, He) weight is weightDq followed by weightDkvKr.  Runs then
 *   need packed_weights (the unpacked kernels read (k, n) weights only:
 *   MLA_ERR_UNSUPPORTED otherwise).  0: (k, n) row-major.
 * x_quant_only: see MLA_INT8_STATIC; 0 in the other scenarios.
 * float_dtype MLA_FP16 (with in_dtype MLA_INT8_STATIC only; else
 *   MLA_ERR_PARAM_INVALID): the preprocess page's FLOAT16 input (its
 *   parameter table, input "FLOAT16, BFLOAT16", and the tensors whose dtype
 *   it ties to the input's).  tokenX, gamma_x/beta_x/quant_scale_x,
 *   gamma_cq/beta_cq/quant_scale_cq, gamma_ckv, rope_sin/rope_cos and
 *   weightUk are fp16, and so are queryOut, queryRopeOut and both caches;
 *   q^C enters the W^UK product rounded to fp16.  The deScale arguments stay
 *   fp32 (the page's INT64 deScale of the FLOAT16 input is an encoding of the
 *   same per-channel scale that this boundary does not take).  Runs need
 *   packed_weights (MLA_ERR_UNSUPPORTED otherwise).  MLA_BF16: those tensors
 *   are bf16.
 * check_index 1: every run first copies cacheIndex to the host, which waits
 *   for the stream, and returns MLA_ERR_PARAM_INVALID with nothing enqueued
 *   if an entry lies outside [0, block_num*block_size) (the prolog page's
 *   "Parameters" table, cacheIndex: the values must lie in that range).  A
 *   debugging aid: it costs a device-to-host copy and a wait per run.  With
 *   0, out-of-range entries are skipped on the device (their rows are
 *   written nowhere) and nothing is reported.  No check is made when
 *   block_num is 0 (no cache update).
 * max_tokens bounds T of every run; it sizes the handle's workspace.
 * eps_cq / eps_ckv: the two RmsNorm epsilons (the page recommends 1e-5);
 *   eps_x: that of the RmsNorm of x (MLA_INT8_STATIC; the preprocess page
 *   has one epsilon for its three norms).
 */
typedef struct {
  int64_t He, Hcq, Hckv, N, D, Dr;
  int64_t block_num, block_size; /* paged caches [block_num, block_size, 1, .] */
  int64_t max_tokens;
  double eps_cq, eps_ckv;
  int32_t in_dtype;    /* mla_dtype */
  int32_t query_dtype; /* mla_dtype */
  int32_t device;      /* HIP device ordinal the handle and all tensors live on */
  int32_t cache_dtype; /* mla_dtype: MLA_BF16, or MLA_INT8 (quantised caches) */
  int32_t concat;      /* 0 or 1 */
  int32_t weights_nk;  /* 0 or 1 */
  int32_t x_quant_only; /* 0 or 1 */
  int32_t check_index; /* 0 or 1 (a debugging aid, see below) */
  double eps_x;
  int32_t float_dtype; /* mla_dtype: MLA_BF16, or MLA_FP16 (MLA_INT8_STATIC only) */
  int32_t reserved;    /* 0 */
} mla_prolog_desc;

/*
 * Tensors of one run (the page's parameter table), all device pointers:
 *   token_x          (T, He)            bf16, or int8
 *   weight_dq        (He, Hcq)          (k, n) row-major (see weights_nk), bf16 or int8
 *   weight_uq_qr     (Hcq, N*(D+Dr))    head-interleaved columns: column
 *                                       h*(D+Dr)+j is W^UQ column h*D+j for
 *                                       j < D, W^QR column h*Dr+j-D otherwise
 *   weight_uk        (N, D, Hckv)       bf16
 *   weight_dkv_kr    (He, Hckv+Dr)      W^DKV columns first, then W^KR
 *   gamma_cq (Hcq), gamma_ckv (Hckv)    bf16
 *   rope_sin, rope_cos (T, Dr)          bf16
 *   cache_index      (T)                int64 flat slot block*block_size+offset;
 *                                       entries outside [0, block_num*block_size)
 *                                       are skipped; duplicates are undefined
 *   kv_cache (block_num, block_size, 1, Hckv), kr_cache (.., Dr)
 *                                       bf16 (or int8, see cache_dtype),
 *                                       updated in place at the named slots
 *                                       only; may be NULL iff block_num is 0
 *                                       (no cache update)
 *   scale_x (T), scale_w_dq (Hcq), scale_w_uq_qr (N*(D+Dr)),
 *   scale_w_dkv_kr (Hckv+Dr)            fp32, int8 mode only, else NULL;
 *                                       partial quantisation takes
 *                                       scale_w_uq_qr alone; the static
 *                                       scenario all but scale_x
 *   query_out        (T, N, Hckv)       bf16, or int8 when query_dtype is INT8
 *                                       ((T, N, Hckv+Dr) with concat)
 *   query_rope_out   (T, N, Dr)         bf16 (NULL with concat)
 *   dequant_scale_q_nope (T, N)         fp32 when query_dtype is INT8, else NULL
 *   packed_weights                      optional (NULL = none): the output of
 *                                       mla_prolog_pack_weights for these
 *                                       four weights, 256-byte aligned.  When
 *                                       given, every run streams the weights
 *                                       from it, and weight_dq, weight_uq_qr,
 *                                       weight_uk and weight_dkv_kr may be
 *                                       NULL (no kernel of the run reads
 *                                       them); when NULL, all four are
 *                                       required.
 *   smooth_scales_cq (Hcq)              fp32 smoothScalesCq, optional (NULL =
 *                                       none) with an int8 weightUqQr, NULL
 *                                       otherwise
 *   quant_scale_ckv (Hckv), quant_scale_ckr (Dr)
 *                                       fp32 quantScaleCkv / quantScaleCkr:
 *                                       each given exactly when its cache is
 *                                       int8 (see cache_dtype), else NULL
 * MLA_INT8_STATIC only (NULL otherwise), the preprocess page's names after
 * the equals sign:
 *   gamma_x = gamma0, beta_x = beta0   (He) bf16; NULL with x_quant_only
 *   quant_scale_x = quantScale0 (1) bf16, quant_offset_x = quantOffset0 (1) int8
 *   bias_dqkv = bias0 (Hcq+Hckv+Dr)     int32, optional (NULL = zeros); each
 *                                       biased sum acc + bias must fit int32,
 *                                       like the accumulator (as for bias1)
 *   beta_cq = beta1 (Hcq)               bf16
 *   quant_scale_cq = quantScale1 (1) bf16, quant_offset_cq = quantOffset1 (1) int8
 *   bias_uq_qr = bias1 (N*(D+Dr))       int32, optional (NULL = zeros)
 * Outputs must not alias inputs.
 */
typedef struct {
  const void* token_x;
  const void* weight_dq;
  const void* weight_uq_qr;
  const void* weight_uk;
  const void* weight_dkv_kr;
  const void* gamma_cq;
  const void* gamma_ckv;
  const void* rope_sin;
  const void* rope_cos;
  const int64_t* cache_index;
  void* kv_cache;
  void* kr_cache;
  const float* scale_x;
  const float* scale_w_dq;
  const float* scale_w_uq_qr;
  const float* scale_w_dkv_kr;
  void* query_out;
  void* query_rope_out;
  float* dequant_scale_q_nope;
  const void* packed_weights; /* optional: the four weights in the library's packed layout */
  const float* smooth_scales_cq;
  const float* quant_scale_ckv;
  const float* quant_scale_ckr;
  const void* gamma_x;
  const void* beta_x;
  const void* quant_scale_x;
  const int8_t* quant_offset_x;
  const int32_t* bias_dqkv;
  const void* beta_cq;
  const void* quant_scale_cq;
  const int8_t* quant_offset_cq;
  const int32_t* bias_uq_qr;
} mla_prolog_tensors;

typedef struct mla_prolog* mla_prolog_t;

/* Checks a description and, when tensors is not NULL, one run's pointers
 * (presence, 16-byte alignment) and T (0 <= T <= max_tokens).  Pure host
 * code: it touches no device and no device memory.  It stands for the
 * parameter validation of the page's first-phase call
 * (aclnnMlaPrologV2WeightNzGetWorkspaceSize, "Function Prototype"), with the
 * error classes of its "Return Value" table: MLA_ERR_NULLPTR where a required
 * pointer is missing, MLA_ERR_PARAM_INVALID where a shape, dtype, alignment
 * or size is outside the domain, MLA_ERR_UNSUPPORTED where the sizes are
 * legal but no kernel tiling takes them. */
mla_status mla_prolog_validate(const mla_prolog_desc* desc, const mla_prolog_tensors* tensors,
                               int64_t T);

/* Bytes of device workspace a handle for desc owns (0 if desc is invalid):
 * the workspaceSize output of the page's first-phase call
 * (aclnnMlaPrologV2WeightNzGetWorkspaceSize, "Parameters"), fixed here by
 * the description and max_tokens. */
size_t mla_prolog_workspace_bytes(const mla_prolog_desc* desc);

/* Bytes of the packed-weight buffer for desc (0 if desc is invalid). */
size_t mla_prolog_packed_weights_bytes(const mla_prolog_desc* desc);

/* Writes weight_dq, weight_uq_qr, weight_uk and weight_dkv_kr of tensors
 * (row-major, as for mla_prolog_run) into packed, a caller-owned device
 * buffer of mla_prolog_packed_weights_bytes bytes, 256-byte aligned, in the
 * library's packed layout: per matrix, windows of 64 columns, each stored as
 * its k-stages (32 bf16 or 64 int8 rows, 4 KB) in MFMA operand order, so that
 * a run streams every window as one contiguous region.  Like the operator
 * page's weights, which its API takes in a pre-tiled format (the NZ format
 * of weightDq, weightUqQr and weightDkvKr in its "Parameters" table), this
 * is a one-time conversion per weight set; the tiling is the library's own.
 * Stream-ordered; the other tensor fields are ignored.  Returns
 * MLA_ERR_NULLPTR for a missing weight or buffer, MLA_ERR_PARAM_INVALID for
 * a misaligned one, MLA_ERR_RUNTIME if the launch fails. */
mla_status mla_prolog_pack_weights(mla_prolog_t handle, const mla_prolog_tensors* tensors,
                                   void* packed, void* stream);

/* Validates desc, allocates the handle and its device workspace on
 * desc->device (the caller's current device is restored).  It stands for the
 * page's first phase (aclnnMlaPrologV2WeightNzGetWorkspaceSize, "Function
 * Prototype"), whose workspace the caller allocates: here the handle owns
 * it, sized for max_tokens, and every run reuses it.  The handle belongs to
 * the caller until mla_prolog_destroy.  Returns the validation codes of
 * mla_prolog_validate, or MLA_ERR_RUNTIME if the allocation fails (the
 * "Return Value" table's runtime class).  On error *out is set to NULL.  Two environment variables, read here, are for diagnosis:
 * MLA_PROLOG_FUSED=0 keeps small-T runs off the one-launch kernel, and
 * MLA_PROLOG_FUSED_SPIN=n (a whole number in 1..2^20) caps the poll steps of
 * the small-T kernels' bounded waits (see mla_prolog_check); any other value
 * of it makes create return MLA_ERR_PARAM_INVALID. */
mla_status mla_prolog_create(const mla_prolog_desc* desc, mla_prolog_t* out);

/* Enqueues one prolog over T tokens on stream (a hipStream_t; NULL = the
 * default stream): the page's second-phase call (aclnnMlaPrologV2WeightNz,
 * "Function Prototype" and its "Parameters": workspace, executor, stream),
 * with the tensors given per run and the workspace the handle's.  Every
 * pointer and T are validated first (as by mla_prolog_validate; nothing is
 * enqueued on an error); MLA_ERR_RUNTIME if a launch fails.  Returns after
 * enqueueing; the outputs and caches are ready when the stream reaches this
 * point.  T = 0 enqueues nothing.  A
 * handle's workspace is shared by its runs: runs of one handle on different
 * streams must be ordered by the caller.  The result is deterministic: the
 * same inputs give bit-identical outputs.
 * Small-T runs on packed weights (T <= 32) launch kernels whose blocks wait
 * for data from other blocks of the same launch, so such a run needs those
 * blocks resident on the device together: kernels from other streams or
 * processes must not occupy the device while it runs.  Otherwise a bounded
 * wait gives up and mla_prolog_check reports the run; MLA_PROLOG_FUSED=0
 * (see mla_prolog_create) keeps small-T runs on kernels that wait only
 * between the two blocks of a head.  A wait that gives up marks a word in
 * host-visible memory: once an earlier run's mark is visible to the host,
 * mla_prolog_run returns MLA_ERR_RUNTIME with nothing enqueued, until
 * mla_prolog_check has reported it (a run enqueued before the mark became
 * visible still runs; mla_prolog_check is the one certain report).
 * A run enqueued while stream is being captured into a HIP graph takes
 * only the kernels that hand no data across blocks (the selection of
 * mla_prolog_run_noalloc), since a captured launch would replay the run
 * number it was captured with: every replay of the graph then computes the
 * prolog of the tensors' contents at that time.  Replays use the handle's
 * workspace like runs do, so they must be ordered with the handle's other
 * runs and replays.  No profiling events are recorded for such a run, and
 * with check_index set it returns MLA_ERR_PARAM_INVALID (the check waits
 * for the device). */
mla_status mla_prolog_run(mla_prolog_t handle, const mla_prolog_tensors* tensors, int64_t T,
                          void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one
 * prolog as mla_prolog_run, with no handle.  Its workspace is a static
 * array of the library, 64 MiB on each device (held from the library's
 * first use on that device until the process ends); the call allocates
 * nothing, also no host memory, and never waits for the device.
 *   desc, tensors, T, stream: as for mla_prolog_validate and
 *     mla_prolog_run (T <= desc->max_tokens); packed_weights, when given,
 *     come from mla_prolog_pack_weights of a handle with the same
 *     description.  desc->check_index must be 0.
 *   Returns the validation codes of mla_prolog_validate;
 *     MLA_ERR_PARAM_INVALID also when the run's workspace would exceed the
 *     64 MiB (at the model shapes of the prolog page's samples, He 7168,
 *     Hcq 1536, Hckv 512, N 128, D 128, Dr 64: up to about 400 tokens) or
 *     check_index is set; MLA_ERR_RUNTIME if the array's device address
 *     cannot be had or a launch fails.  Nothing is enqueued on an error.
 * Small token counts take the kernels that hand no data across blocks (the
 * ones mla_prolog_run takes with MLA_PROLOG_FUSED=0 and no paired blocks),
 * so runs are not faster than mla_prolog_run's.  Every call on a device
 * shares its one array: calls that overlap on one device (on different
 * streams, or from different threads without ordering) race and give wrong
 * results; calls ordered on one stream are safe.  Nothing in the array has
 * to start at zero: each call writes what it reads. */
mla_status mla_prolog_run_noalloc(const mla_prolog_desc* desc, const mla_prolog_tensors* tensors, int64_t T,
                                  void* stream);

/* Frees the workspace and the handle (after synchronising its device): the
 * teardown that follows the page's sample call sequence (releasing the
 * workspace and the executor).  MLA_ERR_NULLPTR for a NULL handle,
 * MLA_ERR_RUNTIME if the device reports an error; the handle is freed in
 * either case. */
mla_status mla_prolog_destroy(mla_prolog_t handle);

/* Waits for the handle's device and reports whether any earlier run gave up
 * waiting for another block of its own launch (MLA_ERR_RUNTIME, the runtime
 * class of the page's "Return Value" table; then the outputs of those runs
 * are not to be trusted), else MLA_OK; clears the record, after which
 * mla_prolog_run accepts runs again.  On the small-T kernels the blocks of one launch hand data to one
 * another and wait, with a bounded spin, for it; that can only fail when
 * the launch does not get the whole device (the library checks at create
 * time that all of its blocks fit on the device at once). */
mla_status mla_prolog_check(mla_prolog_t handle);

/* Sets the poll steps after which a bounded wait of the small-T kernels
 * gives up (see mla_prolog_check), from the next run on: steps in
 * 1..2^20, or 0 for the default (2^20 steps, about a second).  Other values
 * return MLA_ERR_PARAM_INVALID.  For diagnosis and tests of the failure
 * report; a wait that gave up leaves nothing behind that a later run could
 * mistake for its own data (flags and tags carry the number of their run). */
mla_status mla_prolog_set_poll_limit(mla_prolog_t handle, int32_t steps);

/* Kernel timing with HIP events, for benchmarks (no passage of the page:
 * instrumentation of this library).  After
 * mla_prolog_profile_enable(h, 1) every run of h records HIP events on its
 * stream before its first kernel and after each of its four kernels
 * (down_proj, norm_rope_cache, up_proj, uk; where one kernel does both
 * up_proj and uk, its time is booked to up_proj and uk reads 0; where one
 * kernel does the whole run, its time is booked to up_proj and the other
 * three read 0).
 * mla_prolog_profile_read waits
 * for the recorded events and returns, per kernel, the elapsed milliseconds
 * summed over the runs since the previous read (kernel_ms[4]) and the number
 * of those runs; at most 2048 runs are kept between reads (more is an
 * MLA_ERR_PARAM_INVALID at read time).  Enabling creates the events;
 * disabling destroys them. */
mla_status mla_prolog_profile_enable(mla_prolog_t handle, int enable);
mla_status mla_prolog_profile_read(mla_prolog_t handle, double* kernel_ms, int64_t* runs);

/* Text of a status code (the descriptions of the page's "Return Value"
 * table, in short). */
const char* mla_prolog_status_string(mla_status status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_PROLOG_H */
