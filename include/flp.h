/*
 * flp.h -- C ABI of the fused linear selected-token log-probability library
 * for AMD MI355X (gfx950).
 *
 * For token rows i = 0..N-1, vocabulary columns v = 0..V-1:
 *
 *   z_iv   = (hidden_i . W_v + b_v) / T_i            scaled logits (never stored)
 *   lse_i  = log sum_v exp(z_iv)
 *   logp_i = z_i[t_i] - lse_i     if 0 <= t_i < V, else exactly 0
 *
 * The operation is the one of the "Fused Linear LogP" docs page (section
 * "Reference Semantics": linear layer, log_softmax, gather at the target;
 * section "Tensor Contract": shapes, dtypes, float32 output
 * z[target] - logsumexp(z)).  The optional per-row temperature and the
 * fail-closed gates follow the "Feat/nemotron h lm head logprob cuda" page
 * (PR #555, summary bullets); the temperature divides the biased logits.
 * Out-of-range targets give logp = 0 and zero gradient (PR #234 inline
 * review; PR #547 page, section "What", indexed semantics).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers on the current HIP device,
 *     row-major and densely packed, owned by the caller.  The library
 *     allocates no device memory and keeps no state besides a once-
 *     initialised per-device property cache (and, only while the optional
 *     kernel timing below is enabled, a pool of HIP events); the calls are
 *     re-entrant.
 *   - Work is enqueued on `stream` (a hipStream_t, or NULL for the default
 *     stream) and the call returns at once (the measurement probes at the end
 *     are the one exception).  Outputs are valid once the stream has
 *     synchronised; device faults surface there.
 *   - Inputs are read-only.  Outputs are overwritten, never accumulated.
 *     No output may overlap any input or another output (checked from the
 *     address ranges; FLP_INVALID_ARGUMENT otherwise).
 *   - Every argument is validated before anything is enqueued.  On any
 *     non-OK status nothing has been enqueued and no output was touched.
 *     There is no fallback path: an unsupported case is an error.
 *   - N = 0 enqueues nothing, except that the backward calls still write
 *     d_weight and d_bias (when given) as zeros: they are sums over the
 *     rows, and a sum over no rows is zero.
 *   - Results are deterministic and batch-invariant: logp, lse and each row
 *     of d_hidden are bitwise the same whatever the other rows are, whatever
 *     N is and wherever the row sits; d_weight and d_bias are bitwise the
 *     same from run to run and for any backward workspace size.
 */
#ifndef FLP_H_
#define FLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum flp_status {
  FLP_OK = 0,
  FLP_INVALID_ARGUMENT = 1,      /* null required pointer, N < 0, V < 1, D < 1, overlap */
  FLP_UNSUPPORTED_DTYPE = 2,     /* a dtype outside the lists below */
  FLP_UNSUPPORTED_SHAPE = 3,     /* D % 32 != 0, 256 * D * element size >= 2^31 (32-bit row
                                    offsets inside a 256-row tile), or a size beyond the
                                    64-bit index range */
  FLP_MISALIGNED = 4,            /* hidden/weight/workspace not 16-byte aligned, others not
                                    aligned to their element size */
  FLP_WORKSPACE_TOO_SMALL = 5,   /* workspace_bytes below the *_workspace_bytes minimum */
  FLP_UNSUPPORTED_DEVICE = 6,    /* current device is not gfx950 */
  FLP_HIP_ERROR = 7              /* a HIP runtime call or kernel launch failed */
} flp_status;

typedef enum flp_dtype {
  FLP_BF16 = 0,   /* bfloat16, 2 bytes */
  FLP_F32 = 1,    /* IEEE binary32 */
  FLP_I64 = 2,    /* int64 target ids */
  FLP_I32 = 3,    /* int32 target ids */
  FLP_F16 = 4     /* IEEE binary16 */
} flp_dtype;

/*
 * Forward workspace in bytes for (N, D, V): per-row, per-vocabulary-tile
 * partial (max, sum-of-exp) pairs and the target logits.  16-byte aligned.
 * These are the per-row softmax statistics of each vocabulary slab that the
 * "Fused Linear LogP" docs page folds instead of materialising the logits
 * (intro and "Tensor Parallel Vocab Shards": per-slab partials combined in a
 * fixed order); the caller provides the memory so that the library allocates
 * nothing.  Returns 0 for N < 0, D < 1 or V < 1.
 */
size_t flp_forward_workspace_bytes(int64_t N, int64_t D, int64_t V);

/*
 * Forward: out_logp[i] and (optionally) out_lse[i] for every row.
 *
 *   x_dtype      FLP_BF16, FLP_F16 or FLP_F32: element type of hidden and weight
 *                (the docs page's Tensor Contract lists bf16 / fp16 / fp32).
 *   hidden       [N, D] x_dtype, 16-byte aligned.
 *   weight       [V, D] x_dtype, 16-byte aligned.
 *   bias         [V] float32, or NULL for no bias.
 *   targets      [N] ids of t_dtype (FLP_I64 or FLP_I32); any value is legal,
 *                an id outside [0, V) marks the row as ignored (logp = 0).
 *   temperature  [N] float32 (> 0, finite; not checked), or NULL for T = 1.
 *   out_logp     [N] float32.
 *   out_lse      [N] float32 log-sum-exp of the scaled logits, or NULL
 *                (rollout).  logp is bitwise the same either way.
 *   workspace    >= flp_forward_workspace_bytes(N, D, V) bytes, 16-byte
 *                aligned; scratch, contents undefined after the call.
 *   stream       hipStream_t to enqueue on.
 *
 * Requirements: D % 32 == 0, V >= 1, N >= 0.
 */
flp_status flp_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                       const void* hidden, const void* weight, const float* bias,
                       const void* targets, flp_dtype t_dtype,
                       const float* temperature,
                       float* out_logp, float* out_lse,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Largest forward workspace (flp_forward_workspace_bytes) that the
 * allocation-free forward serves: the size of its fixed per-device scratch
 * array, 33 MiB (at V = 131072, batches of up to 8439 rows).
 */
#define FLP_FORWARD_NOALLOC_MAX_BYTES ((size_t)33 << 20)

/*
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The same computation as flp_forward, with the same bits, but the
 * workspace is a fixed array of FLP_FORWARD_NOALLOC_MAX_BYTES that the library
 * holds on every device it runs on (from the first call on that device until
 * the process ends); the caller passes only inputs and outputs.  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library routine
 * (keep the optional kernel timing below off, since it creates HIP events).
 *
 * Arguments, gates and statuses as for flp_forward, plus FLP_WORKSPACE_TOO_SMALL
 * when flp_forward_workspace_bytes(N, D, V) exceeds FLP_FORWARD_NOALLOC_MAX_BYTES.
 * All calls on one device share its array: calls that overlap in time on one
 * device (two streams, two threads) race and must be serialised by the caller.
 */
flp_status flp_forward_noalloc(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                               const void* hidden, const void* weight, const float* bias,
                               const void* targets, flp_dtype t_dtype,
                               const float* temperature, float* out_logp, float* out_lse,
                               void* stream);

/*
 * Vocabulary shards ("Fused Linear LogP" docs page, "Tensor Parallel Vocab
 * Shards"): a rank that holds rows [vocab_start, vocab_start + V_local) of the
 * weight computes the per-tile partials of its slice; the partials of all
 * shards, concatenated in ascending vocabulary order, are folded by flp_merge
 * exactly as flp_forward folds its own, so the result is bitwise that of the
 * unsharded call.
 *
 * Bytes of the partial block of a shard of V_local rows: ceil(V_local / 256)
 * slabs x N (max, sum-of-exp) float pairs, slab-major ([slab][N] float2).
 */
size_t flp_forward_partial_bytes(int64_t N, int64_t V_local);

/*
 * Partial forward over one vocabulary shard.
 *
 *   weight       [V_local, D] x_dtype: rows vocab_start .. vocab_start + V_local - 1
 *                of the full weight.
 *   bias         [V_local] float32 slice of the full bias, or NULL.
 *   targets      [N] global ids (as for flp_forward).
 *   hidden, x_dtype, t_dtype, temperature: as for flp_forward.
 *   partial      flp_forward_partial_bytes(N, V_local) bytes, 16-byte aligned:
 *                the shard's [slab][N] (max, sum-of-exp) pairs.
 *   zt           [N] float32: the scaled target logit for rows whose target is
 *                in this shard, 0.0 for every other row, so that the shards' zt
 *                add up exactly to the full target logits.
 *
 * Requirements: vocab_start % 256 == 0; V_local % 256 == 0 unless the shard
 * ends the vocabulary (vocab_start + V_local == V_total); D % 32 == 0.
 */
flp_status flp_forward_partial(int64_t N, int64_t D, int64_t V_local, int64_t vocab_start,
                               int64_t V_total, flp_dtype x_dtype, const void* hidden,
                               const void* weight, const float* bias, const void* targets,
                               flp_dtype t_dtype, const float* temperature, void* partial,
                               float* zt, void* stream);

/*
 * Merge of the partials of all shards of a V_total vocabulary.
 *
 *   partials     [ceil(V_total / 256)][N] (max, sum-of-exp) float pairs: the
 *                shards' partial blocks concatenated in ascending vocabulary
 *                order; 16-byte aligned.
 *   zt           [N] float32: the sum of the shards' zt.
 *   targets      [N] global ids of t_dtype.
 *   out_logp     [N] float32; out_lse [N] float32 or NULL (as for flp_forward).
 */
flp_status flp_merge(int64_t N, int64_t V_total, const void* partials, const float* zt,
                     const void* targets, flp_dtype t_dtype, float* out_logp, float* out_lse,
                     void* stream);

/*
 * The sibling operator on materialised logits ("Fused LogP": the docs page's
 * intro contrasts it with the linear op; PR #234 "Summary" and "Implementation
 * details", PR #547 "What"): the same lse, selected log-probability and dlogits
 * definitions applied to given logits, with no projection, bias or temperature.
 *
 *   logits       [N, V] x_dtype (FLP_BF16, FLP_F16 or FLP_F32), row-major,
 *                16-byte aligned; V * element size must be a multiple of 16.
 *   targets      [N] ids of t_dtype; an id outside [0, V) gives logp = 0 and a
 *                zero gradient row.
 *   out_logp     [N] float32; out_lse [N] float32 or NULL.
 *
 * One wave per row streams the row once (online max / sum of exp per lane in
 * chunk order, then a fixed butterfly across the wave): a row's results do not
 * depend on the other rows.
 */
flp_status flp_logits_forward(int64_t N, int64_t V, flp_dtype x_dtype, const void* logits,
                              const void* targets, flp_dtype t_dtype, float* out_logp,
                              float* out_lse, void* stream);

/*
 *   d_logits[i, v] = G_i (onehot(t_i)_v - exp(logits[i, v] - lse_i)),
 *   G_i = grad_out[i] for in-range targets, else 0.
 *
 *   grad_out     [N] float32;  lse [N] float32 from flp_logits_forward.
 *   d_logits     [N, V] x_dtype (RNE from fp32), 16-byte aligned; must not
 *                overlap the inputs.
 */
flp_status flp_logits_backward(int64_t N, int64_t V, flp_dtype x_dtype, const float* grad_out,
                               const float* lse, const void* logits, const void* targets,
                               flp_dtype t_dtype, void* d_logits, void* stream);

/*
 * Backward workspace in bytes: the dlogits tile buffers the backward keeps
 * between its recompute and its two GEMMs ("Fused Linear LogP" docs page,
 * intro: tiled dlogits workspaces), the transposed operands, the d_bias
 * partials and, when the rows run in several chunks, the fp32 d_weight
 * accumulator that makes the chunking bit-neutral (PR #555 summary bullets:
 * chunked deterministic backward).  chunk_rows = 0 asks for the minimum (row
 * chunks of 256, or one chunk of the whole batch when that needs less because a
 * single chunk needs no fp32 d_W accumulator); a positive chunk_rows asks for the size that lets the
 * backward process that many rows per chunk (rounded up to a multiple of
 * 256, capped at N rounded up).  Any workspace at least the minimum is
 * accepted; a larger one gives larger chunks and the same bits.
 */
size_t flp_backward_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                    flp_dtype dw_dtype, int64_t chunk_rows);

/*
 * Rows per chunk that flp_backward uses with `workspace_bytes` of workspace
 * when the outputs flagged by need_* (0 or 1) are requested: a multiple of 256,
 * at most N rounded up to 256, or 0 when the workspace is below the minimum.
 * Pure host arithmetic (no device needed); the chunking never changes the bits.
 */
int64_t flp_backward_chunk_rows(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                flp_dtype dw_dtype, size_t workspace_bytes, int need_d_hidden,
                                int need_d_weight, int need_d_bias);

/*
 * Backward of L = sum_i grad_out[i] * logp[i]:
 *
 *   dz_iv     = G_i (onehot(t_i)_v - exp(z_iv - lse_i)) / T_i,
 *               G_i = grad_out[i] if 0 <= t_i < V else 0
 *   d_hidden  = dz W          [N, D] in x_dtype (RNE from fp32 accumulation)
 *   d_weight  = dz^T hidden   [V, D] in dw_dtype (fp32 accumulation over the
 *                              tokens in ascending order, one final rounding)
 *   d_bias    = sum_i dz_i    [V] float32
 *
 * (PR #234, "Implementation details": grad_out * (one_hot - softmax) from the
 * saved statistics; PR #555 summary: chunked deterministic backward whose
 * chunking is bit-neutral.)
 *
 *   grad_out     [N] float32.
 *   lse          [N] float32 as written by flp_forward for the same inputs.
 *   hidden, weight, bias, targets, t_dtype, temperature: as in flp_forward.
 *   d_hidden     [N, D] x_dtype, or NULL to skip.
 *   d_weight     [V, D] dw_dtype (x_dtype or FLP_F32), or NULL to skip.
 *   d_bias       [V] float32, or NULL to skip (allowed with bias == NULL).
 *   workspace    >= flp_backward_workspace_bytes(N, D, V, x_dtype, dw_dtype, 0).
 */
flp_status flp_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                        const float* grad_out, const float* lse,
                        const void* hidden, const void* weight, const float* bias,
                        const void* targets, flp_dtype t_dtype,
                        const float* temperature,
                        void* d_hidden, void* d_weight, flp_dtype dw_dtype,
                        float* d_bias,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Indexed (row-subset) variants (PR #547 "What", indexed semantics; PR #234
 * "Implementation details": rows left out by an indexed call get exactly zero
 * gradients).  A list of row ids selects which rows of the batch are computed:
 *
 *   rows         [n_rows] ids of r_dtype (FLP_I64 or FLP_I32), any order; may be
 *                NULL when n_rows == 0.  An id listed more than once selects its
 *                row once; an id outside [0, N) is ignored.
 *
 * Outputs keep the full row shape.  A selected row gets exactly the bits the
 * dense call gives it; every other row gets logp = 0, lse = 0 and zero
 * gradient rows.  d_weight and d_bias sum over the selected rows only.  The
 * linear variants gather the selected rows into the workspace (ascending row
 * order), run the dense kernels on them and scatter the results back, so their
 * cost scales with min(n_rows, N), not N.  No host synchronisation: the number
 * of distinct selected rows stays on the device, and the capacity min(n_rows, N)
 * sizes the work.  Row ids must be below 2^31.
 *
 * Workspace sizes depend on n_rows; flp_backward_indexed_workspace_bytes's
 * chunk_rows has the meaning it has for flp_backward_workspace_bytes, applied
 * to the selected rows.
 */
size_t flp_forward_indexed_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                           int64_t n_rows);
flp_status flp_forward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                               const void* hidden, const void* weight, const float* bias,
                               const void* targets, flp_dtype t_dtype, const float* temperature,
                               const void* rows, flp_dtype r_dtype, int64_t n_rows,
                               float* out_logp, float* out_lse, void* workspace,
                               size_t workspace_bytes, void* stream);
size_t flp_backward_indexed_workspace_bytes(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                            flp_dtype dw_dtype, int64_t n_rows,
                                            int64_t chunk_rows);
/* lse: [N] as written by flp_forward_indexed (or flp_forward) for the same
 * inputs; only the selected rows are read. */
flp_status flp_backward_indexed(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                const float* grad_out, const float* lse, const void* hidden,
                                const void* weight, const float* bias, const void* targets,
                                flp_dtype t_dtype, const float* temperature, const void* rows,
                                flp_dtype r_dtype, int64_t n_rows, void* d_hidden,
                                void* d_weight, flp_dtype dw_dtype, float* d_bias,
                                void* workspace, size_t workspace_bytes, void* stream);

/* The operator on materialised logits, indexed: the workspace holds one byte
 * per row (the selection mask). */
size_t flp_logits_indexed_workspace_bytes(int64_t N);
flp_status flp_logits_forward_indexed(int64_t N, int64_t V, flp_dtype x_dtype,
                                      const void* logits, const void* targets, flp_dtype t_dtype,
                                      const void* rows, flp_dtype r_dtype, int64_t n_rows,
                                      float* out_logp, float* out_lse, void* workspace,
                                      size_t workspace_bytes, void* stream);
flp_status flp_logits_backward_indexed(int64_t N, int64_t V, flp_dtype x_dtype,
                                       const float* grad_out, const float* lse,
                                       const void* logits, const void* targets,
                                       flp_dtype t_dtype, const void* rows, flp_dtype r_dtype,
                                       int64_t n_rows, void* d_logits, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Untied embedding lookup ("Feat/nemotron h lm head logprob cuda", PR #555
 * summary bullets: the untied embedding lookup of the same model row, with a
 * sorted-segment deterministic grad_weight; its Known issues: the pages'
 * version accumulates repeated ids in BF16 and misses FP64 parity, so here each
 * segment accumulates in fp32 and is rounded once).
 *
 *   out[i]    = weight[ids[i]]                        [N, D] x_dtype
 *   d_weight  = sum over i with ids[i] == v of grad[i], summed in ascending i
 *
 *   x_dtype   FLP_BF16, FLP_F16 or FLP_F32 (weight, out, grad); D * element
 *             size must be a multiple of 16.
 *   ids       [N] of id_dtype (FLP_I64 or FLP_I32).  An id outside [0, V)
 *             reads as a zero row and contributes no gradient.
 *   d_weight  [V, D] of dw_dtype (x_dtype or FLP_F32); every row is written
 *             (zero for ids that do not occur).
 *   workspace >= flp_embedding_backward_workspace_bytes(N, D, V): radix-sort
 *             buffers, per-id segment bounds and fp32 pieces of segments that
 *             span several 32-position groups of the sorted list.
 *
 * The backward sorts (id, token) pairs with a stable radix sort and sums each
 * id's segment in fp32 in a fixed order (token order inside each group of 32
 * sorted positions, groups in ascending order): d_weight is bitwise
 * reproducible.  N < 2^31,
 * V < 2^31 - 1.
 */
flp_status flp_embedding_forward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                 const void* weight, const void* ids, flp_dtype id_dtype,
                                 void* out, void* stream);
size_t flp_embedding_backward_workspace_bytes(int64_t N, int64_t D, int64_t V);
flp_status flp_embedding_backward(int64_t N, int64_t D, int64_t V, flp_dtype x_dtype,
                                  const void* grad, const void* ids, flp_dtype id_dtype,
                                  void* d_weight, flp_dtype dw_dtype, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Measurement probes (not part of the operator): the achievable dense bf16
 * MFMA rate and the shader clock it runs at, and the achievable streaming-read
 * bandwidth, so that figures can be quoted against measured peaks as well as
 * nominal ones.  Unlike every other call these synchronise `stream` and return
 * their results in host memory.
 *
 *   scratch        device buffer of >= flp_probe_scratch_bytes() bytes, 16-byte
 *                  aligned; contents undefined afterwards.
 *   flp_probe_mfma 2048 workgroups x 4 waves each run `iters` x 128
 *                  v_mfma_f32_16x16x32_bf16 on register operands (random bf16
 *                  values with |x| in [2^-7, 2), or zeros when zero_operands is
 *                  nonzero), timed by HIP events after one untimed launch;
 *                  *out_tflops = flops / time; *out_clock_ghz = median over
 *                  workgroups of shader-clock cycles / real-time ticks during
 *                  the loop x the real-time clock rate.  1 <= iters <= 10^6.
 *   flp_probe_read reads `bytes` (a multiple of 16, 16-byte aligned) of
 *                  `buffer` five times with streaming loads after one untimed
 *                  pass; *out_gbs = bytes read / time.
 */
size_t flp_probe_scratch_bytes(void);
flp_status flp_probe_mfma(int zero_operands, int64_t iters, void* scratch, size_t scratch_bytes,
                          double* out_tflops, double* out_clock_ghz, void* stream);
flp_status flp_probe_read(const void* buffer, size_t bytes, void* scratch, size_t scratch_bytes,
                          double* out_gbs, void* stream);

/*
 * Optional per-kernel timing with HIP events, for benchmarks.  While enabled,
 * every kernel the library enqueues is bracketed by two events recorded on
 * the same stream; flp_profile_read synchronises those events and returns, per
 * kernel kind, the summed duration in milliseconds and the launch count since
 * the previous read (then clears them).  Enabling it adds two event records
 * per kernel and nothing else; results are unaffected.  Process-wide, guarded
 * by a mutex.
 */
typedef enum flp_kernel_kind {
  FLP_K_FORWARD = 0,    /* logits tile + per-tile (max, sum of exp) + target logit */
  FLP_K_MERGE = 1,      /* fixed-tree merge of the tile partials -> lse, logp */
  FLP_K_DLOGITS = 2,    /* logits tile recompute -> dz, dz^T, d_bias partials */
  FLP_K_TRANSPOSE = 3,  /* W -> W^T, hidden chunk -> hidden^T (K-blocked) */
  FLP_K_DHIDDEN = 4,    /* d_hidden = dz W */
  FLP_K_DWEIGHT = 5,    /* d_weight (+)= dz^T hidden */
  FLP_K_DBIAS = 6,      /* ascending fold of the d_bias partials */
  FLP_K_LOGITS_FORWARD = 7,   /* flp_logits_forward */
  FLP_K_LOGITS_BACKWARD = 8,  /* flp_logits_backward */
  FLP_K_ROWS = 9,       /* indexed variants: row selection, gather, scatter */
  FLP_K_EMBEDDING = 10, /* flp_embedding_forward / flp_embedding_backward */
  FLP_K_COUNT = 11
} flp_kernel_kind;

void flp_profile_enable(int on);
/* ms[k] and count[k] for k < min(n, FLP_K_COUNT); returns FLP_HIP_ERROR if an
 * event query fails. */
flp_status flp_profile_read(double* ms, int64_t* count, int n);

/*
 * Static text for a status code.  Every unsupported case is reported as an
 * error, never served by another path: the fail-closed gates of PR #555
 * (summary bullets and "Acceptance checks").  Unknown codes give
 * "FLP_UNKNOWN_STATUS".  The string is owned by the library.
 */
const char* flp_status_string(flp_status status);

/*
 * Build provenance: library version, target architecture, git revision and the
 * kernel ids and tile shapes, plus "fallback=none" (this library has no
 * fallback path).  PR #555 (summary bullets, "Acceptance checks") records which
 * backend and kernels produced a result and that no fallback ran; this string
 * is that record for this library.  Static storage owned by the library.
 */
const char* flp_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* FLP_H_ */
