/*
 * ce_fused.h - C ABI of the fused vocabulary cross-entropy (forward + backward)
 * for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every row r of a [T, V] logit matrix z with target
 * column t_r:
 *
 *   LSE_nt  = log sum_{j != t_r} exp(z_rj)           (target dropped before the sum)
 *   NLL_r   = softplus(LSE_nt - z_{r t_r})
 *   lse_r   = logaddexp(LSE_nt, z_{r t_r})            (the full logsumexp)
 *   loss_r  = NLL_r + z_alpha * lse_r^2
 *   grad_rj = s_r * (1 + 2 z_alpha lse_r) * exp(z_rj - lse_r)          j != t_r
 *   grad_rt = s_r * (-sigmoid(LSE_nt - z_t) + 2 z_alpha lse_r sigmoid(z_t - LSE_nt))
 *
 * with s_r = grad_scale, or grad_scale / (rows in r's segment) under
 * CE_FLAG_SEGMENT_MEAN. Sources: torchtitan PR #5661 "fix softmax collapse with
 * improved CE perf" (revised PR description, Numerics: the softplus NLL, the
 * target dropped before the non-target sum, the target gradient as minus the
 * non-target probability, ignored labels zeroed; approving review: backward
 * rebuilds the softmax, puts the target gradient in the target slot and scales
 * by the incoming gradient); Fast-LLM PR #552 "Fuse GSPO into the monolithic
 * compiled loss" (PR body: z-loss shares the vocabulary softmax with the CE;
 * the GSPO seam sums per-token values per segment over a per-batch number of
 * segments); xtuner PR #1963 "[FSDP][Loss] Switch gradient reduction to SUM"
 * (PR body: the global token mean is a caller scale, not a reduction inside
 * the loss). The z-loss form alpha * lse^2 is this library's reading; the
 * pages only say z-loss shares the softmax.
 *
 * Conventions
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library never frees or retains it. ``stream`` is a hipStream_t (NULL =
 *    the default stream).
 *  - The call is asynchronous: it validates on the host, enqueues its kernels
 *    on ``stream`` and returns without synchronising. It allocates nothing.
 *  - On any validation error it returns a ce_status != CE_OK and enqueues
 *    nothing. CE_ERR_HIP means a HIP call failed (no device, launch error).
 *  - Device-side conventions (never a trap): a valid row (target !=
 *    ignore_index and mask byte != 0) whose target lies outside [0, V) gets a
 *    NaN loss and a NaN gradient row. Unsorted segment ids give unspecified
 *    values (never an out-of-bounds access).
 *  - Results are bitwise reproducible run to run (no floating-point atomics).
 */
#ifndef CE_FUSED_H
#define CE_FUSED_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the logits and of the gradient. */
typedef enum ce_dtype {
  CE_DTYPE_F32 = 0,   /* IEEE binary32 */
  CE_DTYPE_BF16 = 1   /* bfloat16 (upper half of a binary32) */
} ce_dtype;

typedef enum ce_status {
  CE_OK = 0,
  CE_ERR_INVALID_ARG = 1,  /* null pointer, negative size, ld < V, bad dtype ... */
  CE_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
  CE_ERR_ALIAS = 3,        /* grad_out overlaps logits other than exactly in place */
  CE_ERR_WORKSPACE = 4,    /* workspace missing or smaller than ce_workspace_bytes() */
  CE_ERR_HIP = 5,          /* a HIP runtime call failed */
  CE_ERR_TIMEOUT = 6       /* CE_FLAG_VALIDATE only: a two-workgroup fp32 row gave up
                              waiting for its other half (that row's outputs are NaN) */
} ce_status;

/* Divide row r's gradient scale by the number of rows that carry r's segment
 * id (ignored rows included). Requires S > 0. */
#define CE_FLAG_SEGMENT_MEAN 0x1u

/* Debug check, for ce_fused_fwd_bwd and ce_fused_forward only. Before any
 * output is written, a device scan checks that every target is ignore_index
 * or in [0, V) and that segment ids are non-decreasing and in [0, S); the
 * call then waits for the stream (so it cannot be captured in a graph) and
 * returns CE_ERR_INVALID_ARG, with nothing else enqueued, if any check fails.
 * Without the flag an out-of-range target gives a NaN row and unsorted ids
 * are undefined. The scan's per-block results take 4096 bytes of workspace
 * (counted by ce_workspace_bytes). A gradient call on fp32 rows of
 * 102404..204803 columns (two workgroups per row, which exchange their
 * halves' statistics through the workspace with a bounded wait) also waits
 * for its kernels and returns CE_ERR_TIMEOUT if any half row stopped waiting
 * for its partner; such rows are NaN. The wait ends only when something
 * outside the call holds the partner workgroup off the GPU for well over
 * 0.1 s. Environment variable CE_PAIR_SPIN_LIMIT, when set to a number up
 * to 2097152, replaces that wait's poll limit (0: no wait at all, every such
 * row NaN); a test hook. */
#define CE_FLAG_VALIDATE 0x2u

/* Shape and options of one call. */
typedef struct ce_problem {
  int64_t T;              /* rows (T >= 0; T == 0 only writes seg_loss_out zeros) */
  int64_t V;              /* vocabulary columns (V >= 1) */
  int64_t ld_logits;      /* elements between consecutive logit rows (>= V) */
  int64_t ld_grad;        /* elements between consecutive gradient rows (>= V) */
  int32_t logits_dtype;   /* ce_dtype */
  int32_t grad_dtype;     /* ce_dtype; must equal logits_dtype when in place */
  int64_t ignore_index;   /* target value that marks an ignored row (e.g. -100) */
  int32_t num_segments;   /* S >= 0; S > 0 iff segment_ids != NULL (when T > 0) */
  uint32_t flags;         /* CE_FLAG_* */
} ce_problem;

/* Device workspace (bytes) a call with this problem needs: room for a [T]
 * float NLL staging array and [S+1] segment offsets when S > 0; for the
 * gradient pass's row scheduling, 256 bytes (a ticket counter) when rows
 * hold 8193..25600 16-byte chunks (bf16: 65544..204807 columns, fp32:
 * 32772..102403), and for fp32 logits of 102404..204803 columns (two
 * workgroups per row) 32 bytes per row plus 8 (the counter and a give-up
 * count); plus 4096 bytes
 * under CE_FLAG_VALIDATE; zero otherwise. This is what a call that
 * writes a gradient needs; a forward-only call (grad_out NULL, or
 * ce_fused_forward) needs no exchange slots, so it accepts a workspace
 * smaller by those bytes. Returns 0 for a null or invalid problem. */
size_t ce_workspace_bytes(const ce_problem* p);

/*
 * Fused forward + backward.
 *
 *  logits        [T, ld_logits] of logits_dtype, row-major. Read only, unless
 *                grad_out == logits (in place: same dtype and ld required).
 *                Ignored rows are never read.
 *  targets       [T] int64 target column per row; ignore_index marks an
 *                ignored row.
 *  mask          [T] uint8 or NULL; 0 marks an ignored row (ANDed with the
 *                ignore_index test).
 *  segment_ids   [T] int32, non-decreasing, values in [0, S); NULL iff S == 0
 *                (with T == 0 it is never read and may be NULL).
 *                targets, mask and segment_ids must stay unchanged until the
 *                call completes and must not overlap an output or the
 *                workspace (the kernels read them through the scalar cache);
 *                such an overlap is not detected.
 *  z_alpha       z-loss weight (0 disables it).
 *  grad_scale    upstream factor of the gradient (e.g. 1 / number of valid
 *                rows for a token mean).
 *  loss_out      [T] float: NLL_r + z_alpha lse_r^2 for valid rows, +0.0 for
 *                ignored rows. Required.
 *  seg_loss_out  [S] float or NULL: per segment, the sum of NLL_r over its
 *                valid rows (z-loss excluded); overwritten, never accumulated.
 *                Requires S > 0.
 *  grad_out      [T, ld_grad] of grad_dtype, or NULL for a forward-only call.
 *                Ignored rows are written as +0.0. May equal logits (in
 *                place); any other overlap with logits is CE_ERR_ALIAS.
 *  lse_out       [T] float or NULL: the full logsumexp lse_r of each valid
 *                row (the per-row statistic a separate backward would save:
 *                torchtitan PR #5661, revised PR description, Memory/perf),
 *                +0.0 for ignored rows, NaN for a valid row whose target is
 *                outside [0, V). Written by the same pass as loss_out (no
 *                extra read of the logits). May not overlap the logits
 *                (CE_ERR_ALIAS).
 *  workspace     device buffer of at least ce_workspace_bytes(p) bytes (may be
 *                NULL when that is 0). Contents on entry do not matter. The
 *                call uses it until it completes on the stream: calls that may
 *                run concurrently need workspaces of their own.
 *  stream        hipStream_t to enqueue on.
 */
ce_status ce_fused_fwd_bwd(const ce_problem* p,
                           const void* logits,
                           const int64_t* targets,
                           const uint8_t* mask,
                           const int32_t* segment_ids,
                           float z_alpha,
                           float grad_scale,
                           float* loss_out,
                           float* seg_loss_out,
                           void* grad_out,
                           float* lse_out,
                           void* workspace,
                           size_t workspace_bytes,
                           void* stream);

/*
 * ce_fused_fwd_bwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. It computes exactly what
 * ce_fused_fwd_bwd computes (the same kernels, bit for bit) and allocates
 * nothing: the workspace lives in a fixed device array of
 * CE_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU, reserved
 * when the library is loaded and held until the process ends. Its device
 * address is looked up on the first call on each device.
 *
 *  Arguments as for ce_fused_fwd_bwd, minus workspace / workspace_bytes.
 *  Returns CE_ERR_WORKSPACE when the call would need more than
 *  CE_NOALLOC_SCRATCH_BYTES (ce_workspace_bytes(p) for a gradient call; less
 *  without a gradient): with S segments, 4 T + 4 (S + 1) bytes (each rounded
 *  up to 256); with a gradient, 256 bytes for rows of 8193..25600 16-byte
 *  chunks, or 32 T + 8 bytes for the two-workgroup fp32 rows; 4096 more
 *  under CE_FLAG_VALIDATE. That is up to about 2 million rows with
 *  segments, or 262143 rows of the two-workgroup fp32 mode. CE_ERR_INVALID_ARG when the stream belongs to another device than
 *  the current one.
 *  Every call on one GPU shares that GPU's array and leaves the last call's
 *  contents in it: two calls that may run at the same time on one GPU (on
 *  different streams, or on one stream from different host threads without
 *  ordering) race on it and must not be issued; calls on one stream are
 *  ordered and safe. Nothing in it needs clearing between calls (every
 *  kernel writes what it later reads).
 */
#define CE_NOALLOC_SCRATCH_BYTES (8u << 20)

ce_status ce_fused_fwd_bwd_noalloc(const ce_problem* p,
                                   const void* logits,
                                   const int64_t* targets,
                                   const uint8_t* mask,
                                   const int32_t* segment_ids,
                                   float z_alpha,
                                   float grad_scale,
                                   float* loss_out,
                                   float* seg_loss_out,
                                   void* grad_out,
                                   float* lse_out,
                                   void* stream);

/*
 * Forward only, with per-row statistics a caller may want from the same read
 * of the logits: the full logsumexp and the entropy of the row's softmax.
 * torchtitan PR #5661 "fix softmax collapse with improved CE perf" (fourth
 * review, inline diff) keeps the input logits unmodified because callers
 * reuse them for such quantities, entropy named among them; this entry
 * computes them in the loss pass instead of a second read.
 *
 *  p, logits, targets, mask, segment_ids, z_alpha, loss_out, seg_loss_out,
 *  workspace, stream: as for ce_fused_fwd_bwd (p->grad_dtype and p->ld_grad
 *                are not used; the logits are never written).
 *  lse_out       [T] float or NULL: logsumexp_j z_j (all columns) of valid
 *                rows, +0.0 for ignored rows, NaN for a valid row whose
 *                target is outside [0, V).
 *  entropy_out   [T] float or NULL: -sum_j p_j ln p_j of the row's softmax
 *                (0 ln 0 = 0), formed without cancellation: the target's
 *                term as p_t NLL_r, every other term as p_j (lse - z_j) >= 0.
 *                +0.0 for ignored rows, NaN for out-of-range targets.
 *  Neither output may overlap the logits (CE_ERR_ALIAS).
 */
ce_status ce_fused_forward(const ce_problem* p,
                           const void* logits,
                           const int64_t* targets,
                           const uint8_t* mask,
                           const int32_t* segment_ids,
                           float z_alpha,
                           float* loss_out,
                           float* seg_loss_out,
                           float* lse_out,
                           float* entropy_out,
                           void* workspace,
                           size_t workspace_bytes,
                           void* stream);

/*
 * Cross-entropy + z-loss with a distillation child on the same softmax pass.
 *
 * Fast-LLM PR #552 "Fuse GSPO into the monolithic compiled loss" (PR body,
 * What) names distillation with CE and z-loss among the losses that share
 * the vocabulary softmax and finish loss and gradient in one pass. The
 * pages give no formula; this library's reading is the forward KL divergence
 * from the teacher's softmax to the student's, per valid row:
 *   loss_r = NLL_r + z_alpha lse_r^2 + kl_beta KL(softmax(y_r) || softmax(z_r))
 *   grad_r = s (1 + 2 z_alpha lse_r + kl_beta) softmax(z_r) - s kl_beta softmax(y_r)
 * with the target column formed from the non-target logsumexps (revised PR
 * description of torchtitan #5661, Numerics):
 *   grad_rt = s (-pS_nt + 2 z_alpha lse_r pS_t + kl_beta (pT_nt - pS_nt)).
 *
 *  p             as for ce_fused_fwd_bwd: the student logits' shape, strides
 *                and dtypes, ignore_index; num_segments must be 0
 *                (CE_ERR_UNSUPPORTED otherwise) and flags 0.
 *  logits        [T, ld_logits] student logits (differentiated).
 *  teacher       [T, ld_teacher] of teacher_dtype (CE_DTYPE_F32 or
 *                CE_DTYPE_BF16), read only; never written.
 *  targets, mask, z_alpha, grad_scale: as for ce_fused_fwd_bwd.
 *  kl_beta       weight of the KL term (0: the gradient does not read the
 *                teacher; the forward still does, for kl_out).
 *  loss_out      [T] float, required; kl_out [T] float or NULL: KL_r.
 *                Ignored rows +0.0; a valid row whose target is outside
 *                [0, V) gets NaN in both and a NaN gradient row.
 *  grad_out      [T, ld_grad] or NULL (forward only); may equal logits (in
 *                place, same dtype and stride); may not overlap teacher.
 * One pass over both matrices computes the statistics; the gradient pass
 * reads them again. Asynchronous, deterministic, allocates nothing.
 */
ce_status ce_fused_distill(const ce_problem* p,
                           const void* logits,
                           const void* teacher,
                           int64_t ld_teacher,
                           int32_t teacher_dtype,
                           const int64_t* targets,
                           const uint8_t* mask,
                           float z_alpha,
                           float kl_beta,
                           float grad_scale,
                           float* loss_out,
                           float* kl_out,
                           void* grad_out,
                           void* stream);

/*
 * Split form: statistics over column shards, a per-row finish, and a
 * gradient pass from saved per-row state.
 *
 * This is the vocabulary-parallel layout of torchtitan PR #5661 "fix softmax
 * collapse with improved CE perf" (third review, inline diff: each rank
 * reduces its [T, V_local] shard, the target logit comes from the rank that
 * owns the target column, and the per-row statistics are combined across
 * ranks) and its final recompute design (approving review, "What this PR
 * does": forward saves the input logits and per-row statistics; backward
 * rebuilds the softmax, puts the precomputed target gradient in the target
 * slot and scales by the incoming gradient). Fast-LLM PR #552 (PR body,
 * Approach) shares one softmax pass plus its tensor-parallel reduction the
 * same way. With one shard it is a forward/backward split of
 * ce_fused_fwd_bwd: ce_shard_stats + ce_rows_finish forward,
 * ce_shard_grad backward.
 */

/* A column shard: columns [v0, v0 + V) of a vocabulary of V_total columns
 * (V_total is the ce_problem V given to ce_rows_finish). */
typedef struct ce_shard {
  int64_t T;              /* rows (T >= 0) */
  int64_t V;              /* columns held by this shard (V >= 1) */
  int64_t v0;             /* global index of the shard's first column (>= 0) */
  int64_t ld_logits;      /* elements between consecutive rows of the shard (>= V) */
  int64_t ld_grad;        /* elements between consecutive gradient rows (>= V) */
  int32_t logits_dtype;   /* ce_dtype */
  int32_t grad_dtype;     /* ce_dtype (gradient pass only) */
  int64_t ignore_index;
} ce_shard;

/*
 * Pass 1 over a shard. For each row, stats[3 r .. 3 r + 2] =
 *   (m, s, z): with the shard's non-target columns j (the target column is
 *   excluded when the shard holds it), s = sum_j 2^(z_j log2(e) - m) for a
 *   float shift m in log2 units (m = -inf, s = 0 when no column remains);
 *   z = the target logit when the shard holds the target column, else -inf.
 * Ignored rows (target == ignore_index, or mask byte 0) get (-inf, 0, -inf)
 * and are not read. stats is a device [T, 3] float array.
 */
ce_status ce_shard_stats(const ce_shard* s, const void* logits, const int64_t* targets,
                         const uint8_t* mask, float* stats, void* stream);

/*
 * Per-row finish over num_shards shards whose statistics are stored
 * back to back in stats ([num_shards, T, 3], shard order). p gives T, the
 * full vocabulary V, ignore_index, num_segments and flags (strides and
 * dtypes are unused). Writes loss_out[T] and seg_loss_out[S] exactly as
 * ce_fused_fwd_bwd does, and the saved per-row state row_state[T, 8]:
 *   [0] lse * log2(e)
 *   [1] p_nt = sigmoid(LSE_nt - z_t)      (probability off the target)
 *   [2] p_t  = sigmoid(z_t - LSE_nt)      (target probability)
 *   [3] 2 z_alpha lse                    (z-loss gradient factor)
 *   [4] f_r = 1 / segment length under CE_FLAG_SEGMENT_MEAN, else 1
 *   [5] kind: 0 valid, 1 ignored, 2 poisoned (target outside [0, V): NaN loss)
 *   [6..7] 0.
 * The merge runs in fp64 in shard order (deterministic). workspace: with
 * segments, the [T] NLL staging array and [S+1] offsets (ce_workspace_bytes
 * of the same p is always enough); may be NULL without segments.
 */
ce_status ce_rows_finish(const ce_problem* p, int32_t num_shards, const float* stats,
                         const int64_t* targets, const uint8_t* mask,
                         const int32_t* segment_ids, float z_alpha, float* loss_out,
                         float* seg_loss_out, float* row_state, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Pass 2 over a shard from the saved row state. With w_r the weight of row
 * r's NLL term -- row_weight[r] when row_weight is given, else
 * grad_scale * f_r -- and u_r = grad_scale * f_r the weight of its z-loss
 * term, the gradient is
 *   g_rj = (w_r + u_r 2 z_alpha lse) exp(z_rj - lse)          j != t
 *   g_rt = -w_r p_nt + u_r 2 z_alpha lse p_t,
 * so with row_weight == NULL it equals ce_fused_fwd_bwd's gradient.
 * row_weight lets per-row weights chosen after the forward -- the seam of a
 * GSPO/GRPO-style loss that shares this softmax, Fast-LLM PR #552 "Fuse GSPO
 * into the monolithic compiled loss" (PR body, Approach: a deferred child
 * whose backward runs after an eager per-segment step) -- scale the NLL
 * gradient row by row. Ignored rows are +0.0 and poisoned rows NaN without
 * reading the logits. grad_out may equal logits (in place, same dtype and
 * ld); any other overlap is CE_ERR_ALIAS.
 */
ce_status ce_shard_grad(const ce_shard* s, const void* logits, const int64_t* targets,
                        const float* row_state, const float* row_weight, float grad_scale,
                        void* grad_out, void* stream);

/*
 * The loss behind a linear LM head, with the logits never stored whole.
 *
 * The logits are z = X W^T for hidden states X [T, H] and the head's weight W
 * [V, H] (one row per vocabulary entry), both bf16; the per-row loss, z-loss,
 * ignore rules and scales are those of ce_fused_fwd_bwd (the collapse-free
 * loss of torchtitan PR #5661, revised PR description, Numerics). Fast-LLM PR
 * #552 (PR body, the LM-head layer tests) puts the loss directly after such a
 * head; fusing the head's product into the loss is this library's design, not
 * the pages'. Forward: logit tiles are formed on the matrix cores and reduced
 * to per-row statistics over vocabulary ranges, merged as by ce_rows_finish.
 * Backward (dhidden or dweight given): per chunk of chunk_cols vocabulary
 * columns the logit tiles of every row are recomputed and turned into dL/dz
 * (bf16, one chunk at a time in the workspace), then the chunk's rows of
 * dW = G^T X and its share of dX = sum over chunks of G W_chunk.
 *
 *  T, V, H       rows, vocabulary size, hidden size (H a multiple of 8).
 *  ld_hidden     elements between rows of hidden (>= H, multiple of 8).
 *  ld_weight     elements between rows of weight (>= H, multiple of 8).
 *  ignore_index  target value of an ignored row.
 *  dhidden_dtype CE_DTYPE_F32 or CE_DTYPE_BF16.
 *  chunk_cols    vocabulary columns per backward chunk (0: 8192); rounded
 *                up to 256. The workspace grows with it (about 4 T chunk_cols
 *                bytes, plus 2 H T for X^T and 4 H T for a bf16 dX's fp32
 *                accumulator).
 */
typedef struct ce_lmhead {
  int64_t T;
  int64_t V;
  int64_t H;
  int64_t ld_hidden;
  int64_t ld_weight;
  int64_t ignore_index;
  int32_t dhidden_dtype;
  int32_t chunk_cols;
} ce_lmhead;

/* Device workspace (bytes) of ce_lmhead_fwd_bwd: forward only (backward ==
 * 0) or with a backward. 0 for a null or invalid problem. */
size_t ce_lmhead_workspace_bytes(const ce_lmhead* p, int32_t backward);

/*
 *  hidden        [T, ld_hidden] bf16, 16-byte aligned. Read only.
 *  weight        [V, ld_weight] bf16, 16-byte aligned. Read only.
 *  targets, mask, z_alpha, grad_scale: as for ce_fused_fwd_bwd.
 *  loss_out      [T] float, as for ce_fused_fwd_bwd. Required.
 *  lse_out       [T] float or NULL: full logsumexp (0 ignored, NaN poisoned).
 *  dhidden       [T, H] (contiguous) of dhidden_dtype or NULL: dL/dX.
 *  dweight       [V, H] float (contiguous) or NULL: dL/dW, overwritten.
 *  workspace     at least ce_lmhead_workspace_bytes(p, dhidden || dweight)
 *                bytes, 256-byte aligned; contents on entry do not matter.
 * Here L = sum_r s_r loss_r over valid rows. A valid row with a target outside
 * [0, V) gives a NaN loss, a NaN dX row and NaN in every dW element (its
 * gradient row enters every column sum). Outputs may not overlap the inputs
 * or the workspace (CE_ERR_ALIAS). Unaligned operands, H % 8 != 0 or a
 * product of more than 2^31 - 1 256 x 256 tiles return CE_ERR_UNSUPPORTED; a
 * failed launch or device query returns CE_ERR_HIP. The call is asynchronous
 * and deterministic.
 */
ce_status ce_lmhead_fwd_bwd(const ce_lmhead* p, const void* hidden, const void* weight,
                            const int64_t* targets, const uint8_t* mask, float z_alpha,
                            float grad_scale, float* loss_out, float* lse_out, void* dhidden,
                            float* dweight, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Static, human-readable name of a status code. */
const char* ce_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CE_FUSED_H */
