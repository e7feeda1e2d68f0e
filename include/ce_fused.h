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
  CE_ERR_HIP = 5           /* a HIP runtime call failed */
} ce_status;

/* Divide row r's gradient scale by the number of rows that carry r's segment
 * id (ignored rows included). Requires S > 0. */
#define CE_FLAG_SEGMENT_MEAN 0x1u

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

/* Device workspace (bytes) a call with this problem needs: zero without
 * segments, else room for a [T] float NLL staging array and [S+1] segment
 * offsets. Returns 0 for a null or invalid problem. */
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
 *  workspace     device buffer of at least ce_workspace_bytes(p) bytes (may be
 *                NULL when that is 0). Contents on entry do not matter.
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
                           void* workspace,
                           size_t workspace_bytes,
                           void* stream);

/* Static, human-readable name of a status code. */
const char* ce_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* CE_FUSED_H */
