/*
 * lce.h - strip-wise linear cross-entropy on AMD CDNA4 (gfx950).
 *
 * Computes loss = CE(h . W^T, targets) and its gradients for hidden states
 * h [N, H] and a projection weight W [V, H] without ever holding the N x V
 * logits.  This is the loss primitive that the page "Running 128K-Sequence MoE
 * RL on 32 H100s" calls Linear CE (section "Linear CE: Avoiding
 * Materialization of Full Logits"), computed the way the page "Flattening
 * Every Memory Peak in Long-Context Mixture-of-Experts Training" describes for
 * Ring-DTP on one device's share (section 3.2 and appendix C): each logit strip
 * h . W[v0:v0+Vs]^T is folded into a running per-token state (max, sum of
 * exponentials, target logit) and released; the backward pass recomputes each
 * strip, forms G = grad_scale * (softmax - onehot) for it, and feeds
 * dH += G . W_strip and dW_strip = G^T . h.  Section 2 of the second page
 * fixes the contract: forward values and gradients equal those of the dense
 * implementation up to the order of floating-point operations.
 *
 * Conventions for every call
 *  - All tensors are dense row-major and live in device memory, unless stated.
 *    hidden [N, H] and weight rows [*, H] have the element type of `dtype`;
 *    targets are int32 [N]; every float output is float32.
 *  - Device pointers must be 16-byte aligned.  H must be a multiple of 8 for
 *    bf16 and of 4 for f32 (LCE_ERR_UNSUPPORTED otherwise).
 *  - The library never allocates device memory.  The caller passes a
 *    workspace of at least lce_workspace_bytes(p) bytes; it is scratch, its
 *    contents are not kept between calls, and two calls that run at the same
 *    time need two workspaces.
 *  - Work is enqueued on `stream` and is asynchronous: no call waits for the
 *    device.  Argument errors are detected on the host and returned before
 *    anything is enqueued.  A failed kernel launch returns LCE_ERR_LAUNCH.
 *  - A non-ignored target outside [0, V) is a precondition violation: the
 *    kernels stay memory-safe (targets are compared, never used as
 *    addresses) and that row's loss, and so the reduced loss, is NaN.
 */
#ifndef LCE_H
#define LCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum lce_status {
  LCE_OK = 0,
  LCE_ERR_INVALID_VALUE = 1, /* null pointer, size <= 0, bad enum, strip range */
  LCE_ERR_UNSUPPORTED = 2,   /* H not a multiple of the 16-byte chunk */
  LCE_ERR_WORKSPACE = 3,     /* workspace null or smaller than lce_workspace_bytes */
  LCE_ERR_LAUNCH = 4         /* a kernel launch failed (hipGetLastError) */
} lce_status_t;

typedef enum lce_dtype { LCE_F32 = 0, LCE_BF16 = 1 } lce_dtype_t;

typedef enum lce_reduction {
  LCE_MEAN = 0, /* sum of row losses / number of non-ignored rows (NaN if none) */
  LCE_SUM = 1   /* sum of row losses */
} lce_reduction_t;

/* The problem: sizes, element type, reduction and strip width.
 * strip (Vs) is the widest vocabulary slice folded per step; it fixes the
 * workspace size.  0 selects lce_pick_strip(p, LCE_DEFAULT_BUDGET). */
typedef struct lce_problem {
  int64_t n_tokens;     /* N in [1, 2^31] */
  int64_t hidden;       /* H in [1, 2^20] */
  int64_t vocab;        /* V in [1, 2^31] */
  int64_t strip;        /* Vs in [1, min(V, 2^21)], or 0 */
  int32_t dtype;        /* lce_dtype_t of hidden and weight */
  int32_t reduction;    /* lce_reduction_t */
  int32_t ignore_index; /* rows with this target are left out */
  int32_t reserved;     /* must be 0 */
} lce_problem_t;

#define LCE_DEFAULT_BUDGET ((size_t)2 << 30) /* 2 GiB of workspace */

/* Human-readable name of a status code (static storage). */
const char* lce_status_string(lce_status_t s);

/* Widest strip width Vs whose workspace (lce_workspace_bytes of the problem
 * with that strip) fits in budget_bytes: a multiple of 256 (the kernels'
 * vocabulary tile), at most V rounded up to 256 and at most 2^21, then
 * clamped to V.  The workspace counted is the whole of it - the backward's
 * gradient strip, or, for a handful of tokens, the forward's partials and
 * running state when they are larger, plus the header - so the returned
 * width's workspace never exceeds the budget.  Returns -1 when not even a
 * 256-wide strip fits, and for an invalid problem; p->strip is ignored.
 * (A problem with strip = 0 then uses 256, or V if smaller, whatever its
 * workspace.)  Follows from the second page's sections 3.5 and 6: a
 * device's working set is fixed by the launch configuration and can be
 * checked before launch. */
int64_t lce_pick_strip(const lce_problem_t* p, size_t budget_bytes);

/* Workspace bytes needed by every call below for problem p (with its strip,
 * or the default policy when p->strip == 0): one gradient strip of
 * round_up(N, 16) x round_up(Vs, 256) elements (bf16 strips are kept in
 * blocks of 16 tokens) plus a 256-byte header (the forward keeps its
 * partials and running state inside the strip region; for a handful of tokens
 * those are larger than the strip and set the size).  This is the extra
 * device memory of the whole path: the second page's section 3.2 bounds the
 * projection's working set by one logit strip instead of the N x V logits,
 * and its section 2 asks that the bound hold in the backward pass too, which
 * recomputes strips into this same region.
 * Returns 0 for an invalid problem. */
size_t lce_workspace_bytes(const lce_problem_t* p);

/* Widest vocabulary range one forward fold (lce_forward_fold and its steps
 * call) may take: at least Vs, and as many rows as the workspace's partials
 * hold beside the running state (8 bytes per token and 128 rows), at most
 * 2^21 and at most V.  lce_forward folds in ranges of this width.  Returns -1
 * for an invalid problem. */
int64_t lce_forward_fold_max(const lce_problem_t* p);

/* Forward: loss[0] (float32, device), lse[N] (log-sum-exp of every row,
 * needed by lce_backward) and, if row_loss != NULL, row_loss[N] (0 for
 * ignored rows).  This is the forward half of the first page's Linear CE
 * (section "Linear CE: Avoiding Materialization of Full Logits"): the loss of
 * the vocabulary projection without the logits tensor.  The vocabulary is
 * folded in natural order into the running per-token state of the second
 * page's section 3.2 (max, sum of exponentials, target logit).  Equivalent to
 * lce_forward_begin + lce_forward_fold over consecutive ranges of
 * lce_forward_fold_max(p) rows + lce_forward_end: the forward keeps only 8
 * bytes of partial state per token and 128 vocabulary rows, so the workspace
 * holds those of about 32 strips (bf16; 64 for f32) and each fold takes as
 * many.  Results agree with strip-by-strip calls up to the order of
 * floating-point operations (the second page's section 2). */
lce_status_t lce_forward(const lce_problem_t* p, const void* hidden, const void* weight,
                         const int32_t* targets, float* loss, float* lse, float* row_loss,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Backward: d_hidden [N, H] and d_weight [V, H] (float32, fully overwritten)
 * of grad_out[0] * loss.  lse is the forward's output; grad_out is a device
 * scalar.  Ignored rows get zero d_hidden rows and add nothing to d_weight.
 * The second page's section 3.2: the backward recomputes each strip's logits
 * and forms their gradient strip by strip (G = scale * (softmax - onehot),
 * dH += G . W_strip, dW_strip = G^T . h), so the logit gradients never exist
 * for the whole vocabulary either.  Equivalent to lce_backward_begin + one
 * lce_backward_fold per strip of Vs rows in natural order. */
lce_status_t lce_backward(const lce_problem_t* p, const void* hidden, const void* weight,
                          const int32_t* targets, const float* lse, const float* grad_out,
                          float* d_hidden, float* d_weight, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/* ---- Strip-level calls: the caller chooses the strips and their order ----
 * One fold is one meeting of the token batch with one vocabulary shard in the
 * second page's Ring-DTP (appendix C): any order that visits every vocabulary
 * row exactly once gives the same result up to rounding.  weight_strip points
 * at row v_begin of the weight (v_len rows of H elements), 1 <= v_len <= Vs
 * (backward) or lce_forward_fold_max(p) (forward), and
 * 0 <= v_begin, v_begin + v_len <= V. */

/* Reset the running per-token state (max = -inf, sum = 0, target logit = NaN). */
lce_status_t lce_forward_begin(const lce_problem_t* p, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Fold the logits of vocabulary rows [v_begin, v_begin + v_len) into the
 * state; v_len may be up to lce_forward_fold_max(p) (>= Vs) rows. */
lce_status_t lce_forward_fold(const lce_problem_t* p, const void* hidden,
                              const void* weight_strip, int64_t v_begin, int64_t v_len,
                              const int32_t* targets, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Turn the state into lse[N], optional row_loss[N] and the reduced loss[0]. */
lce_status_t lce_forward_end(const lce_problem_t* p, const int32_t* targets, float* loss,
                             float* lse, float* row_loss, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);

/* ---- Merging running states: a vocabulary split across devices ----
 * When every device holds the whole token batch and one vocabulary shard
 * (the vocabulary-parallel reduction that the second page's section 5
 * contrasts with Ring-DTP, and the vocab_partition of the first page's
 * full-logits formula), each device folds its shard into its own running
 * state, and the states are combined token by token: (max, sum of
 * exponentials) by the associative log-sum-exp merge, the target logit from
 * the shard that holds the target.  These two calls export a state and fold
 * an exported one into a workspace, so that states can be exchanged between
 * devices (an all-gather, a ring) and merged before lce_forward_end.  The
 * backward pass then needs no exchange but the sum of the devices'
 * d_hidden: each device runs lce_backward_begin and lce_backward_fold over
 * its own shard with the merged lse. */

/* Copy the workspace's running state to state[3 * N] (float32): row 0 the
 * per-token max, row 1 the sum of exp(z - max), row 2 the target logit (NaN
 * while the target has not been folded). */
lce_status_t lce_forward_state(const lce_problem_t* p, float* state, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* Fold a state written by lce_forward_state, for the same tokens and a part of
 * the vocabulary disjoint from the one already folded here, into the
 * workspace's running state (a target logit is taken from whichever side has
 * one; with both, this side's is kept). */
lce_status_t lce_forward_merge_state(const lce_problem_t* p, const float* state, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* Count the non-ignored rows and form the per-row gradient scale from the
 * device scalar grad_out (grad_out / n_valid for mean, grad_out for sum),
 * kept in the workspace header for the folds that follow.  This is the
 * factor grad_out * d loss / d row_loss of the dense loss that the second
 * page's section 2 asks the gradients to reproduce: a row whose target is
 * ignore_index gets 0, and the mean divides by the non-ignored rows. */
lce_status_t lce_backward_begin(const lce_problem_t* p, const int32_t* targets,
                                const float* grad_out, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/* Bits of the `accumulate` argument of the backward folds. */
typedef enum lce_accumulate {
  LCE_ACC_NONE = 0,
  LCE_ACC_DHIDDEN = 1, /* d_hidden += G . W_strip instead of = */
  LCE_ACC_DWEIGHT = 2  /* d_weight_strip += G^T . h instead of = */
} lce_accumulate_t;

/* Recompute the strip, form its logit gradient G in the workspace, then
 * d_hidden (+)= G . W_strip and d_weight_strip[v_len, H] (+)= G^T . h, each
 * added to the buffer's contents where its bit of `accumulate` is set
 * (lce_accumulate_t) and overwriting them otherwise; any other bit is
 * LCE_ERR_INVALID_VALUE.  The first fold of a backward pass clears
 * LCE_ACC_DHIDDEN.  LCE_ACC_DWEIGHT serves the second page's Ring-DTP
 * (section 3.2, appendix C), where one vocabulary shard meets the distinct
 * batches of several ranks: its weight gradient is the sum of the gradients
 * of those meetings, and each meeting after the first adds to it. */
lce_status_t lce_backward_fold(const lce_problem_t* p, const void* hidden,
                               const void* weight_strip, int64_t v_begin, int64_t v_len,
                               const int32_t* targets, const float* lse, float* d_hidden,
                               int accumulate, float* d_weight_strip, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* ---- Backward with no workspace argument ----
 * For callers that cannot allocate device memory (code under stream capture,
 * tight serving loops, harnesses that forbid allocation): lce_backward with
 * its workspace taken from a static device array of LCE_STATIC_SCRATCH_BYTES
 * inside the library instead of the caller.  Each GPU the library runs on
 * holds its own copy of that array from the first call on it until the
 * process ends; the call itself allocates nothing.  Problems whose
 * lce_workspace_bytes exceeds LCE_STATIC_SCRATCH_BYTES are rejected with
 * LCE_ERR_WORKSPACE before anything is enqueued (choose a narrower strip,
 * e.g. lce_pick_strip(p, LCE_STATIC_SCRATCH_BYTES)).  Every call on one GPU
 * uses the same array: two calls that can overlap on one GPU (different
 * streams, or different host threads) race and must be serialised by the
 * caller.  The array keeps the previous call's contents; the backward writes
 * every byte it reads, so nothing needs clearing.  LCE_ERR_LAUNCH also
 * reports a failed lookup of the array's device address.  Arguments and
 * results are otherwise those of lce_backward. */
#define LCE_STATIC_SCRATCH_BYTES ((size_t)256 << 20) /* 256 MiB per GPU */

lce_status_t lce_backward_static(const lce_problem_t* p, const void* hidden, const void* weight,
                                 const int32_t* targets, const float* lse, const float* grad_out,
                                 float* d_hidden, float* d_weight, hipStream_t stream);

/* ---- Backward without a strip buffer ----
 * The fused alternative that the second page's section 5 sets beside
 * Ring-DTP (cross-entropy kernels that keep the logit gradient out of memory
 * for a batch resident on one device): the gradient G is formed one
 * 256 x 256 (token x vocabulary) tile at a time and multiplied at once into
 * the rows of d_hidden and d_weight that tile feeds, so no strip of G exists.
 * Each tile's logits are recomputed as in section 3.2 of that page.
 *   LCE_FUSED_ONE_SWEEP: every tile is visited once and feeds both
 *     gradients (6 N H V multiply-adds of the backward, as the strip path).
 *     The device is shared out as a grid of token groups x vocabulary groups;
 *     each group's contribution goes to its own fp32 partial copy of d_hidden
 *     (one per vocabulary group) and of d_weight (one per token group), and
 *     the copies are summed in a fixed order afterwards.
 *   LCE_FUSED_TWO_SWEEPS: a first sweep forms d_hidden with each token group
 *     owning its rows, a second sweep recomputes every tile and forms
 *     d_weight with each vocabulary group owning its rows (8 N H V: the
 *     logits are formed twice), so partial copies appear only when the
 *     device has more compute units than a dimension has tiles.
 * Both are deterministic (fixed order of additions, no atomics).  The
 * workspace is lce_backward_fused_workspace_bytes(p, mode): a 256-byte
 * header, one G tile per block (128 KiB for bf16) and the partial copies.
 * Arguments and results are otherwise those of lce_backward; H must be a
 * multiple of 4.  The strip path (lce_backward) stays the default: its
 * workspace is one strip, and at the pages' sizes the partial copies of the
 * one-sweep form exceed it (they grow with H, a strip does not). */
typedef enum lce_fused_mode { LCE_FUSED_ONE_SWEEP = 1, LCE_FUSED_TWO_SWEEPS = 2 } lce_fused_mode_t;

/* Workspace bytes of lce_backward_fused for problem p and mode; 0 if invalid. */
size_t lce_backward_fused_workspace_bytes(const lce_problem_t* p, int mode);

lce_status_t lce_backward_fused(const lce_problem_t* p, const void* hidden, const void* weight,
                                const int32_t* targets, const float* lse, const float* grad_out,
                                float* d_hidden, float* d_weight, int mode, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ---- The steps of one fold, one kernel each ----
 * lce_forward_fold and lce_backward_fold run every step of their fold in
 * order; the calls below run only the steps named in `steps` (a bit set of
 * lce_step_t), so that a caller can time each kernel on its stream, as the
 * first page's paired test does for time next to loss, gradient and peak
 * (section 8, "Paired Testing").  Running the steps of a fold in order in
 * separate calls is the same computation as one fold call.
 *   forward:  LCE_STEP_STRIP - logits of the strip and their per-token
 *             (max, sum of exp) partials plus the target logit, in registers;
 *             LCE_STEP_MERGE - fold the partials into the running state.
 *   backward: LCE_STEP_GRAD - recompute the strip and write its G;
 *             LCE_STEP_DHIDDEN - d_hidden (+)= G . W_strip;
 *             LCE_STEP_DWEIGHT - d_weight_strip = G^T . h. */
typedef enum lce_step {
  LCE_STEP_STRIP = 1,
  LCE_STEP_MERGE = 2,
  LCE_STEP_GRAD = 1,
  LCE_STEP_DHIDDEN = 2,
  LCE_STEP_DWEIGHT = 4,
  LCE_STEP_ALL = 7
} lce_step_t;

/* How a backward fold of v_len rows launches its two output GEMMs on the
 * current device: 2 for two launches (d_hidden, then d_weight_strip), 1 for
 * one launch that shares the compute units between them (taken when one of
 * the two alone has too few tiles to fill the device).  Lets a caller that
 * times each step match the launches the whole fold makes.  -1 for an
 * invalid problem or v_len outside [1, Vs]. */
int lce_backward_fold_gemm_launches(const lce_problem_t* p, int64_t v_len);

lce_status_t lce_forward_fold_steps(const lce_problem_t* p, const void* hidden,
                                    const void* weight_strip, int64_t v_begin, int64_t v_len,
                                    const int32_t* targets, void* workspace,
                                    size_t workspace_bytes, unsigned steps, hipStream_t stream);

lce_status_t lce_backward_fold_steps(const lce_problem_t* p, const void* hidden,
                                     const void* weight_strip, int64_t v_begin, int64_t v_len,
                                     const int32_t* targets, const float* lse, float* d_hidden,
                                     int accumulate, float* d_weight_strip, void* workspace,
                                     size_t workspace_bytes, unsigned steps, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H */
