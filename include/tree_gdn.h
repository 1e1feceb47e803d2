/*
 * tree_gdn.h -- C ABI of the tree conv + tree Gated DeltaNet library (forward and
 * backward), with a tree Mamba2 (SSD) forward beside it,
 * for AMD Instinct MI355X (gfx950).
 *
 * The library runs the forward pass of a recurrent mixer over a prefix trie
 * whose segments are packed one after another (depth-first order, "Tree
 * Training: Accelerating Agentic LLMs Training via Shared Prefix Reuse",
 * arXiv 2511.00413, section 3.1 Eq. 8):
 *
 *   - tree_conv: a short causal depthwise conv1d in which every segment reads
 *     the last W-1 inputs of its own root-to-segment path (same paper,
 *     section 3.2 "Causal convolution", Eq. 11; tree-recurrence 0.1.0 project
 *     page, "How a tree runs": a single conv launch covers every segment,
 *     each one given the inputs that precede it on its path).
 *   - tree_gdn_scan: a chunked gated delta rule in which every segment starts
 *     from the final state of its parent segment and a root from zero (same
 *     paper, section 3.2 "SSM Layers (GDN)", Eq. 10; appendix A.2), so
 *     sibling branches never see each other's state.  Per value head, with
 *     a_t = exp(g_t):
 *         S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
 *         o_t = scale * S_t q_t.
 *
 * Every token's result equals the one a standalone forward over its own
 * root-to-leaf path produces (same paper, section 3.1 Eq. 6).
 *
 * Conventions
 *   - All functions return 0 (TREE_OK) or a negative TREE_ERR_* code; no
 *     exception crosses the ABI.  tree_last_error() gives a message for the
 *     last failure on the calling thread.
 *   - Arguments are validated before any device work is enqueued; on failure
 *     nothing is written.  That includes the device plan `dplan`: an entry
 *     point accepts only a buffer that tree_plan_upload filled from the same
 *     plan, with dplan_bytes >= tree_plan_device_bytes(plan) and no larger
 *     than the size it was uploaded with; any other pointer is rejected
 *     (INVALID_ARG, or WORKSPACE when dplan_bytes is too small).  The record
 *     lives as long as the plan: free a dplan buffer only after the plan.
 *   - "device" pointers are HIP device memory owned by the caller.  The
 *     library never allocates or frees device memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device
 *     work is asynchronous and stream-ordered; buffers must stay alive until
 *     the stream reaches the work.  Device faults surface at the caller's
 *     next synchronisation.
 *   - Tensors are packed token-major in segment order (token t of segment s
 *     is row seg_off[s] + t).
 */
#ifndef TREE_GDN_H
#define TREE_GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TREE_OK 0
#define TREE_ERR_INVALID_ARG (-1) /* null pointer, bad enum, bad dimension      */
#define TREE_ERR_BAD_TREE (-2)    /* parent not in [-1, i), length <= 0, n <= 0  */
#define TREE_ERR_SIZE (-3)        /* n_tokens differs from the plan's token count */
#define TREE_ERR_UNSUPPORTED (-4) /* head size / dtype / width not compiled in   */
#define TREE_ERR_WORKSPACE (-5)   /* device plan or workspace too small          */
#define TREE_ERR_HIP (-6)         /* a HIP runtime call failed                   */

#define TREE_DTYPE_F32 0
#define TREE_DTYPE_BF16 1

#define TREE_ACT_NONE 0
#define TREE_ACT_SILU 1

/* Scan schedules (tree-recurrence 0.1.0 project page, "How a tree runs": a
 * tree scan either forks or rescans).  Both give bitwise the same outputs and
 * states: the chunks are segment-local either way and the state handed from
 * a segment to its child is the same fp32 value. */
#define TREE_SCHED_LEVEL 0  /* fork: one launch per trie level, each segment
                               starting from its parent's final state; stream
                               order is the barrier between levels            */
#define TREE_SCHED_RESCAN 1 /* rescan: one launch over every root-to-leaf
                               path, the state carried from segment to
                               segment in registers; shared prefixes are
                               scanned once per path through them and each
                               segment's outputs and state are written by one
                               of those paths                                 */
#define TREE_SCHED_AUTO 2   /* tree_plan_choose_schedule with
                               TREE_FORK_MIN_SAVED_TOKENS                     */

/* Default price, in scanned tokens, of one extra launch (one more trie level)
 * in the fork/rescan choice.  On MI355X a level launch is stream-ordered with
 * no host round trip and costs about the scan of a hundred or so tokens;
 * measured over RL-batch-shaped tries (1..64 prompts of 16..4096 tokens with
 * 8 completions each, 16/32 heads of 128), thresholds from 113 to 448 lose
 * the least time against the faster schedule
 * (python -m prefix_tree_packed_plan_amd.calibrate_policy re-measures it). */
#define TREE_FORK_MIN_SAVED_TOKENS 256

typedef struct tree_plan tree_plan_t; /* opaque, host memory, immutable once built */

typedef struct tree_plan_stats {
  int64_t n_tokens;        /* N: sum of seg_lens (unique tokens)                       */
  int64_t path_tokens;     /* sum over leaves of the root-to-leaf path length        */
  int64_t max_path_tokens; /* longest root-to-leaf path                               */
  double por;              /* potential overlap ratio 1 - N / path_tokens ("Tree
                              Training" section 4.1, Eq. 12)                          */
  int32_t n_seg;
  int32_t n_roots;
  int32_t n_leaves;
  int32_t n_parents; /* segments with at least one child (they own a state slot) */
  int32_t n_levels;  /* 1 + the largest depth                                    */
  int32_t conv_width;
  int64_t path_entries; /* rescan walk table size: sum over leaves of (depth + 1),
                           or -1 when it is too large to build (2^26 entries)
                           and TREE_SCHED_RESCAN is unavailable               */
} tree_plan_stats_t;

/*
 * tree_plan -- build the host plan of a trie (host only, no device work).
 *
 * parents[i]  parent segment of segment i, or -1 for a root; must lie in
 *             [-1, i) (any topological numbering; depth-first pre-order is
 *             the packed layout of "Tree Training" Eq. 8).  Several roots (a
 *             forest) are allowed.
 * seg_lens[i] tokens of segment i, >= 1.  Sum must be < 2^31.
 * n_seg       number of segments, >= 1.
 * conv_width  W of the causal conv, 1..8; n_seg (W-1) must be < 2^31.
 * out         receives a library-owned plan; free it with tree_plan_free.
 *
 * The plan holds: segment offsets; depths and the per-level segment order
 * (longest segment first within a level); the state slot of every segment
 * with children; and the conv history table hist[s][0..W-2], the packed row
 * indices of the W-1 inputs preceding segment s on its path: the last W-1
 * entries of hist[parent] followed by the parent's own rows.  A negative
 * entry -1 - (r (W-1) + j) names context row j (oldest first) of the r-th
 * root in segment order (init_ctx of tree_conv; zeros when that is NULL).
 * Inputs are copied; the plan is immutable and may be shared across threads.
 */
int tree_plan(const int32_t* parents, const int32_t* seg_lens, int32_t n_seg,
              int32_t conv_width, tree_plan_t** out);

/* Free a plan (NULL is a no-op).  Stream work that uses a device copy of the
 * plan does not need the host plan to stay alive. */
void tree_plan_free(tree_plan_t* plan);

/* Copy the plan's statistics into *out. */
int tree_plan_query(const tree_plan_t* plan, tree_plan_stats_t* out);

/* Copy the conv history table (n_seg * (W-1) int32, row-major) into hist. */
int tree_plan_conv_history(const tree_plan_t* plan, int32_t* hist);

/* Copy the level schedule: level_start[0..n_levels] (int32) and
 * order[0..n_seg-1] (segments of level L are order[level_start[L] ..
 * level_start[L+1]-1], longest first, ties by index). */
int tree_plan_levels(const tree_plan_t* plan, int32_t* level_start, int32_t* order);

/*
 * tree_plan_paths -- copy the rescan walk table: path_off[0..n_leaves]
 * (int32) and path_seg[0..path_entries-1].  Walk w covers path_seg[path_off[w]
 * .. path_off[w+1]-1], the segments of one leaf's root path from the root
 * down; walks are ordered by path length, longest first (ties by leaf
 * index).  An entry is the segment index s when this walk writes s's outputs
 * and state (the walk of the lowest-indexed leaf below s), ~s otherwise, so
 * every segment is written by exactly one walk.
 * Errors: INVALID_ARG, UNSUPPORTED (table not built: path_entries == -1).
 */
int tree_plan_paths(const tree_plan_t* plan, int32_t* path_off, int32_t* path_seg);

/*
 * tree_plan_choose_schedule -- the fork/rescan policy (tree-recurrence 0.1.0
 * project page, "How a tree runs": forking pays off when the shared-prefix
 * tokens it avoids rescanning are worth more than the extra launch each trie
 * level costs).  With saved = path_tokens -
 * n_tokens (tokens a rescan would scan twice or more) and n_levels - 1 extra
 * launches for the fork, *sched = TREE_SCHED_LEVEL when
 *     saved >= fork_min_saved_tokens * (n_levels - 1)
 * (always for a single-level trie, where both are one launch), else
 * TREE_SCHED_RESCAN; LEVEL whenever the walk table is unavailable.
 * fork_min_saved_tokens >= 0 is the price of one launch in scanned tokens
 * (TREE_FORK_MIN_SAVED_TOKENS by default).
 * Errors: INVALID_ARG.
 */
int tree_plan_choose_schedule(const tree_plan_t* plan, int64_t fork_min_saved_tokens, int32_t* sched);

/* Bytes of device memory tree_plan_upload writes (the device copy of the plan). */
size_t tree_plan_device_bytes(const tree_plan_t* plan);

/*
 * tree_plan_upload -- copy the plan into caller-owned device memory `dplan`
 * (dplan_bytes >= tree_plan_device_bytes) with an asynchronous host-to-device
 * copy on `stream`.  Do it once per plan; every tree_conv / tree_gdn_scan that
 * names this plan then takes the same `dplan` and `dplan_bytes` (e.g. every
 * layer of a forward).  The plan records (dplan, dplan_bytes), under a lock,
 * so that the entry points can reject any other buffer before launching.
 * The source is the plan's own pageable host buffer, so the plan must stay
 * alive until the copy has run (synchronise `stream` before freeing it).
 * Errors: INVALID_ARG, WORKSPACE (dplan_bytes too small), HIP.
 */
int tree_plan_upload(const tree_plan_t* plan, void* dplan, size_t dplan_bytes, void* stream);

/*
 * tree_conv -- tree-aware causal depthwise conv1d ("Tree Training" section
 * 3.2 Eq. 11; the per-path definition of section 3.1 Eq. 6):
 *
 *   y[t, c] = act( sum_{i=0}^{W-1} w[c, i] * xin(t, i - (W-1), c) + bias[c] )
 *
 * with w[c, W-1] multiplying token t itself,
 * where xin(t, -j, c) is the input j steps back along t's root path; before
 * the root it is the root's context row (init_ctx) or zero.
 *
 * x        device, [n_tokens, channels], dtype        (read)
 * w        device, [channels, W], dtype               (read)
 * bias     device, [channels], dtype, or NULL         (read)
 * y        device, [n_tokens, channels], dtype        (written; must not alias x)
 * init_ctx device, [n_roots, W-1, channels], dtype, or NULL: for the r-th
 *          root in segment order, the W-1 inputs in front of it, oldest
 *          first -- the conv state a partition gateway hands over across a
 *          cut ("Tree Training" section 3.3 and appendix B.7).  NULL = zeros.
 *                                                     (read)
 * ctx_out  device, [n_seg, W-1, channels], dtype, or NULL: for every
 *          segment, the W-1 path inputs ending at its last token, oldest
 *          first (the conv state a child, or the next partition, continues
 *          from).  Ignored when W = 1.                (written)
 * dtype TREE_DTYPE_F32 or TREE_DTYPE_BF16; arithmetic in fp32.
 * act   TREE_ACT_NONE or TREE_ACT_SILU (y = z * sigmoid(z)).
 * dplan, dplan_bytes  device copy of `plan` made by tree_plan_upload, and
 *       the size it was uploaded with (see Conventions).
 * Errors: INVALID_ARG (also: dplan not an upload of this plan), SIZE
 * (n_tokens != plan N), UNSUPPORTED (W > 4), WORKSPACE (dplan_bytes too
 * small), HIP.
 */
int tree_conv(const void* x, const void* w, const void* bias, void* y, const void* init_ctx,
              void* ctx_out, int64_t n_tokens, int32_t channels, int32_t dtype, int32_t act,
              const tree_plan_t* plan, const void* dplan, size_t dplan_bytes, void* stream);

/*
 * tree_conv_backward_workspace_bytes -- device workspace tree_conv_backward
 * needs for `channels`: the dz of every segment's first W-1 tokens and the
 * per-block partial sums of dw and dbias, fp32.
 */
size_t tree_conv_backward_workspace_bytes(const tree_plan_t* plan, int32_t channels);

/*
 * tree_conv_backward -- gradients of the tree conv ("Tree Training"
 * section 3.2 Eq. 11; the backward of the per-path definition, section 3.1
 * Eq. 6, each token's output counted once).  With z the pre-activation and
 * dz = dy * act'(z):
 *
 *   dx[j, c]   = sum_{d=0}^{W-1} w[c, W-1-d] * sum of dz[t, c] over the tokens
 *                t that lie d steps after j on some root-to-leaf path,
 *   dw[c, i]   = sum_t dz[t, c] * xin(t, i - (W-1), c),
 *   dbias[c]   = sum_t dz[t, c],
 *   dinit_ctx  = the same gradient for the roots' given context rows.
 *
 * Past the end of its segment a token's successors are the first tokens of
 * every child (and deeper, for children shorter than W-1): a parent's last
 * W-1 inputs receive the sum over all children (same paper, section 3.2 and
 * appendix A.2, sibling gradients accumulate in what the parent hands them;
 * appendix B.7, fp32 accumulation).  Sums run in a fixed order: the result
 * is deterministic.
 *
 * x, w, bias, init_ctx   the forward's inputs (bias, init_ctx may be NULL).
 * dy        device, [n_tokens, channels], dtype       (read)
 * dx        device, [n_tokens, channels], dtype       (written)
 * dw        device, [channels, W] fp32                (written)
 * dbias     device, [channels] fp32, or NULL          (written)
 * dinit_ctx device, [n_roots, W-1, channels] fp32, or NULL (written; W > 1)
 * dplan, dplan_bytes  as for tree_conv.
 * ws        device workspace of ws_bytes >= tree_conv_backward_workspace_bytes.
 * Errors: INVALID_ARG, SIZE, UNSUPPORTED (W > 4), WORKSPACE, HIP.
 */
int tree_conv_backward(const void* x, const void* w, const void* bias, const void* dy, const void* init_ctx,
                       void* dx, float* dw, float* dbias, float* dinit_ctx, int64_t n_tokens, int32_t channels,
                       int32_t dtype, int32_t act, const tree_plan_t* plan, const void* dplan, size_t dplan_bytes,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * tree_scan_workspace_bytes -- device workspace tree_gdn_scan needs under
 * TREE_SCHED_LEVEL (or AUTO): one fp32 state [h_v, d_k, d_v] per segment with
 * children (0 when the caller passes `states`, which then carries the parent
 * states).  TREE_SCHED_RESCAN needs none.
 */
size_t tree_scan_workspace_bytes(const tree_plan_t* plan, int32_t h_v, int32_t d_k, int32_t d_v,
                                 int32_t with_states);

/*
 * tree_workspace_bytes -- device workspace tree_gdn_scan needs under schedule
 * `sched` when the caller does not ask for `states` (the largest case): the
 * parent state slots under TREE_SCHED_LEVEL, nothing under TREE_SCHED_RESCAN;
 * TREE_SCHED_AUTO is resolved with tree_plan_choose_schedule and
 * TREE_FORK_MIN_SAVED_TOKENS.  The device plan is not part of it: it is the
 * separate `dplan` buffer, uploaded once per forward and shared by every
 * call that names the plan.  0 for a NULL plan.
 */
size_t tree_workspace_bytes(const tree_plan_t* plan, int32_t h_v, int32_t d_k, int32_t d_v, int32_t sched);

/*
 * tree_gdn_scan -- chunked gated delta rule over the trie ("Tree Training"
 * section 3.2 Eq. 10 and appendix A.2; the recurrence at the top of this file).
 *
 * q, k   device, [n_tokens, h_qk, d_k], dtype          (read)
 * v      device, [n_tokens, h_v, d_v], dtype           (read)
 * g      device, [n_tokens, h_v], fp32: log decay, a_t = exp(g_t); g <= 0
 *        keeps every exponent the kernel forms non-positive       (read)
 * beta   device, [n_tokens, h_v], fp32                 (read)
 * o      device, [n_tokens, h_v, d_v], dtype           (written)
 * init_states device, [n_roots, h_v, d_k, d_v] fp32, or NULL: the state the
 *        r-th root (in segment order) starts from, as a partition gateway
 *        hands it over ("Tree Training" appendix B.7).  NULL = zero.  (read)
 * states device, [n_seg, h_v, d_k, d_v] fp32, or NULL: every segment's
 *        state after its last token, [d_k, d_v] orientation (the appendix's
 *        state tensor).  When given, children read their parents' states
 *        from it and the workspace may be empty.         (written)
 * Value head h uses query/key head h / (h_v / h_qk).
 * scale  multiplies q (1.0 = the plain recurrence).
 * dtype  TREE_DTYPE_BF16 (bf16 MFMA, fp32 accumulation, compensated
 *        split-bf16 on the state path) or TREE_DTYPE_F32 (inputs split into
 *        two bf16 parts on every product).  At d = 128 in bf16, a chunk's
 *        later rows skip the products their decay scales below the error
 *        the other rows already carry; the results depend on the inputs only
 *        (both schedules give the same bits).
 * sched  TREE_SCHED_LEVEL, TREE_SCHED_RESCAN or TREE_SCHED_AUTO (see
 *        tree_plan_choose_schedule).
 * dplan, dplan_bytes  as for tree_conv.
 * ws     device workspace of ws_bytes >= tree_scan_workspace_bytes (may be
 *        NULL under TREE_SCHED_RESCAN).
 * Compiled head sizes: d_k = d_v in {32, 64, 128} for bf16, {32, 64} for fp32.
 * Errors: INVALID_ARG, SIZE, UNSUPPORTED (also: RESCAN without a walk
 * table), WORKSPACE, HIP.
 */
int tree_gdn_scan(const void* q, const void* k, const void* v, const float* g,
                  const float* beta, void* o, const float* init_states, float* states,
                  int64_t n_tokens, int32_t h_qk,
                  int32_t h_v, int32_t d_k, int32_t d_v, float scale, int32_t dtype,
                  int32_t sched, const tree_plan_t* plan, const void* dplan, size_t dplan_bytes,
                  void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch array behind tree_gdn_scan_noalloc (one
 * per GPU the library runs on, held until the process ends). */
#define TREE_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * tree_gdn_scan_noalloc -- tree_gdn_scan for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * tree_gdn_scan, without dplan and ws: the device plan and the parent-state
 * slots live in a library-owned static device array of
 * TREE_NOALLOC_SCRATCH_BYTES on each GPU.  The call copies the plan into it
 * (an asynchronous host-to-device copy on `stream`; the plan must stay alive
 * until the stream has run it) and launches the same kernels as
 * tree_gdn_scan; it calls no hipMalloc, hipFree or other allocating routine.
 * Needs tree_plan_device_bytes(plan), rounded up to 256, plus
 * tree_scan_workspace_bytes(plan, h_v, d_k, d_v, states != NULL) under the
 * level schedule (nothing under rescan) to fit in the array; a larger call is
 * rejected with TREE_ERR_WORKSPACE before any device work.  `stream` must
 * belong to the calling thread's current device.  Every call on a GPU shares
 * that GPU's array and leaves its contents behind: calls that overlap on one
 * GPU (different streams, or several threads) race and must be serialised
 * by the caller; calls on one stream are ordered by it.
 */
int tree_gdn_scan_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta, void* o,
                          const float* init_states, float* states, int64_t n_tokens, int32_t h_qk, int32_t h_v,
                          int32_t d_k, int32_t d_v, float scale, int32_t dtype, int32_t sched,
                          const tree_plan_t* plan, void* stream);

/*
 * tree_gdn_scan_backward_workspace_bytes -- device workspace
 * tree_gdn_scan_backward needs: the start state ([h_v, d_k, d_v] fp32) of
 * every 8th 16-token chunk of each segment (a checkpoint; the chunks between
 * two checkpoints are re-run forward from it when the backward reaches
 * them), three [h_v, 16, 16] fp32 matrices of every chunk, one start-state
 * gradient ([h_v, d_k, d_v] fp32) per segment, room for 7 re-run start
 * states per work-group of the largest trie level ([7, d_k, d_v] fp32 per
 * segment of that level and value head), plus per-value-head dq and dk
 * ([n_tokens, h_v, d_k] fp32 each) when h_v > 2 h_qk.
 */
size_t tree_gdn_scan_backward_workspace_bytes(const tree_plan_t* plan, int32_t h_qk, int32_t h_v, int32_t d_k,
                                              int32_t d_v);

/*
 * tree_gdn_scan_backward -- gradients of tree_gdn_scan ("Tree Training"
 * section 3.1 Eq. 6, every token's output counted once; section 3.2 Eq. 10
 * and appendix A.2, each segment starting from its parent's final state).
 * Given do = dL/do (and optionally dstates = dL/dstates), returns dL/dq,
 * dL/dk, dL/dv, dL/dg, dL/dbeta and dL/dinit_states.  A parent's final
 * state receives the sum of the gradients of all its children's start
 * states, in fp32 and in child index order (appendix A.2, sibling
 * gradients accumulate in the shared parent state; appendix B.5, fp32
 * accumulation); levels run from the deepest up.  The result is
 * deterministic.  Within a segment the chunked form is differentiated
 * chunk by chunk (16-token chunks, fp32 MFMA), each chunk's start state
 * recomputed from the parent's final state (every 8th stored, the others
 * re-run from the last stored one).
 * q, k, v, g, beta, init_states, scale, dtype   as passed to tree_gdn_scan.
 * dout    device, [n_tokens, h_v, d_v], dtype        (read)
 * dstates device, [n_seg, h_v, d_k, d_v] fp32, or NULL (no gradient on the
 *         final states)                               (read)
 * states  device, [n_seg, h_v, d_k, d_v] fp32: the final states the
 *         forward wrote (tree_gdn_scan's `states`)    (read)
 * dq, dk  device, [n_tokens, h_qk, d_k] fp32 (summed over the value heads
 *         of each query/key head, in head order; with two value heads
 *         per q/k head the first stores its part and the second adds to
 *         it, which rounds as the ordered sum)        (written)
 * dv      device, [n_tokens, h_v, d_v] fp32           (written)
 * dg, dbeta device, [n_tokens, h_v] fp32              (written)
 * dinit_states device, [n_roots, h_v, d_k, d_v] fp32, or NULL (written)
 * dplan, dplan_bytes  as for tree_conv.
 * ws      device workspace of ws_bytes >= tree_gdn_scan_backward_workspace_bytes.
 * Compiled head sizes: d_k = d_v in {32, 64, 128}; bf16 or fp32 inputs.
 * Errors: INVALID_ARG, SIZE, UNSUPPORTED, WORKSPACE, HIP.
 */
int tree_gdn_scan_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           const void* dout, const float* dstates, const float* init_states,
                           const float* states, float* dq, float* dk, float* dv, float* dg, float* dbeta,
                           float* dinit_states, int64_t n_tokens, int32_t h_qk, int32_t h_v, int32_t d_k,
                           int32_t d_v, float scale, int32_t dtype, const tree_plan_t* plan, const void* dplan,
                           size_t dplan_bytes, void* ws, size_t ws_bytes, void* stream);

/*
 * tree_ssd_scan -- Mamba2 (SSD) forward with the state forked over the trie
 * (tree-recurrence 0.1.0 project page: "How a tree runs", a fork starts each
 * segment from its parent's final state, and "Not yet", forking the Mamba2
 * state; "Tree Training" section 3.1 Eq. 6, every token's result equals the
 * standalone forward of its own root path).  Per head h, with group
 * h / (n_heads / n_groups):
 *     S_t = exp(dt_t A_h) S_{t-1} + dt_t B_t x_t^T,   y_t = S_t^T C_t + D_h x_t,
 * S [d_state, head_dim] fp32; one launch per trie level, each segment
 * starting from its parent's final state (a root from init_states or zero).
 * x      device, [n_tokens, n_heads, head_dim], dtype      (read)
 * dt     device, [n_tokens, n_heads] fp32, the step after softplus (>= 0)
 *                                                          (read)
 * A      device, [n_heads] fp32, the decay rate (< 0)      (read)
 * B, C   device, [n_tokens, n_groups, d_state], dtype      (read)
 * D      device, [n_heads] fp32, or NULL (no skip term)    (read)
 * y      device, [n_tokens, n_heads, head_dim], dtype      (written)
 * init_states device, [n_roots, n_heads, d_state, head_dim] fp32, or NULL
 *                                                          (read)
 * states device, [n_seg, n_heads, d_state, head_dim] fp32, or NULL: every
 *        segment's final state (then the workspace may be empty)  (written)
 * dplan, dplan_bytes  as for tree_conv.
 * ws     device workspace of ws_bytes >= tree_scan_workspace_bytes(plan,
 *        n_heads, d_state, head_dim, states != NULL).
 * dtype  TREE_DTYPE_BF16 (bf16 MFMA; the products with the state take it as
 *        hi + lo bf16) or TREE_DTYPE_F32 (fp32 MFMA).
 * Compiled sizes: d_state in {64, 128}, head_dim in {32, 64}.
 * Errors: INVALID_ARG, SIZE, UNSUPPORTED, WORKSPACE, HIP.
 */
int tree_ssd_scan(const void* x, const float* dt, const float* A, const void* B, const void* C, const float* D,
                  void* y, const float* init_states, float* states, int64_t n_tokens, int32_t n_groups,
                  int32_t n_heads, int32_t d_state, int32_t head_dim, int32_t dtype, const tree_plan_t* plan,
                  const void* dplan, size_t dplan_bytes, void* ws, size_t ws_bytes, void* stream);

/* Message for the last failed call on this thread ("" if none). */
const char* tree_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TREE_GDN_H */
