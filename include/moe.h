/*
 * moe.h -- C ABI of the DeepSeekMoE layer forward on one MI355X (gfx950).
 *
 * The layer (source: "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化",
 * section "Method details: formulas and load balance"):
 *
 *   s_{r,t} = softmax_r(u_t . e_r)                over the N' routed experts
 *   g_{r,t} = s_{r,t} if r in Topk(s_t, K') else 0
 *   h_t     = sum_{i < K_s} FFN_i(u_t) + sum_r g_{r,t} FFN_{K_s + r}(u_t) + u_t
 *
 * with the first K_s experts shared (always active), the remaining N' routed,
 * each expert a SwiGLU FFN  FFN(u) = W2 (SiLU(W1 u) * (W3 u))  of intermediate
 * width w (1/m of a standard FFN, section "Two core strategies"), and the
 * balance terms of the same section and of "【论文总结】MoE" sections 2.3-2.4:
 *
 *   f_r  = N'/(K'T) * #{t : t selects r},     P_r = mean_t s_{r,t}
 *   f'_g = mean of f over device group g,      P'_g = sum of P over group g
 *   ExpBal = sum_r f_r P_r,                    DevBal = sum_g f'_g P'_g
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every tensor pointer is device memory owned by the caller (contiguous,
 *    row-major, 16-byte aligned).  The library allocates nothing and keeps no
 *    mutable global state; calls on different streams with different
 *    workspaces are independent.
 *  - Every call validates its arguments on the host first.  On an error it
 *    returns a negative status, enqueues nothing and leaves outputs untouched.
 *    Launch failures return MOE_ERR_HIP.  Faults inside kernels surface at
 *    the caller's next synchronisation.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *    default stream).  Outputs are overwritten, never accumulated into.
 *  - dtype (moe_problem.dtype) applies to x, the expert weights, y_routed and
 *    h.  Centroids, bias, gates, probabilities and statistics are fp32;
 *    indices and counts are int32.
 *  - Shapes: d % 64 == 0, w % 64 == 0, T >= 0, K_s >= 0, N' >= 0;
 *    N' == 0 (a dense, shared-only layer) requires K' == 0, otherwise
 *    1 <= K' <= N'.  T*K' and T*K_s*w must fit in int32.  Each of these
 *    stays below 2^31 bytes (the GEMMs address them with 32-bit offsets):
 *    x [T, d], y_routed [T*K', d], twice the routed activations [T*K', w]
 *    and twice the shared ones [T, K_s*w] (the backward keeps dp and dq side
 *    by side), and the shared expert stack [K_s, d, w].  Every call returns
 *    MOE_ERR_UNSUPPORTED outside this envelope.
 *  - Routing inputs must be finite.  Expert indices handed to moe_permute
 *    must lie in [0, N') and be distinct within a token; entries that are
 *    not are skipped (memory stays safe, results for that token are
 *    undefined).
 *  - Expert weights, per expert, "out x in": W1 and W3 are [w, d], W2 is
 *    [d, w].  Shared experts are stacked [K_s, ...], routed [N', ...].
 *  - The workspace `ws` (size from moe_workspace_size, 256-byte aligned)
 *    holds the per-block partial routing statistics, the grouping scratch,
 *    the SwiGLU activations, the gates in grouped order (accumulating
 *    expert FFN) and the control words of the fused expert FFN launch
 *    (cleared by moe_expert_ffn itself before each use; no initialisation
 *    is needed).  The calls use disjoint parts of it, so one
 *    workspace serves a whole layer pass on one stream; calls that overlap
 *    in time (other streams) need workspaces of their own.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK               0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, bad shape, bad group count     */
#define MOE_ERR_UNSUPPORTED (-2)  /* outside the supported envelope (see each call) */
#define MOE_ERR_WORKSPACE   (-3)  /* workspace missing or smaller than required    */
#define MOE_ERR_HIP         (-4)  /* a HIP launch or runtime call failed           */
#define MOE_ERR_STALLED     (-5)  /* a device-side wait gave up (moe_expert_ffn_status) */

/* element types of x, weights, y_routed and h */
#define MOE_F32  0
#define MOE_BF16 1

typedef struct moe_problem {
    int32_t T;         /* tokens in the batch                                  */
    int32_t d;         /* hidden size                                          */
    int32_t n_shared;  /* K_s: shared experts, always active                   */
    int32_t n_routed;  /* N': routed experts                                   */
    int32_t top_k;     /* K': routed experts selected per token                */
    int32_t inter;     /* w: expert intermediate width                         */
    int32_t dtype;     /* MOE_F32 or MOE_BF16                                  */
} moe_problem;

/* Human-readable text of a status code (static storage). */
const char *moe_status_str(int status);

/* Library build/version tag (static storage). */
const char *moe_version(void);

/* Bytes of workspace one layer pass needs for `p` (written to *bytes).
 * Returns MOE_ERR_INVALID_ARG on a bad problem or null pointers. */
int moe_workspace_size(const moe_problem *p, size_t *bytes);

/*
 * moe_route -- gating: token-to-centroid affinities, softmax, Top-K'.
 * Source: "[ACL 2024] DeepSeekMoE ..." section "Method details" (gates from
 * Top-k of the affinities; only routed experts are selected), "【论文总结】MoE"
 * section 2.2 (centroids e_i).
 *
 *   x        [T, d]   dtype      token activations u_t
 *   centroids[N', d]  fp32       e_r
 *   bias     [N']     fp32       optional additive logit bias (NULL = none)
 *   idx      [T, K']  int32  out selected routed experts, order (z desc, r asc)
 *   gate     [T, K']  fp32   out s_{idx[t,k], t}
 *   probs    [T, N']  fp32   out all affinities s (NULL = not written)
 *   counts   [N']     int32  out tokens per routed expert
 *   prob_sum [N']     fp32   out sum_t s_{r,t}
 *
 * Logits z_{t,r} are accumulated in fp32 as one fused multiply-add chain over
 * k = 0..d-1 in ascending order starting from +0, then the bias is added in
 * one fp32 add; selection compares z (ties go to the lower index), so the
 * selected experts do not depend on how exp is evaluated.  Deterministic:
 * counts and prob_sum are reduced in a fixed order without atomics.
 * Envelope: 1 <= K' <= min(N', 16), 1 <= N' <= 256 (MOE_ERR_UNSUPPORTED).
 */
int moe_route(const moe_problem *p, const void *x, const float *centroids,
              const float *bias, int32_t *idx, float *gate, float *probs,
              int32_t *counts, float *prob_sum, void *ws, size_t ws_bytes,
              void *stream);

/*
 * moe_route_noalloc -- moe_route for callers that cannot allocate or manage
 * a workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments and results as moe_route, without
 * ws: the per-workgroup partial statistics live in a static device array of
 * the library (4 MiB per GPU, held until the process ends; its address is
 * looked up once per device, with that device current, on the first call).
 * The call itself allocates nothing.  Problems whose partials need more
 * than 4 MiB (ceil(T / tokens per routing workgroup) * N' * 12 bytes, about
 * 43 K tokens at N' = 256) return MOE_ERR_UNSUPPORTED.  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race and must be serialised by the caller.
 */
int moe_route_noalloc(const moe_problem *p, const void *x, const float *centroids,
                      const float *bias, int32_t *idx, float *gate, float *probs,
                      int32_t *counts, float *prob_sum, void *stream);

/*
 * moe_route_ablate -- moe_route with each token's `disabled_top` highest
 * ranked routed experts disabled: the token takes the experts of ranks
 * disabled_top .. disabled_top+K'-1 in the order (z desc, r asc).  This is the
 * redundancy ablation of "[ACL 2024] DeepSeekMoE ..." section "Expert
 * specialization analysis" (Fig. 4, disabling the top routed experts).
 * Affinities, gates (not renormalised), probs and prob_sum are as in
 * moe_route; counts count the taken experts.  disabled_top = 0 is moe_route.
 * Envelope: disabled_top + K' <= min(N', 16).
 */
int moe_route_ablate(const moe_problem *p, int32_t disabled_top, const void *x, const float *centroids,
                     const float *bias, int32_t *idx, float *gate, float *probs, int32_t *counts, float *prob_sum,
                     void *ws, size_t ws_bytes, void *stream);

/*
 * moe_route_hash -- fixed hash routing, the Hash Layer baseline of "[ACL
 * 2024] DeepSeekMoE ..." section "Experiment design": one expert per token
 * from its token id, gate 1 (no learned gate).  K' must be 1.
 *   token_ids [T] int32 in;  idx [T, 1] int32 out;  gate [T, 1] fp32 out (1.0)
 *   counts [N'] int32 out
 *   expert = floor(h * N' / 2^32),  h = id * 2654435761 mod 2^32 (uint32)
 * (Knuth's multiplicative hash with a multiply-shift range reduction; the
 * pages name the baseline, not its hash).  The rest of the layer (permute,
 * expert FFNs, combine) runs unchanged on this routing.
 */
int moe_route_hash(const moe_problem *p, const int32_t *token_ids, int32_t *idx, float *gate, int32_t *counts,
                   void *stream);

/*
 * moe_permute -- group (token, expert) pairs by routed expert: histogram,
 * exclusive scan, stable scatter (tokens ascending within an expert).  This
 * is the bookkeeping behind "token t selects expert i" ("【论文总结】MoE"
 * section 2.3).  It recounts from idx, so any routing can be supplied.
 *
 *   idx          [T, K']   int32 in   routed expert of each (t, k)
 *   offsets      [N'+1]    int32 out  offsets[r] = pairs of experts < r
 *   sorted_token [T*K']    int32 out  tokens of expert 0, then expert 1, ...
 *   slot_of      [T, K']   int32 out  position of (t, idx[t,k]) in sorted_token
 *
 * Envelope: N' <= 1024; 1 <= K' <= N' (any K', e.g. every expert active).
 */
int moe_permute(const moe_problem *p, const int32_t *idx, int32_t *offsets,
                int32_t *sorted_token, int32_t *slot_of, void *ws,
                size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn -- the expert FFNs (SwiGLU, no biases) on MFMA.
 * Source: "[ACL 2024] DeepSeekMoE ..." sections "Two core strategies" (m
 * fine-grained experts of width 1/m; K_s shared experts always active) and
 * "Method details" (FFN_i terms of the layer output and their gate-weighted
 * sum).
 *
 *   x            [T, d]         dtype in
 *   offsets      [N'+1]         int32 in   from moe_permute
 *   sorted_token [T*K']         int32 in   from moe_permute
 *   w1_routed, w3_routed [N', w, d]  dtype;  w2_routed [N', d, w]  dtype
 *   w1_shared, w3_shared [K_s, w, d] dtype;  w2_shared [K_s, d, w] dtype
 *   y_routed     [T*K', d]      dtype out  (nullable, selects the mode below)
 *   y_acc        [T, d]         fp32  out
 *   gate         [T, K']        fp32  in   from moe_route (accumulating mode only)
 *   slot_of      [T, K']        int32 in   from moe_permute (accumulating mode only)
 *
 * Two modes:
 *  - gather (y_routed != NULL, the default of the layer pass):
 *      y_routed[j] = FFN_{e(j)}(u_{sorted_token[j]})   unweighted, grouped order
 *      y_acc[t]    = sum_{i < K_s} FFN_i(u_t)           (y_acc may be NULL when K_s == 0)
 *    moe_combine then sums the gate-weighted rows of each token in k order:
 *    bitwise reproducible.
 *  - accumulating (y_routed == NULL and T*K' > 0): the down projection adds
 *    gate[t,k] * FFN_{idx[t,k]}(u_t) of every routed pair, and every shared
 *    FFN_i(u_t), straight into y_acc (zeroed by the call first), so
 *      y_acc[t] = sum_{i < K_s} FFN_i(u_t) + sum_k gate[t,k] FFN_{idx[t,k]}(u_t)
 *    and moe_combine (with y_routed = NULL) only adds the residual.  This
 *    saves the round trip of y_routed through HBM.  The adds are fp32
 *    atomics in memory: their order, and so the last bits of y_acc, vary
 *    from run to run (NOT bitwise reproducible).  gate and slot_of are
 *    required; the gates are copied into grouped order in the workspace.
 *
 * The K_s shared experts run as one dense expert of width K_s*w over all T
 * rows.  Accumulation is fp32; the SwiGLU activation is rounded to dtype
 * before the down projection.  Routed pointers may be NULL when N' == 0 and
 * shared pointers when K_s == 0.
 *
 * In bf16 both projections run as one persistent launch (one workgroup per
 * CU) whose down-projection tiles wait, on counters in the workspace, for
 * the up-projection tiles of their token rows; a small kernel clears those
 * counters first (it runs on every call, also when there is no work).  In
 * gather mode the results are the same as moe_expert_up followed by
 * moe_expert_down.  fp32 runs the two projections as two launches.
 */
int moe_expert_ffn(const moe_problem *p, const void *x, const int32_t *offsets,
                   const int32_t *sorted_token, const void *w1_routed,
                   const void *w3_routed, const void *w2_routed,
                   const void *w1_shared, const void *w3_shared,
                   const void *w2_shared, void *y_routed, float *y_acc,
                   const float *gate, const int32_t *slot_of,
                   void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_status -- error word of the most recent moe_expert_ffn
 * enqueued with this workspace.  Waits for `stream` to finish, then reads
 * the word.  Returns MOE_OK, or MOE_ERR_STALLED when a down-projection tile
 * of the fused launch gave up waiting for the up-projection tiles of its
 * token rows (bounded wait of about 2^22 sleeps).  Such a tile computes
 * nothing and writes NaN over its outputs, so no result is silently built
 * from partial activations.  MOE_ERR_HIP if the stream or the read fails.
 * Must be called before the next moe_expert_ffn with the same workspace
 * (which clears the word).  Test hook: with the environment variable
 * MOE_DEBUG_FFN_STALL=<n> (n > 0) set when moe_expert_ffn is called, every
 * such wait is made unmeetable and gives up after n sleeps.
 */
int moe_expert_ffn_status(const moe_problem *p, const void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn_kernel -- name of the GPU kernel (template instantiation)
 * that moe_expert_ffn launches for `p` (accumulate != 0: accumulating
 * mode), as it appears in a kernel trace; "" when the call has no work;
 * NULL for an invalid problem.  Static storage.
 */
const char *moe_expert_ffn_kernel(const moe_problem *p, int accumulate);

/*
 * moe_expert_up / moe_expert_down -- the two halves of moe_expert_ffn, for
 * callers that schedule or time them separately.  moe_expert_up computes the
 * SwiGLU activations act = SiLU(W1 u) * (W3 u) (rounded to dtype) of every
 * shared row and grouped routed row into the workspace; moe_expert_down
 * reads them from the same workspace (same problem, same ws, same stream, in
 * that order) and writes y_routed and y_shared exactly as moe_expert_ffn
 * does in gather mode (y_shared: the y_acc of that mode).  Arguments have
 * the meanings given above.
 */
int moe_expert_up(const moe_problem *p, const void *x, const int32_t *offsets,
                  const int32_t *sorted_token, const void *w1_routed,
                  const void *w3_routed, const void *w1_shared,
                  const void *w3_shared, void *ws, size_t ws_bytes, void *stream);

int moe_expert_down(const moe_problem *p, const int32_t *offsets,
                    const void *w2_routed, const void *w2_shared, void *y_routed,
                    float *y_shared, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_combine -- layer output, "[ACL 2024] DeepSeekMoE ..." section "Method
 * details" (output formula):
 *   h_t = u_t + y_acc_t + sum_{k < K'} gate[t,k] * y_routed[slot_of[t,k]]
 * summed in k order in fp32 (deterministic), written as dtype.
 *
 *   x [T, d] dtype, y_routed [T*K', d] dtype, y_acc [T, d] fp32 (NULL =
 *   zero), gate [T, K'] fp32, slot_of [T, K'] int32, h [T, d] dtype out.
 * With y_routed == NULL (after the accumulating moe_expert_ffn, whose y_acc
 * already holds the whole expert sum) h_t = u_t + y_acc_t and gate/slot_of
 * are not read.  With x all zero, h is the expert sum y itself.
 */
int moe_combine(const moe_problem *p, const void *x, const void *y_routed,
                const float *y_acc, const float *gate, const int32_t *slot_of,
                void *h, void *stream);

/*
 * moe_balance_stats -- expert-level and device-level balance terms.
 * Source: "[ACL 2024] DeepSeekMoE ..." section "Method details" (expert-level
 * and device-level balance losses), "【论文总结】MoE" sections 2.3 (symbols T,
 * N', K', indicator, factor N'/K') and 2.4 (f'_i, P'_i of a device).
 *
 *   groups D: routed experts are split into D contiguous equal groups
 *   counts [N'] int32, prob_sum [N'] fp32       in (from moe_route)
 *   f [N'], P [N'], f_dev [D], P_dev [D]        fp32 out
 *   exp_bal [1], dev_bal [1]                    fp32 out (alpha_1, alpha_2 not applied)
 *
 *   f_r = RN_fp32((double)N' * counts[r] / ((double)K' * T))
 *   P_r = prob_sum[r] / T
 *   f'_g = RN_fp32((double)N' * C_g / ((double)K' * T * (N'/D))), C_g = sum of counts in g
 *   P'_g = sum of P over g;  ExpBal = sum f P;  DevBal = sum f' P'  (fp64, then fp32)
 * T == 0 gives f = P = 0.  Requires N' >= 1, 1 <= K' <= N', D >= 1, D | N'.
 */
int moe_balance_stats(const moe_problem *p, int32_t groups, const int32_t *counts,
                      const float *prob_sum, float *f, float *P, float *f_dev,
                      float *P_dev, float *exp_bal, float *dev_bal, void *stream);

/*
 * moe_layer_forward -- one whole layer pass in one call: moe_route,
 * moe_permute, moe_expert_ffn (gather mode), moe_combine and moe_balance_stats
 * in that order on `stream`, over one workspace of moe_workspace_size(p).
 * Source: the five calls above (the layer output of "[ACL 2024] DeepSeekMoE
 * ..." section "Method details", with its balance terms).
 *
 * Every pointer of `io` has the meaning, layout, dtype and ownership it has in
 * those calls (io->probs may be NULL, io->bias may be NULL; io->y_routed is
 * required when routed pairs exist, io->y_shared when K_s > 0), and every
 * output is bitwise the output of the five calls.  All arguments are checked
 * before anything is enqueued: the first failing check of the five calls is
 * returned and nothing runs.  Requires N' >= 1 and D = groups as in
 * moe_balance_stats.
 *
 * Decode batches (at most 256 tokens whose routing takes the one-workgroup-
 * per-token kernel, T K' > 0) run as four kernels instead of seven: routing,
 * then one kernel whose two workgroups group the pairs and clear the expert
 * FFN's control words, and sum the routing partials and compute the balance
 * terms, then
 * the fused expert FFN and the combine.  Other batches run as six kernels
 * instead of eight: routing; the grouping's histogram with the routing's
 * reduction in one launch (more than 256 tokens; else the two apart); the
 * grouping's scatter; one kernel that computes the balance terms and clears
 * the expert FFN's control words; the expert FFN and the combine.
 * moe_expert_ffn_status reports on the expert FFN of this call.
 */
typedef struct moe_layer_io {
    /* inputs (moe_route, moe_expert_ffn) */
    const void *x;
    const float *centroids;
    const float *bias;
    const void *w1_routed, *w3_routed, *w2_routed;
    const void *w1_shared, *w3_shared, *w2_shared;
    /* outputs of moe_route */
    int32_t *idx;
    float *gate;
    float *probs;
    int32_t *counts;
    float *prob_sum;
    /* outputs of moe_permute */
    int32_t *offsets;
    int32_t *sorted_token;
    int32_t *slot_of;
    /* outputs of moe_expert_ffn (y_shared: its y_acc argument) and moe_combine */
    void *y_routed;
    float *y_shared;
    void *h;
    /* outputs of moe_balance_stats */
    float *f, *P, *f_dev, *P_dev, *exp_bal, *dev_bal;
} moe_layer_io;

int moe_layer_forward(const moe_problem *p, int32_t groups, const moe_layer_io *io, void *ws, size_t ws_bytes,
                      void *stream);


/* ========================================================================
 * Backward pass.  Training is the pages' setting ("[ACL 2024] DeepSeekMoE
 * ..." section "Method details": the loss adds alpha_1 * ExpBal +
 * alpha_2 * DevBal to the task loss).  Given dh = dL_task/dh of the layer
 * output, three calls mirror the forward ones (same problem, same stream):
 *
 *   moe_combine_backward     dh -> dy_routed (= gate * dh per grouped row), dgate
 *   moe_expert_ffn_backward  -> dx_ffn and the expert weight gradients
 *   moe_route_backward       -> dx (= dh + dx_ffn + router part), dcentroids, dbias
 *
 * Chain rule on the forward definitions, with the Top-K selection held fixed
 * (it is piecewise constant) and f, f' (counts of that selection) constant;
 * P and P' are differentiable through the softmax:
 *   per used (t, e), dy = gate * dh_t (routed) or dh_t (shared):
 *     da = W2^T dy, dq = da SiLU(p), dp = da q s (1 + p (1 - s)), s = sigmoid(p)
 *     dx_t += W1^T dp + W3^T dq; dW2 += dy a^T; dW1 += dp u_t^T; dW3 += dq u_t^T
 *   dgate[t,k] = dh_t . y_routed[slot_of[t,k]]
 *   ds[t,r] = dgate[t,k] (r = idx[t,k]) + (alpha1 f_r + alpha2 f'_{g(r)}) / T
 *   dz[t,r] = s[t,r] (ds[t,r] - sum_r' s[t,r'] ds[t,r'])
 *   dx_t += sum_r dz[t,r] e_r;  dcentroids = dz^T x;  dbias = column sums of dz
 * The backward workspace (moe_backward_workspace_size, 256-byte aligned) is
 * separate from the forward one; it holds the per-row intermediates (da,
 * dp, dq, a and the grouped rows' dx, all in dtype; the shared experts' dx
 * in fp32) and the router's dz.
 * Gradients are fp32; accumulation is fp32; the intermediates are rounded
 * to dtype as the forward rounds its activations.  Every output is
 * overwritten.  Deterministic: no atomics, fixed summation orders.
 * ====================================================================== */

int moe_backward_workspace_size(const moe_problem *p, size_t *bytes);

/*
 * moe_combine_backward -- gradient through h = u + y_shared + sum_k g y_routed.
 *   dh         [T, d]      dtype in   upstream gradient
 *   y_routed   [T*K', d]   dtype in   from moe_expert_ffn
 *   gate, slot_of [T, K']             from moe_route / moe_permute
 *   dy_routed  [T*K', d]   dtype out  dy_routed[slot_of[t,k]] = gate[t,k] dh_t
 *   dgate      [T, K']     fp32  out  dh_t . y_routed[slot_of[t,k]] (fp32 sum)
 * Envelope: K' <= 16 (as moe_route), MOE_ERR_UNSUPPORTED otherwise.
 */
int moe_combine_backward(const moe_problem *p, const void *dh, const void *y_routed, const float *gate,
                         const int32_t *slot_of, void *dy_routed, float *dgate, void *stream);

/*
 * moe_expert_ffn_backward -- expert FFN gradients ("[ACL 2024] DeepSeekMoE
 * ..." sections "Two core strategies" and "Method details").
 *   x, offsets, sorted_token, weights     as in moe_expert_ffn
 *   slot_of   [T, K']        from moe_permute
 *   dh        [T, d]   dtype upstream gradient (the shared experts' dy)
 *   dy_routed [T*K', d] dtype from moe_combine_backward
 *   dx_ffn    [T, d]   fp32 out  sum over the token's experts of W1^T dp + W3^T dq
 *   dw1_*, dw3_* [E, w, d], dw2_* [E, d, w]  fp32 out (routed E = N', shared
 *             E = K_s; every expert written, unused ones with zeros)
 * The SwiGLU pre-activations are recomputed (one more up-projection).
 */
int moe_expert_ffn_backward(const moe_problem *p, const void *x, const int32_t *offsets,
                            const int32_t *sorted_token, const int32_t *slot_of, const void *w1_routed,
                            const void *w3_routed, const void *w2_routed, const void *w1_shared,
                            const void *w3_shared, const void *w2_shared, const void *dh, const void *dy_routed,
                            float *dx_ffn, float *dw1_routed, float *dw3_routed, float *dw2_routed,
                            float *dw1_shared, float *dw3_shared, float *dw2_shared, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * moe_route_backward -- router gradient and the layer's input gradient.
 * Source: "[ACL 2024] DeepSeekMoE ..." section "Method details" (gates,
 * balance losses), "【论文总结】MoE" sections 2.2-2.4.
 *   groups D, alpha1, alpha2    weights of ExpBal and DevBal in the loss
 *   x [T, d] dtype, centroids [N', d] fp32
 *   probs [T, N'] fp32          the forward's affinities (required)
 *   idx [T, K'], dgate [T, K']  from moe_route / moe_combine_backward
 *   f [N'], f_dev [D]           from moe_balance_stats
 *   dh [T, d] dtype, dx_ffn [T, d] fp32 (NULL = 0)
 *   dx [T, d] fp32 out          dh + dx_ffn + sum_r dz[t,r] e_r
 *   dcentroids [N', d] fp32 out, dbias [N'] fp32 out (NULL = not written)
 * Envelope: N' <= 256, D | N'.
 */
int moe_route_backward(const moe_problem *p, int32_t groups, float alpha1, float alpha2, const void *x,
                       const float *centroids, const float *probs, const int32_t *idx, const float *dgate,
                       const float *f, const float *f_dev, const void *dh, const float *dx_ffn, float *dx,
                       float *dcentroids, float *dbias, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
