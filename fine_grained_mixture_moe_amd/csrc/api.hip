// api.hip -- the extern "C" entry points declared in include/moe.h.
//
// Host side only: argument validation (before anything is enqueued), the
// workspace layout, and dispatch to the kernels of route.hip, permute.hip,
// expert_ffn.hip, combine_stats.hip and backward.hip.
#include <stdint.h>

#include "moe_internal.h"

using namespace moe;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_problem(const moe_problem *p) {
    if (!p) return MOE_ERR_INVALID_ARG;
    if (p->T < 0 || p->d <= 0 || p->n_shared < 0 || p->n_routed < 0 || p->top_k < 0 || p->inter <= 0)
        return MOE_ERR_INVALID_ARG;
    if (p->dtype != MOE_F32 && p->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
    if (p->d % 64 != 0 || p->inter % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (p->n_routed == 0) {
        if (p->top_k != 0) return MOE_ERR_INVALID_ARG;
    } else if (p->top_k < 1 || p->top_k > p->n_routed) {
        return MOE_ERR_INVALID_ARG;
    }
    if (p->n_routed > kPermuteMaxExperts) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)p->T * p->top_k > INT32_MAX || (int64_t)p->n_shared * p->inter > INT32_MAX / 64 ||
        (int64_t)p->T * p->top_k * p->inter > (int64_t)1 << 40)
        return MOE_ERR_UNSUPPORTED;
    // The GEMMs address whole operands through buffer resources with 32-bit
    // offsets: x [T, d], y_routed / dy_routed [T*K', d], the routed and the
    // shared activations (the backward's dp and dq side by side: twice that),
    // and a shared expert stack [K_s, d, w] must each stay below 2^31 bytes.
    const int64_t es = dtype_bytes(p->dtype), lim = (int64_t)1 << 31, tk = (int64_t)p->T * p->top_k;
    if ((int64_t)p->T * p->d * es >= lim || tk * p->d * es >= lim || 2 * tk * p->inter * es + 256 >= lim ||
        2 * (int64_t)p->T * p->n_shared * p->inter * es + 256 >= lim ||
        (int64_t)p->n_shared * p->d * p->inter * es >= lim)
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

int check_ws(const moe_problem *p, const void *ws, size_t ws_bytes, WsLayout *L) {
    *L = ws_layout(*p);
    if (L->total > 0 && (!ws || ws_bytes < L->total)) return MOE_ERR_WORKSPACE;
    if (ws && ((uintptr_t)ws & 255u) != 0) return MOE_ERR_WORKSPACE;
    return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Argument checks of moe_route_ablate (moe_route: disabled_top = 0).
int check_route(const moe_problem *p, int32_t disabled_top, const void *x, const float *centroids,
                const int32_t *idx, const float *gate, const int32_t *counts, const float *prob_sum, const void *ws,
                size_t ws_bytes, WsLayout *L) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->n_routed < 1 || disabled_top < 0) return MOE_ERR_INVALID_ARG;
    if (disabled_top + p->top_k > p->n_routed) return MOE_ERR_INVALID_ARG;
    if (p->n_routed > kRouteMaxExperts || disabled_top + p->top_k > kRouteMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (!centroids || !counts || !prob_sum) return MOE_ERR_INVALID_ARG;
    if (p->T > 0 && (!x || !idx || !gate)) return MOE_ERR_INVALID_ARG;
    if ((x && !aligned16(x)) || !aligned16(centroids)) return MOE_ERR_INVALID_ARG;
    return check_ws(p, ws, ws_bytes, L);
}

// Argument checks of moe_permute.
int check_permute(const moe_problem *p, const int32_t *idx, const int32_t *offsets, const int32_t *sorted_token,
                  const int32_t *slot_of, const void *ws, size_t ws_bytes, WsLayout *L) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (!offsets) return MOE_ERR_INVALID_ARG;
    if ((int64_t)p->T * p->top_k > 0 && (!idx || !sorted_token || !slot_of)) return MOE_ERR_INVALID_ARG;
    return check_ws(p, ws, ws_bytes, L);
}

// Argument checks of moe_combine (with T > 0).
int check_combine(const moe_problem *p, const void *x, const void *y_routed, const float *y_shared,
                  const float *gate, const int32_t *slot_of, const void *h) {
    if (!x || !h) return MOE_ERR_INVALID_ARG;
    if (p->top_k > 0 && y_routed && (!gate || !slot_of)) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(h) || (y_routed && !aligned16(y_routed)) ||
        (y_shared && !aligned16(y_shared)))
        return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

// Argument checks of moe_balance_stats.
int check_stats(const moe_problem *p, int32_t groups, const int32_t *counts, const float *prob_sum, const float *f,
                const float *P, const float *f_dev, const float *P_dev, const float *exp_bal, const float *dev_bal) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->n_routed < 1 || groups < 1 || p->n_routed % groups != 0) return MOE_ERR_INVALID_ARG;
    if (!counts || !prob_sum || !f || !P || !f_dev || !P_dev || !exp_bal || !dev_bal) return MOE_ERR_INVALID_ARG;
    return MOE_OK;
}

uint8_t *at(void *ws, size_t off) { return (uint8_t *)ws + off; }

}  // namespace

extern "C" {

const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, misaligned pointer or bad shape";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the supported envelope";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
        case MOE_ERR_HIP: return "MOE_ERR_HIP: HIP launch or runtime error";
        case MOE_ERR_STALLED:
            return "MOE_ERR_STALLED: a wait inside the fused expert FFN launch gave up; its outputs hold NaN";
        default: return "unknown moe status";
    }
}

const char *moe_version(void) { return "moe-mi355x 0.2 (gfx950)"; }

int moe_workspace_size(const moe_problem *p, size_t *bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    const int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    *bytes = ws_layout(*p).total;
    return MOE_OK;
}

int moe_route_ablate(const moe_problem *p, int32_t disabled_top, const void *x, const float *centroids,
                     const float *bias, int32_t *idx, float *gate, float *probs, int32_t *counts, float *prob_sum,
                     void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    const int rc = check_route(p, disabled_top, x, centroids, idx, gate, counts, prob_sum, ws, ws_bytes, &L);
    if (rc != MOE_OK) return rc;
    return hip_status(launch_route(*p, disabled_top, x, centroids, bias, idx, gate, probs,
                                   (int32_t *)at(ws, L.route_counts), (double *)at(ws, L.route_psum), counts,
                                   prob_sum, (hipStream_t)stream));
}

int moe_route(const moe_problem *p, const void *x, const float *centroids, const float *bias, int32_t *idx,
              float *gate, float *probs, int32_t *counts, float *prob_sum, void *ws, size_t ws_bytes, void *stream) {
    return moe_route_ablate(p, 0, x, centroids, bias, idx, gate, probs, counts, prob_sum, ws, ws_bytes, stream);
}

int moe_route_noalloc(const moe_problem *p, const void *x, const float *centroids, const float *bias, int32_t *idx,
                      float *gate, float *probs, int32_t *counts, float *prob_sum, void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->n_routed < 1) return MOE_ERR_INVALID_ARG;
    if (p->n_routed > kRouteMaxExperts || p->top_k > kRouteMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (!centroids || !counts || !prob_sum) return MOE_ERR_INVALID_ARG;
    if (p->T > 0 && (!x || !idx || !gate)) return MOE_ERR_INVALID_ARG;
    if ((x && !aligned16(x)) || !aligned16(centroids)) return MOE_ERR_INVALID_ARG;
    if (route_partial_bytes(*p) > kRouteScratchBytes) return MOE_ERR_UNSUPPORTED;
    void *sp = nullptr;
    if (route_scratch_ptr(&sp) != hipSuccess) return MOE_ERR_HIP;
    uint8_t *base = (uint8_t *)sp;
    return hip_status(launch_route(*p, 0, x, centroids, bias, idx, gate, probs, (int32_t *)base,
                                   (double *)(base + route_psum_offset(*p)), counts, prob_sum,
                                   (hipStream_t)stream));
}

int moe_route_hash(const moe_problem *p, const int32_t *token_ids, int32_t *idx, float *gate, int32_t *counts,
                   void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->n_routed < 1 || p->top_k != 1) return MOE_ERR_INVALID_ARG;
    if (!counts || (p->T > 0 && (!token_ids || !idx || !gate))) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_route_hash(*p, token_ids, idx, gate, counts, (hipStream_t)stream));
}

int moe_permute(const moe_problem *p, const int32_t *idx, int32_t *offsets, int32_t *sorted_token,
                int32_t *slot_of, void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    const int rc = check_permute(p, idx, offsets, sorted_token, slot_of, ws, ws_bytes, &L);
    if (rc != MOE_OK) return rc;
    return hip_status(launch_permute(*p, idx, offsets, sorted_token, slot_of, (int32_t *)at(ws, L.perm_hist),
                                     (int32_t *)at(ws, L.perm_base), (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation shared by the expert-FFN calls.  `up` / `down` select which
// weights and outputs the call touches.
// accum: the accumulating form of the down projection (y_routed == NULL with
// routed pairs present; gate, slot_of and y_shared = y_acc required).
int check_ffn(const moe_problem *p, bool up, bool down, const void *x, const int32_t *offsets,
              const int32_t *sorted_token, const void *w1_routed, const void *w3_routed, const void *w2_routed,
              const void *w1_shared, const void *w3_shared, const void *w2_shared, const void *y_routed,
              const float *y_shared, const void *ws, size_t ws_bytes, WsLayout *L, bool *routed, bool *shared,
              bool accum = false, const float *gate = nullptr, const int32_t *slot_of = nullptr) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    *routed = p->n_routed > 0 && (int64_t)p->T * p->top_k > 0;
    *shared = p->n_shared > 0 && p->T > 0;
    if (*routed) {
        if (!offsets) return MOE_ERR_INVALID_ARG;
        if (up && (!x || !sorted_token || !w1_routed || !w3_routed)) return MOE_ERR_INVALID_ARG;
        if (down && !w2_routed) return MOE_ERR_INVALID_ARG;
        if (down && !accum && !y_routed) return MOE_ERR_INVALID_ARG;
        if (accum && (!gate || !slot_of || !y_shared || !sorted_token)) return MOE_ERR_INVALID_ARG;
        if ((w1_routed && !aligned16(w1_routed)) || (w3_routed && !aligned16(w3_routed)) ||
            (w2_routed && !aligned16(w2_routed)) || (y_routed && !aligned16(y_routed)))
            return MOE_ERR_INVALID_ARG;
    }
    if (*shared) {
        if (up && (!x || !w1_shared || !w3_shared)) return MOE_ERR_INVALID_ARG;
        if (down && (!w2_shared || !y_shared)) return MOE_ERR_INVALID_ARG;
        if ((w1_shared && !aligned16(w1_shared)) || (w3_shared && !aligned16(w3_shared)) ||
            (w2_shared && !aligned16(w2_shared)) || (y_shared && !aligned16(y_shared)))
            return MOE_ERR_INVALID_ARG;
    }
    if ((x && !aligned16(x)) || (y_shared && !aligned16(y_shared))) return MOE_ERR_INVALID_ARG;
    return check_ws(p, ws, ws_bytes, L);
}

FfnArgs ffn_args(const void *x, const int32_t *offsets, const int32_t *sorted_token, const void *w1_routed,
                 const void *w3_routed, const void *w2_routed, const void *w1_shared, const void *w3_shared,
                 const void *w2_shared, void *y_routed, float *y_shared, void *ws, const WsLayout &L) {
    FfnArgs a{};
    a.x = x;
    a.offsets = offsets;
    a.sorted_token = sorted_token;
    a.w1_r = w1_routed; a.w3_r = w3_routed; a.w2_r = w2_routed;
    a.w1_s = w1_shared; a.w3_s = w3_shared; a.w2_s = w2_shared;
    a.act_shared = at(ws, L.act_shared);
    a.act_routed = at(ws, L.act_routed);
    a.y_routed = y_routed;
    a.y_shared = y_shared;
    return a;
}

moe_problem active_part(const moe_problem &p, bool routed, bool shared) {
    moe_problem q = p;
    if (!routed) q.n_routed = 0, q.top_k = 0;
    if (!shared) q.n_shared = 0;
    return q;
}

}  // namespace

extern "C" {

int moe_expert_up(const moe_problem *p, const void *x, const int32_t *offsets, const int32_t *sorted_token,
                  const void *w1_routed, const void *w3_routed, const void *w1_shared, const void *w3_shared,
                  void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    bool routed, shared;
    int rc = check_ffn(p, true, false, x, offsets, sorted_token, w1_routed, w3_routed, nullptr, w1_shared,
                       w3_shared, nullptr, nullptr, nullptr, ws, ws_bytes, &L, &routed, &shared);
    if (rc != MOE_OK) return rc;
    if (!routed && !shared) return MOE_OK;
    const FfnArgs a = ffn_args(x, offsets, sorted_token, w1_routed, w3_routed, nullptr, w1_shared, w3_shared,
                               nullptr, nullptr, nullptr, ws, L);
    return hip_status(launch_expert_up(active_part(*p, routed, shared), a, (hipStream_t)stream));
}

int moe_expert_down(const moe_problem *p, const int32_t *offsets, const void *w2_routed, const void *w2_shared,
                    void *y_routed, float *y_shared, void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    bool routed, shared;
    int rc = check_ffn(p, false, true, nullptr, offsets, nullptr, nullptr, nullptr, w2_routed, nullptr, nullptr,
                       w2_shared, y_routed, y_shared, ws, ws_bytes, &L, &routed, &shared);
    if (rc != MOE_OK) return rc;
    if (!routed && !shared) return MOE_OK;
    const FfnArgs a = ffn_args(nullptr, offsets, nullptr, nullptr, nullptr, w2_routed, nullptr, nullptr, w2_shared,
                               y_routed, y_shared, ws, L);
    return hip_status(launch_expert_down(active_part(*p, routed, shared), a, (hipStream_t)stream));
}

int moe_expert_ffn(const moe_problem *p, const void *x, const int32_t *offsets, const int32_t *sorted_token,
                   const void *w1_routed, const void *w3_routed, const void *w2_routed, const void *w1_shared,
                   const void *w3_shared, const void *w2_shared, void *y_routed, float *y_acc, const float *gate,
                   const int32_t *slot_of, void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    bool routed, shared;
    const bool accum = y_routed == nullptr && p && p->n_routed > 0 && (int64_t)p->T * p->top_k > 0;
    int rc = check_ffn(p, true, true, x, offsets, sorted_token, w1_routed, w3_routed, w2_routed, w1_shared,
                       w3_shared, w2_shared, y_routed, y_acc, ws, ws_bytes, &L, &routed, &shared, accum, gate,
                       slot_of);
    if (rc != MOE_OK) return rc;
    FfnArgs a = ffn_args(x, offsets, sorted_token, w1_routed, w3_routed, w2_routed, w1_shared, w3_shared,
                         w2_shared, y_routed, y_acc, ws, L);
    if (accum) {
        a.y_acc = y_acc;
        a.gate = gate;
        a.slot_of = slot_of;
        a.gate_sorted = (float *)at(ws, L.gate_sorted);
    }
    // always launched (the preparation kernel clears the error flag of moe_expert_ffn_status)
    const moe_problem q = active_part(*p, routed, shared);
    return hip_status(launch_expert_ffn(q, a, (int32_t *)at(ws, L.ffn_ctl), (hipStream_t)stream));
}

int moe_expert_ffn_status(const moe_problem *p, const void *ws, size_t ws_bytes, void *stream) {
    WsLayout L;
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if ((rc = check_ws(p, ws, ws_bytes, &L)) != MOE_OK) return rc;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return MOE_ERR_HIP;
    int32_t err = 0;
    if (hipMemcpy(&err, (const uint8_t *)ws + L.ffn_ctl + kFfnCtlErr * sizeof(int32_t), sizeof(err),
                  hipMemcpyDeviceToHost) != hipSuccess)
        return MOE_ERR_HIP;
    return err ? MOE_ERR_STALLED : MOE_OK;
}

const char *moe_expert_ffn_kernel(const moe_problem *p, int accumulate) {
    if (check_problem(p) != MOE_OK) return nullptr;
    const bool routed = p->n_routed > 0 && (int64_t)p->T * p->top_k > 0;
    const bool shared = p->n_shared > 0 && p->T > 0;
    if (!routed && !shared) return "";
    return expert_ffn_kernel_name(active_part(*p, routed, shared), accumulate && routed);
}

int moe_combine(const moe_problem *p, const void *x, const void *y_routed, const float *y_shared,
                const float *gate, const int32_t *slot_of, void *h, void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->T == 0) return MOE_OK;
    if ((rc = check_combine(p, x, y_routed, y_shared, gate, slot_of, h)) != MOE_OK) return rc;
    return hip_status(launch_combine(*p, x, y_routed, y_shared, gate, slot_of, h, (hipStream_t)stream));
}

int moe_balance_stats(const moe_problem *p, int32_t groups, const int32_t *counts, const float *prob_sum,
                      float *f, float *P, float *f_dev, float *P_dev, float *exp_bal, float *dev_bal,
                      void *stream) {
    const int rc = check_stats(p, groups, counts, prob_sum, f, P, f_dev, P_dev, exp_bal, dev_bal);
    if (rc != MOE_OK) return rc;
    return hip_status(launch_balance_stats(*p, groups, counts, prob_sum, f, P, f_dev, P_dev, exp_bal, dev_bal,
                                           (hipStream_t)stream));
}

int moe_layer_forward(const moe_problem *p, int32_t groups, const moe_layer_io *io, void *ws, size_t ws_bytes,
                      void *stream) {
    if (!io) return MOE_ERR_INVALID_ARG;
    WsLayout L;
    bool routed = false, shared = false;
    int rc = check_route(p, 0, io->x, io->centroids, io->idx, io->gate, io->counts, io->prob_sum, ws, ws_bytes, &L);
    if (rc == MOE_OK)
        rc = check_permute(p, io->idx, io->offsets, io->sorted_token, io->slot_of, ws, ws_bytes, &L);
    if (rc == MOE_OK)
        rc = check_ffn(p, true, true, io->x, io->offsets, io->sorted_token, io->w1_routed, io->w3_routed,
                       io->w2_routed, io->w1_shared, io->w3_shared, io->w2_shared, io->y_routed, io->y_shared, ws,
                       ws_bytes, &L, &routed, &shared);
    if (rc == MOE_OK && p->T > 0)
        rc = check_combine(p, io->x, io->y_routed, io->y_shared, io->gate, io->slot_of, io->h);
    if (rc == MOE_OK)
        rc = check_stats(p, groups, io->counts, io->prob_sum, io->f, io->P, io->f_dev, io->P_dev, io->exp_bal,
                         io->dev_bal);
    if (rc != MOE_OK) return rc;
    // decode batches: routing, the one-workgroup tail (partials summed, statistics, grouping, the
    // FFN's control words), the fused FFN without its preparation kernel, the combine
    if (routed && p->T <= kPermuteTokens && route_decode_batch(*p)) {
        hipStream_t s = (hipStream_t)stream;
        int32_t *pc = (int32_t *)at(ws, L.route_counts);
        double *pp = (double *)at(ws, L.route_psum);
        int32_t *ctl = (int32_t *)at(ws, L.ffn_ctl);
        const moe_problem q = active_part(*p, routed, shared);
        hipError_t e = launch_route(*p, 0, io->x, io->centroids, io->bias, io->idx, io->gate, io->probs, pc, pp,
                                    io->counts, io->prob_sum, s, /*reduce=*/false);
        if (e == hipSuccess)
            e = launch_layer_decode_tail(*p, groups, pp, io->counts, io->prob_sum, io->idx, io->offsets,
                                         io->sorted_token, io->slot_of, io->f, io->P, io->f_dev, io->P_dev,
                                         io->exp_bal, io->dev_bal, ctl, ffn_ctl_ints(q), s);
        const FfnArgs a = ffn_args(io->x, io->offsets, io->sorted_token, io->w1_routed, io->w3_routed, io->w2_routed,
                                   io->w1_shared, io->w3_shared, io->w2_shared, io->y_routed, io->y_shared, ws, L);
        if (e == hipSuccess) e = launch_expert_ffn(q, a, ctl, s, /*prep=*/false);
        if (e == hipSuccess)
            e = launch_combine(*p, io->x, io->y_routed, io->y_shared, io->gate, io->slot_of, io->h, s);
        return hip_status(e);
    }
    // other batches: the routing; the grouping's histogram with the routing's reduction in one
    // launch (more than kPermuteTokens tokens with routed pairs; else the two apart, as moe_route
    // and moe_permute); the grouping; one kernel for the statistics and the FFN's control words;
    // the fused FFN without its preparation kernel; the combine (their checks have passed above)
    hipStream_t s = (hipStream_t)stream;
    int32_t *pc = (int32_t *)at(ws, L.route_counts);
    double *pp = (double *)at(ws, L.route_psum);
    const bool merge = p->n_routed > 0 && p->top_k > 0 && cdiv(p->T, kPermuteTokens) >= 2;
    hipError_t e = launch_route(*p, 0, io->x, io->centroids, io->bias, io->idx, io->gate, io->probs, pc, pp,
                                io->counts, io->prob_sum, s, /*reduce=*/!merge);
    const RouteReduce rr{p->T > 0 ? route_blocks(p->T, p->d, p->n_routed) : 0, pc, pp, io->counts, io->prob_sum};
    if (e == hipSuccess)
        e = launch_permute(*p, io->idx, io->offsets, io->sorted_token, io->slot_of, (int32_t *)at(ws, L.perm_hist),
                           (int32_t *)at(ws, L.perm_base), s, merge ? &rr : nullptr);
    int32_t *ctl = (int32_t *)at(ws, L.ffn_ctl);
    const moe_problem q = active_part(*p, routed, shared);
    if (e == hipSuccess) e = launch_layer_stats_ctl(*p, groups, io->counts, io->prob_sum, io->f, io->P, io->f_dev, io->P_dev,
                                          io->exp_bal, io->dev_bal, ctl, ffn_ctl_ints(q), s);
    const FfnArgs a = ffn_args(io->x, io->offsets, io->sorted_token, io->w1_routed, io->w3_routed, io->w2_routed,
                               io->w1_shared, io->w3_shared, io->w2_shared, io->y_routed, io->y_shared, ws, L);
    if (e == hipSuccess) e = launch_expert_ffn(q, a, ctl, s, /*prep=*/false);
    if (e == hipSuccess)
        e = launch_combine(*p, io->x, io->y_routed, io->y_shared, io->gate, io->slot_of, io->h, s);
    return hip_status(e);
}

// ---------------------------------------------------------------------------
// backward pass
// ---------------------------------------------------------------------------

int moe_backward_workspace_size(const moe_problem *p, size_t *bytes) {
    if (!bytes) return MOE_ERR_INVALID_ARG;
    const int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    *bytes = bwd_ws_layout(*p).total;
    return MOE_OK;
}

int moe_combine_backward(const moe_problem *p, const void *dh, const void *y_routed, const float *gate,
                         const int32_t *slot_of, void *dy_routed, float *dgate, void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if ((int64_t)p->T * p->top_k == 0) return MOE_OK;
    if (p->top_k > kRouteMaxTopK) return MOE_ERR_UNSUPPORTED;
    if (!dh || !y_routed || !gate || !slot_of || !dy_routed || !dgate) return MOE_ERR_INVALID_ARG;
    if (!aligned16(dh) || !aligned16(y_routed) || !aligned16(dy_routed)) return MOE_ERR_INVALID_ARG;
    return hip_status(launch_combine_backward(*p, dh, y_routed, gate, slot_of, dy_routed, dgate,
                                              (hipStream_t)stream));
}

int moe_expert_ffn_backward(const moe_problem *p, const void *x, const int32_t *offsets,
                            const int32_t *sorted_token, const int32_t *slot_of, const void *w1_routed,
                            const void *w3_routed, const void *w2_routed, const void *w1_shared,
                            const void *w3_shared, const void *w2_shared, const void *dh, const void *dy_routed,
                            float *dx_ffn, float *dw1_routed, float *dw3_routed, float *dw2_routed,
                            float *dw1_shared, float *dw3_shared, float *dw2_shared, void *ws, size_t ws_bytes,
                            void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    const bool routed = p->n_routed > 0, shared = p->n_shared > 0;
    if (routed && (!offsets || !w1_routed || !w3_routed || !w2_routed || !dw1_routed || !dw3_routed || !dw2_routed))
        return MOE_ERR_INVALID_ARG;
    if (routed && p->T > 0 && (!sorted_token || !slot_of || !dy_routed)) return MOE_ERR_INVALID_ARG;
    if (shared && (!w1_shared || !w3_shared || !w2_shared || !dw1_shared || !dw3_shared || !dw2_shared))
        return MOE_ERR_INVALID_ARG;
    if (p->T > 0 && (!x || !dh || !dx_ffn)) return MOE_ERR_INVALID_ARG;
    for (const void *q : {x, dh, dy_routed, (const void *)dx_ffn, w1_routed, w3_routed, w2_routed, w1_shared,
                          w3_shared, w2_shared, (const void *)dw1_routed, (const void *)dw3_routed,
                          (const void *)dw2_routed, (const void *)dw1_shared, (const void *)dw3_shared,
                          (const void *)dw2_shared})
        if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
    const BwdWsLayout L = bwd_ws_layout(*p);
    if (L.total > 0 && (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u) != 0)) return MOE_ERR_WORKSPACE;
    BwdFfnArgs a{};
    a.x = x; a.dh = dh; a.dy_routed = dy_routed;
    a.offsets = offsets; a.sorted_token = sorted_token; a.slot_of = slot_of;
    a.w1_r = w1_routed; a.w3_r = w3_routed; a.w2_r = w2_routed;
    a.w1_s = w1_shared; a.w3_s = w3_shared; a.w2_s = w2_shared;
    a.da_r = at(ws, L.da_r); a.dp_r = at(ws, L.dp_r); a.dq_r = at(ws, L.dq_r); a.a_r = at(ws, L.a_r);
    a.da_s = at(ws, L.da_s); a.dp_s = at(ws, L.dp_s); a.dq_s = at(ws, L.dq_s); a.a_s = at(ws, L.a_s);
    a.dxr = at(ws, L.dxr); a.dxs = (float *)at(ws, L.dxs); a.dx_ffn = dx_ffn;
    a.dw1_r = dw1_routed; a.dw3_r = dw3_routed; a.dw2_r = dw2_routed;
    a.dw1_s = dw1_shared; a.dw3_s = dw3_shared; a.dw2_s = dw2_shared;
    return hip_status(launch_expert_backward(*p, a, (hipStream_t)stream));
}

int moe_route_backward(const moe_problem *p, int32_t groups, float alpha1, float alpha2, const void *x,
                       const float *centroids, const float *probs, const int32_t *idx, const float *dgate,
                       const float *f, const float *f_dev, const void *dh, const float *dx_ffn, float *dx,
                       float *dcentroids, float *dbias, void *ws, size_t ws_bytes, void *stream) {
    int rc = check_problem(p);
    if (rc != MOE_OK) return rc;
    if (p->n_routed < 1) return MOE_ERR_INVALID_ARG;
    if (p->n_routed > kRouteMaxExperts) return MOE_ERR_UNSUPPORTED;
    if (groups < 1 || p->n_routed % groups != 0) return MOE_ERR_INVALID_ARG;
    if (!centroids || !f || !f_dev || !dcentroids) return MOE_ERR_INVALID_ARG;
    if (p->T > 0 && (!x || !probs || !idx || !dgate || !dh || !dx)) return MOE_ERR_INVALID_ARG;
    for (const void *q : {x, dh, (const void *)dx_ffn, (const void *)dx, (const void *)centroids})
        if (q && !aligned16(q)) return MOE_ERR_INVALID_ARG;
    const BwdWsLayout L = bwd_ws_layout(*p);
    if (L.total > 0 && (!ws || ws_bytes < L.total || ((uintptr_t)ws & 255u) != 0)) return MOE_ERR_WORKSPACE;
    return hip_status(launch_route_backward(*p, groups, alpha1, alpha2, x, centroids, probs, idx, dgate, f, f_dev,
                                            dh, dx_ffn, dx, dcentroids, dbias, (float *)at(ws, L.dz),
                                            (float *)at(ws, L.de_part), (hipStream_t)stream));
}

}  // extern "C"
