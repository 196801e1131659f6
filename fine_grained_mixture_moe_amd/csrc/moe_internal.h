// moe_internal.h -- private declarations shared by the HIP sources of libmoe.
// Not installed, not part of the C ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Tokens handled by one grouping (permute) workgroup.
constexpr int kPermuteTokens = 256;
// Largest N' the routing kernel supports, and K' bound.
constexpr int kRouteMaxExperts = 256;
constexpr int kRouteMaxTopK = 16;
// Largest N' the grouping kernels support.
constexpr int kPermuteMaxExperts = 1024;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }
__host__ __device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline size_t dtype_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// Byte offsets of each call's scratch inside the caller's workspace.  The
// regions are disjoint, so one workspace serves a whole layer pass.
struct WsLayout {
    size_t route_counts;   // int32  [route_blocks, N']  per-block expert counts
    size_t route_psum;     // double [route_blocks, N']  per-block affinity sums
    size_t perm_hist;      // int32  [N', perm_blocks]   per-block histogram (expert-major)
    size_t perm_base;      // int32  [N', perm_blocks]   first slot of each (expert, block)
    size_t act_shared;     // dtype  [T, K_s*w]          SwiGLU activations, shared experts
    size_t act_routed;     // dtype  [T*K', w]           SwiGLU activations, grouped order
    size_t ffn_ctl;        // int32  [ffn_ctl_ints]      fused expert FFN: queue heads, error flag, per-run counters
    size_t total;
};

// Control words of the fused expert FFN launch: 8 queue heads, an error
// flag, and one counter per token run; a group of c rows has ceil(c/128)
// runs at most, so sum_g ceil(c_g/128) <= T K'/128 + N' (+ T/128 shared).
inline int ffn_ctl_ints(const moe_problem &p) {
    const int64_t runs = (p.n_shared > 0 ? cdiv(p.T, 128) : 0) +
                         (p.n_routed > 0 ? ((int64_t)p.T * p.top_k) / 128 + p.n_routed : 0);
    return (int)(8 + 1 + runs);
}

// Routing workgroups for T tokens (route.hip).
int route_blocks(int T);

inline WsLayout ws_layout(const moe_problem &p) {
    WsLayout L{};
    const size_t nr = (size_t)p.n_routed;
    const size_t rb = p.T > 0 ? (size_t)route_blocks(p.T) : 0;
    const size_t pb = (size_t)cdiv(p.T, kPermuteTokens);
    const size_t es = dtype_bytes(p.dtype);
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes, 256); return at; };
    L.route_counts = take(rb * nr * sizeof(int32_t));
    L.route_psum = take(rb * nr * sizeof(double));
    L.perm_hist = take(pb * nr * sizeof(int32_t));
    L.perm_base = take(pb * nr * sizeof(int32_t));
    L.act_shared = take((size_t)p.T * p.n_shared * p.inter * es);
    L.act_routed = take((size_t)p.T * p.top_k * p.inter * es);
    L.ffn_ctl = take((size_t)ffn_ctl_ints(p) * sizeof(int32_t));
    L.total = off;
    return L;
}

// ---- launchers (each returns hipSuccess or the launch error) -------------

hipError_t launch_route(const moe_problem &p, int skip, const void *x, const float *centroids,
                        const float *bias, int32_t *idx, float *gate, float *probs,
                        int32_t *part_counts, double *part_psum,
                        int32_t *counts, float *prob_sum, hipStream_t s);

hipError_t launch_route_hash(const moe_problem &p, const int32_t *token_ids, int32_t *idx, float *gate,
                             int32_t *counts, hipStream_t s);

hipError_t launch_permute(const moe_problem &p, const int32_t *idx, int32_t *offsets,
                          int32_t *sorted_token, int32_t *slot_of, int32_t *hist,
                          int32_t *base, hipStream_t s);

struct FfnArgs {
    const void *x;
    const int32_t *offsets;
    const int32_t *sorted_token;
    const void *w1_r, *w3_r, *w2_r;
    const void *w1_s, *w3_s, *w2_s;
    void *act_shared, *act_routed;
    void *y_routed;
    float *y_shared;
};

// up: act = SiLU(X W1^T) * (X W3^T) into the workspace; down: y = act W2^T.
hipError_t launch_expert_up(const moe_problem &p, const FfnArgs &a, hipStream_t s);
hipError_t launch_expert_down(const moe_problem &p, const FfnArgs &a, hipStream_t s);
// both projections: bf16 as one fused persistent launch (ctl: the workspace's
// control words), fp32 as the two launches above
hipError_t launch_expert_ffn(const moe_problem &p, const FfnArgs &a, int32_t *ctl, hipStream_t s);
// backward: the up projection recomputed, with a = SiLU(p) q written to act_*
// and dp, dq formed from da in the epilogue (bf16 only)
hipError_t launch_expert_up_backward(const moe_problem &p, const FfnArgs &a, const void *da_shared,
                                     const void *da_routed, void *dp_shared, void *dp_routed, void *dq_shared,
                                     void *dq_routed, hipStream_t s);

hipError_t launch_combine(const moe_problem &p, const void *x, const void *y_routed,
                          const float *y_shared, const float *gate, const int32_t *slot_of,
                          void *h, hipStream_t s);

hipError_t launch_balance_stats(const moe_problem &p, int groups, const int32_t *counts,
                                const float *prob_sum, float *f, float *P, float *f_dev,
                                float *P_dev, float *exp_bal, float *dev_bal, hipStream_t s);

// ---- backward pass (backward.hip) ------------------------------------------

// Token chunks of the centroid-gradient partial sums.
int route_backward_chunks(int T);

// Byte offsets of the backward scratch inside the caller's backward workspace.
struct BwdWsLayout {
    size_t da_r, dp_r, dq_r, a_r;   // dtype [T*K', w]
    size_t da_s, dp_s, dq_s, a_s;   // dtype [T, K_s*w]
    size_t dxr;                     // fp32  [T*K', d]   dx of every grouped row
    size_t dxs;                     // fp32  [T, d]      dx of the shared experts
    size_t dz;                      // fp32  [T, N']     router logit gradient
    size_t de_part;                 // fp32  [chunks, N', d+4] centroid-gradient partials
    size_t total;
};

inline BwdWsLayout bwd_ws_layout(const moe_problem &p) {
    BwdWsLayout L{};
    const size_t es = dtype_bytes(p.dtype);
    const size_t tk = (size_t)p.T * p.top_k, ts = (size_t)p.T * p.n_shared;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes, 256); return at; };
    L.da_r = take(tk * p.inter * es);
    L.dp_r = take(tk * p.inter * es);
    L.dq_r = take(tk * p.inter * es);
    L.a_r = take(tk * p.inter * es);
    L.da_s = take(ts * p.inter * es);
    L.dp_s = take(ts * p.inter * es);
    L.dq_s = take(ts * p.inter * es);
    L.a_s = take(ts * p.inter * es);
    L.dxr = take(tk * p.d * sizeof(float));
    L.dxs = take((p.n_shared > 0 ? (size_t)p.T : 0) * p.d * sizeof(float));
    L.dz = take((size_t)p.T * p.n_routed * sizeof(float));
    L.de_part = take((size_t)route_backward_chunks(p.T) * p.n_routed * (p.d + 4) * sizeof(float));
    L.total = off;
    return L;
}

hipError_t launch_combine_backward(const moe_problem &p, const void *dh, const void *y_routed,
                                   const float *gate, const int32_t *slot_of, void *dy_routed,
                                   float *dgate, hipStream_t s);

struct BwdFfnArgs {
    const void *x, *dh, *dy_routed;
    const int32_t *offsets, *sorted_token, *slot_of;
    const void *w1_r, *w3_r, *w2_r, *w1_s, *w3_s, *w2_s;
    void *da_r, *dp_r, *dq_r, *a_r, *da_s, *dp_s, *dq_s, *a_s;
    float *dxr, *dxs, *dx_ffn;
    float *dw1_r, *dw3_r, *dw2_r, *dw1_s, *dw3_s, *dw2_s;
};
hipError_t launch_expert_backward(const moe_problem &p, const BwdFfnArgs &a, hipStream_t s);

hipError_t launch_route_backward(const moe_problem &p, int groups, float alpha1, float alpha2,
                                 const void *x, const float *centroids, const float *probs,
                                 const int32_t *idx, const float *dgate, const float *f,
                                 const float *f_dev, const void *dh, const float *dx_ffn, float *dx,
                                 float *dcentroids, float *dbias, float *dz, float *part,
                                 hipStream_t s);

}  // namespace moe
