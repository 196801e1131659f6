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
    size_t gate_sorted;    // fp32   [T*K']              gates in grouped order (accumulating expert FFN)
    size_t ffn_ctl;        // int32  [ffn_ctl_ints]      fused expert FFN: queue heads, error flag, per-run counters
    size_t total;
};

// Control words of the fused expert FFN launch: kFfnQueues queue heads, an
// error flag (index kFfnCtlErr), and one counter per token run; a group of c
// rows has ceil(c/128) runs at most, so sum_g ceil(c_g/128) <= T K'/128 + N'
// (+ T/128 shared).
constexpr int kFfnQueues = 8;
constexpr int kFfnCtlErr = kFfnQueues;
inline int ffn_ctl_ints(const moe_problem &p) {
    const int64_t runs = (p.n_shared > 0 ? cdiv(p.T, 128) : 0) +
                         (p.n_routed > 0 ? ((int64_t)p.T * p.top_k) / 128 + p.n_routed : 0);
    return (int)(kFfnQueues + 1 + runs);
}

// Routing workgroups for T tokens of hidden size d (route.hip).
int route_blocks(int T, int d, int Nr);

inline WsLayout ws_layout(const moe_problem &p) {
    WsLayout L{};
    const size_t nr = (size_t)p.n_routed;
    const size_t rb = p.T > 0 ? (size_t)route_blocks(p.T, p.d, p.n_routed) : 0;
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
    L.gate_sorted = take((size_t)p.T * p.top_k * sizeof(float));
    L.ffn_ctl = take((size_t)ffn_ctl_ints(p) * sizeof(int32_t));
    L.total = off;
    return L;
}

// ---- balance statistics of one workgroup (moe_balance_stats, and the decode tail of
//      moe_layer_forward): "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化",
//      section "Method details: formulas and load balance" (expert- and device-level balance
//      losses), with the symbols of "【论文总结】MoE" sections 2.3 and 2.4 ----
// One workgroup of 256 threads.  f and f' are exact functions of integer
// counts (fp64 quotient rounded once to fp32); ExpBal and DevBal are fp64
// sums: strided per-thread sums, a butterfly within each wave, then the four
// wave sums in order (a fixed order, so deterministic).
__device__ __forceinline__ double stats_block_sum4(double v, double *s_w) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

// One workgroup of 256 threads for expert r: counts[r] = sum_b part_counts[b, r] and
// prob_sum[r] = sum_b part_psum[b, r] over the nblk routing workgroups, in fp64: strided
// per-thread sums, a butterfly within each wave, then the 4 wave sums in order (fixed order).
__device__ inline void route_reduce_block(int r, int nblk, int Nr, const int32_t *__restrict__ part_counts,
                                          const double *__restrict__ part_psum, int32_t *__restrict__ counts,
                                          float *__restrict__ prob_sum) {
    __shared__ double s_p[4];
    __shared__ long long s_c[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double a = 0.0;
    long long c = 0;
    for (int b = threadIdx.x; b < nblk; b += 256) {
        a += part_psum[(size_t)b * Nr + r];
        c += part_counts[(size_t)b * Nr + r];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        a += __shfl_xor(a, o, 64);
        c += __shfl_xor(c, o, 64);
    }
    if (lane == 0) { s_p[wave] = a; s_c[wave] = c; }
    __syncthreads();
    if (threadIdx.x == 0) {
        counts[r] = (int32_t)(s_c[0] + s_c[1] + s_c[2] + s_c[3]);
        prob_sum[r] = (float)(((s_p[0] + s_p[1]) + s_p[2]) + s_p[3]);
    }
}

__device__ inline void balance_stats_block(int T, int Nr, int K, int D, const int32_t *counts,
                                           const float *prob_sum, float *__restrict__ f,
                                           float *__restrict__ P, float *__restrict__ f_dev,
                                           float *__restrict__ P_dev, float *__restrict__ exp_bal,
                                           float *__restrict__ dev_bal) {
    __shared__ double s_a[4], s_b[4];
    __shared__ double s_P[kPermuteMaxExperts];
    __shared__ int s_c[kPermuteMaxExperts];
    const int gsz = Nr / D;
    double eb = 0.0, db = 0.0;
    for (int r = threadIdx.x; r < Nr; r += 256) {
        const int c = counts[r];
        const double fr = T > 0 ? ((double)Nr * (double)c) / ((double)K * (double)T) : 0.0;
        const double pr = T > 0 ? (double)prob_sum[r] / (double)T : 0.0;
        const float ff = (float)fr, pf = (float)pr;
        f[r] = ff;
        P[r] = pf;
        s_P[r] = pr;
        s_c[r] = c;
        eb += (double)ff * (double)pf;
    }
    __syncthreads();
    for (int g = threadIdx.x; g < D; g += 256) {
        int64_t C = 0;
        double ps = 0.0;
        for (int r = g * gsz; r < (g + 1) * gsz; ++r) {
            C += s_c[r];
            ps += s_P[r];
        }
        const double fg = T > 0 ? ((double)Nr * (double)C) / ((double)K * (double)T * (double)gsz) : 0.0;
        const float ff = (float)fg, pf = (float)ps;
        f_dev[g] = ff;
        P_dev[g] = pf;
        db += (double)ff * (double)pf;
    }
    const double e_all = stats_block_sum4(eb, s_a);
    const double d_all = stats_block_sum4(db, s_b);
    if (threadIdx.x == 0) {
        *exp_bal = (float)e_all;
        *dev_bal = (float)d_all;
    }
}

// ---- launchers (each returns hipSuccess or the launch error) -------------

// reduce = false leaves the partials unsummed (moe_layer_forward's decode tail sums them)
hipError_t launch_route(const moe_problem &p, int skip, const void *x, const float *centroids,
                        const float *bias, int32_t *idx, float *gate, float *probs,
                        int32_t *part_counts, double *part_psum,
                        int32_t *counts, float *prob_sum, hipStream_t s, bool reduce = true);
// True when the routing of p takes the decode kernel (one workgroup per token, nblk = T).
bool route_decode_batch(const moe_problem &p);

// Allocation-free routing: bytes of the static device scratch that holds the
// routing partials, and its address on the current device (taken once per
// device).
constexpr size_t kRouteScratchBytes = (size_t)4 << 20;
hipError_t route_scratch_ptr(void **ptr);
// Bytes of the routing partials (counts, then fp64 sums) for p, laid out as
// in the workspace: counts at 0, sums at route_psum_offset(p).
inline size_t route_psum_offset(const moe_problem &p) {
    const size_t rb = p.T > 0 ? (size_t)route_blocks(p.T, p.d, p.n_routed) : 0;
    return align_up(rb * (size_t)p.n_routed * sizeof(int32_t), 256);
}
inline size_t route_partial_bytes(const moe_problem &p) {
    const size_t rb = p.T > 0 ? (size_t)route_blocks(p.T, p.d, p.n_routed) : 0;
    return route_psum_offset(p) + rb * (size_t)p.n_routed * sizeof(double);
}

hipError_t launch_route_hash(const moe_problem &p, const int32_t *token_ids, int32_t *idx, float *gate,
                             int32_t *counts, hipStream_t s);

// The routing's reduction over its nblk workgroups' partials (route_reduce_block), when
// launch_permute runs it beside its histogram (moe_layer_forward).
struct RouteReduce {
    int nblk;
    const int32_t *part_counts;
    const double *part_psum;
    int32_t *counts;
    float *prob_sum;
};
// rr: also run the routing's reduction, in the histogram's launch; only with more than
// kPermuteTokens tokens and routed pairs (else hipErrorInvalidValue, nothing launched).
hipError_t launch_permute(const moe_problem &p, const int32_t *idx, int32_t *offsets,
                          int32_t *sorted_token, int32_t *slot_of, int32_t *hist,
                          int32_t *base, hipStream_t s, const RouteReduce *rr = nullptr);
// The decode tail of moe_layer_forward (T <= kPermuteTokens, decode routing, T K' > 0): two
// independent workgroups. One groups the pairs (the single-block permute) and clears the nctl
// control words of the fused expert FFN; the other counts each expert's selections in idx, sums
// the affinity partials of the T decode workgroups into prob_sum (the order of
// route_reduce_kernel) and runs the balance statistics on them.
hipError_t launch_layer_decode_tail(const moe_problem &p, int groups, const double *part_psum,
                                    int32_t *counts, float *prob_sum,
                                    const int32_t *idx, int32_t *offsets, int32_t *sorted_token,
                                    int32_t *slot_of, float *f, float *P, float *f_dev, float *P_dev,
                                    float *exp_bal, float *dev_bal, int32_t *ctl, int nctl, hipStream_t s);

struct FfnArgs {
    const void *x;
    const int32_t *offsets;
    const int32_t *sorted_token;
    const void *w1_r, *w3_r, *w2_r;
    const void *w1_s, *w3_s, *w2_s;
    void *act_shared, *act_routed;
    void *y_routed;
    float *y_shared;
    // accumulating mode (moe_expert_ffn with y_routed == NULL): y_acc [T, d]
    // receives the whole expert sum (zeroed first); the gates and slots of
    // the (t, k) pairs and the workspace's grouped-order gate array.
    // Null outside that mode.
    float *y_acc;
    const float *gate;
    const int32_t *slot_of;
    float *gate_sorted;
};

// up: act = SiLU(X W1^T) * (X W3^T) into the workspace; down: y = act W2^T.
hipError_t launch_expert_up(const moe_problem &p, const FfnArgs &a, hipStream_t s);
hipError_t launch_expert_down(const moe_problem &p, const FfnArgs &a, hipStream_t s);
// both projections: bf16 as one fused persistent launch (ctl: the workspace's
// control words), fp32 as the two launches above.  A preparation kernel
// always runs first: it clears the control words (so the error flag reports
// this call only) and, in accumulating mode, zeroes y_acc and writes the
// gates in grouped order.  p may have no active part (then only the
// preparation runs).
// prep = false: the control words are already clear (moe_layer_forward's decode tail cleared
// them; gather mode only).
hipError_t launch_expert_ffn(const moe_problem &p, const FfnArgs &a, int32_t *ctl, hipStream_t s,
                             bool prep = true);
// name of the kernel (template instantiation) launch_expert_ffn runs for p
const char *expert_ffn_kernel_name(const moe_problem &p, bool accum);
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
// The balance statistics and the clearing of the fused expert FFN's nctl control words in one
// launch (moe_layer_forward beyond decode batches, gather mode): workgroup 0 runs
// balance_stats_block, the others clear the words. Both only need the routing's counts.
hipError_t launch_layer_stats_ctl(const moe_problem &p, int groups, const int32_t *counts,
                                  const float *prob_sum, float *f, float *P, float *f_dev,
                                  float *P_dev, float *exp_bal, float *dev_bal, int32_t *ctl, int nctl,
                                  hipStream_t s);

// ---- backward pass (backward.hip) ------------------------------------------

// Token chunks of the centroid-gradient partial sums.
int route_backward_chunks(int T);

// Byte offsets of the backward scratch inside the caller's backward workspace.
struct BwdWsLayout {
    size_t da_r, dp_r, dq_r, a_r;   // dtype [T*K', w]
    size_t da_s, dp_s, dq_s, a_s;   // dtype [T, K_s*w]
    size_t dxr;                     // dtype [T*K', d]   dx of every grouped row
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
    L.dxr = take(tk * p.d * es);
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
    void *dxr;
    float *dxs, *dx_ffn;
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
