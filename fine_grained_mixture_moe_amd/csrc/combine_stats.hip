// combine_stats.hip -- layer output and balance statistics on gfx950.
//
// Layer output, "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化",
// section "Method details: formulas and load balance" (output formula):
//   h_t = u_t + sum_{shared} FFN_i(u_t) + sum_k g_{t,k} FFN_{idx[t,k]}(u_t)
// Each thread owns 8 consecutive hidden units of one token and gathers the
// token's K' routed rows in k order (fp32, deterministic); HBM-bound, 16-byte
// accesses.
//
// Balance terms, same page and section (expert-level and device-level balance
// losses) with the symbols of "【论文总结】MoE" sections 2.3 and 2.4.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

// The combine reads and writes every row once: non-temporal accesses (nt), which stream past
// the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const u32x4_t q = __builtin_nontemporal_load((const u32x4_t *)p);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const f32x4_t a = __builtin_nontemporal_load((const f32x4_t *)p);
    const f32x4_t b = __builtin_nontemporal_load((const f32x4_t *)(p + 4));
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ void store8(uint16_t *p, const float v[8]) {
    uint4 q;
    q.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    q.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    q.z = (uint32_t)f2bf(v[4]) | ((uint32_t)f2bf(v[5]) << 16);
    q.w = (uint32_t)f2bf(v[6]) | ((uint32_t)f2bf(v[7]) << 16);
    u32x4_t w;
    w.x = q.x; w.y = q.y; w.z = q.z; w.w = q.w;
    __builtin_nontemporal_store(w, (u32x4_t *)p);
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
    f32x4_t a, b;
    a.x = v[0]; a.y = v[1]; a.z = v[2]; a.w = v[3];
    b.x = v[4]; b.y = v[5]; b.z = v[6]; b.w = v[7];
    __builtin_nontemporal_store(a, (f32x4_t *)p);
    __builtin_nontemporal_store(b, (f32x4_t *)(p + 4));
}

template <typename DT>
__global__ __launch_bounds__(256) void combine_kernel(int T, int d, int K, const DT *__restrict__ x,
                                                      const DT *__restrict__ y_routed,
                                                      const float *__restrict__ y_shared,
                                                      const float *__restrict__ gate,
                                                      const int32_t *__restrict__ slot_of,
                                                      DT *__restrict__ h) {
    const int per_tok = d / 8;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)T * per_tok) return;
    const int t = (int)(i / per_tok);
    const int c = (int)(i % per_tok) * 8;
    float acc[8];
    if (y_shared) {
        load8(y_shared + (size_t)t * d + c, acc);
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    }
    // k in batches of 4: the batch's slots and gates, then its rows, are
    // loaded before any use (independent loads in flight); the sums still run
    // in k order
    constexpr int KB = 4;
    for (int k0 = 0; k0 < K; k0 += KB) {
        int slot[KB];
        float g[KB];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            const bool in = k0 + u < K;
            slot[u] = in ? slot_of[(size_t)t * K + k0 + u] : -1;
            g[u] = in ? gate[(size_t)t * K + k0 + u] : 0.0f;
        }
        float y[KB][8];
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            if (slot[u] >= 0) load8(y_routed + (size_t)slot[u] * d + c, y[u]);
        }
#pragma unroll
        for (int u = 0; u < KB; ++u) {
            if (slot[u] < 0) continue;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] = __builtin_fmaf(g[u], y[u][j], acc[j]);
        }
    }
    float u[8];
    load8(x + (size_t)t * d + c, u);
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = u[j] + acc[j];
    store8(h + (size_t)t * d + c, acc);
}

// One workgroup of 256 threads (balance_stats_block, moe_internal.h).
__global__ __launch_bounds__(256) void balance_stats_kernel(int T, int Nr, int K, int D,
                                                            const int32_t *__restrict__ counts,
                                                            const float *__restrict__ prob_sum,
                                                            float *__restrict__ f, float *__restrict__ P,
                                                            float *__restrict__ f_dev,
                                                            float *__restrict__ P_dev,
                                                            float *__restrict__ exp_bal,
                                                            float *__restrict__ dev_bal) {
    balance_stats_block(T, Nr, K, D, counts, prob_sum, f, P, f_dev, P_dev, exp_bal, dev_bal);
}

// Workgroup 0: balance_stats_block; workgroups 1.. clear ctl[0, nctl) (what the fused expert
// FFN's preparation kernel does in gather mode), so the two share one kernel boundary.
__global__ __launch_bounds__(256) void layer_stats_ctl_kernel(int T, int Nr, int K, int D,
                                                              const int32_t *__restrict__ counts,
                                                              const float *__restrict__ prob_sum,
                                                              float *__restrict__ f, float *__restrict__ P,
                                                              float *__restrict__ f_dev,
                                                              float *__restrict__ P_dev,
                                                              float *__restrict__ exp_bal,
                                                              float *__restrict__ dev_bal, int32_t *ctl,
                                                              int nctl) {
    if (blockIdx.x == 0) {
        balance_stats_block(T, Nr, K, D, counts, prob_sum, f, P, f_dev, P_dev, exp_bal, dev_bal);
        return;
    }
    const int stride = (int)(gridDim.x - 1) * 256;
    for (int i = (int)(blockIdx.x - 1) * 256 + (int)threadIdx.x; i < nctl; i += stride) ctl[i] = 0;
}

}  // namespace

hipError_t launch_combine(const moe_problem &p, const void *x, const void *y_routed,
                          const float *y_shared, const float *gate, const int32_t *slot_of, void *h,
                          hipStream_t s) {
    const int64_t n = (int64_t)p.T * (p.d / 8);
    if (n == 0) return hipSuccess;
    const int grid = (int)((n + 255) / 256);
    // no y_routed: the accumulating expert FFN already added the routed terms into y_shared
    const int K = y_routed ? p.top_k : 0;
    if (p.dtype == MOE_BF16)
        combine_kernel<uint16_t><<<grid, 256, 0, s>>>(p.T, p.d, K, (const uint16_t *)x,
                                                      (const uint16_t *)y_routed, y_shared, gate, slot_of,
                                                      (uint16_t *)h);
    else
        combine_kernel<float><<<grid, 256, 0, s>>>(p.T, p.d, K, (const float *)x, (const float *)y_routed,
                                                   y_shared, gate, slot_of, (float *)h);
    return hipGetLastError();
}

hipError_t launch_balance_stats(const moe_problem &p, int groups, const int32_t *counts,
                                const float *prob_sum, float *f, float *P, float *f_dev, float *P_dev,
                                float *exp_bal, float *dev_bal, hipStream_t s) {
    balance_stats_kernel<<<1, 256, 0, s>>>(p.T, p.n_routed, p.top_k, groups, counts, prob_sum, f, P, f_dev,
                                           P_dev, exp_bal, dev_bal);
    return hipGetLastError();
}

hipError_t launch_layer_stats_ctl(const moe_problem &p, int groups, const int32_t *counts,
                                  const float *prob_sum, float *f, float *P, float *f_dev,
                                  float *P_dev, float *exp_bal, float *dev_bal, int32_t *ctl, int nctl,
                                  hipStream_t s) {
    const int grid = 1 + std::min(std::max((nctl + 255) / 256, 1), 64);
    layer_stats_ctl_kernel<<<grid, 256, 0, s>>>(p.T, p.n_routed, p.top_k, groups, counts, prob_sum, f, P,
                                                f_dev, P_dev, exp_bal, dev_bal, ctl, nctl);
    return hipGetLastError();
}

}  // namespace moe
