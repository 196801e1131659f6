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
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const uint4 q = *(const uint4 *)p;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16);
        v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
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
    *(uint4 *)p = q;
}
__device__ __forceinline__ void store8(float *p, const float v[8]) {
    *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4 *)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
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

// One workgroup of 256 threads.  f and f' are exact functions of integer
// counts (fp64 quotient rounded once to fp32); ExpBal and DevBal are fp64
// sums: strided per-thread sums, a butterfly within each wave, then the four
// wave sums in order (a fixed order, so deterministic).
__device__ __forceinline__ double block_sum4(double v, double *s_w) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = v;
    __syncthreads();
    return ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

__global__ __launch_bounds__(256) void balance_stats_kernel(int T, int Nr, int K, int D,
                                                            const int32_t *__restrict__ counts,
                                                            const float *__restrict__ prob_sum,
                                                            float *__restrict__ f, float *__restrict__ P,
                                                            float *__restrict__ f_dev,
                                                            float *__restrict__ P_dev,
                                                            float *__restrict__ exp_bal,
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
    const double e_all = block_sum4(eb, s_a);
    const double d_all = block_sum4(db, s_b);
    if (threadIdx.x == 0) {
        *exp_bal = (float)e_all;
        *dev_bal = (float)d_all;
    }
}

}  // namespace

hipError_t launch_combine(const moe_problem &p, const void *x, const void *y_routed,
                          const float *y_shared, const float *gate, const int32_t *slot_of, void *h,
                          hipStream_t s) {
    const int64_t n = (int64_t)p.T * (p.d / 8);
    if (n == 0) return hipSuccess;
    const int grid = (int)((n + 255) / 256);
    if (p.dtype == MOE_BF16)
        combine_kernel<uint16_t><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, (const uint16_t *)x,
                                                      (const uint16_t *)y_routed, y_shared, gate, slot_of,
                                                      (uint16_t *)h);
    else
        combine_kernel<float><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, (const float *)x, (const float *)y_routed,
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

}  // namespace moe
