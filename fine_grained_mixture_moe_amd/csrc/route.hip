// route.hip -- gating of the DeepSeekMoE layer on gfx950.
//
// "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section "Method
// details: formulas and load balance": gates come from the Top-k of the
// token-to-expert affinities s_{j,t}, and only routed experts are selected;
// "【论文总结】MoE" section 2.2: the affinity is computed against a learnable
// centroid e_i per expert.
//
// One workgroup (256 threads, 4 wave64) owns 64 tokens and all N' experts:
//   1. logits z[64 x N'] as a register-tiled SIMT GEMM in fp32.  Every
//      z_{t,r} is ONE fused multiply-add chain over k = 0..d-1 in ascending
//      order starting from +0 (then + bias_r), so the value - and therefore
//      the selected experts - is reproducible bit for bit on any IEEE host.
//      No MFMA and no split-K: both would change the summation order.
//   2. per token, one wave computes softmax over the routed experts
//      (max/sum butterflies) and selects the Top-K' by repeated wave argmax
//      on a 64-bit key (ordered logit bits, then inverted expert index), so
//      equal logits go to the lower index and -0.0 ties +0.0.
//   3. the workgroup writes its per-expert token counts and affinity sums
//      (fp64, tokens in order); a second one-block kernel reduces the
//      partials over workgroups in a fixed order (only integer LDS atomics,
//      whose result does not depend on order).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int KC = 32;  // k-chunk staged in LDS

// Order-preserving map fp32 -> uint32 (larger float -> larger key); zero is
// canonicalised so that -0.0 and +0.0 get the same key.
__device__ __forceinline__ uint32_t ordered_key(float z) {
    uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
        uint64_t w = ((uint64_t)hi << 32) | lo;
        v = w > v ? w : v;
    }
    return v;
}

// NRP: N' padded to a multiple of 64 (64, 128 or 256).
template <int NRP>
__global__ __launch_bounds__(256) void route_kernel(
    int T, int d, int Nr, int K, const void *__restrict__ x, int x_bf16,
    const float *__restrict__ E, const float *__restrict__ bias, int32_t *__restrict__ idx,
    float *__restrict__ gate, float *__restrict__ probs, int32_t *__restrict__ part_counts,
    double *__restrict__ part_psum) {
    constexpr int TB = kRouteTokens;      // 64 tokens
    constexpr int EG = NRP / 4;           // expert groups of 4 consecutive experts
    constexpr int TG = 256 / EG;          // token groups
    constexpr int RT = TB / TG;           // tokens per thread
    constexpr int NJ = NRP / 64;          // experts per lane in the selection phase

    __shared__ float xs[KC][TB];
    __shared__ __attribute__((aligned(16))) float es[KC][NRP];
    __shared__ float zs[TB][NRP + 1];
    __shared__ int cnt[NRP];

    const int tid = threadIdx.x;
    const int t0 = blockIdx.x * TB;
    const int eg = tid % EG, tg = tid / EG;

    float acc[RT][4];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < d; k0 += KC) {
        // x chunk [TB x KC] -> xs[k][t]; 8 consecutive k of one token per thread
        {
            const int tt = tid >> 2, kk = (tid & 3) * 8;
            const int t = t0 + tt;
            float v[8];
            if (t >= T) {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = 0.0f;
            } else if (x_bf16) {
                const uint4 q = *(const uint4 *)((const uint16_t *)x + (size_t)t * d + k0 + kk);
                const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[2 * j] = __uint_as_float(w[j] << 16);
                    v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4 *)((const float *)x + (size_t)t * d + k0 + kk);
                const float4 b = *(const float4 *)((const float *)x + (size_t)t * d + k0 + kk + 4);
                v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
                v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) xs[kk + j][tt] = v[j];
        }
        // E chunk [NRP x KC] -> es[k][r]
        for (int c = tid; c < NRP * (KC / 4); c += 256) {
            const int r = c / (KC / 4), kq = (c % (KC / 4)) * 4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < Nr) v = *(const float4 *)(E + (size_t)r * d + k0 + kq);
            es[kq + 0][r] = v.x;
            es[kq + 1][r] = v.y;
            es[kq + 2][r] = v.z;
            es[kq + 3][r] = v.w;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < KC; ++k) {
            const float4 ev = *(const float4 *)&es[k][eg * 4];
#pragma unroll
            for (int i = 0; i < RT; ++i) {
                const float xv = xs[k][tg + i * TG];
                acc[i][0] = __builtin_fmaf(xv, ev.x, acc[i][0]);
                acc[i][1] = __builtin_fmaf(xv, ev.y, acc[i][1]);
                acc[i][2] = __builtin_fmaf(xv, ev.z, acc[i][2]);
                acc[i][3] = __builtin_fmaf(xv, ev.w, acc[i][3]);
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = eg * 4 + j;
            float z = acc[i][j];
            if (bias && r < Nr) z = z + bias[r];
            zs[tg + i * TG][r] = z;
        }
    for (int r = tid; r < NRP; r += 256) cnt[r] = 0;
    __syncthreads();

    // ---- per-token softmax + Top-K' (one wave per token) ----
    const int wave = tid >> 6, lane = tid & 63;
    for (int tt = wave; tt < TB; tt += 4) {
        const int t = t0 + tt;
        if (t >= T) break;
        float z[NJ], e[NJ];
        bool valid[NJ];
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = lane + 64 * j;
            valid[j] = r < Nr;
            z[j] = zs[tt][r];
            if (valid[j]) m = fmaxf(m, z[j]);
        }
        m = wave_max(m);
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            e[j] = valid[j] ? expf(z[j] - m) : 0.0f;
            sum += e[j];
        }
        sum = wave_sum(sum);
        const float inv = 1.0f / sum;
        float s[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            s[j] = e[j] * inv;
            const int r = lane + 64 * j;
            if (valid[j] && probs) probs[(size_t)t * Nr + r] = s[j];
        }
        // Top-K' by repeated wave argmax.  key = (ordered z) << 32 | ~r.
        uint32_t taken = 0;
        for (int k = 0; k < K; ++k) {
            uint64_t best = 0;  // below every real key (ordered keys of finite z are > 0)
            float best_s = 0.0f;
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                if (!valid[j] || (taken >> j & 1u)) continue;
                const uint32_t r = (uint32_t)(lane + 64 * j);
                const uint64_t key = ((uint64_t)ordered_key(z[j]) << 32) | (uint32_t)(~r);
                if (key > best) { best = key; best_s = s[j]; }
            }
            const uint64_t win = wave_max_u64(best);
            const int r = (int)(~(uint32_t)win);
            const int owner = r & 63;
            const float g = __shfl(best_s, owner, 64);
            if (lane == owner) taken |= 1u << (r >> 6);
            if (lane == 0) {
                idx[(size_t)t * K + k] = r;
                gate[(size_t)t * K + k] = g;
                atomicAdd(&cnt[r], 1);  // integer: order-independent result
            }
        }
        // keep s for the per-block affinity sums
#pragma unroll
        for (int j = 0; j < NJ; ++j) zs[tt][lane + 64 * j] = s[j];
    }
    __syncthreads();

    // ---- per-block partial statistics (tokens in order, fp64) ----
    const int nt = min(TB, T - t0);
    for (int r = tid; r < Nr; r += 256) {
        double ps = 0.0;
        for (int tt = 0; tt < nt; ++tt) ps += (double)zs[tt][r];
        part_psum[(size_t)blockIdx.x * Nr + r] = ps;
        part_counts[(size_t)blockIdx.x * Nr + r] = cnt[r];
    }
}

// counts[r] = sum_b part_counts[b, r]; prob_sum[r] = sum_b part_psum[b, r] (fp64, b ascending)
__global__ __launch_bounds__(256) void route_reduce_kernel(
    int nblk, int Nr, const int32_t *__restrict__ part_counts, const double *__restrict__ part_psum,
    int32_t *__restrict__ counts, float *__restrict__ prob_sum) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= Nr) return;
    int64_t c = 0;
    double ps = 0.0;
    for (int b = 0; b < nblk; ++b) {
        c += part_counts[(size_t)b * Nr + r];
        ps += part_psum[(size_t)b * Nr + r];
    }
    counts[r] = (int32_t)c;
    prob_sum[r] = (float)ps;
}

}  // namespace

hipError_t launch_route(const moe_problem &p, const void *x, const float *centroids,
                        const float *bias, int32_t *idx, float *gate, float *probs,
                        int32_t *part_counts, double *part_psum, int32_t *counts,
                        float *prob_sum, hipStream_t s) {
    const int nblk = cdiv(p.T, kRouteTokens);
    const int xb = p.dtype == MOE_BF16;
    if (nblk > 0) {
        if (p.n_routed <= 64)
            route_kernel<64><<<nblk, 256, 0, s>>>(p.T, p.d, p.n_routed, p.top_k, x, xb, centroids, bias,
                                                  idx, gate, probs, part_counts, part_psum);
        else if (p.n_routed <= 128)
            route_kernel<128><<<nblk, 256, 0, s>>>(p.T, p.d, p.n_routed, p.top_k, x, xb, centroids, bias,
                                                   idx, gate, probs, part_counts, part_psum);
        else
            route_kernel<256><<<nblk, 256, 0, s>>>(p.T, p.d, p.n_routed, p.top_k, x, xb, centroids, bias,
                                                   idx, gate, probs, part_counts, part_psum);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    route_reduce_kernel<<<cdiv(p.n_routed, 256), 256, 0, s>>>(nblk, p.n_routed, part_counts, part_psum,
                                                              counts, prob_sum);
    return hipGetLastError();
}

}  // namespace moe
