// route.hip -- gating of the DeepSeekMoE layer on gfx950.
//
// "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section "Method
// details: formulas and load balance": gates come from the Top-k of the
// token-to-expert affinities s_{j,t}, and only routed experts are selected;
// "【论文总结】MoE" section 2.2: the affinity is computed against a learnable
// centroid e_i per expert.
//
// Large batches: one launch (route_kernel) computes logits, softmax, Top-K'
// and partial statistics per 16 tokens.  Small batches: three launches:
//   1. logits: z[T x N'] in fp32 as a register-tiled SIMT GEMM (lane = token,
//      a wave's experts read as LDS broadcasts).  Every z_{t,r} is ONE fused
//      multiply-add chain over k = 0..d-1 in ascending order starting from +0,
//      so the value - and therefore the selected experts - is reproducible
//      bit for bit on any IEEE host.  No MFMA and no split-K: both would
//      change the summation order.
//   2. select: one wave per token adds the bias, computes softmax over the
//      routed experts (max/sum butterflies) and selects the Top-K' by repeated
//      wave argmax on a 64-bit key (ordered logit bits, then inverted expert
//      index), so equal logits go to the lower index and -0.0 ties +0.0; each
//      workgroup writes its per-expert token counts and fp64 affinity sums
//      (tokens in order).
//   3. reduce (both shapes): one workgroup per expert sums the partials in a
//      fixed order.
// No atomics: results are identical on every run.
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

// Softmax over the routed experts and Top-K' selection for one token whose
// logits (before bias) the wave holds: lane l has experts l + 64 j.  Writes
// idx/gate (and probs), and adds the token's affinities and selections to
// the lane's running per-expert sums ps / cnt.
template <int NJ>
__device__ __forceinline__ void finish_token(int t, int Nr, int K, int lane, float (&z)[NJ], const bool (&ev)[NJ],
                                             const float *__restrict__ bias, int32_t *__restrict__ idx,
                                             float *__restrict__ gate, float *__restrict__ probs,
                                             double (&ps)[NJ], int (&cnt)[NJ]) {
    float e[NJ], s[NJ];
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        if (bias && ev[j]) z[j] = z[j] + bias[lane + 64 * j];
        if (ev[j]) m = fmaxf(m, z[j]);
    }
    m = wave_max(m);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        e[j] = ev[j] ? expf(z[j] - m) : 0.0f;
        sum += e[j];
    }
    sum = wave_sum(sum);
    const float inv = 1.0f / sum;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        s[j] = e[j] * inv;
        ps[j] += (double)s[j];
        if (ev[j] && probs) probs[(size_t)t * Nr + lane + 64 * j] = s[j];
    }
    // Top-K' by repeated wave argmax on key = (ordered z) << 32 | ~r
    uint32_t taken = 0;
    for (int k = 0; k < K; ++k) {
        uint64_t best = 0;  // below every real key (ordered keys of finite z are > 0)
        float best_s = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (!ev[j] || (taken >> j & 1u)) continue;
            const uint32_t r = (uint32_t)(lane + 64 * j);
            const uint64_t key = ((uint64_t)ordered_key(z[j]) << 32) | (uint32_t)(~r);
            if (key > best) { best = key; best_s = s[j]; }
        }
        const uint64_t win = wave_max_u64(best);
        const int r = (int)(~(uint32_t)win);
        const int owner = r & 63;
        const float g = __shfl(best_s, owner, 64);
        if (lane == owner) {
            taken |= 1u << (r >> 6);
#pragma unroll
            for (int j = 0; j < NJ; ++j) cnt[j] += (j == (r >> 6)) ? 1 : 0;
        }
        if (lane == 0) {
            idx[(size_t)t * K + k] = r;
            gate[(size_t)t * K + k] = g;
        }
    }
}

// Per-workgroup partial statistics: the 4 waves' per-expert sums combined in
// wave order (fixed), written to part_* at row blockIdx.x.
template <int NJ>
__device__ __forceinline__ void write_partials(int Nr, int wave, int lane, const double (&ps)[NJ],
                                               const int (&cnt)[NJ], double (*s_ps)[NJ * 64],
                                               int (*s_cnt)[NJ * 64], int32_t *__restrict__ part_counts,
                                               double *__restrict__ part_psum) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        s_ps[wave][lane + 64 * j] = ps[j];
        s_cnt[wave][lane + 64 * j] = cnt[j];
    }
    __syncthreads();
    for (int r = threadIdx.x; r < Nr; r += blockDim.x) {
        double a = 0.0;
        int c = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) { a += s_ps[w][r]; c += s_cnt[w][r]; }
        part_psum[(size_t)blockIdx.x * Nr + r] = a;
        part_counts[(size_t)blockIdx.x * Nr + r] = c;
    }
}

// One wave owns RT tokens and all N' experts: lane l holds experts l + 64 j
// (j < NJ).  Every (token, expert) logit is one fma chain over k ascending.
// The four waves of a workgroup share each KC-wide chunk of the centroids and
// of their 4*RT token rows through LDS (fp32, double-buffered, one barrier
// per chunk; row pitch KC+4 floats keeps the 16-byte centroid reads of 16
// consecutive lanes on distinct banks; token reads are wave-uniform
// broadcasts).  After the chain the wave holds every logit of its tokens in
// registers: softmax and Top-K' need no LDS round trip.
template <int RT, int NJ, int KC>
__global__ __launch_bounds__(256) void route_kernel(
    int T, int d, int Nr, int K, const void *__restrict__ x, int x_bf16,
    const float *__restrict__ E, const float *__restrict__ bias, int32_t *__restrict__ idx,
    float *__restrict__ gate, float *__restrict__ probs, int32_t *__restrict__ part_counts,
    double *__restrict__ part_psum) {
    constexpr int NE = NJ * 64;            // expert rows covered by a wave
    constexpr int TB = 4 * RT;             // tokens of the workgroup
    constexpr int PITCH = KC + 4;          // LDS row pitch (floats)
    constexpr int NL = NE * KC / 4 / 256;  // centroid float4 staged per thread per chunk
    constexpr int NX = TB * KC / 8;        // threads staging 8 token values each
    static_assert(NL >= 1 && NX <= 256, "chunk shape");
    __shared__ __attribute__((aligned(16))) float s_e[2][NE * PITCH];
    __shared__ __attribute__((aligned(16))) float s_x[2][TB * PITCH];
    __shared__ double s_ps[4][NE];
    __shared__ int s_cnt[4][NE];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int tb0 = blockIdx.x * TB;
    const int t0 = tb0 + wave * RT;

    bool ev[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) ev[j] = lane + 64 * j < Nr;

    float acc[RT][NJ];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = 0.0f;

    // staging registers: centroid float4s, and 8 token values (thread < NX)
    float4 stage[NL];
    float xst[8];
    const int xt = tid / (KC / 8), xk = (tid % (KC / 8)) * 8;   // token row / k offset staged by this thread
    const size_t xrow = (size_t)min(tb0 + xt, T - 1) * d;
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int c = tid + 256 * q;
            const int row = c / (KC / 4), c4 = c % (KC / 4);
            stage[q] = row < Nr ? *(const float4 *)(E + (size_t)row * d + k0 + 4 * c4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (tid < NX) {
            if (x_bf16) {
                const uint4 w = *(const uint4 *)((const uint16_t *)x + xrow + k0 + xk);
                const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xst[2 * h] = __uint_as_float(wv[h] << 16);
                    xst[2 * h + 1] = __uint_as_float(wv[h] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4 *)((const float *)x + xrow + k0 + xk);
                const float4 b = *(const float4 *)((const float *)x + xrow + k0 + xk + 4);
                xst[0] = a.x; xst[1] = a.y; xst[2] = a.z; xst[3] = a.w;
                xst[4] = b.x; xst[5] = b.y; xst[6] = b.z; xst[7] = b.w;
            }
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < NL; ++q) {
            const int c = tid + 256 * q;
            const int row = c / (KC / 4), c4 = c % (KC / 4);
            *(float4 *)&s_e[buf][row * PITCH + 4 * c4] = stage[q];
        }
        if (tid < NX) {
            *(float4 *)&s_x[buf][xt * PITCH + xk] = make_float4(xst[0], xst[1], xst[2], xst[3]);
            *(float4 *)&s_x[buf][xt * PITCH + xk + 4] = make_float4(xst[4], xst[5], xst[6], xst[7]);
        }
    };

    const int nchunk = d / KC;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kc = 0; kc < nchunk; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nchunk) gload((kc + 1) * KC);
        if (t0 < T) {
#pragma unroll
            for (int v = 0; v < KC / 4; ++v) {
                float4 e4[NJ];
#pragma unroll
                for (int j = 0; j < NJ; ++j) e4[j] = *(const float4 *)&s_e[buf][(lane + 64 * j) * PITCH + 4 * v];
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const float4 x4 = *(const float4 *)&s_x[buf][(wave * RT + i) * PITCH + 4 * v];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        acc[i][j] = __builtin_fmaf(x4.x, e4[j].x, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(x4.y, e4[j].y, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(x4.z, e4[j].z, acc[i][j]);
                        acc[i][j] = __builtin_fmaf(x4.w, e4[j].w, acc[i][j]);
                    }
                }
            }
        }
        if (kc + 1 < nchunk) sstore(buf ^ 1);
        __syncthreads();
    }

    double ps[NJ];
    int cnt[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { ps[j] = 0.0; cnt[j] = 0; }

#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int t = t0 + i;
        if (t >= T) break;
        float z[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) z[j] = acc[i][j];
        finish_token<NJ>(t, Nr, K, lane, z, ev, bias, idx, gate, probs, ps, cnt);
    }

    write_partials<NJ>(Nr, wave, lane, ps, cnt, s_ps, s_cnt, part_counts, part_psum);
}

// Logits.  A workgroup owns 64 tokens x 4*EW experts: lane = token, wave w
// the experts 4*EW*blockIdx.y + EW*w + (0..EW-1).  Every z_{t,r} is one fp32
// fma chain over k = 0..d-1 in ascending order from +0 (the bias is added
// by the select kernel).  The workgroup streams KC-wide chunks of its 64
// token rows (converted to fp32, shared by the 4 waves; row pitch KC+4 keeps
// the 16-byte per-lane reads on distinct banks) and of its experts' centroid
// rows (read as wave-uniform broadcasts) through double-buffered LDS.
template <int EW, int KC>
__global__ __launch_bounds__(256) void route_logits_kernel(int T, int d, int Nr, const void *__restrict__ x,
                                                           int x_bf16, const float *__restrict__ E,
                                                           float *__restrict__ z) {
    constexpr int NE = 4 * EW;           // experts of the workgroup
    constexpr int XP = KC + 4;           // token row pitch (floats)
    constexpr int XV = 64 * KC / 8 / 256;  // 8-value token pieces per thread
    constexpr int EV = (NE * KC / 4 + 255) / 256;  // centroid float4 per thread
    static_assert(XV >= 1, "chunk shape");
    __shared__ __attribute__((aligned(16))) float s_x[2][64 * XP];
    __shared__ __attribute__((aligned(16))) float s_e[2][NE * KC];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = blockIdx.x * 64, r0 = blockIdx.y * NE;

    float xs[XV][8];
    float4 es[EV];
    auto gload = [&](int k0) {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int c = tid + 256 * v;                // piece: token c / (KC/8), k offset 8*(c % (KC/8))
            const int tt = c / (KC / 8), kk = (c % (KC / 8)) * 8;
            const int t = t0 + tt;
            if (t >= T) {
#pragma unroll
                for (int j = 0; j < 8; ++j) xs[v][j] = 0.0f;
            } else if (x_bf16) {
                const uint4 w = *(const uint4 *)((const uint16_t *)x + (size_t)t * d + k0 + kk);
                const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xs[v][2 * h] = __uint_as_float(wv[h] << 16);
                    xs[v][2 * h + 1] = __uint_as_float(wv[h] & 0xffff0000u);
                }
            } else {
                const float4 a = *(const float4 *)((const float *)x + (size_t)t * d + k0 + kk);
                const float4 b = *(const float4 *)((const float *)x + (size_t)t * d + k0 + kk + 4);
                xs[v][0] = a.x; xs[v][1] = a.y; xs[v][2] = a.z; xs[v][3] = a.w;
                xs[v][4] = b.x; xs[v][5] = b.y; xs[v][6] = b.z; xs[v][7] = b.w;
            }
        }
#pragma unroll
        for (int q = 0; q < EV; ++q) {
            const int c = tid + 256 * q;
            es[q] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (c < NE * KC / 4) {
                const int e = c / (KC / 4), c4 = c % (KC / 4);
                if (r0 + e < Nr) es[q] = *(const float4 *)(E + (size_t)(r0 + e) * d + k0 + 4 * c4);
            }
        }
    };
    auto sstore = [&](int b) {
#pragma unroll
        for (int v = 0; v < XV; ++v) {
            const int c = tid + 256 * v;
            const int tt = c / (KC / 8), kk = (c % (KC / 8)) * 8;
            *(float4 *)&s_x[b][tt * XP + kk] = make_float4(xs[v][0], xs[v][1], xs[v][2], xs[v][3]);
            *(float4 *)&s_x[b][tt * XP + kk + 4] = make_float4(xs[v][4], xs[v][5], xs[v][6], xs[v][7]);
        }
#pragma unroll
        for (int q = 0; q < EV; ++q)
            if (tid + 256 * q < NE * KC / 4) *(float4 *)&s_e[b][(tid + 256 * q) * 4] = es[q];
    };

    float acc[EW];
#pragma unroll
    for (int e = 0; e < EW; ++e) acc[e] = 0.0f;
    const int nchunk = d / KC;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kc = 0; kc < nchunk; ++kc) {
        const int b = kc & 1;
        if (kc + 1 < nchunk) gload((kc + 1) * KC);
#pragma unroll 4
        for (int v = 0; v < KC / 4; ++v) {
            const float4 x4 = *(const float4 *)&s_x[b][lane * XP + 4 * v];
#pragma unroll
            for (int e = 0; e < EW; ++e) {
                const float4 e4 = *(const float4 *)&s_e[b][(wave * EW + e) * KC + 4 * v];
                acc[e] = __builtin_fmaf(x4.x, e4.x, acc[e]);
                acc[e] = __builtin_fmaf(x4.y, e4.y, acc[e]);
                acc[e] = __builtin_fmaf(x4.z, e4.z, acc[e]);
                acc[e] = __builtin_fmaf(x4.w, e4.w, acc[e]);
            }
        }
        if (kc + 1 < nchunk) sstore(b ^ 1);
        __syncthreads();
    }
    const int t = t0 + lane;
    if (t < T)
#pragma unroll
        for (int e = 0; e < EW; ++e) {
            const int r = r0 + wave * EW + e;
            if (r < Nr) z[(size_t)t * Nr + r] = acc[e];
        }
}

// Select.  One wave per token (its shuffle chains are latency-bound, so
// tokens run in parallel waves), 4 per workgroup: add the bias, softmax,
// Top-K', and the per-workgroup partial statistics (waves in a fixed order).
template <int NJ>
__global__ __launch_bounds__(256) void route_select_kernel(int T, int Nr, int K, const float *__restrict__ z,
                                                           const float *__restrict__ bias,
                                                           int32_t *__restrict__ idx, float *__restrict__ gate,
                                                           float *__restrict__ probs,
                                                           int32_t *__restrict__ part_counts,
                                                           double *__restrict__ part_psum) {
    __shared__ double s_ps[4][NJ * 64];
    __shared__ int s_cnt[4][NJ * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    bool ev[NJ];
    double ps[NJ];
    int cnt[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { ev[j] = lane + 64 * j < Nr; ps[j] = 0.0; cnt[j] = 0; }
    const int t = blockIdx.x * 4 + wave;
    if (t < T) {
        float zz[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) zz[j] = ev[j] ? z[(size_t)t * Nr + lane + 64 * j] : 0.0f;
        finish_token<NJ>(t, Nr, K, lane, zz, ev, bias, idx, gate, probs, ps, cnt);
    }
    write_partials<NJ>(Nr, wave, lane, ps, cnt, s_ps, s_cnt, part_counts, part_psum);
}

// One workgroup per expert: counts[r] = sum_b part_counts[b, r],
// prob_sum[r] = sum_b part_psum[b, r] in fp64: strided per-thread sums, a
// butterfly within each wave, then the 4 wave sums in order (fixed order).
__global__ __launch_bounds__(256) void route_reduce_kernel(
    int nblk, int Nr, const int32_t *__restrict__ part_counts, const double *__restrict__ part_psum,
    int32_t *__restrict__ counts, float *__restrict__ prob_sum) {
    __shared__ double s_p[4];
    __shared__ long long s_c[4];
    const int r = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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

}  // namespace

// Two shapes of the same computation (identical fma chains, so identical
// results):
//   T >= 8192: route_kernel, lane = expert, 4 tokens per wave, centroid
//     chunks staged once per 16 tokens (each LDS read feeds 4 token chains);
//   T <  8192: route_logits_kernel + route_select_kernel, lane = token, so
//     even a decode batch spreads over many workgroups (2 experts per wave
//     from 2048 tokens, else 1), then one wave per token selects.
constexpr int kRouteTiledT = 8192;

int route_blocks(int T) { return T >= kRouteTiledT ? cdiv(T, 16) : cdiv(T, 4); }

hipError_t launch_route(const moe_problem &p, const void *x, const float *centroids,
                        const float *bias, int32_t *idx, float *gate, float *probs, float *z,
                        int32_t *part_counts, double *part_psum, int32_t *counts,
                        float *prob_sum, hipStream_t s) {
    const int nblk = p.T > 0 ? route_blocks(p.T) : 0;
    const int xb = p.dtype == MOE_BF16;
    const int nj = cdiv(p.n_routed, 64);
    if (nblk > 0) {
        if (p.T >= kRouteTiledT) {
#define MOE_ARGS p.T, p.d, p.n_routed, p.top_k, x, xb, centroids, bias, idx, gate, probs, part_counts, part_psum
            if (nj == 1) route_kernel<4, 1, 32><<<nblk, 256, 0, s>>>(MOE_ARGS);
            else if (nj == 2) route_kernel<4, 2, 32><<<nblk, 256, 0, s>>>(MOE_ARGS);
            else route_kernel<4, 4, 16><<<nblk, 256, 0, s>>>(MOE_ARGS);
#undef MOE_ARGS
        } else {
            // chunk of 128 when it divides d (d is a multiple of 64), else 64
            const bool k128 = p.d % 128 == 0;
            if (p.T >= 2048) {
                const dim3 grid(cdiv(p.T, 64), cdiv(p.n_routed, 8));
                if (k128) route_logits_kernel<2, 128><<<grid, 256, 0, s>>>(p.T, p.d, p.n_routed, x, xb, centroids, z);
                else route_logits_kernel<2, 64><<<grid, 256, 0, s>>>(p.T, p.d, p.n_routed, x, xb, centroids, z);
            } else {
                const dim3 grid(cdiv(p.T, 64), cdiv(p.n_routed, 4));
                if (k128) route_logits_kernel<1, 128><<<grid, 256, 0, s>>>(p.T, p.d, p.n_routed, x, xb, centroids, z);
                else route_logits_kernel<1, 64><<<grid, 256, 0, s>>>(p.T, p.d, p.n_routed, x, xb, centroids, z);
            }
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
#define MOE_SEL(NJ) route_select_kernel<NJ><<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, z, bias, idx, gate, \
                                                                 probs, part_counts, part_psum)
            if (nj == 1) MOE_SEL(1);
            else if (nj == 2) MOE_SEL(2);
            else MOE_SEL(4);
#undef MOE_SEL
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    route_reduce_kernel<<<p.n_routed, 256, 0, s>>>(nblk, p.n_routed, part_counts, part_psum, counts, prob_sum);
    return hipGetLastError();
}

}  // namespace moe
