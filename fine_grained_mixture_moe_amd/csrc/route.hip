// route.hip -- gating of the DeepSeekMoE layer on gfx950.
//
// "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section "Method
// details: formulas and load balance": gates come from the Top-k of the
// token-to-expert affinities s_{j,t}, and only routed experts are selected;
// "【论文总结】MoE" section 2.2: the affinity is computed against a learnable
// centroid e_i per expert.
//
// Three launches: the centroids are copied into a blocked layout (see
// route_kernel), one launch computes logits, softmax, Top-K' and
// per-workgroup partial statistics, and one sums the partials in a fixed
// order.
//
// Logits.  Every z_{t,r} is ONE fused multiply-add chain over k = 0..d-1 in
// ascending order starting from +0, so the value - and therefore the
// selected experts - is reproducible bit for bit on any IEEE host.  No MFMA
// and no split of k: both would change the summation order.  The work is
// T*N' independent chains of length d; the kernel is built so that nothing
// but the fma issue rate bounds it:
//   * lane = expert (l + 64 j for j < NJ), a wave owns RT consecutive tokens,
//     so each lane runs RT*NJ independent chains;
//   * the token values are the same in every lane, so they feed the fma as
//     its scalar operand: the wave loads its RT token rows in 128-byte
//     chunks (one 16-byte piece per lane, ordinary vector loads issued 3
//     to 4 chunks ahead), and each step moves the packed bf16 pairs it needs to
//     SGPRs with v_readlane (one VALU op per two fmas of a lane's chain) and
//     unpacks them on the scalar unit.  Scalar loads would save that op but
//     return out of order, so a wave could not keep several in flight;
//   * each lane streams its centroid values from L2 through a ring of P
//     register stages (loads issued P steps of 8 k ahead), reused by the
//     wave's RT tokens; no LDS and no barrier in the chain.
// Measured on MI355X (why not more tokens per wave): with one wave per SIMD
// an fma with independent neighbours still costs ~9-11 cycles of issue, with
// 2-4 waves per SIMD ~5, so the kernel trades centroid reuse for waves.
//
// Selection, per token, with the wave holding every logit (bias added) of it:
//   * softmax over the routed experts: maximum and sum by DPP row reductions
//     (fixed order, so deterministic), fp32 exp;
//   * Top-K' on key = order-preserving uint32 image of z (-0 and +0 equal):
//     the K'-th largest key tau is found by a 32-step radix search on wave
//     ballots; keys above tau are taken, and of the keys equal to tau the
//     lowest expert indices; each taken expert's place in idx[t, :] is the
//     number of taken experts ahead of it in (z desc, r asc) order.
// The per-expert counts and fp64 affinity sums run over the wave's tokens in
// order, then over the 4 waves in order.
#include <algorithm>

#include "moe_internal.h"

namespace moe {
namespace {

// Order-preserving map fp32 -> uint32 (larger float -> larger key); zero is
// canonicalised so that -0.0 and +0.0 get the same key.  Every finite z maps
// above 0, the key of an absent expert.
__device__ __forceinline__ uint32_t ordered_key(float z) {
    const uint32_t u = __float_as_uint(z == 0.0f ? 0.0f : z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP controls (within rows of 16 lanes)
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i of 8 <- lane 7-i
constexpr int kRowMirror = 0x140;     // lane i of 16 <- lane 15-i

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// After these four steps every lane of a row of 16 holds the row's result.
__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp<kQuadSwap1>(v));
    v = fmaxf(v, dpp<kQuadSwap2>(v));
    v = fmaxf(v, dpp<kRowHalfMirror>(v));
    return fmaxf(v, dpp<kRowMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dpp<kQuadSwap1>(v);
    v += dpp<kQuadSwap2>(v);
    v += dpp<kRowHalfMirror>(v);
    return v + dpp<kRowMirror>(v);
}
__device__ __forceinline__ float lane_value(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_max(float v) {
    v = row_max(v);
    return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum(v);
    return ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
}
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Softmax and Top-K' of the wave's tokens t0 .. t0+nt-1 (nt <= RT);
// acc[i][j] is the logit (before bias) of token t0+i and expert lane + 64 j.
// The RT tokens go through every phase together, so the latencies of their
// cross-lane steps overlap.  Adds each token's affinities and selections, in
// token order, to the lane's running ps / cnt.
template <int RT, int NJ>
__device__ __forceinline__ void finish_tokens(int t0, int nt, int Nr, int K, int lane, const float (&acc)[RT][NJ],
                                              const float *__restrict__ bias, int32_t *__restrict__ idx,
                                              float *__restrict__ gate, float *__restrict__ probs,
                                              double (&ps)[NJ], int (&cnt)[NJ]) {
    bool ev[NJ];
    float b[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = lane + 64 * j;
        ev[j] = r < Nr;
        b[j] = (bias && ev[j]) ? bias[r] : 0.0f;
    }
    float z[RT][NJ], s[RT][NJ];
    uint32_t key[RT][NJ];
    float m[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        m[i] = -INFINITY;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            z[i][j] = bias ? acc[i][j] + b[j] : acc[i][j];   // one fp32 add, only with a bias
            if (ev[j]) m[i] = fmaxf(m[i], z[i][j]);
            key[i][j] = ev[j] ? ordered_key(z[i][j]) : 0u;
        }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) m[i] = wave_max(m[i]);
    float part[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        part[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            s[i][j] = ev[j] ? expf(z[i][j] - m[i]) : 0.0f;
            part[i] += s[i][j];
        }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const float inv = 1.0f / wave_sum(part[i]);
        if (i >= nt) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            s[i][j] *= inv;
            ps[j] += (double)s[i][j];
            if (ev[j] && probs) probs[(size_t)(t0 + i) * Nr + lane + 64 * j] = s[i][j];
        }
    }

    // tau[i] = the K-th largest key of token i (counted with multiplicity)
    uint32_t tau[RT];
#pragma unroll
    for (int i = 0; i < RT; ++i) tau[i] = 0;
    for (int bit = 31; bit >= 0; --bit) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const uint32_t cand = tau[i] | (1u << bit);
            int c = 0;
#pragma unroll
            for (int j = 0; j < NJ; ++j) c += __popcll(__builtin_amdgcn_ballot_w64(key[i][j] >= cand));
            tau[i] = c >= K ? cand : tau[i];
        }
    }
    // taken: keys above tau, then keys equal to tau by lowest index
    bool sel[RT][NJ];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        int above = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) above += __popcll(__builtin_amdgcn_ballot_w64(key[i][j] > tau[i]));
        const int need = K - above;   // >= 1
        int eq_before = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const uint64_t eq = __builtin_amdgcn_ballot_w64(key[i][j] == tau[i]);
            sel[i][j] = key[i][j] > tau[i] || (key[i][j] == tau[i] && eq_before + lanes_below(eq) < need);
            eq_before += __popcll(eq);
        }
    }
    // place of each taken expert in idx[t, :]: taken experts with a larger
    // key, or an equal key and a lower index, come first.  Every token has
    // exactly K taken experts, so the K rounds serve all tokens at once.
    int place[RT][NJ];
    uint64_t mask[RT][NJ];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            place[i][j] = 0;
            mask[i][j] = __builtin_amdgcn_ballot_w64(sel[i][j]);
        }
    for (int round = 0; round < K; ++round) {
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            // next taken expert of token i: lowest set bit of the first non-empty group
            int js = 0;
#pragma unroll
            for (int j = NJ - 1; j >= 0; --j)
                if (mask[i][j]) js = j;
            uint64_t mj = mask[i][0];
#pragma unroll
            for (int j = 1; j < NJ; ++j)
                if (js == j) mj = mask[i][j];
            const int ls = __builtin_ctzll(mj);
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                if (js == j) mask[i][j] &= mask[i][j] - 1;
            uint32_t kv = key[i][0];
#pragma unroll
            for (int j = 1; j < NJ; ++j)
                if (js == j) kv = key[i][j];
            const uint32_t ks = (uint32_t)__builtin_amdgcn_readlane((int)kv, ls);
            const int rs = ls + 64 * js;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                place[i][j] += (ks > key[i][j] || (ks == key[i][j] && rs < lane + 64 * j)) ? 1 : 0;
        }
    }
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        if (i >= nt) continue;
        const size_t t = (size_t)(t0 + i);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            if (sel[i][j]) {
                idx[t * K + place[i][j]] = lane + 64 * j;
                gate[t * K + place[i][j]] = s[i][j];
                cnt[j] += 1;
            }
    }
}

// RT tokens per wave, NJ expert lanes per lane, P register stages of 8 k of
// centroids, PX stages of 128-byte token chunks.  The centroids come in the
// blocked layout Eb[d/8][N'][8]: one step of a wave's 64 experts is one
// contiguous 2 KB span (row-major rows would put the 64 lanes of every load
// d*4 bytes apart; measured 2-3x slower at d >= 2048).
template <int RT, int NJ, int P, int PX, bool XB>
__global__ __launch_bounds__(256) void route_kernel(int T, int d, int Nr, int K, const void *__restrict__ x,
                                                    const float *__restrict__ E, const float *__restrict__ bias,
                                                    int32_t *__restrict__ idx, float *__restrict__ gate,
                                                    float *__restrict__ probs, int32_t *__restrict__ part_counts,
                                                    double *__restrict__ part_psum) {
    constexpr int SPC = XB ? 8 : 4;   // steps of 8 k in a 128-byte token chunk
    static_assert(RT <= 8, "one chunk load per wave");
    static_assert((PX * SPC) % P == 0, "centroid ring slots repeat every PX chunks");
    static_assert(P <= PX * SPC, "ring within a chunk group");
    __shared__ double s_ps[4][NJ * 64];
    __shared__ int s_cnt[4][NJ * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int t0 = (blockIdx.x * 4 + wave) * RT;

    double ps[NJ];
    int cnt[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { ps[j] = 0.0; cnt[j] = 0; }

    if (t0 < T) {
        // this lane's experts in the blocked centroids (absent experts read expert Nr-1; their logits are dropped)
        const float *erow[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) erow[j] = E + (size_t)min(lane + 64 * j, Nr - 1) * 8;
        const size_t estep = (size_t)Nr * 8;   // floats from one step to the next
        // token chunks: lane 8i+q (i < RT) holds bytes [16q, 16q+16) of token t0+i's
        // current 128-byte chunk (lanes past 8*RT repeat the last token; tokens
        // past T read row T-1 and are not finished)
        const int xi = min(lane >> 3, RT - 1), xq = lane & 7;
        const uint8_t *xrow = (const uint8_t *)x + (size_t)min(t0 + xi, T - 1) * d * (XB ? 2 : 4) + xq * 16;
        auto xload = [&](int c) -> uint4 { return *(const uint4 *)(xrow + (size_t)c * 128); };

        float acc[RT][NJ];
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[i][j] = 0.0f;

        float4 ering[P][NJ][2];
        auto eload = [&](int st, int pe) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                ering[pe][j][0] = *(const float4 *)(erow[j] + (size_t)st * estep);
                ering[pe][j][1] = *(const float4 *)(erow[j] + (size_t)st * estep + 4);
            }
        };
        // nch is a multiple of PX (the launcher's choice) and nst of P, so the
        // loop body has no branch: prefetches past the end re-read the last
        // chunk / step (clamped), which keeps the load order the same in every
        // iteration and lets each wait cover only the stage it consumes.
        const int nch = d / (SPC * 8);
        const int nst = d / 8;
        uint4 xring[PX];
#pragma unroll
        for (int pc = 0; pc < PX; ++pc) xring[pc] = xload(pc);
#pragma unroll
        for (int pe = 0; pe < P; ++pe) eload(pe, pe);

        for (int c0 = 0; c0 < nch; c0 += PX) {
#pragma unroll
            for (int pc = 0; pc < PX; ++pc) {
                const int c = c0 + pc;
                const uint4 xc = xring[pc];
#pragma unroll
                for (int q = 0; q < SPC; ++q) {
                    const int st = c * SPC + q;
                    const int pe = (pc * SPC + q) % P;
                    float ev[NJ][8];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const float4 a = ering[pe][j][0], b = ering[pe][j][1];
                        ev[j][0] = a.x; ev[j][1] = a.y; ev[j][2] = a.z; ev[j][3] = a.w;
                        ev[j][4] = b.x; ev[j][5] = b.y; ev[j][6] = b.z; ev[j][7] = b.w;
                    }
                    eload(min(st + P, nst - 1), pe);
                    // the RT tokens' words of this step, moved to scalar registers;
                    // then, for each k of the step, the fmas of all RT*NJ chains
                    // (independent, so back-to-back issue never waits on a result)
                    constexpr int NW = XB ? 4 : 8;
                    uint32_t w[RT][NW];
#pragma unroll
                    for (int i = 0; i < RT; ++i)
#pragma unroll
                        for (int h = 0; h < NW; ++h) {
                            const int src = XB ? i * 8 + q : i * 8 + 2 * q + (h >> 2);
                            const uint32_t v = (h & 3) == 0 ? xc.x : (h & 3) == 1 ? xc.y : (h & 3) == 2 ? xc.z : xc.w;
                            w[i][h] = (uint32_t)__builtin_amdgcn_readlane((int)v, src);
                        }
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                        for (int i = 0; i < RT; ++i) {
                            const float xv = XB ? __uint_as_float((kk & 1) ? (w[i][kk >> 1] & 0xffff0000u)
                                                                           : (w[i][kk >> 1] << 16))
                                                : __uint_as_float(w[i][kk]);
#pragma unroll
                            for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_fmaf(xv, ev[j][kk], acc[i][j]);
                        }
                    __builtin_amdgcn_sched_barrier(0);
                }
                // the chunk is consumed: its stage takes chunk c + PX
                xring[pc] = xload(min(c + PX, nch - 1));
            }
        }

        finish_tokens<RT, NJ>(t0, min(RT, T - t0), Nr, K, lane, acc, bias, idx, gate, probs, ps, cnt);
    }

    // the 4 waves' per-expert sums, combined in wave order, at row blockIdx.x
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        s_ps[wave][lane + 64 * j] = ps[j];
        s_cnt[wave][lane + 64 * j] = cnt[j];
    }
    __syncthreads();
    for (int r = threadIdx.x; r < Nr; r += 256) {
        double a = 0.0;
        int c = 0;
#pragma unroll
        for (int w = 0; w < 4; ++w) { a += s_ps[w][r]; c += s_cnt[w][r]; }
        part_psum[(size_t)blockIdx.x * Nr + r] = a;
        part_counts[(size_t)blockIdx.x * Nr + r] = c;
    }
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

// Tokens per wave: more waves per SIMD hide the chain and load latencies,
// more tokens per wave reuse each centroid load; measured best: 4 from 8192
// tokens, 2 from 1024, else 1.
int route_tokens_per_wave(int T) { return T >= 8192 ? 4 : T >= 1024 ? 2 : 1; }

// Centroid register stages: about 16 steps of lookahead in fmas per lane
// (RT*NJ*8 per step), at least 2, at most the steps of the token ring.  Token chunk
// stages: 4 chunks ahead when the chunk count allows it, else 1.
constexpr int ring_stages(int rt, int nj, int steps) {
    return (16 / (rt * nj) < 2 ? 2 : 16 / (rt * nj)) < steps ? (16 / (rt * nj) < 2 ? 2 : 16 / (rt * nj)) : steps;
}

template <int RT, int NJ, int PX, bool XB>
void launch_rtj(const moe_problem &p, int nblk, const void *x, const float *E, const float *bias, int32_t *idx,
                float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    constexpr int P = ring_stages(RT, NJ, PX * (XB ? 8 : 4));
    route_kernel<RT, NJ, P, PX, XB><<<nblk, 256, 0, s>>>(p.T, p.d, p.n_routed, p.top_k, x, E, bias, idx,
                                                               gate, probs, pc, pp);
}

template <int RT, bool XB>
void launch_rt(const moe_problem &p, int nblk, const void *x, const float *E, const float *bias, int32_t *idx,
               float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    const int nj = cdiv(p.n_routed, 64);
    const int nch = p.d / (XB ? 64 : 32);
#define MOE_L(NJ) (nch % 4 == 0 ? launch_rtj<RT, NJ, 4, XB>(p, nblk, x, E, bias, idx, gate, probs, pc, pp, s) \
                                : launch_rtj<RT, NJ, 1, XB>(p, nblk, x, E, bias, idx, gate, probs, pc, pp, s))
    if (nj == 1) MOE_L(1);
    else if (nj == 2) MOE_L(2);
    else MOE_L(4);
#undef MOE_L
}

template <bool XB>
void launch_route_typed(const moe_problem &p, int nblk, const void *x, const float *E, const float *bias,
                        int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    switch (route_tokens_per_wave(p.T)) {
        case 4: launch_rt<4, XB>(p, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        case 2: launch_rt<2, XB>(p, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        default: launch_rt<1, XB>(p, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
    }
}

// Centroids [N'][d] -> blocked [d/8][N'][8].
__global__ __launch_bounds__(256) void block_centroids_kernel(int Nr, int d, const float *__restrict__ E,
                                                              float *__restrict__ Eb) {
    const int64_t n = (int64_t)Nr * d / 4;   // float4 units (d % 64 == 0)
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t e = i * 4;
        const int r = (int)(e / d), k = (int)(e % d);
        *(float4 *)(Eb + ((int64_t)(k / 8) * Nr + r) * 8 + (k % 8)) = *(const float4 *)(E + e);
    }
}

}  // namespace

int route_blocks(int T) { return cdiv(T, 4 * route_tokens_per_wave(T)); }

hipError_t launch_route(const moe_problem &p, const void *x, const float *centroids, const float *bias,
                        int32_t *idx, float *gate, float *probs, float *centroids_blocked, int32_t *part_counts,
                        double *part_psum, int32_t *counts, float *prob_sum, hipStream_t s) {
    const int nblk = p.T > 0 ? route_blocks(p.T) : 0;
    if (nblk > 0) {
        const int64_t n4 = (int64_t)p.n_routed * p.d / 4;
        const int gb = (int)std::min<int64_t>((n4 + 255) / 256, 1024);
        block_centroids_kernel<<<gb, 256, 0, s>>>(p.n_routed, p.d, centroids, centroids_blocked);
        if (p.dtype == MOE_BF16)
            launch_route_typed<true>(p, nblk, x, centroids_blocked, bias, idx, gate, probs, part_counts, part_psum, s);
        else
            launch_route_typed<false>(p, nblk, x, centroids_blocked, bias, idx, gate, probs, part_counts, part_psum, s);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    route_reduce_kernel<<<p.n_routed, 256, 0, s>>>(nblk, p.n_routed, part_counts, part_psum, counts, prob_sum);
    return hipGetLastError();
}

}  // namespace moe
