// route.hip -- gating of the DeepSeekMoE layer on gfx950.
//
// "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section "Method
// details: formulas and load balance": gates come from the Top-k of the
// token-to-expert affinities s_{j,t}, and only routed experts are selected;
// "【论文总结】MoE" section 2.2: the affinity is computed against a learnable
// centroid e_i per expert.
//
// Two launches: one computes logits, softmax, Top-K' and per-workgroup
// partial statistics, one sums the partials in a fixed order.
//
// Logits.  Every z_{t,r} is ONE fused multiply-add chain over k = 0..d-1 in
// ascending order starting from +0, so the value - and therefore the
// selected experts - is reproducible bit for bit on any IEEE host.  No split
// of k: it would change the summation order.  For 65 to 128 experts the
// chains run on the matrix cores (route_mfma_kernel below: an fp32 MFMA adds
// each product as a fused multiply-add of its own, in k order); otherwise,
// and for decode batches, on the VALU.  The VALU work is T*N' independent
// chains of length d:
//   * lane = expert (l + 64 j for j < NJ), a wave owns RT consecutive tokens,
//     so each lane runs RT*NJ independent chains;
//   * the centroids are staged in LDS in chunks of 32 KB (KC values of k for
//     all experts), double-buffered, and every wave of the workgroup reads
//     them from there: one L2 read of E per workgroup instead of one per
//     wave.  A chunk is stored as slices of 8 k, each as two halves of 4 k,
//     [slice][half][expert][4]: a lane's 16-byte read of one half sits next
//     to its neighbours', so the 64 lanes read one contiguous 1 KB span (a
//     32-byte stride per lane would use half of each bank cycle); E itself
//     is read in its natural [N'][d] layout;
//   * the token values are the same in every lane.  Each wave loads its RT
//     token rows of a chunk with ordinary vector loads (one 16-byte piece
//     per lane, a chunk ahead); three forms then feed them to the fmas:
//     several tokens per wave (bf16): a DPP row broadcast inside the fma;
//     one token and one expert per lane: the chunk as fp32 in LDS, read by
//     all lanes at one address, so the single chain per lane issues its
//     fmas back to back on VGPR operands; otherwise: v_readlane to SGPRs
//     and the fma's scalar operand.  Scalar loads would save the readlane
//     but return out of order, and they share their wait counter with the
//     LDS reads.
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
#include <mutex>
#include <type_traits>
#include <utility>

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
__device__ __forceinline__ void finish_tokens(int t0, int nt, int Nr, int K, int skip, int lane,
                                              const float (&acc)[RT][NJ],
                                              const float *__restrict__ bias, int32_t *__restrict__ idx,
                                              float *__restrict__ gate, float *__restrict__ probs,
                                              double (&ps)[NJ], int (&cnt)[NJ]) {
    const int KS = K + skip;   // selected, then the first `skip` dropped
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
            tau[i] = c >= KS ? cand : tau[i];
        }
    }
    // taken: keys above tau, then keys equal to tau by lowest index
    bool sel[RT][NJ];
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        int above = 0;
#pragma unroll
        for (int j = 0; j < NJ; ++j) above += __popcll(__builtin_amdgcn_ballot_w64(key[i][j] > tau[i]));
        const int need = KS - above;   // >= 1
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
    for (int round = 0; round < KS; ++round) {
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
            if (sel[i][j] && place[i][j] >= skip) {   // the top `skip` are disabled
                idx[t * K + place[i][j] - skip] = lane + 64 * j;
                gate[t * K + place[i][j] - skip] = s[i][j];
                cnt[j] += 1;
            }
    }
}

// acc += x * e with x taken from lane ST of the lane's 16-lane row (DPP
// row_newbcast): the wave-uniform token value reaches every lane without a
// readlane; one fused multiply-add, the same rounding as fmaf.
//
// A DPP instruction must not read a VGPR that a VALU instruction wrote in the
// two wait states before it, and the compiler's hazard check does not see
// into inline asm.  The operands are covered by construction: the centroid
// values come straight from LDS loads (no VALU writer), the token values are
// unpacked once per chunk and fenced off by two wait states (compute_bcast),
// and an accumulator was last written by its chain's previous fma, C - 1
// fmas back for C interleaved chains, so the asm adds NOPS = max(0, 3 - C)
// wait states.  tests/test_route_dpp_hazards.py checks the generated code.
template <int ST, int NOPS>
__device__ __forceinline__ void fmac_row_bcast(float &acc, float x, float e) {
    if constexpr (NOPS == 0)
        asm volatile("v_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc)
                     : "v"(x), "v"(e), "i"(ST));
    else
        asm volatile("s_nop %4\n\tv_fmac_f32_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                     : "+v"(acc)
                     : "v"(x), "v"(e), "i"(ST), "i"(NOPS - 1));
}
template <typename F, int... S>
__device__ __forceinline__ void for_each_step(F &&f, std::integer_sequence<int, S...>) {
    (f(std::integral_constant<int, S>{}), ...);
}

// W waves of RT tokens; NJ experts per lane.  Centroid chunks of KC k for
// the padded NE = 64*NJ experts (64 B per thread: 32 KB with 8 waves) are
// double-buffered in LDS; each thread fills two 32-byte pieces (8 k of one
// expert), the KC/8 threads of an expert row reading its KC values
// contiguously.  The pad after each slice puts those writes on distinct
// banks.
template <int RT, int NJ, int W, bool XB>
__global__ __launch_bounds__(W * 64) void route_kernel(int T, int d, int Nr, int K, int skip, const void *x,
                                                        const float *E,
                                                        const float *__restrict__ bias,
                                                        int32_t *__restrict__ idx, float *__restrict__ gate,
                                                        float *__restrict__ probs, int32_t *__restrict__ part_counts,
                                                        double *__restrict__ part_psum) {
    constexpr int NT = W * 64;
    constexpr int NE = NJ * 64;
    constexpr int KC = 16 * NT / NE;         // k per chunk (two 32-byte fill pieces per thread)
    constexpr int SL = KC / 8;               // steps of 8 k per chunk
    static_assert(KC >= 8 && KC <= 128 && KC % 8 == 0, "chunk of whole steps");
    // slice pitch (bytes): the two halves of the slice, then a pad that puts
    // the fill writes of each 8 lanes (rows r, slices s) on distinct banks
    constexpr int SS = NE * 32 + 128 / (SL < 8 ? SL : 8);
    constexpr int FR = NE * SL / NT;         // 32-byte fill pieces per thread
    constexpr int ES = XB ? 2 : 4;           // token element bytes
    constexpr int PPT = KC * ES / 16;        // 16-byte token pieces per token and chunk
    constexpr int XPL = (RT * PPT + 63) / 64;
    constexpr int NW = XB ? 4 : 8;           // 32-bit token words per step
    static_assert(NE * SL % NT == 0, "whole fill rounds");
    static_assert(W * NE * (8 + 4) <= 2 * SL * SS, "statistics fit in the chunk stages");
    __shared__ __attribute__((aligned(16))) uint8_t s_e[2][SL * SS];
    // LDS form (one token, one expert per lane): the chunk's token values as fp32, per
    // stage and wave, read by all lanes at one address (a broadcast), so the
    // fmas take VGPR operands and the chain has no SGPR round trip
    constexpr bool LB = RT == 1 && NJ == 1;
    __shared__ __attribute__((aligned(16))) float s_xf[LB ? 2 * W * KC : 4];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = (blockIdx.x * W + wave) * RT;

    // ---- centroid fill: piece f of this thread is (expert row, slice) ----
    int frow[FR], fsl[FR];
    const float *fsrc[FR];
#pragma unroll
    for (int f = 0; f < FR; ++f) {
        const int pc = tid + f * NT;
        frow[f] = pc / SL;
        fsl[f] = pc % SL;
        fsrc[f] = E + (size_t)min(frow[f], Nr - 1) * d;   // rows of absent experts repeat row N'-1
    }
    // (named registers, not an array: the array ended up in scratch memory)
    static_assert(FR == 2, "two fill pieces per thread");
    float4 fe0a, fe0b, fe1a, fe1b;
    const float *fs0 = fsrc[0] + 8 * fsl[0], *fs1 = fsrc[1] + 8 * fsl[1];
    const int flim0 = d - 8 - 8 * fsl[0], flim1 = d - 8 - 8 * fsl[1];
    uint8_t *fd0 = &s_e[0][0] + fsl[0] * SS + frow[0] * 16, *fd1 = &s_e[0][0] + fsl[1] * SS + frow[1] * 16;
#define MOE_FILL_LOAD_TO(c, A0, B0, A1, B1)                           \
    {                                                                 \
        const float *a_ = fs0 + min((c) * KC, flim0);                 \
        const float *b_ = fs1 + min((c) * KC, flim1);                 \
        A0 = *(const float4 *)a_;                                     \
        B0 = *(const float4 *)(a_ + 4);                               \
        A1 = *(const float4 *)b_;                                     \
        B1 = *(const float4 *)(b_ + 4);                               \
    }
#define MOE_FILL_STORE_FROM(stg, A0, B0, A1, B1)                      \
    {                                                                 \
        const int o_ = (stg) * (SL * SS);                             \
        *(float4 *)(fd0 + o_) = A0;                                   \
        *(float4 *)(fd0 + o_ + NE * 16) = B0;                         \
        *(float4 *)(fd1 + o_) = A1;                                   \
        *(float4 *)(fd1 + o_ + NE * 16) = B1;                         \
    }
#define MOE_FILL_LOAD(c) MOE_FILL_LOAD_TO(c, fe0a, fe0b, fe1a, fe1b)
#define MOE_FILL_STORE(stg) MOE_FILL_STORE_FROM(stg, fe0a, fe0b, fe1a, fe1b)
    // ---- token pieces: piece p = i*PPT + q is bytes [16q, 16q+16) of token
    //      t0+i within the chunk; lane l holds pieces l + 64u ----
    //      (readlane form).  Broadcast form (bf16 tokens, RT >= 2): every
    //      16-lane row holds the chunk's pieces of all RT tokens, lane 16r+q
    //      piece q (one step of 8 k), so step q of the chunk broadcasts lane
    //      q of each row.  With a single token per wave the chain's DPP wait
    //      states are not hidden, and the readlane form is faster (decode
    //      batches: c5a 28.6 vs 29.4 us, c5c 76.7 vs 81.7 us) ----
    constexpr bool BC = XB && RT >= 2;
    constexpr int XR = BC ? RT : XPL;   // 16-byte pieces per lane and chunk
    const uint8_t *xsrc[XR];
    int xoff[XR];
#pragma unroll
    for (int u = 0; u < XR; ++u) {
        const int pc = BC ? u * PPT + min(lane & 15, PPT - 1) : lane + 64 * u;
        const int i = min(pc / PPT, RT - 1);
        xsrc[u] = (const uint8_t *)x + (size_t)max(min(t0 + i, T - 1), 0) * d * ES;
        xoff[u] = (pc % PPT) * 16;
    }
    // LDS form: lane l < PPT converts its 16-byte piece of the token (k
    // [l*16/ES, (l+1)*16/ES) of the chunk) to fp32 and stores it
#define MOE_XSTORE(stg, xr)                                                               \
    if constexpr (LB) {                                                                   \
        if (lane < PPT) {                                                                 \
            float *xd_ = s_xf + ((stg) * W + wave) * KC + lane * (16 / ES);               \
            const uint4 v_ = xr[0];                                                       \
            if constexpr (XB) {                                                           \
                *(float4 *)xd_ = make_float4(__uint_as_float(v_.x << 16),                 \
                                             __uint_as_float(v_.x & 0xffff0000u),         \
                                             __uint_as_float(v_.y << 16),                 \
                                             __uint_as_float(v_.y & 0xffff0000u));        \
                *(float4 *)(xd_ + 4) = make_float4(__uint_as_float(v_.z << 16),           \
                                                   __uint_as_float(v_.z & 0xffff0000u),   \
                                                   __uint_as_float(v_.w << 16),           \
                                                   __uint_as_float(v_.w & 0xffff0000u));  \
            } else {                                                                      \
                *(uint4 *)xd_ = v_;                                                       \
            }                                                                             \
        }                                                                                 \
    }
#define MOE_XLOAD(c, xr)                                                                  \
    _Pragma("unroll") for (int u = 0; u < XR; ++u)                                        \
        xr[u] = *(const uint4 *)(xsrc[u] + min((c) * KC * ES + xoff[u], d * ES - 16));

    float acc[RT][NJ];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = 0.0f;

    // NS steps of chunk stage stg with token words xc: per step, the wave's
    // centroid values from LDS, the RT tokens' words to SGPRs, then for each
    // k of the step the fmas of all RT*NJ chains (independent neighbours)
    auto compute_bcast = [&](auto ns_t, int stg, const uint4 (&xc)[XR]) {
        constexpr int NS = decltype(ns_t)::value;
        const uint8_t *eb = s_e[stg] + lane * 16;
        float x8[RT][8];   // the lane's piece of each token, as fp32
#pragma unroll
        for (int i = 0; i < RT; ++i) {
            const uint32_t wv[4] = {xc[i].x, xc[i].y, xc[i].z, xc[i].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                x8[i][2 * h] = __uint_as_float(wv[h] << 16);
                x8[i][2 * h + 1] = __uint_as_float(wv[h] & 0xffff0000u);
            }
        }
        // the unpacked token values are read through DPP: two wait states
        // after their last VALU write, with no instruction moved across
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 1");
        __builtin_amdgcn_sched_barrier(0);
        float4 ev[2][NJ][2];
        auto eread = [&](int st, float4 (&e)[NJ][2]) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                e[j][0] = *(const float4 *)(eb + st * SS + j * 64 * 16);
                e[j][1] = *(const float4 *)(eb + st * SS + j * 64 * 16 + NE * 16);
            }
        };
        eread(0, ev[0]);
        for_each_step(
            [&](auto st_t) {
                constexpr int ST = decltype(st_t)::value;
                if (ST + 1 < NS) eread(ST + 1, ev[(ST + 1) & 1]);
                float e8[NJ][8];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float4 a = ev[ST & 1][j][0], b = ev[ST & 1][j][1];
                    e8[j][0] = a.x; e8[j][1] = a.y; e8[j][2] = a.z; e8[j][3] = a.w;
                    e8[j][4] = b.x; e8[j][5] = b.y; e8[j][6] = b.z; e8[j][7] = b.w;
                }
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int i = 0; i < RT; ++i)
#pragma unroll
                        for (int j = 0; j < NJ; ++j)
                            fmac_row_bcast<ST, (RT * NJ >= 3 ? 0 : 3 - RT * NJ)>(acc[i][j], x8[i][kk], e8[j][kk]);
                __builtin_amdgcn_sched_barrier(0);
            },
            std::make_integer_sequence<int, NS>{});
    };
    auto compute = [&](auto ns_t, int stg, const uint4 (&xc)[XR]) {
        if constexpr (BC) {
            compute_bcast(ns_t, stg, xc);
        } else if constexpr (LB) {
            constexpr int NS = decltype(ns_t)::value;
            const uint8_t *eb = s_e[stg] + lane * 16;
            const float *xb = s_xf + (stg * W + wave) * KC;
            float4 ev[3][NJ][2], xv[3][2];   // step st in [st % 3]; steps st+1, st+2 are in flight
            auto rd = [&](int st, float4 (&e)[NJ][2], float4 (&xx)[2]) {
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    e[j][0] = *(const float4 *)(eb + st * SS + j * 64 * 16);
                    e[j][1] = *(const float4 *)(eb + st * SS + j * 64 * 16 + NE * 16);
                }
                xx[0] = *(const float4 *)(xb + 8 * st);
                xx[1] = *(const float4 *)(xb + 8 * st + 4);
            };
            rd(0, ev[0], xv[0]);
            if (NS > 1) rd(1, ev[1], xv[1]);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                if (st + 2 < NS) rd(st + 2, ev[(st + 2) % 3], xv[(st + 2) % 3]);
                const float4 xa = xv[st % 3][0], xb4 = xv[st % 3][1];
                const float x8[8] = {xa.x, xa.y, xa.z, xa.w, xb4.x, xb4.y, xb4.z, xb4.w};
                float e8[NJ][8];
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const float4 a = ev[st % 3][j][0], b = ev[st % 3][j][1];
                    e8[j][0] = a.x; e8[j][1] = a.y; e8[j][2] = a.z; e8[j][3] = a.w;
                    e8[j][4] = b.x; e8[j][5] = b.y; e8[j][6] = b.z; e8[j][7] = b.w;
                }
#pragma unroll
                for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[0][j] = __builtin_fmaf(x8[kk], e8[j][kk], acc[0][j]);
                // one step at a time (bounded registers; the reads above run
                // ahead): the empty asm takes the accumulators and clobbers
                // memory, so neither this step's fmas nor later steps' LDS
                // reads move across it
#pragma unroll
                for (int j = 0; j < NJ; ++j) asm volatile("" : "+v"(acc[0][j]) : : "memory");
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
        constexpr int NS = decltype(ns_t)::value;
        const uint8_t *eb = s_e[stg] + lane * 16;
        float4 ev[2][NJ][2];   // step st in ev[st & 1]; step st+1 is read while st computes
        auto eread = [&](int st, float4 (&e)[NJ][2]) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                e[j][0] = *(const float4 *)(eb + st * SS + j * 64 * 16);
                e[j][1] = *(const float4 *)(eb + st * SS + j * 64 * 16 + NE * 16);
            }
        };
        eread(0, ev[0]);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            if (st + 1 < NS) eread(st + 1, ev[(st + 1) & 1]);
            float e8[NJ][8];
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const float4 a = ev[st & 1][j][0], b = ev[st & 1][j][1];
                e8[j][0] = a.x; e8[j][1] = a.y; e8[j][2] = a.z; e8[j][3] = a.w;
                e8[j][4] = b.x; e8[j][5] = b.y; e8[j][6] = b.z; e8[j][7] = b.w;
            }
            uint32_t w[RT][NW];
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int h = 0; h < NW; ++h) {
                    const int pp = i * PPT + (XB ? st : 2 * st + (h >> 2));
                    const uint4 xv = xc[pp / 64];
                    const uint32_t v = (h & 3) == 0 ? xv.x : (h & 3) == 1 ? xv.y : (h & 3) == 2 ? xv.z : xv.w;
                    w[i][h] = (uint32_t)__builtin_amdgcn_readlane((int)v, pp % 64);
                }
#pragma unroll
            for (int kk = 0; kk < 8; ++kk)
#pragma unroll
                for (int i = 0; i < RT; ++i) {
                    const float xv = XB ? __uint_as_float((kk & 1) ? (w[i][kk >> 1] & 0xffff0000u)
                                                                   : (w[i][kk >> 1] << 16))
                                        : __uint_as_float(w[i][kk]);
#pragma unroll
                    for (int j = 0; j < NJ; ++j) acc[i][j] = __builtin_fmaf(xv, e8[j][kk], acc[i][j]);
                }
            // one step at a time: the scheduler would otherwise hoist every
            // step's readlanes and run out of SGPRs
            __builtin_amdgcn_sched_barrier(0);
        }
        }
    };

    // Full chunks in the loop: the loads of chunk c+1 (global -> registers)
    // go out before chunk c is computed, the compiler barrier keeps them
    // there, and they are stored to the other stage afterwards.  d % 64 == 0,
    // so only KC = 128 can leave a last chunk of 64 k; the last iteration
    // loads it (or re-loads the last full chunk into the idle stage).
    const int nchunk = (d + KC - 1) / KC, nfull = d / KC;
    // One token per wave in 4-wave blocks (small batches): a chunk's compute
    // is short, and in a layer step the centroids and tokens come from HBM
    // (the expert weights streamed through the caches since the last
    // routing), so with the next chunk's loads issued one chunk ahead every
    // chunk waits out a memory latency.  Four register sets keep three
    // chunks in flight: at chunk c the set c%4 holds c's token piece, the
    // others chunks c+1..c+3; after c is computed, c+1 goes to the other
    // stage and set c%4 is reloaded with chunk c+4.  Here KC <= 64 divides d
    // (d % 64 == 0), so every chunk is full; loads past the end repeat the
    // last chunk.  No branch in the loop skips a load and the loop has one
    // exit (with loads issued on some paths only, or a loop left from inside
    // the group, the wait counts before the LDS stores fall back to waiting
    // for loads issued a step earlier); steps past the last chunk skip only
    // their compute.  (Named registers through macros: as structs passed to
    // lambdas the sets were kept in scratch memory.)
    if constexpr (RT == 1 && W == 4) {
        static_assert(64 % KC == 0, "whole chunks");
        static_assert(XR == 1, "one token piece per lane and chunk");
#define MOE_SET(n) float4 n##a0, n##b0, n##a1, n##b1; uint4 n##x;
#define MOE_LD(c, n)                                                                     \
    {                                                                                    \
        const int cc_ = min((c), nchunk - 1);                                            \
        MOE_FILL_LOAD_TO(cc_, n##a0, n##b0, n##a1, n##b1)                                \
        n##x = *(const uint4 *)(xsrc[0] + min(cc_ * KC * ES + xoff[0], d * ES - 16));    \
    }
#define MOE_STEP(c, cur, nxt)                                                            \
    {                                                                                    \
        if ((c) < nchunk) {                                                              \
            const uint4 xa_[1] = {cur##x};                                               \
            compute(std::integral_constant<int, SL>{}, (c) & 1, xa_);                   \
        }                                                                                \
        MOE_FILL_STORE_FROM(((c) + 1) & 1, nxt##a0, nxt##b0, nxt##a1, nxt##b1)          \
        MOE_XSTORE(((c) + 1) & 1, (&nxt##x))                                             \
        MOE_LD((c) + 4, cur)                                                             \
        __syncthreads();                                                                 \
    }
        MOE_SET(q0) MOE_SET(q1) MOE_SET(q2) MOE_SET(q3)
        MOE_LD(0, q0)
        MOE_LD(1, q1)
        MOE_LD(2, q2)
        MOE_LD(3, q3)
        MOE_FILL_STORE_FROM(0, q0a0, q0b0, q0a1, q0b1)
        MOE_XSTORE(0, (&q0x))
        __syncthreads();
        for (int c = 0; c < nchunk; c += 4) {
            MOE_STEP(c, q0, q1)
            MOE_STEP(c + 1, q1, q2)
            MOE_STEP(c + 2, q2, q3)
            MOE_STEP(c + 3, q3, q0)
        }
#undef MOE_SET
#undef MOE_LD
#undef MOE_STEP
    } else {
    uint4 xc[XR], xn[XR];
    MOE_FILL_LOAD(0)
    MOE_XLOAD(0, xc)
    MOE_FILL_STORE(0)
    MOE_XSTORE(0, xc)
    __syncthreads();
    for (int c = 0; c < nfull; ++c) {
        const int cn = min(c + 1, nchunk - 1);
        MOE_FILL_LOAD(cn)
        MOE_XLOAD(cn, xn)
        // keeps the loads above ahead of the compute
        __builtin_amdgcn_sched_barrier(0);
        compute(std::integral_constant<int, SL>{}, c & 1, xc);
        MOE_FILL_STORE((c + 1) & 1)
        MOE_XSTORE((c + 1) & 1, xn)
#pragma unroll
        for (int u = 0; u < XR; ++u) xc[u] = xn[u];
        __syncthreads();
    }
    if (nfull < nchunk) compute(std::integral_constant<int, (SL / 2 > 0 ? SL / 2 : 1)>{}, nfull & 1, xc);
    }
#undef MOE_FILL_LOAD
#undef MOE_FILL_STORE
#undef MOE_FILL_LOAD_TO
#undef MOE_FILL_STORE_FROM
#undef MOE_XLOAD
#undef MOE_XSTORE

    double ps[NJ];
    int cnt[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { ps[j] = 0.0; cnt[j] = 0; }
    if (t0 < T)
        finish_tokens<RT, NJ>(t0, min(RT, T - t0), Nr, K, skip, lane, acc, bias, idx, gate, probs, ps, cnt);

    // the W waves' per-expert sums, combined in wave order, at row blockIdx.x
    // (the chunk stages are free after the last barrier of the loop)
    double *s_ps = (double *)&s_e[0][0];
    int *s_cnt = (int *)(s_ps + W * NE);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        s_ps[wave * NE + lane + 64 * j] = ps[j];
        s_cnt[wave * NE + lane + 64 * j] = cnt[j];
    }
    __syncthreads();
    for (int r = tid; r < Nr; r += NT) {
        double a = 0.0;
        int cc = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) { a += s_ps[w * NE + r]; cc += s_cnt[w * NE + r]; }
        part_psum[(size_t)blockIdx.x * Nr + r] = a;
        part_counts[(size_t)blockIdx.x * Nr + r] = cc;
    }
}

// Decode batches (few tokens): one workgroup per token and NW = ceil(N'/64)
// waves, wave w running the chains of experts 64w + lane.  Every lane's
// chain is sequential in k (the fixed fma order), so with few tokens the
// work is T*N' chains of d dependent fmas and the time is the chain length,
// as long as a wave issues little besides its fmas and never waits for data.
//   * Centroids: each wave streams its 64 expert rows in chunks of CK = 32 k
//     (8 KB) straight into LDS (buffer_load ... lds: no staging registers, no
//     LDS stores), S stages per wave, S - 2 chunks ahead of the one being
//     read, so that several chunks per wave are in flight against the memory
//     latency.  Load instruction i of a chunk fills rows 8i .. 8i+7 (1 KB,
//     lane L the 16 bytes at 16 L); the 16-byte piece q of row r sits at
//     piece q ^ (r & 7) ^ ((r >> 3) & 1) of the row, so the 16 lanes of a
//     row-wise read phase (rows r .. r+15 at one q) hit 16 distinct 4-bank
//     groups.  A wave waits for its own loads only (vmcnt): the waves of a
//     workgroup do not synchronise inside the k loop.
//   * Token: the row is converted to fp32 once into LDS; each chunk's values
//     are read at one address by all lanes (a broadcast).
//   * The LDS reads of chunk c+1 are interleaved with the fmas of chunk c
//     (after each half of them, the next chunk's pieces of that half, in
//     descending order), so every read is a whole chunk of fmas ahead of its
//     use, 8 reads are in flight at each wait (the counter holds 15), and a
//     chunk takes two waits.
// The logits of the NW waves meet in LDS and wave 0 runs the same softmax
// and Top-K' as the batched kernel.  The partial statistics go to row
// `token` of the partials (nblk = T).
constexpr int kRouteDecodeMaxD = 16384;
constexpr int kDecodeCK = 32;                          // k per chunk
constexpr int kDecodeChunk = 64 * kDecodeCK * 4;       // bytes of one chunk of one wave
constexpr size_t kDecodeLdsMax = 160 * 1024 - 1024;    // dynamic LDS budget (the logits take the rest)
// dynamic LDS of the decode kernel: NW waves x S stages, then the token row as fp32 and a zero chunk
constexpr size_t decode_lds_bytes(int NW, int S, int d) {
    return (size_t)NW * S * kDecodeChunk + ((size_t)d + kDecodeCK) * 4;
}
// stages per wave: as many as fit, up to 8 (at most 6 chunks, 48 loads, in flight)
int decode_stages(int NW, int d) {
    for (int S = 8; S >= 4; S -= 2)
        if (decode_lds_bytes(NW, S, d) <= kDecodeLdsMax) return S;
    return 0;
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
// Buffer descriptor (four dwords, the layout __builtin_amdgcn_make_buffer_rsrc
// builds): base, no stride, `bytes` in range; offsets at or past it read zeros.
__device__ __forceinline__ i32x4_t decode_rsrc(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4_t r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}
// Four loads of 16 bytes per lane straight into LDS: load i (immediate offset
// 1024 i) lane L writes LDS bytes [lds + 1024 i + 16 L, +16) and reads memory
// at voff[i] + soff + 1024 i (the immediate offset moves both addresses, so
// voff[i] carries -1024 i).  Inline asm, so the compiler neither tracks nor
// waits for them; the kernel waits for its own loads with s_waitcnt vmcnt.
// The s_nop is the wait state between the write of M0 and its first read.
__device__ __forceinline__ void decode_dma16x4(i32x4_t rsrc, uint32_t lds, const uint32_t *voff, uint32_t soff) {
    asm volatile("s_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %5, %6 offen lds\n\t"
                 "buffer_load_dwordx4 %2, %5, %6 offen offset:1024 lds\n\t"
                 "buffer_load_dwordx4 %3, %5, %6 offen offset:2048 lds\n\t"
                 "buffer_load_dwordx4 %4, %5, %6 offen offset:3072 lds"
                 :
                 : "{m0}"(lds), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(rsrc), "s"(soff)
                 : "memory");
}
__device__ __forceinline__ uint32_t decode_lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
// s_waitcnt vmcnt(VM), no wait on the other counters
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(VM >= 0 && VM < 64, "vmcnt immediate");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
}

template <int NW, int S, bool XB>
__global__ __launch_bounds__(NW * 64) void route_decode_kernel(int T, int d, int Nr, int K, int skip, const void *x,
                                                               const float *__restrict__ E,
                                                               const float *__restrict__ bias,
                                                               int32_t *__restrict__ idx, float *__restrict__ gate,
                                                               float *__restrict__ probs,
                                                               int32_t *__restrict__ part_counts,
                                                               double *__restrict__ part_psum) {
    static_assert(S >= 4 && S % 2 == 0 && 8 * (S - 2) < 64, "stages: even, 4..8");
    constexpr int CK = kDecodeCK;
    constexpr int NQ = CK / 4;       // 16-byte pieces of a row segment; also load instructions per chunk
    // dynamic LDS: [NW waves][S stages][64 rows][128 bytes], then the token row [d] fp32 and CK zeros
    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    __shared__ float s_z[NW * 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = blockIdx.x;
    const int nch = d / CK;          // d % 64 == 0: even, at least 2
    float *s_x = (float *)(s_dyn + (size_t)NW * S * kDecodeChunk);
    const uint8_t *const stg0 = s_dyn + (size_t)wave * S * kDecodeChunk;   // this wave's stages
    const uint32_t lds0 = decode_lds_addr(stg0);

    // load instruction i of a chunk: row 8i + (lane >> 3) (rows past N' repeat row N'-1),
    // physical piece lane & 7, which holds logical piece q
    const i32x4_t re = decode_rsrc(E, (uint32_t)((size_t)Nr * d * 4));
    uint32_t voff[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int q = (lane & 7) ^ (r & 7) ^ ((r >> 3) & 1);
        // less the immediate offset of load i within its group of four (row r >= 8 i, so the
        // value stays positive)
        voff[i] = (uint32_t)(((size_t)min(wave * 64 + r, Nr - 1) * d + 4 * q) * 4) - 1024u * (i & 3);
    }
    // loads 4h .. 4h+3 of chunk c (clamped: the loads past the last chunk repeat it, so every
    // step issues the same number of loads and the vmcnt waits stay exact) into stage stg
    auto dma = [&](int c, int stg, int h) {
        decode_dma16x4(re, lds0 + stg * kDecodeChunk + 4096 * h, voff + 4 * h, (uint32_t)min(c, nch - 1) * (CK * 4));
    };
#pragma unroll
    for (int s = 0; s < S - 1; ++s) {
        dma(s, s, 0);
        dma(s, s, 1);
    }

    // the token row, as fp32, into LDS (its loads go out after the chunks' and the first wait
    // for them covers the chunks too; with SB pieces per thread at most 8 (S - 1) + SB <= 60
    // loads are outstanding)
    {
        constexpr int NT = NW * 64, SB = 4;
        const int n16 = d * (XB ? 2 : 4) / 16;     // 16-byte pieces of the row
        const uint4 *xr = (const uint4 *)((const uint8_t *)x + (size_t)t * d * (XB ? 2 : 4));
        auto put = [&](int i, const uint4 v) {
            if constexpr (XB) {
                *(float4 *)(s_x + 8 * i) = make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
                                                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u));
                *(float4 *)(s_x + 8 * i + 4) =
                    make_float4(__uint_as_float(v.z << 16), __uint_as_float(v.z & 0xffff0000u),
                                __uint_as_float(v.w << 16), __uint_as_float(v.w & 0xffff0000u));
            } else {
                *(uint4 *)(s_x + 4 * i) = v;
            }
        };
        uint4 v[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u)
            if (tid + u * NT < n16) v[u] = xr[tid + u * NT];
#pragma unroll
        for (int u = 0; u < SB; ++u)
            if (tid + u * NT < n16) put(tid + u * NT, v[u]);
        for (int i = tid + SB * NT; i < n16; i += NT) put(i, xr[i]);
        if (tid < CK / 4) *(float4 *)(s_x + d + 4 * tid) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    wait_vmcnt<0>();
    __syncthreads();

    // the lane's row: logical piece q at physical piece q ^ sw
    const int sw = (lane & 7) ^ ((lane >> 3) & 1);
    uint32_t eo[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) eo[q] = (uint32_t)(lane * 128 + 16 * (q ^ sw));
    float4 e[2][NQ], xv[2][NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        e[0][q] = *(const float4 *)(stg0 + eo[q]);
        xv[0][q] = *(const float4 *)(s_x + 4 * q);
    }
    float acc = 0.0f;
    // step c (stage j = c % S, register set j & 1): chunk c+1 is in its stage once the loads
    // after it, chunks c+2 .. c+S-2, are the only ones outstanding; its reads go out between the
    // fma groups of chunk c; chunk c+S-1 then refills the stage of chunk c-1, read a step ago.
    auto step = [&](auto jt, int c) {
        constexpr int j = decltype(jt)::value, P = j & 1, N = P ^ 1;
        constexpr int SN = (j + 1) % S, SF = (j + S - 1) % S;
        wait_vmcnt<8 * (S - 3)>();
        const float *xs = s_x + min(c + 1, nch) * CK;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int q = 4 * h; q < 4 * h + 4; ++q) {
                acc = __builtin_fmaf(xv[P][q].x, e[P][q].x, acc);
                acc = __builtin_fmaf(xv[P][q].y, e[P][q].y, acc);
                acc = __builtin_fmaf(xv[P][q].z, e[P][q].z, acc);
                acc = __builtin_fmaf(xv[P][q].w, e[P][q].w, acc);
            }
            __builtin_amdgcn_sched_barrier(0);
            // in descending q: the first fma of the half then waits for all of them at once
#pragma unroll
            for (int q = 4 * h + 3; q >= 4 * h; --q) {
                xv[N][q] = *(const float4 *)(xs + 4 * q);
                __builtin_amdgcn_sched_barrier(0);
                e[N][q] = *(const float4 *)(stg0 + SN * kDecodeChunk + eo[q]);
                __builtin_amdgcn_sched_barrier(0);
            }
            dma(c + S - 1, SF, h);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // whole rounds of S steps, no branch inside: steps past the last chunk add x = 0 (the zero
    // chunk after the token row) times a copy of the last centroid chunk, which leaves acc as it
    // is (for finite centroids; acc is never -0, as the chain starts from +0)
    for (int c0 = 0; c0 < nch; c0 += S)
        for_each_step([&](auto jt) { step(jt, c0 + decltype(jt)::value); }, std::make_integer_sequence<int, S>{});
    wait_vmcnt<0>();   // the loads past the last chunk land before the workgroup's LDS is released
    s_z[wave * 64 + lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    float z[1][NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) z[0][j] = s_z[lane + 64 * j];
    double ps[NW];
    int cnt[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) { ps[j] = 0.0; cnt[j] = 0; }
    finish_tokens<1, NW>(t, 1, Nr, K, skip, lane, z, bias, idx, gate, probs, ps, cnt);
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int rr = lane + 64 * j;
        if (rr < Nr) {
            part_psum[(size_t)t * Nr + rr] = ps[j];
            part_counts[(size_t)t * Nr + rr] = cnt[j];
        }
    }
}

// One workgroup per expert (route_reduce_block, moe_internal.h).
__global__ __launch_bounds__(256) void route_reduce_kernel(
    int nblk, int Nr, const int32_t *__restrict__ part_counts, const double *__restrict__ part_psum,
    int32_t *__restrict__ counts, float *__restrict__ prob_sum) {
    route_reduce_block(blockIdx.x, nblk, Nr, part_counts, part_psum, counts, prob_sum);
}

// ---------------------------------------------------------------------------
// Logits on the matrix cores (batches beyond the decode path, 64 < N' <= 128,
// d a multiple of 64).  v_mfma_f32_32x32x2_f32 adds to each output the product
// of the k pair's first value (the operands of lanes 0-31) and then that of
// its second (lanes 32-63), as two fused multiply-adds with one rounding
// each: measured bit-identical to fmaf chains in ascending k, subnormal
// values included.  A run of these instructions over the k pairs in
// ascending order is therefore the same single fma chain over k = 0..d-1
// from +0 as route_kernel's, at the matrix cores' fp32 rate.
//   * a workgroup takes 32 tokens and every expert; wave e computes the
//     32 x 32 block of experts 32e .. 32e+31 (EBK waves, N' <= 32 EBK);
//   * each 64-deep k chunk of the token rows and the centroid rows is staged
//     in LDS, two stages filled through registers a chunk ahead, every row
//     split into its even and its odd k (lanes 0-31 take the even k of each
//     pair, lanes 32-63 the odd one), so one 16-byte read of a lane feeds
//     four instructions; rows are 272 bytes apart, so the rows of a read
//     phase hit distinct 16-byte bank groups;
//   * the logits then go through LDS into the lane-per-expert layout of the
//     selection (finish_tokens, 8 tokens of a wave at a time), and the
//     statistics are combined as in route_kernel (tokens in order within a
//     wave, then the waves in order).
// ---------------------------------------------------------------------------
namespace rm {
// Range-checked 16-byte loads: an offset at or past the buffer's size reads zeros.  No branch
// guards a load, so the compiler keeps exact wait counts for the loads in flight.
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
constexpr int TB = 32;              // tokens per workgroup
constexpr int KC = 64;              // k per stage
constexpr int PITCH = KC * 4 + 16;  // a row's 32 even k, its 32 odd k, a pad (bytes)
}  // namespace rm

template <int EBK, bool XB>
__global__ __launch_bounds__(EBK * 64) void route_mfma_kernel(int T, int d, int Nr, int K, int skip, const void *x,
                                                              const float *__restrict__ E,
                                                              const float *__restrict__ bias,
                                                              int32_t *__restrict__ idx, float *__restrict__ gate,
                                                              float *__restrict__ probs,
                                                              int32_t *__restrict__ part_counts,
                                                              double *__restrict__ part_psum) {
    using namespace rm;
    constexpr int W = EBK, NT = W * 64, NE = 32 * EBK, NJ = (NE + 63) / 64;
    constexpr int STAGE = (TB + NE) * PITCH;   // token rows, then centroid rows
    constexpr int PR = XB ? KC / 8 : KC / 4;   // 16-byte token pieces per row and chunk
    constexpr int XPT = TB * PR / NT;          // token pieces per thread
    constexpr int EPT = NE * (KC / 4) / NT;    // centroid pieces per thread (4)
    static_assert(TB * PR % NT == 0 && NE * (KC / 4) % NT == 0, "whole pieces per thread");
    constexpr int ZP = NE + 4;                 // pitch (floats) of the logits tile
    static_assert(TB * ZP * 4 <= 2 * STAGE && W * NJ * 64 * 12 <= 2 * STAGE, "tile and statistics fit");
    __shared__ __attribute__((aligned(16))) uint8_t s_m[2 * STAGE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, hi = lane >> 5;
    const int t0 = blockIdx.x * TB;
    const int nchunk = d / KC;

    // staging: token piece p = row p / PR, piece p % PR; centroid piece p = row p / 16, piece p % 16.
    // Piece c of a row covers k = 4c..4c+3 (fp32; 8c..8c+7 for bf16 tokens): its even k go to
    // [8c, 8c+8) of the row's even half (bf16: [16c, 16c+16)), its odd k to the same place + 128.
    constexpr int XE = XB ? 2 : 4;
    const __amdgpu_buffer_rsrc_t rx = rsrc(x, (uint32_t)((size_t)T * d * XE));
    const __amdgpu_buffer_rsrc_t re = rsrc(E, (uint32_t)((size_t)Nr * d * 4));
    uint32_t xo[XPT], eo[EPT];   // byte offsets of the pieces in chunk 0 (kOob: a row past the end)
    int xd[XPT], ed[EPT];
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
        const int pc = tid + i * NT, r = pc / PR, c = pc % PR;
        const int t = t0 + r;
        xo[i] = t < T ? (uint32_t)(((size_t)t * d + (size_t)c * (16 / XE)) * XE) : kOob;
        xd[i] = r * PITCH + c * (XB ? 16 : 8);
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int pc = tid + i * NT, r = pc / 16, c = pc % 16;
        eo[i] = r < Nr ? (uint32_t)(((size_t)r * d + 4 * c) * 4) : kOob;   // rows of absent experts read zeros
        ed[i] = (TB + r) * PITCH + c * 8;
    }
    uint4 xr[XPT], er[EPT];
    auto load = [&](int c) {
#pragma unroll
        for (int i = 0; i < XPT; ++i) xr[i] = ld16(rx, xo[i], (uint32_t)(c * KC * XE));
#pragma unroll
        for (int i = 0; i < EPT; ++i) er[i] = ld16(re, eo[i], (uint32_t)(c * KC * 4));
    };
    // the 4 fp32 values of a piece: even k at p, p + 4, odd k at p + 128, p + 132
    auto put4 = [](uint8_t *p, const uint4 &v) {
        *(uint2 *)p = make_uint2(v.x, v.z);
        *(uint2 *)(p + 128) = make_uint2(v.y, v.w);
    };
    auto store = [&](int st) {
        uint8_t *b = s_m + st * STAGE;
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const uint4 v = xr[i];
            if (XB) {   // 8 bf16 -> fp32 (exact): even k, then odd k
                *(uint4 *)(b + xd[i]) = make_uint4(v.x << 16, v.y << 16, v.z << 16, v.w << 16);
                *(uint4 *)(b + xd[i] + 128) =
                    make_uint4(v.x & 0xffff0000u, v.y & 0xffff0000u, v.z & 0xffff0000u, v.w & 0xffff0000u);
            } else {
                put4(b + xd[i], v);
            }
        }
#pragma unroll
        for (int i = 0; i < EPT; ++i) put4(b + ed[i], er[i]);
    };

    f32x16 acc;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
    // lane (l32, hi): token row l32 and centroid row 32 wave + l32, their hi-parity k
    const int aoff = l32 * PITCH + hi * 128, boff = (TB + 32 * wave + l32) * PITCH + hi * 128;
    // chunk c in stage c & 1; chunk c+1's loads go out before chunk c's MFMAs and are stored
    // into the other stage after them
    load(0);
    store(0);
    __syncthreads();
    for (int c = 0; c < nchunk; ++c) {
        if (c + 1 < nchunk) load(c + 1);
        const uint8_t *b = s_m + (c & 1) * STAGE;
#pragma unroll
        for (int u = 0; u < KC / 8; ++u) {   // k pairs 4u .. 4u+3 of the chunk, in order
            const float4 a4 = *(const float4 *)(b + aoff + 16 * u);
            const float4 b4 = *(const float4 *)(b + boff + 16 * u);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.x, b4.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.y, b4.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.z, b4.z, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a4.w, b4.w, acc, 0, 0, 0);
        }
        if (c + 1 < nchunk) store((c + 1) & 1);
        __syncthreads();
    }

    // the 32 x NE logits through LDS: register e of lane (l32, hi) holds token
    // 8 (e / 4) + 4 hi + e % 4 and expert 32 wave + l32
    float *s_z = (float *)s_m;
#pragma unroll
    for (int e = 0; e < 16; ++e) s_z[((e / 4) * 8 + hi * 4 + (e % 4)) * ZP + 32 * wave + l32] = acc[e];
    __syncthreads();

    constexpr int TPW = TB / W;               // tokens of each wave
    constexpr int RR = TPW < 8 ? TPW : 8;     // tokens per selection round
    double ps[NJ];
    int cnt[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) { ps[j] = 0.0; cnt[j] = 0; }
    for (int q = 0; q < TPW; q += RR) {
        const int tl = wave * TPW + q;
        const int tg = t0 + tl;
        if (tg >= T) break;
        float a[RR][NJ];
#pragma unroll
        for (int i = 0; i < RR; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e = lane + 64 * j;
                a[i][j] = e < NE ? s_z[(tl + i) * ZP + e] : 0.0f;
            }
        finish_tokens<RR, NJ>(tg, min(RR, T - tg), Nr, K, skip, lane, a, bias, idx, gate, probs, ps, cnt);
    }

    // the waves' per-expert sums, combined in wave order, at row blockIdx.x
    __syncthreads();
    double *s_ps = (double *)s_m;
    int *s_cnt = (int *)(s_ps + W * NJ * 64);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        s_ps[wave * NJ * 64 + lane + 64 * j] = ps[j];
        s_cnt[wave * NJ * 64 + lane + 64 * j] = cnt[j];
    }
    __syncthreads();
    for (int r = tid; r < Nr; r += NT) {
        double a = 0.0;
        int cc = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) { a += s_ps[w * NJ * 64 + r]; cc += s_cnt[w * NJ * 64 + r]; }
        part_psum[(size_t)blockIdx.x * Nr + r] = a;
        part_counts[(size_t)blockIdx.x * Nr + r] = cc;
    }
}

// Waves per workgroup and tokens per wave, from a sweep of (2, 4, 8) x
// (1, 2, 4) on MI355X: 8 waves from 2048 tokens (one centroid chunk read
// serves 8 waves), 4 below (more CUs stream the centroids for small
// batches); 2 tokens per wave from 4096 tokens and 4 from 8192 (each
// centroid value read from LDS feeds more chains, while the chip keeps about
// two waves per SIMD).
int route_waves(int T) { return T >= 2048 ? 8 : 4; }
int route_tokens_per_wave(int T) { return T >= 8192 ? 4 : T >= 4096 ? 2 : 1; }
// Batches of at most this many tokens take the decode kernel (one workgroup per token).
constexpr int kRouteDecodeTokens = 256;
// ... and whose LDS stages fit (decode_stages); N' up to 256.
bool route_decode_path(int T, int d, int Nr) {
    return T <= kRouteDecodeTokens && d <= kRouteDecodeMaxD && decode_stages(cdiv(Nr, 64), d) > 0;
}
// Batched tokens that take route_mfma_kernel: 65 to 128 experts (four 32-expert waves) and whole
// 64-deep k chunks.  Measured against route_kernel (bf16 tokens, one box): T = 8192, d = 4096,
// N' = 128: 231-255 -> 150 us.  With N' <= 64 (two waves per workgroup, less than a microsecond
// of MFMAs per chunk) the chunk loads' latency dominates and route_kernel stays faster (T = 16384,
// d = 1280, N' = 63: 61 -> 92 us; T = 4096, N' = 64: 25 -> 57 us).
bool route_mfma_path(int T, int d, int Nr) {
    return !route_decode_path(T, d, Nr) && Nr > 64 && Nr <= 128 && d % rm::KC == 0;
}

template <bool XB>
void launch_route_mfma(const moe_problem &p, int skip, int nblk, const void *x, const float *E, const float *bias,
                       int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
#define MOE_L(EBK) route_mfma_kernel<EBK, XB><<<nblk, EBK * 64, 0, s>>>( \
        p.T, p.d, p.n_routed, p.top_k, skip, x, E, bias, idx, gate, probs, pc, pp)
    MOE_L(4);   // 65..128 experts: four waves (65..96 with a zero block: the staging splits evenly)
#undef MOE_L
}

template <int NW, int S, bool XB>
hipError_t launch_decode_form(const moe_problem &p, int skip, const void *x, const float *E, const float *bias,
                              int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    const size_t lds = decode_lds_bytes(NW, S, p.d);
    // dynamic LDS beyond 64 KB: raise the kernel's limit, once per form and device (the largest d
    // so far wins)
    constexpr int kDevices = 64;
    static size_t granted[kDevices] = {};
    static std::mutex mu;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kDevices) return hipErrorInvalidDevice;
    {
        std::lock_guard<std::mutex> lock(mu);
        if (lds > granted[dev]) {
            e = hipFuncSetAttribute((const void *)route_decode_kernel<NW, S, XB>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            if (e != hipSuccess) return e;
            granted[dev] = lds;
        }
    }
    route_decode_kernel<NW, S, XB><<<p.T, NW * 64, lds, s>>>(p.T, p.d, p.n_routed, p.top_k, skip, x, E, bias, idx,
                                                             gate, probs, pc, pp);
    return hipGetLastError();
}

template <bool XB>
hipError_t launch_route_decode(const moe_problem &p, int skip, const void *x, const float *E, const float *bias,
                               int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    const int nw = cdiv(p.n_routed, 64);
#define MOE_L(NW, S) return launch_decode_form<NW, S, XB>(p, skip, x, E, bias, idx, gate, probs, pc, pp, s)
    switch (nw * 16 + decode_stages(nw, p.d)) {
        case 1 * 16 + 8: MOE_L(1, 8);
        case 2 * 16 + 8: MOE_L(2, 8);
        case 2 * 16 + 6: MOE_L(2, 6);
        case 2 * 16 + 4: MOE_L(2, 4);
        case 3 * 16 + 6: MOE_L(3, 6);
        case 3 * 16 + 4: MOE_L(3, 4);
        case 4 * 16 + 4: MOE_L(4, 4);
        default: return hipErrorInvalidValue;   // route_decode_path excludes every other form
    }
#undef MOE_L
}

template <int RT, int W, bool XB>
void launch_rtw(const moe_problem &p, int skip, int nblk, const void *x, const float *E, const float *bias,
                int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    const int nj = cdiv(p.n_routed, 64);
#define MOE_L(NJ) route_kernel<RT, NJ, W, XB><<<nblk, W * 64, 0, s>>>( \
        p.T, p.d, p.n_routed, p.top_k, skip, x, E, bias, idx, gate, probs, pc, pp)
    if (nj == 1) MOE_L(1);
    else if (nj == 2) MOE_L(2);
    else MOE_L(4);
#undef MOE_L
}

template <int RT, bool XB>
void launch_rt(const moe_problem &p, int skip, int nblk, const void *x, const float *E, const float *bias,
               int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    switch (route_waves(p.T)) {
        case 8: launch_rtw<RT, 8, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        case 4: launch_rtw<RT, 4, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        default: launch_rtw<RT, 2, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
    }
}

template <bool XB>
void launch_route_typed(const moe_problem &p, int skip, int nblk, const void *x, const float *E, const float *bias,
                        int32_t *idx, float *gate, float *probs, int32_t *pc, double *pp, hipStream_t s) {
    switch (route_tokens_per_wave(p.T)) {
        case 4: launch_rt<4, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        case 2: launch_rt<2, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
        default: launch_rt<1, XB>(p, skip, nblk, x, E, bias, idx, gate, probs, pc, pp, s); break;
    }
}

}  // namespace

int route_blocks(int T, int d, int Nr) {
    if (route_decode_path(T, d, Nr)) return T;
    if (route_mfma_path(T, d, Nr)) return cdiv(T, rm::TB);
    return cdiv(T, route_waves(T) * route_tokens_per_wave(T));
}

// ---------------------------------------------------------------------------
// Allocation-free routing (moe_route_noalloc): the per-workgroup partial
// statistics live in a file-scope device array instead of the caller's
// workspace.  Each device holds its own copy of the array until the process
// ends; its device address is taken once per device with hipGetSymbolAddress
// (the host-side name is only a stand-in and is never passed to a kernel).
// Every call on a device shares that device's array: each routing workgroup
// overwrites its own partials before the reduction reads them, so nothing
// needs clearing, but calls that overlap in time on one device race.
// ---------------------------------------------------------------------------
namespace {
constexpr int kScratchDevices = 64;
__device__ __align__(256) uint8_t scratch[kRouteScratchBytes];
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices] = {};
}  // namespace

hipError_t route_scratch_ptr(void **ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *q = nullptr;
        e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = q;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool route_decode_batch(const moe_problem &p) { return p.T > 0 && route_decode_path(p.T, p.d, p.n_routed); }

hipError_t launch_route(const moe_problem &p, int skip, const void *x, const float *centroids, const float *bias,
                        int32_t *idx, float *gate, float *probs, int32_t *part_counts, double *part_psum,
                        int32_t *counts, float *prob_sum, hipStream_t s, bool reduce) {
    const int nblk = p.T > 0 ? route_blocks(p.T, p.d, p.n_routed) : 0;
    if (nblk > 0) {
        if (route_mfma_path(p.T, p.d, p.n_routed)) {
            if (p.dtype == MOE_BF16)
                launch_route_mfma<true>(p, skip, nblk, x, centroids, bias, idx, gate, probs, part_counts, part_psum, s);
            else
                launch_route_mfma<false>(p, skip, nblk, x, centroids, bias, idx, gate, probs, part_counts, part_psum,
                                         s);
        } else if (route_decode_path(p.T, p.d, p.n_routed)) {
            const hipError_t e =
                p.dtype == MOE_BF16
                    ? launch_route_decode<true>(p, skip, x, centroids, bias, idx, gate, probs, part_counts, part_psum, s)
                    : launch_route_decode<false>(p, skip, x, centroids, bias, idx, gate, probs, part_counts, part_psum,
                                                 s);
            if (e != hipSuccess) return e;
        } else if (p.dtype == MOE_BF16) {
            launch_route_typed<true>(p, skip, nblk, x, centroids, bias, idx, gate, probs, part_counts, part_psum, s);
        } else {
            launch_route_typed<false>(p, skip, nblk, x, centroids, bias, idx, gate, probs, part_counts, part_psum,
                                      s);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!reduce) return hipSuccess;
    route_reduce_kernel<<<p.n_routed, 256, 0, s>>>(nblk, p.n_routed, part_counts, part_psum, counts, prob_sum);
    return hipGetLastError();
}

// Hash routing (the Hash Layer baseline): expert = floor(h * N' / 2^32) with
// h = id * 2654435761 mod 2^32 (Knuth's multiplicative hash), gate 1; then
// one workgroup per expert counts its tokens (integer, fixed order).
namespace {
__global__ __launch_bounds__(256) void route_hash_kernel(int T, int Nr, const int32_t *__restrict__ ids,
                                                         int32_t *__restrict__ idx, float *__restrict__ gate) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const uint32_t h = (uint32_t)ids[t] * 2654435761u;
    idx[t] = (int32_t)(((uint64_t)h * (uint64_t)Nr) >> 32);
    gate[t] = 1.0f;
}
__global__ __launch_bounds__(256) void route_hash_counts_kernel(int T, const int32_t *__restrict__ idx,
                                                                int32_t *__restrict__ counts) {
    __shared__ int s_c[4];
    const int r = blockIdx.x;
    int c = 0;
    for (int t = threadIdx.x; t < T; t += 256) c += idx[t] == r ? 1 : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    if ((threadIdx.x & 63) == 0) s_c[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) counts[r] = s_c[0] + s_c[1] + s_c[2] + s_c[3];
}
}  // namespace

hipError_t launch_route_hash(const moe_problem &p, const int32_t *token_ids, int32_t *idx, float *gate,
                             int32_t *counts, hipStream_t s) {
    if (p.T > 0) route_hash_kernel<<<cdiv(p.T, 256), 256, 0, s>>>(p.T, p.n_routed, token_ids, idx, gate);
    route_hash_counts_kernel<<<p.n_routed, 256, 0, s>>>(p.T, idx, counts);
    return hipGetLastError();
}

}  // namespace moe
