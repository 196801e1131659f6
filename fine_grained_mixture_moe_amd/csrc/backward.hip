// backward.hip -- backward pass of the DeepSeekMoE layer on gfx950.
//
// Training is the setting of "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致
// 专家特化", section "Method details: formulas and load balance": the loss
// adds alpha_1 * ExpBal + alpha_2 * DevBal to the task loss.  Given the
// upstream gradient dh = dL/dh of the layer output, the chain rule through the
// output sum, the SwiGLU experts and the softmax router gives (per used
// token-expert pair, dy = gate * dh for a routed pair and dh for a shared
// expert):
//   da = W2^T dy;  dp = da q s (1 + p (1 - s)), dq = da SiLU(p), s = sigmoid(p)
//   dx += W1^T dp + W3^T dq;  dW2 += dy a^T;  dW1 += dp x^T;  dW3 += dq x^T
//   dgate = dh . y;  ds_r = dgate (r selected) + (alpha_1 f_r + alpha_2 f'_g(r)) / T
//   dz = s (ds - <s, ds>);  dx += sum_r dz_r e_r;  dE = dz^T x;  dbias = sum_t dz
// with the Top-K selection held fixed and f, f' (counts) constant.
//
// Kernels:
//   combine_bwd_kernel   dy rows (gate * dh) and dgate (dot products), one wave per token
//   grouped GEMMs on MFMA, five products (MODE):
//      0  da   = dy . W2              (A rows k-contiguous, B = W2 read transposed)
//      1  dxr  = dp . W1 + dq . W3    (A k-contiguous, B transposed; rows in the
//                                      layer dtype, as the forward's y_routed)
//      2  dW2  = dy^T . a             (A and B transposed; k runs over the group's rows)
//      3  dW13 = [dp|dq]^T . x        (A and B transposed; x rows gathered)
//      4  p, q = x . [W1;W3]^T, then the SwiGLU backward in the epilogue:
//         reads da, writes dp, dq and a (A and B k-contiguous); fp32 layers
//         only: bf16 layers recompute p, q on the forward up kernel with its
//         backward epilogue (expert_ffn.hip)
//   bgemm_wide_kernel    bf16 modes 0-3 on 256 x 256 tiles (8 waves, two LDS
//                        stages, raw buffer loads whose offsets are fixed per
//                        tile, an LDS-staged epilogue)
//   bgemm_kernel<MODE>   fp32 layers: all five modes on 128 x 128 tiles
//   (both with an XCD-aware tile order, see bgemm_kernel)
//   gather_dx_kernel     dx_ffn[t] = dxs[t] + sum_k dxr[slot_of[t,k]] (k order)
//   router_dz_kernel     ds, dz per token (wave per token, lane = expert)
//   router_dx_kernel     dx = dh + dx_ffn + dz E (LDS-tiled, 128 or 64 tokens x 128 columns, 8 or 4 x 8
//                        per thread)
//   router_de_part/sum   dE, dbias partials over token chunks (8 columns x 4 or 8 experts per thread),
//                        then a fixed-order sum
//
// Operands are staged through LDS; a "transposed" operand (stored with its
// m index contiguous) is read into MFMA fragments with ds_read_b64_tr_b16:
// within each 16-lane group, element e of lane 4a+b is element b of the
// 8-byte piece addressed by lane a+4e, so two such reads give a lane the 8
// consecutive k of its row.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef short v4s __attribute__((ext_vector_type(4)));
typedef short v8s __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Raw buffer loads for the bf16 GEMM staging.  The range is the whole 2 GB
// window: a chunk outside its tile's M/N bounds or past K carries the offset
// kOob, which the hardware answers with zeros (no branch, no null pointer).
constexpr uint32_t kOob = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bg_rsrc(const void *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ uint4 bg_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

template <typename DT> __device__ __forceinline__ float to_f(DT v);
template <> __device__ __forceinline__ float to_f<uint16_t>(uint16_t v) { return bf2f(v); }
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <typename DT> __device__ __forceinline__ DT from_f(float v);
template <> __device__ __forceinline__ uint16_t from_f<uint16_t>(float v) { return f2bf(v); }
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }

// ---------------------------------------------------------------------------
// combine backward: one wave per token.  Lane l covers columns 8l + 512 i
// with 16-byte accesses; dh_t is read once for all K' slots.
// dy_routed[slot_of[t,k]] = gate[t,k] * dh_t (rounded to dtype);
// dgate[t,k] = sum_i dh_t[i] * y_routed[slot][i] in fp32, lane partials summed
// by a fixed butterfly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8(const uint16_t *p, float v[8]) {
    const uint4 q = *(const uint4 *)p;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float *p, float v[8]) {
    const float4 a = *(const float4 *)p, b = *(const float4 *)(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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
__global__ __launch_bounds__(256) void combine_bwd_kernel(int T, int d, int K, const DT *__restrict__ dh,
                                                          const DT *__restrict__ y, const float *__restrict__ gate,
                                                          const int32_t *__restrict__ slot_of, DT *__restrict__ dy,
                                                          float *__restrict__ dgate) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    float part[kRouteMaxTopK];
#pragma unroll
    for (int k = 0; k < kRouteMaxTopK; ++k) part[k] = 0.0f;
    for (int c = lane * 8; c < d; c += 512) {
        float hv[8];
        load8(dh + (size_t)t * d + c, hv);
        // K' in batches of 4: the batch's slots, then its 4 independent row loads
#pragma unroll
        for (int k0 = 0; k0 < kRouteMaxTopK; k0 += 4) {
            if (k0 >= K) break;
            int slot[4];
            float g[4], yv[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool in = k0 + u < K;
                slot[u] = in ? slot_of[(size_t)t * K + k0 + u] : -1;
                g[u] = in ? gate[(size_t)t * K + k0 + u] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (slot[u] >= 0) load8(y + (size_t)slot[u] * d + c, yv[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (slot[u] < 0) continue;
                float o[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    part[k0 + u] = __builtin_fmaf(hv[e], yv[u][e], part[k0 + u]);
                    o[e] = g[u] * hv[e];
                }
                store8(dy + (size_t)slot[u] * d + c, o);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kRouteMaxTopK; ++k) {
        if (k >= K) break;
        float v = part[k];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == 0) dgate[(size_t)t * K + k] = v;
    }
}

// ---------------------------------------------------------------------------
// Grouped backward GEMMs.
// ---------------------------------------------------------------------------
struct BgArgs {
    int T, d, Ks, Nr, w;
    const int32_t *offsets, *sorted_token;
    const void *x, *dh, *dy_r;
    const void *w1_r, *w3_r, *w2_r, *w1_s, *w3_s, *w2_s;
    void *da_r, *da_s;                   // [T*K', w], [T, K_s*w] dtype
    void *dp_r, *dq_r, *a_r;             // [T*K', w] dtype
    void *dp_s, *dq_s, *a_s;             // [T, K_s*w] dtype
    void *dxr;                           // [T*K', d] dtype: dx of every grouped row
    float *dxs;                          // [T, d]: dx of the shared experts
    float *dw1_r, *dw3_r, *dw2_r;        // [N', w, d], [N', w, d], [N', d, w]
    float *dw1_s, *dw3_s, *dw2_s;        // [K_s, ...]
};

constexpr int BG_MAXG = 1 + kPermuteMaxExperts;

struct Group {
    bool sh;
    int r, rows, roff, wg;
};

__device__ __forceinline__ Group group_of(const BgArgs &A, int g) {
    Group G;
    G.sh = A.Ks > 0 && g == 0;
    G.r = g - (A.Ks > 0 ? 1 : 0);
    G.rows = G.sh ? A.T : A.offsets[G.r + 1] - A.offsets[G.r];
    G.roff = G.sh ? 0 : A.offsets[G.r];
    G.wg = G.sh ? A.Ks * A.w : A.w;
    return G;
}

// M, N, K of a group's product; N counts B rows (mode 4: W1 and W3 rows).
template <int MODE>
__device__ __forceinline__ void dims(const BgArgs &A, const Group &G, int &M, int &N, int &K) {
    if (MODE == 0) { M = G.rows; N = G.wg; K = A.d; }
    if (MODE == 1) { M = G.rows; N = A.d; K = 2 * G.wg; }
    if (MODE == 2) { M = A.d; N = G.wg; K = G.rows; }
    if (MODE == 3) { M = 2 * G.wg; N = A.d; K = G.rows; }
    if (MODE == 4) { M = G.rows; N = 2 * G.wg; K = A.d; }
}
constexpr bool a_transposed(int mode) { return mode == 2 || mode == 3; }
constexpr bool b_transposed(int mode) { return mode != 4; }

// Element pointer of operand A at (m, k) (a chunk of 8 bf16 / 4 fp32 along the
// contiguous index starts there); nullptr when outside the group.
template <int MODE, typename DT>
__device__ __forceinline__ const DT *a_ptr(const BgArgs &A, const Group &G, int m, int k, int M, int K) {
    if (m >= M || k >= K) return nullptr;
    const size_t w = A.w, d = A.d, wg = G.wg;
    if (MODE == 0) {
        const DT *dy = G.sh ? (const DT *)A.dh : (const DT *)A.dy_r;
        return dy + (size_t)(G.roff + m) * d + k;
    }
    if (MODE == 1) {
        const bool p = k < G.wg;
        const int kk = p ? k : k - G.wg;
        const DT *b = G.sh ? (const DT *)(p ? A.dp_s : A.dq_s) : (const DT *)(p ? A.dp_r : A.dq_r);
        return b + (size_t)(G.roff + m) * wg + kk;
    }
    if (MODE == 2) {   // A(m, k) = dy[row k][m]
        const DT *dy = G.sh ? (const DT *)A.dh : (const DT *)A.dy_r;
        return dy + (size_t)(G.roff + k) * d + m;
    }
    if (MODE == 3) {   // A(m, k) = [dp | dq][row k][m]
        const bool p = m < G.wg;
        const int mm = p ? m : m - G.wg;
        const DT *b = G.sh ? (const DT *)(p ? A.dp_s : A.dq_s) : (const DT *)(p ? A.dp_r : A.dq_r);
        return b + (size_t)(G.roff + k) * wg + mm;
    }
    // MODE 4: x rows gathered through sorted_token
    const int tok = G.sh ? m : A.sorted_token[G.roff + m];
    (void)w;
    return (const DT *)A.x + (size_t)tok * d + k;
}

// Operand B at (n, k): mode 4 row n of [W1; W3] interleaved per 32 units
// (k contiguous); otherwise B(k, n) with n contiguous.
template <int MODE, typename DT>
__device__ __forceinline__ const DT *b_ptr(const BgArgs &A, const Group &G, int n, int k, int N, int K) {
    if (n >= N || k >= K) return nullptr;
    const size_t w = A.w, d = A.d;
    if (MODE == 0) {   // W2 [seg][d][w]: B(k = hidden i, n = unit)
        const int seg = n / A.w, nn = n % A.w;
        const DT *w2 = G.sh ? (const DT *)A.w2_s + (size_t)seg * d * w : (const DT *)A.w2_r + (size_t)G.r * d * w;
        return w2 + (size_t)k * w + nn;
    }
    if (MODE == 1) {   // [W1; W3] rows: B(k = unit row, n = hidden)
        const bool p = k < G.wg;
        const int kk = p ? k : k - G.wg;
        const int seg = kk / A.w, kr = kk % A.w;
        const DT *wb = G.sh ? (const DT *)(p ? A.w1_s : A.w3_s) + (size_t)seg * w * d
                            : (const DT *)(p ? A.w1_r : A.w3_r) + (size_t)G.r * w * d;
        return wb + (size_t)kr * d + n;
    }
    if (MODE == 2) {   // a[row k][n]
        const DT *a = G.sh ? (const DT *)A.a_s : (const DT *)A.a_r;
        return a + (size_t)(G.roff + k) * G.wg + n;
    }
    if (MODE == 3) {   // x[tok(row k)][n]
        const int tok = G.sh ? k : A.sorted_token[G.roff + k];
        return (const DT *)A.x + (size_t)tok * d + n;
    }
    // MODE 4: tile row n -> unit (n / 64) * 32 + n % 32 of W1 (bit 5 of n clear) or W3
    const int unit = (n >> 6) * 32 + (n & 31);
    const bool p = ((n >> 5) & 1) == 0;
    const int seg = unit / A.w, ur = unit % A.w;
    const DT *wb = G.sh ? (const DT *)(p ? A.w1_s : A.w3_s) + (size_t)seg * w * d
                        : (const DT *)(p ? A.w1_r : A.w3_r) + (size_t)G.r * w * d;
    return wb + (size_t)ur * d + k;
}

__device__ __forceinline__ uint4 ld16(const void *p) {
    return p ? *(const uint4 *)p : make_uint4(0u, 0u, 0u, 0u);
}

// fp32 layers.  128 x 128 tile (mode 4: 128 rows x 64 units, both halves of
// B), 32 k per step, 4 waves in 2 x 2, each 64 x 64 = 2 x 2 MFMA blocks of
// 32 x 32 (v_mfma_f32_32x32x2f32).
template <int MODE>
__global__ __launch_bounds__(256, 4) void bgemm_kernel(BgArgs A) {
    using DT = float;
    constexpr int ES = sizeof(DT);
    constexpr int EC = 16 / ES;                       // elements per 16-byte chunk
    constexpr bool AT = a_transposed(MODE), BT = b_transposed(MODE);
    // LDS pitches (bytes): k-contiguous tiles [128][32], transposed tiles [32][128]
    constexpr int PK = 32 * ES + 16;                  // 144: conflict-free fragment rows
    constexpr int PT = 128 * ES + 128;                // 640
    constexpr int SA = AT ? 32 * PT : 128 * PK;
    constexpr int SB = BT ? 32 * PT : 128 * PK;
    constexpr int CA = AT ? 32 * (128 / EC) : 128 * (32 / EC);   // chunks per A tile
    constexpr int CB = BT ? 32 * (128 / EC) : 128 * (32 / EC);
    constexpr int RA = CA / 256, RB = CB / 256;                   // chunks per thread
    __shared__ __attribute__((aligned(16))) uint8_t s_a2[1][SA];
    __shared__ __attribute__((aligned(16))) uint8_t s_b2[1][SB];
    __shared__ int s_pref[BG_MAXG + 1];
    __shared__ int s_maxg;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int G = (A.Ks > 0 ? 1 : 0) + A.Nr;
    if (wave == 0) {
        int carry = 0, mx = 0;
        if (lane == 0) s_pref[0] = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            int tiles = 0;
            if (g < G) {
                const Group Gr = group_of(A, g);
                int M, N, K;
                dims<MODE>(A, Gr, M, N, K);
                tiles = cdiv(M, 128) * cdiv(N, 128);
            }
            mx = max(mx, tiles);
            int incl = tiles;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            if (g < G) s_pref[g + 1] = carry + incl;
            carry += __shfl(incl, 63, 64);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
        if (lane == 0) s_maxg = mx;
    }
    __syncthreads();
    const int bid = blockIdx.x;
    const int NT = s_pref[G];
    if (bid >= NT) return;
    // XCD-aware order.  Workgroup b runs on XCD b % 8; spread(j, n) gives the
    // j-th of n workgroups the position j % 8 * per + j / 8 (ragged classes
    // shortened), so each XCD works through a contiguous eighth of the range
    // and tiles that share an operand share its L2.  The range is the whole
    // tile list (whole groups on one XCD: each operand read into one L2) when
    // every tile costs the same and no group holds more than an eighth of the
    // tiles: da (k = d), and the dx rows with at most one shared expert
    // (k = 2 K_s w vs 2 w).  Otherwise each group is spread over all XCDs, so
    // every XCD gets the same share of it whatever it costs (hot experts
    // under skewed routing, several shared experts, the weight gradients'
    // k = the group's rows).
    auto spread = [](int j, int n) {
        const int per = (n + 7) / 8, tall = n % 8 == 0 ? 8 : n % 8, x = j % 8, l = j / 8;
        return x < tall ? x * per + l : tall * per + (x - tall) * (per - 1) + l;
    };
    auto group_at = [&](int v) {
        int lo = 0, hi = G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pref[mid] <= v) lo = mid; else hi = mid;
        }
        return lo;
    };
    const bool whole = (MODE == 0 || (MODE == 1 && A.Ks <= 1)) && s_maxg * 8 <= NT;
    int lo, lt;
    if (whole) {
        const int v = spread(bid, NT);
        lo = group_at(v);
        lt = v - s_pref[lo];
    } else {
        lo = group_at(bid);
        lt = spread(bid - s_pref[lo], s_pref[lo + 1] - s_pref[lo]);
    }
    const Group Gr = group_of(A, lo);
    int M, N, K;
    dims<MODE>(A, Gr, M, N, K);
    const int mt = cdiv(M, 128);
    const int m0 = (lt % mt) * 128, n0 = (lt / mt) * 128;

    // ---- staging: chunk c of a tile -> (row, column) in the tile ----
    uint4 ra[RA], rb[RB];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int c = tid + 256 * i;
            const void *p;
            if (AT) { const int kr = c / (128 / EC), mc = c % (128 / EC); p = a_ptr<MODE, DT>(A, Gr, m0 + mc * EC, k0 + kr, M, K); }
            else { const int mr = c / (32 / EC), kc = c % (32 / EC); p = a_ptr<MODE, DT>(A, Gr, m0 + mr, k0 + kc * EC, M, K); }
            ra[i] = ld16(p);
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int c = tid + 256 * i;
            const void *p;
            if (BT) { const int kr = c / (128 / EC), nc = c % (128 / EC); p = b_ptr<MODE, DT>(A, Gr, n0 + nc * EC, k0 + kr, N, K); }
            else { const int nr = c / (32 / EC), kc = c % (32 / EC); p = b_ptr<MODE, DT>(A, Gr, n0 + nr, k0 + kc * EC, N, K); }
            rb[i] = ld16(p);
        }
    };
    auto store_tiles = [&](int stg) {
        uint8_t *s_a = s_a2[stg], *s_b = s_b2[stg];
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int c = tid + 256 * i;
            uint8_t *q = AT ? s_a + (c / (128 / EC)) * PT + (c % (128 / EC)) * 16
                            : s_a + (c / (32 / EC)) * PK + (c % (32 / EC)) * 16;
            *(uint4 *)q = ra[i];
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int c = tid + 256 * i;
            uint8_t *q = BT ? s_b + (c / (128 / EC)) * PT + (c % (128 / EC)) * 16
                            : s_b + (c / (32 / EC)) * PK + (c % (32 / EC)) * 16;
            *(uint4 *)q = rb[i];
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    const int l32 = lane & 31, lhi = lane >> 5;
    // fragment of a 32-row block at tile row r0 for k sub-step ks (2 k)
    auto frag_f32 = [&](const uint8_t *s, bool tr, int r0, int ks) -> float {
        const int k = 2 * ks + lhi;
        return tr ? *(const float *)(s + k * PT + (r0 + l32) * 4) : *(const float *)(s + (r0 + l32) * PK + k * 4);
    };
    auto compute = [&](int stg) {
        const uint8_t *s_a = s_a2[stg], *s_b = s_b2[stg];
        {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                float fa[2], fb[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    fa[b] = frag_f32(s_a, AT, wm * 64 + b * 32, ks);
                    fb[b] = frag_f32(s_b, BT, wn * 64 + b * 32, ks);
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
            }
        }
    };

    // One LDS stage; the registers prefetch the next step during the
    // compute of the current one.  (Two stages with one barrier per step
    // measured slower: the extra registers cost a wave per SIMD.)
    const int nk = cdiv(K, 32);
    if (nk > 0) {
        load_tiles(0);
        store_tiles(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            if (kt + 1 < nk) load_tiles((kt + 1) * 32);
            compute(0);
            __syncthreads();
            if (kt + 1 < nk) {
                store_tiles(0);
                __syncthreads();
            }
        }
    }

    // ---- epilogue: lane holds column n = l32 of each block and rows
    //      8q + 4*lhi + e (register 4q+e) ----
    if constexpr (MODE == 4) {
        // acc[mb][0] = p (W1 rows), acc[mb][1] = q (W3 rows) of unit
        // n0/2 + wn*32 + l32 for rows m0 + wm*64 + mb*32 + 8q + 4lhi + e
        const int unit = n0 / 2 + wn * 32 + l32;
        if (unit >= Gr.wg) return;
        DT *dpo = (DT *)(Gr.sh ? A.dp_s : A.dp_r), *dqo = (DT *)(Gr.sh ? A.dq_s : A.dq_r);
        DT *ao = (DT *)(Gr.sh ? A.a_s : A.a_r);
        const DT *dai = (const DT *)(Gr.sh ? A.da_s : A.da_r);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 64 + mb * 32 + 8 * (e >> 2) + 4 * lhi + (e & 3);
                if (m >= M) continue;
                const size_t o = (size_t)(Gr.roff + m) * Gr.wg + unit;
                const float p = acc[mb][0][e], q = acc[mb][1][e];
                const float sg = 1.0f / (1.0f + __expf(-p));
                const float da = to_f(dai[o]);
                ao[o] = from_f<DT>(p * sg * q);
                dqo[o] = from_f<DT>(da * p * sg);
                dpo[o] = from_f<DT>(da * q * sg * (1.0f + p * (1.0f - sg)));
            }
    } else {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int n = n0 + wn * 64 + nb * 32 + l32;
                if (n >= N) continue;
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int m = m0 + wm * 64 + mb * 32 + 8 * (e >> 2) + 4 * lhi + (e & 3);
                    if (m >= M) continue;
                    const float v = acc[mb][nb][e];
                    if (MODE == 0) {
                        DT *o = (DT *)(Gr.sh ? A.da_s : A.da_r);
                        o[(size_t)(Gr.roff + m) * Gr.wg + n] = from_f<DT>(v);
                    } else if (MODE == 1) {
                        float *o = Gr.sh ? A.dxs : (float *)A.dxr;
                        o[(size_t)(Gr.roff + m) * A.d + n] = v;
                    } else if (MODE == 2) {
                        const int seg = n / A.w, nn = n % A.w;
                        float *o = Gr.sh ? A.dw2_s + (size_t)seg * A.d * A.w : A.dw2_r + (size_t)Gr.r * A.d * A.w;
                        o[(size_t)m * A.w + nn] = v;
                    } else {
                        const bool p = m < Gr.wg;
                        const int mm = p ? m : m - Gr.wg;
                        const int seg = mm / A.w, mr = mm % A.w;
                        float *o = Gr.sh ? (p ? A.dw1_s : A.dw3_s) + (size_t)seg * A.w * A.d
                                         : (p ? A.dw1_r : A.dw3_r) + (size_t)Gr.r * A.w * A.d;
                        o[(size_t)mr * A.d + n] = v;
                    }
                }
            }
    }
}

// ---------------------------------------------------------------------------
// bf16 grouped GEMMs of modes 0-3 on 256 x 256 tiles.
//
// 512 threads (8 waves, 2 per SIMD) in 2 x 4: a wave owns 4 blocks of 32 A
// rows (tile rows (2b + wm) * 32, so the live blocks of a short tile split
// evenly between the two wave rows) times 2 blocks of 32 B rows, 8 MFMAs of
// 32 x 32 x 16 per 6 fragment reads (the 128 x 128 kernel above: 4 per 4).
// 64 k per step in two LDS stages; the registers hold the step after next,
// written into the idle stage a quarter at a time between the MFMAs of the
// current step, so one barrier per step.
// Stage layouts: a k-contiguous operand is 256 rows of 128 B, 16-byte chunk c
// of row r at c ^ (r & 7) ^ ((r >> 3) & 1) (a ds_read_b128 of 32 rows hits
// distinct banks); a transposed operand is 64 k rows of 256 values with a
// 576-byte pitch, read through ds_read_b64_tr_b16 (the four k rows that one
// 32-lane half reads lie 64 B apart modulo the 256-byte bank cycle).
// Modes 1-3 share one launch (no product among them needs another's output):
// the dx rows first (k = 2 w, the longest), then dW1/dW3, then dW2.
// ---------------------------------------------------------------------------
namespace wide {
constexpr int NT = 512;
constexpr int KC = 128;          // k-contiguous stage: bytes per row (64 k)
constexpr int KT = 576;          // transposed stage: pitch of a k row (256 values + 64 B)
constexpr int SKC = 256 * KC;    // 32 KB
constexpr int STR = 64 * KT;     // 36 KB
constexpr int SMEM = 4 * STR;    // two stages of two transposed operands (the largest)
}  // namespace wide

// The modes of one launch and their block counts in units of 8 (a mode's
// block j runs on XCD j % 8), in block order.  (Interleaving the modes 8
// blocks at a time measured slower: fewer co-running tiles of one expert
// share an XCD's L2.)
struct WideRange {
    int mode[3];
    int oct[3];
};

// Tile (m0, nr rows; n0) of group Gr for product MODE, K its depth.
template <int MODE>
__device__ __forceinline__ void wide_tile(const BgArgs &A, const Group &Gr, int m0, int nr, int n0, int M, int N,
                                          int K, uint8_t *smem) {
    using namespace wide;
    constexpr bool AT = a_transposed(MODE), BT = b_transposed(MODE);
    constexpr int SA = AT ? STR : SKC, SB = BT ? STR : SKC;
    static_assert(2 * (SA + SB) <= SMEM, "stages fit");
    auto stA = [&](int s) { return smem + s * (SA + SB); };
    auto stB = [&](int s) { return smem + s * (SA + SB) + SA; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    // staging geometry: k-contiguous chunk i = row rsub + 64 i, 16-byte part `part`;
    // transposed chunk i = k row kr + 16 i, values 8 mc .. 8 mc + 7
    const int part = tid & 7, rsub = tid >> 3;
    const int swz = part ^ (rsub & 7) ^ ((rsub >> 3) & 1);
    const int mc = tid & 31, kr = tid >> 5;
    auto lds_off = [&](bool tr, int i) { return tr ? (kr + 16 * i) * KT + mc * 16 : (rsub + 64 * i) * KC + swz * 16; };

    const size_t d = A.d, w = A.w, wg = Gr.wg, ro = Gr.roff;
    const uint16_t *dy = (const uint16_t *)(Gr.sh ? A.dh : A.dy_r);
    const uint16_t *dp = (const uint16_t *)(Gr.sh ? A.dp_s : A.dp_r);
    const uint16_t *dq = (const uint16_t *)(Gr.sh ? A.dq_s : A.dq_r);
    const uint32_t dq_off = (uint32_t)((const char *)dq - (const char *)dp);   // dq follows dp in the workspace

    // fixed byte offsets of each thread's chunks (kOob: outside the tile's rows or columns)
    uint32_t va[4], vb[4];
    __amdgpu_buffer_rsrc_t rsA, rsB, rsB2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (MODE == 0) {   // A = dy rows (k = d), B = W2 [seg][d][w] read along its units
            const int m = rsub + 64 * i;
            va[i] = m < nr ? (uint32_t)(((m0 + m) * d + part * 8) * 2) : kOob;
            const int n = n0 + 8 * mc;
            const size_t seg = (size_t)n / w;
            vb[i] = n < N ? (uint32_t)((seg * d * w + (size_t)(kr + 16 * i) * w + (n - seg * w)) * 2) : kOob;
        } else if (MODE == 1) {   // A = [dp | dq] rows (k = unit), B = [W1; W3] rows read along d
            const int m = rsub + 64 * i;
            va[i] = m < nr ? (uint32_t)(((m0 + m) * wg + part * 8) * 2) : kOob;
            const int n = n0 + 8 * mc;
            vb[i] = n < N ? (uint32_t)(((size_t)(kr + 16 * i) * d + n) * 2) : kOob;
        } else if (MODE == 2) {   // A(m = column of dy, k = row), B(n = unit, k = row) of a
            const int m = m0 + 8 * mc, n = n0 + 8 * mc;
            va[i] = 8 * mc < nr ? (uint32_t)(((size_t)(kr + 16 * i) * d + m) * 2) : kOob;
            vb[i] = n < N ? (uint32_t)(((size_t)(kr + 16 * i) * wg + n) * 2) : kOob;
        } else {   // A(m = unit of [dp | dq], k = row), B(n = column of x, k = row: gathered token)
            const int m = m0 + 8 * mc, n = n0 + 8 * mc;
            const bool q = m >= (int)wg;
            const size_t mm = q ? m - wg : m;
            va[i] = 8 * mc < nr ? (uint32_t)(((size_t)(kr + 16 * i) * wg + mm) * 2) + (q ? dq_off : 0u) : kOob;
            vb[i] = n < N ? (uint32_t)(n * 2) : kOob;
        }
    }
    if (MODE == 0) {
        rsA = bg_rsrc(dy + ro * d);
        rsB = bg_rsrc(Gr.sh ? (const uint16_t *)A.w2_s : (const uint16_t *)A.w2_r + (size_t)Gr.r * d * w);
    } else if (MODE == 1) {
        rsA = bg_rsrc(dp + ro * wg);
        rsB = bg_rsrc(Gr.sh ? (const uint16_t *)A.w1_s : (const uint16_t *)A.w1_r + (size_t)Gr.r * w * d);
        rsB2 = bg_rsrc(Gr.sh ? (const uint16_t *)A.w3_s : (const uint16_t *)A.w3_r + (size_t)Gr.r * w * d);
    } else if (MODE == 2) {
        rsA = bg_rsrc(dy + ro * d);
        rsB = bg_rsrc((const uint16_t *)(Gr.sh ? A.a_s : A.a_r) + ro * wg);
    } else {
        rsA = bg_rsrc(dp + ro * wg);
        rsB = bg_rsrc(A.x);
    }
    if (MODE != 1) rsB2 = rsB;
    // mode 3: byte offset of the token row of chunk i's k row in the step whose loads go out next
    uint32_t tkb[4] = {0u, 0u, 0u, 0u};
    auto tok_row = [&](int i, int k0) -> uint32_t {
        const int k = min(k0 + kr + 16 * i, K - 1);
        const int t = Gr.sh ? k : A.sorted_token[ro + k];
        return (uint32_t)t * (uint32_t)(d * 2);
    };

    // offsets of k step kt: uniform (scalar) adds to the fixed chunk offsets
    struct KS {
        uint32_t sa, sb;
        int k0;
        bool b3;
    };
    auto kstate = [&](int kt) -> KS {
        KS s;
        s.k0 = kt * 64;
        s.b3 = false;
        if (MODE == 0) { s.sa = (uint32_t)kt * 128u; s.sb = (uint32_t)(kt * 64 * w * 2); }
        if (MODE == 1) {
            s.b3 = s.k0 >= (int)wg;
            const int kk = s.b3 ? s.k0 - (int)wg : s.k0;
            s.sa = (s.b3 ? dq_off : 0u) + (uint32_t)kk * 2u;
            s.sb = (uint32_t)((size_t)kk * d * 2);
        }
        if (MODE == 2) { s.sa = (uint32_t)((size_t)s.k0 * d * 2); s.sb = (uint32_t)((size_t)s.k0 * wg * 2); }
        if (MODE == 3) { s.sa = (uint32_t)((size_t)s.k0 * wg * 2); s.sb = 0u; }
        return s;
    };
    uint4 ra[4], rb[4];
    // quarter ph of step s: chunk ph of both operands
    auto gload = [&](const KS &s, int ph) {
        const bool kv = MODE < 2 || s.k0 + kr + 16 * ph < K;   // the transposed chunks' k row is inside the group
        ra[ph] = bg_load(rsA, kv ? va[ph] : kOob, s.sa);
        if (MODE == 3) {
            rb[ph] = bg_load(rsB, (kv && vb[ph] != kOob) ? tkb[ph] + vb[ph] : kOob, 0u);
            tkb[ph] = tok_row(ph, s.k0 + 64);   // the same chunk's row one step on
        } else {
            rb[ph] = bg_load(s.b3 ? rsB2 : rsB, kv ? vb[ph] : kOob, s.sb);
        }
    };
    auto sstore = [&](int st, int ph) {
        *(uint4 *)(stA(st) + lds_off(AT, ph)) = ra[ph];
        *(uint4 *)(stB(st) + lds_off(BT, ph)) = rb[ph];
    };

    f32x16 acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    // fragment of the 32-row block at `base` for k sub-step ks (16 k)
    const int lsw = (l32 & 7) ^ ((l32 >> 3) & 1);
    const int g4 = lane >> 4, j16 = lane & 15;
    const int trow = 8 * (g4 >> 1) + (j16 >> 2), tcol = 16 * (g4 & 1) + 4 * (j16 & 3);
    auto frag = [&](const uint8_t *s, bool tr, int base, int ks) -> bf16x8 {
        if (!tr) return *(const bf16x8 *)(s + (base + l32) * KC + ((2 * ks + lhi) ^ lsw) * 16);
        const uint8_t *p = s + (16 * ks + trow) * KT + (base + tcol) * 2;
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)p);
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(p + 4 * KT));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto frags = [&](auto ml_t, int st, int ks, bf16x8 (&fa)[4], bf16x8 (&fb)[2]) {
        constexpr int ML = decltype(ml_t)::value;
#pragma unroll
        for (int ma = 0; ma < ML; ++ma) fa[ma] = frag(stA(st), AT, (2 * ma + wm) * 32, ks);
        if (ML > 0) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) fb[nb] = frag(stB(st), BT, wn * 64 + nb * 32, ks);
        }
    };
    auto mma = [&](auto ml_t, const bf16x8 (&fa)[4], const bf16x8 (&fb)[2]) {
        constexpr int ML = decltype(ml_t)::value;
#pragma unroll
        for (int ma = 0; ma < ML; ++ma)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                acc[ma][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ma], fb[nb], acc[ma][nb], 0, 0, 0);
    };

    using yes = std::true_type;
    using no = std::false_type;
    const int nk = cdiv(K, 64);
    const int nblk = cdiv(nr, 32);
    const int ml = __builtin_amdgcn_readfirstlane(min(4, (nblk - wm + 1) >> 1));
    if (nk > 0) {
        const KS s0 = kstate(0);
        if (MODE == 3) {
#pragma unroll
            for (int i = 0; i < 4; ++i) tkb[i] = tok_row(i, 0);
        }
#pragma unroll
        for (int ph = 0; ph < 4; ++ph) gload(s0, ph);
#pragma unroll
        for (int ph = 0; ph < 4; ++ph) sstore(0, ph);
        __syncthreads();
        auto kloop = [&](auto ml_t) {
            if (nk > 1) {
                const KS s1 = kstate(1);
#pragma unroll
                for (int ph = 0; ph < 4; ++ph) {
                    gload(s1, ph);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // sub-step 0's fragments of each step are read under the last MFMAs of the
            // step before, after its barrier (as in the forward's k loop)
            bf16x8 fa0[4], fb0[2], fa1[4], fb1[2];
            frags(ml_t, 0, 0, fa0, fb0);
            auto kstep = [&](int kt, auto more_t, auto more2_t) {
                constexpr bool MORE = decltype(more_t)::value, MORE2 = decltype(more2_t)::value;
                const int st = kt & 1;
                KS sn;
                if (MORE2) sn = kstate(kt + 2);
                frags(ml_t, st, 1, fa1, fb1);
                if (MORE) { sstore(st ^ 1, 0); if (MORE2) gload(sn, 0); }
                __builtin_amdgcn_sched_barrier(0);
                mma(ml_t, fa0, fb0);
                frags(ml_t, st, 2, fa0, fb0);
                if (MORE) { sstore(st ^ 1, 1); if (MORE2) gload(sn, 1); }
                __builtin_amdgcn_sched_barrier(0);
                mma(ml_t, fa1, fb1);
                frags(ml_t, st, 3, fa1, fb1);
                if (MORE) { sstore(st ^ 1, 2); if (MORE2) gload(sn, 2); }
                __builtin_amdgcn_sched_barrier(0);
                mma(ml_t, fa0, fb0);
                if (MORE) { sstore(st ^ 1, 3); if (MORE2) gload(sn, 3); }
                __builtin_amdgcn_sched_barrier(0);
                if (MORE) {
                    __syncthreads();
                    frags(ml_t, st ^ 1, 0, fa0, fb0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma(ml_t, fa1, fb1);
                } else {
                    mma(ml_t, fa1, fb1);
                    __syncthreads();
                }
            };
            int kt = 0;
            for (; kt + 2 < nk; ++kt) kstep(kt, yes{}, yes{});
            if (kt + 1 < nk) kstep(kt++, yes{}, no{});
            kstep(kt, no{}, no{});
        };
        using std::integral_constant;
        if (ml >= 4) kloop(integral_constant<int, 4>{});
        else if (ml == 3) kloop(integral_constant<int, 3>{});
        else if (ml == 2) kloop(integral_constant<int, 2>{});
        else if (ml == 1) kloop(integral_constant<int, 1>{});
        else kloop(integral_constant<int, 0>{});
    }

    // ---- epilogue: lane holds column n = l32 of each B block; register 4q + e
    //      holds tile row (2 ma + wm) * 32 + 8q + 4 lhi + e.  The tile goes out
    //      through the idle LDS stages as whole rows of 16-byte stores (a row
    //      per wave instruction; bf16: two rows): stored straight from the
    //      MFMA layout, every instruction would write 4-byte pieces of two rows,
    //      4x the store instructions, which took 7-12 us per tile.  fp32 tiles
    //      go in two passes of 128 rows (pitch 1056 B), bf16 tiles in one pass
    //      (pitch 544 B); either pitch puts the rows r and r + 4 of a fragment
    //      write on different banks.
    const bool obf = MODE == 0 || (MODE == 1 && !Gr.sh);   // bf16 output rows
    // element offset of columns [n, n + 8) (bf16) / [n, n + 4) (fp32) in an output
    // row, per lane; mode 2: in its W2 segment, whose base goes in too
    const int ncol = obf ? 8 * l32 : 4 * lane;
    const int nabs = n0 + ncol;
    size_t nofs = (size_t)nabs;
    if (MODE == 2) {
        const size_t seg = (size_t)nabs / w;
        nofs = seg * d * w + (nabs - seg * w);
    }
    const bool ncol_ok = nabs < N;
    auto row_ptr = [&](int tr) -> uint8_t * {   // output row of tile row tr (bytes; the lane's columns)
        const size_t m = (size_t)(m0 + tr);
        if (MODE == 0) return (uint8_t *)((uint16_t *)(Gr.sh ? A.da_s : A.da_r) + (ro + m) * wg + nofs);
        if (MODE == 1) {
            if (obf) return (uint8_t *)((uint16_t *)A.dxr + (ro + m) * d + nofs);
            return (uint8_t *)(A.dxs + m * d + nofs);
        }
        if (MODE == 2) return (uint8_t *)((Gr.sh ? A.dw2_s : A.dw2_r + (size_t)Gr.r * d * w) + m * w + nofs);
        const bool q = m >= wg;
        float *o = Gr.sh ? (q ? A.dw3_s : A.dw1_s) : (q ? A.dw3_r : A.dw1_r) + (size_t)Gr.r * w * d;
        return (uint8_t *)(o + (q ? m - wg : m) * d + nofs);
    };
    auto emit = [&](auto bf_t) {
        constexpr bool BF = decltype(bf_t)::value;
        constexpr int PR = BF ? 256 : 128;        // tile rows per pass
        constexpr int PITCH = BF ? 544 : 1056;
#pragma unroll
        for (int pass = 0; pass < 256 / PR; ++pass) {
            if (pass * PR >= nr) break;
            if (pass > 0) __syncthreads();         // the previous pass's rows are read
#pragma unroll
            for (int ma = 0; ma < 4; ++ma) {
                const int rb0 = (2 * ma + wm) * 32;
                if (rb0 < pass * PR || rb0 >= (pass + 1) * PR || rb0 >= nr) continue;
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int c = wn * 64 + nb * 32 + l32;
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int lr = rb0 - pass * PR + 8 * (e >> 2) + 4 * lhi + (e & 3);
                        if (BF) *(uint16_t *)(smem + lr * PITCH + c * 2) = f2bf(acc[ma][nb][e]);
                        else *(float *)(smem + lr * PITCH + c * 4) = acc[ma][nb][e];
                    }
                }
            }
            __syncthreads();
            // wave w stores rows w, w + 8, ... of the pass (bf16: a row per half-wave)
            constexpr int RPI = BF ? 2 : 1;       // rows per store instruction
#pragma unroll
            for (int i = 0; i < PR / (8 * RPI); ++i) {
                const int lr = (i * 8 + wave) * RPI + (BF ? lhi : 0);
                const int tr = pass * PR + lr;
                const uint4 v = *(const uint4 *)(smem + lr * PITCH + (BF ? l32 : lane) * 16);
                if (tr < nr && ncol_ok) *(uint4 *)row_ptr(tr) = v;
            }
        }
    };
    if (obf) emit(std::true_type{});
    else emit(std::false_type{});
}

// Locates block lb of a mode's range and runs its tile.  The tile list is
// ordered group by group; a group's rows (modes 0, 1) or its M (modes 2, 3)
// are cut into mt runs of equal length rounded up to 32, as in the forward.
// XCD-aware order: as in bgemm_kernel (a mode's range starts on XCD 0).
template <int MODE>
__device__ __forceinline__ void wide_run(const BgArgs &A, int lb, uint8_t *smem, int *s_pref, int &s_maxg) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (A.Ks > 0 ? 1 : 0) + A.Nr;
    if (wave == 0) {
        int carry = 0, mx = 0;
        if (lane == 0) s_pref[0] = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            int tiles = 0;
            if (g < G) {
                const Group Gr = group_of(A, g);
                int M, N, K;
                dims<MODE>(A, Gr, M, N, K);
                tiles = cdiv(M, 256) * cdiv(N, 256);
            }
            mx = max(mx, tiles);
            int incl = tiles;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            if (g < G) s_pref[g + 1] = carry + incl;
            carry += __shfl(incl, 63, 64);
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
        if (lane == 0) s_maxg = mx;
    }
    __syncthreads();
    const int NT = s_pref[G];
    if (lb >= NT) return;
    auto spread = [](int j, int n) {
        const int per = (n + 7) / 8, tall = n % 8 == 0 ? 8 : n % 8, x = j % 8, l = j / 8;
        return x < tall ? x * per + l : tall * per + (x - tall) * (per - 1) + l;
    };
    auto group_at = [&](int v) {
        int lo = 0, hi = G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_pref[mid] <= v) lo = mid; else hi = mid;
        }
        return lo;
    };
    const bool whole = (MODE == 0 || (MODE == 1 && A.Ks <= 1)) && s_maxg * 8 <= NT;
    int g, lt;
    if (whole) {
        const int v = spread(lb, NT);
        g = group_at(v);
        lt = v - s_pref[g];
    } else {
        g = group_at(lb);
        lt = spread(lb - s_pref[g], s_pref[g + 1] - s_pref[g]);
    }
    // the group and tile are the same in every lane: in SGPRs, the buffer descriptors built from
    // them are too (a descriptor in VGPRs puts a waterfall loop around every load that uses it)
    g = __builtin_amdgcn_readfirstlane(g);
    lt = __builtin_amdgcn_readfirstlane(lt);
    Group Gr = group_of(A, g);
    Gr.rows = __builtin_amdgcn_readfirstlane(Gr.rows);
    Gr.roff = __builtin_amdgcn_readfirstlane(Gr.roff);
    int M, N, K;
    dims<MODE>(A, Gr, M, N, K);
    const int mt = cdiv(M, 256);
    const int run = (cdiv(M, mt) + 31) & ~31;
    const int m0 = (lt % mt) * run, n0 = (lt / mt) * 256;
    wide_tile<MODE>(A, Gr, m0, min(run, M - m0), n0, M, N, K, smem);
}

__global__ __launch_bounds__(512) void bgemm_wide_kernel(BgArgs A, WideRange R) {
    __shared__ __attribute__((aligned(16))) uint8_t smem[wide::SMEM];
    __shared__ int s_pref[BG_MAXG + 1];
    __shared__ int s_maxg;
    const int o = blockIdx.x >> 3;
    const int slot = o < R.oct[0] ? 0 : (o < R.oct[0] + R.oct[1] ? 1 : 2);
    const int lb = blockIdx.x - 8 * (slot == 0 ? 0 : (slot == 1 ? R.oct[0] : R.oct[0] + R.oct[1]));
    switch (R.mode[slot]) {
        case 0: wide_run<0>(A, lb, smem, s_pref, s_maxg); break;
        case 1: wide_run<1>(A, lb, smem, s_pref, s_maxg); break;
        case 2: wide_run<2>(A, lb, smem, s_pref, s_maxg); break;
        default: wide_run<3>(A, lb, smem, s_pref, s_maxg); break;
    }
}

// dx_ffn[t] = dxs[t] (shared experts, or 0) + sum_k dxr[slot_of[t,k]], k in
// order.  A thread owns 8 columns of a token: its K' slots are read first,
// then the K' row pieces go out together (4 at a time), summed in k order.
template <typename RT>
__global__ __launch_bounds__(256) void gather_dx_kernel(int T, int d, int K, const float *__restrict__ dxs,
                                                        const RT *__restrict__ dxr,
                                                        const int32_t *__restrict__ slot_of,
                                                        float *__restrict__ dx) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 8 columns of one token
    const int q = d / 8;
    if (i >= (int64_t)T * q) return;
    const int t = (int)(i / q), c = (int)(i % q) * 8;
    float acc[8];
    if (dxs) {
        load8(dxs + (size_t)t * d + c, acc);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    }
    int slot[kRouteMaxTopK];
#pragma unroll
    for (int k = 0; k < kRouteMaxTopK; ++k) slot[k] = k < K ? slot_of[(size_t)t * K + k] : -1;
#pragma unroll
    for (int k0 = 0; k0 < kRouteMaxTopK; k0 += 4) {
        if (k0 >= K) break;
        float v[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (slot[k0 + u] >= 0) load8(dxr + (size_t)slot[k0 + u] * d + c, v[u]);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (slot[k0 + u] >= 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
            }
    }
    for (int k = kRouteMaxTopK; k < K; ++k) {   // K' beyond the routing kernels' limit (other routers)
        const int sl = slot_of[(size_t)t * K + k];
        if (sl < 0) continue;
        float v[8];
        load8(dxr + (size_t)sl * d + c, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += v[e];
    }
    store8(dx + (size_t)t * d + c, acc);
}

// ---------------------------------------------------------------------------
// Router backward.  One wave per token, lane = expert (up to 4 per lane).
// ds_r = dgate (r selected) + (alpha1 f_r + alpha2 f'_{g(r)}) / T;
// dz_r = s_r (ds_r - sum_r' s_r' ds_r'), in fp64 (ds_r - <s, ds> cancels when
// the balance terms dominate), the sum by a fixed butterfly, rounded to fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void router_dz_kernel(int T, int Nr, int K, int D, float alpha1, float alpha2,
                                                        const float *__restrict__ probs,
                                                        const int32_t *__restrict__ idx,
                                                        const float *__restrict__ dgate,
                                                        const float *__restrict__ f, const float *__restrict__ fdev,
                                                        float *__restrict__ dz) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (t >= T) return;
    const int gsz = Nr / D;
    double ds[4], s[4];
    double dot = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = lane + 64 * j;
        ds[j] = 0.0;
        s[j] = 0.0;
        if (r < Nr) {
            s[j] = (double)probs[(size_t)t * Nr + r];
            ds[j] = ((double)alpha1 * (double)f[r] + (double)alpha2 * (double)fdev[r / gsz]) / (double)T;
        }
    }
    for (int k = 0; k < K; ++k) {
        const int r = idx[(size_t)t * K + k];
        const double g = (double)dgate[(size_t)t * K + k];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (r == lane + 64 * j) ds[j] += g;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) dot += s[j] * ds[j];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) dot += __shfl_xor(dot, o, 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = lane + 64 * j;
        if (r < Nr) dz[(size_t)t * Nr + r] = (float)(s[j] * (ds[j] - dot));
    }
}

// dx = dh + dx_ffn + dz E.  Workgroup tile: 16 TPT tokens x 128 columns,
// thread (token group tg, column group cg) owns TPT tokens x 8 columns (TPT =
// 8: 64 accumulators, 4 LDS reads of 16 bytes per 64 fmas; TPT = 4 for small
// batches, twice the workgroups).  The expert dimension goes through LDS 32
// at a time: dz transposed to [r][t], E as [r][c]; every output's sum over r
// runs in ascending order.
template <typename DT, int TPT>
__global__ __launch_bounds__(256) void router_dx_kernel(int T, int d, int Nr, const DT *__restrict__ dh,
                                                        const float *__restrict__ dx_ffn,
                                                        const float *__restrict__ dz, const float *__restrict__ E,
                                                        float *__restrict__ dx) {
    constexpr int TT = 16 * TPT;   // tokens of the tile
    __shared__ __attribute__((aligned(16))) float s_z[32][TT];
    __shared__ __attribute__((aligned(16))) float s_e[32][128];
    const int t0 = blockIdx.x * TT, c0 = blockIdx.y * 128;
    const int tid = threadIdx.x, cg = tid & 15, tg = tid >> 4;
    float acc[TPT][8];
#pragma unroll
    for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
    for (int r0 = 0; r0 < Nr; r0 += 32) {
        // dz[t0 + t][r0 + 4q .. 4q + 3] -> s_z[4q + e][t]; E rows r0 .. r0 + 31 -> s_e
#pragma unroll
        for (int i = 0; i < TPT / 2; ++i) {
            const int t = tid % TT, q = tid / TT + (256 / TT) * i;   // q: 0..7
            const int r = r0 + 4 * q;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t0 + t < T) {
                const float *src = dz + (size_t)(t0 + t) * Nr + r;
                if ((Nr & 3) == 0 && r + 3 < Nr) v = *(const float4 *)src;   // 16-byte aligned rows
                else {
                    v.x = r < Nr ? src[0] : 0.f;
                    v.y = r + 1 < Nr ? src[1] : 0.f;
                    v.z = r + 2 < Nr ? src[2] : 0.f;
                    v.w = r + 3 < Nr ? src[3] : 0.f;
                }
            }
            s_z[4 * q][t] = v.x;
            s_z[4 * q + 1][t] = v.y;
            s_z[4 * q + 2][t] = v.z;
            s_z[4 * q + 3][t] = v.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int idx = tid + 256 * i, rr = idx >> 5, c4 = (idx & 31) * 4;
            const int r = r0 + rr, c = c0 + c4;
            *(float4 *)&s_e[rr][c4] = (r < Nr && c < d) ? *(const float4 *)(E + (size_t)r * d + c)
                                                        : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __syncthreads();
        const int nr = min(32, Nr - r0);
        for (int r = 0; r < nr; ++r) {
            float z[TPT];
#pragma unroll
            for (int i = 0; i < TPT; i += 4) {
                const float4 z4 = *(const float4 *)&s_z[r][tg * TPT + i];
                z[i] = z4.x; z[i + 1] = z4.y; z[i + 2] = z4.z; z[i + 3] = z4.w;
            }
            const float4 e0 = *(const float4 *)&s_e[r][cg * 8], e1 = *(const float4 *)&s_e[r][cg * 8 + 4];
            const float e[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
            for (int i = 0; i < TPT; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(z[i], e[j], acc[i][j]);
        }
        __syncthreads();
    }
    const int c = c0 + cg * 8;
    if (c >= d) return;   // d % 64 == 0: a thread's 8 columns are all inside or all outside
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int t = t0 + tg * TPT + i;
        if (t >= T) continue;
        float hv[8], fv[8], o[8];
        load8(dh + (size_t)t * d + c, hv);
        if (dx_ffn) load8(dx_ffn + (size_t)t * d + c, fv);
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = (hv[j] + (dx_ffn ? fv[j] : 0.0f)) + acc[i][j];
        store8(dx + (size_t)t * d + c, o);
    }
}

// dE partials over token chunks of kDeTokens: workgroup (chunk j, 16 RT
// experts, 128 columns); thread (expert group eg, column group cg) owns RT
// experts x 8 columns and accumulates, t ascending, dz[t, r] x[t, c]; the
// chunk's dz rows and x rows (as fp32) go through LDS 32 tokens at a time.
// part[j][r][c], row pitch d + 4; column d carries sum_t dz (the bias
// gradient), from the workgroups of the first column tile.
constexpr int kDeTokens = 128;
template <typename DT, int RT>
__global__ __launch_bounds__(256) void router_de_part_kernel(int T, int d, int Nr, const DT *__restrict__ x,
                                                             const float *__restrict__ dz,
                                                             float *__restrict__ part) {
    constexpr int TR = 16 * RT;   // experts of the tile
    __shared__ __attribute__((aligned(16))) float s_z[32][TR];
    __shared__ __attribute__((aligned(16))) float s_x[32][128];
    const int j = blockIdx.x, rt0 = blockIdx.z * TR, c0 = blockIdx.y * 128;
    const int tid = threadIdx.x, cg = tid & 15, eg = tid >> 4;
    const int tc0 = j * kDeTokens, n = min(kDeTokens, T - tc0);
    float acc[RT][8];
#pragma unroll
    for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[i][k] = 0.0f;
    float bsum = 0.0f;   // thread tid < TR of the first column tile: sum over t of dz[t, rt0 + tid]
    for (int s0 = 0; s0 < n; s0 += 32) {
        // dz rows of 32 tokens (TR experts each), x rows (128 columns) as fp32
        for (int i = tid; i < 32 * TR / 4; i += 256) {
            const int tt = i / (TR / 4), r4 = (i % (TR / 4)) * 4;
            const int t = tc0 + s0 + tt, r = rt0 + r4;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (s0 + tt < n) {
                const float *src = dz + (size_t)t * Nr + r;
                if ((Nr & 3) == 0 && r + 3 < Nr) v = *(const float4 *)src;   // 16-byte aligned rows
                else {
                    v.x = r < Nr ? src[0] : 0.f;
                    v.y = r + 1 < Nr ? src[1] : 0.f;
                    v.z = r + 2 < Nr ? src[2] : 0.f;
                    v.w = r + 3 < Nr ? src[3] : 0.f;
                }
            }
            *(float4 *)&s_z[tt][r4] = v;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int idx = tid + 256 * i, tt = idx >> 4, c8 = (idx & 15) * 8;
            float v[8];
            if (s0 + tt < n && c0 + c8 < d) load8(x + (size_t)(tc0 + s0 + tt) * d + c0 + c8, v);
            else {
#pragma unroll
                for (int k = 0; k < 8; ++k) v[k] = 0.0f;
            }
            *(float4 *)&s_x[tt][c8] = make_float4(v[0], v[1], v[2], v[3]);
            *(float4 *)&s_x[tt][c8 + 4] = make_float4(v[4], v[5], v[6], v[7]);
        }
        __syncthreads();
        const int m = min(32, n - s0);
        if (blockIdx.y == 0 && tid < TR)
            for (int tt = 0; tt < m; ++tt) bsum += s_z[tt][tid];
        for (int tt = 0; tt < m; ++tt) {
            float z[RT], xv[8];
#pragma unroll
            for (int i = 0; i < RT; i += 4) {
                const float4 z4 = *(const float4 *)&s_z[tt][eg * RT + i];
                z[i] = z4.x; z[i + 1] = z4.y; z[i + 2] = z4.z; z[i + 3] = z4.w;
            }
            const float4 x0 = *(const float4 *)&s_x[tt][cg * 8], x1 = *(const float4 *)&s_x[tt][cg * 8 + 4];
            xv[0] = x0.x; xv[1] = x0.y; xv[2] = x0.z; xv[3] = x0.w;
            xv[4] = x1.x; xv[5] = x1.y; xv[6] = x1.z; xv[7] = x1.w;
#pragma unroll
            for (int i = 0; i < RT; ++i)
#pragma unroll
                for (int k = 0; k < 8; ++k) acc[i][k] = __builtin_fmaf(z[i], xv[k], acc[i][k]);
        }
        __syncthreads();
    }
    const int c = c0 + cg * 8;
#pragma unroll
    for (int i = 0; i < RT; ++i) {
        const int r = rt0 + eg * RT + i;
        if (r >= Nr || c >= d) continue;
        float *o = part + ((size_t)j * Nr + r) * (d + 4) + c;
        *(float4 *)o = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
        *(float4 *)(o + 4) = make_float4(acc[i][4], acc[i][5], acc[i][6], acc[i][7]);
    }
    if (blockIdx.y == 0 && tid < TR && rt0 + tid < Nr) part[((size_t)j * Nr + rt0 + tid) * (d + 4) + d] = bsum;
}

// dE[r][c] = sum_j part[j][r][c] (j ascending); dbias[r] = sum_j part[j][r][d].
__global__ __launch_bounds__(256) void router_de_sum_kernel(int nchunk, int d, int Nr, const float *__restrict__ part,
                                                            float *__restrict__ dE, float *__restrict__ dbias) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)Nr * (d + 1)) return;
    const int r = (int)(i / (d + 1)), c = (int)(i % (d + 1));
    float a = 0.0f;
    for (int j = 0; j < nchunk; ++j) a += part[((size_t)j * Nr + r) * (d + 4) + c];
    if (c < d) dE[(size_t)r * d + c] = a;
    else if (dbias) dbias[r] = a;
}

template <int MODE>
hipError_t launch_bg(const BgArgs &a, int tiles, hipStream_t s) {
    if (tiles <= 0) return hipSuccess;
    bgemm_kernel<MODE><<<tiles, 256, 0, s>>>(a);
    return hipGetLastError();
}

// Upper bounds of the tile counts: routed row tiles <= T K'/128 + N'.
int row_tile_bound(const moe_problem &p) {
    const int rt = p.n_routed > 0 ? (int)(((int64_t)p.T * p.top_k) / 128) + p.n_routed : 0;
    return rt + (p.n_shared > 0 ? cdiv(p.T, 128) : 0);
}

}  // namespace

// ---------------------------------------------------------------------------
hipError_t launch_combine_backward(const moe_problem &p, const void *dh, const void *y_routed, const float *gate,
                                   const int32_t *slot_of, void *dy_routed, float *dgate, hipStream_t s) {
    if (p.T == 0 || p.top_k == 0) return hipSuccess;
    const int grid = cdiv(p.T, 4);
    if (p.dtype == MOE_BF16)
        combine_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, (const uint16_t *)dh,
                                                          (const uint16_t *)y_routed, gate, slot_of,
                                                          (uint16_t *)dy_routed, dgate);
    else
        combine_bwd_kernel<float><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, (const float *)dh, (const float *)y_routed,
                                                       gate, slot_of, (float *)dy_routed, dgate);
    return hipGetLastError();
}

hipError_t launch_expert_backward(const moe_problem &p, const BwdFfnArgs &b, hipStream_t s) {
    BgArgs a{};
    a.T = p.T; a.d = p.d; a.Ks = p.n_shared; a.Nr = p.n_routed; a.w = p.inter;
    a.offsets = b.offsets; a.sorted_token = b.sorted_token;
    a.x = b.x; a.dh = b.dh; a.dy_r = b.dy_routed;
    a.w1_r = b.w1_r; a.w3_r = b.w3_r; a.w2_r = b.w2_r; a.w1_s = b.w1_s; a.w3_s = b.w3_s; a.w2_s = b.w2_s;
    a.da_r = b.da_r; a.da_s = b.da_s; a.dp_r = b.dp_r; a.dq_r = b.dq_r; a.a_r = b.a_r;
    a.dp_s = b.dp_s; a.dq_s = b.dq_s; a.a_s = b.a_s;
    a.dxr = b.dxr; a.dxs = b.dxs;
    a.dw1_r = b.dw1_r; a.dw3_r = b.dw3_r; a.dw2_r = b.dw2_r; a.dw1_s = b.dw1_s; a.dw3_s = b.dw3_s;
    a.dw2_s = b.dw2_s;
    const int G = (p.n_shared > 0 ? 1 : 0) + p.n_routed;
    const int wmax = std::max(p.inter, p.n_shared * p.inter);
    const int rt = row_tile_bound(p);
    const int t0 = rt * cdiv(wmax, 128);                       // da
    const int t1 = rt * cdiv(p.d, 128);                        // dxr
    const int t2 = G * cdiv(p.d, 128) * cdiv(wmax, 128);       // dW2
    const int t3 = G * cdiv(2 * wmax, 128) * cdiv(p.d, 128);   // dW1, dW3
    const int t4 = rt * cdiv(2 * wmax, 128);                   // p, q -> dp, dq, a
    hipError_t e;
    (void)t4;
    if (p.dtype == MOE_BF16) {
        // 256 x 256 tiles: da alone, then (after the recompute) dx rows, dW1/dW3, dW2 in one launch
        const int rw = (p.n_routed > 0 ? (int)(((int64_t)p.T * p.top_k) / 256) + p.n_routed : 0) +
                       (p.n_shared > 0 ? cdiv(p.T, 256) : 0);
        const int o0 = cdiv(rw * cdiv(wmax, 256), 8);
        const int o1 = cdiv(rw * cdiv(p.d, 256), 8);
        const int o3 = cdiv(G * cdiv(2 * wmax, 256) * cdiv(p.d, 256), 8);
        const int o2 = cdiv(G * cdiv(p.d, 256) * cdiv(wmax, 256), 8);
        if (o0 > 0) {
            const WideRange r0{{0, 0, 0}, {o0, 0, 0}};
            bgemm_wide_kernel<<<8 * o0, wide::NT, 0, s>>>(a, r0);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        // p, q recomputed by the forward up kernel, with the backward epilogue
        FfnArgs f{};
        f.x = b.x; f.offsets = b.offsets; f.sorted_token = b.sorted_token;
        f.w1_r = b.w1_r; f.w3_r = b.w3_r; f.w1_s = b.w1_s; f.w3_s = b.w3_s;
        f.act_shared = b.a_s; f.act_routed = b.a_r;
        moe_problem q = p;
        if (p.T == 0 || p.top_k == 0) q.n_routed = 0, q.top_k = 0;
        if (p.T == 0) q.n_shared = 0;
        if ((q.n_routed > 0 || q.n_shared > 0) &&
            (e = launch_expert_up_backward(q, f, b.da_s, b.da_r, b.dp_s, b.dp_r, b.dq_s, b.dq_r, s)) != hipSuccess)
            return e;
        if (o1 + o3 + o2 > 0) {
            const WideRange r{{1, 3, 2}, {o1, o3, o2}};
            bgemm_wide_kernel<<<8 * (o1 + o3 + o2), wide::NT, 0, s>>>(a, r);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    } else {
        if ((e = launch_bg<0>(a, t0, s)) != hipSuccess) return e;
        if ((e = launch_bg<4>(a, t4, s)) != hipSuccess) return e;
        if ((e = launch_bg<1>(a, t1, s)) != hipSuccess) return e;
        if ((e = launch_bg<2>(a, t2, s)) != hipSuccess) return e;
        if ((e = launch_bg<3>(a, t3, s)) != hipSuccess) return e;
    }
    if (p.T > 0) {
        const int64_t n = (int64_t)p.T * (p.d / 8);
        const int grid = (int)((n + 255) / 256);
        const float *dxs = p.n_shared > 0 ? b.dxs : nullptr;
        if (p.dtype == MOE_BF16)
            gather_dx_kernel<uint16_t><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, dxs, (const uint16_t *)b.dxr,
                                                            b.slot_of, b.dx_ffn);
        else
            gather_dx_kernel<float><<<grid, 256, 0, s>>>(p.T, p.d, p.top_k, dxs, (const float *)b.dxr, b.slot_of,
                                                         b.dx_ffn);
    }
    return hipGetLastError();
}

hipError_t launch_route_backward(const moe_problem &p, int groups, float alpha1, float alpha2, const void *x,
                                 const float *centroids, const float *probs, const int32_t *idx,
                                 const float *dgate, const float *f, const float *f_dev, const void *dh,
                                 const float *dx_ffn, float *dx, float *dcentroids, float *dbias, float *dz,
                                 float *part, hipStream_t s) {
    if (p.T > 0) {
        router_dz_kernel<<<cdiv(p.T, 4), 256, 0, s>>>(p.T, p.n_routed, p.top_k, groups, alpha1, alpha2, probs, idx,
                                                      dgate, f, f_dev, dz);
        // 64-token tiles while 128-token ones would leave fewer than two workgroups per CU
        const bool small = (int64_t)cdiv(p.T, 128) * cdiv(p.d, 128) < 512;
        const dim3 gx(cdiv(p.T, small ? 64 : 128), cdiv(p.d, 128));
#define MOE_DX(DT, TPT) router_dx_kernel<DT, TPT><<<gx, 256, 0, s>>>(p.T, p.d, p.n_routed, (const DT *)dh, dx_ffn, \
                                                                     dz, centroids, dx)
        if (p.dtype == MOE_BF16) {
            if (small) MOE_DX(uint16_t, 4); else MOE_DX(uint16_t, 8);
        } else {
            if (small) MOE_DX(float, 4); else MOE_DX(float, 8);
        }
#undef MOE_DX
    }
    const int nchunk = cdiv(p.T, kDeTokens);
    if (nchunk > 0) {
        // 64-expert tiles up to 64 routed experts, else 128-expert tiles
        const bool small = p.n_routed <= 64;
        const dim3 g(nchunk, cdiv(p.d, 128), cdiv(p.n_routed, small ? 64 : 128));
#define MOE_DE(DT, RT) router_de_part_kernel<DT, RT><<<g, 256, 0, s>>>(p.T, p.d, p.n_routed, (const DT *)x, dz, part)
        if (p.dtype == MOE_BF16) {
            if (small) MOE_DE(uint16_t, 4); else MOE_DE(uint16_t, 8);
        } else {
            if (small) MOE_DE(float, 4); else MOE_DE(float, 8);
        }
#undef MOE_DE
    }
    const int64_t m = (int64_t)p.n_routed * (p.d + 1);
    router_de_sum_kernel<<<(int)((m + 255) / 256), 256, 0, s>>>(nchunk, p.d, p.n_routed, part, dcentroids, dbias);
    return hipGetLastError();
}

int route_backward_chunks(int T) { return cdiv(T, kDeTokens); }

}  // namespace moe
