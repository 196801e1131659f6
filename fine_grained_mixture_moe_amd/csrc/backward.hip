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
//   bgemm_kernel<MODE>   one grouped GEMM on MFMA for the five products below
//      0  da   = dy . W2              (A rows k-contiguous, B = W2 read transposed)
//      1  dxr  = dp . W1 + dq . W3    (A k-contiguous, B transposed)
//      2  dW2  = dy^T . a             (A and B transposed; k runs over the group's rows)
//      3  dW13 = [dp|dq]^T . x        (A and B transposed; x rows gathered)
//      4  p, q = x . [W1;W3]^T, then the SwiGLU backward in the epilogue:
//         reads da, writes dp, dq and a (A and B k-contiguous); fp32 layers
//         only: bf16 layers recompute p, q on the forward up kernel with its
//         backward epilogue (expert_ffn.hip)
//      bf16 operands come in through raw buffer loads whose offsets are fixed
//      per tile (a chunk out of range reads zeros), and the tile order is
//      XCD-aware (see the kernel)
//   gather_dx_kernel     dx_ffn[t] = dxs[t] + sum_k dxr[slot_of[t,k]] (k order)
//   router_dz_kernel     ds, dz per token (wave per token, lane = expert)
//   router_dx_kernel     dx = dh + dx_ffn + dz E (LDS-tiled, 64 tokens x 64 columns)
//   router_de_part/sum   dE, dbias partials over token chunks (x read once), then a fixed-order sum
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
    float *dxr, *dxs;                    // [T*K', d], [T, d]
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

// 128 x 128 tile (mode 4: 128 rows x 64 units, both halves of B), 32 k per
// step, 4 waves in 2 x 2, each 64 x 64 = 2 x 2 MFMA blocks of 32 x 32.
template <int MODE, typename DT>
__global__ __launch_bounds__(256, 4) void bgemm_kernel(BgArgs A) {
    constexpr bool BF = std::is_same<DT, uint16_t>::value;
    constexpr int ES = sizeof(DT);
    constexpr int EC = 16 / ES;                       // elements per 16-byte chunk
    constexpr bool AT = a_transposed(MODE), BT = b_transposed(MODE);
    // LDS pitches (bytes): k-contiguous tiles [128][32], transposed tiles [32][128]
    constexpr int PK = 32 * ES + 16;                  // 80 (bf16) / 144 (fp32): conflict-free fragment rows
    constexpr int PT = 128 * ES + (BF ? 64 : 128);    // 320 / 640: the four rows of a transposed read hit distinct banks
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
    // bf16 products: every chunk's byte offset is fixed per tile and a step
    // adds a uniform scalar offset (mode 3's B rows follow the gathered
    // tokens, loaded one step ahead); no address arithmetic, division or
    // branch per chunk in the k loop.  Column offsets within a chunk never
    // cross a segment or a [dp | dq] boundary: w % 64 == 0 and chunks are 8
    // elements.  dq follows dp in the same workspace, so one window with dq
    // at a positive byte offset covers both.
    constexpr bool BUF = BF && MODE <= 3;
    __amdgpu_buffer_rsrc_t rsA = bg_rsrc(A.x), rsB = rsA, rsB2 = rsA;
    uint32_t va[RA], vb[RB], sA = 0, sB = 0, dA = 0;
    int klA[RA], klB[RB], tkB[RB];
    if constexpr (BUF) {
        const size_t w = A.w, d = A.d, wg = Gr.wg, ro = Gr.roff;
        const DT *dy = (const DT *)(Gr.sh ? A.dh : A.dy_r);
        const DT *dp = (const DT *)(Gr.sh ? A.dp_s : A.dp_r), *dq = (const DT *)(Gr.sh ? A.dq_s : A.dq_r);
        const uint32_t dq_off = (uint32_t)((const char *)dq - (const char *)dp);
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const int c = tid + 256 * i;
            int m, kofs;
            if (AT) { kofs = c / (128 / EC); m = m0 + (c % (128 / EC)) * EC; }
            else { m = m0 + c / (32 / EC); kofs = (c % (32 / EC)) * EC; }
            size_t e = 0;
            if (MODE == 0) e = (ro + m) * d + kofs;
            if (MODE == 1) e = (ro + m) * wg + kofs;
            if (MODE == 2) e = (size_t)kofs * d + m;
            if (MODE == 3) e = (ro + kofs) * wg + (m < (int)wg ? m : m - (int)wg);
            uint32_t off = (uint32_t)(e * ES);
            if (MODE == 3 && m >= (int)wg) off += dq_off;
            va[i] = m < M ? off : kOob;
            klA[i] = K - kofs;   // the chunk is live while k0 < klA
        }
        if (MODE == 0) { rsA = bg_rsrc(dy); sA = 32 * ES; }
        if (MODE == 1) { rsA = bg_rsrc(dp); dA = dq_off; }
        if (MODE == 2) { rsA = bg_rsrc(dy + ro * d); sA = (uint32_t)(32 * d * ES); }
        if (MODE == 3) { rsA = bg_rsrc(dp); sA = (uint32_t)(32 * wg * ES); }

#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const int c = tid + 256 * i;
            const int kofs = c / (128 / EC), n = n0 + (c % (128 / EC)) * EC;   // B is transposed in modes 0-3
            size_t e = 0;
            if (MODE == 0) e = ((size_t)(n / A.w) * d + kofs) * w + n % A.w;
            if (MODE == 1) e = (size_t)kofs * d + n;
            if (MODE == 2) e = (size_t)kofs * wg + n;
            if (MODE == 3) e = (size_t)n;
            vb[i] = n < N ? (uint32_t)(e * ES) : kOob;
            klB[i] = K - kofs;
            tkB[i] = 0;
        }
        if (MODE == 0) {
            rsB = bg_rsrc(Gr.sh ? (const DT *)A.w2_s : (const DT *)A.w2_r + (size_t)Gr.r * d * w);
            sB = (uint32_t)(32 * w * ES);
        }
        if (MODE == 1) {
            rsB = bg_rsrc(Gr.sh ? (const DT *)A.w1_s : (const DT *)A.w1_r + (size_t)Gr.r * w * d);
            rsB2 = bg_rsrc(Gr.sh ? (const DT *)A.w3_s : (const DT *)A.w3_r + (size_t)Gr.r * w * d);
            sB = (uint32_t)(d * ES);   // per k row
        }
        if (MODE == 2) { rsB = bg_rsrc((const DT *)(Gr.sh ? A.a_s : A.a_r) + ro * wg); sB = (uint32_t)(32 * wg * ES); }
        if (MODE == 3) rsB = bg_rsrc(A.x);
    }
    // mode 3: token of k row k0 + kofs of chunk i (clamped into the group)
    auto tok_of = [&](int i, int k0) -> int {
        const int c = tid + 256 * i, k = min(k0 + c / (128 / EC), max(K - 1, 0));
        return Gr.sh ? k : A.sorted_token[Gr.roff + k];
    };
    auto load_buf = [&](int k0) {
        // A
        uint32_t so = 0;
        if (MODE == 1) so = k0 < Gr.wg ? (uint32_t)(k0 * ES) : dA + (uint32_t)((k0 - Gr.wg) * ES);
        else so = (uint32_t)(k0 / 32) * sA;
#pragma unroll
        for (int i = 0; i < RA; ++i) {
            const uint32_t v = (MODE >= 2 && k0 >= klA[i]) ? kOob : va[i];
            ra[i] = bg_load(rsA, v, so);
        }
        // B
        if (MODE == 3) {
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const uint32_t v = (k0 >= klB[i] || vb[i] == kOob) ? kOob : (uint32_t)(tkB[i] * A.d * ES) + vb[i];
                rb[i] = bg_load(rsB, v, 0);
            }
            // tokens of the next step's rows, a step ahead of their use
#pragma unroll
            for (int i = 0; i < RB; ++i) tkB[i] = tok_of(i, k0 + 32);
        } else {
            const bool w3 = MODE == 1 && k0 >= Gr.wg;
            const uint32_t sob = MODE == 1 ? (uint32_t)(w3 ? k0 - Gr.wg : k0) * sB : (uint32_t)(k0 / 32) * sB;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const uint32_t v = (MODE >= 2 && k0 >= klB[i]) ? kOob : vb[i];
                rb[i] = bg_load(w3 ? rsB2 : rsB, v, sob);
            }
        }
    };
    auto load_tiles = [&](int k0) {
      if constexpr (BUF) {
        load_buf(k0);
      } else {
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
    // fragment of a 32-row block at tile row r0 for the k16 (bf16) / k2 (fp32) sub-step s
    auto frag_bf = [&](const uint8_t *s, bool tr, int r0, int ks) -> bf16x8 {
        if (!tr) return *(const bf16x8 *)(s + (r0 + l32) * PK + (16 * ks + 8 * lhi) * 2);
        const int g = lane >> 4, j = lane & 15;
        const int col = r0 + 16 * (g & 1) + 4 * (j & 3);
        const int row = 16 * ks + 8 * (g >> 1) + (j >> 2);
        const v4s lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(s + row * PT + col * 2));
        const v4s hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(s + (row + 4) * PT + col * 2));
        // whole-vector shuffle and bit cast (element-wise assembly of the
        // fragment was miscompiled: the second dword of each read was lost)
        const v8s both = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, both);
    };
    auto frag_f32 = [&](const uint8_t *s, bool tr, int r0, int ks) -> float {
        const int k = 2 * ks + lhi;
        return tr ? *(const float *)(s + k * PT + (r0 + l32) * 4) : *(const float *)(s + (r0 + l32) * PK + k * 4);
    };
    auto compute = [&](int stg) {
        const uint8_t *s_a = s_a2[stg], *s_b = s_b2[stg];
        if constexpr (BF) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 fa[2], fb[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    fa[b] = frag_bf(s_a, AT, wm * 64 + b * 32, ks);
                    fb[b] = frag_bf(s_b, BT, wn * 64 + b * 32, ks);
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mb], fb[nb], acc[mb][nb], 0, 0, 0);
            }
        } else {
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
    if (MODE == 3 && BUF && nk > 0) {
#pragma unroll
        for (int i = 0; i < RB; ++i) tkB[i] = tok_of(i, 0);
    }
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
                        float *o = Gr.sh ? A.dxs : A.dxr;
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

// dx_ffn[t] = dxs[t] (shared experts, or 0) + sum_k dxr[slot_of[t,k]], k in order.
__global__ __launch_bounds__(256) void gather_dx_kernel(int T, int d, int K, const float *__restrict__ dxs,
                                                        const float *__restrict__ dxr,
                                                        const int32_t *__restrict__ slot_of,
                                                        float *__restrict__ dx) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // one float4 of one token
    const int q = d / 4;
    if (i >= (int64_t)T * q) return;
    const int t = (int)(i / q), c = (int)(i % q) * 4;
    float4 acc = dxs ? *(const float4 *)(dxs + (size_t)t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
        const int slot = slot_of[(size_t)t * K + k];
        if (slot < 0) continue;
        const float4 v = *(const float4 *)(dxr + (size_t)slot * d + c);
        acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    *(float4 *)(dx + (size_t)t * d + c) = acc;
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

// dx = dh + dx_ffn + dz E.  Workgroup tile: 64 tokens x 64 columns, thread
// (token group tg, column group cg) owns 4 tokens x 4 columns; dz rows of the
// tile and E columns of the tile are staged in LDS; the sum over r runs in
// ascending order.
template <typename DT, int NJ>
__global__ __launch_bounds__(256) void router_dx_kernel(int T, int d, int Nr, const DT *__restrict__ dh,
                                                        const float *__restrict__ dx_ffn,
                                                        const float *__restrict__ dz, const float *__restrict__ E,
                                                        float *__restrict__ dx) {
    constexpr int NE = 64 * NJ;
    __shared__ float s_dz[64][NE + 1];
    __shared__ __attribute__((aligned(16))) float s_e[NE][64];
    const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    for (int i = tid; i < 64 * NE; i += 256) {
        const int tt = i / NE, r = i % NE;
        s_dz[tt][r] = (t0 + tt < T && r < Nr) ? dz[(size_t)(t0 + tt) * Nr + r] : 0.0f;
    }
    for (int i = tid; i < NE * 16; i += 256) {
        const int r = i / 16, c4 = (i % 16) * 4;
        *(float4 *)&s_e[r][c4] = (r < Nr && c0 + c4 < d) ? *(const float4 *)(E + (size_t)r * d + c0 + c4)
                                                        : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    const int cg = tid & 15, tg = tid >> 4;
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
    for (int r = 0; r < Nr; ++r) {
        const float4 e4 = *(const float4 *)&s_e[r][cg * 4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float z = s_dz[tg * 4 + i][r];
            acc[i][0] = __builtin_fmaf(z, e4.x, acc[i][0]);
            acc[i][1] = __builtin_fmaf(z, e4.y, acc[i][1]);
            acc[i][2] = __builtin_fmaf(z, e4.z, acc[i][2]);
            acc[i][3] = __builtin_fmaf(z, e4.w, acc[i][3]);
        }
    }
    const int c = c0 + cg * 4;
    if (c >= d) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = t0 + tg * 4 + i;
        if (t >= T) continue;
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = to_f(dh[(size_t)t * d + c + j]) + (dx_ffn ? dx_ffn[(size_t)t * d + c + j] : 0.0f) + acc[i][j];
        *(float4 *)(dx + (size_t)t * d + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// dE partials over token chunks of kDeTokens: workgroup (chunk j, 64
// columns); thread (column col, expert group eg) accumulates, t ascending,
// dz[t, r] x[t, c] for its 16 NJ consecutive experts r = eg * 16 NJ + i,
// reading each x value once; dz of the chunk is staged in LDS, read as
// 16-byte broadcasts (a wave shares eg).  part[j][r][c], row pitch d + 4;
// column d carries sum_t dz (the bias gradient).
constexpr int kDeTokens = 128;
template <typename DT, int NJ>
__global__ __launch_bounds__(256) void router_de_part_kernel(int T, int d, int Nr, const DT *__restrict__ x,
                                                             const float *__restrict__ dz,
                                                             float *__restrict__ part) {
    constexpr int NE = 64 * NJ, PER = 16 * NJ;
    __shared__ __attribute__((aligned(16))) float s_dz[kDeTokens][NE];
    const int j = blockIdx.x, c0 = blockIdx.y * 64;
    const int tid = threadIdx.x, col = tid & 63, eg = tid >> 6;
    const int c = c0 + col;
    const int t0 = j * kDeTokens, n = min(kDeTokens, T - t0);
    for (int i = tid; i < kDeTokens * NE; i += 256) {
        const int tt = i / NE, r = i % NE;
        s_dz[tt][r] = (tt < n && r < Nr) ? dz[(size_t)(t0 + tt) * Nr + r] : 0.0f;
    }
    __syncthreads();
    float acc[PER];
    float bsum[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) { acc[i] = 0.0f; bsum[i] = 0.0f; }
    for (int tt = 0; tt < n; ++tt) {
        const float xv = to_f(x[(size_t)(t0 + tt) * d + c]);
#pragma unroll
        for (int i = 0; i < PER; i += 4) {
            const float4 z = *(const float4 *)&s_dz[tt][eg * PER + i];
            acc[i] = __builtin_fmaf(z.x, xv, acc[i]);
            acc[i + 1] = __builtin_fmaf(z.y, xv, acc[i + 1]);
            acc[i + 2] = __builtin_fmaf(z.z, xv, acc[i + 2]);
            acc[i + 3] = __builtin_fmaf(z.w, xv, acc[i + 3]);
            bsum[i] += z.x; bsum[i + 1] += z.y; bsum[i + 2] += z.z; bsum[i + 3] += z.w;
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int r = eg * PER + i;
        if (r >= Nr) continue;
        float *o = part + ((size_t)j * Nr + r) * (d + 4);
        o[c] = acc[i];
        if (blockIdx.y == 0 && col == 0) o[d] = bsum[i];
    }
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

template <int MODE, typename DT>
hipError_t launch_bg(const BgArgs &a, int tiles, hipStream_t s) {
    if (tiles <= 0) return hipSuccess;
    bgemm_kernel<MODE, DT><<<tiles, 256, 0, s>>>(a);
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
        if ((e = launch_bg<0, uint16_t>(a, t0, s)) != hipSuccess) return e;
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
        if ((e = launch_bg<1, uint16_t>(a, t1, s)) != hipSuccess) return e;
        if ((e = launch_bg<2, uint16_t>(a, t2, s)) != hipSuccess) return e;
        if ((e = launch_bg<3, uint16_t>(a, t3, s)) != hipSuccess) return e;
    } else {
        if ((e = launch_bg<0, float>(a, t0, s)) != hipSuccess) return e;
        if ((e = launch_bg<4, float>(a, t4, s)) != hipSuccess) return e;
        if ((e = launch_bg<1, float>(a, t1, s)) != hipSuccess) return e;
        if ((e = launch_bg<2, float>(a, t2, s)) != hipSuccess) return e;
        if ((e = launch_bg<3, float>(a, t3, s)) != hipSuccess) return e;
    }
    if (p.T > 0) {
        const int64_t n = (int64_t)p.T * (p.d / 4);
        gather_dx_kernel<<<(int)((n + 255) / 256), 256, 0, s>>>(p.T, p.d, p.top_k, p.n_shared > 0 ? b.dxs : nullptr,
                                                                 b.dxr, b.slot_of, b.dx_ffn);
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
        const dim3 gx(cdiv(p.T, 64), cdiv(p.d, 64));
        const int nj = cdiv(p.n_routed, 64);
#define MOE_DX(DT, NJ) router_dx_kernel<DT, NJ><<<gx, 256, 0, s>>>(p.T, p.d, p.n_routed, (const DT *)dh, dx_ffn, \
                                                                   dz, centroids, dx)
        if (p.dtype == MOE_BF16) {
            if (nj == 1) MOE_DX(uint16_t, 1); else if (nj == 2) MOE_DX(uint16_t, 2); else MOE_DX(uint16_t, 4);
        } else {
            if (nj == 1) MOE_DX(float, 1); else if (nj == 2) MOE_DX(float, 2); else MOE_DX(float, 4);
        }
#undef MOE_DX
    }
    const int nchunk = cdiv(p.T, kDeTokens);
    if (nchunk > 0) {
        const dim3 g(nchunk, cdiv(p.d, 64));
        const int nj = cdiv(p.n_routed, 64);
#define MOE_DE(DT, NJ) router_de_part_kernel<DT, NJ><<<g, 256, 0, s>>>(p.T, p.d, p.n_routed, (const DT *)x, dz, part)
        if (p.dtype == MOE_BF16) {
            if (nj == 1) MOE_DE(uint16_t, 1); else if (nj == 2) MOE_DE(uint16_t, 2); else MOE_DE(uint16_t, 4);
        } else {
            if (nj == 1) MOE_DE(float, 1); else if (nj == 2) MOE_DE(float, 2); else MOE_DE(float, 4);
        }
#undef MOE_DE
    }
    const int64_t m = (int64_t)p.n_routed * (p.d + 1);
    router_de_sum_kernel<<<(int)((m + 255) / 256), 256, 0, s>>>(nchunk, p.d, p.n_routed, part, dcentroids, dbias);
    return hipGetLastError();
}

int route_backward_chunks(int T) { return cdiv(T, kDeTokens); }

}  // namespace moe
