// expert_ffn.hip -- the expert FFNs of the DeepSeekMoE layer on gfx950 MFMA.
//
// "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化", section "Two core
// strategies": mN fine-grained experts whose intermediate width is 1/m of a
// standard FFN, and K_s shared experts that every token uses.  Each expert is
// a SwiGLU FFN (no biases): FFN(u) = W2 (SiLU(W1 u) * (W3 u)).
//
// Two grouped GEMM launches:
//   up   : for every group, act = SiLU(X W1^T) * (X W3^T), the SwiGLU fused into
//          the epilogue (W1 and W3 rows of the same unit sit in one tile);
//   down : y = act W2^T, written per grouped row.
// Groups: the K_s shared experts form ONE dense group of width K_s*w over all
// T rows (their W1/W3 stacks [K_s, w, d] are already one [K_s*w, d] matrix;
// W2 is read segment by segment), then one group per routed expert whose rows
// are its tokens in grouped order (gathered through sorted_token in the up
// GEMM, contiguous in the down GEMM).
//
// Tiles: 128 weight rows x 128 tokens x 128 bytes of K per step, 256 threads
// (4 wave64, 2x2), each wave 64x64 = 2x2 MFMA 32x32 blocks.  The MFMA A
// operand is the weight tile, B the token tile, so each lane owns one token
// column and 4 consecutive output columns per register quad (8/16-byte
// stores).  bf16 uses v_mfma_f32_32x32x16_bf16; fp32 uses 8 x
// v_mfma_f32_32x32x2_f32 per 16-wide k step over the same LDS fragments.
// Every workgroup derives its (group, row-tile, column-tile) from the
// device-side offsets, so no host round trip sizes the grid: the grid is an
// upper bound and surplus workgroups exit at once.
#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int BM = 128;        // tokens per tile
constexpr int BN = 128;        // weight rows per tile
constexpr int KB = 128;        // bytes of K per tile step (64 bf16 / 32 fp32)
constexpr int PITCH = KB + 16; // padded LDS row pitch (bytes)
constexpr int MAXG = 1 + kPermuteMaxExperts;

template <typename DT> struct Elt;
template <> struct Elt<float> { static constexpr int size = 4; };

__device__ __forceinline__ uint16_t f2bf(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ void store4(uint16_t *dst, const float v[4]) {
    uint2 q;
    q.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    q.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *(uint2 *)dst = q;
}
__device__ __forceinline__ void store4(float *dst, const float v[4]) {
    *(float4 *)dst = make_float4(v[0], v[1], v[2], v[3]);
}

// One 16-wide k step of a 32x32 block: a = weight fragment, b = token fragment.
__device__ __forceinline__ void mfma_k16(f32x16 &acc, const uint8_t *a, const uint8_t *b, uint16_t) {
    const bf16x8 av = *(const bf16x8 *)a;
    const bf16x8 bv = *(const bf16x8 *)b;
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_k16(f32x16 &acc, const uint8_t *a, const uint8_t *b, float) {
    const float4 a0 = *(const float4 *)a, a1 = *(const float4 *)(a + 16);
    const float4 b0 = *(const float4 *)b, b1 = *(const float4 *)(b + 16);
    const float av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
    const float bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av[j], bv[j], acc, 0, 0, 0);
}

struct GemmParams {
    int T, d, Ks, Nr, w;
    int TK;                      // T*K': rows of the routed grouped arrays
    const int32_t *offsets;
    const int32_t *sorted_token;
    const uint8_t *x;            // up: [T, d]
    const uint8_t *act_shared;   // down: [T, Ks*w]
    const uint8_t *act_routed;   // down: [T*K', w]
    const uint8_t *wa_r, *wb_r;  // up: W1_r, W3_r  | down: W2_r
    const uint8_t *wa_s, *wb_s;  // up: W1_s, W3_s  | down: W2_s
    uint8_t *out_shared;         // up: act_shared  | down: y_shared (fp32)
    uint8_t *out_routed;         // up: act_routed  | down: y_routed
    // backward recompute of the up projection (BWD): da in, dp and dq out
    // (act_* above take the recomputed activations a)
    const uint8_t *da_shared, *da_routed;
    uint8_t *dp_shared, *dp_routed, *dq_shared, *dq_routed;
    // accumulating down projection: y_acc[t] += gate * y for every grouped row
    // of token t (gate_sorted in grouped order), y_acc[t] += y for the shared rows
    const float *gate_sorted;
    float *y_acc;
};

// fp32 add into y, performed in memory (no return value): the hardware float
// atomic, coherent across the XCDs' L2s (agent scope); the order of the adds
// into one element is not fixed
__device__ __forceinline__ void acc_add(float *dst, float v) { unsafeAtomicAdd(dst, v); }

// UP: true for the gate/up projection with SwiGLU epilogue, false for the down projection.
template <typename DT, bool UP>
__global__ __launch_bounds__(256) void grouped_ffn_kernel(GemmParams P) {
    constexpr int ES = Elt<DT>::size;
    constexpr int KSTEP = 16 * ES;          // bytes of one 16-wide k step
    __shared__ int s_pref[MAXG + 1];
    __shared__ int s_src[BM];
    __shared__ __attribute__((aligned(16))) uint8_t s_w[BN * PITCH];
    __shared__ __attribute__((aligned(16))) uint8_t s_x[BM * PITCH];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (P.Ks > 0 ? 1 : 0) + P.Nr;
    const int ntn_s = UP ? P.Ks * P.w / 64 : cdiv(P.d, BN);
    const int ntn_r = UP ? P.w / 64 : cdiv(P.d, BN);

    // ---- tile prefix over groups (wave 0), then locate this workgroup's tile ----
    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_pref[0] = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            int tiles = 0;
            if (g < G) {
                const bool sh = P.Ks > 0 && g == 0;
                const int r = g - (P.Ks > 0 ? 1 : 0);
                const int rows = sh ? P.T : P.offsets[r + 1] - P.offsets[r];
                tiles = cdiv(rows, BM) * (sh ? ntn_s : ntn_r);
            }
            int incl = tiles;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            if (g < G) s_pref[g + 1] = carry + incl;
            carry += __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    const int bid = blockIdx.x;
    if (bid >= s_pref[G]) return;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= bid) lo = mid; else hi = mid;
    }
    const int g = lo;
    const bool shared = P.Ks > 0 && g == 0;
    const int r = g - (P.Ks > 0 ? 1 : 0);
    const int row_off = shared ? 0 : P.offsets[r];
    const int rows = shared ? P.T : P.offsets[r + 1] - row_off;
    const int mt = cdiv(rows, BM);
    const int lt = bid - s_pref[g];
    const int m_tile = lt % mt, n_tile = lt / mt;
    const int m0 = m_tile * BM;

    // K extent and operand geometry of this group
    const int K = UP ? P.d : (shared ? P.Ks * P.w : P.w);
    const size_t a_pitch = (size_t)K * ES;               // token-side row pitch (bytes)
    const uint8_t *a_base;
    if (UP) a_base = P.x;
    else a_base = shared ? P.act_shared : P.act_routed;
    if (tid < BM) {
        const int row = m0 + tid;
        int src = -1;
        if (row < rows) {
            if (UP) src = shared ? row : P.sorted_token[row_off + row];
            else src = row_off + row;
        }
        s_src[tid] = src;
    }
    __syncthreads();

    // weight-side rows handled by this thread's 4 load chunks
    const uint8_t *wsrc[4];
    bool wvalid[4];
    int wrow[4];
    const uint8_t *xsrc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + 256 * i;
        const int row = c >> 3, part = c & 7;
        wrow[i] = row;
        if (UP) {
            const uint8_t *base = (row < 64) ? (shared ? P.wa_s : P.wa_r + (size_t)r * P.w * P.d * ES)
                                             : (shared ? P.wb_s : P.wb_r + (size_t)r * P.w * P.d * ES);
            const int wr = n_tile * 64 + (row & 63);
            wsrc[i] = base + (size_t)wr * P.d * ES + part * 16;
            wvalid[i] = true;
        } else {
            const int col = n_tile * BN + row;
            wvalid[i] = col < P.d;
            // W2 row `col` of expert r (routed) or of shared segment 0 (advanced per k tile)
            const uint8_t *base = shared ? P.wa_s : P.wa_r + (size_t)r * P.d * P.w * ES;
            wsrc[i] = base + (size_t)(wvalid[i] ? col : 0) * P.w * ES + part * 16;
        }
        const int src = s_src[row];
        xsrc[i] = src >= 0 ? a_base + (size_t)src * a_pitch + part * 16 : nullptr;
    }

    uint4 rw[4], rx[4];
    auto load_tile = [&](int kt) {
        const size_t kbyte = (size_t)kt * KB;
        size_t wk = kbyte;
        if (!UP && shared) {
            // shared down projection: k runs over K_s segments of width w
            const int k_el = kt * (KB / ES);
            const int seg = k_el / P.w;
            wk = ((size_t)seg * P.d * P.w + (k_el - seg * P.w)) * ES;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            rw[i] = wvalid[i] ? *(const uint4 *)(wsrc[i] + wk) : make_uint4(0, 0, 0, 0);
            rx[i] = xsrc[i] ? *(const uint4 *)(xsrc[i] + kbyte) : make_uint4(0, 0, 0, 0);
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    // LDS byte offsets of this lane's fragments (k step 0)
    int wfrag[2], xfrag[2];
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int wr = UP ? (ni * 64 + wn * 32 + l32) : (wn * 64 + ni * 32 + l32);
        wfrag[ni] = wr * PITCH + lhi * (8 * ES);
    }
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) xfrag[mi] = (wm * 64 + mi * 32 + l32) * PITCH + lhi * (8 * ES);

    const int nk = K * ES / KB;
    load_tile(0);
    for (int kt = 0; kt < nk; ++kt) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + 256 * i;
            const int off = (c >> 3) * PITCH + (c & 7) * 16;
            *(uint4 *)(s_w + off) = rw[i];
            *(uint4 *)(s_x + off) = rx[i];
        }
        __syncthreads();
        if (kt + 1 < nk) load_tile(kt + 1);
#pragma unroll
        for (int ks = 0; ks < KB / KSTEP; ++ks) {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    mfma_k16(acc[ni][mi], s_w + wfrag[ni] + ks * KSTEP, s_x + xfrag[mi] + ks * KSTEP, DT{});
        }
    }

    // ---- epilogue: lane owns token column l32; register quad q holds 4 consecutive
    //      weight rows 8q + 4*lhi + {0..3} of each 32x32 block ----
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
        const int row = m0 + wm * 64 + mi * 32 + l32;
        if (row >= rows) continue;
        if (UP) {
            const int ld = shared ? P.Ks * P.w : P.w;
            DT *dst = (DT *)(shared ? P.out_shared : P.out_routed) + (size_t)(row_off + row) * ld;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p = acc[0][mi][4 * q + e];
                    const float u = acc[1][mi][4 * q + e];
                    v[e] = p / (1.0f + __expf(-p)) * u;
                }
                store4(dst + n_tile * 64 + wn * 32 + 8 * q + 4 * lhi, v);
            }
        } else {
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n_tile * BN + wn * 64 + ni * 32 + 8 * q + 4 * lhi;
                    if (col >= P.d) continue;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[ni][mi][4 * q + e];
                    if (P.y_acc) {
                        // accumulating mode: y_acc[t] += gate * y (gate 1 for the shared rows)
                        const int t = shared ? row : P.sorted_token[row_off + row];
                        const float g = shared ? 1.0f : P.gate_sorted[row_off + row];
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc_add(P.y_acc + (size_t)t * P.d + col + e, g * v[e]);
                    } else if (shared) {
                        store4((float *)P.out_shared + (size_t)row * P.d + col, v);
                    } else {
                        store4((DT *)P.out_routed + (size_t)(row_off + row) * P.d + col, v);
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 path: 256 weight rows x BM tokens per tile, 64 k per step.
//
// LDS rows are 128 bytes (64 bf16) with no padding; the 16-byte chunk c of
// row r lives at chunk c ^ (r & 7) ^ ((r >> 3) & 1), so the 32 rows a fragment
// read touches spread over all banks.  Two LDS stages, filled by direct-to-LDS
// buffer loads (no registers, no LDS store instructions; on a 64 KB-per-step
// loop the LDS stores cost about a tenth of the MFMA rate, and their power
// the shader clock): a step reads all its weight fragments first, so its
// stage's weight rows are refilled with the step after next from the
// barrier after its first MFMA group, and its token rows from the barrier
// before its last group.  Per-thread 32-bit row offsets are fixed for the
// whole k loop and the k position is a scalar offset; rows outside the group
// read as zero (range-checked loads), so no masking is needed.
// 8 waves (2 per SIMD, so one wave's LDS and memory latency hides behind
// the other's MFMAs), laid out 2 (tokens) x 4 (weights): a wave owns 64
// weight rows (2 blocks of 32) x BM/2 tokens (BM/64 blocks of 32).  In the
// up projection the wave's two weight blocks are the W1 rows and the W3 rows
// of the same 32 intermediate units, so the SwiGLU pairs up in registers.
// ---------------------------------------------------------------------------
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
constexpr uint32_t kOOB = 0x80000000u;   // offset beyond any buffer: reads as zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
// Cache policy of the stores that carry data between workgroups of one
// launch: sc1, the agent-coherent form (what the compiler emits for relaxed
// agent-scope atomic stores), written through to memory so that every XCD
// sees it.  The reads of that data are ordinary cached loads: a reading XCD's
// L2 cannot hold an older copy of those lines (the kernel launch starts with
// the L2s invalidated, and within the launch the lines are read only after
// they are written), so the first read on an XCD fetches the written data
// and the later ones hit in that L2.
constexpr int kCoherent = 16;
constexpr int kNonTemporal = 2;   // nt: a streaming access
template <int AUX = 0>
__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Direct-to-LDS load of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane L
// writes LDS bytes [lds_base + 16 L, +16); lanes whose offset lies past the
// descriptor's size write zeros.  The descriptor is four dwords in SGPRs (the
// layout __builtin_amdgcn_make_buffer_rsrc builds).  Issued from inline asm: the
// compiler does not track these loads, which keeps it from making later LDS
// reads of the other stage wait for them (it cannot tell the stages apart); the
// caller orders them with s_waitcnt vmcnt and barriers, and any wait the
// compiler places for its own loads only counts more loads than it knows of.
// The s_nop covers the hazard between the write of M0 and its read by the load.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_rsrc4(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    i32x4 r;
    r.x = (int)(uint32_t)a;
    r.y = (int)((uint32_t)(a >> 32) & 0xffffu);
    r.z = (int)bytes;
    r.w = 0x00020000;
    return r;
}
template <int AUX>
__device__ __forceinline__ void dma16(i32x4 r, uint32_t lds_base, uint32_t voff, uint32_t soff) {
    static_assert(AUX == 0 || AUX == kNonTemporal, "cache policy of a direct-to-LDS load");
    if constexpr (AUX == kNonTemporal)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                     :
                     : "{m0}"(lds_base), "v"(voff), "s"(r), "s"(soff)
                     : "memory");
    else
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                     :
                     : "{m0}"(lds_base), "v"(voff), "s"(r), "s"(soff)
                     : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}
template <int AUX = 0>
__device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint4 v) {
    v4u w;
    w.x = v.x; w.y = v.y; w.z = v.z; w.w = v.w;
    __builtin_amdgcn_raw_buffer_store_b128(w, r, voff, 0, AUX);
}

// One tile of the bf16 grouped GEMM: rows [m0, m0+nr) of a group (the
// shared experts, or routed expert r) against weight tile n_tile.  FUSED:
// the tile runs inside the fused up+down launch, whose activations pass
// between workgroups through agent-coherent stores (read back as cached loads).
struct TileDesc {
    bool shared;
    int r, row_off, m0, nr, n_tile;
};

// WAUX: cache policy of the weight loads (0, or kNonTemporal for decode-sized batches, where
// the routed experts average at most 64 rows and the shared group, if any, is one token tile:
// most experts' weights are then read by a single tile; a skewed expert with more than one
// tile re-reads them from memory).  ACC (down projection only): instead of writing y per grouped
// row, add gate * y into the fp32 rows of y_acc of the rows' tokens.
template <int BM, bool UP, bool BWD, bool FUSED, int WAUX = 0, bool ACC = false>
__device__ __forceinline__ void ffn_tile_bf16(const GemmParams &P, const TileDesc td, uint8_t (&s_w)[2][256 * 128],
                                              uint8_t (&s_x)[2][BM * 128], int (&s_src)[BM],
                                              int *head = nullptr, int *next = nullptr) {
    static_assert(!BWD || UP, "the backward epilogue belongs to the up projection");
    static_assert(!ACC || !UP, "only the down projection accumulates");
    constexpr int NT = 512;          // threads: 8 waves, 2 per SIMD
    constexpr int BN = 256;          // weight rows per tile
    constexpr int RB = 128;          // LDS row bytes
    constexpr int MB = BM / 64;      // 32-token blocks per wave
    constexpr int NB = 2;            // 32-row weight blocks per wave
    constexpr int CW = BN * 8 / NT;  // weight chunks per thread (4)
    constexpr int CX = BM * 8 / NT;  // token chunks per thread (4 or 2)
    int tid_ = threadIdx.x;
    // in the persistent launch, keep the lane-dependent offsets inside the tile:
    // hoisted out of the tile loop they would stay live across both projections
    // and spill (the empty asm is opaque to loop-invariant code motion)
    if constexpr (FUSED) asm volatile("" : "+v"(tid_));
    const int tid = tid_, lane = tid & 63, wave = tid >> 6;
    const bool shared = td.shared;
    const int r = td.r, row_off = td.row_off, m0 = td.m0, nr = td.nr, n_tile = td.n_tile;

    const int K = UP ? P.d : (shared ? P.Ks * P.w : P.w);
    const uint32_t xpitch = (uint32_t)K * 2u;   // token-side row bytes
    // ---- buffer resources and fixed per-thread offsets ----
    const int part = tid & 7;               // physical 16-byte chunk of the row in LDS
    const int rsub = tid >> 3;              // row within a group of 64
    // Logical chunk c of row r sits at physical chunk c ^ (r & 7) ^ ((r >> 3) & 1)
    // (an involution): any 8 consecutive rows, and any 16 consecutive rows split by
    // parity, land on distinct 16-byte bank groups.  The stages are filled by
    // direct-to-LDS loads, lane L of a wave writing the L-th 16 bytes after the
    // wave's base, so the lane at physical chunk `part` fetches logical chunk swz.
    const int swz = part ^ (rsub & 7) ^ ((rsub >> 3) & 1);
    i32x4 rw_a, rw_b, rx;
    uint32_t ow[CW], ox[CX];
    int n_valid;                            // weight-side rows of this group
    uint32_t wpitch;
    if (UP) {
        const size_t ebytes = (size_t)P.w * P.d * 2;
        const uint8_t *b1 = shared ? P.wa_s : P.wa_r + (size_t)r * ebytes;
        const uint8_t *b3 = shared ? P.wb_s : P.wb_r + (size_t)r * ebytes;
        n_valid = shared ? P.Ks * P.w : P.w;
        wpitch = (uint32_t)P.d * 2u;
        rw_a = make_rsrc4(b1, (uint32_t)((size_t)n_valid * wpitch));
        rw_b = make_rsrc4(b3, (uint32_t)((size_t)n_valid * wpitch));
        rx = make_rsrc4(P.x, (uint32_t)((size_t)P.T * P.d * 2));
    } else {
        const size_t ebytes = (size_t)P.d * P.w * 2;
        const uint8_t *b2 = shared ? P.wa_s : P.wa_r + (size_t)r * ebytes;
        n_valid = P.d;
        wpitch = (uint32_t)P.w * 2u;
        rw_a = make_rsrc4(b2, (uint32_t)(shared ? (size_t)P.Ks * ebytes : ebytes));
        rw_b = rw_a;
        const uint8_t *xb = shared ? P.act_shared : P.act_routed;
        // the routed activations' region holds T*K' rows (a bound known without a
        // load: read from memory, the descriptor was built from a vector register,
        // every buffer load got a waterfall loop, and the k loop's first wait covered
        // that load's register)
        const size_t xrows = shared ? (size_t)P.T : (size_t)P.TK;
        rx = make_rsrc4(xb, (uint32_t)(xrows * xpitch));
    }
#pragma unroll
    for (int i = 0; i < CW; ++i) {
        const int j = rsub + 64 * i;                     // tile row 0..255
        int wr;
        if (UP) wr = n_tile * 128 + (j & 127);           // W1 (j < 128) or W3 row
        else wr = n_tile * BN + j;                       // W2 row = output column
        ow[i] = wr < n_valid ? (uint32_t)wr * wpitch + swz * 16 : kOOB;
    }
    // Byte offsets of k step kt in the weight rows and the token rows.  In the
    // down projection of the shared experts, k runs over the K_s segments
    // [d, w] of the stacked W2, w/64 steps per segment.  The k loop advances
    // them by one step at a time (a scalar add, and a segment jump every w/64
    // steps); a division per step, if-converted by the compiler into every
    // down tile, cost the down k loop about 80 scalar instructions per step
    // and wave on the CU's one scalar unit.
    const bool segd = !UP && shared;
    const int spw = P.w / 64;
    const uint32_t sstr = (uint32_t)((size_t)P.d * P.w * 2);
    struct KOff {
        uint32_t kw, kx, kseg;
        int kin;
    };
    auto koff = [&](int kt) -> KOff {
        KOff o;
        o.kx = (uint32_t)kt * RB;
        if (segd) {
            o.kseg = (uint32_t)(kt / spw) * sstr;
            o.kin = kt % spw;
            o.kw = o.kseg + (uint32_t)o.kin * RB;
        } else {
            o.kseg = 0;
            o.kin = 0;
            o.kw = o.kx;
        }
        return o;
    };
    auto kadvance = [&](KOff &o) {
        o.kx += RB;
        if (segd) {
            if (++o.kin == spw) {
                o.kin = 0;
                o.kseg += sstr;
            }
            o.kw = o.kseg + (uint32_t)o.kin * RB;
        } else {
            o.kw = o.kx;
        }
    };
    // The loads of k step o into stage stg, straight into LDS: instruction i of
    // wave wv fills tile rows 64 i + 8 wv .. +7, 1 KB contiguous from the wave's
    // base.  Rows past the operand (offset kOOB) are filled with zeros.  They
    // count on vmcnt like any load: a wave waits for its own with s_waitcnt
    // vmcnt, and a barrier after that wait publishes them to the others.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    auto dma = [&](const KOff &o, int stg, bool wts, bool toks) {
        if (wts) {
#pragma unroll
            for (int i = 0; i < CW; ++i)
                dma16<WAUX>((UP && i >= CW / 2) ? rw_b : rw_a, lds_addr(s_w[stg] + (64 * i + 8 * wv) * RB), ow[i], o.kw);
        }
        if (toks) {
#pragma unroll
            for (int i = 0; i < CX; ++i) dma16<0>(rx, lds_addr(s_x[stg] + (64 * i + 8 * wv) * RB), ox[i], o.kx);
        }
    };
    // Barrier that waits for this wave's LDS accesses and its direct-to-LDS loads
    // except the newest VM of them (an immediate), not for more: __syncthreads'
    // fence would wait for every outstanding load.  The empty asm statements keep
    // the compiler from moving LDS accesses across it.
    auto lds_sync = [&](auto vm_t) {
        constexpr int VM = decltype(vm_t)::value;
        static_assert(VM < 16, "vmcnt immediate");
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(0x0070 | VM);   // vmcnt(VM) expcnt(7) lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };

    f32x16 acc[NB][MB];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < MB; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

    const int wm = wave & 1, wn = wave >> 1;
    const int l32 = lane & 31, lhi = lane >> 5;
    int wrow[NB], xrow[MB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        wrow[nb] = UP ? (nb * 128 + wn * 32 + l32) : (wn * 64 + nb * 32 + l32);
    // token block j (tile rows 32j..32j+31) belongs to wave row j & 1 as its
    // block j >> 1, so the live blocks of a short tile split evenly
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) xrow[mb] = (2 * mb + wm) * 32 + l32;
    const int nblk = cdiv(nr, 32);
    // live token blocks of this wave (the same in all its lanes)
    const int ml = __builtin_amdgcn_readfirstlane(min(MB, (nblk - wm + 1) >> 1));
    const int lsw = (l32 & 7) ^ ((l32 >> 3) & 1);   // swizzle of every fragment row of this lane

    // ML (below): live token blocks of the wave, a compile-time count so that
    // the k loop stays straight-line code
    auto mma = [&](auto ml_t, const bf16x8 (&fa)[NB], const bf16x8 (&fb)[MB]) {
        constexpr int ML = decltype(ml_t)::value;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < ML; ++mb)
                acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[nb], fb[mb], acc[nb][mb], 0, 0, 0);
    };

    using yes = std::true_type;
    using no = std::false_type;
    const int nk = K / 64;
    {
        // The weight rows of step 0 depend on the tile alone: their loads go out
        // before the token sources are gathered (for the up projection a dependent
        // global read), so the two latencies overlap.
        const KOff k0 = koff(0);
        dma(k0, 0, true, false);
        if (tid < BM) {
            const int row = m0 + tid;
            int src = -1;
            if (tid < nr) {
                if (UP) src = shared ? row : P.sorted_token[row_off + row];
                else src = row_off + row;
            }
            s_src[tid] = src;
        }
        lds_sync(std::integral_constant<int, 15>{});   // s_src written; the weight loads stay in flight
#pragma unroll
        for (int i = 0; i < CX; ++i) {
            const int src = s_src[rsub + 64 * i];
            ox[i] = src >= 0 ? (uint32_t)src * xpitch + swz * 16 : kOOB;
        }
        dma(k0, 0, false, true);
        // step 1 into stage 1; then stage 0 complete (step 1's loads, issued after
        // it, may stay in flight: vmcnt counts down in issue order)
        if (nk > 1) {
            dma(koff(1), 1, true, true);
            lds_sync(std::integral_constant<int, CW + CX>{});
        } else {
            lds_sync(std::integral_constant<int, 0>{});
        }
        // MORE: step kt+1 exists (wait for its stage), MORE2: step kt+2 exists (load it)
        auto kloop = [&](auto ml_t) {
            constexpr int ML = decltype(ml_t)::value;
            // Stage kt&1 holds step kt; step kt+1's loads into the other stage are in
            // flight.  A step reads all four of its weight fragments up front; the
            // barrier after its first group of MFMAs then frees the stage's weight
            // rows, and step kt+2's weight loads go out there, two steps ahead of
            // their use.  The barrier before the step's last group (its fragments are
            // in registers by then) waits for step kt+1, frees the token rows (step
            // kt+2's token loads go out), and the next step's first fragments are
            // read under that last group.
            KOff kn = koff(2);   // the step whose loads go out next (kt + 2 in the loop)
            bf16x8 fw[4][NB], fx0[MB], fx1[MB];
            auto wfr = [&](int stg, int ks, bf16x8 (&fa)[NB]) {
                if (ML > 0) {
                    const int ch = ((2 * ks + lhi) ^ lsw) * 16;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) fa[nb] = *(const bf16x8 *)(s_w[stg] + wrow[nb] * RB + ch);
                }
            };
            auto xfr = [&](int stg, int ks, bf16x8 (&fb)[MB]) {
                const int ch = ((2 * ks + lhi) ^ lsw) * 16;
#pragma unroll
                for (int mb = 0; mb < ML; ++mb) fb[mb] = *(const bf16x8 *)(s_x[stg] + xrow[mb] * RB + ch);
            };
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) wfr(0, ks, fw[ks]);
            xfr(0, 0, fx0);
            auto kstep = [&](int kt, auto more_t, auto more2_t) {
                constexpr bool MORE = decltype(more_t)::value, MORE2 = decltype(more2_t)::value;
                const int st = kt & 1;
                xfr(st, 1, fx1);
                mma(ml_t, fw[0], fx0);
                // every wave has its weight fragments of this stage
                lds_sync(std::integral_constant<int, 15>{});
                if (MORE2) dma(kn, st, true, false);
                xfr(st, 2, fx0);
                mma(ml_t, fw[1], fx1);
                xfr(st, 3, fx1);
                mma(ml_t, fw[2], fx0);
                if (MORE) {
                    // step kt+1 complete (step kt+2's weight loads may stay in flight)
                    if (MORE2) lds_sync(std::integral_constant<int, CW>{});
                    else lds_sync(std::integral_constant<int, 0>{});
                    if (MORE2) {
                        dma(kn, st, false, true);
                        kadvance(kn);
                    }
#pragma unroll
                    for (int ks = 0; ks < 3; ++ks) wfr(st ^ 1, ks, fw[ks]);
                    xfr(st ^ 1, 0, fx0);
                    __builtin_amdgcn_sched_barrier(0);
                    mma(ml_t, fw[3], fx1);
                    wfr(st ^ 1, 3, fw[3]);
                } else {
                    mma(ml_t, fw[3], fx1);
                    __syncthreads();
                }
            };
            int kt = 0;
            for (; kt + 2 < nk; ++kt) kstep(kt, yes{}, yes{});
            if (kt + 1 < nk) kstep(kt++, yes{}, no{});
            kstep(kt, no{}, no{});
        };
        // every wave runs every k step (loads, LDS stores, barriers); only its
        // fragment reads and MFMAs follow its live blocks
        using std::integral_constant;
        if (ml >= MB) kloop(integral_constant<int, MB>{});
        else if (MB > 3 && ml == 3) kloop(integral_constant<int, (MB > 3 ? 3 : 0)>{});
        else if (MB > 2 && ml == 2) kloop(integral_constant<int, (MB > 2 ? 2 : 0)>{});
        else if (ml == 1) kloop(integral_constant<int, 1>{});
        else kloop(integral_constant<int, 0>{});
    }

    // the fused launch takes its next ticket here: a device-scope atomic has
    // microseconds of latency, which the epilogue hides (issued before the
    // tile, the first wait on the tile's loads would wait for it as well)
    if constexpr (FUSED) {
        if (tid == 0) *next = atomicAdd(head, 1);
    }
    // ---- epilogue: lane owns token column l32 of each block; register quad q
    //      holds weight rows 8q + 4*lhi + {0..3} of the block ----
    if constexpr (ACC) {
        // Accumulating form.  The fp32 tile goes through LDS 64 token rows at
        // a time (the two 32-row blocks of pass pb, 64 KB in the weight
        // stages): row lr (0..63) holds the 256 output columns as 64 chunks of
        // 16 B, chunk c stored at c ^ lr, so the fragment writes (16 rows of a
        // fragment per LDS cycle) and the row reads (one row per wave, 64
        // consecutive floats) are both conflict-free.  Then each wave adds
        // whole row segments (64 consecutive floats per instruction) into the
        // rows of y_acc of the tile rows' tokens, scaled by the row's gate.
        float *stage = (float *)&s_w[0][0];
        auto sidx = [](int lr, int col) { return lr * 256 + (((col >> 2) ^ lr) << 2) + (col & 3); };
        const int ncol = min(BN, P.d - n_tile * BN);
        const int npass = cdiv(nr, 64);
#pragma unroll
        for (int pb = 0; pb < MB; ++pb) {
            if (pb >= npass) break;
            const int lr = wm * 32 + l32;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = wn * 64 + nb * 32 + 8 * q + 4 * lhi;
                    *(float4 *)(stage + sidx(lr, col)) =
                        make_float4(acc[nb][pb][4 * q], acc[nb][pb][4 * q + 1], acc[nb][pb][4 * q + 2],
                                    acc[nb][pb][4 * q + 3]);
                }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int lrow = __builtin_amdgcn_readfirstlane(wave + 8 * i);
                const int r = pb * 64 + lrow;          // tile row
                if (r < nr) {
                    const int j = row_off + m0 + r;     // grouped row
                    const int t = shared ? m0 + r : P.sorted_token[j];
                    const float g = shared ? 1.0f : P.gate_sorted[j];
                    float *dst = P.y_acc + (size_t)t * P.d + n_tile * BN;
#pragma unroll
                    for (int c4 = 0; c4 < 4; ++c4) {
                        const int col = c4 * 64 + lane;
                        if (col < ncol) acc_add(dst + col, g * stage[sidx(lrow, col)]);
                    }
                }
            }
            __syncthreads();
        }
        return;
    } else {
    if (!UP && shared) {
        // fp32 output of the shared experts: stored straight from registers
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if (xrow[mb] >= nr) continue;
            const int row = m0 + xrow[mb];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int col = n_tile * BN + wn * 64 + nb * 32 + 8 * q + 4 * lhi;
                    if (col >= P.d) continue;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][4 * q + e];
                    store4((float *)P.out_shared + (size_t)row * P.d + col, v);
                }
        }
        return;
    }
    if constexpr (BWD) {
        // Backward recompute: p, q are in registers (acc[0], acc[1]); da of the
        // same rows and units comes in through LDS (coalesced row loads into
        // the weight stages), and a = SiLU(p) q, dq = da SiLU(p),
        // dp = da q s (1 + p (1 - s)), s = sigmoid(p), go out through the
        // token stages, one output at a time, as row-wise 16-byte stores.
        constexpr int C16B = 16;                       // 128 units = 16 chunks of 16 B per row
        constexpr int ITB = BM * C16B / NT;
        const int ldb = shared ? P.Ks * P.w : P.w;
        const int colb = n_tile * 128;
        auto slot_in = [&](int r, int c) -> uint8_t * { return &s_w[0][0] + r * 256 + (c ^ (r & 15)) * 16; };
        auto slot_out = [&](int r, int c) -> uint8_t * { return &s_x[0][0] + r * 256 + (c ^ (r & 15)) * 16; };
        const uint16_t *dain = (const uint16_t *)(shared ? P.da_shared : P.da_routed);
#pragma unroll
        for (int it = 0; it < ITB; ++it) {
            const int i = tid + it * NT;
            const int r = i / C16B, c = i % C16B;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (r < nr && colb + c * 8 < ldb) v = *(const uint4 *)(dain + (size_t)(row_off + m0 + r) * ldb + colb + c * 8);
            *(uint4 *)slot_in(r, c) = v;
        }
        __syncthreads();
        // one output at a time (which = 0: a, 1: dp, 2: dq), recomputed from the
        // accumulators, to keep the registers of a single packed tile live
        auto pack = [&](int which, uint2 (&v)[MB][4]) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint2 dav = *(const uint2 *)(slot_in(xrow[mb], wn * 4 + q) + lhi * 8);
                    const uint32_t dw[2] = {dav.x, dav.y};
                    uint16_t h[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float da = __uint_as_float((e & 1) ? (dw[e >> 1] & 0xffff0000u) : (dw[e >> 1] << 16));
                        const float pg = acc[0][mb][4 * q + e];
                        const float pu = acc[1][mb][4 * q + e];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-pg));
                        const float o = which == 0 ? pg * sg * pu
                                      : which == 1 ? da * pu * sg * (1.0f + pg * (1.0f - sg))
                                                   : da * pg * sg;
                        h[e] = f2bf(o);
                    }
                    v[mb][q] = make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
                }
        };
        auto emit = [&](const uint2 (&v)[MB][4], uint8_t *outp) {
            __syncthreads();   // the previous output's reads of the token stages are done
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int q = 0; q < 4; ++q) *(uint2 *)(slot_out(xrow[mb], wn * 4 + q) + lhi * 8) = v[mb][q];
            __syncthreads();
            uint16_t *out = (uint16_t *)outp;
            uint4 piece[ITB];
#pragma unroll
            for (int it = 0; it < ITB; ++it) {
                const int i = tid + it * NT;
                piece[it] = *(const uint4 *)slot_out(i / C16B, i % C16B);
            }
#pragma unroll
            for (int it = 0; it < ITB; ++it) {
                const int i = tid + it * NT;
                const int r = i / C16B, c = i % C16B;
                if (r < nr && colb + c * 8 < ldb)
                    *(uint4 *)(out + (size_t)(row_off + m0 + r) * ldb + colb + c * 8) = piece[it];
            }
        };
        uint2 pv[MB][4];
        pack(0, pv);
        emit(pv, shared ? P.out_shared : P.out_routed);
        pack(1, pv);
        emit(pv, shared ? P.dp_shared : P.dp_routed);
        pack(2, pv);
        emit(pv, shared ? P.dq_shared : P.dq_routed);
        return;
    } else {
    // bf16 output tile (BM tokens x NC features) staged in the now idle LDS
    // stages, then written row by row with 16-byte stores: a wave covers whole
    // rows, where direct stores from the MFMA layout would touch 32 rows with
    // 16 bytes each.  Row pitch NC*2 bytes (C16 chunks of 16 B); chunk c of
    // row r sits at chunk c ^ (r % C16), so the 32 rows of a fragment write,
    // and the consecutive chunks of a row read, hit distinct banks.
    constexpr int NC = UP ? 128 : BN;           // features of the tile
    constexpr int C16 = NC / 8;                 // 16-byte chunks per row
    constexpr int ROWS_W = (2 * BN * RB) / (NC * 2);   // rows that fit in the weight stages
    static_assert(BM <= ROWS_W || BM - ROWS_W <= (2 * BM * RB) / (NC * 2), "output tile fits in LDS");
    auto slot = [&](int r, int c) -> uint8_t * {
        const int pc = c ^ (r & (C16 - 1));
        return r < ROWS_W ? &s_w[0][0] + r * (NC * 2) + pc * 16 : &s_x[0][0] + (r - ROWS_W) * (NC * 2) + pc * 16;
    };
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int r = xrow[mb];
        if (UP) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pg = acc[0][mb][4 * q + e];
                    const float pu = acc[1][mb][4 * q + e];
                    // SiLU(p) * q with the hardware reciprocal (about 1 ulp; an IEEE
                    // divide here costs more VALU time than the tile's MFMAs leave)
                    v[e] = pg * pu * __builtin_amdgcn_rcpf(1.0f + __expf(-pg));
                }
                store4((uint16_t *)(slot(r, wn * 4 + q) + lhi * 8), v);
            }
        } else {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = acc[nb][mb][4 * q + e];
                    store4((uint16_t *)(slot(r, wn * 8 + nb * 4 + q) + lhi * 8), v);
                }
        }
    }
    __syncthreads();
    const int ld = UP ? (shared ? P.Ks * P.w : P.w) : P.d;   // features of an output row
    const int col0 = n_tile * NC;
    uint16_t *out = (uint16_t *)(UP && shared ? P.out_shared : P.out_routed);
    // in the fused launch the activations go out as agent-coherent stores: the
    // down tiles that read them may run on another XCD, behind another L2
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + (size_t)(row_off + m0) * ld, (uint32_t)((size_t)nr * ld * 2));
    constexpr int ITER = BM * C16 / NT;   // 16-byte pieces per thread
    uint4 piece[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {   // every LDS read first, then the stores
        const int i = tid + it * NT;
        piece[it] = *(const uint4 *)slot(i / C16, i % C16);
    }
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int i = tid + it * NT;
        const int r = i / C16, c = i % C16;
        if (r < nr && col0 + c * 8 < ld) {
            if constexpr (FUSED && UP) bstore<kCoherent>(rout, ((uint32_t)r * ld + col0 + c * 8) * 2u, piece[it]);
            else *(uint4 *)(out + (size_t)(row_off + m0 + r) * ld + col0 + c * 8) = piece[it];
        }
    }
    }
    }
}

template <int BM, bool UP, bool BWD = false>
__global__ __launch_bounds__(512) void grouped_ffn_bf16_kernel(GemmParams P) {
    constexpr int BN = 256;          // weight rows per tile
    __shared__ __attribute__((aligned(16))) uint8_t s_w[2][256 * 128];
    __shared__ __attribute__((aligned(16))) uint8_t s_x[2][BM * 128];
    __shared__ int s_pref[MAXG + 1];
    __shared__ int s_src[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (P.Ks > 0 ? 1 : 0) + P.Nr;
    const int ntn_s = UP ? cdiv(P.Ks * P.w, 128) : cdiv(P.d, BN);
    const int ntn_r = UP ? cdiv(P.w, 128) : cdiv(P.d, BN);

    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_pref[0] = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            int tiles = 0;
            if (g < G) {
                const bool sh = P.Ks > 0 && g == 0;
                const int r = g - (P.Ks > 0 ? 1 : 0);
                const int rows = sh ? P.T : P.offsets[r + 1] - P.offsets[r];
                tiles = cdiv(rows, BM) * (sh ? ntn_s : ntn_r);
            }
            int incl = tiles;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            if (g < G) s_pref[g + 1] = carry + incl;
            carry += __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    const int total = s_pref[G];
    const int bid = blockIdx.x;
    if (bid >= total) return;
    // Renumbering: workgroups reach the 8 XCDs round-robin, so within each run
    // of 256 workgroups XCD x gets the 32 consecutive tiles [32x, 32x+32) of
    // that run (they are co-resident there and share operands in its L2);
    // runs follow each other in tile order, which keeps the XCDs balanced.
    // The tail run (< 256 tiles) keeps the identity order.
    const int L = (bid < (total & ~255)) ? ((bid & ~255) + (bid & 7) * 32 + ((bid >> 3) & 31)) : bid;
    int lo = 0, hi = G;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= L) lo = mid; else hi = mid;
    }
    const int g = lo;
    const bool shared = P.Ks > 0 && g == 0;
    const int r = g - (P.Ks > 0 ? 1 : 0);
    const int row_off = shared ? 0 : P.offsets[r];
    const int rows = shared ? P.T : P.offsets[r + 1] - row_off;
    const int mt = cdiv(rows, BM);
    const int lt = L - s_pref[g];
    const int m_tile = lt % mt, n_tile = lt / mt;
    // The group's rows are cut into mt runs of equal length rounded up to 32
    // (never above BM, never empty), so a group of 530 rows makes tiles of
    // 192, 192 and 146 rows instead of 256, 256 and 18: the work of a tile
    // follows its live 32-row blocks, which the waves skip when empty.
    const int run = (cdiv(rows, mt) + 31) & ~31;
    const int m0 = m_tile * run;
    const int nr = min(run, rows - m0);
    ffn_tile_bf16<BM, UP, BWD, false>(P, TileDesc{shared, r, row_off, m0, nr, n_tile}, s_w, s_x, s_src);
}

// ---------------------------------------------------------------------------
// Fused expert FFN: the up and the down projection of every group in ONE
// persistent launch of one workgroup per CU.
//
// Separate launches leave each projection with its own partial last round of
// tiles (c2b: 640 up tiles = 2.5 per CU, 800 down tiles = 3.1 per CU), so a
// third of the up launch and a quarter of the down launch run with most CUs
// idle.  Here the tiles of both projections share one schedule:
//   * a token run is one of the mt equal row runs of a group (as in the
//     separate kernels); its up tiles write the run's activations, its down
//     tiles read them;
//   * the runs are split into kQueues contiguous ranges of equal work, one
//     queue per XCD (workgroup b starts on queue b % 8, the XCD the hardware
//     gives it), so the tiles of one expert stay on one XCD and share its L2;
//   * inside a queue, tickets are taken in order from an atomic counter: all
//     up tiles of the queue's runs (the shared runs in blocks of a few runs,
//     weight-tile-major; the routed runs run-major), then all its down tiles
//     in the same order; a workgroup whose queue is empty takes tickets from
//     the other queues;
//   * a down tile waits until the up tiles of its run are done (a per-run
//     counter, bumped after the tile's coherent activation stores complete).
// No wait can deadlock: a ticket is only ever held by a running workgroup,
// up tiles never wait, a down tile's up tiles precede it in its queue, and a
// workgroup takes its next ticket only after the current tile's wait is
// over.  The wait is still bounded (spin_limit sleeps): a down tile whose
// wait gives up sets the error flag, skips its GEMM and writes NaN over its
// outputs instead (so no output is ever computed from partial activations),
// and the launch goes on; the host reads the flag through
// moe_expert_ffn_status.
// ---------------------------------------------------------------------------
constexpr int kQueues = kFfnQueues;
constexpr int kSpinLimit = 1 << 22;

struct FusedCtl {
    int *head;        // [kQueues] next ticket of each queue
    int *err;         // [1] set when a wait ran out of its budget
    int *done;        // [runs] finished up tiles of each token run
    int spin_limit;   // sleeps before a wait gives up
    int need_extra;   // added to every wait's target (0; 1 makes every wait unmeetable, for tests)
};

// NaN over the outputs of a down tile whose wait gave up.
template <bool ACC>
__device__ void poison_down_tile(const GemmParams &P, const TileDesc &td) {
    const int c0 = td.n_tile * 256, nc = min(256, P.d - c0);
    const float qnan = __builtin_nanf("");
    for (int i = threadIdx.x; i < td.nr * nc; i += 512) {
        const int r = i / nc, c = c0 + i % nc;
        if constexpr (ACC) {
            const int t = td.shared ? td.m0 + r : P.sorted_token[td.row_off + td.m0 + r];
            acc_add(P.y_acc + (size_t)t * P.d + c, qnan);
        } else if (td.shared) {
            ((float *)P.out_shared)[(size_t)(td.m0 + r) * P.d + c] = qnan;
        } else {
            ((uint16_t *)P.out_routed)[(size_t)(td.row_off + td.m0 + r) * P.d + c] = 0x7fc0;
        }
    }
}

template <int BM, int WAUX, bool ACC>
__global__ __launch_bounds__(512) void grouped_ffn_fused_kernel(GemmParams Pu, GemmParams Pd, FusedCtl C) {
    __shared__ __attribute__((aligned(16))) uint8_t s_w[2][256 * 128];
    __shared__ __attribute__((aligned(16))) uint8_t s_x[2][BM * 128];
    __shared__ int s_src[BM];
    __shared__ int s_runp[MAXG + 1];   // prefix of the token runs over the groups
    __shared__ int s_offs[MAXG + 1];   // the routed group offsets
    __shared__ int s_ticket;
    __shared__ int s_met;              // the down tile's wait was met

    const GemmParams &P = Pu;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int G = (P.Ks > 0 ? 1 : 0) + P.Nr;
    if (wave == 0) {
        int carry = 0;
        if (lane == 0) s_runp[0] = 0;
        for (int g0 = 0; g0 < G; g0 += 64) {
            const int g = g0 + lane;
            int runs = 0;
            if (g < G) {
                int rows = P.T;
                if (!(P.Ks > 0 && g == 0)) {
                    const int r = g - (P.Ks > 0 ? 1 : 0);
                    const int a = P.offsets[r], b = P.offsets[r + 1];
                    rows = b - a;
                    s_offs[r] = a;
                    if (r + 1 == P.Nr) s_offs[P.Nr] = b;
                }
                runs = cdiv(rows, BM);
            }
            int incl = runs;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int v = __shfl_up(incl, o, 64);
                if (lane >= o) incl += v;
            }
            if (g < G) s_runp[g + 1] = carry + incl;
            carry += __shfl(incl, 63, 64);
        }
    }
    __syncthreads();
    // wave-uniform bookkeeping lives in SGPRs (readfirstlane of the LDS values):
    // the tile bodies need every VGPR
    auto uni = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    const int R = uni(s_runp[G]);
    const int mts = P.Ks > 0 ? uni(s_runp[1]) : 0;                  // runs of the shared group
    const int nus = cdiv(P.Ks * P.w, 128), nur = cdiv(P.w, 128);    // up tiles per run
    const int nd = cdiv(P.d, 256);                                  // down tiles per run
    // Queue q serves the runs [qstart(q), qstart(q+1)): equal shares of the work, counted in
    // 64-wide k steps (a shared run, of width K_s*w, weighs more than a routed one), so the
    // queues drain together and few tiles leave their XCD.
    const int64_t ws = (int64_t)nus * (P.d / 64) + (int64_t)nd * (P.Ks * P.w / 64);
    const int64_t wr = (int64_t)nur * (P.d / 64) + (int64_t)nd * (P.w / 64);
    const int64_t wtot = (int64_t)mts * ws + (int64_t)(R - mts) * wr;
    auto qstart = [&](int q) -> int {
        const int64_t tau = wtot * q / kQueues;
        int r;
        if (mts > 0 && tau <= (int64_t)mts * ws) r = (int)((tau + ws - 1) / ws);
        else r = mts + (int)((tau - (int64_t)mts * ws + wr - 1) / wr);
        return q >= kQueues ? R : min(r, R);
    };
    // The shared runs of a queue go in blocks of kShBlock runs, each block weight-tile-major
    // (tile n of every run of the block, then tile n+1): the workgroups of one XCD then work on a
    // few runs and a few weight tiles at a time and share both in L2, where run-major order
    // streamed the whole shared weight stack once per run.  l counts the tiles of the queue's
    // shared runs [s0, s1), `per` tiles per run.
    constexpr int kShBlock = 4;
    auto blocked = [&](int l, int s0, int s1, int per, int &run, int &n) {
        const int j = l / (kShBlock * per);
        const int b0 = s0 + j * kShBlock;
        const int bsz = min(kShBlock, s1 - b0);
        const int lo = l - j * kShBlock * per;
        n = lo / bsz;
        run = b0 + lo % bsz;
    };

    const int q0 = blockIdx.x % kQueues;
    for (int qi = 0; qi < kQueues; ++qi) {
        const int q = (q0 + qi) % kQueues;
        const int ra = qstart(q), rb = qstart(q + 1);
        const int se = min(rb, mts), rs = max(ra, mts);    // shared runs [ra, se), routed runs [rs, rb)
        const int nsh = max(se - ra, 0), nro = max(rb - rs, 0);
        const int nUs = nsh * nus, nU = nUs + nro * nur, nDs = nsh * nd;
        const int len = nU + (nsh + nro) * nd;
        if (len == 0) continue;
        if (tid == 0) s_ticket = atomicAdd(&C.head[q], 1);
        __syncthreads();
        int t = uni(s_ticket);
        __syncthreads();   // every wave has read the ticket before it is rewritten
        while (t < len) {
            // tickets: the up tiles (shared blocks, then routed runs run-major), then the down
            // tiles in the same order
            const bool up = t < nU;
            int run, n;
            if (t < nUs) {
                blocked(t, ra, se, nus, run, n);
            } else if (up) {
                const int v = t - nUs;
                run = rs + v / nur;
                n = v % nur;
            } else if (t < nU + nDs) {
                blocked(t - nU, ra, se, nd, run, n);
            } else {
                const int v = t - nU - nDs;
                run = rs + v / nd;
                n = v % nd;
            }
            // group of the run: the number of prefix entries s_runp[1..G] <= run,
            // one ballot per 64 groups (each wave on its own)
            int g = 0;
            for (int g0 = 1; g0 <= G; g0 += 64) {
                const int gi = g0 + lane;
                const bool le = gi <= G && s_runp[gi] <= run;
                g += __builtin_popcountll(__ballot(le));
            }
            g = uni(g);
            TileDesc td;
            td.shared = P.Ks > 0 && g == 0;
            td.r = g - (P.Ks > 0 ? 1 : 0);
            td.row_off = td.shared ? 0 : uni(s_offs[td.r]);
            const int rows = td.shared ? P.T : uni(s_offs[td.r + 1]) - td.row_off;
            const int rp = uni(s_runp[g]);
            const int mt = uni(s_runp[g + 1]) - rp;
            const int rl = (cdiv(rows, mt) + 31) & ~31;
            td.m0 = (run - rp) * rl;
            td.nr = min(rl, rows - td.m0);
            td.n_tile = n;
            int met = 1;
            if (!up) {
                const int need = (td.shared ? nus : nur) + C.need_extra;
                if (tid == 0) {
                    int spins = 0, ok = 1;
                    while (__hip_atomic_load(&C.done[run], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
                        if (++spins > C.spin_limit) {
                            __hip_atomic_store(C.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            ok = 0;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(4);
                    }
                    s_met = ok;
                }
                __syncthreads();
                met = uni(s_met);
            }
            int next = 0;
            if (up) {
                ffn_tile_bf16<BM, true, false, true, WAUX>(Pu, td, s_w, s_x, s_src, &C.head[q], &next);
                __builtin_amdgcn_s_waitcnt(0);   // this thread's activation stores are complete
                __syncthreads();
                if (tid == 0) __hip_atomic_fetch_add(&C.done[run], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            } else if (met) {
                ffn_tile_bf16<BM, false, false, true, WAUX, ACC>(Pd, td, s_w, s_x, s_src, &C.head[q], &next);
            } else {
                poison_down_tile<ACC>(Pd, td);
                if (tid == 0) next = atomicAdd(&C.head[q], 1);
            }
            if (tid == 0) s_ticket = next;
            __syncthreads();
            t = uni(s_ticket);
            __syncthreads();
        }
    }
}

// Runs before every moe_expert_ffn: clears the control words of the fused
// launch (queue heads, error flag, run counters) and, in accumulating mode,
// zeroes y_acc [T, d] and writes the gates in grouped order
// (gate_sorted[slot_of[t,k]] = gate[t,k]; slots of skipped pairs are -1).
__global__ __launch_bounds__(256) void ffn_prep_kernel(int *ctl, int n, float *y_acc, int64_t n4,
                                                       const float *gate, const int32_t *slot_of,
                                                       float *gate_sorted, int npairs) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int64_t i = i0; i < n; i += stride) ctl[i] = 0;
    if (y_acc) {
        for (int64_t i = i0; i < n4; i += stride) ((float4 *)y_acc)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int64_t i = i0; i < npairs; i += stride) {
            const int j = slot_of[i];
            if (j >= 0 && j < npairs) gate_sorted[j] = gate[i];
        }
    }
}

GemmParams make_params(const moe_problem &p, const FfnArgs &a, bool up) {
    GemmParams P{};
    P.T = p.T; P.d = p.d; P.Ks = p.n_shared; P.Nr = p.n_routed; P.w = p.inter;
    P.TK = p.T * p.top_k;
    P.offsets = a.offsets;
    P.sorted_token = a.sorted_token;
    P.x = (const uint8_t *)a.x;
    P.act_shared = (const uint8_t *)a.act_shared;
    P.act_routed = (const uint8_t *)a.act_routed;
    P.gate_sorted = a.gate_sorted;
    P.y_acc = up ? nullptr : a.y_acc;
    if (up) {
        P.wa_r = (const uint8_t *)a.w1_r; P.wb_r = (const uint8_t *)a.w3_r;
        P.wa_s = (const uint8_t *)a.w1_s; P.wb_s = (const uint8_t *)a.w3_s;
        P.out_shared = (uint8_t *)a.act_shared; P.out_routed = (uint8_t *)a.act_routed;
    } else {
        P.wa_r = (const uint8_t *)a.w2_r; P.wb_r = nullptr;
        P.wa_s = (const uint8_t *)a.w2_s; P.wb_s = nullptr;
        P.out_shared = (uint8_t *)a.y_shared; P.out_routed = (uint8_t *)a.y_routed;
    }
    return P;
}

// Upper bound of the tile count for token tiles of bm rows and weight
// tiles of `wn` rows (act columns in the up projection):
// sum_r ceil(c_r / bm) <= floor(T K' / bm) + N'.
int tile_bound(const moe_problem &p, bool up, int bm, int wn_up, int wn_down) {
    const int rt_bound = (int)(((int64_t)p.T * p.top_k) / bm) + p.n_routed;
    const int mts = p.n_shared > 0 ? cdiv(p.T, bm) : 0;
    if (up) return mts * cdiv(p.n_shared * p.inter, wn_up) + (p.n_routed > 0 ? rt_bound * cdiv(p.inter, wn_up) : 0);
    return mts * cdiv(p.d, wn_down) + (p.n_routed > 0 ? rt_bound * cdiv(p.d, wn_down) : 0);
}

template <typename DT, bool UP>
hipError_t launch_typed(const moe_problem &p, const FfnArgs &a, hipStream_t s) {
    const int tiles = tile_bound(p, UP, BM, 64, BN);
    if (tiles == 0) return hipSuccess;
    grouped_ffn_kernel<DT, UP><<<tiles, 256, 0, s>>>(make_params(p, a, UP));
    return hipGetLastError();
}

// Token tile of the bf16 path: 256 rows when the routed experts average at
// least 256 rows (measured: the larger tile's lower LDS traffic per MFMA
// outweighs its edge waste down to ~2 tiles per expert), else 128.
template <bool UP>
hipError_t launch_bf16(const moe_problem &p, const FfnArgs &a, hipStream_t s) {
    const int64_t avg = p.n_routed > 0 ? ((int64_t)p.T * p.top_k) / p.n_routed : (int64_t)p.T;
    if (avg >= 256) {
        const int tiles = tile_bound(p, UP, 256, 128, 256);
        if (tiles == 0) return hipSuccess;
        grouped_ffn_bf16_kernel<256, UP><<<tiles, 512, 0, s>>>(make_params(p, a, UP));
    } else {
        const int tiles = tile_bound(p, UP, 128, 128, 256);
        if (tiles == 0) return hipSuccess;
        grouped_ffn_bf16_kernel<128, UP><<<tiles, 512, 0, s>>>(make_params(p, a, UP));
    }
    return hipGetLastError();
}

// The preparation kernel of every moe_expert_ffn call (see ffn_prep_kernel).
hipError_t launch_prep(const moe_problem &p, const FfnArgs &a, int32_t *ctl, hipStream_t s) {
    const int n = ffn_ctl_ints(p);
    const bool accum = a.y_acc != nullptr && p.T > 0;
    const int64_t n4 = accum ? (int64_t)p.T * p.d / 4 : 0;
    const int npairs = accum ? p.T * p.top_k : 0;
    const int64_t work = std::max<int64_t>(std::max<int64_t>(n, n4), npairs);
    const int grid = (int)std::min<int64_t>(std::max<int64_t>((work + 255) / 256, 1), 2048);
    ffn_prep_kernel<<<grid, 256, 0, s>>>(ctl, n, accum ? a.y_acc : nullptr, n4, a.gate, a.slot_of,
                                         a.gate_sorted, npairs);
    return hipGetLastError();
}

// Which fused instantiation a problem takes: the token tile (256 rows when the routed experts
// average at least 256 rows, else 128) and the weight loads' cache policy. Decode batches (at
// most 64 rows per expert on average, no shared group or at most 128 tokens) read each
// expert's weights with a single token tile: there the weight loads are non-temporal, so the
// streamed weights leave L2 to the token rows and activations that are read again (c5a expert
// FFN 207.5 -> 193.2 us, c5c 548 -> 510 us). With more rows an expert's second tile re-reads
// its weights from L2, and the hint costs 4-13% (192 rows per expert on average: 491 ->
// 555 us); a shared group over more than 128 tokens is such a case too.
enum class FusedForm { k256, k128nt, k128 };
FusedForm fused_form(const moe_problem &p) {
    const int64_t avg = p.n_routed > 0 ? ((int64_t)p.T * p.top_k) / p.n_routed : (int64_t)p.T;
    if (avg >= 256) return FusedForm::k256;
    if (avg <= 64 && (p.n_shared == 0 || p.T <= 128)) return FusedForm::k128nt;
    return FusedForm::k128;
}

// Test hook: MOE_DEBUG_FFN_STALL=<n> (n > 0) makes every wait of the fused launch unmeetable and
// gives up after n sleeps, so the error path runs with every kernel exiting normally.
void stall_hook(int *spin_limit, int *need_extra) {
    *spin_limit = kSpinLimit;
    *need_extra = 0;
    if (const char *e = getenv("MOE_DEBUG_FFN_STALL")) {
        const int n = atoi(e);
        if (n > 0) {
            *spin_limit = n;
            *need_extra = 1;
        }
    }
}

hipError_t launch_fused(const moe_problem &p, const FfnArgs &a, int32_t *ctl, hipStream_t s) {
    int dev = 0, ncu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const GemmParams Pu = make_params(p, a, true), Pd = make_params(p, a, false);
    FusedCtl C{ctl, ctl + kQueues, ctl + kQueues + 1, 0, 0};
    stall_hook(&C.spin_limit, &C.need_extra);
    const bool accum = a.y_acc != nullptr;
    switch (fused_form(p)) {
        case FusedForm::k256:
            if (accum) grouped_ffn_fused_kernel<256, 0, true><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            else grouped_ffn_fused_kernel<256, 0, false><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            break;
        case FusedForm::k128nt:
            if (accum) grouped_ffn_fused_kernel<128, kNonTemporal, true><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            else grouped_ffn_fused_kernel<128, kNonTemporal, false><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            break;
        case FusedForm::k128:
            if (accum) grouped_ffn_fused_kernel<128, 0, true><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            else grouped_ffn_fused_kernel<128, 0, false><<<ncu, 512, 0, s>>>(Pu, Pd, C);
            break;
    }
    return hipGetLastError();
}

}  // namespace

// Backward recompute of the up projection (bf16): act_* <- a, dp_*, dq_* from da_*.
hipError_t launch_expert_up_backward(const moe_problem &p, const FfnArgs &a, const void *da_shared,
                                     const void *da_routed, void *dp_shared, void *dp_routed, void *dq_shared,
                                     void *dq_routed, hipStream_t s) {
    GemmParams P = make_params(p, a, true);
    P.da_shared = (const uint8_t *)da_shared;
    P.da_routed = (const uint8_t *)da_routed;
    P.dp_shared = (uint8_t *)dp_shared;
    P.dp_routed = (uint8_t *)dp_routed;
    P.dq_shared = (uint8_t *)dq_shared;
    P.dq_routed = (uint8_t *)dq_routed;
    const int64_t avg = p.n_routed > 0 ? ((int64_t)p.T * p.top_k) / p.n_routed : (int64_t)p.T;
    if (avg >= 256) {
        const int tiles = tile_bound(p, true, 256, 128, 256);
        if (tiles == 0) return hipSuccess;
        grouped_ffn_bf16_kernel<256, true, true><<<tiles, 512, 0, s>>>(P);
    } else {
        const int tiles = tile_bound(p, true, 128, 128, 256);
        if (tiles == 0) return hipSuccess;
        grouped_ffn_bf16_kernel<128, true, true><<<tiles, 512, 0, s>>>(P);
    }
    return hipGetLastError();
}

hipError_t launch_expert_up(const moe_problem &p, const FfnArgs &a, hipStream_t s) {
    if (p.dtype == MOE_BF16) return launch_bf16<true>(p, a, s);
    return launch_typed<float, true>(p, a, s);
}

hipError_t launch_expert_down(const moe_problem &p, const FfnArgs &a, hipStream_t s) {
    if (p.dtype == MOE_BF16) return launch_bf16<false>(p, a, s);
    return launch_typed<float, false>(p, a, s);
}

hipError_t launch_expert_ffn(const moe_problem &p, const FfnArgs &a, int32_t *ctl, hipStream_t s, bool prep) {
    hipError_t e = prep ? launch_prep(p, a, ctl, s) : hipSuccess;
    const bool active = p.T > 0 && (p.n_shared > 0 || (p.n_routed > 0 && p.top_k > 0));
    if (e != hipSuccess || !active) return e;
    if (p.dtype == MOE_BF16) return launch_fused(p, a, ctl, s);
    e = launch_typed<float, true>(p, a, s);
    if (e == hipSuccess) e = launch_typed<float, false>(p, a, s);
    return e;
}

const char *expert_ffn_kernel_name(const moe_problem &p, bool accum) {
    if (p.dtype != MOE_BF16) return "grouped_ffn_kernel<float, true> + grouped_ffn_kernel<float, false>";
    switch (fused_form(p)) {
        case FusedForm::k256:
            return accum ? "grouped_ffn_fused_kernel<256, 0, true>" : "grouped_ffn_fused_kernel<256, 0, false>";
        case FusedForm::k128nt:
            return accum ? "grouped_ffn_fused_kernel<128, 2, true>" : "grouped_ffn_fused_kernel<128, 2, false>";
        default:
            return accum ? "grouped_ffn_fused_kernel<128, 0, true>" : "grouped_ffn_fused_kernel<128, 0, false>";
    }
}

}  // namespace moe
