// permute.hip -- group (token, expert) pairs by routed expert on gfx950.
//
// The bookkeeping behind "token t selects expert i" ("【论文总结】MoE" section
// 2.3): a stable counting sort of the T*K' pairs by expert, so each expert's
// tokens sit contiguously (tokens ascending) for the grouped expert GEMMs.
//
//   hist     <<<ceil(T/256), 256>>>  per-block expert histogram (LDS int atomics),
//                                    stored expert-major: hist[r][b]
//   scatter  <<<ceil(T/256), 256>>>  each block first derives what it needs from the
//                                    whole histogram: expert totals, their exclusive
//                                    scan (= offsets; block 0 stores them) and the
//                                    first slot of (expert, this block) = offsets[r]
//                                    + earlier blocks' counts.  Then each wave builds,
//                                    per expert, the 64-bit mask of its lanes (tokens)
//                                    that chose it; a pair's rank inside the expert is
//                                    popcount of the masks of earlier waves plus its
//                                    lanes below -> stable.
// A single block (T <= 256, decode batches) counts its own pairs and scans
// them itself: one launch instead of two.
// When the histogram is large (blocks x experts above kFusedScanMax) every
// scatter block re-reading it would cost more than one more launch, so a
// separate scan kernel <<<1, 1024>>> computes offsets and the per-(expert,
// block) first slots once.
// Integer-only, so the result is identical on every run.
#include "moe_internal.h"

namespace moe {
namespace {

// The (t, k) entries of a block's tokens are one contiguous run of idx: the
// threads read it together (consecutive threads, consecutive entries, 4
// independent loads in flight per thread).
constexpr int kUnroll = 4;

// Workgroup b of nblk: the expert histogram of tokens [256 b, 256 b + 256) into hist[r, b].
__device__ inline void perm_hist_block(int T, int Nr, int K, const int32_t *__restrict__ idx,
                                       int32_t *__restrict__ hist, int b, int nblk) {
    __shared__ int cnt[kPermuteMaxExperts];
    for (int r = threadIdx.x; r < Nr; r += 256) cnt[r] = 0;
    __syncthreads();
    const int t0 = b * kPermuteTokens;
    const int n = min(kPermuteTokens, T - t0) * K;
    const int32_t *run = idx + (size_t)t0 * K;
    for (int e = threadIdx.x; e < n; e += kUnroll * 256) {
        int v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = e + u * 256 < n ? run[e + u * 256] : -1;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if ((unsigned)v[u] < (unsigned)Nr) atomicAdd(&cnt[v[u]], 1);
    }
    __syncthreads();
    for (int r = threadIdx.x; r < Nr; r += 256) hist[(size_t)r * nblk + b] = cnt[r];
}

__global__ __launch_bounds__(256) void perm_hist_kernel(int T, int Nr, int K,
                                                        const int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ hist) {
    perm_hist_block(T, Nr, K, idx, hist, blockIdx.x, gridDim.x);
}

// Workgroups 0 .. nblk-1: perm_hist_block; workgroups nblk .. nblk+Nr-1: the routing's reduction
// for expert blockIdx.x - nblk (route_reduce_block over rblk partials). Both read only what the
// routing wrote, so they share one launch (moe_layer_forward).
__global__ __launch_bounds__(256) void perm_hist_reduce_kernel(int T, int Nr, int K, const int32_t *__restrict__ idx,
                                                               int32_t *__restrict__ hist, int nblk, int rblk,
                                                               const int32_t *__restrict__ part_counts,
                                                               const double *__restrict__ part_psum,
                                                               int32_t *__restrict__ counts,
                                                               float *__restrict__ prob_sum) {
    if ((int)blockIdx.x < nblk)
        perm_hist_block(T, Nr, K, idx, hist, blockIdx.x, nblk);
    else
        route_reduce_block((int)blockIdx.x - nblk, rblk, Nr, part_counts, part_psum, counts, prob_sum);
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int nblk, int Nr,
                                                         const int32_t *__restrict__ hist,
                                                         int32_t *__restrict__ base,
                                                         int32_t *__restrict__ offsets) {
    __shared__ int wsum[16];
    const int r = threadIdx.x, lane = r & 63, wave = r >> 6;
    const int32_t *row = hist + (size_t)r * nblk;
    int total = 0;
    if (r < Nr)
        for (int b = 0; b < nblk; ++b) total += row[b];
    // inclusive scan within the wave, then across the 16 wave totals
    int incl = total;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const int excl = before + incl - total;
    if (r < Nr) {
        offsets[r] = excl;
        int run = excl;
        int32_t *brow = base + (size_t)r * nblk;
        for (int b = 0; b < nblk; ++b) {
            brow[b] = run;
            run += row[b];
        }
    }
    if (r == 0) {
        int all = 0;
        for (int w = 0; w < 16; ++w) all += wsum[w];
        offsets[Nr] = all;
    }
}

constexpr int kFusedScanMax = 16384;   // histogram entries each scatter block may read

// Exclusive scan over experts of tot[0..Nr) in place (Nr <= 1024), 256
// threads: each takes a run of 4 consecutive experts.  Returns the total.
__device__ int block_exscan_experts(int *tot, int Nr, int *s_w) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int r0 = tid * 4;
    int loc[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        loc[i] = r0 + i < Nr ? tot[r0 + i] : 0;
        sum += loc[i];
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
    }
    if (lane == 63) s_w[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_w[w];
    const int all = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (r0 + i < Nr) tot[r0 + i] = run;
        run += loc[i];
    }
    __syncthreads();
    return all;
}

// HM (where the counts come from): kFromHist derives offsets and this
// block's first slots from hist (see above); kFromBase reads the first slots
// from base (written by perm_scan_kernel); kSelf, for a single block (up to
// 256 tokens, decode batches), counts its own pairs, so no histogram launch
// precedes it.
enum { kFromBase = 0, kFromHist = 1, kSelf = 2 };
// The scatter of block b of nblk (256 threads); the kernel below and the decode tail kernel
// (layer_decode_tail_kernel) run it.  kSelf: the block's entries are read from memory once
// and kept in LDS for the later passes when they fit (at most kSelfCache), and tot_out (LDS of
// the caller, or null) receives each expert's count of pairs.
constexpr int kSelfCache = 4096;
template <int HM>
__device__ __forceinline__ void perm_scatter_block(int T, int Nr, int K, int nblk, int b,
                                                   const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ hist,
                                                   const int32_t *__restrict__ base,
                                                   int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ sorted_token,
                                                   int32_t *__restrict__ slot_of, int *tot_out = nullptr) {
    __shared__ unsigned long long mask[4][kPermuteMaxExperts];
    __shared__ int s_first[kPermuteMaxExperts];
    __shared__ int s_tot[kPermuteMaxExperts];
    __shared__ int s_w[4];
    __shared__ int s_idx[HM == kSelf ? kSelfCache : 1];
    for (int i = threadIdx.x; i < 4 * Nr; i += 256) mask[i / Nr][i % Nr] = 0ull;
    const bool cached = HM == kSelf && min(kPermuteTokens, T) * K <= kSelfCache;
    if (HM == kSelf) {
        for (int r = threadIdx.x; r < Nr; r += 256) s_tot[r] = 0;
        __syncthreads();
        const int n = min(kPermuteTokens, T) * K;
        for (int e = threadIdx.x; e < n; e += kUnroll * 256) {
            int v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = e + u * 256 < n ? idx[e + u * 256] : -1;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                if ((unsigned)v[u] < (unsigned)Nr) atomicAdd(&s_tot[v[u]], 1);
                if (cached && e + u * 256 < n) s_idx[e + u * 256] = v[u];
            }
        }
        __syncthreads();
        if (tot_out)
            for (int r = threadIdx.x; r < Nr; r += 256) tot_out[r] = s_tot[r];
        const int all = block_exscan_experts(s_tot, Nr, s_w);
        for (int r = threadIdx.x; r < Nr; r += 256) {
            s_first[r] = s_tot[r];
            offsets[r] = s_tot[r];
        }
        if (threadIdx.x == 0) offsets[Nr] = all;
    } else if (HM == kFromHist) {
        for (int r = threadIdx.x; r < Nr; r += 256) { s_tot[r] = 0; s_first[r] = 0; }
        __syncthreads();
        // expert totals and this block's preceding counts: every (expert,
        // block) entry of hist read once, summed with integer LDS atomics
        const int nh = Nr * nblk;
        for (int e = threadIdx.x; e < nh; e += kUnroll * 256) {
            int v[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) v[u] = e + u * 256 < nh ? hist[e + u * 256] : 0;
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int f = e + u * 256;
                if (f < nh && v[u] != 0) {
                    const int r = f / nblk, j = f % nblk;
                    atomicAdd(&s_tot[r], v[u]);
                    if (j < b) atomicAdd(&s_first[r], v[u]);
                }
            }
        }
        __syncthreads();
        const int all = block_exscan_experts(s_tot, Nr, s_w);
        for (int r = threadIdx.x; r < Nr; r += 256) {
            s_first[r] += s_tot[r];
            if (b == 0) offsets[r] = s_tot[r];
        }
        if (b == 0 && threadIdx.x == 0) offsets[Nr] = all;
    } else {
        for (int r = threadIdx.x; r < Nr; r += 256) s_first[r] = base[(size_t)r * nblk + b];
    }
    __syncthreads();
    // entries of this block: token t0 + e / K, slot k = e % K; its wave and lane
    // are those of the token within the block (64 tokens per wave)
    const int t0 = b * kPermuteTokens;
    const int n = min(kPermuteTokens, T - t0) * K;
    const int32_t *run = idx + (size_t)t0 * K;
    auto entry = [&](int i) { return cached ? s_idx[i] : run[i]; };
    for (int e = threadIdx.x; e < n; e += kUnroll * 256) {
        int v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = e + u * 256 < n ? entry(e + u * 256) : -1;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int tt = (e + u * 256) / K;
            if ((unsigned)v[u] < (unsigned)Nr) atomicOr(&mask[tt >> 6][v[u]], 1ull << (tt & 63));
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kUnroll * 256) {
        int v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) v[u] = e + u * 256 < n ? entry(e + u * 256) : -1;
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int f = e + u * 256;
            if (f >= n) continue;
            const int r = v[u];
            if ((unsigned)r >= (unsigned)Nr) {
                slot_of[(size_t)t0 * K + f] = -1;
                continue;
            }
            // rank of token tt among this block's tokens that chose r, in token order
            const int tt = f / K, w = tt >> 6, l = tt & 63;
            const unsigned long long below = l == 0 ? 0ull : (~0ull >> (64 - l));
            int rank = __popcll(mask[w][r] & below);
            for (int ww = 0; ww < w; ++ww) rank += __popcll(mask[ww][r]);
            const int pos = s_first[r] + rank;
            sorted_token[pos] = t0 + tt;
            slot_of[(size_t)t0 * K + f] = pos;
        }
    }
}

template <int HM>
__global__ __launch_bounds__(256) void perm_scatter_kernel(int T, int Nr, int K,
                                                           const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ hist,
                                                           const int32_t *__restrict__ base,
                                                           int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ sorted_token,
                                                           int32_t *__restrict__ slot_of) {
    perm_scatter_block<HM>(T, Nr, K, gridDim.x, blockIdx.x, idx, hist, base, offsets, sorted_token, slot_of);
}

__global__ void perm_empty_kernel(int Nr, int32_t *__restrict__ offsets) {
    for (int r = threadIdx.x; r <= Nr; r += blockDim.x) offsets[r] = 0;
}

// The decode tail of moe_layer_forward, two independent workgroups of 256 threads (T <= 256
// decode workgroups of routing partials, N' <= 256). Workgroup 0 does what the expert FFN after
// it needs:
//   * the single-block grouping (as moe_permute for T <= 256);
//   * the fused expert FFN's control words cleared (as its preparation kernel in gather mode).
// Workgroup 1, beside it:
//   * the expert counts as a histogram of idx, the integers moe_route sums from its count
//     partials;
//   * affinity sums: thread r sums expert r's partials as route_reduce_kernel's tree does (each
//     group of 64 workgroup rows pairwise at distances 32, 16, ..., 1 -- the butterfly of its
//     waves -- rows past T adding +0, then the four group sums in order), so prob_sum is bitwise
//     that of moe_route;
//   * the balance statistics on them (balance_stats_block, as moe_balance_stats).
__global__ __launch_bounds__(256) void layer_decode_tail_kernel(
    int T, int Nr, int K, int D, const double *__restrict__ part_psum,
    int32_t *__restrict__ counts, float *__restrict__ prob_sum, const int32_t *__restrict__ idx,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_token, int32_t *__restrict__ slot_of,
    float *__restrict__ f, float *__restrict__ P, float *__restrict__ f_dev, float *__restrict__ P_dev,
    float *__restrict__ exp_bal, float *__restrict__ dev_bal, int32_t *__restrict__ ctl, int nctl) {
    __shared__ int s_cnt[kRouteMaxExperts];
    __shared__ float s_ps[kRouteMaxExperts];
    if (blockIdx.x == 0) {
        perm_scatter_block<kSelf>(T, Nr, K, 1, 0, idx, nullptr, nullptr, offsets, sorted_token, slot_of);
        for (int i = threadIdx.x; i < nctl; i += 256) ctl[i] = 0;
        return;
    }
    // each expert's count of selections: the same integers as the sum of the routing's count
    // partials
    for (int e = threadIdx.x; e < Nr; e += 256) s_cnt[e] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < T * K; e += 256) {
        const int v = idx[e];
        if ((unsigned)v < (unsigned)Nr) atomicAdd(&s_cnt[v], 1);
    }
    __syncthreads();
    const int r = threadIdx.x;
    if (r < Nr) {
        double total = 0.0;
#pragma nounroll
        for (int w = 0; w < 4; ++w) {
            double g = 0.0;   // a group with no rows sums to +0, as in route_reduce_kernel
            if (64 * w < T) {
                // the group's 64 rows are loaded together (rows past T clamped and replaced by
                // zero), then summed
                double a[64];
#pragma unroll
                for (int i = 0; i < 64; ++i) a[i] = part_psum[(size_t)min(64 * w + i, T - 1) * Nr + r];
#pragma unroll
                for (int i = 0; i < 64; ++i) a[i] = 0.0 + (64 * w + i < T ? a[i] : 0.0);
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
                    for (int i = 0; i < o; ++i) a[i] = a[i] + a[i + o];
                g = a[0];
            }
            total = w == 0 ? g : total + g;   // ((g0 + g1) + g2) + g3
        }
        const float ps = (float)total;
        counts[r] = s_cnt[r];
        prob_sum[r] = ps;
        s_ps[r] = ps;
    }
    __syncthreads();
    balance_stats_block(T, Nr, K, D, s_cnt, s_ps, f, P, f_dev, P_dev, exp_bal, dev_bal);
}

}  // namespace

hipError_t launch_layer_decode_tail(const moe_problem &p, int groups, const double *part_psum, int32_t *counts, float *prob_sum,
                                    const int32_t *idx, int32_t *offsets, int32_t *sorted_token,
                                    int32_t *slot_of, float *f, float *P, float *f_dev, float *P_dev,
                                    float *exp_bal, float *dev_bal, int32_t *ctl, int nctl, hipStream_t s) {
    if (p.T > kPermuteTokens || p.n_routed > kRouteMaxExperts) return hipErrorInvalidValue;
    layer_decode_tail_kernel<<<2, 256, 0, s>>>(p.T, p.n_routed, p.top_k, groups, part_psum, counts,
                                               prob_sum, idx, offsets, sorted_token, slot_of, f, P, f_dev, P_dev,
                                               exp_bal, dev_bal, ctl, nctl);
    return hipGetLastError();
}

hipError_t launch_permute(const moe_problem &p, const int32_t *idx, int32_t *offsets,
                          int32_t *sorted_token, int32_t *slot_of, int32_t *hist, int32_t *base,
                          hipStream_t s, const RouteReduce *rr) {
    const int nblk = cdiv(p.T, kPermuteTokens);
    if (rr && (nblk < 2 || p.top_k == 0 || p.n_routed == 0)) return hipErrorInvalidValue;
    if (nblk == 0 || p.top_k == 0 || p.n_routed == 0) {
        perm_empty_kernel<<<1, 256, 0, s>>>(p.n_routed, offsets);
        return hipGetLastError();
    }
    if (nblk == 1) {
        perm_scatter_kernel<kSelf><<<1, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, nullptr, nullptr, offsets,
                                                     sorted_token, slot_of);
        return hipGetLastError();
    }
    if (rr)
        perm_hist_reduce_kernel<<<nblk + p.n_routed, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, hist, nblk,
                                                                  rr->nblk, rr->part_counts, rr->part_psum,
                                                                  rr->counts, rr->prob_sum);
    else
        perm_hist_kernel<<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, hist);
    if ((int64_t)nblk * p.n_routed <= kFusedScanMax) {
        perm_scatter_kernel<kFromHist><<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, hist, nullptr, offsets,
                                                            sorted_token, slot_of);
    } else {
        perm_scan_kernel<<<1, 1024, 0, s>>>(nblk, p.n_routed, hist, base, offsets);
        perm_scatter_kernel<kFromBase><<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, hist, base, offsets,
                                                            sorted_token, slot_of);
    }
    return hipGetLastError();
}

}  // namespace moe
