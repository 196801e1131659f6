// permute.hip -- group (token, expert) pairs by routed expert on gfx950.
//
// The bookkeeping behind "token t selects expert i" ("【论文总结】MoE" section
// 2.3): a stable counting sort of the T*K' pairs by expert, so each expert's
// tokens sit contiguously (tokens ascending) for the grouped expert GEMMs.
//
//   hist     <<<ceil(T/256), 256>>>  per-block expert histogram (LDS int atomics)
//   scan     <<<1, 1024>>>           expert totals -> offsets; per (block, expert)
//                                    first slot = offsets[r] + earlier blocks' counts
//   scatter  <<<ceil(T/256), 256>>>  each wave builds, per expert, the 64-bit mask of
//                                    its lanes (tokens) that chose it; a pair's rank
//                                    inside the expert is popcount of the masks of
//                                    earlier waves plus its lanes below -> stable.
// Integer-only, so the result is identical on every run.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void perm_hist_kernel(int T, int Nr, int K,
                                                        const int32_t *__restrict__ idx,
                                                        int32_t *__restrict__ hist) {
    __shared__ int cnt[kPermuteMaxExperts];
    for (int r = threadIdx.x; r < Nr; r += 256) cnt[r] = 0;
    __syncthreads();
    const int t = blockIdx.x * kPermuteTokens + threadIdx.x;
    if (t < T) {
        for (int k = 0; k < K; ++k) {
            const int r = idx[(size_t)t * K + k];
            if ((unsigned)r < (unsigned)Nr) atomicAdd(&cnt[r], 1);
        }
    }
    __syncthreads();
    for (int r = threadIdx.x; r < Nr; r += 256) hist[(size_t)blockIdx.x * Nr + r] = cnt[r];
}

__global__ __launch_bounds__(1024) void perm_scan_kernel(int nblk, int Nr,
                                                         const int32_t *__restrict__ hist,
                                                         int32_t *__restrict__ base,
                                                         int32_t *__restrict__ offsets) {
    __shared__ int tot[kPermuteMaxExperts];
    const int r = threadIdx.x;
    int total = 0;
    if (r < Nr)
        for (int b = 0; b < nblk; ++b) total += hist[(size_t)b * Nr + r];
    tot[r] = total;
    __syncthreads();
    // inclusive Hillis-Steele scan over the (<= 1024) expert totals
    for (int o = 1; o < 1024; o <<= 1) {
        const int v = r >= o ? tot[r - o] : 0;
        __syncthreads();
        tot[r] += v;
        __syncthreads();
    }
    const int excl = tot[r] - total;
    if (r < Nr) {
        offsets[r] = excl;
        int run = excl;
        for (int b = 0; b < nblk; ++b) {
            base[(size_t)b * Nr + r] = run;
            run += hist[(size_t)b * Nr + r];
        }
    }
    if (r == 0) offsets[Nr] = tot[1023];
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(int T, int Nr, int K,
                                                           const int32_t *__restrict__ idx,
                                                           const int32_t *__restrict__ base,
                                                           int32_t *__restrict__ sorted_token,
                                                           int32_t *__restrict__ slot_of) {
    __shared__ unsigned long long mask[4][kPermuteMaxExperts];
    for (int i = threadIdx.x; i < 4 * Nr; i += 256) mask[i / Nr][i % Nr] = 0ull;
    __syncthreads();
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int t = blockIdx.x * kPermuteTokens + threadIdx.x;
    const bool live = t < T;
    if (live)
        for (int k = 0; k < K; ++k) {
            const int r = idx[(size_t)t * K + k];
            if ((unsigned)r < (unsigned)Nr) atomicOr(&mask[wave][r], 1ull << lane);
        }
    __syncthreads();
    if (!live) return;
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int k = 0; k < K; ++k) {
        const int r = idx[(size_t)t * K + k];
        if ((unsigned)r >= (unsigned)Nr) {
            slot_of[(size_t)t * K + k] = -1;
            continue;
        }
        int rank = __popcll(mask[wave][r] & below);
        for (int w = 0; w < wave; ++w) rank += __popcll(mask[w][r]);
        const int pos = base[(size_t)blockIdx.x * Nr + r] + rank;
        sorted_token[pos] = t;
        slot_of[(size_t)t * K + k] = pos;
    }
}

__global__ void perm_empty_kernel(int Nr, int32_t *__restrict__ offsets) {
    for (int r = threadIdx.x; r <= Nr; r += blockDim.x) offsets[r] = 0;
}

}  // namespace

hipError_t launch_permute(const moe_problem &p, const int32_t *idx, int32_t *offsets,
                          int32_t *sorted_token, int32_t *slot_of, int32_t *hist, int32_t *base,
                          hipStream_t s) {
    const int nblk = cdiv(p.T, kPermuteTokens);
    if (nblk == 0 || p.top_k == 0 || p.n_routed == 0) {
        perm_empty_kernel<<<1, 256, 0, s>>>(p.n_routed, offsets);
        return hipGetLastError();
    }
    perm_hist_kernel<<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, hist);
    perm_scan_kernel<<<1, 1024, 0, s>>>(nblk, p.n_routed, hist, base, offsets);
    perm_scatter_kernel<<<nblk, 256, 0, s>>>(p.T, p.n_routed, p.top_k, idx, base, sorted_token, slot_of);
    return hipGetLastError();
}

}  // namespace moe
