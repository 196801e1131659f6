/*
 * moe_oracle.c -- plain, slow CPU oracle of the DeepSeekMoE layer forward and
 * its backward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the HIP path is
 * compared against.  Only the tests, the smoke check and the benchmark's CPU
 * baseline may load it; the product path never calls it, and it shares no
 * code, header or constant with the HIP library.
 *
 * Sources (web pages about DeepSeekMoE, arXiv 2401.06066):
 *   [S]  "[ACL 2024] DeepSeekMoE: 混合专家语言模型中的极致专家特化" (blog
 *        summary): section "Two core strategies" (fine-grained segmentation,
 *        shared-expert isolation), section "Method details: formulas and load
 *        balance" (layer output h_t, Top-k gates, shared isolation rule,
 *        expert-level and device-level balance losses).
 *   [N]  "【论文总结】MoE" (paper notes): section 2.2 (expert centroids e_i used
 *        for token affinity), section 2.3 (symbols of the expert-level balance
 *        loss: T, N', K', indicator; why the factor N'/K'), section 2.4
 *        (device-level terms: f'_i average usage frequency of a device's
 *        experts, P'_i affinity of the device's experts).
 *   [C]  DeepSeekMoE concept page, section "技術原理" (generic MoE: gate =
 *        linear + softmax, output = weighted sum of the selected experts).
 *
 * Precision.  Only the routing *decision* (which experts a token selects)
 * is made in fp32: the logit z_{t,r} = u_t . e_r is one fmaf chain over k in
 * ascending order (plus one fp32 add of the optional bias), the convention
 * the GPU route kernel also follows, so indices can be compared bit for bit.
 * Everything else (softmax, expert FFNs, the weighted sum, statistics) is
 * computed in fp64 straight from the definitions.
 *
 * Readings of the pages taken here (the pages leave these open):
 *   - gates are the softmax affinities of the selected experts, with no
 *     renormalisation over the Top-K (the softmax is the normalisation);
 *   - the softmax runs over the N' routed experts only;
 *   - ties in z go to the lower expert index; -0.0 == +0.0;
 *   - each expert FFN is SwiGLU without biases: W2 (SiLU(W1 u) * (W3 u));
 *   - f_i = N'/(K'T) * #{t : t selects i};  P_i = mean_t s_{i,t};
 *   - device groups are D contiguous equal blocks of routed experts;
 *     f'_g = mean of f over the group, P'_g = sum of P over the group;
 *   - ExpBal = sum_i f_i P_i, DevBal = sum_g f'_g P'_g (alpha_1, alpha_2 are
 *     not applied);  T = 0 gives f = P = 0.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------
 * Token-to-expert affinity logits, [N] section 2.2 / [S] "Method details":
 * z_{t,r} = u_t . e_r, accumulated as acc = fmaf(u[k], e[k], acc) for
 * k = 0 .. d-1 in order, starting from +0.0f; then z += bias_r (one fp32
 * add) when a bias is given.
 * ---------------------------------------------------------------------- */
void oracle_logits(int T, int d, int Nr, const float *x, const float *E,
                   const float *bias, float *z) {
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int r = 0; r < Nr; ++r) {
            float acc = 0.0f;
            for (int k = 0; k < d; ++k)
                acc = fmaf(x[(size_t)t * d + k], E[(size_t)r * d + k], acc);
            if (bias) acc = acc + bias[r];
            z[(size_t)t * Nr + r] = acc;
        }
    }
}

/* 1 if expert a ranks before expert b: larger logit first, lower index on ties. */
static int ranks_before(float za, int a, float zb, int b) {
    if (za > zb) return 1;
    if (za < zb) return 0;
    return a < b;
}

/* ------------------------------------------------------------------------
 * Routing for T tokens, [S] "Method details" (gates from Top-k of the
 * affinities s_{j,t}; only routed experts are selected) and [C] (linear +
 * softmax gate):
 *   s_{t,r} = exp(z_{t,r}) / sum_j exp(z_{t,j})    over routed experts, fp64
 *   idx[t, 0..K-1] = the K routed experts in order (z desc, r asc)
 *   gate[t,k] = (float) s_{t, idx[t,k]}
 *   probs[t,r] = (float) s_{t,r}              (optional, may be NULL)
 *   counts[r]  = #{t : r in idx[t,:]}
 *   prob_sum[r] = sum_t s_{t,r}               (fp64)
 * Selection uses z: softmax is strictly increasing in z, so Top-K of s and of
 * z are the same set, and the order does not depend on how exp is computed.
 * ---------------------------------------------------------------------- */
void oracle_route(int T, int d, int Nr, int K, const float *x, const float *E,
                  const float *bias, int32_t *idx, float *gate, float *probs,
                  int32_t *counts, double *prob_sum) {
    float *z = (float *)malloc((size_t)(T > 0 ? T : 1) * (Nr > 0 ? Nr : 1) * sizeof(float));
    double *s = (double *)malloc((size_t)(T > 0 ? T : 1) * (Nr > 0 ? Nr : 1) * sizeof(double));
    oracle_logits(T, d, Nr, x, E, bias, z);

    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *zt = z + (size_t)t * Nr;
        double *st = s + (size_t)t * Nr;
        double m = -INFINITY;
        for (int r = 0; r < Nr; ++r) if ((double)zt[r] > m) m = (double)zt[r];
        double sum = 0.0;
        for (int r = 0; r < Nr; ++r) { st[r] = exp((double)zt[r] - m); sum += st[r]; }
        for (int r = 0; r < Nr; ++r) st[r] = st[r] / sum;
        if (probs) for (int r = 0; r < Nr; ++r) probs[(size_t)t * Nr + r] = (float)st[r];

        /* selection by repeated best-of-remaining: plain and obviously ordered */
        unsigned char *taken = (unsigned char *)calloc((size_t)Nr, 1);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int r = 0; r < Nr; ++r) {
                if (taken[r]) continue;
                if (best < 0 || ranks_before(zt[r], r, zt[best], best)) best = r;
            }
            taken[best] = 1;
            idx[(size_t)t * K + k] = best;
            gate[(size_t)t * K + k] = (float)st[best];
        }
        free(taken);
    }

    for (int r = 0; r < Nr; ++r) { counts[r] = 0; prob_sum[r] = 0.0; }
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) counts[idx[(size_t)t * K + k]] += 1;
        for (int r = 0; r < Nr; ++r) prob_sum[r] += s[(size_t)t * Nr + r];
    }
    free(z);
    free(s);
}

/* ------------------------------------------------------------------------
 * Routing variants of the ablations on [S] "Expert specialization analysis"
 * (Fig. 4: disabling the top routed experts) and the baselines of [S]
 * "Experiment design" (Hash Layer's fixed hash routing; Switch's top-1 and
 * GShard's top-2 are oracle_route with K' = 1, 2).
 *
 * oracle_route_ablate: as oracle_route, but each token's `skip` highest
 * ranked routed experts (order z desc, r asc) are disabled and the token
 * takes the next K: idx[t, 0..K-1] = ranks skip .. skip+K-1.  Affinities,
 * gates (no renormalisation) and prob_sum are those of oracle_route.
 * ---------------------------------------------------------------------- */
void oracle_route_ablate(int T, int d, int Nr, int K, int skip, const float *x, const float *E,
                         const float *bias, int32_t *idx, float *gate, float *probs,
                         int32_t *counts, double *prob_sum) {
    float *z = (float *)malloc((size_t)(T > 0 ? T : 1) * (Nr > 0 ? Nr : 1) * sizeof(float));
    double *s = (double *)malloc((size_t)(T > 0 ? T : 1) * (Nr > 0 ? Nr : 1) * sizeof(double));
    oracle_logits(T, d, Nr, x, E, bias, z);
    #pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const float *zt = z + (size_t)t * Nr;
        double *st = s + (size_t)t * Nr;
        double m = -INFINITY;
        for (int r = 0; r < Nr; ++r) if ((double)zt[r] > m) m = (double)zt[r];
        double sum = 0.0;
        for (int r = 0; r < Nr; ++r) { st[r] = exp((double)zt[r] - m); sum += st[r]; }
        for (int r = 0; r < Nr; ++r) st[r] = st[r] / sum;
        if (probs) for (int r = 0; r < Nr; ++r) probs[(size_t)t * Nr + r] = (float)st[r];
        unsigned char *taken = (unsigned char *)calloc((size_t)Nr, 1);
        for (int k = 0; k < skip + K; ++k) {
            int best = -1;
            for (int r = 0; r < Nr; ++r) {
                if (taken[r]) continue;
                if (best < 0 || ranks_before(zt[r], r, zt[best], best)) best = r;
            }
            taken[best] = 1;
            if (k < skip) continue;   /* disabled */
            idx[(size_t)t * K + (k - skip)] = best;
            gate[(size_t)t * K + (k - skip)] = (float)st[best];
        }
        free(taken);
    }
    for (int r = 0; r < Nr; ++r) { counts[r] = 0; prob_sum[r] = 0.0; }
    for (int t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) counts[idx[(size_t)t * K + k]] += 1;
        for (int r = 0; r < Nr; ++r) prob_sum[r] += s[(size_t)t * Nr + r];
    }
    free(z);
    free(s);
}

/* oracle_route_hash: one expert per token from a fixed hash of its token id
 * (the Hash Layer baseline), gate 1:
 *   h = (uint32) id * 2654435761 (mod 2^32)   (Knuth's multiplicative hash)
 *   idx[t] = floor(h * N' / 2^32)              (multiply-shift range reduction)
 *   counts[r] = #{t : idx[t] = r}                                          */
void oracle_route_hash(int T, int Nr, const int32_t *token_ids, int32_t *idx, float *gate,
                       int32_t *counts) {
    for (int r = 0; r < Nr; ++r) counts[r] = 0;
    for (int t = 0; t < T; ++t) {
        const uint32_t h = (uint32_t)token_ids[t] * 2654435761u;
        const int r = (int)(((uint64_t)h * (uint64_t)Nr) >> 32);
        idx[t] = r;
        gate[t] = 1.0f;
        counts[r] += 1;
    }
}

/* ------------------------------------------------------------------------
 * Grouping of (token, expert) pairs by routed expert, the bookkeeping behind
 * "token t selects expert i" ([N] section 2.3).  A counting sort:
 *   offsets[r] = sum_{r' < r} counts[r'],  offsets[Nr] = T*K
 *   sorted_token lists, for r ascending, the tokens t ascending that chose r
 *   slot_of[t*K + k] = position of pair (t, idx[t,k]) in sorted_token
 * Returns 0, or -1 if an index is out of range or repeated within a token.
 * ---------------------------------------------------------------------- */
int oracle_permute(int T, int Nr, int K, const int32_t *idx, int32_t *offsets,
                   int32_t *sorted_token, int32_t *slot_of) {
    int64_t *fill = (int64_t *)calloc((size_t)Nr + 1, sizeof(int64_t));
    int64_t *cnt = (int64_t *)calloc((size_t)Nr + 1, sizeof(int64_t));
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int r = idx[(size_t)t * K + k];
            if (r < 0 || r >= Nr) { free(fill); free(cnt); return -1; }
            for (int k2 = 0; k2 < k; ++k2)
                if (idx[(size_t)t * K + k2] == r) { free(fill); free(cnt); return -1; }
            cnt[r] += 1;
        }
    int64_t run = 0;
    for (int r = 0; r < Nr; ++r) { offsets[r] = (int32_t)run; run += cnt[r]; }
    offsets[Nr] = (int32_t)run;
    for (int t = 0; t < T; ++t)
        for (int k = 0; k < K; ++k) {
            int r = idx[(size_t)t * K + k];
            int64_t pos = offsets[r] + fill[r]++;
            sorted_token[pos] = t;
            slot_of[(size_t)t * K + k] = (int32_t)pos;
        }
    free(fill);
    free(cnt);
    return 0;
}

/* ------------------------------------------------------------------------
 * One expert FFN on one token ("each expert is an independent FFN", [C];
 * SwiGLU form, no biases), fp64:
 *   p_j = sum_k W1[j,k] u_k,  q_j = sum_k W3[j,k] u_k      (j < w)
 *   a_j = SiLU(p_j) * q_j,    SiLU(v) = v / (1 + exp(-v))
 *   y_i = sum_j W2[i,j] a_j                                 (i < d)
 * W1, W3 are [w, d] and W2 is [d, w], row-major.  y is accumulated into
 * (y += scale * FFN(u)).
 * ---------------------------------------------------------------------- */
static void expert_ffn_accumulate(int d, int w, const float *u, const float *W1,
                                  const float *W3, const float *W2, double scale,
                                  double *y, double *a /* scratch [w] */) {
    for (int j = 0; j < w; ++j) {
        double p = 0.0, q = 0.0;
        const float *r1 = W1 + (size_t)j * d;
        const float *r3 = W3 + (size_t)j * d;
        for (int k = 0; k < d; ++k) {
            p += (double)r1[k] * (double)u[k];
            q += (double)r3[k] * (double)u[k];
        }
        a[j] = p / (1.0 + exp(-p)) * q;
    }
    for (int i = 0; i < d; ++i) {
        const float *r2 = W2 + (size_t)i * w;
        double acc = 0.0;
        for (int j = 0; j < w; ++j) acc += (double)r2[j] * a[j];
        y[i] += scale * acc;
    }
}

/* Public single-expert FFN (y = FFN(u)), for the special-case tests. */
void oracle_expert_ffn(int d, int w, const float *u, const float *W1,
                       const float *W3, const float *W2, double *y) {
    double *a = (double *)malloc((size_t)(w > 0 ? w : 1) * sizeof(double));
    for (int i = 0; i < d; ++i) y[i] = 0.0;
    expert_ffn_accumulate(d, w, u, W1, W3, W2, 1.0, y, a);
    free(a);
}

/* ------------------------------------------------------------------------
 * Layer output for a list of tokens, [S] "Method details" output formula:
 *   h_t = sum_{i <= K_s} FFN_i(u_t) + sum_{routed} g_{i,t} FFN_i(u_t) + u_t
 * with the first K_s experts shared (always active) and the routed experts
 * weighted by their gates (zero off the Top-K).  For each listed token t
 * (tokens[n]) this writes, in fp64:
 *   y_shared[n, :]    = sum_{e < Ks} FFN_e(u_t)
 *   y_routed[n, k, :] = FFN_{Ks + idx[t,k]}(u_t)   (unweighted, k < K)
 *   y[n, :]           = y_shared + sum_k gate[t,k] * y_routed[n,k]
 *   h[n, :]           = u_t + y[n, :]
 * Any of the four outputs may be NULL.  Shared weights are [Ks, w, d] /
 * [Ks, d, w]; routed weights [Nr, w, d] / [Nr, d, w].
 * ---------------------------------------------------------------------- */
void oracle_layer_tokens(int n_tok, const int32_t *tokens, int d, int Ks, int Nr,
                         int K, int w, const float *x, const int32_t *idx,
                         const float *gate, const float *W1s, const float *W3s,
                         const float *W2s, const float *W1r, const float *W3r,
                         const float *W2r, double *y_shared, double *y_routed,
                         double *y, double *h) {
    (void)Nr;
    const size_t up = (size_t)w * d, down = (size_t)d * w;
    #pragma omp parallel
    {
        double *a = (double *)malloc((size_t)(w > 0 ? w : 1) * sizeof(double));
        double *ys = (double *)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
        double *yk = (double *)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
        double *yt = (double *)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int n = 0; n < n_tok; ++n) {
            const int t = tokens[n];
            const float *u = x + (size_t)t * d;
            for (int i = 0; i < d; ++i) ys[i] = 0.0;
            for (int e = 0; e < Ks; ++e)
                expert_ffn_accumulate(d, w, u, W1s + e * up, W3s + e * up, W2s + e * down, 1.0, ys, a);
            for (int i = 0; i < d; ++i) yt[i] = ys[i];
            for (int k = 0; k < K; ++k) {
                const int r = idx[(size_t)t * K + k];
                for (int i = 0; i < d; ++i) yk[i] = 0.0;
                expert_ffn_accumulate(d, w, u, W1r + r * up, W3r + r * up, W2r + r * down, 1.0, yk, a);
                if (y_routed) memcpy(y_routed + ((size_t)n * K + k) * d, yk, (size_t)d * sizeof(double));
                const double g = (double)gate[(size_t)t * K + k];
                for (int i = 0; i < d; ++i) yt[i] += g * yk[i];
            }
            if (y_shared) memcpy(y_shared + (size_t)n * d, ys, (size_t)d * sizeof(double));
            if (y) memcpy(y + (size_t)n * d, yt, (size_t)d * sizeof(double));
            if (h)
                for (int i = 0; i < d; ++i) h[(size_t)n * d + i] = (double)u[i] + yt[i];
        }
        free(a); free(ys); free(yk); free(yt);
    }
}

/* ------------------------------------------------------------------------
 * Balance statistics, [S] "Method details" (expert-level and device-level
 * balance losses) with the symbols of [N] sections 2.3 and 2.4:
 *   f_r  = N'/(K'T) * counts[r]            (fp64 quotient, rounded to fp32)
 *   P_r  = prob_sum[r] / T                 (mean affinity)
 *   group g = experts [g*N'/D, (g+1)*N'/D)
 *   f'_g = mean_{r in g} f_r = N' * C_g / (K' T (N'/D)),  C_g = sum counts
 *   P'_g = sum_{r in g} P_r
 *   ExpBal = sum_r f_r P_r,  DevBal = sum_g f'_g P'_g   (fp64, then fp32)
 * Returns -1 if D does not divide N' or an argument is out of range.
 * ---------------------------------------------------------------------- */
int oracle_balance_stats(int T, int Nr, int K, int D, const int32_t *counts,
                         const double *prob_sum, float *f, float *P, float *fdev,
                         float *Pdev, float *exp_bal, float *dev_bal) {
    if (Nr <= 0 || K <= 0 || K > Nr || D <= 0 || Nr % D != 0 || T < 0) return -1;
    const int gsz = Nr / D;
    double eb = 0.0, db = 0.0;
    double *Pd = (double *)malloc((size_t)Nr * sizeof(double));
    for (int r = 0; r < Nr; ++r) {
        double fr = T > 0 ? ((double)Nr * (double)counts[r]) / ((double)K * (double)T) : 0.0;
        Pd[r] = T > 0 ? prob_sum[r] / (double)T : 0.0;
        f[r] = (float)fr;
        P[r] = (float)Pd[r];
        eb += (double)f[r] * (double)P[r];
    }
    for (int g = 0; g < D; ++g) {
        int64_t C = 0;
        double Ps = 0.0;
        for (int r = g * gsz; r < (g + 1) * gsz; ++r) { C += counts[r]; Ps += Pd[r]; }
        double fg = T > 0 ? ((double)Nr * (double)C) / ((double)K * (double)T * (double)gsz) : 0.0;
        fdev[g] = (float)fg;
        Pdev[g] = (float)Ps;
        db += (double)fdev[g] * (double)Pdev[g];
    }
    *exp_bal = (float)eb;
    *dev_bal = (float)db;
    free(Pd);
    return 0;
}

/* ------------------------------------------------------------------------
 * The whole layer pass on the first n_tok tokens, as one call: route,
 * group, expert FFNs, weighted sum with residual, statistics.  Used to time
 * the oracle as a CPU baseline; outputs h in fp64 [n_tok, d].
 * ---------------------------------------------------------------------- */
int oracle_forward(int n_tok, int d, int Ks, int Nr, int K, int w, int D,
                   const float *x, const float *E, const float *bias,
                   const float *W1s, const float *W3s, const float *W2s,
                   const float *W1r, const float *W3r, const float *W2r,
                   double *h, float *exp_bal, float *dev_bal) {
    const size_t tk = (size_t)(n_tok > 0 ? n_tok : 1) * (K > 0 ? K : 1);
    int32_t *idx = (int32_t *)calloc(tk, sizeof(int32_t));
    float *gate = (float *)calloc(tk, sizeof(float));
    int32_t *counts = (int32_t *)calloc((size_t)Nr + 1, sizeof(int32_t));
    double *psum = (double *)calloc((size_t)Nr + 1, sizeof(double));
    int32_t *offsets = (int32_t *)malloc(((size_t)Nr + 1) * sizeof(int32_t));
    int32_t *sorted = (int32_t *)malloc(tk * sizeof(int32_t));
    int32_t *slot = (int32_t *)malloc(tk * sizeof(int32_t));
    int32_t *tokens = (int32_t *)malloc((size_t)(n_tok > 0 ? n_tok : 1) * sizeof(int32_t));
    float *f = (float *)malloc(((size_t)Nr + 1) * sizeof(float));
    float *P = (float *)malloc(((size_t)Nr + 1) * sizeof(float));
    float *fd = (float *)malloc(((size_t)D + 1) * sizeof(float));
    float *Pd = (float *)malloc(((size_t)D + 1) * sizeof(float));
    int rc = 0;
    for (int n = 0; n < n_tok; ++n) tokens[n] = n;
    if (Nr > 0) oracle_route(n_tok, d, Nr, K, x, E, bias, idx, gate, NULL, counts, psum);
    if (Nr > 0 && oracle_permute(n_tok, Nr, K, idx, offsets, sorted, slot) != 0) rc = -1;
    if (rc == 0)
        oracle_layer_tokens(n_tok, tokens, d, Ks, Nr, K, w, x, idx, gate, W1s, W3s, W2s,
                            W1r, W3r, W2r, NULL, NULL, NULL, h);
    if (rc == 0 && Nr > 0)
        rc = oracle_balance_stats(n_tok, Nr, K, D, counts, psum, f, P, fd, Pd, exp_bal, dev_bal);
    free(idx); free(gate); free(counts); free(psum); free(offsets); free(sorted);
    free(slot); free(tokens); free(f); free(P); free(fd); free(Pd);
    return rc;
}

/* ========================================================================
 * Backward pass of the layer (training is the setting of [S] "Method
 * details", whose loss adds alpha_1 * ExpBal + alpha_2 * DevBal to the task
 * loss).  Given dh = dL_task/dh [T, d] the gradients follow from the chain
 * rule on the forward definitions above, in fp64:
 *
 *   per used (t, e) with upstream dy (dy = g_{t,k} dh_t for a routed pair,
 *   dy = dh_t for a shared expert):
 *     da_j = sum_i W2[i,j] dy_i
 *     dq_j = da_j SiLU(p_j),  dp_j = da_j q_j sig_j (1 + p_j (1 - sig_j))
 *     dx_t += sum_j W1[j,:] dp_j + W3[j,:] dq_j
 *     dW2 += dy a^T,  dW1 += dp x_t^T,  dW3 += dq x_t^T
 *   routed pair:  dg_{t,k} = dh_t . FFN_e(u_t)
 *   router:  ds_{t,r} = dg_{t,k} (r = idx[t,k]) + alpha_1 f_r / T
 *                       + alpha_2 f'_{group(r)} / T
 *            dz_{t,r} = s_{t,r} (ds_{t,r} - sum_r' s_{t,r'} ds_{t,r'})
 *            dx_t += sum_r dz_{t,r} e_r,  dE_r = sum_t dz_{t,r} u_t,
 *            dbias_r = sum_t dz_{t,r}
 *   plus the residual: dx_t += dh_t.
 *
 * Readings (the pages give the losses, not their gradients): the Top-K
 * selection is held fixed (it is piecewise constant); f and f' are counts
 * of that selection, so they are constants; P and P' are differentiable
 * through the softmax.  The affinities s and gates g are the forward's
 * outputs (probs, gate).
 * ====================================================================== */

/* p, q, a of one expert on one token (fp64). */
static void ffn_hidden(int d, int w, const float *u, const float *W1, const float *W3,
                       double *p, double *q, double *a) {
    for (int j = 0; j < w; ++j) {
        double pj = 0.0, qj = 0.0;
        const float *r1 = W1 + (size_t)j * d, *r3 = W3 + (size_t)j * d;
        for (int k = 0; k < d; ++k) {
            pj += (double)r1[k] * (double)u[k];
            qj += (double)r3[k] * (double)u[k];
        }
        p[j] = pj;
        q[j] = qj;
        a[j] = pj / (1.0 + exp(-pj)) * qj;
    }
}

/* da -> dp, dq (SwiGLU backward). */
static void swiglu_backward(int w, const double *p, const double *q, const double *da,
                            double *dp, double *dq) {
    for (int j = 0; j < w; ++j) {
        const double sg = 1.0 / (1.0 + exp(-p[j]));
        dq[j] = da[j] * p[j] * sg;
        dp[j] = da[j] * q[j] * sg * (1.0 + p[j] * (1.0 - sg));
    }
}

/* da_j = sum_i W2[i,j] dy_i */
static void down_backward(int d, int w, const float *W2, const double *dy, double *da) {
    for (int j = 0; j < w; ++j) da[j] = 0.0;
    for (int i = 0; i < d; ++i) {
        const float *r2 = W2 + (size_t)i * w;
        const double v = dy[i];
        for (int j = 0; j < w; ++j) da[j] += (double)r2[j] * v;
    }
}

/* dx += W1^T dp + W3^T dq */
static void up_backward_dx(int d, int w, const float *W1, const float *W3, const double *dp,
                           const double *dq, double *dx) {
    for (int j = 0; j < w; ++j) {
        const float *r1 = W1 + (size_t)j * d, *r3 = W3 + (size_t)j * d;
        for (int k = 0; k < d; ++k) dx[k] += (double)r1[k] * dp[j] + (double)r3[k] * dq[j];
    }
}

/* ------------------------------------------------------------------------
 * Per-token part of the backward for the listed tokens (tokens[n]):
 *   dgate[n, k]  = dh_t . FFN_{idx[t,k]}(u_t)
 *   dz[n, r]     = router logit gradient (NULL: not written)
 *   dx[n, :]     = dh_t + FFN part + router part
 * T is the whole batch (it scales the balance-loss terms).  groups D
 * divides N'.  f [N'], fdev [D] are the forward's statistics.
 * ---------------------------------------------------------------------- */
void oracle_backward_tokens(int n_tok, const int32_t *tokens, int T, int d, int Ks, int Nr,
                            int K, int w, int D, double alpha1, double alpha2,
                            const float *x, const float *E, const int32_t *idx,
                            const float *gate, const float *probs, const float *f,
                            const float *fdev, const float *W1s, const float *W3s,
                            const float *W2s, const float *W1r, const float *W3r,
                            const float *W2r, const float *dh, double *dgate, double *dz,
                            double *dx) {
    const size_t up = (size_t)w * d, down = (size_t)d * w;
    const int gsz = (Nr > 0 && D > 0) ? Nr / D : 1;
    #pragma omp parallel
    {
        const size_t nw = (size_t)(w > 0 ? w : 1), nd = (size_t)(d > 0 ? d : 1);
        double *p = (double *)malloc(nw * sizeof(double)), *q = (double *)malloc(nw * sizeof(double));
        double *a = (double *)malloc(nw * sizeof(double)), *da = (double *)malloc(nw * sizeof(double));
        double *dp = (double *)malloc(nw * sizeof(double)), *dq = (double *)malloc(nw * sizeof(double));
        double *dy = (double *)malloc(nd * sizeof(double)), *dxt = (double *)malloc(nd * sizeof(double));
        double *ds = (double *)malloc((size_t)(Nr > 0 ? Nr : 1) * sizeof(double));
        #pragma omp for schedule(dynamic, 1)
        for (int n = 0; n < n_tok; ++n) {
            const int t = tokens[n];
            const float *u = x + (size_t)t * d, *g = dh + (size_t)t * d;
            for (int i = 0; i < d; ++i) dxt[i] = (double)g[i];
            for (int e = 0; e < Ks; ++e) {
                for (int i = 0; i < d; ++i) dy[i] = (double)g[i];
                ffn_hidden(d, w, u, W1s + e * up, W3s + e * up, p, q, a);
                down_backward(d, w, W2s + e * down, dy, da);
                swiglu_backward(w, p, q, da, dp, dq);
                up_backward_dx(d, w, W1s + e * up, W3s + e * up, dp, dq, dxt);
            }
            for (int r = 0; r < Nr; ++r) ds[r] = 0.0;
            for (int k = 0; k < K; ++k) {
                const int r = idx[(size_t)t * K + k];
                const float *W1 = W1r + r * up, *W3 = W3r + r * up, *W2 = W2r + r * down;
                ffn_hidden(d, w, u, W1, W3, p, q, a);
                double dgk = 0.0;
                for (int i = 0; i < d; ++i) {
                    double yi = 0.0;
                    const float *r2 = W2 + (size_t)i * w;
                    for (int j = 0; j < w; ++j) yi += (double)r2[j] * a[j];
                    dgk += (double)g[i] * yi;
                }
                if (dgate) dgate[(size_t)n * K + k] = dgk;
                ds[r] += dgk;
                const double gk = (double)gate[(size_t)t * K + k];
                for (int i = 0; i < d; ++i) dy[i] = gk * (double)g[i];
                down_backward(d, w, W2, dy, da);
                swiglu_backward(w, p, q, da, dp, dq);
                up_backward_dx(d, w, W1, W3, dp, dq, dxt);
            }
            if (Nr > 0) {
                double dot = 0.0;
                for (int r = 0; r < Nr; ++r) {
                    ds[r] += alpha1 * (double)f[r] / (double)T + alpha2 * (double)fdev[r / gsz] / (double)T;
                    dot += (double)probs[(size_t)t * Nr + r] * ds[r];
                }
                for (int r = 0; r < Nr; ++r) {
                    const double z = (double)probs[(size_t)t * Nr + r] * (ds[r] - dot);
                    if (dz) dz[(size_t)n * Nr + r] = z;
                    const float *er = E + (size_t)r * d;
                    for (int i = 0; i < d; ++i) dxt[i] += z * (double)er[i];
                }
            }
            if (dx) memcpy(dx + (size_t)n * d, dxt, (size_t)d * sizeof(double));
        }
        free(p); free(q); free(a); free(da); free(dp); free(dq); free(dy); free(dxt); free(ds);
    }
}

/* ------------------------------------------------------------------------
 * Router parameter gradients from the logit gradients of ALL T tokens
 * (dz [T, N'] from oracle_backward_tokens over every token):
 *   dE[r, :] = sum_t dz[t, r] u_t (t ascending),  dbias[r] = sum_t dz[t, r]
 * ---------------------------------------------------------------------- */
void oracle_backward_router(int T, int d, int Nr, const float *x, const double *dz,
                            double *dE, double *dbias) {
    #pragma omp parallel for schedule(static)
    for (int r = 0; r < Nr; ++r) {
        double *er = dE + (size_t)r * d;
        double b = 0.0;
        for (int i = 0; i < d; ++i) er[i] = 0.0;
        for (int t = 0; t < T; ++t) {
            const double z = dz[(size_t)t * Nr + r];
            b += z;
            const float *u = x + (size_t)t * d;
            for (int i = 0; i < d; ++i) er[i] += z * (double)u[i];
        }
        dbias[r] = b;
    }
}

/* ------------------------------------------------------------------------
 * Weight gradients of one expert, selected rows only.  Expert e is global
 * (e < Ks shared, else routed r = e - Ks).  Its tokens: every token for a
 * shared expert (dy = dh_t); the tokens t with idx[t,k] == r for a routed
 * one (dy = gate[t,k] dh_t), t ascending.
 *   dW1[rows1[n], :], dW3[rows1[n], :]   (n < n1; rows of [w, d])
 *   dW2[rows2[n], :]                     (n < n2; rows of [d, w])
 * ---------------------------------------------------------------------- */
void oracle_backward_weight_rows(int e, int T, int d, int Ks, int K, int w, const float *x,
                                 const int32_t *idx, const float *gate, const float *W1s,
                                 const float *W3s, const float *W2s, const float *W1r,
                                 const float *W3r, const float *W2r, const float *dh,
                                 int n1, const int32_t *rows1, double *dW1, double *dW3,
                                 int n2, const int32_t *rows2, double *dW2) {
    const size_t up = (size_t)w * d, down = (size_t)d * w;
    const int sh = e < Ks;
    const int r = e - Ks;
    const float *W1 = sh ? W1s + e * up : W1r + r * up;
    const float *W3 = sh ? W3s + e * up : W3r + r * up;
    const float *W2 = sh ? W2s + e * down : W2r + r * down;
    for (size_t i = 0; i < (size_t)n1 * d; ++i) { dW1[i] = 0.0; dW3[i] = 0.0; }
    for (size_t i = 0; i < (size_t)n2 * w; ++i) dW2[i] = 0.0;
    const size_t nw = (size_t)(w > 0 ? w : 1), nd = (size_t)(d > 0 ? d : 1);
    double *p = (double *)malloc(nw * sizeof(double)), *q = (double *)malloc(nw * sizeof(double));
    double *a = (double *)malloc(nw * sizeof(double)), *da = (double *)malloc(nw * sizeof(double));
    double *dp = (double *)malloc(nw * sizeof(double)), *dq = (double *)malloc(nw * sizeof(double));
    double *dy = (double *)malloc(nd * sizeof(double));
    for (int t = 0; t < T; ++t) {
        double scale;
        if (sh) {
            scale = 1.0;
        } else {
            int kk = -1;
            for (int k = 0; k < K; ++k)
                if (idx[(size_t)t * K + k] == r) kk = k;
            if (kk < 0) continue;
            scale = (double)gate[(size_t)t * K + kk];
        }
        const float *u = x + (size_t)t * d, *g = dh + (size_t)t * d;
        for (int i = 0; i < d; ++i) dy[i] = scale * (double)g[i];
        ffn_hidden(d, w, u, W1, W3, p, q, a);
        down_backward(d, w, W2, dy, da);
        swiglu_backward(w, p, q, da, dp, dq);
        for (int n = 0; n < n1; ++n) {
            const int j = rows1[n];
            for (int k = 0; k < d; ++k) {
                dW1[(size_t)n * d + k] += dp[j] * (double)u[k];
                dW3[(size_t)n * d + k] += dq[j] * (double)u[k];
            }
        }
        for (int n = 0; n < n2; ++n) {
            const double v = dy[rows2[n]];
            for (int j = 0; j < w; ++j) dW2[(size_t)n * w + j] += v * a[j];
        }
    }
    free(p); free(q); free(a); free(da); free(dp); free(dq); free(dy);
}
