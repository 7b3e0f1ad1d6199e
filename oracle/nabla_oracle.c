/*
 * nabla_oracle.c -- plain CPU reference of the NABLA hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The product path
 * (the HIP library) never does, and shares no code with it.
 *
 * Source: "NABLA: Neighborhood Adaptive Block-Level Attention" (arXiv 2507.13546),
 *   section 2.1 eq. (2)-(3)       dense attention,
 *   section 2.2 eq. (4)-(5)       masked (sliding-tile) attention and its block count,
 *   section 3.1.2, Algorithm 1    the block mask (pooling, reduced softmax, CDF),
 *   section 3.1.3                 the union with the STA mask.
 *
 * Inputs are fp32 arrays holding exactly the values the GPU consumes (bf16
 * widened to fp32). Every sum (pool sums, dot products, softmax denominators,
 * masses) is accumulated in double. Layouts: tensors [BH][S][D] row-major with
 * BH = batch*heads flattened; block maps [BH][n][n] with n = S/N.
 *
 * Readings of points the paper leaves open (each also listed in the design notes):
 *  - Algorithm 1 sorts each row ascending: keeping the entries whose ascending
 *    cumulative sum reaches 1 - thr keeps the largest probabilities, and Table 1
 *    shows a larger thr giving a lower sparsity.
 *  - The ascending cumulative sum at entry j equals 1 - G_ij where G_ij is the
 *    mass of entries strictly larger than entry j (ties counted together), so
 *    "cvals >= 1 - thr" is "G_ij <= thr". thr >= 1 keeps every block.
 *  - The STA window is centred on the query tile and clipped at the grid edges.
 *
 * The attention functions follow eq. (4): keys in dropped blocks get an additive
 * -inf, i.e. contribute exp(-inf) = 0; the loops therefore visit kept blocks
 * only ("blocked" form) and use a two-pass softmax (maximum first, then sums).
 */

#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

EXPORT int nabla_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Algorithm 1, steps 2-5: reshape to [h, S/N, N, D] and average over the N
 * tokens of each block. out[bh][i][d] = (1/N) * sum_r x[bh][i*N + r][d]. */
EXPORT void nabla_oracle_pool(const float* x, int64_t BH, int64_t S, int64_t D, int64_t N,
                              double* out) {
    const int64_t n = S / N;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t i = 0; i < n; ++i) {
            for (int64_t d = 0; d < D; ++d) {
                double s = 0.0;
                for (int64_t r = 0; r < N; ++r)
                    s += (double)x[(bh * S + i * N + r) * D + d];
                out[(bh * n + i) * D + d] = s / (double)N;
            }
        }
    }
}

/* Algorithm 1, steps 6-7: A = softmax(Q_a K_a^T * scale) along the last
 * dimension; the paper's scale is 1/sqrt(D) (eq. (2)). a is [BH][n][n]. */
EXPORT void nabla_oracle_reduced_map(const double* qa, const double* ka, int64_t BH, int64_t n,
                                     int64_t D, double scale, double* a) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t i = 0; i < n; ++i) {
            const double* qi = qa + (bh * n + i) * D;
            double* row = a + (bh * n + i) * n;
            double m = -INFINITY;
            for (int64_t j = 0; j < n; ++j) {
                const double* kj = ka + (bh * n + j) * D;
                double dot = 0.0;
                for (int64_t d = 0; d < D; ++d) dot += qi[d] * kj[d];
                row[j] = dot * scale;
                if (row[j] > m) m = row[j];
            }
            double z = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                row[j] = exp(row[j] - m);
                z += row[j];
            }
            for (int64_t j = 0; j < n; ++j) row[j] /= z;
        }
    }
}

/* Algorithm 1, steps 8-11 rewritten without the sort: for every entry j of a
 * row, G_ij = sum of the row's entries strictly larger than entry j. With an
 * ascending sort the cumulative sum at j's sorted position is 1 - G_ij (equal
 * entries counted together), so the binarisation keeps j iff G_ij <= thr.
 * g is [BH][n][n]. Quadratic per row: the plain definition, no cleverness. */
EXPORT void nabla_oracle_mass_above(const double* a, int64_t BH, int64_t n, double* g) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t i = 0; i < n; ++i) {
            const double* row = a + (bh * n + i) * n;
            double* grow = g + (bh * n + i) * n;
            for (int64_t j = 0; j < n; ++j) {
                const double pj = row[j];
                double s = 0.0;
                for (int64_t l = 0; l < n; ++l)
                    if (row[l] > pj) s += row[l];
                grow[j] = s;
            }
        }
    }
}

/* Top-k selector, the fixed-budget alternative the CDF rule is compared with
 * (review record of arXiv 2507.13546, comment on Appendix C, Theorem 1): for
 * every entry j of a row, c[j] = number of entries of the same row strictly
 * larger than a[j]. Keeping j iff c[j] < k keeps the k largest entries, with
 * entries tied at the k-th value kept together (the same tie rule as G). */
EXPORT void nabla_oracle_count_above(const double* a, int64_t BH, int64_t n, int64_t* c) {
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t i = 0; i < n; ++i) {
            const double* row = a + (bh * n + i) * n;
            int64_t* crow = c + (bh * n + i) * n;
            for (int64_t j = 0; j < n; ++j) {
                int64_t cnt = 0;
                for (int64_t l = 0; l < n; ++l) cnt += row[l] > row[j];
                crow[j] = cnt;
            }
        }
    }
}

/* Binarisation (Algorithm 1, step 10 in the G form): keep iff thr >= 1 or
 * G <= thr. count = number of entries of g and m. */
EXPORT void nabla_oracle_cdf_mask(const double* g, int64_t count, double thr, uint8_t* m) {
    const int keep_all = thr >= 1.0;
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < count; ++e) m[e] = (uint8_t)(keep_all || g[e] <= thr);
}

/* Number of tile coordinates c' in [c - lo, c + hi] clipped to [0, L). */
static int64_t clipped_lo(int64_t c, int64_t w) { int64_t v = c - (w - 1) / 2; return v < 0 ? 0 : v; }
static int64_t clipped_hi(int64_t c, int64_t w, int64_t L) { int64_t v = c + w / 2; return v > L - 1 ? L - 1 : v; }

/* STA mask (section 2.2, eq. (4); STA_mask(T, H, W, W_T, W_H, W_W) of section
 * 3.1.3). Tiles are (1 frame) x P x P tokens, i.e. one block each; block
 * i sits at tile coordinates (t, y, x) = (i / (tH*tW), (i / tW) % tH, i % tW).
 * The window in tiles is (win_t, win_h/P, win_w/P), centred on the query tile
 * (lo = (w-1)/2 below, hi = w/2 above) and clipped at the grid edges.
 * m is [n][n], n = T * (Hs/P) * (Ws/P). */
EXPORT void nabla_oracle_sta_mask(int64_t T, int64_t Hs, int64_t Ws, int64_t P, int64_t win_t,
                                  int64_t win_h, int64_t win_w, uint8_t* m) {
    const int64_t tH = Hs / P, tW = Ws / P, n = T * tH * tW;
    const int64_t wt = win_t, wh = win_h / P, ww = win_w / P;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const int64_t ti = i / (tH * tW), yi = (i / tW) % tH, xi = i % tW;
        for (int64_t j = 0; j < n; ++j) {
            const int64_t tj = j / (tH * tW), yj = (j / tW) % tH, xj = j % tW;
            const int in_t = tj >= clipped_lo(ti, wt) && tj <= clipped_hi(ti, wt, T);
            const int in_h = yj >= clipped_lo(yi, wh) && yj <= clipped_hi(yi, wh, tH);
            const int in_w = xj >= clipped_lo(xi, ww) && xj <= clipped_hi(xi, ww, tW);
            m[i * n + j] = (uint8_t)(in_t && in_h && in_w);
        }
    }
}

/* Section 3.1.3: M = M_nabla OR M_STA, the STA map [n][n] applied to every head. */
EXPORT void nabla_oracle_union(uint8_t* m, const uint8_t* sta, int64_t BH, int64_t n) {
#pragma omp parallel for schedule(static)
    for (int64_t e = 0; e < BH * n * n; ++e) m[e] = (uint8_t)(m[e] | sta[e % (n * n)]);
}

/* Mask-fidelity diagnostic (review record of arXiv 2507.13546 on pith.science:
 * the referee's per-block fidelity test and the skeptic's falsifier). True block
 * mass of full (dense) attention: for query block i and key block j,
 *   M_ij = (1/N) * sum over tokens s of block i, u of block j of P_su,
 *   P_su = exp(x_su - m_s) / sum_{u'} exp(x_su' - m_s),  x_su = scale * q_s . k_u,
 * the softmax running over ALL S keys (eq. (2)). Each row of M sums to 1.
 * blocks lists flattened query blocks (bh*n + i) to compute (NULL = all);
 * m is [BH][n][n] and only the listed rows are written. */
EXPORT void nabla_oracle_block_mass(const float* q, const float* k, int64_t BH, int64_t S,
                                    int64_t D, int64_t N, double scale, const int64_t* blocks,
                                    int64_t nblocks, double* m) {
    const int64_t n = S / N;
    const int64_t total = blocks ? nblocks : BH * n;
#pragma omp parallel
    {
        double* x = (double*)malloc(sizeof(double) * S);
        double* row = (double*)malloc(sizeof(double) * n);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            const int64_t blk = blocks ? blocks[t] : t;
            const int64_t bh = blk / n, i = blk % n;
            for (int64_t j = 0; j < n; ++j) row[j] = 0.0;
            for (int64_t r = 0; r < N; ++r) {
                const float* qs = q + (bh * S + i * N + r) * D;
                double mx = -INFINITY;
                for (int64_t u = 0; u < S; ++u) {
                    const float* ku = k + (bh * S + u) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += (double)qs[d] * (double)ku[d];
                    x[u] = scale * dot;
                    if (x[u] > mx) mx = x[u];
                }
                double z = 0.0;
                for (int64_t u = 0; u < S; ++u) {
                    x[u] = exp(x[u] - mx);
                    z += x[u];
                }
                for (int64_t j = 0; j < n; ++j) {
                    double sj = 0.0;
                    for (int64_t c = 0; c < N; ++c) sj += x[j * N + c];
                    row[j] += sj / z;
                }
            }
            for (int64_t j = 0; j < n; ++j) m[(bh * n + i) * n + j] = row[j] / (double)N;
        }
        free(x);
        free(row);
    }
}

/* Kept keys of query block i: the tokens of every block j with mask[i][j]. */
static int64_t kept_keys(const uint8_t* mrow, int64_t n, int64_t N, int64_t* keys) {
    int64_t c = 0;
    for (int64_t j = 0; j < n; ++j)
        if (mrow[j])
            for (int64_t r = 0; r < N; ++r) keys[c++] = j * N + r;
    return c;
}

/* Masked attention, eq. (4) with the block mask expanded to tokens:
 * for each token s of query block i,
 *   x_su   = scale * q_s . k_u   over kept keys u,
 *   O_s    = sum_u exp(x_su - m_s) v_u / sum_u exp(x_su - m_s),
 *   LSE_s  = m_s + log sum_u exp(x_su - m_s),   m_s = max_u x_su.
 * blocks lists flattened query blocks (bh*n + i) to compute (NULL = all).
 * o is [BH][S][D] and lse [BH][S]; only the listed rows are written. */
EXPORT void nabla_oracle_attn_fwd(const float* q, const float* k, const float* v, int64_t BH,
                                  int64_t S, int64_t D, int64_t N, const uint8_t* mask,
                                  double scale, const int64_t* blocks, int64_t nblocks,
                                  double* o, double* lse) {
    const int64_t n = S / N;
    const int64_t total = blocks ? nblocks : BH * n;
#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * S);
        double* x = (double*)malloc(sizeof(double) * S);
        double* acc = (double*)malloc(sizeof(double) * D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            const int64_t blk = blocks ? blocks[t] : t;
            const int64_t bh = blk / n, i = blk % n;
            const int64_t nk = kept_keys(mask + (bh * n + i) * n, n, N, keys);
            for (int64_t r = 0; r < N; ++r) {
                const int64_t s = i * N + r;
                const float* qs = q + (bh * S + s) * D;
                double m = -INFINITY;
                for (int64_t c = 0; c < nk; ++c) {
                    const float* ku = k + (bh * S + keys[c]) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += (double)qs[d] * (double)ku[d];
                    x[c] = scale * dot;
                    if (x[c] > m) m = x[c];
                }
                double z = 0.0;
                for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
                for (int64_t c = 0; c < nk; ++c) {
                    const double e = exp(x[c] - m);
                    const float* vu = v + (bh * S + keys[c]) * D;
                    z += e;
                    for (int64_t d = 0; d < D; ++d) acc[d] += e * (double)vu[d];
                }
                double* os = o + (bh * S + s) * D;
                for (int64_t d = 0; d < D; ++d) os[d] = acc[d] / z;
                lse[bh * S + s] = m + log(z);
            }
        }
        free(keys);
        free(x);
        free(acc);
    }
}

/* Row statistics of token s over its kept keys: probabilities P_su (into p),
 * and Delta_s = sum_u P_su * (dO_s . v_u), which equals dO_s . O_s. */
static void row_probs(const float* qs, const float* dos, const float* kbh, const float* vbh,
                      const int64_t* keys, int64_t nk, int64_t D, double scale, double* p,
                      double* dp, double* delta) {
    double m = -INFINITY;
    for (int64_t c = 0; c < nk; ++c) {
        const float* ku = kbh + keys[c] * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)qs[d] * (double)ku[d];
        p[c] = scale * dot;
        if (p[c] > m) m = p[c];
    }
    double z = 0.0;
    for (int64_t c = 0; c < nk; ++c) {
        p[c] = exp(p[c] - m);
        z += p[c];
    }
    double dl = 0.0;
    for (int64_t c = 0; c < nk; ++c) {
        p[c] /= z;
        const float* vu = vbh + keys[c] * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += (double)dos[d] * (double)vu[d];
        dp[c] = dot;
        dl += p[c] * dot;
    }
    *delta = dl;
}

/* Gradient of eq. (4) with respect to Q, the mask held constant (it is a
 * piecewise-constant function of Q and K and passes no gradient):
 *   dP_su = dO_s . v_u,  dS_su = P_su (dP_su - Delta_s),
 *   dQ_s  = scale * sum_u dS_su k_u.
 * blocks lists flattened query blocks (NULL = all); only their rows of dq are written. */
EXPORT void nabla_oracle_attn_bwd_dq(const float* q, const float* k, const float* v,
                                     const float* dout, int64_t BH, int64_t S, int64_t D,
                                     int64_t N, const uint8_t* mask, double scale,
                                     const int64_t* blocks, int64_t nblocks, double* dq) {
    const int64_t n = S / N;
    const int64_t total = blocks ? nblocks : BH * n;
#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * S);
        double* p = (double*)malloc(sizeof(double) * S);
        double* dp = (double*)malloc(sizeof(double) * S);
#pragma omp for schedule(dynamic, 1)
        for (int64_t t = 0; t < total; ++t) {
            const int64_t blk = blocks ? blocks[t] : t;
            const int64_t bh = blk / n, i = blk % n;
            const int64_t nk = kept_keys(mask + (bh * n + i) * n, n, N, keys);
            const float* kbh = k + bh * S * D;
            const float* vbh = v + bh * S * D;
            for (int64_t r = 0; r < N; ++r) {
                const int64_t s = i * N + r;
                double delta;
                row_probs(q + (bh * S + s) * D, dout + (bh * S + s) * D, kbh, vbh, keys, nk, D,
                          scale, p, dp, &delta);
                double* dqs = dq + (bh * S + s) * D;
                for (int64_t d = 0; d < D; ++d) dqs[d] = 0.0;
                for (int64_t c = 0; c < nk; ++c) {
                    const double ds = p[c] * (dp[c] - delta);
                    const float* ku = kbh + keys[c] * D;
                    for (int64_t d = 0; d < D; ++d) dqs[d] += scale * ds * (double)ku[d];
                }
            }
        }
        free(keys);
        free(p);
        free(dp);
    }
}

/* Gradients with respect to K and V, the mask held constant:
 *   dV_u = sum_s P_su dO_s,   dK_u = scale * sum_s dS_su q_s,
 * the sums over every token s whose query block keeps u's block.
 * First pass: for every query row s that keeps one of the listed key blocks,
 * its softmax statistics over all its kept keys -- maximum m_s, denominator
 * Z_s -- and Delta_s = sum_u P_su (dO_s . v_u). Second pass: for each listed
 * key block, P_su = exp(x_su - m_s) / Z_s and dS_su for its keys u only.
 * kv_blocks lists flattened key blocks (bh*n + j) (NULL = all); only their
 * rows of dk and dv are written. */
EXPORT void nabla_oracle_attn_bwd_dkdv(const float* q, const float* k, const float* v,
                                       const float* dout, int64_t BH, int64_t S, int64_t D,
                                       int64_t N, const uint8_t* mask, double scale,
                                       const int64_t* kv_blocks, int64_t nblocks, double* dk,
                                       double* dv) {
    const int64_t n = S / N;
    const int64_t total = kv_blocks ? nblocks : BH * n;
    /* query blocks whose row statistics are needed */
    uint8_t* need = (uint8_t*)calloc((size_t)(BH * n), 1);
    double* rm = (double*)malloc(sizeof(double) * BH * S);
    double* rz = (double*)malloc(sizeof(double) * BH * S);
    double* rdelta = (double*)malloc(sizeof(double) * BH * S);
    for (int64_t t = 0; t < total; ++t) {
        const int64_t blk = kv_blocks ? kv_blocks[t] : t;
        const int64_t bh = blk / n, j = blk % n;
        for (int64_t i = 0; i < n; ++i)
            if (mask[(bh * n + i) * n + j]) need[bh * n + i] = 1;
    }
#pragma omp parallel
    {
        int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * S);
        double* x = (double*)malloc(sizeof(double) * S);
#pragma omp for collapse(2) schedule(dynamic, 4)
        for (int64_t qb = 0; qb < BH * n; ++qb) {
            for (int64_t r = 0; r < N; ++r) {
                if (!need[qb]) continue;
                const int64_t bh = qb / n, i = qb % n;
                const int64_t nk = kept_keys(mask + qb * n, n, N, keys);
                const int64_t s = i * N + r;
                const float* qs = q + (bh * S + s) * D;
                const float* dos = dout + (bh * S + s) * D;
                double m = -INFINITY;
                for (int64_t c = 0; c < nk; ++c) {
                    const float* ku = k + (bh * S + keys[c]) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += (double)qs[d] * (double)ku[d];
                    x[c] = scale * dot;
                    if (x[c] > m) m = x[c];
                }
                double z = 0.0;
                for (int64_t c = 0; c < nk; ++c) {
                    x[c] = exp(x[c] - m);
                    z += x[c];
                }
                double dl = 0.0;
                for (int64_t c = 0; c < nk; ++c) {
                    const float* vu = v + (bh * S + keys[c]) * D;
                    double dot = 0.0;
                    for (int64_t d = 0; d < D; ++d) dot += (double)dos[d] * (double)vu[d];
                    dl += (x[c] / z) * dot;
                }
                rm[bh * S + s] = m;
                rz[bh * S + s] = z;
                rdelta[bh * S + s] = dl;
            }
        }
        free(keys);
        free(x);
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < total; ++t) {
        const int64_t blk = kv_blocks ? kv_blocks[t] : t;
        const int64_t bh = blk / n, j = blk % n;
        for (int64_t r = 0; r < N; ++r) {
            double* dku = dk + (bh * S + j * N + r) * D;
            double* dvu = dv + (bh * S + j * N + r) * D;
            for (int64_t d = 0; d < D; ++d) dku[d] = dvu[d] = 0.0;
        }
        for (int64_t i = 0; i < n; ++i) {
            if (!mask[(bh * n + i) * n + j]) continue;
            for (int64_t rq = 0; rq < N; ++rq) {
                const int64_t s = i * N + rq;
                const float* qs = q + (bh * S + s) * D;
                const float* dos = dout + (bh * S + s) * D;
                for (int64_t r = 0; r < N; ++r) {
                    const int64_t u = j * N + r;
                    const float* ku = k + (bh * S + u) * D;
                    const float* vu = v + (bh * S + u) * D;
                    double xs = 0.0, dp = 0.0;
                    for (int64_t d = 0; d < D; ++d) {
                        xs += (double)qs[d] * (double)ku[d];
                        dp += (double)dos[d] * (double)vu[d];
                    }
                    const double p = exp(scale * xs - rm[bh * S + s]) / rz[bh * S + s];
                    const double ds = p * (dp - rdelta[bh * S + s]);
                    double* dku = dk + (bh * S + u) * D;
                    double* dvu = dv + (bh * S + u) * D;
                    for (int64_t d = 0; d < D; ++d) {
                        dvu[d] += p * (double)dos[d];
                        dku[d] += scale * ds * (double)qs[d];
                    }
                }
            }
        }
    }
    free(need);
    free(rm);
    free(rz);
    free(rdelta);
}
