/*
 * attn_oracle.c -- plain, slow CPU fp64 implementation of attention forward and
 * backward.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this library.  It shares no code, header
 * or constant with the GPU library, and the GPU library never calls it.
 *
 * Sources (the web pages on the FlashAttention-2 backward):
 *   [FA2-ch16]  "CUDA 算子工程：手写 FlashAttention v2 之路", chapter 16
 *               "FA2 反向：dQ/dK/dV 的重计算":
 *               sec 16.1 (chain rule: dV = P^T dO, dP = dO V^T,
 *               dS = P o (dP - D), D_i = sum_k P_ik dP_ik, dQ = dS K,
 *               dK = dS^T Q, and the identity D_i = dO_i . O_i),
 *               sec 16.2 (K blocks outer, Q blocks inner),
 *               sec 16.4 (LSE_i = m_i + log l_i; P = exp(S - LSE)),
 *               sec 16.6 (dK multiplied by the softmax scale at write-out,
 *               dQ scaled by the convert step),
 *               sec 16.8 items 1-2 (D precomputed from O and dO; whole
 *               tiles above the causal diagonal skipped).
 *   [gsyq]      gsyq.cn, "FlashAttention 的反向传播设计：在 SRAM 内部重计算
 *               Softmax 的显存收益", part 一 (S = Q K^T / sqrt(d);
 *               dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d)).
 *   [1p3a]      1point3acres, "最近准备面试的时候手扒了FlashAttention":
 *               online-softmax recurrence (m, l, a; m', alpha, l', a'),
 *               logsumexp L_i = m_i + log l_i, P_ij = exp(S_ij - L_i),
 *               softmax-backward reduction delta = g . o.
 *   [cs349e]    CS349E lecture 11 "03_flash_backward.py", demo 1
 *               (gradient check, tiles 16 x 12).
 *
 * Conventions (readings of the pages):
 *   - tensors are contiguous [BH, N, d] row-major (d fastest), float64;
 *     L and D are [BH, N];
 *   - s_ij = scale * Q_i . K_j; the softmax and L are over scaled scores;
 *     dQ and dK carry the scale, dV does not ([gsyq] part 一, [FA2-ch16] 16.6);
 *   - causal: key j is visible to query i iff j <= i (0-based, diagonal kept);
 *   - L uses the natural logarithm.
 *
 * Every function works one query row (or one key row) at a time, so no N x N
 * matrix is held.  OpenMP splits rows across threads; per-thread partial dK and
 * dV are summed in thread order, so results are deterministic for a fixed
 * thread count.
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

static double dot(const double* a, const double* b, long d) {
    double s = 0.0;
    for (long k = 0; k < d; ++k) s += a[k] * b[k];
    return s;
}

static long n_visible(long i, long N, int causal) { return causal ? i + 1 : N; }

/* Softmax of one query row over its visible keys, by definition
 * ([FA2-ch16] 16.1; [1p3a]): s_j = scale * q . K_j, m = max_j s_j,
 * l = sum_j exp(s_j - m), P_j = exp(s_j - m) / l.  Writes P_j for the n visible
 * keys into p and returns L = m + log l ([FA2-ch16] 16.4). */
static double row_softmax(const double* q, const double* K, long n, long d,
                          double scale, double* p) {
    double m = -INFINITY;
    for (long j = 0; j < n; ++j) {
        p[j] = scale * dot(q, K + j * d, d);
        if (p[j] > m) m = p[j];
    }
    double l = 0.0;
    for (long j = 0; j < n; ++j) {
        p[j] = exp(p[j] - m);
        l += p[j];
    }
    for (long j = 0; j < n; ++j) p[j] /= l;
    return m + log(l);
}

int orc_max_threads(void) { return omp_get_max_threads(); }
void orc_set_threads(int n) { if (n > 0) omp_set_num_threads(n); }

/* Standard attention forward: O = softmax(scale * Q K^T [+ causal mask]) V, and
 * L_i = m_i + log l_i.  [FA2-ch16] 16.1, [gsyq] part 一, [1p3a] logsumexp. */
void orc_attn_fwd(const double* Q, const double* K, const double* V,
                  long BH, long N, long d, double scale, int causal,
                  double* O, double* L) {
    for (long bh = 0; bh < BH; ++bh) {
        const double* q = Q + bh * N * d;
        const double* k = K + bh * N * d;
        const double* v = V + bh * N * d;
        double* o = O + bh * N * d;
        double* lse = L + bh * N;
#pragma omp parallel
        {
            double* p = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 4)
            for (long i = 0; i < N; ++i) {
                long n = n_visible(i, N, causal);
                lse[i] = row_softmax(q + i * d, k, n, d, scale, p);
                double* oi = o + i * d;
                for (long c = 0; c < d; ++c) oi[c] = 0.0;
                for (long j = 0; j < n; ++j)
                    for (long c = 0; c < d; ++c) oi[c] += p[j] * v[j * d + c];
            }
            free(p);
        }
    }
}

/* Standard attention backward by the chain rule of [FA2-ch16] 16.1:
 *   dV_j = sum_i P_ij dO_i
 *   dP_ij = dO_i . V_j
 *   D_i = sum_j P_ij dP_ij          (the definition, not the O.dO identity)
 *   dS_ij = P_ij (dP_ij - D_i)
 *   dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i  ([gsyq] part 一)
 * P is the softmax of the scaled, masked scores, recomputed per row.
 * D (may be NULL) receives D_i. */
void orc_attn_bwd(const double* Q, const double* K, const double* V,
                  const double* dO, long BH, long N, long d, double scale,
                  int causal, double* dQ, double* dK, double* dV, double* D) {
    int T = omp_get_max_threads();
    double** part = (double**)calloc((size_t)T, sizeof(double*));
    for (long bh = 0; bh < BH; ++bh) {
        const double* q = Q + bh * N * d;
        const double* k = K + bh * N * d;
        const double* v = V + bh * N * d;
        const double* g = dO + bh * N * d;
        double* dq = dQ + bh * N * d;
        double* dk = dK + bh * N * d;
        double* dv = dV + bh * N * d;
        int nt = 1;
#pragma omp parallel
        {
            int t = omp_get_thread_num();
#pragma omp single
            nt = omp_get_num_threads();
            /* private accumulators: [dK | dV], each N x d */
            double* acc = (double*)calloc((size_t)(2 * N * d), sizeof(double));
            double* p = (double*)malloc(sizeof(double) * (size_t)N);
            double* dp = (double*)malloc(sizeof(double) * (size_t)N);
            part[t] = acc;
#pragma omp for schedule(dynamic, 4)
            for (long i = 0; i < N; ++i) {
                long n = n_visible(i, N, causal);
                const double* qi = q + i * d;
                const double* gi = g + i * d;
                row_softmax(qi, k, n, d, scale, p);
                double Di = 0.0;
                for (long j = 0; j < n; ++j) {
                    dp[j] = dot(gi, v + j * d, d);
                    Di += p[j] * dp[j];
                }
                if (D) D[bh * N + i] = Di;
                double* dqi = dq + i * d;
                for (long c = 0; c < d; ++c) dqi[c] = 0.0;
                for (long j = 0; j < n; ++j) {
                    double ds = p[j] * (dp[j] - Di);
                    const double* kj = k + j * d;
                    double* dkj = acc + j * d;
                    double* dvj = acc + N * d + j * d;
                    for (long c = 0; c < d; ++c) {
                        dqi[c] += scale * ds * kj[c];
                        dkj[c] += scale * ds * qi[c];
                        dvj[c] += p[j] * gi[c];
                    }
                }
            }
            /* implicit barrier: every part[] is complete; sum in thread order */
#pragma omp for schedule(static)
            for (long e = 0; e < N * d; ++e) {
                double sk = 0.0, sv = 0.0;
                for (int u = 0; u < nt; ++u) {
                    sk += part[u][e];
                    sv += part[u][N * d + e];
                }
                dk[e] = sk;
                dv[e] = sv;
            }
            free(dp);
            free(p);
#pragma omp barrier
            free(acc);
        }
    }
    free(part);
}

/* ---- sampled outputs for large problems (one head at a time) ------------ */

/* L_i and D_i for every row of one head, each by its definition:
 * L_i = log sum_j exp(s_ij) (as m_i + log l_i), D_i = sum_j P_ij dP_ij. */
void orc_row_stats(const double* Q, const double* K, const double* V,
                   const double* dO, long N, long d, double scale, int causal,
                   double* L, double* D) {
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 8)
        for (long i = 0; i < N; ++i) {
            long n = n_visible(i, N, causal);
            L[i] = row_softmax(Q + i * d, K, n, d, scale, p);
            double Di = 0.0;
            for (long j = 0; j < n; ++j) Di += p[j] * dot(dO + i * d, V + j * d, d);
            D[i] = Di;
        }
        free(p);
    }
}

/* O_i and L_i for selected rows of one head (forward definition). */
void orc_fwd_rows(const double* Q, const double* K, const double* V,
                  long N, long d, double scale, int causal,
                  const long* rows, long nrows, double* O, double* L) {
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            long i = rows[r];
            long n = n_visible(i, N, causal);
            L[r] = row_softmax(Q + i * d, K, n, d, scale, p);
            double* o = O + r * d;
            for (long c = 0; c < d; ++c) o[c] = 0.0;
            for (long j = 0; j < n; ++j)
                for (long c = 0; c < d; ++c) o[c] += p[j] * V[j * d + c];
        }
        free(p);
    }
}

/* dQ_i for selected rows of one head: the whole chain rule restricted to row i
 * (softmax, dP, D_i by definition, dS, dQ_i = scale sum_j dS_ij K_j). */
void orc_dq_rows(const double* Q, const double* K, const double* V,
                 const double* dO, long N, long d, double scale, int causal,
                 const long* rows, long nrows, double* dQ) {
#pragma omp parallel
    {
        double* p = (double*)malloc(sizeof(double) * (size_t)N);
        double* dp = (double*)malloc(sizeof(double) * (size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            long i = rows[r];
            long n = n_visible(i, N, causal);
            row_softmax(Q + i * d, K, n, d, scale, p);
            double Di = 0.0;
            for (long j = 0; j < n; ++j) {
                dp[j] = dot(dO + i * d, V + j * d, d);
                Di += p[j] * dp[j];
            }
            double* out = dQ + r * d;
            for (long c = 0; c < d; ++c) out[c] = 0.0;
            for (long j = 0; j < n; ++j) {
                double ds = p[j] * (dp[j] - Di);
                for (long c = 0; c < d; ++c) out[c] += scale * ds * K[j * d + c];
            }
        }
        free(dp);
        free(p);
    }
}

/* dK_j and dV_j for selected keys of one head.  Needs every row's L_i and D_i
 * (from orc_row_stats); P_ij = exp(s_ij - L_i) is the softmax written with the
 * row's logsumexp ([1p3a]), dS_ij = P_ij (dP_ij - D_i),
 * dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i over the rows i that
 * see key j. */
void orc_dkdv_rows(const double* Q, const double* K, const double* V,
                   const double* dO, const double* L, const double* D,
                   long N, long d, double scale, int causal,
                   const long* keys, long nkeys, double* dK, double* dV) {
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < nkeys; ++r) {
        long j = keys[r];
        double* dk = dK + r * d;
        double* dv = dV + r * d;
        for (long c = 0; c < d; ++c) { dk[c] = 0.0; dv[c] = 0.0; }
        for (long i = causal ? j : 0; i < N; ++i) {
            double P = exp(scale * dot(Q + i * d, K + j * d, d) - L[i]);
            double ds = P * (dot(dO + i * d, V + j * d, d) - D[i]);
            for (long c = 0; c < d; ++c) {
                dk[c] += scale * ds * Q[i * d + c];
                dv[c] += P * dO[i * d + c];
            }
        }
    }
}

/* ---- tiled variant, used only to check the definition above ------------ */

#define ORC_FLAG_FORGET_ALPHA_ON_ACC 1

/* Tiled forward with the online-softmax recurrence of [1p3a]: per query row,
 * running max m, denominator l and unnormalised accumulator a start at
 * (-inf, 0, 0); for each key block b: m' = max(m, max s_b), p_b = exp(s_b - m'),
 * alpha = exp(m - m'), l' = alpha l + sum p_b, a' = alpha a + p_b V_b; at the end
 * O = a / l and L = m + log l.  Row blocks of Br, key blocks of Bc; under the
 * causal mask, key blocks lying wholly above the row block are skipped
 * ([FA2-ch16] 16.8 item 2).  flags & ORC_FLAG_FORGET_ALPHA_ON_ACC plants the
 * pitfall [1p3a] warns about (a' = a + p_b V_b); only the negative-control test
 * sets it. */
void orc_flash_fwd_tiled(const double* Q, const double* K, const double* V,
                         long BH, long N, long d, double scale, int causal,
                         long Br, long Bc, int flags, double* O, double* L) {
    for (long bh = 0; bh < BH; ++bh) {
        const double* q = Q + bh * N * d;
        const double* k = K + bh * N * d;
        const double* v = V + bh * N * d;
#pragma omp parallel for schedule(dynamic, 1)
        for (long r0 = 0; r0 < N; r0 += Br) {
            long r1 = r0 + Br < N ? r0 + Br : N;
            long nr = r1 - r0;
            double* m = (double*)malloc(sizeof(double) * (size_t)nr);
            double* l = (double*)calloc((size_t)nr, sizeof(double));
            double* a = (double*)calloc((size_t)(nr * d), sizeof(double));
            double* s = (double*)malloc(sizeof(double) * (size_t)Bc);
            for (long t = 0; t < nr; ++t) m[t] = -INFINITY;
            for (long c0 = 0; c0 < N; c0 += Bc) {
                if (causal && c0 > r1 - 1) break; /* every key in this block > every row */
                long c1 = c0 + Bc < N ? c0 + Bc : N;
                for (long i = r0; i < r1; ++i) {
                    long t = i - r0;
                    long cend = c1;
                    if (causal && cend > i + 1) cend = i + 1;
                    if (cend <= c0) continue;          /* row sees nothing here */
                    double mb = -INFINITY;
                    for (long j = c0; j < cend; ++j) {
                        s[j - c0] = scale * dot(q + i * d, k + j * d, d);
                        if (s[j - c0] > mb) mb = s[j - c0];
                    }
                    double mn = m[t] > mb ? m[t] : mb;
                    double alpha = (m[t] == -INFINITY) ? 0.0 : exp(m[t] - mn);
                    double psum = 0.0;
                    double* at = a + t * d;
                    if (!(flags & ORC_FLAG_FORGET_ALPHA_ON_ACC))
                        for (long c = 0; c < d; ++c) at[c] *= alpha;
                    for (long j = c0; j < cend; ++j) {
                        double pj = exp(s[j - c0] - mn);
                        psum += pj;
                        for (long c = 0; c < d; ++c) at[c] += pj * v[j * d + c];
                    }
                    l[t] = alpha * l[t] + psum;
                    m[t] = mn;
                }
            }
            for (long i = r0; i < r1; ++i) {
                long t = i - r0;
                for (long c = 0; c < d; ++c) O[bh * N * d + i * d + c] = a[t * d + c] / l[t];
                L[bh * N + i] = m[t] + log(l[t]);
            }
            free(s); free(a); free(l); free(m);
        }
    }
}

/* Tiled backward in the loop order of [FA2-ch16] 16.2: key blocks outer, query
 * blocks inner; dV and dK accumulate per key block and are written once, dQ
 * receives one partial per (key block, query block).  D_i = dO_i . O_i is
 * computed first ([FA2-ch16] 16.8 item 1); P = exp(S - L) uses the stored
 * logsumexp ([FA2-ch16] 16.4).  dK is scaled at write-out and dQ at the end
 * ([FA2-ch16] 16.6).  Under the causal mask whole tiles above the diagonal are
 * skipped and diagonal tiles are masked element by element. */
void orc_flash_bwd_tiled(const double* Q, const double* K, const double* V,
                         const double* O, const double* dO, const double* L,
                         long BH, long N, long d, double scale, int causal,
                         long Br, long Bc, double* dQ, double* dK, double* dV) {
    for (long bh = 0; bh < BH; ++bh) {
        const double* q = Q + bh * N * d;
        const double* k = K + bh * N * d;
        const double* v = V + bh * N * d;
        const double* o = O + bh * N * d;
        const double* g = dO + bh * N * d;
        const double* lse = L + bh * N;
        double* dq = dQ + bh * N * d;
        double* Dv = (double*)malloc(sizeof(double) * (size_t)N);
        for (long i = 0; i < N; ++i) Dv[i] = dot(o + i * d, g + i * d, d);
        for (long e = 0; e < N * d; ++e) dq[e] = 0.0;
        /* key blocks are independent except for dQ, so run them in order */
        double* dka = (double*)malloc(sizeof(double) * (size_t)(Bc * d));
        double* dva = (double*)malloc(sizeof(double) * (size_t)(Bc * d));
        double* P = (double*)malloc(sizeof(double) * (size_t)(Br * Bc));
        double* dS = (double*)malloc(sizeof(double) * (size_t)(Br * Bc));
        for (long c0 = 0; c0 < N; c0 += Bc) {
            long c1 = c0 + Bc < N ? c0 + Bc : N;
            memset(dka, 0, sizeof(double) * (size_t)(Bc * d));
            memset(dva, 0, sizeof(double) * (size_t)(Bc * d));
            for (long r0 = 0; r0 < N; r0 += Br) {
                long r1 = r0 + Br < N ? r0 + Br : N;
                if (causal && r1 - 1 < c0) continue;   /* every q < every k */
                for (long i = r0; i < r1; ++i)
                    for (long j = c0; j < c1; ++j) {
                        long e = (i - r0) * Bc + (j - c0);
                        if (causal && j > i) { P[e] = 0.0; dS[e] = 0.0; continue; }
                        double s = scale * dot(q + i * d, k + j * d, d);
                        P[e] = exp(s - lse[i]);
                        double dp = dot(g + i * d, v + j * d, d);
                        dS[e] = P[e] * (dp - Dv[i]);
                    }
                for (long j = c0; j < c1; ++j)
                    for (long i = r0; i < r1; ++i) {
                        long e = (i - r0) * Bc + (j - c0);
                        for (long c = 0; c < d; ++c) {
                            dva[(j - c0) * d + c] += P[e] * g[i * d + c];
                            dka[(j - c0) * d + c] += dS[e] * q[i * d + c];
                        }
                    }
                for (long i = r0; i < r1; ++i)
                    for (long j = c0; j < c1; ++j) {
                        long e = (i - r0) * Bc + (j - c0);
                        for (long c = 0; c < d; ++c) dq[i * d + c] += dS[e] * k[j * d + c];
                    }
            }
            for (long j = c0; j < c1; ++j)
                for (long c = 0; c < d; ++c) {
                    dV[bh * N * d + j * d + c] = dva[(j - c0) * d + c];
                    dK[bh * N * d + j * d + c] = scale * dka[(j - c0) * d + c];
                }
        }
        for (long e = 0; e < N * d; ++e) dq[e] *= scale;
        free(dS); free(P); free(dva); free(dka); free(Dv);
    }
}
