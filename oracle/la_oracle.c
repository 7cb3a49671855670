/*
 * la_oracle.c -- plain fp64 CPU oracle for kernelized linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link,
 * load or call this file.  Its only users are the tests, the smoke check and
 * the CPU-baseline leg of the benchmark.  It shares no code, header, table or
 * helper with the HIP library; the two meet only in the seeded input arrays.
 *
 * Sources (web pages on Katharopoulos et al., "Transformers are RNNs: Fast
 * Autoregressive Transformers with Linear Attention", ICML 2020):
 *   [review]  nubint.ai, "[Paper Review] Transformers are RNNs: ...",
 *             section "Proposed method".
 *   [summary] paperlayer.ai, "Transformers are RNNs: ..." (arXiv 2006.16236v3
 *             summary), sections 3.2, 3.2.1, 3.3, 3.3.1, 3.3.2, 3.4 and
 *             appendix "A. Gradient Derivation".
 *   [deck]    zhengyuhong.cn, "Transformers are RNNs: ... 解读", slide 3
 *             (associativity, feature map) and slide 4 (causal prefix states).
 *
 * Every routine below follows the per-token recurrence literally, in double
 * precision, with no chunking, blocking or reordering.  Arrays are dense and
 * row-major: q,k are [B][H][N][D], v,out are [B][H][N][M].  The (b,h) slices
 * are independent recurrences, so they are spread over OpenMP threads; the
 * order of operations inside one slice is the plain sequential order.
 *
 * Readings where the pages are silent:
 *   - feature map phi(x) = elu(x) + 1 with alpha = 1, i.e. x + 1 for x > 0
 *     and exp(x) otherwise ([deck] slide 3; [summary] 3.2.1).  Both branches
 *     give value 1 and slope 1 at x = 0, so the branch choice at 0 is moot.
 *   - causal prefix states include token i itself (j <= i) ([deck] slide 4).
 *   - no 1/sqrt(D) scaling and no epsilon in the denominator; phi > 0 makes
 *     every denominator positive.
 *   - the decode step updates the state first and then reads it out, so it
 *     reproduces the inclusive causal forward ([review] "Proposed method",
 *     two-step update; [deck] slide 4).
 *   - the backward pass differentiates with respect to the raw Q, K, V,
 *     through phi and through the denominator.  The pages only sketch the
 *     numerator part ([summary] appendix A) and leave the rest to autograd;
 *     the formulas used here are derived in the comments of
 *     orc_backward_causal and pinned by finite differences in the tests.
 *   - the gradient of the degree-2 polynomial form is written as its plain
 *     pairwise definition (every pair j <= i, by the chain rule), not as a
 *     recurrence: an independent form, pinned by finite differences of the
 *     polynomial forward.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* phi(x) = elu(x) + 1 ([deck] slide 3; [summary] 3.2.1). */
static double phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* d phi / dx: 1 for x > 0, exp(x) otherwise. */
static double dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Elementwise phi and phi' over n values (used to pin phi itself). */
void orc_feature_map(const double *x, double *y, double *dy, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) {
        y[i] = phi(x[i]);
        if (dy) dy[i] = dphi(x[i]);
    }
}

/*
 * Causal forward ([deck] slide 4; [review] "Proposed method"; [summary] 3.3):
 *   S_i = S_{i-1} + phi(K_i) V_i^T        (D x M)
 *   Z_i = Z_{i-1} + phi(K_i)              (D)
 *   out_i = S_i^T phi(Q_i) / (phi(Q_i) . Z_i)
 * S_io / Z_io (nullable, [B][H][D][M] and [B][H][D]) hold the starting state
 * on entry and the final state S_N, Z_N on return; when null the state starts
 * at zero.  den (nullable, [B][H][N]) receives each denominator.
 */
void orc_forward_causal(const double *q, const double *k, const double *v,
                        double *out, double *S_io, double *Z_io, double *den,
                        int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M;
        double *O = out + bh * N * M;
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *Z = (double *)calloc((size_t)D, sizeof(double));
        double *qh = (double *)malloc((size_t)D * sizeof(double));
        double *kh = (double *)malloc((size_t)D * sizeof(double));
        if (S_io) memcpy(S, S_io + bh * D * M, (size_t)(D * M) * sizeof(double));
        if (Z_io) memcpy(Z, Z_io + bh * D, (size_t)D * sizeof(double));
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t d = 0; d < D; ++d) {
                kh[d] = phi(K[i * D + d]);
                qh[d] = phi(Q[i * D + d]);
            }
            /* state update, token i included */
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += kh[d] * V[i * M + m];
                Z[d] += kh[d];
            }
            /* readout */
            double dd = 0.0;
            for (int64_t d = 0; d < D; ++d) dd += qh[d] * Z[d];
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t d = 0; d < D; ++d) n += qh[d] * S[d * M + m];
                O[i * M + m] = n / dd;
            }
            if (den) den[bh * N + i] = dd;
        }
        if (S_io) memcpy(S_io + bh * D * M, S, (size_t)(D * M) * sizeof(double));
        if (Z_io) memcpy(Z_io + bh * D, Z, (size_t)D * sizeof(double));
        free(S); free(Z); free(qh); free(kh);
    }
}

/*
 * Non-causal forward ([review] "Proposed method"; [summary] 3.2; [deck]
 * slide 3): S = sum_j phi(K_j) V_j^T and Z = sum_j phi(K_j) over all N
 * tokens, then out_i = S^T phi(Q_i) / (phi(Q_i) . Z).
 */
void orc_forward_noncausal(const double *q, const double *k, const double *v,
                           double *out, int64_t B, int64_t H, int64_t N,
                           int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M;
        double *O = out + bh * N * M;
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *Z = (double *)calloc((size_t)D, sizeof(double));
        double *qh = (double *)malloc((size_t)D * sizeof(double));
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t d = 0; d < D; ++d) {
                double kd = phi(K[j * D + d]);
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += kd * V[j * M + m];
                Z[d] += kd;
            }
        }
        for (int64_t i = 0; i < N; ++i) {
            double dd = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                qh[d] = phi(Q[i * D + d]);
                dd += qh[d] * Z[d];
            }
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t d = 0; d < D; ++d) n += qh[d] * S[d * M + m];
                O[i * M + m] = n / dd;
            }
        }
        free(S); free(Z); free(qh);
    }
}

/*
 * Causal backward.  With loss L = sum_i G_i . out_i (G = dout), write
 * qh_i = phi(Q_i), kh_j = phi(K_j), a_ij = qh_i . kh_j for j <= i,
 * d_i = sum_{j<=i} a_ij and out_i = sum_{j<=i} a_ij V_j / d_i.  Then
 *   dL/da_ij = G_i . (V_j - out_i) / d_i = g_i . V_j + h_i,
 *   with g_i = G_i / d_i and h_i = -(G_i . out_i) / d_i.
 * Summing over the indices each a_ij touches:
 *   dL/dqh_i = sum_{j<=i} (g_i . V_j + h_i) kh_j = S_i g_i + h_i Z_i
 *              (no sum over later tokens: [summary] appendix A, eq. 13),
 *   dL/dkh_j = sum_{i>=j} (g_i . V_j + h_i) qh_i = R_j V_j + u_j,
 *   dL/dV_j  = sum_{i>=j} a_ij g_i = R_j^T kh_j,
 *   with the reverse prefix sums R_j = sum_{i>=j} qh_i g_i^T (D x M) and
 *   u_j = sum_{i>=j} h_i qh_i (D) ([summary] appendix A, eqs. 14-15: key j
 *   affects every output i >= j, and this sum runs in the opposite direction
 *   to the forward one).  Finally dQ = dL/dqh * phi'(Q), dK = dL/dkh * phi'(K).
 * Pass 1 runs i = 1..N and rebuilds S_i, Z_i, d_i, out_i as the forward does;
 * it keeps only g (N x M) and h (N), never the N states S_i.  Pass 2 runs
 * j = N..1 carrying R and u.
 */
void orc_backward_causal(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv,
                         int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M, *G = dout + bh * N * M;
        double *dQ = dq + bh * N * D, *dK = dk + bh * N * D, *dV = dv + bh * N * M;
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *Z = (double *)calloc((size_t)D, sizeof(double));
        double *g = (double *)malloc((size_t)(N * M) * sizeof(double));
        double *h = (double *)malloc((size_t)N * sizeof(double));
        double *qh = (double *)malloc((size_t)D * sizeof(double));
        double *kh = (double *)malloc((size_t)D * sizeof(double));
        double *o = (double *)malloc((size_t)M * sizeof(double));

        /* pass 1: forward direction */
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t d = 0; d < D; ++d) {
                kh[d] = phi(K[i * D + d]);
                qh[d] = phi(Q[i * D + d]);
            }
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += kh[d] * V[i * M + m];
                Z[d] += kh[d];
            }
            double dd = 0.0;
            for (int64_t d = 0; d < D; ++d) dd += qh[d] * Z[d];
            double go = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t d = 0; d < D; ++d) n += qh[d] * S[d * M + m];
                o[m] = n / dd;
                go += G[i * M + m] * o[m];
            }
            for (int64_t m = 0; m < M; ++m) g[i * M + m] = G[i * M + m] / dd;
            h[i] = -go / dd;
            for (int64_t d = 0; d < D; ++d) {
                double acc = h[i] * Z[d];
                for (int64_t m = 0; m < M; ++m) acc += S[d * M + m] * g[i * M + m];
                dQ[i * D + d] = acc * dphi(Q[i * D + d]);
            }
        }

        /* pass 2: reverse direction; S is reused as R, Z as u */
        memset(S, 0, (size_t)(D * M) * sizeof(double));
        memset(Z, 0, (size_t)D * sizeof(double));
        for (int64_t j = N - 1; j >= 0; --j) {
            for (int64_t d = 0; d < D; ++d) {
                qh[d] = phi(Q[j * D + d]);
                kh[d] = phi(K[j * D + d]);
            }
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += qh[d] * g[j * M + m];
                Z[d] += h[j] * qh[d];
            }
            for (int64_t d = 0; d < D; ++d) {
                double acc = Z[d];
                for (int64_t m = 0; m < M; ++m) acc += S[d * M + m] * V[j * M + m];
                dK[j * D + d] = acc * dphi(K[j * D + d]);
            }
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += S[d * M + m] * kh[d];
                dV[j * M + m] = acc;
            }
        }
        free(S); free(Z); free(g); free(h); free(qh); free(kh); free(o);
    }
}

/*
 * Non-causal backward.  The derivation of orc_backward_causal with every
 * token seeing every other (a_ij = qh_i . kh_j for all i, j; [summary] 3.2:
 * the non-causal form through associativity): S = sum_j kh_j V_j^T and
 * Z = sum_j kh_j are the full sums, d_i = qh_i . Z, out_i = S^T qh_i / d_i,
 * g_i = G_i / d_i, h_i = -(G_i . out_i) / d_i, and
 *   dL/dqh_i = S g_i + h_i Z,
 *   dL/dkh_j = R V_j + u,   dL/dV_j = R^T kh_j,
 *   with R = sum_i qh_i g_i^T and u = sum_i h_i qh_i over all i (no prefix:
 *   every output depends on every key).  dQ = dL/dqh * phi'(Q),
 *   dK = dL/dkh * phi'(K).
 */
void orc_backward_noncausal(const double *q, const double *k, const double *v,
                            const double *dout, double *dq, double *dk, double *dv,
                            int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M, *G = dout + bh * N * M;
        double *dQ = dq + bh * N * D, *dK = dk + bh * N * D, *dV = dv + bh * N * M;
        double *S = (double *)calloc((size_t)(D * M), sizeof(double));
        double *Z = (double *)calloc((size_t)D, sizeof(double));
        double *R = (double *)calloc((size_t)(D * M), sizeof(double));
        double *u = (double *)calloc((size_t)D, sizeof(double));
        double *qh = (double *)malloc((size_t)D * sizeof(double));
        double *kh = (double *)malloc((size_t)D * sizeof(double));
        double *g = (double *)malloc((size_t)M * sizeof(double));

        /* the full sums S, Z */
        for (int64_t j = 0; j < N; ++j)
            for (int64_t d = 0; d < D; ++d) {
                const double kj = phi(K[j * D + d]);
                for (int64_t m = 0; m < M; ++m) S[d * M + m] += kj * V[j * M + m];
                Z[d] += kj;
            }
        /* per query: out_i, d_i, g_i, h_i; dQ_i; accumulate R, u */
        for (int64_t i = 0; i < N; ++i) {
            double dd = 0.0;
            for (int64_t d = 0; d < D; ++d) {
                qh[d] = phi(Q[i * D + d]);
                dd += qh[d] * Z[d];
            }
            double go = 0.0;
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t d = 0; d < D; ++d) n += qh[d] * S[d * M + m];
                go += G[i * M + m] * (n / dd);
                g[m] = G[i * M + m] / dd;
            }
            const double h = -go / dd;
            for (int64_t d = 0; d < D; ++d) {
                double acc = h * Z[d];
                for (int64_t m = 0; m < M; ++m) acc += S[d * M + m] * g[m];
                dQ[i * D + d] = acc * dphi(Q[i * D + d]);
                for (int64_t m = 0; m < M; ++m) R[d * M + m] += qh[d] * g[m];
                u[d] += h * qh[d];
            }
        }
        /* per key: dK_j, dV_j */
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t d = 0; d < D; ++d) kh[d] = phi(K[j * D + d]);
            for (int64_t d = 0; d < D; ++d) {
                double acc = u[d];
                for (int64_t m = 0; m < M; ++m) acc += R[d * M + m] * V[j * M + m];
                dK[j * D + d] = acc * dphi(K[j * D + d]);
            }
            for (int64_t m = 0; m < M; ++m) {
                double acc = 0.0;
                for (int64_t d = 0; d < D; ++d) acc += R[d * M + m] * kh[d];
                dV[j * M + m] = acc;
            }
        }
        free(S); free(Z); free(R); free(u); free(qh); free(kh); free(g);
    }
}

/*
 * Random Fourier features ([summary] 5: approximating the RBF kernel with
 * random Fourier features is named as a way to reuse softmax-pretrained
 * models; the construction is the standard one of Rahimi and Recht):
 *   phi_r(x) = sqrt(2 / R) cos(sum_d x_d omega[d][r] + b_r),  r < R,
 * with omega [D][R] and b [R] drawn by the caller (omega ~ N(0, 1/sigma^2),
 * b ~ U[0, 2 pi)), so that phi(q) . phi(k) estimates the RBF kernel
 * exp(-|q - k|^2 / (2 sigma^2)).  x: [rows][D]; out: [rows][R].
 */
void orc_rff_features(const double *x, const double *omega, const double *b, double *out,
                      int64_t rows, int64_t D, int64_t R)
{
    const double scale = sqrt(2.0 / (double)R);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t r = 0; r < R; ++r) {
            double a = b[r];
            for (int64_t d = 0; d < D; ++d) a += x[i * D + d] * omega[d * R + r];
            out[i * R + r] = scale * cos(a);
        }
    }
}

/*
 * Causal forward with the feature map already applied: fq = phi(Q) and
 * fk = phi(K) are given, [B][H][N][F].  The recurrence of orc_forward_causal
 * with phi the identity: S_i = S_{i-1} + fk_i V_i^T, Z_i = Z_{i-1} + fk_i,
 * out_i = S_i^T fq_i / (fq_i . Z_i).  Features of any sign are accepted; the
 * result is whatever the division gives.
 */
void orc_forward_causal_features(const double *fq, const double *fk, const double *v, double *out,
                                 int64_t B, int64_t H, int64_t N, int64_t F, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = fq + bh * N * F, *K = fk + bh * N * F;
        const double *V = v + bh * N * M;
        double *O = out + bh * N * M;
        double *S = (double *)calloc((size_t)(F * M), sizeof(double));
        double *Z = (double *)calloc((size_t)F, sizeof(double));
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t f = 0; f < F; ++f) {
                for (int64_t m = 0; m < M; ++m) S[f * M + m] += K[i * F + f] * V[i * M + m];
                Z[f] += K[i * F + f];
            }
            double dd = 0.0;
            for (int64_t f = 0; f < F; ++f) dd += Q[i * F + f] * Z[f];
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t f = 0; f < F; ++f) n += Q[i * F + f] * S[f * M + m];
                O[i * M + m] = n / dd;
            }
        }
        free(S); free(Z);
    }
}

/*
 * Causal forward with the degree-2 polynomial kernel ([summary] 3.2.1: a
 * degree-2 polynomial kernel has an exact finite feature map).  Reading:
 * sim(q, k) = (q . k)^2, whose feature map is phi(x) = vec(x x^T) (D^2
 * features, phi(q) . phi(k) = sum_{a,b} q_a q_b k_a k_b = (q . k)^2).  The
 * recurrence of orc_forward_causal with that phi: S_i = S_{i-1} +
 * phi(K_i) V_i^T (D^2 x M), Z_i = Z_{i-1} + phi(K_i), out_i =
 * S_i^T phi(Q_i) / (phi(Q_i) . Z_i).  q, k: [B][H][N][D]; v, out: [B][H][N][M].
 */
void orc_forward_causal_poly2(const double *q, const double *k, const double *v, double *out,
                              int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H, F = D * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M;
        double *O = out + bh * N * M;
        double *S = (double *)calloc((size_t)(F * M), sizeof(double));
        double *Z = (double *)calloc((size_t)F, sizeof(double));
        double *pq = (double *)malloc((size_t)F * sizeof(double));
        double *pk = (double *)malloc((size_t)F * sizeof(double));
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t a = 0; a < D; ++a)
                for (int64_t b = 0; b < D; ++b) {
                    pq[a * D + b] = Q[i * D + a] * Q[i * D + b];
                    pk[a * D + b] = K[i * D + a] * K[i * D + b];
                }
            for (int64_t f = 0; f < F; ++f) {
                for (int64_t m = 0; m < M; ++m) S[f * M + m] += pk[f] * V[i * M + m];
                Z[f] += pk[f];
            }
            double dd = 0.0;
            for (int64_t f = 0; f < F; ++f) dd += pq[f] * Z[f];
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t f = 0; f < F; ++f) n += pq[f] * S[f * M + m];
                O[i * M + m] = n / dd;
            }
        }
        free(S); free(Z); free(pq); free(pk);
    }
}

/*
 * Non-causal forward with the same kernel ([summary] 3.2.1; every key
 * attends): S = sum_j phi(K_j) V_j^T and Z = sum_j phi(K_j) over all j with
 * phi(x) = vec(x x^T), then out_i = S^T phi(Q_i) / (phi(Q_i) . Z).
 */
void orc_forward_noncausal_poly2(const double *q, const double *k, const double *v, double *out,
                                 int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H, F = D * D;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M;
        double *O = out + bh * N * M;
        double *S = (double *)calloc((size_t)(F * M), sizeof(double));
        double *Z = (double *)calloc((size_t)F, sizeof(double));
        double *pf = (double *)malloc((size_t)F * sizeof(double));
        for (int64_t j = 0; j < N; ++j) {
            for (int64_t a = 0; a < D; ++a)
                for (int64_t b = 0; b < D; ++b) pf[a * D + b] = K[j * D + a] * K[j * D + b];
            for (int64_t f = 0; f < F; ++f) {
                for (int64_t m = 0; m < M; ++m) S[f * M + m] += pf[f] * V[j * M + m];
                Z[f] += pf[f];
            }
        }
        for (int64_t i = 0; i < N; ++i) {
            for (int64_t a = 0; a < D; ++a)
                for (int64_t b = 0; b < D; ++b) pf[a * D + b] = Q[i * D + a] * Q[i * D + b];
            double dd = 0.0;
            for (int64_t f = 0; f < F; ++f) dd += pf[f] * Z[f];
            for (int64_t m = 0; m < M; ++m) {
                double n = 0.0;
                for (int64_t f = 0; f < F; ++f) n += pf[f] * S[f * M + m];
                O[i * M + m] = n / dd;
            }
        }
        free(S); free(Z); free(pf);
    }
}

/*
 * Selected rows of the polynomial forwards, each from the kernel itself
 * ([summary] 3.2.1; the attention form sim(q_i, k_j) summed over j <= i, or
 * over all j when causal is 0):
 *   out_i = sum_j (q_i . k_j)^2 v_j / sum_j (q_i . k_j)^2,
 * O(i (D + M)) per row, for checking long sequences at sampled rows.
 * rows: nrows token indices in [0, N); out: [B][H][nrows][M].
 */
void orc_forward_poly2_rows(const double *q, const double *k, const double *v, const int64_t *rows,
                            double *out, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                            int64_t nrows, int64_t causal)
{
    const int64_t BH = B * H;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = rows[r];
            const int64_t last = causal ? i : N - 1;
            const double *qi = q + (bh * N + i) * D;
            double *o = out + (bh * nrows + r) * M;
            double den = 0.0;
            for (int64_t m = 0; m < M; ++m) o[m] = 0.0;
            for (int64_t j = 0; j <= last; ++j) {
                const double *kj = k + (bh * N + j) * D, *vj = v + (bh * N + j) * M;
                double dot = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * kj[a];
                const double w = dot * dot;
                den += w;
                for (int64_t m = 0; m < M; ++m) o[m] += w * vj[m];
            }
            for (int64_t m = 0; m < M; ++m) o[m] /= den;
        }
}

/*
 * Gradients of L = sum(dout * out) for the causal forward with the degree-2
 * polynomial kernel ([summary] 3.2.1 for the kernel; 3.3.1: the gradient of
 * the linear form).  Plain definition by the chain rule, O(N^2) per (b, h):
 *   s_ij = (q_i . k_j)^2 (j <= i), d_i = sum_j s_ij, out_i = sum_j s_ij v_j / d_i;
 *   dL/ds_ij = (dout_i . v_j - dout_i . out_i) / d_i = e_ij;
 *   dq_i = sum_{j<=i} e_ij 2 (q_i . k_j) k_j,  dk_j = sum_{i>=j} e_ij 2 (q_i . k_j) q_i,
 *   dv_j = sum_{i>=j} s_ij dout_i / d_i.
 * q, k, dq, dk: [B][H][N][D]; v, dout, dv: [B][H][N][M].
 */
void orc_backward_causal_poly2(const double *q, const double *k, const double *v, const double *dout,
                               double *dq, double *dk, double *dv,
                               int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M, *G = dout + bh * N * M;
        double *dQ = dq + bh * N * D, *dK = dk + bh * N * D, *dV = dv + bh * N * M;
        for (int64_t x = 0; x < N * D; ++x) { dQ[x] = 0.0; dK[x] = 0.0; }
        for (int64_t x = 0; x < N * M; ++x) dV[x] = 0.0;
        double *o = (double *)malloc((size_t)M * sizeof(double));
        for (int64_t i = 0; i < N; ++i) {
            const double *qi = Q + i * D, *gi = G + i * M;
            /* the forward row: d_i and out_i */
            double den = 0.0;
            for (int64_t m = 0; m < M; ++m) o[m] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * K[j * D + a];
                den += dot * dot;
                for (int64_t m = 0; m < M; ++m) o[m] += dot * dot * V[j * M + m];
            }
            for (int64_t m = 0; m < M; ++m) o[m] /= den;
            double go = 0.0;
            for (int64_t m = 0; m < M; ++m) go += gi[m] * o[m];
            /* every pair (i, j <= i) */
            for (int64_t j = 0; j <= i; ++j) {
                const double *kj = K + j * D, *vj = V + j * M;
                double dot = 0.0, gv = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * kj[a];
                for (int64_t m = 0; m < M; ++m) gv += gi[m] * vj[m];
                const double e = (gv - go) / den;
                for (int64_t a = 0; a < D; ++a) {
                    dQ[i * D + a] += e * 2.0 * dot * kj[a];
                    dK[j * D + a] += e * 2.0 * dot * qi[a];
                }
                for (int64_t m = 0; m < M; ++m) dV[j * M + m] += dot * dot * gi[m] / den;
            }
        }
        free(o);
    }
}

/*
 * Selected rows of orc_backward_causal_poly2, each summed pair by pair from
 * the same definition: dq at the rows rq[0 .. nq) (O(i (D + M)) per row),
 * dk and dv at the rows rk[0 .. nk) (every later token's out_i and d_i are
 * formed first, once: O((N - min rk) N (D + M)), for rows near the end).
 * dq: [B][H][nq][D]; dk: [B][H][nk][D]; dv: [B][H][nk][M].
 */
void orc_backward_causal_poly2_rows(const double *q, const double *k, const double *v, const double *dout,
                                    const int64_t *rq, int64_t nq, const int64_t *rk, int64_t nk,
                                    double *dq, double *dk, double *dv,
                                    int64_t B, int64_t H, int64_t N, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
    int64_t jmin = N;
    for (int64_t r = 0; r < nk; ++r) if (rk[r] < jmin) jmin = rk[r];
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *Q = q + bh * N * D, *K = k + bh * N * D;
        const double *V = v + bh * N * M, *G = dout + bh * N * M;
        const int64_t nt = N - jmin;
        /* out_i . dout_i and d_i of token i (jmin <= i < N) */
        double *go = (double *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(double));
        double *den = (double *)malloc((size_t)(nt > 0 ? nt : 1) * sizeof(double));
        double *o = (double *)malloc((size_t)M * sizeof(double));
        for (int64_t i = jmin; i < N; ++i) {
            double dd = 0.0;
            for (int64_t m = 0; m < M; ++m) o[m] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += Q[i * D + a] * K[j * D + a];
                dd += dot * dot;
                for (int64_t m = 0; m < M; ++m) o[m] += dot * dot * V[j * M + m];
            }
            double g = 0.0;
            for (int64_t m = 0; m < M; ++m) g += G[i * M + m] * o[m] / dd;
            go[i - jmin] = g;
            den[i - jmin] = dd;
        }
        for (int64_t r = 0; r < nq; ++r) {
            const int64_t i = rq[r];
            const double *qi = Q + i * D, *gi = G + i * M;
            double *out = dq + (bh * nq + r) * D;
            double dd = 0.0, g = 0.0;
            for (int64_t m = 0; m < M; ++m) o[m] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dot = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * K[j * D + a];
                dd += dot * dot;
                for (int64_t m = 0; m < M; ++m) o[m] += dot * dot * V[j * M + m];
            }
            for (int64_t m = 0; m < M; ++m) g += gi[m] * o[m] / dd;
            for (int64_t a = 0; a < D; ++a) out[a] = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                const double *kj = K + j * D, *vj = V + j * M;
                double dot = 0.0, gv = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * kj[a];
                for (int64_t m = 0; m < M; ++m) gv += gi[m] * vj[m];
                const double e = (gv - g) / dd;
                for (int64_t a = 0; a < D; ++a) out[a] += e * 2.0 * dot * kj[a];
            }
        }
        for (int64_t r = 0; r < nk; ++r) {
            const int64_t j = rk[r];
            const double *kj = K + j * D, *vj = V + j * M;
            double *ok = dk + (bh * nk + r) * D, *ov = dv + (bh * nk + r) * M;
            for (int64_t a = 0; a < D; ++a) ok[a] = 0.0;
            for (int64_t m = 0; m < M; ++m) ov[m] = 0.0;
            for (int64_t i = j; i < N; ++i) {
                const double *qi = Q + i * D, *gi = G + i * M;
                double dot = 0.0, gv = 0.0;
                for (int64_t a = 0; a < D; ++a) dot += qi[a] * kj[a];
                for (int64_t m = 0; m < M; ++m) gv += gi[m] * vj[m];
                const double dd = den[i - jmin];
                const double e = (gv - go[i - jmin]) / dd;
                for (int64_t a = 0; a < D; ++a) ok[a] += e * 2.0 * dot * qi[a];
                for (int64_t m = 0; m < M; ++m) ov[m] += dot * dot * gi[m] / dd;
            }
        }
        free(go); free(den); free(o);
    }
}

/*
 * One RNN-style decode step for B*H independent streams ([review] "Proposed
 * method", attention memory s and normalizer memory z; [summary] 3.3.2, 3.4;
 * [deck] slide 4): S += phi(k) v^T, Z += phi(k), then
 * out = S^T phi(q) / (phi(q) . Z).  q,k: [B][H][D]; v,out: [B][H][M];
 * S: [B][H][D][M]; Z: [B][H][D]; S and Z are updated in place.
 */
void orc_decode_step(const double *q, const double *k, const double *v,
                     double *S, double *Z, double *out,
                     int64_t B, int64_t H, int64_t D, int64_t M)
{
    const int64_t BH = B * H;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < BH; ++bh) {
        const double *qq = q + bh * D, *kk = k + bh * D, *vv = v + bh * M;
        double *SS = S + bh * D * M, *ZZ = Z + bh * D, *oo = out + bh * M;
        double dd = 0.0;
        for (int64_t d = 0; d < D; ++d) {
            double kd = phi(kk[d]);
            for (int64_t m = 0; m < M; ++m) SS[d * M + m] += kd * vv[m];
            ZZ[d] += kd;
            dd += phi(qq[d]) * ZZ[d];
        }
        for (int64_t m = 0; m < M; ++m) {
            double n = 0.0;
            for (int64_t d = 0; d < D; ++d) n += phi(qq[d]) * SS[d * M + m];
            oo[m] = n / dd;
        }
    }
}
