/*
 * sanity_main.c -- a driver that runs every oracle routine on small shapes
 * (one token, one feature, ragged lengths, several (b, h) slices) so that the
 * oracle can be built and run under AddressSanitizer and
 * UndefinedBehaviorSanitizer on the CPU.  TEST INFRASTRUCTURE ONLY, like
 * la_oracle.c.  Its inputs come from a fixed-seed xorshift generator (memory
 * safety and finite results are checked here; the values are pinned by the
 * Python tests).  Exits 0 when every routine ran and returned finite values.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_feature_map(const double *x, double *y, double *dy, int64_t n);
void orc_forward_causal(const double *q, const double *k, const double *v, double *out, double *S_io,
                        double *Z_io, double *den, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);
void orc_forward_noncausal(const double *q, const double *k, const double *v, double *out, int64_t B,
                           int64_t H, int64_t N, int64_t D, int64_t M);
void orc_backward_causal(const double *q, const double *k, const double *v, const double *g, double *dq,
                         double *dk, double *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);
void orc_backward_noncausal(const double *q, const double *k, const double *v, const double *g, double *dq,
                            double *dk, double *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);
void orc_rff_features(const double *x, const double *omega, const double *b, double *out, int64_t rows,
                      int64_t D, int64_t R);
void orc_forward_causal_features(const double *fq, const double *fk, const double *v, double *out, int64_t B,
                                 int64_t H, int64_t N, int64_t F, int64_t M);
void orc_forward_causal_poly2(const double *q, const double *k, const double *v, double *out, int64_t B,
                              int64_t H, int64_t N, int64_t D, int64_t M);
void orc_decode_step(const double *q, const double *k, const double *v, double *S, double *Z, double *out,
                     int64_t B, int64_t H, int64_t D, int64_t M);
void orc_backward_causal_poly2(const double *q, const double *k, const double *v, const double *dout, double *dq,
                               double *dk, double *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);
void orc_backward_causal_poly2_rows(const double *q, const double *k, const double *v, const double *dout,
                                    const int64_t *rq, int64_t nq, const int64_t *rk, int64_t nk, double *dq,
                                    double *dk, double *dv, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M);

static uint64_t state = 0x9E3779B97F4A7C15ull;

static double draw(void) {   /* xorshift64*, mapped to [-2, 2) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0 * 4.0 - 2.0;
}

static double *arr(int64_t n, int fill) {
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    if (!p) exit(3);
    for (int64_t i = 0; i < n; ++i) p[i] = fill ? draw() : 0.0;
    return p;
}

static int finite_all(const double *p, int64_t n, const char *what) {
    for (int64_t i = 0; i < n; ++i)
        if (!isfinite(p[i])) {
            fprintf(stderr, "%s: element %lld is not finite\n", what, (long long)i);
            return 0;
        }
    return 1;
}

static int run(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M) {
    const int64_t nq = B * H * N * D, nv = B * H * N * M, ns = B * H * D * M, nz = B * H * D;
    double *q = arr(nq, 1), *k = arr(nq, 1), *v = arr(nv, 1), *g = arr(nv, 1);
    double *out = arr(nv, 0), *den = arr(B * H * N, 0), *S = arr(ns, 1), *Z = arr(nz, 0);
    double *dq = arr(nq, 0), *dk = arr(nq, 0), *dv = arr(nv, 0), *y = arr(nq, 0), *dy = arr(nq, 0);
    int ok = 1;
    for (int64_t i = 0; i < nz; ++i) Z[i] = 1.0 + fabs(draw());   /* a reachable start state */
    orc_feature_map(q, y, dy, nq);
    ok &= finite_all(y, nq, "phi") & finite_all(dy, nq, "phi'");
    orc_forward_causal(q, k, v, out, NULL, NULL, NULL, B, H, N, D, M);
    ok &= finite_all(out, nv, "forward_causal");
    orc_forward_causal(q, k, v, out, S, Z, den, B, H, N, D, M);
    ok &= finite_all(out, nv, "forward_causal from a state") & finite_all(S, ns, "S_N") &
          finite_all(den, B * H * N, "den");
    orc_forward_noncausal(q, k, v, out, B, H, N, D, M);
    ok &= finite_all(out, nv, "forward_noncausal");
    orc_backward_causal(q, k, v, g, dq, dk, dv, B, H, N, D, M);
    ok &= finite_all(dq, nq, "dq") & finite_all(dk, nq, "dk") & finite_all(dv, nv, "dv");
    orc_backward_noncausal(q, k, v, g, dq, dk, dv, B, H, N, D, M);
    ok &= finite_all(dq, nq, "dq nc") & finite_all(dk, nq, "dk nc") & finite_all(dv, nv, "dv nc");
    {   /* random features, R = M, then attention on positive-shifted features */
        double *om = arr(D * M, 1), *b = arr(M, 1), *f = arr(B * H * N * M, 0);
        orc_rff_features(q, om, b, f, B * H * N, D, M);
        ok &= finite_all(f, B * H * N * M, "rff");
        for (int64_t i = 0; i < B * H * N * M; ++i) f[i] = 2.0 + f[i];
        orc_forward_causal_features(f, f, v, out, B, H, N, M, M);
        ok &= finite_all(out, nv, "forward on features");
        free(om); free(b); free(f);
    }
    orc_forward_causal_poly2(q, k, v, out, B, H, N, D, M);   /* (q.k)^2 may vanish: no finiteness check */
    orc_backward_causal_poly2(q, k, v, g, dq, dk, dv, B, H, N, D, M);   /* likewise */
    {   /* the first and last rows, each summed on its own */
        const int64_t rq[2] = {0, N - 1}, rk[2] = {N - 1, N > 1 ? N - 2 : 0};
        double *sq = arr(B * H * 2 * D, 0), *sk = arr(B * H * 2 * D, 0), *sv = arr(B * H * 2 * M, 0);
        orc_backward_causal_poly2_rows(q, k, v, g, rq, 2, rk, 2, sq, sk, sv, B, H, N, D, M);
        free(sq); free(sk); free(sv);
    }
    for (int64_t i = 0; i < ns; ++i) S[i] = 0.0;
    for (int64_t i = 0; i < nz; ++i) Z[i] = 0.0;
    for (int64_t t = 0; t < 3; ++t) {
        orc_decode_step(q, k, v, S, Z, out, B, H, D, M);
        ok &= finite_all(out, B * H * M, "decode");
    }
    free(q); free(k); free(v); free(g); free(out); free(den); free(S); free(Z);
    free(dq); free(dk); free(dv); free(y); free(dy);
    return ok;
}

int main(void) {
    static const int64_t shapes[][5] = {{1, 1, 1, 1, 1}, {1, 2, 17, 3, 5}, {2, 1, 33, 4, 2}, {1, 1, 64, 8, 8}};
    int ok = 1;
    for (size_t i = 0; i < sizeof shapes / sizeof shapes[0]; ++i)
        ok &= run(shapes[i][0], shapes[i][1], shapes[i][2], shapes[i][3], shapes[i][4]);
    printf(ok ? "oracle sanity: ok\n" : "oracle sanity: FAILED\n");
    return ok ? 0 : 1;
}
