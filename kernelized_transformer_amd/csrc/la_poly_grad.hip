// la_poly_grad.hip -- gradient of the causal forward with the degree-2
// polynomial kernel on gfx950.
//
// [summary] 3.2.1 (sim(q, k) = (q . k)^2 has an exact finite feature map)
// and 3.3.1 (the gradient of the linear form takes linear time and constant
// memory, with running sums in both directions).  With s_ij = (q_i . k_j)^2
// for j <= i, d_i = sum_j s_ij and out_i = sum_j s_ij v_j / d_i, the chain
// rule gives dL/ds_ij = e_ij = w_i . u_j with
//   w_i = [g_i, h_i],  g_i = dout_i / d_i,  h_i = -(dout_i . out_i) / d_i,
//   u_j = [v_j, 1]    (M + 1 columns, the last one the normalizer),
// and then
//   dq_i = 2 sum_{j<=i} e_ij (q_i . k_j) k_j = 2 sum_m w_im A_i^(m) q_i,
//          A_i^(m) = sum_{j<=i} u_jm k_j k_j^T                (D x D each);
//   dk_j = 2 sum_{i>=j} e_ij (q_i . k_j) q_i = 2 sum_m u_jm B_j^(m) k_j,
//          B_j^(m) = sum_{i>=j} w_im q_i q_i^T;
//   dv_jm = sum_{i>=j} s_ij g_im = k_j^T B_j^(m) k_j          (m < M).
// Both directions are one computation, run twice: a "query" row x_a reads
// out against the running sum over the "key" rows y_b of the past (b <= a
// forwards, b >= a backwards), C^(m) = sum_b u_bm y_b y_b^T, giving
//   p_a = sum_m w_am C^(m) x_a (plus the chunk's own pairs)  and
//   r_am = x_a^T C^(m) x_a (plus the chunk's own pairs).
// Forwards: x = q, y = k, u = [v, 1], w = [g, h]: 2 p = dq.  Backwards:
// x = k, y = q, u = [g, h], w = [v, 1]: 2 p = dk and r = dv.
//
// Precision.  The gradient is a sum of terms that cancel (sum_j s_ij e_ij
// = 0 for every i, and at N = 65536 the cancelled sums are tens of times the
// result), so out and d are not taken from the polynomial forward (its state
// enters the readout rounded to bf16): the forwards direction first reads
// them out of the same sums its dq pass then uses, which keeps the
// cancellation exact to the sums' precision.  Taking them from the forward
// gave dq errors of 13% at B1 H8 N65536 D = M = 32 bf16.  fp32 I/O runs on
// the fp32 matrix instruction.  bf16 I/O rounds the state and u y to bf16
// operands, as the forward's state is, and carries the chunk's pair weights
// as bf16 hi + lo parts paired with the exact bf16 rows in one 32-deep
// instruction per tile ([y, y] . [hi, lo]).  Measured on the bf16 parity
// cases: dq, dk, dv errors of 2.0e-3 to 3.8e-3 (per 16-row chunk), against
// 1.7e-3 to 2.1e-3 with the state and u y split as well (23% slower).
//
// Launches, forwards: the segments' sums of C, their exclusive prefixes,
// the readout (the forward's numerators and denominators), the weights w,
// the dq pass (these three as one pass when one workgroup holds every column)
// and the sum over the column blocks; backwards: the segments' sums, their
// exclusive suffixes, the dk / dv pass and the sum.  The state is kept
// as plain D x D fp32 matrices (one per column m) in accumulator tiles:
// a workgroup of 11 wavefronts owns one segment and a block of 11 NMW
// columns m (NMW = 3 at D = 32, 1 at D = 64, i.e. 48 or 64 state registers
// per wavefront), so that M + 1 = 33 or 65 columns fill one to six blocks.
// Per 16-row chunk each wavefront forms, for its columns, T = x C^(m)
// (matrix cores, the state as the operand), its share of p (T scaled by
// w_am) and of r, its share of the chunk's own pairs (scores x . y on the
// matrix cores, masked to the past, weighted by its columns' u . w), and
// the update C^(m) += y^T diag(u_m) y.  The wavefronts' partial p meet in
// LDS (added in wavefront order); the column blocks' partial p go to the
// workspace and are added in block order by the last launch, so results
// do not vary from run to run.
#include <type_traits>

#include "la_chunk.h"
#include "la_internal.h"
#include "la_poly_grad.h"

namespace la {

namespace {

constexpr int kPgWaves = 11;
constexpr int kPgThreads = 64 * kPgWaves;

template <int D> struct PgCfg {
    static constexpr int DT = D / 16;                 // 16-row tiles of D
    static constexpr int NMW = D == 32 ? 3 : 1;       // columns m per wavefront
    static constexpr int MBK = kPgWaves * NMW;        // columns m per workgroup
    static constexpr int XS = D + 4;                  // floats per staged row
    static constexpr int US = MBK + 1;                // floats per staged u, w row
};

__host__ __device__ constexpr int64_t pg_blocks(int64_t D, int64_t M) {
    return (M + 1 + kPgWaves * (D == 32 ? 3 : 1) - 1) / (kPgWaves * (D == 32 ? 3 : 1));
}

template <typename T> __device__ __forceinline__ float ld1(const T *p) { return static_cast<float>(*p); }

// acc += A B^T over one 16-wide tile, A exact in bf16 and B split into bf16
// hi + lo parts: [a, a] . [hi, lo] = a (hi + lo) in one 32-deep instruction.
// fp32 operands: the fp32 instruction.
__device__ __forceinline__ void mma_xs(f32x4 &acc, bf16x4 a, split4 b) {
    const bf16x8 aa = __builtin_shufflevector(a, a, 0, 1, 2, 3, 0, 1, 2, 3);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aa, b.hl, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_xs(f32x4 &acc, f32x4 a, f32x4 b) { mma1(acc, a, b); }

// Element (token t, column m) of u or w: from V ([v, 1]) or from the weights
// buffer ([g, h]).
template <typename T, bool FROM_V, int M>
__device__ __forceinline__ float col_value(const T *V, const float *Wb, int row, int m) {
    if constexpr (FROM_V) return m < M ? ld1<T>(V + row * M + m) : 1.f;
    else return Wb[row * (M + 1) + m];
}

// DIR 0: forwards (x = q, y = k, u = [v, 1], w = [g, h]); DIR 1: backwards
// (x = k, y = q, u = [g, h], w = [v, 1]).  SEG: only sum the segment's
// C^(m) from zero and store it (no x, no outputs).
// RMODE (passes): 0 p only; 1 p and r for m < M into dv (backwards); 2 r for
// every m <= M into rb (fp32, [BH][N][M + 1]) and no p: the readout of the
// forward itself, numerators and denominator, from the same sums the dq pass
// uses; 3 (forwards, all M + 1 columns in one workgroup) both in one pass:
// per chunk the readout r, then w = [dout / d, -(dout . out) / d] from it in
// LDS (also stored to rb for the backwards direction), then p.
template <typename T, int D, int M, int DIR, bool SEG, int RMODE = 0>
__global__ __launch_bounds__(kPgThreads) void k_pg(const T *__restrict__ X, const T *__restrict__ Y,
                                                   const T *__restrict__ V, const float *__restrict__ Wb,
                                                   const T *__restrict__ Gd, float *__restrict__ recs,
                                                   float *__restrict__ pbuf,
                                                   T *__restrict__ dv, float *__restrict__ rb, int64_t N,
                                                   int64_t nseg, int64_t seg_tokens, int64_t BH) {
    typedef PgCfg<D> C;
    // XF: operands exact in the I/O type (x, y); SF: computed ones (the
    // state, u y, the chunk's pair weights), split into hi + lo for bf16
    typedef typename std::conditional<sizeof(T) == 2, bf16x4, f32x4>::type XF;
    typedef typename std::conditional<sizeof(T) == 2, split4, f32x4>::type SF;
    constexpr int DT = C::DT, NMW = C::NMW, MBK = C::MBK, XS = C::XS, US = C::US;
    constexpr int64_t REC = int64_t(M + 1) * D * D;
    constexpr int NMB = int(pg_blocks(D, M));
    constexpr bool U_FROM_V = DIR == 0, W_FROM_V = DIR == 1;
    constexpr bool P_OUT = !SEG && RMODE != 2;   // p formed (and w staged; dout for RMODE 3)
    static_assert(RMODE != 3 || (DIR == 0 && NMB == 1), "the fused readout needs every column in the workgroup");

    __shared__ __align__(16) float xs[SEG ? 4 : 16 * XS];
    __shared__ __align__(16) float ys[16 * XS];
    __shared__ float us[16 * US];
    __shared__ float wsh[P_OUT ? 16 * US : 1];
    __shared__ f32x4 pred[P_OUT ? kPgWaves * DT * 64 : 1];
    __shared__ float rsh[RMODE == 3 ? 16 * US : 1];

    const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int mb = int(blockIdx.x % NMB);
    const int64_t seg = (blockIdx.x / NMB) % nseg, bh = blockIdx.x / NMB / nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const int64_t nch = (t_end - t_begin + 15) / 16;
    const T *Xh = X + bh * N * D;
    const T *Yh = Y + bh * N * D;
    const T *Vh = V + bh * N * M;
    const float *Wh = Wb + bh * N * (M + 1);
    float *rec = recs ? recs + (bh * nseg + seg) * REC : nullptr;

    // this wavefront's columns: m = mb MBK + wave NMW + k, valid while m <= M
    f32x4 A[NMW][DT][DT];
#pragma unroll
    for (int k = 0; k < NMW; ++k) {
        const int m = mb * MBK + wave * NMW + k;
#pragma unroll
        for (int db = 0; db < DT; ++db)
#pragma unroll
            for (int eb = 0; eb < DT; ++eb)
                A[k][db][eb] = (!SEG && rec && m <= M)
                                   ? reinterpret_cast<const f32x4 *>(rec + int64_t(m) * D * D +
                                                                     (db * DT + eb) * 256)[lane]
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Each thread moves at most NY elements of the chunk's x and y rows and NU
    // of its u and w columns.  The rows of the next PF chunks are in flight in
    // PF register slots while a chunk is worked on, so their latency is hidden
    // behind PF chunks of work.
    constexpr int NY = (16 * D + kPgThreads - 1) / kPgThreads, NU = (16 * MBK + kPgThreads - 1) / kPgThreads;
    constexpr int PF = SEG ? 4 : 2;   // 2 or 4 (the passes hold more registers)
    float ry[PF][NY], rx[PF][NY], ru[PF][NU], rw[PF][NU];
    // (row addresses: the chunk's base is uniform, each element a 32-bit offset from it)
    auto fetch = [&](int64_t ci, float(&fy)[NY], float(&fx)[NY], float(&fu)[NU], float(&fw)[NU]) {
        const int64_t t0 = t_begin + 16 * (DIR == 0 ? ci : nch - 1 - ci);
        const bool live = ci < nch;
        const int rem = live ? int(imin64(16, t_end - t0)) : 0;   // rows present
        const T *yb = Yh + (live ? t0 : 0) * D, *xb = Xh + (live ? t0 : 0) * D;
        const T *vb = Vh + (live ? t0 : 0) * M;
        const float *wb = Wh + (live ? t0 : 0) * (M + 1);
        const T *gb = Gd + (RMODE == 3 && live ? t0 * M + int64_t(bh) * N * M : 0);
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            const int e = tid + i * kPgThreads, row = e / D;
            const bool on = e < 16 * D && row < rem;
            fy[i] = on ? ld1<T>(yb + e) : 0.f;
            if constexpr (!SEG) fx[i] = on ? ld1<T>(xb + e) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = tid + i * kPgThreads, row = e / MBK, j = e % MBK, m = mb * MBK + j;
            const bool on = e < 16 * MBK && row < rem && m <= M;
            fu[i] = on ? col_value<T, U_FROM_V, M>(vb, wb, row, m) : 0.f;
            if constexpr (RMODE == 3) fw[i] = on && m < M ? ld1<T>(gb + row * M + m) : 0.f;
            else if constexpr (P_OUT) fw[i] = on ? col_value<T, W_FROM_V, M>(vb, wb, row, m) : 0.f;
        }
    };
    fetch(0, ry[0], rx[0], ru[0], rw[0]);
    fetch(1, ry[1], rx[1], ru[1], rw[1]);
    if constexpr (PF > 2) {
        fetch(2, ry[2], rx[2], ru[2], rw[2]);
        fetch(3, ry[3], rx[3], ru[3], rw[3]);
    }
    // chunks in groups of PF, chunk c0 + U staged from register slot U, which
    // is then refilled with chunk c0 + U + PF (slots fixed at compile time)
    auto step = [&](int64_t ci, auto uc) {
        constexpr int U = decltype(uc)::value;
        const int64_t cc = DIR == 0 ? ci : nch - 1 - ci;
        const int64_t t0 = t_begin + 16 * cc;
        __syncthreads();   // the previous chunk's LDS reads are done
#pragma unroll
        for (int i = 0; i < NY; ++i) {
            const int e = tid + i * kPgThreads, row = e / D, col = e % D;
            if (e < 16 * D) {
                ys[row * XS + col] = ry[U][i];
                if constexpr (!SEG) xs[row * XS + col] = rx[U][i];
            }
        }
#pragma unroll
        for (int i = 0; i < NU; ++i) {
            const int e = tid + i * kPgThreads, row = e / MBK, j = e % MBK;
            if (e < 16 * MBK) {
                us[row * US + j] = ru[U][i];
                if constexpr (P_OUT) wsh[row * US + j] = rw[U][i];
            }
        }
        __syncthreads();
        fetch(ci + PF, ry[U], rx[U], ru[U], rw[U]);

        // y as token-contiguous tiles: lane (c, g) element r = y[4g + r][16 db + c]
        f32x4 ytf[DT];
#pragma unroll
        for (int db = 0; db < DT; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) ytf[db][r] = ys[(4 * g + r) * XS + 16 * db + c];
        XF yt[DT];
#pragma unroll
        for (int db = 0; db < DT; ++db) yt[db] = frag_from<XF>(ytf[db]);
        float u[NMW][4];
#pragma unroll
        for (int k = 0; k < NMW; ++k)
#pragma unroll
            for (int r = 0; r < 4; ++r) u[k][r] = us[(4 * g + r) * US + wave * NMW + k];

        if constexpr (!SEG) {
            // x and y as row tiles: lane (c, g) element r = x[c][16 db + 4g + r]
            f32x4 xf[DT];
            XF xn[DT], yn[DT];
#pragma unroll
            for (int db = 0; db < DT; ++db) {
                xf[db] = *reinterpret_cast<const f32x4 *>(&xs[c * XS + 16 * db + 4 * g]);
                xn[db] = frag_from<XF>(xf[db]);
                yn[db] = frag_from<XF>(*reinterpret_cast<const f32x4 *>(&ys[c * XS + 16 * db + 4 * g]));
            }
            // scores: lane (c, g) element r = x_c . y_{4g + r}, kept where b = 4g + r
            // lies in a's past (b <= a forwards, b >= a backwards)
            f32x4 P = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int db = 0; db < DT; db += 2) mma2(P, yn[db], yn[db + 1], xn[db], xn[db + 1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int b = 4 * g + r;
                if (DIR == 0 ? b > c : b < c) P[r] = 0.f;
            }
            f32x4 pacc[DT];
#pragma unroll
            for (int eb = 0; eb < DT; ++eb) pacc[eb] = f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 E = {0.f, 0.f, 0.f, 0.f};
            if constexpr (RMODE == 3) {
                // 1. T and the readout r_m of every column; wsh holds this chunk's dout
                f32x4 tk[NMW][DT];
#pragma unroll
                for (int k = 0; k < NMW; ++k) {
                    const int m = wave * NMW + k;
                    if (m > M) continue;   // uniform per wavefront
                    float rv = 0.f;
#pragma unroll
                    for (int eb = 0; eb < DT; ++eb) {
                        tk[k][eb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int db = 0; db < DT; db += 2)
                            mma2(tk[k][eb], frag_from<XF>(A[k][db][eb]), frag_from<XF>(A[k][db + 1][eb]), xn[db],
                                 xn[db + 1]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) rv += tk[k][eb][r] * xf[eb][r];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) rv += P[r] * P[r] * u[k][r];
                    rv += __shfl_xor(rv, 16);
                    rv += __shfl_xor(rv, 32);
                    if (g == 0) rsh[c * US + m] = rv;
                }
                __syncthreads();
                // 2. w per token (zero past the end), in place of dout in wsh
                if (tid < 16) {
                    const int64_t t = t0 + tid;
                    float *wr = wsh + tid * US;
                    const float *rr = rsh + tid * US;
                    if (t < t_end) {
                        const float inv = 1.f / rr[M];
                        float go = 0.f;
                        for (int m = 0; m < M; ++m) {
                            const float gm = wr[m];
                            go += gm * (rr[m] * inv);
                            wr[m] = gm * inv;
                            rb[(bh * N + t) * (M + 1) + m] = wr[m];
                        }
                        wr[M] = -go * inv;
                        rb[(bh * N + t) * (M + 1) + M] = wr[M];
                    } else {
                        for (int m = 0; m <= M; ++m) wr[m] = 0.f;
                    }
                }
                __syncthreads();
                // 3. p from the kept T
#pragma unroll
                for (int k = 0; k < NMW; ++k) {
                    const int m = wave * NMW + k;
                    if (m > M) continue;
                    const float wa = wsh[c * US + m];
#pragma unroll
                    for (int eb = 0; eb < DT; ++eb) pacc[eb] += wa * tk[k][eb];
#pragma unroll
                    for (int r = 0; r < 4; ++r) E[r] += u[k][r] * wa;
                }
            } else {
#pragma unroll
            for (int k = 0; k < NMW; ++k) {
                const int m = mb * MBK + wave * NMW + k;
                if (m > M) continue;   // uniform per wavefront
                const float wa = P_OUT ? wsh[c * US + wave * NMW + k] : 0.f;
                float rv = 0.f;
#pragma unroll
                for (int eb = 0; eb < DT; ++eb) {
                    // T[a = c][e = 16 eb + 4g + r] = sum_d x[c][d] C[d][e]
                    f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int db = 0; db < DT; db += 2)
                        mma2(t, frag_from<XF>(A[k][db][eb]), frag_from<XF>(A[k][db + 1][eb]), xn[db], xn[db + 1]);
                    if constexpr (P_OUT) pacc[eb] += wa * t;
                    if constexpr (RMODE != 0) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) rv += t[r] * xf[eb][r];
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) E[r] += u[k][r] * wa;
                if constexpr (RMODE != 0) {
                    if (RMODE == 2 || m < M) {
                        // r_am: the state part (lanes of every g) and the chunk's own pairs
#pragma unroll
                        for (int r = 0; r < 4; ++r) rv += P[r] * P[r] * u[k][r];
                        rv += __shfl_xor(rv, 16);
                        rv += __shfl_xor(rv, 32);
                        const int64_t t = t0 + c;
                        if (g == 0 && t < t_end) {
                            if constexpr (RMODE == 1) dv[(bh * N + t) * M + m] = static_cast<T>(rv);
                            else rb[(bh * N + t) * (M + 1) + m] = rv;
                        }
                    }
                }
            }
            }   // RMODE
            if constexpr (P_OUT) {
            // the chunk's own pairs: p_a += sum_b (u_b . w_a) (x_a . y_b) y_b
            f32x4 Z;
#pragma unroll
            for (int r = 0; r < 4; ++r) Z[r] = E[r] * P[r];
            const SF zf = frag_from<SF>(Z);
#pragma unroll
            for (int eb = 0; eb < DT; ++eb) mma_xs(pacc[eb], yt[eb], zf);

            // partial p of the wavefronts, added in wavefront order
#pragma unroll
            for (int eb = 0; eb < DT; ++eb) pred[(wave * DT + eb) * 64 + lane] = pacc[eb];
            __syncthreads();
            for (int e = tid; e < DT * 64; e += kPgThreads) {
                const int eb = e / 64, ln = e % 64, a = ln & 15, ga = ln >> 4;
                f32x4 sum = pred[eb * 64 + ln];
                for (int w2 = 1; w2 < kPgWaves; ++w2) sum += pred[(w2 * DT + eb) * 64 + ln];
                const int64_t t = t0 + a;
                if (t < t_end)
                    *reinterpret_cast<f32x4 *>(pbuf + ((int64_t(mb) * BH + bh) * N + t) * D + 16 * eb + 4 * ga) = sum;
            }
            }   // P_OUT
        }

        // C^(m) += y^T diag(u_m) y over the chunk
#pragma unroll
        for (int k = 0; k < NMW; ++k) {
            const int m = mb * MBK + wave * NMW + k;
            if (m > M) continue;
#pragma unroll
            for (int eb = 0; eb < DT; ++eb) {
                f32x4 sy;
#pragma unroll
                for (int r = 0; r < 4; ++r) sy[r] = ytf[eb][r] * u[k][r];
                const XF sf = frag_from<XF>(sy);
#pragma unroll
                for (int db = 0; db < DT; ++db) mma1(A[k][db][eb], yt[db], sf);
            }
        }
    };
    for (int64_t c0 = 0; c0 < nch; c0 += PF) {
        step(c0, std::integral_constant<int, 0>());
        if (c0 + 1 < nch) step(c0 + 1, std::integral_constant<int, 1>());
        if constexpr (PF > 2) {
            if (c0 + 2 < nch) step(c0 + 2, std::integral_constant<int, 2>());
            if (c0 + 3 < nch) step(c0 + 3, std::integral_constant<int, 3>());
        }
    }

    if constexpr (SEG) {
#pragma unroll
        for (int k = 0; k < NMW; ++k) {
            const int m = mb * MBK + wave * NMW + k;
            if (m > M) continue;
#pragma unroll
            for (int db = 0; db < DT; ++db)
#pragma unroll
                for (int eb = 0; eb < DT; ++eb)
                    reinterpret_cast<f32x4 *>(rec + int64_t(m) * D * D + (db * DT + eb) * 256)[lane] = A[k][db][eb];
        }
    }
}

// w = [dout / d, -(dout . out) / d] per token from the readout r = [n, d]
// (out = n / d), in place: row t of rw holds r on entry and w on exit.  One
// thread per token.
template <typename T, int M>
__global__ __launch_bounds__(256) void k_pg_weights(const T *__restrict__ dout, float *__restrict__ rw,
                                                    int64_t rows) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (t >= rows) return;
    float *row = rw + t * (M + 1);
    const float inv = 1.f / row[M];
    float go = 0.f;
    for (int m = 0; m < M; ++m) {
        const float gm = static_cast<float>(dout[t * M + m]);
        go += gm * (row[m] * inv);
        row[m] = gm * inv;
    }
    row[M] = -go * inv;
}

// grad = 2 * (sum over the column blocks of the partial p), block order.
template <typename T, int D>
__global__ __launch_bounds__(256) void k_pg_sum(const float *__restrict__ pbuf, T *__restrict__ grad, int64_t n4,
                                                int nmb) {
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i >= n4) return;
    f32x4 s = reinterpret_cast<const f32x4 *>(pbuf)[i];
    for (int b = 1; b < nmb; ++b) s += reinterpret_cast<const f32x4 *>(pbuf)[int64_t(b) * n4 + i];
    store4<T>(grad + 4 * i, IO<T>::from_f32(2.f * s));
}

struct PgPlan {
    int64_t nmb = 1, nseg = 1, seg_tokens = 16, rec = 0;
    size_t w_off = 0, rec_off = 0, p_off = 0, total = 0;
};

PgPlan make_pg_plan(int64_t BH, int64_t N, int64_t D, int64_t M) {
    PgPlan p;
    p.nmb = pg_blocks(D, M);
    p.rec = (M + 1) * D * D;
    const int64_t nch = ceil_div(N, kChunk);
    int64_t nseg = ceil_div(int64_t(device_cus()), BH * p.nmb);
    nseg = std::max<int64_t>(1, std::min<int64_t>({nseg, nch, kMaxSegPerHead}));
    p.seg_tokens = ceil_div(nch, nseg) * kChunk;
    p.nseg = ceil_div(N, p.seg_tokens);
    size_t off = 256;
    p.w_off = off;   // the readout [n, d], then the weights [g, h], per token
    off += align256(size_t(BH * N * (M + 1)) * 4);
    p.rec_off = off;
    off += p.nseg > 1 ? align256(size_t(BH * p.nseg * p.rec) * 4) : 0;
    p.p_off = off;
    off += align256(size_t(p.nmb * BH * N * D) * 4);
    p.total = off;
    return p;
}

template <typename T, int D, int M>
hipError_t run_pg(const void *q, const void *k, const void *v, const void *dout, void *dq, void *dk, void *dv,
                  int64_t BH, int64_t N, void *ws, hipStream_t s) {
    const PgPlan p = make_pg_plan(BH, N, D, M);
    char *base = static_cast<char *>(ws);
    float *Wb = reinterpret_cast<float *>(base + p.w_off);
    float *recs = p.nseg > 1 ? reinterpret_cast<float *>(base + p.rec_off) : nullptr;
    float *pbuf = reinterpret_cast<float *>(base + p.p_off);
    const T *Q = static_cast<const T *>(q), *K = static_cast<const T *>(k), *V = static_cast<const T *>(v);
    const dim3 grid(unsigned(BH * p.nseg * p.nmb)), block(kPgThreads);
    const int64_t rows = BH * N, n4 = BH * N * D / 4;
    const dim3 gsum(unsigned(ceil_div(n4, 256)));
    hipError_t e;
    // forwards: the segments' sums of [v, 1]_m k k^T and their prefixes, the
    // readout (numerators and denominators), the weights, dq
    if (p.nseg > 1) {
        hipLaunchKernelGGL((k_pg<T, D, M, 0, true>), grid, block, 0, s, Q, K, V, (const float *)Wb, (const T *)nullptr, recs,
                           (float *)nullptr, (T *)nullptr, (float *)nullptr, N, p.nseg, p.seg_tokens, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_scan(recs, BH, p.nseg, p.rec, 0, s)) != hipSuccess) return e;
    }
    if constexpr (pg_blocks(D, M) == 1) {
        // every column in one workgroup: readout, weights and dq in one pass
        hipLaunchKernelGGL((k_pg<T, D, M, 0, false, 3>), grid, block, 0, s, Q, K, V, (const float *)nullptr,
                           static_cast<const T *>(dout), recs, pbuf, (T *)nullptr, Wb, N, p.nseg, p.seg_tokens, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
        hipLaunchKernelGGL((k_pg<T, D, M, 0, false, 2>), grid, block, 0, s, Q, K, V, (const float *)Wb, (const T *)nullptr, recs,
                           (float *)nullptr, (T *)nullptr, Wb, N, p.nseg, p.seg_tokens, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_pg_weights<T, M>), dim3(unsigned(ceil_div(rows, 256))), dim3(256), 0, s,
                           static_cast<const T *>(dout), Wb, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((k_pg<T, D, M, 0, false, 0>), grid, block, 0, s, Q, K, V, (const float *)Wb, (const T *)nullptr, recs, pbuf,
                           (T *)nullptr, (float *)nullptr, N, p.nseg, p.seg_tokens, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_pg_sum<T, D>), gsum, dim3(256), 0, s, (const float *)pbuf, static_cast<T *>(dq), n4,
                       int(p.nmb));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // backwards: the segments' sums of [g, h]_m q q^T and their suffixes, dk and dv
    if (p.nseg > 1) {
        hipLaunchKernelGGL((k_pg<T, D, M, 1, true>), grid, block, 0, s, K, Q, V, (const float *)Wb, (const T *)nullptr, recs,
                           (float *)nullptr, (T *)nullptr, (float *)nullptr, N, p.nseg, p.seg_tokens, BH);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_scan(recs, BH, p.nseg, p.rec, 2, s)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_pg<T, D, M, 1, false, 1>), grid, block, 0, s, K, Q, V, (const float *)Wb, (const T *)nullptr, recs, pbuf,
                       static_cast<T *>(dv), (float *)nullptr, N, p.nseg, p.seg_tokens, BH);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((k_pg_sum<T, D>), gsum, dim3(256), 0, s, (const float *)pbuf, static_cast<T *>(dk), n4,
                       int(p.nmb));
    return hipGetLastError();
}

template <typename T>
hipError_t run_pg_t(int dt, const void *q, const void *k, const void *v, const void *dout, void *dq, void *dk,
                    void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, void *ws, hipStream_t s) {
    if (D == 32 && M == 32) return run_pg<T, 32, 32>(q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 32 && M == 64) return run_pg<T, 32, 64>(q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 64 && M == 32) return run_pg<T, 64, 32>(q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 64 && M == 64) return run_pg<T, 64, 64>(q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    return hipErrorInvalidValue;
}

} // namespace

size_t poly_backward_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, size_t esize) {
    if (!poly_head_sizes(D, M)) return 0;
    (void)esize;
    return make_pg_plan(BH, N, D, M).total;
}

hipError_t launch_poly_backward(int dt, const void *q, const void *k, const void *v, const void *dout, void *dq,
                                void *dk, void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, void *ws,
                                hipStream_t s) {
    if (!poly_head_sizes(D, M)) return hipErrorInvalidValue;
    if (dt == 0) return run_pg_t<float>(dt, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
    return run_pg_t<bf16>(dt, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
}

} // namespace la
