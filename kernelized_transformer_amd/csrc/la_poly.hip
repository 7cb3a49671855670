// la_poly.hip -- causal attention with the degree-2 polynomial kernel on gfx950.
//
// [summary] 3.2.1: a degree-2 polynomial kernel has an exact finite feature
// map.  Reading: sim(q, k) = (q . k)^2, feature map phi(x) = vec(x x^T), so
//   out_i = sum_{j<=i} (q_i . k_j)^2 v_j / sum_{j<=i} (q_i . k_j)^2.
// The D^2 x M state sum_j phi(k_j) v_j^T is kept as M matrices of D x D,
//   S_m = sum_j v_jm k_j k_j^T,   Z = sum_j k_j k_j^T   (the normalizer),
// and phi(q) . vec(X) = q^T X q, so no feature vector is ever formed.
//
// Work split (D = 32): a workgroup of kPolyWaves wavefronts owns one segment
// of one (b, h) and a block of 32 output columns (M = 64 has two blocks per
// segment); wavefront w owns 4 of them, [cb 32 + 4w, cb 32 + 4w + 4), and
// carries their S_m plus its own copy of Z in registers (fp32 Acc tiles:
// 80 registers).  The wavefronts of a workgroup
// never wait for each other.  Per 16-token chunk, for each matrix X it holds:
//   readout  U^T = X^T Q^T on the matrix cores (rows b, cols tokens), then
//            C[i][i'] = sum_b U^T[b][i] q_i'b, whose diagonal is q_i^T X q_i;
//   intra    the same accumulator gets sum_j P[i][j] w(j), P = (Q K^T)^2
//            masked to j <= i, w(j) = v_jm (or 1 for Z): on the diagonal
//            this adds the chunk's own contribution;
//   update   X += (w o K)^T K (contraction over the chunk's tokens).
// out_im = diag of the S_m accumulator / diag of the Z accumulator.
// Segments: k_poly_segment_state sums each segment's matrices into a record
// ([M + 1][D][D] fp32: S_0 .. S_{M-1}, Z), the shared scan turns them into
// exclusive prefixes, and k_poly_output starts each segment from its prefix.
#include "la_chunk.h"
#include "la_internal.h"

namespace la {

constexpr int kPolyWaves = 8;
constexpr int kPolyD = 32;

constexpr int kPolyCols = 32;   // output columns per workgroup

template <typename T, int M> struct PolyCfg {
    typedef typename IO<T>::frag Fr;
    static constexpr int D = kPolyD, DT = D / 16;
    static constexpr int MW = kPolyCols / kPolyWaves;   // output columns per wavefront
    static constexpr int NX = MW + 1;                   // its matrices: S_m of its columns, then Z
    static constexpr int CB = M / kPolyCols;            // column blocks per segment
};

// Load / store / zero a wavefront's matrices: matrix x of the wavefront is
// record matrix m0 + x (x < MW) or M (Z, x = MW).  Tile (at, bt), lane
// (c, g), element r <-> rec[mat][16 at + 4g + r][16 bt + c].
template <int M, int NX>
__device__ __forceinline__ void poly_load(f32x4 (&X)[NX][2][2], const float *rec, int m0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        const float *mat = rec + int64_t(x < NX - 1 ? m0 + x : M) * kPolyD * kPolyD;
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
            for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                for (int r = 0; r < 4; ++r) X[x][at][bt][r] = mat[(16 * at + 4 * g + r) * kPolyD + 16 * bt + c];
    }
}
template <int M, int NX>
__device__ __forceinline__ void poly_store(float *rec, const f32x4 (&X)[NX][2][2], int m0, bool with_z) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        if (x < NX - 1 || with_z) {
            float *mat = rec + int64_t(x < NX - 1 ? m0 + x : M) * kPolyD * kPolyD;
#pragma unroll
            for (int at = 0; at < 2; ++at)
#pragma unroll
                for (int bt = 0; bt < 2; ++bt)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        mat[(16 * at + 4 * g + r) * kPolyD + 16 * bt + c] = X[x][at][bt][r];
        }
    }
}

// Two consecutive chunks (32 tokens from t0) as one wavefront needs them.
// Rows at or beyond t_end read row t_end - 1 (addresses: a uniform base
// pointer per pair plus 32-bit lane offsets).
template <typename T, int M> struct PolyPair {
    typedef PolyCfg<T, M> C;
    typedef typename IO<T>::vec4 V4;
    V4 rq[2][C::DT], rk[2][C::DT];   // natural rows: token 16h + c, features 16 ft + 4g ..
    V4 rv[2][4];                     // rv[h][r] = v[t0 + 16h + 4g + r][m0 .. m0 + 3]

    __device__ __forceinline__ void load(const T *Qh, const T *Kh, const T *Vh, int64_t t0, int64_t t_end, int m0,
                                         bool with_q) {
        const int c = lane_id() & 15, g = lane_id() >> 4;
        const int lim = int(min<int64_t>(t_end - 1 - t0, 64));   // last valid row, relative (may be < 0)
        const T *qb = Qh + t0 * kPolyD, *kb = Kh + t0 * kPolyD, *vb = Vh + t0 * M;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = min(16 * h + c, lim);
#pragma unroll
            for (int ft = 0; ft < C::DT; ++ft) {
                if (with_q) rq[h][ft] = load4<T>(qb + row * kPolyD + 16 * ft + 4 * g);
                rk[h][ft] = load4<T>(kb + row * kPolyD + 16 * ft + 4 * g);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) rv[h][r] = load4<T>(vb + min(16 * h + 4 * g + r, lim) * M + m0);
        }
    }
    // wv[h][x][r] = v[t0 + 16h + 4g + r][m0 + x]
    __device__ __forceinline__ void values(f32x4 (&wv)[2][C::MW]) const {
        static_assert(C::MW == 4, "four columns per wavefront");
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const f32x4 v4 = IO<T>::to_f32(rv[h][r]);
#pragma unroll
                for (int x = 0; x < 4; ++x) wv[h][x][r] = v4[x];
            }
    }
};

// Pairs of chunks in flight per wavefront (the loops are unrolled by this
// many so that pair i always lives in buffer i % PF).
template <typename T, int M> constexpr int poly_ahead() { return (sizeof(T) == 2 && M == 32) ? 2 : 1; }

// X += (w o K)^T K over the pair's 32 tokens (one 32-deep product per tile):
// KT[h] are token-contiguous K fragments of chunk h (lane (c, g):
// k[16h + 4g + r][16 at + c]), KTf the same in fp32.
template <typename T, int NX>
__device__ __forceinline__ void poly_update(f32x4 (&X)[NX][2][2], const typename IO<T>::frag (&KT)[2][kPolyD / 16],
                                            const f32x4 (&KTf)[2][kPolyD / 16], const f32x4 (&wv)[2][NX - 1],
                                            int nx) {
    typedef typename IO<T>::frag Fr;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        if (x < nx) {
#pragma unroll
            for (int at = 0; at < 2; ++at) {
                const Fr a0 = (x < NX - 1) ? IO<T>::to_frag(KTf[0][at] * wv[0][x]) : KT[0][at];
                const Fr a1 = (x < NX - 1) ? IO<T>::to_frag(KTf[1][at] * wv[1][x]) : KT[1][at];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) mma2(X[x][at][bt], a0, a1, KT[0][bt], KT[1][bt]);
            }
        }
    }
}

// Zero the token-contiguous rows (tokens 16h + 4g + r) at or beyond lim + 1.
template <typename T>
__device__ __forceinline__ void poly_mask_rows(typename IO<T>::frag (&KT)[2][kPolyD / 16], f32x4 (&KTf)[2][kPolyD / 16],
                                               int lim) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int ft = 0; ft < kPolyD / 16; ++ft) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * h + 4 * g + r > lim) KTf[h][ft][r] = 0.f;
            KT[h][ft] = IO<T>::to_frag(KTf[h][ft]);
        }
}

template <typename T, int M>
__global__ __launch_bounds__(64 * kPolyWaves) void k_poly_segment_state(const T *__restrict__ k,
                                                                        const T *__restrict__ v,
                                                                        float *__restrict__ ws, int64_t N,
                                                                        int64_t nseg, int64_t seg_tokens,
                                                                        int64_t rec) {
    typedef PolyCfg<T, M> C;
    typedef typename C::Fr Fr;
    const int wave = threadIdx.x >> 6;
    const int cb = blockIdx.x % C::CB;
    const int64_t bh = blockIdx.x / C::CB / nseg, seg = blockIdx.x / C::CB % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = min(N, t_begin + seg_tokens);
    const int m0 = cb * kPolyCols + wave * C::MW;
    const T *K = k + bh * N * kPolyD;
    const T *V = v + bh * N * M;
    __shared__ bf16 stage_mem[kPolyWaves][stage_elems<C::DT, 2>()];
    lds_bf16 *stage = (lds_bf16 *)stage_mem[wave];
    const bool owns_z = cb == 0 && wave == 0;   // Z is summed and stored once per segment

    f32x4 X[C::NX][2][2];
#pragma unroll
    for (int x = 0; x < C::NX; ++x)
#pragma unroll
        for (int at = 0; at < 2; ++at)
#pragma unroll
            for (int bt = 0; bt < 2; ++bt) X[x][at][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nx = owns_z ? C::NX : C::NX - 1;

    constexpr int PF = poly_ahead<T, M>();
    if (t_begin < t_end) {
        PolyPair<T, M> buf[PF];
#pragma unroll
        for (int b = 0; b < PF; ++b) buf[b].load(nullptr, K, V, t_begin + 32 * b, t_end, m0, false);
        for (int64_t t00 = t_begin; t00 < t_end; t00 += 32 * PF) {
#pragma unroll
            for (int b = 0; b < PF; ++b) {
                const int64_t t0 = t00 + 32 * b;   // may lie past t_end: every row masked, adds nothing
                Fr Kn[2][C::DT], KT[2][C::DT];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int ft = 0; ft < C::DT; ++ft) Kn[h][ft] = IO<T>::to_frag(IO<T>::to_f32(buf[b].rk[h][ft]));
                f32x4 wv[2][C::MW];
                buf[b].values(wv);
                buf[b].load(nullptr, K, V, t0 + 32 * PF, t_end, m0, false);
                transpose_frags<C::DT, 2>(KT, Kn, stage);
                f32x4 KTf[2][C::DT];
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int at = 0; at < C::DT; ++at) KTf[h][at] = IO<T>::to_f32(KT[h][at]);
                const int lim = int(min<int64_t>(t_end - 1 - t0, 64));
                if (lim < 31) poly_mask_rows<T>(KT, KTf, lim);   // the segment's last, partial pair
                poly_update<T, C::NX>(X, KT, KTf, wv, nx);
            }
        }
    }
    poly_store<M, C::NX>(ws + (bh * nseg + seg) * rec, X, m0, owns_z);
}

template <typename T, int M>
__global__ __launch_bounds__(64 * kPolyWaves) void k_poly_output(const T *__restrict__ q, const T *__restrict__ k,
                                                                 const T *__restrict__ v, T *__restrict__ out,
                                                                 const float *__restrict__ ws, int64_t N,
                                                                 int64_t nseg, int64_t seg_tokens, int64_t rec) {
    typedef PolyCfg<T, M> C;
    typedef typename C::Fr Fr;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int cb = blockIdx.x % C::CB;
    const int64_t bh = blockIdx.x / C::CB / nseg, seg = blockIdx.x / C::CB % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = min(N, t_begin + seg_tokens);
    if (t_begin >= t_end) return;   // whole workgroup: no barrier below
    const int m0 = cb * kPolyCols + wave * C::MW;
    const T *Q = q + bh * N * kPolyD;
    const T *K = k + bh * N * kPolyD;
    const T *V = v + bh * N * M;
    T *O = out + bh * N * M;
    __shared__ bf16 stage_mem[kPolyWaves][stage_elems<C::DT, 2>()];
    lds_bf16 *stage = (lds_bf16 *)stage_mem[wave];

    f32x4 X[C::NX][2][2];
    poly_load<M, C::NX>(X, ws + (bh * nseg + seg) * rec, m0);
    const Fr ones = frag_ones<Fr>();
    const bool diag = (c >> 2) == g;   // this lane holds token c's results
    const int e = c & 3;               // ... in element c % 4

    // No row masks: rows past t_end only reach outputs that are not stored
    // (the causal mask keeps them out of the others), and the state is not
    // used after the segment's last pair.  fp32 pairs are loaded where they
    // are used (a pair in flight would cost 64 more registers).
    constexpr int PF = poly_ahead<T, M>();
    constexpr bool kAhead = sizeof(T) == 2;
    PolyPair<T, M> buf[PF];
    if (kAhead) {
#pragma unroll
        for (int b = 0; b < PF; ++b) buf[b].load(Q, K, V, t_begin + 32 * b, t_end, m0, true);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += 32 * PF) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + 32 * b;   // may lie past t_end: nothing stored
        if (!kAhead) buf[b].load(Q, K, V, t0, t_end, m0, true);
        Fr Qn[2][C::DT], Kn[2][C::DT], KT[2][C::DT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ft = 0; ft < C::DT; ++ft) {
                Qn[h][ft] = IO<T>::to_frag(IO<T>::to_f32(buf[b].rq[h][ft]));
                Kn[h][ft] = IO<T>::to_frag(IO<T>::to_f32(buf[b].rk[h][ft]));
            }
        f32x4 wv[2][C::MW];
        buf[b].values(wv);
        if (kAhead) buf[b].load(Q, K, V, t0 + 32 * PF, t_end, m0, true);
        transpose_frags<C::DT, 2>(KT, Kn, stage);
        f32x4 KTf[2][C::DT];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int at = 0; at < C::DT; ++at) KTf[h][at] = IO<T>::to_f32(KT[h][at]);

        // P^T[j][i] = (q_i . k_j)^2 for key chunk hk, query chunk hq (masked to
        // j <= i on the diagonal blocks); as fragments they are P (rows i,
        // contraction j)
        Fr Pf[3];   // (keys 0, queries 0), (keys 0, queries 1), (keys 1, queries 1)
#pragma unroll
        for (int pi = 0; pi < 3; ++pi) {
            const int hk = pi == 2 ? 1 : 0, hq = pi == 0 ? 0 : 1;
            f32x4 pt = {0.f, 0.f, 0.f, 0.f};
            mma2(pt, Kn[hk][0], Kn[hk][1], Qn[hq][0], Qn[hq][1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) pt[r] = (hk != hq || 4 * g + r <= c) ? pt[r] * pt[r] : 0.f;
            Pf[pi] = IO<T>::to_frag(pt);
        }

        float res[2][C::NX];
#pragma unroll
        for (int x = 0; x < C::NX; ++x) {
            Fr Xf[2][2];
#pragma unroll
            for (int at = 0; at < 2; ++at)
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) Xf[at][bt] = IO<T>::to_frag(X[x][at][bt]);
            const Fr w0 = (x < C::NX - 1) ? IO<T>::to_frag(wv[0][x]) : ones;
            const Fr w1 = (x < C::NX - 1) ? IO<T>::to_frag(wv[1][x]) : ones;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // U^T tiles (rows b, cols tokens of chunk h) from X^T (the Acc tile is the operand)
                f32x4 u[2];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) {
                    u[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
                    mma2(u[bt], Xf[0][bt], Xf[1][bt], Qn[h][0], Qn[h][1]);
                }
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
                mma2(d, IO<T>::to_frag(u[0]), IO<T>::to_frag(u[1]), Qn[h][0], Qn[h][1]);
                if (h == 0)
                    mma1(d, Pf[0], w0);
                else
                    mma2(d, Pf[1], Pf[2], w0, w1);
                res[h][x] = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
            }
        }
        poly_update<T, C::NX>(X, KT, KTf, wv, C::NX);

#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float inv = __builtin_amdgcn_rcpf(res[h][C::NX - 1]);
            const int64_t t = t0 + 16 * h + c;
            if (diag && t < t_end)
                store4<T>(O + t * M + m0, IO<T>::from_f32(f32x4{res[h][0] * inv, res[h][1] * inv, res[h][2] * inv,
                                                                res[h][3] * inv}));
        }
    }
    }
}

// Segments of whole chunks: about kPolyTargetBlocks workgroups in all.
constexpr int64_t kPolyTargetBlocks = 512;

inline SegPlan make_poly_plan(int64_t BH, int64_t N, int64_t M) {
    SegPlan p;
    const int64_t nch = ceil_div(N, kChunk);
    int64_t nseg = std::max<int64_t>(1, std::min<int64_t>({ceil_div(kPolyTargetBlocks, BH), nch, kMaxSegPerHead}));
    p.seg_tokens = ceil_div(nch, nseg) * kChunk;
    p.nseg = ceil_div(N, p.seg_tokens);
    p.rec = (M + 1) * kPolyD * kPolyD;
    return p;
}

size_t poly_workspace_bytes(int64_t BH, int64_t N, int64_t M) {
    const SegPlan p = make_poly_plan(BH, N, M);
    return align256(size_t(BH * p.nseg * p.rec) * sizeof(float));
}

template <typename T, int M>
static hipError_t run_poly(const void *q, const void *k, const void *v, void *out, int64_t BH, int64_t N, float *ws,
                           hipStream_t s) {
    const SegPlan p = make_poly_plan(BH, N, M);
    const dim3 grid(unsigned(BH * p.nseg * (M / kPolyCols))), block(64 * kPolyWaves);
    hipLaunchKernelGGL((k_poly_segment_state<T, M>), grid, block, 0, s, (const T *)k, (const T *)v, ws, N, p.nseg,
                       p.seg_tokens, p.rec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_scan(ws, BH, p.nseg, p.rec, 0, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((k_poly_output<T, M>), grid, block, 0, s, (const T *)q, (const T *)k, (const T *)v, (T *)out,
                       (const float *)ws, N, p.nseg, p.seg_tokens, p.rec);
    return hipGetLastError();
}

hipError_t launch_poly_forward(int dt, const void *q, const void *k, const void *v, void *out, int64_t BH, int64_t N,
                               int64_t D, int64_t M, float *ws, hipStream_t s) {
    if (D != kPolyD) return hipErrorInvalidValue;
    if (dt == 0) {
        if (M == 32) return run_poly<float, 32>(q, k, v, out, BH, N, ws, s);
        if (M == 64) return run_poly<float, 64>(q, k, v, out, BH, N, ws, s);
    } else {
        if (M == 32) return run_poly<bf16, 32>(q, k, v, out, BH, N, ws, s);
        if (M == 64) return run_poly<bf16, 64>(q, k, v, out, BH, N, ws, s);
    }
    return hipErrorInvalidValue;
}

} // namespace la
