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

// The chunk's inputs as one wavefront needs them.  Rows at or beyond t_end
// read row t_end - 1; their K rows are zeroed, which removes them from every
// product (the rows of Q only reach outputs that are not stored).
template <typename T, int M> struct PolyChunk {
    typedef PolyCfg<T, M> C;
    typedef typename IO<T>::vec4 V4;
    V4 rq[1][C::DT], rk[1][C::DT];
    f32x4 wv[C::MW];   // wv[x][r] = v[t0 + 4g + r][m0 + x]

    __device__ __forceinline__ void load(const T *Q, const T *K, const T *V, int64_t t0, int64_t t_end, int m0,
                                         bool with_q) {
        if (with_q) load_chunk<T, kPolyD, 1>(rq, Q, t0, t_end);
        load_chunk<T, kPolyD, 1>(rk, K, t0, t_end);
        const int g = lane_id() >> 4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t t = min(t0 + 4 * g + r, t_end - 1);
#pragma unroll
            for (int x = 0; x < C::MW; x += 4) {
                const f32x4 v4 = IO<T>::to_f32(load4<T>(V + t * M + m0 + x));
#pragma unroll
                for (int e = 0; e < 4; ++e) wv[x + e][r] = v4[e];
            }
        }
    }
};

// X += (w o K)^T K for every matrix of the wavefront: KT are the chunk's
// token-contiguous K fragments (lane (c, g): k[4g + r][16 at + c]).
template <typename T, int M, int NX>
__device__ __forceinline__ void poly_update(f32x4 (&X)[NX][2][2], const typename IO<T>::frag (&KT)[1][kPolyD / 16],
                                            const f32x4 (&KTf)[kPolyD / 16], const f32x4 *wv, int nx) {
    typedef typename IO<T>::frag Fr;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
        if (x < nx) {
#pragma unroll
            for (int at = 0; at < 2; ++at) {
                const Fr a = (x < NX - 1) ? IO<T>::to_frag(KTf[at] * wv[x]) : KT[0][at];
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) mma1(X[x][at][bt], a, KT[0][bt]);
            }
        }
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
    __shared__ bf16 stage_mem[kPolyWaves][stage_elems<C::DT, 1>()];
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

    if (t_begin < t_end) {
        PolyChunk<T, M> cur, nxt;
        cur.load(nullptr, K, V, t_begin, t_end, m0, false);
        for (int64_t t0 = t_begin; t0 < t_end; t0 += 16) {
            if (t0 + 16 < t_end) nxt.load(nullptr, K, V, t0 + 16, t_end, m0, false);
            Fr Kn[1][C::DT], KT[1][C::DT];
            raw_frags<T, kPolyD, 1>(Kn, cur.rk, t0, t_end);
            transpose_frags<C::DT, 1>(KT, Kn, stage);
            f32x4 KTf[C::DT];
#pragma unroll
            for (int at = 0; at < C::DT; ++at) KTf[at] = IO<T>::to_f32(KT[0][at]);
            poly_update<T, M, C::NX>(X, KT, KTf, cur.wv, nx);
            cur = nxt;
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
    __shared__ bf16 stage_mem[kPolyWaves][stage_elems<C::DT, 1>()];
    lds_bf16 *stage = (lds_bf16 *)stage_mem[wave];

    f32x4 X[C::NX][2][2];
    poly_load<M, C::NX>(X, ws + (bh * nseg + seg) * rec, m0);
    const Fr ones = frag_ones<Fr>();
    const bool diag = (c >> 2) == g;   // this lane holds token c's results

    PolyChunk<T, M> cur, nxt;
    cur.load(Q, K, V, t_begin, t_end, m0, true);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += 16) {
        if (t0 + 16 < t_end) nxt.load(Q, K, V, t0 + 16, t_end, m0, true);
        Fr Qn[1][C::DT], Kn[1][C::DT], KT[1][C::DT];
        raw_frags<T, kPolyD, 1>(Qn, cur.rq, t0, t_end);
        raw_frags<T, kPolyD, 1>(Kn, cur.rk, t0, t_end);
        transpose_frags<C::DT, 1>(KT, Kn, stage);
        f32x4 KTf[C::DT];
#pragma unroll
        for (int at = 0; at < C::DT; ++at) KTf[at] = IO<T>::to_f32(KT[0][at]);

        // P^T[j][i] = (q_i . k_j)^2, j <= i; as a fragment it is P (rows i, contraction j)
        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
        mma2(pt, Kn[0][0], Kn[0][1], Qn[0][0], Qn[0][1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) pt[r] = (4 * g + r <= c) ? pt[r] * pt[r] : 0.f;
        const Fr Pf = IO<T>::to_frag(pt);

        float res[C::NX];
#pragma unroll
        for (int x = 0; x < C::NX; ++x) {
            // U^T tiles (rows b, cols tokens) from X^T (the Acc tile is the operand as it is)
            f32x4 u[2];
#pragma unroll
            for (int bt = 0; bt < 2; ++bt) {
                u[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
                mma2(u[bt], IO<T>::to_frag(X[x][0][bt]), IO<T>::to_frag(X[x][1][bt]), Qn[0][0], Qn[0][1]);
            }
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            mma2(d, IO<T>::to_frag(u[0]), IO<T>::to_frag(u[1]), Qn[0][0], Qn[0][1]);
            const Fr w = (x < C::NX - 1) ? IO<T>::to_frag(cur.wv[x]) : ones;
            mma1(d, Pf, w);
            // diagonal: token c sits in element c % 4 of lane (c, c / 4)
            const int e = c & 3;
            res[x] = e == 0 ? d[0] : e == 1 ? d[1] : e == 2 ? d[2] : d[3];
        }
        poly_update<T, M, C::NX>(X, KT, KTf, cur.wv, C::NX);

        const float inv = __builtin_amdgcn_rcpf(res[C::NX - 1]);
        const int64_t t = t0 + c;
        if (diag && t < t_end) {
#pragma unroll
            for (int x = 0; x < C::MW; x += 4)
                store4<T>(O + t * M + m0 + x,
                          IO<T>::from_f32(f32x4{res[x] * inv, res[x + 1] * inv, res[x + 2] * inv, res[x + 3] * inv}));
        }
        cur = nxt;
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
    if ((e = launch_scan(ws, BH, p.nseg, p.rec, 0, nullptr, nullptr, s)) != hipSuccess) return e;
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
