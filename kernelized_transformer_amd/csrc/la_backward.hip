// la_backward.hip -- causal backward through cumulative sums on gfx950.
//
// Method ([summary] = paperlayer.ai summary of "Transformers are RNNs",
// section 3.3.1 and appendix "A. Gradient Derivation"): the gradient is
// evaluated in linear time with running sums, never storing every S_i; the
// query gradient uses the forward-direction sum and the key/value gradients
// a sum of the same size running in the opposite direction.  The pages give
// the numerator part for feature-mapped inputs; the denominator and phi'
// terms are written out here.  With qh = phi(Q), kh = phi(K),
// a_ij = qh_i . kh_j (j <= i), d_i = sum_{j<=i} a_ij, out_i = num_i / d_i,
// and dout = G:
//   g_i = G_i / d_i,  h_i = -(G_i . out_i) / d_i,  gh_i = [g_i, h_i],
//   vh_j = [V_j, 1],  dA_ij = dL/da_ij = gh_i . vh_j,
//   dL/dqh_i = sum_{j<=i} dA_ij kh_j = S_aug_{i} gh_i          (forward sum)
//   dL/dkh_j = sum_{i>=j} dA_ij qh_i = R_aug_{j} vh_j          (reverse sum)
//   dV_j     = sum_{i>=j} a_ij g_i   = R_j^T kh_j
//   with S_aug = [S | Z] and R_aug = sum_{i>=j} qh_i gh_i^T = [R | u];
//   dQ = dL/dqh * phi'(Q), dK = dL/dkh * phi'(K).
// Chunked exactly like the forward (16-token chunks here, so that the three
// fp32 states of a wavefront fit in registers):
//   1. k_segment_state + scan  -> S_aug at the start of every segment;
//   2. k_bwd_dq    (forward direction, one wavefront per segment): recompute
//      out and d for the chunk, form gh, write dQ, store 1/d and h for pass 4
//      (8 bytes per token; pass 4 forms g = dout / d again from dout, with the
//      same fp32 product and rounding), and accumulate the segment's
//      sum_i qh_i gh_i^T;
//   3. reverse scan            -> R_aug after the end of every segment;
//   4. k_bwd_dkdv  (reverse direction): walk the chunks backwards carrying
//      R_aug, write dK and dV.
// The non-causal backward is the same with every sum taken over the whole
// sequence (a_ij for all i, j): 1. gives the full S_aug, 2. reads only Q and
// dout against it, 3. totals R_aug, 4. reads only K and V against it.
#include "la_chunk.h"
#include "la_internal.h"
#include "la_split.h"

namespace la {

constexpr int BTT = 1;  // token tiles per chunk in the backward kernels
constexpr int BCH = 16 * BTT;
// Operand fragments of the one-wavefront kernels: fp32 data runs on the bf16
// matrix instruction split into hi + lo parts (split4, as in the fp32
// forward), bf16 as is.
template <typename T> using BwdFrag = typename std::conditional<sizeof(T) == 4, split4, typename IO<T>::frag>::type;
// LDS per wavefront: the chunk transposes, or the state's (M + 16) x D
// transpose (split operands: two areas each)
template <typename T, int D, int M>
constexpr int kBwdStage =
    (transpose_stage_elems<BwdFrag<T>, D / 16, BTT>() + transpose_stage_elems<BwdFrag<T>, M / 16 + 1, BTT>() >
     transpose_stage_elems<BwdFrag<T>, D / 16, M / 16 + 1>())
        ? transpose_stage_elems<BwdFrag<T>, D / 16, BTT>() + transpose_stage_elems<BwdFrag<T>, M / 16 + 1, BTT>()
        : transpose_stage_elems<BwdFrag<T>, D / 16, M / 16 + 1>();
template <int D, int M>
constexpr int kBwdTile = 16 * ((D > M ? D : M) + kStagePad);

// ---- pass 2: forward direction --------------------------------------------
// Non-causal (CAUSAL = false): every query sees the full sums S_aug (record 0
// of the head), so K, V are not read, there is no intra-chunk term and no
// state to carry, and 1/d, h are not stored (ibuf, hbuf unused).
template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__(64) void k_bwd_dq(const T *__restrict__ q, const T *__restrict__ k,
                                               const T *__restrict__ v, const T *__restrict__ dout,
                                               T *__restrict__ dq, const float *__restrict__ wsS,
                                               float *__restrict__ wsR, float *__restrict__ ibuf,
                                               float *__restrict__ hbuf, int64_t N, int64_t nseg,
                                               int64_t seg_tokens, int64_t rec) {
    typedef BwdFrag<T> Fr;
    typedef typename IO<T>::vec4 V4;
    constexpr int DT = D / 16, MT = M / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    const T *G = dout + bh * N * M;
    T *DQ = dq + bh * N * D;
    float *IB = ibuf + bh * N;
    float *HB = hbuf + bh * N;

    const float *srec = wsS + (bh * nseg + (CAUSAL ? seg : 0)) * rec;
    f32x4 St[DT][MT + 1];      // S_aug, rows d
    f32x4 Ra[DT][MT + 1];      // this segment's sum_i qh_i gh_i^T, rows d
    state_load<D, M>(St, srec);
    state_zero<D, M>(Ra);

    const Fr ones = frag_row0_ones<Fr>();
    const Fr k0ones = frag_k0_ones<Fr>();
    __shared__ bf16 stage_mem[kBwdStage<T, D, M> + kBwdTile<D, M>];
    lds_bf16 *stage = (lds_bf16 *)(stage_mem);
    lds_bf16 *otile = stage + kBwdStage<T, D, M>;   // one 16-token output tile (bf16)

    V4 rq[BTT][DT], rk[BTT][DT], rv[BTT][MT], rg[BTT][MT];
    load_chunk<T, D, BTT>(rq, Q, t_begin, t_end);
    if (CAUSAL) {
        load_chunk<T, D, BTT>(rk, K, t_begin, t_end);
        load_chunk<T, M, BTT>(rv, V, t_begin, t_end);
    }
    load_chunk<T, M, BTT>(rg, G, t_begin, t_end);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += BCH) {
        Fr Qn[BTT][DT], Kn[BTT][DT], Vn[BTT][MT];
        phi_frags<T, D, BTT>(Qn, rq, t0, t_end);
        if (CAUSAL) {
            phi_frags<T, D, BTT>(Kn, rk, t0, t_end);
            raw_frags<T, M, BTT>(Vn, rv, t0, t_end);
        }
        f32x4 qraw[DT], graw[MT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) qraw[dt] = IO<T>::to_f32(rq[0][dt]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) graw[mt] = IO<T>::to_f32(rg[0][mt]);
        load_chunk<T, D, BTT>(rq, Q, t0 + BCH, t_end);
        if (CAUSAL) {
            load_chunk<T, D, BTT>(rk, K, t0 + BCH, t_end);
            load_chunk<T, M, BTT>(rv, V, t0 + BCH, t_end);
        }
        load_chunk<T, M, BTT>(rg, G, t0 + BCH, t_end);
        const int64_t t = t0 + c;   // this lane's query token
        const bool valid = t < t_end;

        // S_aug as operand tiles in both orientations: SF[mt][dt] (rows m',
        // contraction d) is the accumulator tile itself, SFT[mt][dt] (rows d,
        // contraction m') its transpose through LDS
        Fr SF[MT + 1][DT], SFT[MT + 1][DT];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) SF[mt][dt] = frag_from<Fr>(St[dt][mt]);
        transpose_frags<DT, MT + 1>(SFT, SF, stage);

        Fr KT[BTT][DT], VT[BTT][MT];
        if (CAUSAL) {
            transpose_frags<DT, BTT>(KT, Kn, stage);
            transpose_frags<MT, BTT>(VT, Vn, stage + transpose_stage_elems<Fr, DT, BTT>());
        }

        // recompute out^T (and den in the normalizer block) as the forward does
        f32x4 Ot[MT + 1];
        Fr PT = frag_zero<Fr>();
        if (CAUSAL) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DT; dt += 2) mma2(p, Kn[0][dt], Kn[0][dt + 1], Qn[0][dt], Qn[0][dt + 1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
            PT = frag_from<Fr>(p);
        }
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) {
            Ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DT; dt += 2) mma2(Ot[mt], SF[mt][dt], SF[mt][dt + 1], Qn[0][dt], Qn[0][dt + 1]);
            if (CAUSAL) mma1(Ot[mt], mt < MT ? VT[0][mt] : ones, PT);
        }
        const float den = __shfl(Ot[MT][0], c);
        const float inv = valid ? __builtin_amdgcn_rcpf(den) : 0.f;

        // gh = [G / d, -(G . out) / d]; lane (c, g) holds m = 16 mt + 4g + r of token c
        float go = 0.f;
        f32x4 gv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 o = Ot[mt];   // out times d: the 1/d factors are applied to the sum
            go += graw[mt][0] * o[0] + graw[mt][1] * o[1] + graw[mt][2] * o[2] + graw[mt][3] * o[3];
            gv[mt] = graw[mt] * inv;
        }
        go += __shfl_xor(go, 16);
        go += __shfl_xor(go, 32);
        const float h = -(go * inv) * inv;   // -(dout . out) / d with out = Ot / d
        Fr Gn[BTT][MT + 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) Gn[0][mt] = frag_from<Fr>(gv[mt]);
        Gn[0][MT] = frag_from<Fr>(f32x4{g == 0 ? h : 0.f, 0.f, 0.f, 0.f});
        if (CAUSAL && valid && g == 0) {
            IB[t] = inv;
            HB[t] = h;
        }

        // dA^T[j][i] = vh_j . gh_i, masked to j <= i
        Fr dAT = frag_zero<Fr>();
        if (CAUSAL) {
            f32x4 da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) {
                const Fr a1 = (mt + 1 < MT) ? Vn[0][mt + 1] : k0ones;
                mma2(da, Vn[0][mt], a1, Gn[0][mt], Gn[0][mt + 1]);
            }
            if ((MT & 1) == 0) mma1(da, k0ones, Gn[0][MT]);
#pragma unroll
            for (int r = 0; r < 4; ++r) da[r] = (4 * g + r <= c) ? da[r] : 0.f;
            dAT = frag_from<Fr>(da);
        }

        // dL/dqh^T[d][i] = sum_j kh[j][d] dA^T[j][i] + sum_m' S_aug[d][m'] gh[i][m']
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (CAUSAL) mma1(acc, KT[0][dt], dAT);
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, SFT[mt][dt], SFT[mt + 1][dt], Gn[0][mt], Gn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(acc, SFT[MT][dt], Gn[0][MT]);
            const f32x4 dqv = acc * dphi4(qraw[dt]);
            if constexpr (sizeof(T) == 2)
                tile_put_bf16<D>(otile, dt, IO<bf16>::from_f32(dqv));
            else if (valid)
                store4<T>(DQ + t * D + 16 * dt + 4 * g, IO<T>::from_f32(dqv));
        }
        if constexpr (sizeof(T) == 2) tile_flush_bf16<D>((bf16 *)DQ, t0, t_end, otile);

        // this segment's reverse-sum contribution: Ra += sum_i qh_i gh_i^T
        Fr QT[BTT][DT], GT[BTT][MT + 1];
        transpose_frags<DT, BTT>(QT, Qn, stage);
        transpose_frags<MT + 1, BTT>(GT, Gn, stage + transpose_stage_elems<Fr, DT, BTT>());
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt) mma1(Ra[dt][mt], QT[0][dt], GT[0][mt]);

        // carry S_aug past this chunk
        if (CAUSAL) state_accumulate<Fr, D, M, BTT>(St, KT, VT);
    }
    state_store<D, M>(wsR + (bh * nseg + seg) * rec, Ra);
}

// ---- pass 4: reverse direction --------------------------------------------
// Non-causal (CAUSAL = false): every key sees the full sums R_aug (record 0 of
// the head), so Q, g, h are not read, there is no intra-chunk term and no
// sum to carry.
template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__(64) void k_bwd_dkdv(const T *__restrict__ q, const T *__restrict__ k,
                                                 const T *__restrict__ v, const T *__restrict__ dout,
                                                 const float *__restrict__ ibuf, const float *__restrict__ hbuf,
                                                 T *__restrict__ dk,
                                                 T *__restrict__ dv, const float *__restrict__ wsR, int64_t N,
                                                 int64_t nseg, int64_t seg_tokens, int64_t rec) {
    typedef BwdFrag<T> Fr;
    typedef typename IO<T>::vec4 V4;
    constexpr int DT = D / 16, MT = M / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    const T *G = dout + bh * N * M;
    const float *IB = ibuf + bh * N;
    const float *HB = hbuf + bh * N;
    T *DK = dk + bh * N * D;
    T *DV = dv + bh * N * M;

    const float *rrec = wsR + (bh * nseg + (CAUSAL ? seg : 0)) * rec;
    f32x4 Rr[DT][MT + 1];      // R_aug = [R | u], rows d
    state_load<D, M>(Rr, rrec);

    const Fr k0ones = frag_k0_ones<Fr>();
    __shared__ bf16 stage_mem[kBwdStage<T, D, M> + kBwdTile<D, M>];
    lds_bf16 *stage = (lds_bf16 *)(stage_mem);
    lds_bf16 *otile = stage + kBwdStage<T, D, M>;   // one 16-token output tile (bf16)

    const int64_t nch = (t_end - t_begin + BCH - 1) / BCH;
    V4 rq[BTT][DT], rk[BTT][DT], rv[BTT][MT], rg[BTT][MT];
    float rh, ri;
    auto load_all = [&](int64_t t0) {
        if (CAUSAL) load_chunk<T, D, BTT>(rq, Q, t0, t_end);
        load_chunk<T, D, BTT>(rk, K, t0, t_end);
        load_chunk<T, M, BTT>(rv, V, t0, t_end);
        if (CAUSAL) {
            load_chunk<T, M, BTT>(rg, G, t0, t_end);
            rh = (t0 + c < t_end) ? HB[t0 + c] : 0.f;
            ri = (t0 + c < t_end) ? IB[t0 + c] : 0.f;
        }
    };
    load_all(t_begin + (nch - 1) * BCH);
    for (int64_t ci = nch - 1; ci >= 0; --ci) {
        const int64_t t0 = t_begin + ci * BCH;
        Fr Qn[BTT][DT], Kn[BTT][DT], Vn[BTT][MT + 1], Gn[BTT][MT + 1];
        if (CAUSAL) phi_frags<T, D, BTT>(Qn, rq, t0, t_end);
        phi_frags<T, D, BTT>(Kn, rk, t0, t_end);
        {
            Fr tmp[BTT][MT];
            raw_frags<T, M, BTT>(tmp, rv, t0, t_end);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) Vn[0][mt] = tmp[0][mt];
            Vn[0][MT] = k0ones;
            if (CAUSAL) {   // g = dout / d, formed as in the forward-direction pass; rows past t_end are 0
                const bool ok = t0 + c < t_end;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const f32x4 gv = IO<T>::to_f32(rg[0][mt]) * ri;
                    Gn[0][mt] = frag_from<Fr>(ok ? gv : f32x4{0.f, 0.f, 0.f, 0.f});
                }
                Gn[0][MT] = frag_from<Fr>(f32x4{g == 0 ? rh : 0.f, 0.f, 0.f, 0.f});
            }
        }
        f32x4 kraw[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) kraw[dt] = IO<T>::to_f32(rk[0][dt]);
        if (ci > 0) load_all(t0 - BCH);

        const int64_t t = t0 + c;   // this lane's key token
        const bool valid = t < t_end;

        // R_aug as operand tiles in both orientations (see the forward-direction pass)
        Fr RF[MT + 1][DT], RFT[MT + 1][DT];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) RF[mt][dt] = frag_from<Fr>(Rr[dt][mt]);
        transpose_frags<DT, MT + 1>(RFT, RF, stage);

        Fr QT[BTT][DT], GT[BTT][MT + 1];
        Fr Pf = frag_zero<Fr>(), dAf = frag_zero<Fr>();
        if (CAUSAL) {
            transpose_frags<DT, BTT>(QT, Qn, stage);
            transpose_frags<MT + 1, BTT>(GT, Gn, stage + transpose_stage_elems<Fr, DT, BTT>());

            // P[i][j] = qh_i . kh_j and dA[i][j] = gh_i . vh_j, masked to i >= j
            f32x4 p = {0.f, 0.f, 0.f, 0.f}, da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DT; dt += 2) mma2(p, Qn[0][dt], Qn[0][dt + 1], Kn[0][dt], Kn[0][dt + 1]);
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(da, Gn[0][mt], Gn[0][mt + 1], Vn[0][mt], Vn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(da, Gn[0][MT], Vn[0][MT]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = 4 * g + r >= c;
                p[r] = keep ? p[r] : 0.f;
                da[r] = keep ? da[r] : 0.f;
            }
            Pf = frag_from<Fr>(p);
            dAf = frag_from<Fr>(da);
        }

        // dL/dkh^T[d][j] = sum_i qh[i][d] dA[i][j] + sum_m' R_aug[d][m'] vh[j][m']
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (CAUSAL) mma1(acc, QT[0][dt], dAf);
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, RFT[mt][dt], RFT[mt + 1][dt], Vn[0][mt], Vn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(acc, RFT[MT][dt], Vn[0][MT]);
            const f32x4 dkv = acc * dphi4(kraw[dt]);
            if constexpr (sizeof(T) == 2)
                tile_put_bf16<D>(otile, dt, IO<bf16>::from_f32(dkv));
            else if (valid)
                store4<T>(DK + t * D + 16 * dt + 4 * g, IO<T>::from_f32(dkv));
        }
        if constexpr (sizeof(T) == 2) tile_flush_bf16<D>((bf16 *)DK, t0, t_end, otile);
        // dV^T[m][j] = sum_i g[i][m] P[i][j] + sum_d R[d][m] kh[j][d]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (CAUSAL) mma1(acc, GT[0][mt], Pf);
#pragma unroll
            for (int dt = 0; dt < DT; dt += 2) mma2(acc, RF[mt][dt], RF[mt][dt + 1], Kn[0][dt], Kn[0][dt + 1]);
            if constexpr (sizeof(T) == 2)
                tile_put_bf16<M>(otile, mt, IO<bf16>::from_f32(acc));
            else if (valid)
                store4<T>(DV + t * M + 16 * mt + 4 * g, IO<T>::from_f32(acc));
        }
        if constexpr (sizeof(T) == 2) tile_flush_bf16<M>((bf16 *)DV, t0, t_end, otile);

        // carry R_aug past this chunk, towards earlier tokens
        if (CAUSAL) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int mt = 0; mt <= MT; ++mt) mma1(Rr[dt][mt], QT[0][dt], GT[0][mt]);
        }
    }
}

// ---- bf16, D = 64: two wavefronts per segment ------------------------------
// The kernels above carry D x (M + 16) fp32 states in one wavefront (the
// forward-direction pass two of them) and run one wavefront per SIMD.  Here
// a segment is walked by a workgroup of two wavefronts; wavefront w owns the
// state rows d in [32 w, 32 w + 32) (S_aug and this segment's sum of
// phi(Q) gh^T in the forward direction, R_aug in the reverse one), so each
// carries half the registers and two workgroups share a SIMD pair.  Every
// product that contracts over d (the recomputed out and den, the dV readout)
// is formed as two partial sums, one per wavefront, exchanged once per chunk
// through LDS; the rest is local to a wavefront's rows or (the small [g, h]
// and dA products) computed by both.  Rows move through LDS staging as
// 16-byte loads (a wavefront loads its own 32 columns of Q and K and all of
// V and dout), and phi'(x) = min(phi(x), 1) is read off the staged
// phi(x) (phi(x) <= 1 exactly when x <= 0, where phi' = phi = exp(x)).
template <int M> struct W2Stage {   // one wavefront's private LDS, in elements
    static constexpr int SQ = 16 * (kW2Half + kStagePad);   // phi(Q) or phi(K) columns of the wavefront
    static constexpr int SV = 16 * (M + kStagePad);         // V, dout or g rows
    static constexpr int ROWS = 2 * SQ + 2 * SV;
    static constexpr int ST = stage_elems<kW2Half / 16, M / 16 + 1>();   // a state transpose
    static constexpr int N = ROWS > ST ? ROWS : ST;
    static constexpr int NQ = ROWS > SV + ST ? ROWS : SV + ST;   // the forward-direction layout
};

// Forward direction (see k_bwd_dq): recompute out and den, write dQ, g, h,
// and this segment's sum of phi(Q) gh^T.
template <int D, int M>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq_w2(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, bf16 *__restrict__ dq, const float *__restrict__ wsS, float *__restrict__ wsR,
    float *__restrict__ ibuf, float *__restrict__ hbuf, int64_t N, int64_t nseg, int64_t seg_tokens, int64_t rec) {
    static_assert(D == 2 * kW2Half, "two wavefronts of 32 feature rows");
    typedef bf16x4 Fr;
    constexpr int DTH = kW2Half / 16, MT = M / 16, PF = 1;
    constexpr int NV = Lines<M, 1>::n;
    typedef W2Stage<M> SL;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const bf16 *Qw = q + bh * N * D + w * kW2Half;
    const bf16 *Kw = k + bh * N * D + w * kW2Half;
    const bf16 *V = v + bh * N * M;
    const bf16 *G = dout + bh * N * M;
    bf16 *DQw = dq + bh * N * D + w * kW2Half;
    float *IB = ibuf + bh * N;
    float *HB = hbuf + bh * N;

    // per wavefront: dout rows first, then phi(Q), phi(K), V; the state's
    // transpose goes right after the dout rows, which are read last
    __shared__ __align__(16) bf16 priv_mem[2][SL::NQ];
    __shared__ __align__(16) f32x4 xbuf[2][2][MT + 1][64];   // [chunk parity][wavefront][tile][lane]
    lds_bf16 *sg = (lds_bf16 *)priv_mem[w];
    lds_bf16 *sq = sg + SL::SV;
    lds_bf16 *sk = sq + SL::SQ;
    lds_bf16 *sv = sk + SL::SQ;
    lds_bf16 *sst = sq;   // S_aug^T, over the phi(Q), phi(K), V rows once they are read

    f32x4 St[DTH][MT + 1];   // S_aug rows of this wavefront, normalizer tile replicated
    f32x4 Ra[DTH][MT + 1];   // this segment's sum_i qh_i gh_i^T, same rows
    rows_load<D, M, DTH, true>(St, wsS + (bh * nseg + seg) * rec, w * kW2Half);
#pragma unroll
    for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) Ra[dt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const Fr ones = frag_ones<Fr>();
    const Fr k0ones = frag_k0_ones<Fr>();

    dwordx4 lq[PF], lk[PF], lv[PF][NV], lg[PF][NV];
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t_begin + b * BCH;
        lq[b] = load_cols32<D>(Qw, t0, t_end);
        lk[b] = load_cols32<D>(Kw, t0, t_end);
        load_rows32<M>(lv[b], V, t0, t_end);
        load_rows32<M>(lg[b], G, t0, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * BCH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + b * BCH;
        if (t0 >= t_end) break;   // uniform over the workgroup
        // no row masks: rows past t_end copy row t_end - 1; their g, h are zero
        // (inv = 0 below), the causal mask keeps their keys out of every valid
        // query, and the state is not used after the segment
        stage_cols32_phi(sq, lq[b]);
        stage_cols32_phi(sk, lk[b]);
        stage_lines<M, 1, false, false>(sv, lv[b], t0, t_end);
        stage_lines<M, 1, false, false>(sg, lg[b], t0, t_end);
        {
            const int64_t tn = t0 + PF * BCH;
            lq[b] = load_cols32<D>(Qw, tn, t_end);
            lk[b] = load_cols32<D>(Kw, tn, t_end);
            load_rows32<M>(lv[b], V, tn, t_end);
            load_rows32<M>(lg[b], G, tn, t_end);
        }
        __builtin_amdgcn_sched_barrier(0);
        const int64_t t = t0 + c;   // this lane's query token
        const bool valid = t < t_end;

        Fr Qn[1][DTH], QT[1][DTH], Kn[1][DTH], KT[1][DTH], VT[1][MT], Vn[1][MT];
        natural_frags_lds<kW2Half, 1>(Qn, sq);
        transposed_frags_lds<kW2Half, 1>(QT, sq);
        natural_frags_lds<kW2Half, 1>(Kn, sk);
        transposed_frags_lds<kW2Half, 1>(KT, sk);
        natural_frags_lds<M, 1>(Vn, sv);
        transposed_frags_lds<M, 1>(VT, sv);

        // S_aug as operand tiles: SF[mt][dt] (rows m', contraction d) is the
        // accumulator itself; its transpose (rows d, contraction m') is
        // written to LDS now and read back for dQ
        Fr SF[MT + 1][DTH];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt) SF[mt][dt] = IO<bf16>::to_frag(St[dt][mt]);
        put_frags_lds<DTH, MT + 1>(sst, SF);

        // this wavefront's share (its 32 rows d) of out^T and den
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DTH; dt += 2) mma2(p, Kn[0][dt], Kn[0][dt + 1], Qn[0][dt], Qn[0][dt + 1]);
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
        const Fr PT = IO<bf16>::to_frag(p);
        f32x4 Ot[MT + 1];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) {
            Ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DTH; dt += 2) mma2(Ot[mt], SF[mt][dt], SF[mt][dt + 1], Qn[0][dt], Qn[0][dt + 1]);
            mma1(Ot[mt], mt < MT ? VT[0][mt] : ones, PT);
        }
        // exchange the shares: both wavefronts then hold the same full sums
        const int par = int((t0 - t_begin) / BCH) & 1;
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) xbuf[par][w][mt][lane] = Ot[mt];
        // carry S_aug past this chunk (its operand copies are taken): work
        // that does not need the other wavefront's share, before waiting for it
        state_accumulate<Fr, kW2Half, M, 1, true>(St, KT, VT);
        lds_barrier();
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) Ot[mt] += xbuf[par][1 - w][mt][lane];

        // gh = [G / d, -(G . out) / d]; lane (c, g) holds m = 16 mt + 4g + r of token c
        const float inv = valid ? __builtin_amdgcn_rcpf(Ot[MT][0]) : 0.f;
        Fr Gr[1][MT];
        natural_frags_lds<M, 1>(Gr, sg);
        float go = 0.f;
        f32x4 gv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 graw = IO<bf16>::to_f32(Gr[0][mt]);
            const f32x4 o = Ot[mt];   // out times d: the 1/d factors are applied to the sum
            go += graw[0] * o[0] + graw[1] * o[1] + graw[2] * o[2] + graw[3] * o[3];
            gv[mt] = graw * inv;
        }
        go += __shfl_xor(go, 16);
        go += __shfl_xor(go, 32);
        const float h = -(go * inv) * inv;   // -(dout . out) / d with out = Ot / d
        Fr Gn[1][MT + 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) Gn[0][mt] = IO<bf16>::to_frag(gv[mt]);
        Gn[0][MT] = IO<bf16>::to_frag(f32x4{g == 0 ? h : 0.f, 0.f, 0.f, 0.f});

        // 1/d and h leave from here (wavefront 1); the reverse pass forms g itself
        if (w == 1 && valid && g == 0) {
            IB[uint32_t(t)] = inv;
            HB[uint32_t(t)] = h;
        }

        // dA^T[j][i] = vh_j . gh_i, masked to j <= i (both wavefronts)
        f32x4 da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int mt = 0; mt + 1 <= MT; mt += 2) {
            const Fr a1 = (mt + 1 < MT) ? Vn[0][mt + 1] : k0ones;
            mma2(da, Vn[0][mt], a1, Gn[0][mt], Gn[0][mt + 1]);
        }
        if ((MT & 1) == 0) mma1(da, k0ones, Gn[0][MT]);
#pragma unroll
        for (int r = 0; r < 4; ++r) da[r] = (4 * g + r <= c) ? da[r] : 0.f;
        const Fr dAT = IO<bf16>::to_frag(da);

        // dL/dqh^T for this wavefront's rows d, times phi'(q) = min(phi(q), 1)
        Fr SFT[MT + 1][DTH];
        transposed_frags_lds<16 * DTH, MT + 1>(SFT, sst);
        lds_bf16 *dtile = sg;   // the dout rows are read
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma1(acc, KT[0][dt], dAT);
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, SFT[mt][dt], SFT[mt + 1][dt], Gn[0][mt], Gn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(acc, SFT[MT][dt], Gn[0][MT]);
            const f32x4 qh = IO<bf16>::to_f32(Qn[0][dt]);
            const f32x4 dp = {__builtin_fminf(qh[0], 1.f), __builtin_fminf(qh[1], 1.f), __builtin_fminf(qh[2], 1.f),
                              __builtin_fminf(qh[3], 1.f)};
            tile_put_bf16<kW2Half>(dtile, dt, IO<bf16>::from_f32(acc * dp));
        }
        flush_rows<kW2Half, D, 16>(DQw, t0, t_end, dtile, 0);

        // this segment's reverse-sum contribution (rows d of this wavefront)
        Fr GT[1][MT + 1];
        static_assert(stage_elems<MT + 1, 1>() <= SL::NQ, "transpose of gh fits");
        transpose_frags<MT + 1, 1>(GT, Gn, sg);   // the dQ tile is flushed
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt) mma1(Ra[dt][mt], QT[0][dt], GT[0][mt]);
    }
    }
    rows_store<D, M, DTH>(wsR + (bh * nseg + seg) * rec, Ra, w * kW2Half);
}

// Reverse direction (see k_bwd_dkdv): walk the chunks last to first carrying
// R_aug, write dK and dV.
template <int D, int M>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dkdv_w2(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ dout, const float *__restrict__ ibuf, const float *__restrict__ hbuf,
    bf16 *__restrict__ dk, bf16 *__restrict__ dv, const float *__restrict__ wsR, int64_t N, int64_t nseg,
    int64_t seg_tokens, int64_t rec) {
    static_assert(D == 2 * kW2Half, "two wavefronts of 32 feature rows");
    typedef bf16x4 Fr;
    constexpr int DTH = kW2Half / 16, MT = M / 16, MH = MT / 2, PF = 2;
    constexpr int NV = Lines<M, 1>::n;
    typedef W2Stage<M> SL;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const bf16 *Qw = q + bh * N * D + w * kW2Half;
    const bf16 *Kw = k + bh * N * D + w * kW2Half;
    const bf16 *V = v + bh * N * M;
    const bf16 *G = dout + bh * N * M;
    const float *IB = ibuf + bh * N;
    const float *HB = hbuf + bh * N;
    bf16 *DKw = dk + bh * N * D + w * kW2Half;
    bf16 *DVw = dv + bh * N * M + w * (M / 2);

    __shared__ __align__(16) bf16 priv_mem[2][SL::N];
    __shared__ __align__(16) f32x4 xbuf[2][2][MH][64];   // [chunk parity][wavefront][tile][lane]
    lds_bf16 *sq = (lds_bf16 *)priv_mem[w];
    lds_bf16 *sk = sq + SL::SQ;
    lds_bf16 *sv = sk + SL::SQ;
    lds_bf16 *sg = sv + SL::SV;

    f32x4 Rr[DTH][MT + 1];   // R_aug = [R | u], this wavefront's rows d
    rows_load<D, M, DTH, false>(Rr, wsR + (bh * nseg + seg) * rec, w * kW2Half);
    const Fr k0ones = frag_k0_ones<Fr>();

    const int64_t nch = (t_end - t_begin + BCH - 1) / BCH;
    auto chunk = [&](int64_t step) { return t_begin + imax64(nch - 1 - step, 0) * BCH; };
    dwordx4 lq[PF], lk[PF], lv[PF][NV], lg[PF][NV];
    float lh[PF], li[PF];
    auto load_all = [&](int b, int64_t t0) {
        lq[b] = load_cols32<D>(Qw, t0, t_end);
        lk[b] = load_cols32<D>(Kw, t0, t_end);
        load_rows32<M>(lv[b], V, t0, t_end);
        load_rows32<M>(lg[b], G, t0, t_end);
        const uint32_t tc = min(uint32_t(t0) + uint32_t(c), uint32_t(t_end - 1));
        lh[b] = HB[tc];
        li[b] = IB[tc];
    };
#pragma unroll
    for (int b = 0; b < PF; ++b) load_all(b, chunk(b));
    for (int64_t s0 = 0; s0 < nch; s0 += PF) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t step = s0 + b;
        if (step >= nch) break;   // uniform over the workgroup
        const int64_t t0 = chunk(step);
        // rows past t_end belong to the next segment: their g and h must not
        // enter (zeroed); Q, K, V there only meet those zeros or unstored outputs
        stage_cols32_phi(sq, lq[b]);
        stage_cols32_phi(sk, lk[b]);
        stage_lines<M, 1, false, false>(sv, lv[b], t0, t_end);
        stage_rows_scaled<M>(sg, lg[b], li[b], t0, t_end);   // g = dout / d, as the forward-direction pass forms it
        const float hc = (t0 + c < t_end) ? lh[b] : 0.f;
        load_all(b, chunk(step + PF));
        __builtin_amdgcn_sched_barrier(0);

        Fr Qn[1][DTH], QT[1][DTH], Kn[1][DTH], Vn[1][MT + 1], Gn[1][MT + 1], GT[1][MT + 1];
        natural_frags_lds<kW2Half, 1>(Qn, sq);
        transposed_frags_lds<kW2Half, 1>(QT, sq);
        natural_frags_lds<kW2Half, 1>(Kn, sk);
        {
            Fr tv[1][MT], tg[1][MT], tgt[1][MT];
            natural_frags_lds<M, 1>(tv, sv);
            natural_frags_lds<M, 1>(tg, sg);
            transposed_frags_lds<M, 1>(tgt, sg);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                Vn[0][mt] = tv[0][mt];
                Gn[0][mt] = tg[0][mt];
                GT[0][mt] = tgt[0][mt];
            }
        }
        Vn[0][MT] = k0ones;
        Gn[0][MT] = IO<bf16>::to_frag(f32x4{g == 0 ? hc : 0.f, 0.f, 0.f, 0.f});
        {   // GT[MT]: row 0 holds h of tokens 4g + r (lanes c = 0)
            f32x4 h4;
#pragma unroll
            for (int r = 0; r < 4; ++r) h4[r] = __shfl(hc, 4 * g + r);
            GT[0][MT] = IO<bf16>::to_frag(c == 0 ? h4 : f32x4{0.f, 0.f, 0.f, 0.f});
        }

        // R_aug as operand tiles in both orientations
        Fr RF[MT + 1][DTH], RFT[MT + 1][DTH];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt) RF[mt][dt] = IO<bf16>::to_frag(Rr[dt][mt]);
        transpose_frags<DTH, MT + 1>(RFT, RF, sq);

        // P (this wavefront's share over its rows d) and dA (both), masked to i >= j
        f32x4 p = {0.f, 0.f, 0.f, 0.f}, da = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DTH; dt += 2) mma2(p, Qn[0][dt], Qn[0][dt + 1], Kn[0][dt], Kn[0][dt + 1]);
#pragma unroll
        for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(da, Gn[0][mt], Gn[0][mt + 1], Vn[0][mt], Vn[0][mt + 1]);
        if ((MT & 1) == 0) mma1(da, Gn[0][MT], Vn[0][MT]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const bool keep = 4 * g + r >= c;
            p[r] = keep ? p[r] : 0.f;
            da[r] = keep ? da[r] : 0.f;
        }
        const Fr Pf = IO<bf16>::to_frag(p), dAf = IO<bf16>::to_frag(da);

        // dV^T[m][j] shares: sum_i g[i][m] P[i][j] + sum_d R[d][m] kh[j][d];
        // wavefront w finishes the tiles mt in [w MH, w MH + MH)
        f32x4 dvs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            dvs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma1(dvs[mt], GT[0][mt], Pf);
#pragma unroll
            for (int dt = 0; dt < DTH; dt += 2) mma2(dvs[mt], RF[mt][dt], RF[mt][dt + 1], Kn[0][dt], Kn[0][dt + 1]);
        }
        // (explicit selects: an index computed from w would make the compiler
        // index the register file at run time)
        const int par = int(step & 1);
#pragma unroll
        for (int i = 0; i < MH; ++i) xbuf[par][w][i][lane] = w ? dvs[i] : dvs[MH + i];

        // dL/dkh^T for this wavefront's rows d, times phi'(k) = min(phi(k), 1)
        lds_bf16 *dtile = sv;   // the staged rows are all in registers by now
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            mma1(acc, QT[0][dt], dAf);
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, RFT[mt][dt], RFT[mt + 1][dt], Vn[0][mt], Vn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(acc, RFT[MT][dt], Vn[0][MT]);
            const f32x4 kh = IO<bf16>::to_f32(Kn[0][dt]);
            const f32x4 dp = {__builtin_fminf(kh[0], 1.f), __builtin_fminf(kh[1], 1.f), __builtin_fminf(kh[2], 1.f),
                              __builtin_fminf(kh[3], 1.f)};
            tile_put_bf16<kW2Half>(dtile, dt, IO<bf16>::from_f32(acc * dp));
        }
        flush_rows<kW2Half, D, 16>(DKw, t0, t_end, dtile, 0);

        // carry R_aug past this chunk, towards earlier tokens
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt) mma1(Rr[dt][mt], QT[0][dt], GT[0][mt]);

        lds_barrier();
        lds_bf16 *vtile = dtile;
#pragma unroll
        for (int i = 0; i < MH; ++i)
            tile_put_bf16<M / 2>(vtile, i, IO<bf16>::from_f32((w ? dvs[MH + i] : dvs[i]) + xbuf[par][1 - w][i][lane]));
        flush_rows<M / 2, M, 16>(DVw, t0, t_end, vtile, 0);
    }
    }
}

// Non-causal, two wavefronts per segment: every query sees the full S_aug
// and every key the full R_aug (record 0 of the head), so each wavefront
// converts its rows of the sums to operand tiles, in both orientations, once
// before its chunk loop.  dQ pass: Q (its 32 columns) and dout against S_aug,
// the partial sums over d of out and den exchanged per chunk, plus this
// segment's sum of phi(Q) gh^T.
template <int D, int M>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dq_nc_w2(
    const bf16 *__restrict__ q, const bf16 *__restrict__ dout, bf16 *__restrict__ dq,
    const float *__restrict__ wsS, float *__restrict__ wsR, int64_t N, int64_t nseg, int64_t seg_tokens,
    int64_t rec) {
    static_assert(D == 2 * kW2Half, "two wavefronts of 32 feature rows");
    typedef bf16x4 Fr;
    constexpr int DTH = kW2Half / 16, MT = M / 16, PF = 2;
    constexpr int NV = M / 32;
    constexpr int SQ = 16 * (kW2Half + kStagePad), SV = 16 * (M + kStagePad);
    constexpr int ST = stage_elems<DTH, MT + 1>(), SGT = stage_elems<MT + 1, 1>();
    constexpr int NP = (SQ + SV > ST ? SQ + SV : ST) > SGT ? (SQ + SV > ST ? SQ + SV : ST) : SGT;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const bf16 *Qw = q + bh * N * D + w * kW2Half;
    const bf16 *G = dout + bh * N * M;
    bf16 *DQw = dq + bh * N * D + w * kW2Half;

    __shared__ __align__(16) bf16 priv_mem[2][NP];
    __shared__ __align__(16) f32x4 xbuf[2][2][MT + 1][64];   // [chunk parity][wavefront][tile][lane]
    lds_bf16 *sq = (lds_bf16 *)priv_mem[w];
    lds_bf16 *sg = sq + SQ;

    Fr SF[MT + 1][DTH], SFT[MT + 1][DTH];   // S_aug rows of this wavefront, both orientations
    {
        f32x4 St[DTH][MT + 1];
        rows_load<D, M, DTH, true>(St, wsS + bh * nseg * rec, w * kW2Half);
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt) SF[mt][dt] = IO<bf16>::to_frag(St[dt][mt]);
        transpose_frags<DTH, MT + 1>(SFT, SF, sq);
    }
    f32x4 Ra[DTH][MT + 1];
#pragma unroll
    for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) Ra[dt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};

    dwordx4 lq[PF], lg[PF][NV];
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        lq[b] = load_cols32<D>(Qw, t_begin + b * BCH, t_end);
        load_rows32<M>(lg[b], G, t_begin + b * BCH, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * BCH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + b * BCH;
        if (t0 >= t_end) break;   // uniform over the workgroup
        stage_cols32_phi(sq, lq[b]);   // rows past t_end: gh = 0 below, so no mask
        stage_lines<M, 1, false, false>(sg, lg[b], t0, t_end);
        lq[b] = load_cols32<D>(Qw, t0 + PF * BCH, t_end);
        load_rows32<M>(lg[b], G, t0 + PF * BCH, t_end);
        __builtin_amdgcn_sched_barrier(0);
        const int64_t t = t0 + c;
        const bool valid = t < t_end;

        Fr Qn[1][DTH], QT[1][DTH], Gr[1][MT];
        natural_frags_lds<kW2Half, 1>(Qn, sq);
        transposed_frags_lds<kW2Half, 1>(QT, sq);
        natural_frags_lds<M, 1>(Gr, sg);
        f32x4 Ot[MT + 1];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) {
            Ot[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DTH; dt += 2) mma2(Ot[mt], SF[mt][dt], SF[mt][dt + 1], Qn[0][dt], Qn[0][dt + 1]);
        }
        const int par = int((t0 - t_begin) / BCH) & 1;
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) xbuf[par][w][mt][lane] = Ot[mt];
        lds_barrier();
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) Ot[mt] += xbuf[par][1 - w][mt][lane];

        const float inv = valid ? __builtin_amdgcn_rcpf(Ot[MT][0]) : 0.f;
        float go = 0.f;
        f32x4 gv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 graw = IO<bf16>::to_f32(Gr[0][mt]);
            const f32x4 o = Ot[mt];   // out times d: the 1/d factors are applied to the sum
            go += graw[0] * o[0] + graw[1] * o[1] + graw[2] * o[2] + graw[3] * o[3];
            gv[mt] = graw * inv;
        }
        go += __shfl_xor(go, 16);
        go += __shfl_xor(go, 32);
        const float h = -(go * inv) * inv;   // -(dout . out) / d with out = Ot / d
        Fr Gn[1][MT + 1];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) Gn[0][mt] = IO<bf16>::to_frag(gv[mt]);
        Gn[0][MT] = IO<bf16>::to_frag(f32x4{g == 0 ? h : 0.f, 0.f, 0.f, 0.f});

        // dL/dqh^T for this wavefront's rows d = S_aug gh, times min(phi(q), 1)
        lds_bf16 *dtile = sg;   // the dout rows are read
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, SFT[mt][dt], SFT[mt + 1][dt], Gn[0][mt], Gn[0][mt + 1]);
            if ((MT & 1) == 0) mma1(acc, SFT[MT][dt], Gn[0][MT]);
            const f32x4 qh = IO<bf16>::to_f32(Qn[0][dt]);
            const f32x4 dp = {__builtin_fminf(qh[0], 1.f), __builtin_fminf(qh[1], 1.f), __builtin_fminf(qh[2], 1.f),
                              __builtin_fminf(qh[3], 1.f)};
            tile_put_bf16<kW2Half>(dtile, dt, IO<bf16>::from_f32(acc * dp));
        }
        flush_rows<kW2Half, D, 16>(DQw, t0, t_end, dtile, 0);

        Fr GT[1][MT + 1];
        transpose_frags<MT + 1, 1>(GT, Gn, sq);   // the staged rows are all read
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt) mma1(Ra[dt][mt], QT[0][dt], GT[0][mt]);
    }
    }
    rows_store<D, M, DTH>(wsR + (bh * nseg + seg) * rec, Ra, w * kW2Half);
}

// dK/dV pass: K (its 32 columns) and V against the full R_aug; dV's partial
// sums over d are exchanged per chunk.
template <int D, int M>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_dkdv_nc_w2(
    const bf16 *__restrict__ k, const bf16 *__restrict__ v, bf16 *__restrict__ dk, bf16 *__restrict__ dv,
    const float *__restrict__ wsR, int64_t N, int64_t nseg, int64_t seg_tokens, int64_t rec) {
    static_assert(D == 2 * kW2Half, "two wavefronts of 32 feature rows");
    typedef bf16x4 Fr;
    constexpr int DTH = kW2Half / 16, MT = M / 16, MH = MT / 2, PF = 2;
    constexpr int NV = M / 32;
    constexpr int SQ = 16 * (kW2Half + kStagePad), SV = 16 * (M + kStagePad);
    constexpr int ST = stage_elems<DTH, MT + 1>();
    constexpr int NP = SQ + SV > ST ? SQ + SV : ST;
    const int lane = lane_id();
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const bf16 *Kw = k + bh * N * D + w * kW2Half;
    const bf16 *V = v + bh * N * M;
    bf16 *DKw = dk + bh * N * D + w * kW2Half;
    bf16 *DVw = dv + bh * N * M + w * (M / 2);

    __shared__ __align__(16) bf16 priv_mem[2][NP];
    __shared__ __align__(16) f32x4 xbuf[2][2][MH][64];   // [chunk parity][wavefront][tile][lane]
    lds_bf16 *sk = (lds_bf16 *)priv_mem[w];
    lds_bf16 *sv = sk + SQ;

    Fr RF[MT + 1][DTH], RFT[MT + 1][DTH];   // R_aug rows of this wavefront, both orientations
    {
        f32x4 Rr[DTH][MT + 1];
        rows_load<D, M, DTH, false>(Rr, wsR + bh * nseg * rec, w * kW2Half);
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int dt = 0; dt < DTH; ++dt) RF[mt][dt] = IO<bf16>::to_frag(Rr[dt][mt]);
        transpose_frags<DTH, MT + 1>(RFT, RF, sk);
    }
    const Fr k0ones = frag_k0_ones<Fr>();

    dwordx4 lk[PF], lv[PF][NV];
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        lk[b] = load_cols32<D>(Kw, t_begin + b * BCH, t_end);
        load_rows32<M>(lv[b], V, t_begin + b * BCH, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * BCH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + b * BCH;
        if (t0 >= t_end) break;   // uniform over the workgroup
        // rows past t_end only produce outputs that are not stored
        stage_cols32_phi(sk, lk[b]);
        stage_lines<M, 1, false, false>(sv, lv[b], t0, t_end);
        lk[b] = load_cols32<D>(Kw, t0 + PF * BCH, t_end);
        load_rows32<M>(lv[b], V, t0 + PF * BCH, t_end);
        __builtin_amdgcn_sched_barrier(0);

        Fr Kn[1][DTH], Vn[1][MT];
        natural_frags_lds<kW2Half, 1>(Kn, sk);
        natural_frags_lds<M, 1>(Vn, sv);
        // dV^T shares over this wavefront's rows d: sum_d R[d][m] kh[j][d]
        f32x4 dvs[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            dvs[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DTH; dt += 2) mma2(dvs[mt], RF[mt][dt], RF[mt][dt + 1], Kn[0][dt], Kn[0][dt + 1]);
        }
        const int par = int((t0 - t_begin) / BCH) & 1;
#pragma unroll
        for (int i = 0; i < MH; ++i) xbuf[par][w][i][lane] = w ? dvs[i] : dvs[MH + i];

        // dL/dkh^T for this wavefront's rows d = R_aug vh, times min(phi(k), 1)
        lds_bf16 *dtile = sk;   // the staged rows are read
#pragma unroll
        for (int dt = 0; dt < DTH; ++dt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt + 1 <= MT; mt += 2) mma2(acc, RFT[mt][dt], RFT[mt + 1][dt], Vn[0][mt], Vn[0][mt + 1]);
            mma1(acc, RFT[MT][dt], k0ones);
            const f32x4 kh = IO<bf16>::to_f32(Kn[0][dt]);
            const f32x4 dp = {__builtin_fminf(kh[0], 1.f), __builtin_fminf(kh[1], 1.f), __builtin_fminf(kh[2], 1.f),
                              __builtin_fminf(kh[3], 1.f)};
            tile_put_bf16<kW2Half>(dtile, dt, IO<bf16>::from_f32(acc * dp));
        }
        flush_rows<kW2Half, D, 16>(DKw, t0, t_end, dtile, 0);

        lds_barrier();
        lds_bf16 *vtile = dtile;
#pragma unroll
        for (int i = 0; i < MH; ++i)
            tile_put_bf16<M / 2>(vtile, i, IO<bf16>::from_f32((w ? dvs[MH + i] : dvs[i]) + xbuf[par][1 - w][i][lane]));
        flush_rows<M / 2, M, 16>(DVw, t0, t_end, vtile, 0);
    }
    }
}

template <typename T, int D, int M>
static hipError_t run_backward(bool causal, const void *q, const void *k, const void *v, const void *dout, void *dq,
                               void *dk, void *dv, int64_t BH, int64_t N, float *ws, hipStream_t s) {
    const SegPlan p = make_plan(BH, N, D, M);
    const BwdLayout L = backward_layout(BH, N, D, M, sizeof(T));
    float *wsS = ws;
    float *wsR = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.states);
    float *ibuf = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.inv_off);
    float *hbuf = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.h_off);
    const dim3 grid(unsigned(BH * p.nseg));
    const int dt = sizeof(T) == 4 ? 0 : 1;
    hipError_t e = launch_segment_state(dt, k, v, wsS, BH, N, D, M, s);
    if (e != hipSuccess) return e;
    // two wavefronts per segment (their kernels address a head with 32-bit
    // element offsets)
    const bool w2 = sizeof(T) == 2 && D == 2 * kW2Half && N * (D > M ? D : M) <= int64_t(INT32_MAX);
    if (!causal) {   // full sums S_aug, then R_aug, each into record 0 of the head
        if ((e = launch_scan(wsS, BH, p.nseg, p.rec, 1, s)) != hipSuccess) return e;
        if constexpr (sizeof(T) == 2 && D == 2 * kW2Half) if (w2) {
            hipLaunchKernelGGL((k_bwd_dq_nc_w2<D, M>), grid, dim3(128), 0, s, (const bf16 *)q, (const bf16 *)dout,
                               (bf16 *)dq, (const float *)wsS, wsR, N, p.nseg, p.seg_tokens, p.rec);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if ((e = launch_scan(wsR, BH, p.nseg, p.rec, 1, s)) != hipSuccess) return e;
            hipLaunchKernelGGL((k_bwd_dkdv_nc_w2<D, M>), grid, dim3(128), 0, s, (const bf16 *)k, (const bf16 *)v,
                               (bf16 *)dk, (bf16 *)dv, (const float *)wsR, N, p.nseg, p.seg_tokens, p.rec);
            return hipGetLastError();
        }
        hipLaunchKernelGGL((k_bwd_dq<T, D, M, false>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (T *)dq, (const float *)wsS, wsR, (float *)nullptr,
                           (float *)nullptr, N, p.nseg, p.seg_tokens, p.rec);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_scan(wsR, BH, p.nseg, p.rec, 1, s)) != hipSuccess) return e;
        hipLaunchKernelGGL((k_bwd_dkdv<T, D, M, false>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)nullptr, (const float *)nullptr, (const float *)nullptr,
                           (T *)dk, (T *)dv, (const float *)wsR, N, p.nseg, p.seg_tokens, p.rec);
        return hipGetLastError();
    }
    if ((e = launch_scan(wsS, BH, p.nseg, p.rec, 0, s)) != hipSuccess) return e;
    if constexpr (sizeof(T) == 2 && D == 2 * kW2Half) if (w2) {
        hipLaunchKernelGGL((k_bwd_dq_w2<D, M>), grid, dim3(128), 0, s, (const bf16 *)q, (const bf16 *)k,
                           (const bf16 *)v, (const bf16 *)dout, (bf16 *)dq, (const float *)wsS, wsR, ibuf,
                           hbuf, N, p.nseg, p.seg_tokens, p.rec);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_scan(wsR, BH, p.nseg, p.rec, 2, s)) != hipSuccess) return e;
        hipLaunchKernelGGL((k_bwd_dkdv_w2<D, M>), grid, dim3(128), 0, s, (const bf16 *)q, (const bf16 *)k,
                           (const bf16 *)v, (const bf16 *)dout, (const float *)ibuf, (const float *)hbuf,
                           (bf16 *)dk, (bf16 *)dv, (const float *)wsR, N, p.nseg, p.seg_tokens, p.rec);
        return hipGetLastError();
    }
    {
        hipLaunchKernelGGL((k_bwd_dq<T, D, M, true>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (T *)dq, (const float *)wsS, wsR, ibuf, hbuf, N, p.nseg,
                           p.seg_tokens, p.rec);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = launch_scan(wsR, BH, p.nseg, p.rec, 2, s)) != hipSuccess) return e;
        hipLaunchKernelGGL((k_bwd_dkdv<T, D, M, true>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (const float *)ibuf, (const float *)hbuf, (T *)dk,
                           (T *)dv, (const float *)wsR, N, p.nseg, p.seg_tokens, p.rec);
        return hipGetLastError();
    }
}

template <typename T>
static hipError_t run_backward_t(bool causal, const void *q, const void *k, const void *v, const void *dout,
                                 void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, float *ws,
                                 hipStream_t s) {
    if (D == 32 && M == 32) return run_backward<T, 32, 32>(causal, q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 32 && M == 64) return run_backward<T, 32, 64>(causal, q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 64 && M == 32) return run_backward<T, 64, 32>(causal, q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    if (D == 64 && M == 64) return run_backward<T, 64, 64>(causal, q, k, v, dout, dq, dk, dv, BH, N, ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_backward(bool causal, int dt, const void *q, const void *k, const void *v, const void *dout,
                           void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t D, int64_t M, float *ws,
                           hipStream_t s) {
    if (!fused_head_sizes(D, M))
        return launch_backward_generic(causal, dt, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
    if (dt == 0) return run_backward_t<float>(causal, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
    return run_backward_t<bf16>(causal, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
}

} // namespace la
