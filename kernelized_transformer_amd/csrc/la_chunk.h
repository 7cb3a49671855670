// la_chunk.h -- per-wavefront chunk primitives shared by the forward and
// backward kernels: loading token tiles, the feature map on load, and the
// fp32 state record <-> accumulator tiles.
//
// A chunk is TT token tiles of 16 tokens.  For a row-major tensor X [N][F]
// the "natural" fragment of token tile tt and feature tile ft holds, in lane
// (c, g), the 4 features 16*ft + 4g .. 16*ft + 4g + 3 of token 16*tt + c:
// one 8-byte (bf16) or 16-byte (fp32) load per lane.
#pragma once

#include "la_device.h"

namespace la {

// Raw load of one chunk of rows [t0, t0 + 16 TT) of a [N][F] slice; rows at
// or beyond t_end read as zero.
template <typename T, int F, int TT>
__device__ __forceinline__ void load_chunk(typename IO<T>::vec4 (&x)[TT][F / 16], const T *__restrict__ base,
                                           int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t t = t0 + 16 * tt + c;
        const bool ok = t < t_end;
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) {
            typename IO<T>::vec4 z = {0, 0, 0, 0};
            x[tt][ft] = ok ? load4<T>(base + t * F + 16 * ft + 4 * g) : z;
        }
    }
}

// phi on load: fragments of phi(X); rows at or beyond t_end become exact
// zeros (so they add nothing to any state or sum).
template <typename T, int F, int TT>
__device__ __forceinline__ void phi_frags(typename IO<T>::frag (&y)[TT][F / 16],
                                          const typename IO<T>::vec4 (&x)[TT][F / 16], int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const bool ok = t0 + 16 * tt + c < t_end;
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) {
            f32x4 p = phi4(IO<T>::to_f32(x[tt][ft]));
            if (!ok) p = f32x4{0.f, 0.f, 0.f, 0.f};
            y[tt][ft] = IO<T>::to_frag(p);
        }
    }
}

template <typename T, int F, int TT>
__device__ __forceinline__ void raw_frags(typename IO<T>::frag (&y)[TT][F / 16],
                                          const typename IO<T>::vec4 (&x)[TT][F / 16]) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) y[tt][ft] = IO<T>::to_frag(IO<T>::to_f32(x[tt][ft]));
}

// Token-contiguous copies: yt[tt][ft] holds, in lane (c, g), the 4 tokens
// 16*tt + 4g .. + 3 of feature 16*ft + c.
template <typename Fr, int NF, int TT>
__device__ __forceinline__ void transpose_frags(Fr (&yt)[TT][NF], const Fr (&y)[TT][NF]) {
    const Fr ident = frag_identity<Fr>();
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < NF; ++ft) yt[tt][ft] = transpose_frag(y[tt][ft], ident);
}

// ---- state records --------------------------------------------------------
// A state record is D*M floats of S (row-major [d][m]) followed by D floats
// of Z.  In registers the state is an augmented D x (M + 16) matrix of Acc
// tiles St[dt][mt], dt < D/16, mt <= M/16: tile mt = M/16 holds Z in its
// column 0 and zeros elsewhere, so the products that use S also produce the
// normalizer.  Lane (c, g) element r of St[dt][mt] is row d = 16 dt + 4g + r,
// column m = 16 mt + c.
template <int D, int M>
__device__ __forceinline__ void state_load(f32x4 (&St)[D / 16][M / 16 + 1], const float *__restrict__ rec) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) St[dt][mt][r] = rec[(16 * dt + 4 * g + r) * M + 16 * mt + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) St[dt][M / 16][r] = (c == 0) ? rec[D * M + 16 * dt + 4 * g + r] : 0.f;
    }
}

// The same record as transposed tiles StT[mt][dt] (rows = the M + 16
// augmented columns, cols = d): lane (c, g) element r of StT[mt][dt] is
// S[16 dt + c][16 mt + 4g + r]; block mt = M/16 holds Z[d] in its row 0.
template <int D, int M>
__device__ __forceinline__ void stateT_load(f32x4 (&StT)[M / 16 + 1][D / 16], const float *__restrict__ rec) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) StT[mt][dt][r] = rec[(16 * dt + c) * M + 16 * mt + 4 * g + r];
        StT[M / 16][dt] = f32x4{g == 0 ? rec[D * M + 16 * dt + c] : 0.f, 0.f, 0.f, 0.f};
    }
}

template <int D, int M>
__device__ __forceinline__ void state_zero(f32x4 (&St)[D / 16][M / 16 + 1]) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int mt = 0; mt <= M / 16; ++mt) St[dt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D, int M>
__device__ __forceinline__ void state_store(float *__restrict__ rec, const f32x4 (&St)[D / 16][M / 16 + 1]) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[(16 * dt + 4 * g + r) * M + 16 * mt + c] = St[dt][mt][r];
        if (c == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[D * M + 16 * dt + 4 * g + r] = St[dt][M / 16][r];
        }
    }
}

// St += sum over the chunk's tokens of A_t B_t^T, where KT/VT are
// token-contiguous fragments (KT: rows = the D features of A; VT: rows = the
// M features of B).  The extra column block adds sum_t A_t to the
// normalizer column.
template <typename Fr, int D, int M, int TT>
__device__ __forceinline__ void state_accumulate(f32x4 (&St)[D / 16][M / 16 + 1], const Fr (&KT)[TT][D / 16],
                                                 const Fr (&VT)[TT][M / 16]) {
    const Fr ones = frag_row0_ones<Fr>();
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt <= M / 16; ++mt) {
#pragma unroll
            for (int tt = 0; tt + 1 < TT; tt += 2)
                mma2(St[dt][mt], KT[tt][dt], KT[tt + 1][dt], mt < M / 16 ? VT[tt][mt] : ones,
                     mt < M / 16 ? VT[tt + 1][mt] : ones);
            if (TT & 1) mma1(St[dt][mt], KT[TT - 1][dt], mt < M / 16 ? VT[TT - 1][mt] : ones);
        }
    }
}

// acc += sum over token tiles tt of A[tt] B[tt]^T (pairs tiles on bf16).
template <typename Fr, int TT>
__device__ __forceinline__ void mma_tiles(f32x4 &acc, const Fr (&A)[TT], const Fr (&B)[TT]) {
#pragma unroll
    for (int tt = 0; tt + 1 < TT; tt += 2) mma2(acc, A[tt], A[tt + 1], B[tt], B[tt + 1]);
    if (TT & 1) mma1(acc, A[TT - 1], B[TT - 1]);
}

// Frag with a single one at contraction index 0 of each row: lane (c, 0)
// element 0.  As the last feature tile of a row it appends a constant 1 to
// that row (the augmented [V, 1] or [g, h] rows of the backward pass).
template <typename F> __device__ __forceinline__ F frag_k0_ones() {
    const float o = (lane_id() < 16) ? 1.f : 0.f;
    return frag_from<F>(f32x4{o, 0.f, 0.f, 0.f});
}

} // namespace la
