// la_chunk.h -- per-wavefront chunk primitives shared by the forward and
// backward kernels: loading token tiles, the feature map on load, and the
// fp32 state record <-> accumulator tiles.
//
// A chunk is TT token tiles of 16 tokens.  For a row-major tensor X [N][F]
// the "natural" fragment of token tile tt and feature tile ft holds, in lane
// (c, g), the 4 features 16*ft + 4g .. 16*ft + 4g + 3 of token 16*tt + c:
// one 8-byte (bf16) or 16-byte (fp32) load per lane.
#pragma once
#include <type_traits>

#include "la_device.h"

namespace la {

typedef short i16x4 __attribute__((ext_vector_type(4)));

// Raw load of one chunk of rows [t0, t0 + 16 TT) of a [N][F] slice.  The
// load is issued for every lane (rows at or beyond t_end read row t_end - 1,
// which always exists), so no lane branches around it and the compiler can
// keep several chunks in flight; the consumers (phi_frags, raw_frags) zero
// the rows at or beyond t_end.  Requires t_end >= 1.
template <typename T, int F, int TT>
__device__ __forceinline__ void load_chunk(typename IO<T>::vec4 (&x)[TT][F / 16], const T *__restrict__ base,
                                           int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const int64_t t = min(t0 + 16 * tt + c, t_end - 1);
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) x[tt][ft] = load4<T>(base + t * F + 16 * ft + 4 * g);
    }
}

// phi on load: fragments of phi(X); with MASK rows at or beyond t_end become
// exact zeros (so they add nothing to any state or sum).
template <typename T, int F, int TT, bool MASK = true, typename Fr>
__device__ __forceinline__ void phi_frags(Fr (&y)[TT][F / 16],
                                          const typename IO<T>::vec4 (&x)[TT][F / 16], int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const bool ok = t0 + 16 * tt + c < t_end;
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) {
            f32x4 p = phi4(IO<T>::to_f32(x[tt][ft]));
            if (MASK && !ok) p = f32x4{0.f, 0.f, 0.f, 0.f};
            y[tt][ft] = frag_from<Fr>(p);
        }
    }
}

// V rows as fragments for the forward products, unmasked: every product
// that reads them also multiplies by phi(K) of the same row, which is zero
// past t_end (and the padded rows are copies of row t_end - 1, so finite
// whenever the data is).
__device__ __forceinline__ void value_frags_unmasked(bf16x4 &y, bf16x4 x) { y = x; }
__device__ __forceinline__ void value_frags_unmasked(f32x4 &y, f32x4 x) { y = x; }
__device__ __forceinline__ void value_frags_unmasked(split4 &y, f32x4 x) { y = split_f32(x); }

// The loaded values as fragments, rows at or beyond t_end zeroed (MASK).
template <typename T, int F, int TT, bool MASK = true, typename Fr>
__device__ __forceinline__ void raw_frags(Fr (&y)[TT][F / 16],
                                          const typename IO<T>::vec4 (&x)[TT][F / 16], int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
        const bool ok = t0 + 16 * tt + c < t_end;
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) {
            f32x4 p = IO<T>::to_f32(x[tt][ft]);
            if (MASK && !ok) p = f32x4{0.f, 0.f, 0.f, 0.f};
            y[tt][ft] = frag_from<Fr>(p);
        }
    }
}

// Query/key fragments: phi applied (PHI) or the given features as they are;
// rows at or beyond t_end zeroed either way (MASK).
template <typename T, int F, int TT, bool PHI, bool MASK = true, typename Fr>
__device__ __forceinline__ void feat_frags(Fr (&y)[TT][F / 16],
                                           const typename IO<T>::vec4 (&x)[TT][F / 16], int64_t t0, int64_t t_end) {
    if constexpr (PHI)
        phi_frags<T, F, TT, MASK>(y, x, t0, t_end);
    else
        raw_frags<T, F, TT, MASK>(y, x, t0, t_end);
}

// ---- LDS staging (bf16) ---------------------------------------------------
// A wavefront's private staging area for one chunk of one tensor: rows of
// 16*NF features (bf16), padded to kStagePad extra elements per row.
typedef __attribute__((address_space(3))) bf16 lds_bf16;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
constexpr int kStagePad = 8;

// Token-contiguous copies of bf16 fragments through LDS: the natural
// fragments are written row-major (one 8-byte store per lane and tile), then
// read back with the gfx950 transposing LDS read, which hands lane (c, g) of
// a 16x16 tile the elements [4g + r][c], r = 0..3, when lane (c, g) points at
// row 4g + c/4, columns 4 (c % 4) .. + 3.  Exact (a copy).
template <int NF, int TT>
__device__ __forceinline__ void transpose_frags_lds(bf16x4 (&yt)[TT][NF], const bf16x4 (&y)[TT][NF],
                                                    lds_bf16 *stage) {
    constexpr int S = 16 * NF + kStagePad;
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < NF; ++ft)
            *reinterpret_cast<lds_bf16x4 *>(stage + (16 * tt + c) * S + 16 * ft + 4 * g) = y[tt][ft];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < NF; ++ft) {
            const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                reinterpret_cast<lds_i16x4 *>(stage + (16 * tt + 4 * g + (c >> 2)) * S + 16 * ft + 4 * (c & 3)));
            yt[tt][ft] = __builtin_bit_cast(bf16x4, r);
        }
}

// ---- contiguous chunk loads (bf16) -------------------------------------------
// A chunk of 16 TT rows x F bf16 features is fetched with 16-byte loads in
// row-major order (each load instruction of the wavefront covers 1 KB of
// consecutive memory), which streams HBM far better than per-fragment 8-byte
// loads.  The rows then go through the wavefront's LDS staging area, from
// which the MFMA fragments are read in either orientation.
typedef unsigned int dwordx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) dwordx4 lds_dwordx4;

template <int F, int TT> struct Lines {
    static constexpr int n = TT * F / 32;   // 16-byte loads per lane
};

// Rows at or beyond t_end read row t_end - 1 (always valid); stage_lines
// zeroes them where that matters.  Requires t_end >= 1.
template <int F, int TT>
__device__ __forceinline__ void load_lines(dwordx4 (&x)[TT * F / 32], const bf16 *__restrict__ base, int64_t t0,
                                           int64_t t_end) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < Lines<F, TT>::n; ++i) {
        const int e = (64 * i + l) * 8;          // first element of this lane's 8
        const int64_t t = min(t0 + e / F, t_end - 1);
        x[i] = *reinterpret_cast<const dwordx4 *>(base + t * F + e % F);
    }
}

// phi of 8 packed bf16 values (two per dword), rounded back to bf16.
__device__ __forceinline__ dwordx4 phi8(dwordx4 x) {
    dwordx4 y;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float lo = __builtin_bit_cast(float, x[w] << 16);
        const float hi = __builtin_bit_cast(float, x[w] & 0xffff0000u);
        const bf16x2 p = {(bf16)phi(lo), (bf16)phi(hi)};
        y[w] = __builtin_bit_cast(unsigned int, p);
    }
    return y;
}

// Writes the loaded rows into the staging area (row stride F + kStagePad);
// with PHI the feature map is applied, with MASK rows at or beyond t_end
// become 0.
template <int F, int TT, bool PHI, bool MASK = PHI>
__device__ __forceinline__ void stage_lines(lds_bf16 *stage, const dwordx4 (&x)[TT * F / 32], int64_t t0,
                                            int64_t t_end) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < Lines<F, TT>::n; ++i) {
        const int e = (64 * i + l) * 8;
        const int row = e / F, col = e % F;
        dwordx4 y = x[i];
        if (PHI) y = phi8(y);
        if (MASK && t0 + row >= t_end) y = dwordx4{0u, 0u, 0u, 0u};
        *reinterpret_cast<lds_dwordx4 *>(stage + row * (F + kStagePad) + col) = y;
    }
}

// Natural fragments (token rows, contraction over features) from staging.
template <int F, int TT>
__device__ __forceinline__ void natural_frags_lds(bf16x4 (&y)[TT][F / 16], const lds_bf16 *stage) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft)
            y[tt][ft] = *reinterpret_cast<const lds_bf16x4 *>(stage + (16 * tt + c) * (F + kStagePad) + 16 * ft + 4 * g);
}

// One token-contiguous tile of rows staged with a row stride of S elements:
// rows 16 tt .. 16 tt + 15, feature tile ft (the tile yt[tt][ft] of
// transposed_frags_lds), for reading operand tiles where they are used.
__device__ __forceinline__ bf16x4 transposed_tile_lds(const lds_bf16 *stage, int S, int tt, int ft) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4 *>(
        const_cast<lds_bf16 *>(stage) + (16 * tt + 4 * g + (c >> 2)) * S + 16 * ft + 4 * (c & 3)));
    return __builtin_bit_cast(bf16x4, r);
}

// Token-contiguous fragments from staging (see transpose_frags_lds).
template <int F, int TT>
__device__ __forceinline__ void transposed_frags_lds(bf16x4 (&yt)[TT][F / 16], const lds_bf16 *stage) {
    constexpr int S = F + kStagePad;
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < F / 16; ++ft) {
            const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<lds_i16x4 *>(
                const_cast<lds_bf16 *>(stage) + (16 * tt + 4 * g + (c >> 2)) * S + 16 * ft + 4 * (c & 3)));
            yt[tt][ft] = __builtin_bit_cast(bf16x4, r);
        }
}

// Output tiles of 16 tokens x F bf16 features go through LDS (row stride
// F + kStagePad): each lane puts the 4 consecutive features it holds (Acc
// layout: lane (c, g) has token c, features 16 ft + 4g .. + 3), then every
// store instruction writes 1 KB of whole rows.
template <int F>
__device__ __forceinline__ void tile_put_bf16(lds_bf16 *tile, int ft, bf16x4 x) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    *reinterpret_cast<lds_bf16x4 *>(tile + c * (F + kStagePad) + 16 * ft + 4 * g) = x;
}
template <int F>
__device__ __forceinline__ void tile_flush_bf16(bf16 *__restrict__ dst, int64_t t0, int64_t t_end,
                                                const lds_bf16 *tile) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < F / 32; ++i) {
        const int e = (64 * i + l) * 8, row = e / F, col = e % F;
        const dwordx4 y = *reinterpret_cast<const lds_dwordx4 *>(tile + row * (F + kStagePad) + col);
        if (t0 + row < t_end) *reinterpret_cast<dwordx4 *>(dst + (t0 + row) * F + col) = y;
    }
}

// Elements of LDS staging one wavefront needs per tensor chunk.
template <int NF, int TT> constexpr int stage_elems() { return 16 * TT * (16 * NF + kStagePad); }

// Token-contiguous copies: yt[tt][ft] holds, in lane (c, g), the 4 tokens
// 16*tt + 4g .. + 3 of feature 16*ft + c.  bf16 goes through LDS; fp32 goes
// through an identity product on the matrix cores.
template <int NF, int TT>
__device__ __forceinline__ void transpose_frags(f32x4 (&yt)[TT][NF], const f32x4 (&y)[TT][NF], lds_bf16 *) {
    const f32x4 ident = frag_identity<f32x4>();
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < NF; ++ft) yt[tt][ft] = transpose_frag(y[tt][ft], ident);
}
template <int NF, int TT>
__device__ __forceinline__ void transpose_frags(bf16x4 (&yt)[TT][NF], const bf16x4 (&y)[TT][NF], lds_bf16 *stage) {
    transpose_frags_lds<NF, TT>(yt, y, stage);
}
// Split fp32 operands (split4): the hi parts through the LDS area at `stage`,
// the lo parts through the one after it, so the area is twice
// stage_elems<NF, TT>() elements.  Exact (copies).
template <int NF, int TT>
__device__ __forceinline__ void transpose_frags(split4 (&yt)[TT][NF], const split4 (&y)[TT][NF], lds_bf16 *stage) {
    bf16x4 h[TT][NF], l[TT][NF], ht[TT][NF], lt[TT][NF];
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            h[tt][f] = split_hi(y[tt][f]);
            l[tt][f] = split_lo(y[tt][f]);
        }
    transpose_frags_lds<NF, TT>(ht, h, stage);
    transpose_frags_lds<NF, TT>(lt, l, stage + stage_elems<NF, TT>());
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) yt[tt][f] = split_join(ht[tt][f], lt[tt][f]);
}
// LDS elements a transpose_frags of fragment type Fr takes (split4: two areas).
template <typename Fr, int NF, int TT> constexpr int transpose_stage_elems() {
    return (std::is_same<Fr, split4>::value ? 2 : 1) * stage_elems<NF, TT>();
}

// ---- state records --------------------------------------------------------
// A state record is D*M floats of S (row-major [d][m]) followed by D floats
// of Z.  In registers the state is an augmented D x (M + 16) matrix of Acc
// tiles St[dt][mt], dt < D/16, mt <= M/16: tile mt = M/16 holds Z in its
// column 0 and zeros elsewhere (or Z in every column, see state_load), so
// the products that use S also produce the normalizer.  Lane (c, g) element r of St[dt][mt] is row d = 16 dt + 4g + r,
// column m = 16 mt + c.
// With REP the normalizer tile holds Z in every column instead of column 0
// (the layout the forward kernels use: their normalizer rows come out
// replicated, so each lane holds its tokens' denominators).
template <int D, int M, bool REP = false>
__device__ __forceinline__ void state_load(f32x4 (&St)[D / 16][M / 16 + 1], const float *__restrict__ rec) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) St[dt][mt][r] = rec[(16 * dt + 4 * g + r) * M + 16 * mt + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) St[dt][M / 16][r] = (REP || c == 0) ? rec[D * M + 16 * dt + 4 * g + r] : 0.f;
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

// The same state in fragment order, for records that are only ever summed
// elementwise (the causal forward's block totals and prefixes): the S part
// is the Acc tiles one after another, St[dt][mt] (mt < M/16) as 64 lanes x 4
// consecutive floats, so every lane moves one f32x4 per tile without LDS
// bank conflicts; Z follows in natural order, D floats.  Same size as the
// row-major record.
template <int D, int M>
__device__ __forceinline__ void state_store_frag(float *__restrict__ rec, const f32x4 (&St)[D / 16][M / 16 + 1]) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    f32x4 *r4 = reinterpret_cast<f32x4 *>(rec);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt) r4[(dt * (M / 16) + mt) * 64 + lane] = St[dt][mt];
        if (c == 0) r4[(D * M) / 4 + 4 * dt + g] = St[dt][M / 16];
    }
}
// St = A + B of two fragment-order records (B may be null), normalizer tile
// replicated (the REP layout of state_load).
template <int D, int M>
__device__ __forceinline__ void state_load_frag2(f32x4 (&St)[D / 16][M / 16 + 1], const float *__restrict__ a,
                                                 const float *__restrict__ b) {
    const int lane = lane_id(), g = lane >> 4;
    const f32x4 *a4 = reinterpret_cast<const f32x4 *>(a);
    const f32x4 *b4 = reinterpret_cast<const f32x4 *>(b);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt) {
            const int i = (dt * (M / 16) + mt) * 64 + lane;
            St[dt][mt] = b4 ? a4[i] + b4[i] : a4[i];
        }
        const int i = (D * M) / 4 + 4 * dt + g;
        St[dt][M / 16] = b4 ? a4[i] + b4[i] : a4[i];
    }
}

// Element i4 (an f32x4) of a fragment-order record, from / to a state kept
// as separate row-major S [D][M] and Z [D]: an S element holds rows
// 16 dt + 4g + r (r = 0..3) of column 16 mt + c, where i4 = (dt (M/16) + mt)
// 64 + 16 g + c; past the S part, 4 consecutive Z entries.
template <int D, int M>
__device__ __forceinline__ f32x4 record_frag4_load(const float *S, const float *Z, int i4) {
    if (i4 < D * M / 4) {
        const int ln = i4 & 63, tile = i4 >> 6, dt = tile / (M / 16), mt = tile % (M / 16);
        const float *p = S + (16 * dt + 4 * (ln >> 4)) * M + 16 * mt + (ln & 15);
        return f32x4{p[0], p[M], p[2 * M], p[3 * M]};
    }
    return *reinterpret_cast<const f32x4 *>(Z + 4 * (i4 - D * M / 4));
}
template <int D, int M>
__device__ __forceinline__ void record_frag4_store(float *S, float *Z, int i4, f32x4 x) {
    if (i4 < D * M / 4) {
        const int ln = i4 & 63, tile = i4 >> 6, dt = tile / (M / 16), mt = tile % (M / 16);
        float *p = S + (16 * dt + 4 * (ln >> 4)) * M + 16 * mt + (ln & 15);
        p[0] = x[0];
        p[M] = x[1];
        p[2 * M] = x[2];
        p[3 * M] = x[3];
    } else {
        *reinterpret_cast<f32x4 *>(Z + 4 * (i4 - D * M / 4)) = x;
    }
}

// St += sum over the chunk's tokens of A_t B_t^T, where KT/VT are
// token-contiguous fragments (KT: rows = the D features of A; VT: rows = the
// M features of B).  The extra column block adds sum_t A_t to the
// normalizer column (to every column of that block with REP).
template <typename Fr, int D, int M, int TT, bool REP = false>
__device__ __forceinline__ void state_accumulate(f32x4 (&St)[D / 16][M / 16 + 1], const Fr (&KT)[TT][D / 16],
                                                 const Fr (&VT)[TT][M / 16]) {
    const Fr ones = REP ? frag_ones<Fr>() : frag_row0_ones<Fr>();
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
