// la_poly.hip -- causal attention with the degree-2 polynomial kernel on gfx950.
//
// [summary] 3.2.1: a degree-2 polynomial kernel has an exact finite feature
// map.  Reading: sim(q, k) = (q . k)^2, so
//   out_i = sum_{j<=i} (q_i . k_j)^2 v_j / sum_{j<=i} (q_i . k_j)^2.
//
// Feature map.  (q . k)^2 = sum_a q_a^2 k_a^2 + 2 sum_{a<b} q_a q_b k_a k_b, so
// the D (D + 1) / 2 products x_a x_b, a <= b, make an exact map once the
// off-diagonal terms are counted twice.  The kernels keep every product
// unscaled (state S = sum_j phi(k_j) v_j^T over these features) and apply the
// factor 2 where the readout's partial sums are combined:
//   num_i = 2 phi_off(q_i) . S_off + phi_diag(q_i) . S_diag.
// The normalizer uses the D x D form instead, den_i = q_i^T Z q_i with
// Z = sum_j k_j k_j^T, which needs no features at all.
//
// Feature tiles.  The matrix cores see the features in tiles of 16, one per
// lane c of a row of 16 lanes; lane c "owns" the dimensions c + 16 i
// (i < D / 16).  A tile pairs an owned dimension of lane c with one of lane
// (c + d) % 16 for a lane offset d:
//   d = 0       the pairs {c + 16 i, c + 16 j}, i <= j, within the lane;
//   d = 1..7    {c + 16 i, (c + d) % 16 + 16 j} for i < D / 32, every j;
//   d = 9..15   the same for j >= D / 32, every i;
//   d = 8       lanes c < 8 take i < D / 32, lanes c >= 8 take j >= D / 32.
// Lane c at offset d and lane c + d at offset 16 - d then split the products
// of their dimensions between them, so every unordered pair appears exactly
// once: 33 tiles (528 features) at D = 32, 130 tiles (2080) at D = 64.
//   * In the state update S_f += phi(K)_f^T V the feature index runs along the
//     lanes and the tokens along the contraction: lane (c, g) multiplies its
//     own values k[t][c + 16 i] by the partner's k[t][(c + d) % 16 + 16 j],
//     fetched by a DPP row rotation that the compiler folds into the multiply.
//   * In the readout O^T += S_f^T phi(Q)_f^T the features run along the
//     contraction, four per lane (rows 4g + r of the tile); lane (c, g) holds
//     token c's q rotated by 4g within each 16-dimension block, so every
//     product reads registers at compile-time indices.
//
// Work split.  A workgroup owns one segment of one (b, h) and a block of MB
// output columns.  Its wavefronts split the feature tiles (each carries its
// tiles' fp32 S in registers) and the 16 x 16 tiles of Z; at D = M = 32 one
// more wavefront only stages chunks from memory into LDS.  Per 32-token chunk
// (two token tiles) every state wavefront of the output kernel
//   1. forms phi(q) for its tiles and adds its share of the readout from the
//      prefix state, and its share of q^T Z q; the wavefronts that own output
//      tiles also form the intra-chunk part (q_i . k_j)^2, j <= i, on the
//      matrix cores;
//   2. forms phi(k) for its tiles and updates them (and its Z tiles);
//   3. posts its partial readouts to the owners through LDS; after one
//      workgroup barrier the owners add them up, divide and store.
// Segments: k_poly_segment_state sums each segment's S and Z into a record
// (longer chunks: it exchanges nothing), the shared scan turns the records
// into exclusive prefixes, and k_poly_output starts every segment from its
// prefix.  A single segment per (b, h) skips both.
#include <type_traits>

#include "la_chunk.h"
#include "la_internal.h"

namespace la {

namespace {

// kind 0: diagonal {c + 16i}^2; 1: pair within the lane, i < j; 2: lane
// offset d (1..15 without 8); 3: lane offset 8, slot s, split by lane half.
struct PolyTile {
    int kind, d, i, j, s;
};

template <int NL> constexpr int poly_tiles() { return NL * (NL + 1) / 2 + 15 * NL * NL / 2; }

template <int NL> constexpr PolyTile poly_tile(int f) {
    int n = 0;
    for (int i = 0; i < NL; ++i) {
        if (n == f) return PolyTile{0, 0, i, i, 0};
        ++n;
    }
    for (int i = 0; i < NL; ++i)
        for (int j = i + 1; j < NL; ++j) {
            if (n == f) return PolyTile{1, 0, i, j, 0};
            ++n;
        }
    for (int d = 1; d < 16; ++d) {
        if (d == 8) continue;
        for (int i = 0; i < NL; ++i)
            for (int j = 0; j < NL; ++j)
                if (d < 8 ? i < NL / 2 : j >= NL / 2) {
                    if (n == f) return PolyTile{2, d, i, j, 0};
                    ++n;
                }
    }
    for (int s = 0; s < NL * NL / 2; ++s) {
        if (n == f) return PolyTile{3, 8, 0, 0, s};
        ++n;
    }
    return PolyTile{-1, 0, 0, 0, 0};
}

// The groups of four rotated q values (bit 4 i + x / 4: qr[16 i + x .. + 3])
// that the readout of tiles [f0, f1) reads; group 0 of every block is always
// included (the intra-chunk products and the normalizer use it).  The others
// are never loaded, so they take no registers.
template <int NL> constexpr unsigned poly_qr_groups(int f0, int f1) {
    unsigned m = 0;
    for (int i = 0; i < NL; ++i) m |= 1u << (4 * i);
    for (int f = f0; f < f1; ++f) {
        const PolyTile t = poly_tile<NL>(f);
        for (int r = 0; r < 4; ++r) {
            if (t.kind == 2) {
                m |= 1u << (4 * t.j + ((r + t.d) % 16) / 4);
            } else if (t.kind == 3) {
                m |= 1u << (4 * (t.s % NL) + (r + 8) / 4);
                m |= 1u << (4 * (NL / 2 + t.s / NL) + (r + 8) / 4);
            }
        }
    }
    return m;
}

// x as held by lane (c + d) % 16 of the same row of 16 lanes (a DPP row
// rotation: with row_ror:n, lane l reads lane l - n of its row).
template <int d> __device__ __forceinline__ float from_lane_ahead(float x) {
    static_assert(d >= 1 && d <= 15, "lane offset");
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x120 + (16 - d), 0xf, 0xf, true));
}

// phi(k) of tile F for the update: lane (c, g) element r is the feature of
// lane c for token 4g + r of the token tile; own[i] holds k[token][c + 16 i].
// lo: this lane is one of c < 8.
template <int NL, int F> __device__ __forceinline__ f32x4 phi_k(const f32x4 (&own)[NL], bool lo) {
    constexpr PolyTile t = poly_tile<NL>(F);
    static_assert(t.kind >= 0, "tile index");
    f32x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (t.kind == 0) {
            p[r] = own[t.i][r] * own[t.i][r];
        } else if constexpr (t.kind == 1) {
            p[r] = own[t.i][r] * own[t.j][r];
        } else if constexpr (t.kind == 2) {
            p[r] = own[t.i][r] * from_lane_ahead<t.d>(own[t.j][r]);
        } else {
            // lanes c < 8: own s / NL x partner's s % NL; lanes c >= 8: own
            // s % NL x partner's NL / 2 + s / NL (each lane hands its partner
            // the value the partner needs)
            const float sel = lo ? own[t.s / NL][r] : own[t.s % NL][r];
            const float src = lo ? own[NL / 2 + t.s / NL][r] : own[t.s % NL][r];
            p[r] = sel * from_lane_ahead<8>(src);
        }
    }
    return p;
}

// phi(q) of tile F for the readout: lane (c, g) element r is feature row
// 4g + r of the tile for token c; qr[x + 16 i] = q[c][(4g + x) % 16 + 16 i].
// glo: this lane is one of g < 2 (feature rows below 8).  The diagonal
// features come out halved: every partial readout is doubled when the
// partials are combined, which counts the off-diagonal pairs twice and the
// diagonal once.
template <int NL, int F, bool HALF_DIAG = true>
__device__ __forceinline__ f32x4 phi_q(const float (&qr)[16 * NL], bool glo) {
    constexpr PolyTile t = poly_tile<NL>(F);
    f32x4 p;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (t.kind == 0) {
            p[r] = qr[r + 16 * t.i] * (HALF_DIAG ? 0.5f * qr[r + 16 * t.i] : qr[r + 16 * t.i]);
        } else if constexpr (t.kind == 1) {
            p[r] = qr[r + 16 * t.i] * qr[r + 16 * t.j];
        } else if constexpr (t.kind == 2) {
            p[r] = qr[r + 16 * t.i] * qr[(r + t.d) % 16 + 16 * t.j];
        } else {
            const float a = glo ? qr[r + 16 * (t.s / NL)] : qr[r + 16 * (t.s % NL)];
            const float b = glo ? qr[r + 8 + 16 * (t.s % NL)] : qr[r + 8 + 16 * (NL / 2 + t.s / NL)];
            p[r] = a * b;
        }
    }
    return p;
}

// ---- configuration --------------------------------------------------------
// Two wavefronts per SIMD keep both the matrix cores and the VALU busy (one
// wavefront alone issues them largely one after the other), so a workgroup is
// 8 wavefronts: at D = M = 32, seven hold the state and one (the producer)
// only moves chunks from memory into LDS; otherwise all 8 hold the state and
// load the next chunk while they work on the current one.
template <typename T, int D, int M> struct PolyCfg {
    static constexpr int NL = D / 16;                   // dimension tiles
    static constexpr int FT = poly_tiles<NL>();         // feature tiles
    static constexpr int MB = D == 32 ? M : 16;         // output columns per workgroup
    static constexpr int NMB = M / MB;                  // workgroups per segment
    static constexpr int MT = MB / 16;                  // column tiles per workgroup
    static constexpr int MTOT = M / 16;                 // column tiles of the record
    static constexpr bool PROD = D == 32 && M == 32;    // a producer wavefront feeds the chunks
    static constexpr int W = D == 32 ? (M == 32 ? 7 : 4) : 8;   // wavefronts holding the state
    static constexpr int PF = 3;                        // chunks in flight (producer)
    static constexpr int NWAVE = W + (PROD ? 1 : 0);
    static constexpr int TT = 2;                        // token tiles per chunk (outputs)
    static constexpr int CH = 16 * TT;                  // tokens per chunk (outputs)
    // The segment sums exchange nothing between wavefronts, so they take
    // longer chunks: fewer barriers, more work between them.
    static constexpr int TT1 = 4;
    static constexpr int PF1 = 3;
    // State converted to bf16 once per chunk (else once per token tile,
    // which needs fewer registers).
    static constexpr bool SB_CACHE = D == 32;
    static constexpr bool QR_BOTH = false;
    static constexpr int NZ = NL * NL;                  // Z tiles
    static constexpr int NOUT = TT * MT;                // output tiles per chunk
    static constexpr int REC = (FT * MTOT + NZ) * 256;  // floats per record
    // Feature tiles [split(w), split(w + 1)) of wavefront w: the owners of
    // output tiles (waves 0..NOUT-1) take fewer, since they also form the
    // intra-chunk part and combine the partial sums.  The first NL tiles (the
    // diagonal features) always go to wavefront 0.
    // Wavefronts w and w + 4 share a SIMD, so the producer (wavefront 7)
    // shares one with wavefront 3, which takes fewer tiles.  PASS 1: the
    // segment sums; PASS 2: the outputs.
    static constexpr int split(int w, int pass) {
        if (PROD) {
            constexpr int s1[8] = {0, 5, 10, 15, 17, 22, 27, 33};
            constexpr int s2[8] = {0, 4, 8, 12, 19, 23, 28, 33};
            return pass == 1 ? s1[w] : s2[w];
        }
        return w * FT / W;
    }
    // Z tiles [zsplit(w), zsplit(w + 1)): pairs sharing a row block, on the
    // wavefronts that own no output tiles when there are such.
    static constexpr int zsplit(int w, int pass) {
        if (PROD) {
            constexpr int s1[8] = {0, 0, 0, 0, 2, 2, 4, 4};
            constexpr int s2[8] = {0, 0, 0, 0, 0, 2, 4, 4};
            return pass == 1 ? s1[w] : s2[w];
        }
        return w * NZ / W;
    }
    static_assert(split(0, 1) == 0 && split(W, 1) == FT && split(1, 1) >= NL, "feature tiles");
    static_assert(split(0, 2) == 0 && split(W, 2) == FT && split(1, 2) >= NL, "feature tiles");
    static_assert(zsplit(0, 1) == 0 && zsplit(W, 1) == NZ && zsplit(0, 2) == 0 && zsplit(W, 2) == NZ, "Z tiles");
};

// Owner of output tile (token tile tt, column tile mt).  With four token
// tiles and two wavefronts per column tile, a wavefront takes token tiles
// {0, 3} or {1, 2}, so the intra-chunk work (tt + 1 key tiles) is balanced.
template <int TT, int MT, int W> constexpr int poly_owner(int tt, int mt) {
    if (TT == 4 && 2 * MT == W) return 2 * mt + ((tt == 0 || tt == 3) ? 0 : 1);
    return (tt * MT + mt) % W;
}
struct PolyOwn {
    int n, tt[16], mt[16];
};
template <int TT, int MT, int W> constexpr PolyOwn poly_own(int wi) {
    PolyOwn o{0, {}, {}};
    for (int tt = 0; tt < TT; ++tt)
        for (int mt = 0; mt < MT; ++mt)
            if (poly_owner<TT, MT, W>(tt, mt) == wi) {
                o.tt[o.n] = tt;
                o.mt[o.n] = mt;
                ++o.n;
            }
    return o;
}

// LDS of one workgroup: two chunk buffers (staged q in fp32, k and v in T,
// and k transposed in fp32) and, for the outputs (OUT), two buffers of partial
// results (one per chunk parity).
template <typename T, int D, int M, int TT, bool OUT> struct PolyShared {
    typedef PolyCfg<T, D, M> C;
    static constexpr int CH = 16 * TT;
    static constexpr int QS = D + 4;                    // floats per staged q row
    static constexpr int PAD = sizeof(T) == 2 ? 8 : 4;  // elements of padding per k, v row
    static constexpr int KS = D + PAD, VS = C::MB + PAD;
    static constexpr int KTS = CH + 4;                  // floats per row of the transposed fp32 K
    alignas(16) float q[2][OUT ? CH * QS : 4];
    alignas(16) float kt[2][D * KTS];                   // kt[d][t] = k[t][d]: the feature products' operand
    alignas(16) T k[2][CH * KS];
    alignas(16) T v[2][CH * VS];
    alignas(16) f32x4 part[2][OUT ? TT * C::MT : 1][OUT ? C::W : 1][64];
    alignas(16) float den[2][OUT ? C::W : 1][TT][64];
};

// Global -> register loads of one chunk (16-byte lines spread over NT
// threads), then register -> LDS staging.  Rows at or beyond t_end read row
// t_end - 1 and are staged as zeros.
template <typename T, int D, int M, bool WITH_Q, int NT, int TT> struct PolyLines {
    typedef PolyCfg<T, D, M> C;
    typedef PolyShared<T, D, M, TT, WITH_Q> SM;
    static constexpr int CH = 16 * TT;
    static constexpr int EL = 16 / int(sizeof(T));      // elements per line
    static constexpr int QL = D / EL, VL = C::MB / EL;  // lines per row
    static constexpr int LQ = WITH_Q ? CH * QL : 0, LK = CH * QL, LV = CH * VL;
    static constexpr int L = LQ + LK + LV;
    static constexpr int PER = (L + NT - 1) / NT;
    dwordx4 x[PER];

    __device__ __forceinline__ void load(const T *Q, const T *K, const T *V, int64_t t0, int64_t t_end, int m0,
                                         int tid) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int line = tid + u * NT;
            if (PER * NT > L && line >= L) break;
            const T *p;
            if (line < LQ) {
                const int64_t t = imin64(t0 + line / QL, t_end - 1);
                p = Q + t * D + (line % QL) * EL;
            } else if (line < LQ + LK) {
                const int l = line - LQ;
                const int64_t t = imin64(t0 + l / QL, t_end - 1);
                p = K + t * D + (l % QL) * EL;
            } else {
                const int l = line - LQ - LK;
                const int64_t t = imin64(t0 + l / VL, t_end - 1);
                p = V + t * M + m0 + (l % VL) * EL;
            }
            x[u] = *reinterpret_cast<const dwordx4 *>(p);
        }
    }

    __device__ __forceinline__ void stage(SM &sm, int buf, int64_t t0, int64_t t_end, int tid) const {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int line = tid + u * NT;
            if (PER * NT > L && line >= L) break;
            dwordx4 y = x[u];
            if (line < LQ) {
                const int row = line / QL, col = (line % QL) * EL;
                if (t0 + row >= t_end) y = dwordx4{0u, 0u, 0u, 0u};
                float *dst = &sm.q[buf][row * SM::QS + col];
                if constexpr (sizeof(T) == 2) {
                    f32x4 a, b;
#pragma unroll
                    for (int w = 0; w < 2; ++w) {
                        a[2 * w] = __builtin_bit_cast(float, y[w] << 16);
                        a[2 * w + 1] = __builtin_bit_cast(float, y[w] & 0xffff0000u);
                        b[2 * w] = __builtin_bit_cast(float, y[2 + w] << 16);
                        b[2 * w + 1] = __builtin_bit_cast(float, y[2 + w] & 0xffff0000u);
                    }
                    *reinterpret_cast<f32x4 *>(dst) = a;
                    *reinterpret_cast<f32x4 *>(dst + 4) = b;
                } else {
                    *reinterpret_cast<dwordx4 *>(dst) = y;
                }
            } else if (line < LQ + LK) {
                const int l = line - LQ, row = l / QL, col = (l % QL) * EL;
                if (t0 + row >= t_end) y = dwordx4{0u, 0u, 0u, 0u};
                *reinterpret_cast<dwordx4 *>(&sm.k[buf][row * SM::KS + col]) = y;
                float *kt = &sm.kt[buf][col * SM::KTS + row];
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        kt[(2 * w) * SM::KTS] = __builtin_bit_cast(float, y[w] << 16);
                        kt[(2 * w + 1) * SM::KTS] = __builtin_bit_cast(float, y[w] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int w = 0; w < 4; ++w) {
                        const unsigned int e = y[w];   // (a bit cast of the vector element itself reads element 0)
                        kt[w * SM::KTS] = __builtin_bit_cast(float, e);
                    }
                }
            } else {
                const int l = line - LQ - LK, row = l / VL, col = (l % VL) * EL;
                if (t0 + row >= t_end) y = dwordx4{0u, 0u, 0u, 0u};
                *reinterpret_cast<dwordx4 *>(&sm.v[buf][row * SM::VS + col]) = y;
            }
        }
    }
};

// Token-contiguous fragment of a staged tile: lane (c, g) gets
// x[16 tt + 4g + r][col0 + c], r = 0..3 (bf16: the transposing LDS read).
template <int S> __device__ __forceinline__ bf16x4 tok_frag(const bf16 *stage, int tt, int col0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<lds_i16x4 *>((lds_bf16 *)(stage) + (16 * tt + 4 * g + (c >> 2)) * S + col0 + 4 * (c & 3)));
    return __builtin_bit_cast(bf16x4, r);
}
template <int S> __device__ __forceinline__ f32x4 tok_frag(const float *stage, int tt, int col0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const float *p = stage + (16 * tt + 4 * g) * S + col0 + c;
    return f32x4{p[0], p[S], p[2 * S], p[3 * S]};
}
// Natural fragment: lane (c, g) gets x[16 tt + c][col0 + 4g + r].
template <int S, typename T>
__device__ __forceinline__ typename IO<T>::vec4 nat_frag(const T *stage, int tt, int col0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    return *reinterpret_cast<const typename IO<T>::vec4 *>(stage + (16 * tt + c) * S + col0 + 4 * g);
}

// Rotated q of token tile tt: qr[x + 16 i] = q[16 tt + c][16 i + (4g + x) % 16].
template <int D, int QS, unsigned MASK = ~0u>
__device__ __forceinline__ void load_qr(float (&qr)[D], const float *sq, int tt) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int x0 = 0; x0 < 16; x0 += 4) {
            if (!((MASK >> (4 * i + x0 / 4)) & 1u)) continue;   // never read by this wavefront
            const f32x4 y =
                *reinterpret_cast<const f32x4 *>(sq + (16 * tt + c) * QS + 16 * i + 4 * ((g + x0 / 4) & 3));
#pragma unroll
            for (int e = 0; e < 4; ++e) qr[16 * i + x0 + e] = y[e];
        }
}

template <typename T> __device__ __forceinline__ f32x4 unpack(typename IO<T>::vec4 x) { return IO<T>::to_f32(x); }

// q of token c, dimensions 16 x + 4g .. + 3, from the rotated copy.
template <typename T, int D> __device__ __forceinline__ typename IO<T>::frag q_frag(const float (&qr)[D], int x) {
    return IO<T>::to_frag(f32x4{qr[16 * x], qr[16 * x + 1], qr[16 * x + 2], qr[16 * x + 3]});
}

// ---- per-wavefront state ----------------------------------------------------
template <typename T, int D, int M, int WI, int PASS> struct PolyWave {
    typedef PolyCfg<T, D, M> C;
    typedef typename IO<T>::frag Fr;
    static constexpr int NL = C::NL, MT = C::MT;
    static constexpr int F0 = C::split(WI, PASS), F1 = C::split(WI + 1, PASS), NF = F1 - F0;
    static constexpr int Z0 = C::zsplit(WI, PASS), Z1 = C::zsplit(WI + 1, PASS), NZW = Z1 - Z0;
    static_assert(NF >= 1, "feature tiles per wavefront");
    static_assert(NZW <= 2 && (NZW == 0 || (Z1 - 1) / NL == Z0 / NL), "Z tiles of a wavefront share a row block");

    f32x4 S[NF][MT];
    f32x4 Zt[NZW > 0 ? NZW : 1];

    __device__ __forceinline__ void load_state(const float *rec, int mb) {
        const int l = lane_id();
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                S[f][mt] = rec ? reinterpret_cast<const f32x4 *>(
                                     rec + int64_t((F0 + f) * C::MTOT + mb * MT + mt) * 256)[l]
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int z = 0; z < NZW; ++z)
            Zt[z] = rec ? reinterpret_cast<const f32x4 *>(rec + int64_t(C::FT * C::MTOT + Z0 + z) * 256)[l]
                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ __forceinline__ void store_state(float *rec, int mb) const {
        const int l = lane_id();
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                reinterpret_cast<f32x4 *>(rec + int64_t((F0 + f) * C::MTOT + mb * MT + mt) * 256)[l] = S[f][mt];
        if (mb == 0) {
#pragma unroll
            for (int z = 0; z < NZW; ++z)
                reinterpret_cast<f32x4 *>(rec + int64_t(C::FT * C::MTOT + Z0 + z) * 256)[l] = Zt[z];
        }
    }

    // The chunk's K as token-contiguous fragments (T for the Z products, fp32
    // for the feature products).
    template <int TT, typename SM>
    __device__ __forceinline__ void read_k(const SM &sm, int buf, Fr (&kt)[TT][NL], f32x4 (&own)[TT][NL]) const {
        const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                own[tt][i] = *reinterpret_cast<const f32x4 *>(&sm.kt[buf][(16 * i + c) * SM::KTS + 16 * tt + 4 * g]);
                if constexpr (NZW > 0) kt[tt][i] = tok_frag<SM::KS>(sm.k[buf], tt, 16 * i);
            }
    }
    // V of this workgroup's columns, token-contiguous.
    template <int TT, typename SM>
    __device__ __forceinline__ void read_v(const SM &sm, int buf, Fr (&vf)[TT][MT]) const {
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) vf[tt][mt] = tok_frag<SM::VS>(sm.v[buf], tt, 16 * mt);
    }

    // S_f += phi(K)_f^T V over the chunk, Z += K^T K on this wavefront's tiles.
    template <int TT>
    __device__ __forceinline__ void update(const Fr (&kt)[TT][NL], const f32x4 (&own)[TT][NL],
                                           const Fr (&vf)[TT][MT]) {
        const bool lo = (lane_id() & 15) < 8;
        update_tiles<0, TT>(own, vf, lo);
#pragma unroll
        for (int z = 0; z < NZW; ++z) {
            const int x = (Z0 + z) % NL, y = (Z0 + z) / NL;
#pragma unroll
            for (int tt = 0; tt < TT; tt += 2) mma2(Zt[z], kt[tt][x], kt[tt + 1][x], kt[tt][y], kt[tt + 1][y]);
        }
    }
    template <int f, int TT>
    __device__ __forceinline__ void update_tiles(const f32x4 (&own)[TT][NL], const Fr (&vf)[TT][MT], bool lo) {
        if constexpr (f < NF) {
            Fr a[TT];
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) a[tt] = IO<T>::to_frag(phi_k<NL, F0 + f>(own[tt], lo));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int tt = 0; tt < TT; tt += 2) mma2(S[f][mt], a[tt], a[tt + 1], vf[tt][mt], vf[tt + 1][mt]);
            update_tiles<f + 1, TT>(own, vf, lo);
        }
    }

    // The same update read straight from a staged chunk of TT token tiles,
    // two token tiles at a time (fewer registers for long chunks).
    template <int TT, typename SM> __device__ __forceinline__ void update_lds(const SM &sm, int buf) {
        const bool lo = (lane_id() & 15) < 8;
        const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
        for (int tp = 0; tp < TT; tp += 2) {
            f32x4 own[2][NL];
            Fr kt[2][NL], vf[2][MT];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
#pragma unroll
                for (int i = 0; i < NL; ++i) {
                    own[u][i] = *reinterpret_cast<const f32x4 *>(
                        &sm.kt[buf][(16 * i + c) * SM::KTS + 16 * (tp + u) + 4 * g]);
                    if constexpr (NZW > 0) kt[u][i] = tok_frag<SM::KS>(sm.k[buf], tp + u, 16 * i);
                }
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) vf[u][mt] = tok_frag<SM::VS>(sm.v[buf], tp + u, 16 * mt);
            }
            update_tiles<0, 2>(own, vf, lo);
#pragma unroll
            for (int z = 0; z < NZW; ++z) {
                const int x = (Z0 + z) % NL, y = (Z0 + z) / NL;
                mma2(Zt[z], kt[0][x], kt[1][x], kt[0][y], kt[1][y]);
            }
        }
    }

    // The state as bf16 fragments (rows = output columns, contraction = features).
    __device__ __forceinline__ void state_frags(Fr (&sb)[NF][MT]) const {
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) sb[f][mt] = IO<T>::to_frag(S[f][mt]);
    }

    // Readout of token tile tt from the prefix state: acc[mt][tt] +=
    // S_f^T phi(Q)_f^T over this wavefront's tiles (state fragments from sb,
    // or converted here when sb is not kept).
    template <int f, bool CACHE, int TT>
    __device__ __forceinline__ void readout_tt(f32x4 (&acc)[MT][TT], const Fr (&sb)[NF][MT], const float (&qr)[D],
                                               int tt, bool glo) const {
        if constexpr (f < NF) {
            constexpr bool pair = f + 1 < NF;
            const Fr pa = IO<T>::to_frag(phi_q<NL, F0 + f>(qr, glo));
            Fr pb;
            if constexpr (pair) pb = IO<T>::to_frag(phi_q<NL, F0 + f + 1>(qr, glo));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const Fr sa = CACHE ? sb[f][mt] : IO<T>::to_frag(S[f][mt]);
                if constexpr (pair) {
                    const Fr sc = CACHE ? sb[f + 1][mt] : IO<T>::to_frag(S[f + 1][mt]);
                    mma2(acc[mt][tt], sa, sc, pa, pb);
                } else {
                    mma1(acc[mt][tt], sa, pa);
                }
            }
            readout_tt<pair ? f + 2 : f + 1, CACHE, TT>(acc, sb, qr, tt, glo);
        }
    }

    // Partial q^T Z q per lane (this wavefront's Z tiles and the lane's 4
    // rows of them; the owners add the four lanes of a column).
    __device__ __forceinline__ float den_part(const float (&qr)[D]) const {
        if constexpr (NZW == 0) return 0.f;
        constexpr int y = Z0 / NL;
        f32x4 u = {0.f, 0.f, 0.f, 0.f};
        if constexpr (NZW == 2)
            mma2(u, IO<T>::to_frag(Zt[0]), IO<T>::to_frag(Zt[1]), q_frag<T, D>(qr, Z0 % NL),
                 q_frag<T, D>(qr, (Z0 + 1) % NL));
        else
            mma1(u, IO<T>::to_frag(Zt[0]), q_frag<T, D>(qr, Z0 % NL));
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) s += u[r] * qr[16 * y + r];
        return s;
    }
};

// Intra-chunk part for query tile qt: P^T[key][query] = (k . q)^2 for key
// tiles kt <= qt (masked to key <= query on the diagonal tile), as fragments
// (rows queries, contraction keys), and the lane's partial denominator (its 4
// keys of each tile).
template <typename T, int D, int TT, typename SM>
__device__ __forceinline__ float intra_p(typename IO<T>::frag (&pf)[TT], const SM &sm, int buf, const float (&qr)[D],
                                         int qt) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    float den = 0.f;
#pragma unroll
    for (int kt = 0; kt < TT; ++kt) {
        if (kt > qt) break;
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int x = 0; x < D / 16; x += 2)
            mma2(p, IO<T>::to_frag(unpack<T>(nat_frag<SM::KS>(sm.k[buf], kt, 16 * x))),
                 IO<T>::to_frag(unpack<T>(nat_frag<SM::KS>(sm.k[buf], kt, 16 * x + 16))), q_frag<T, D>(qr, x),
                 q_frag<T, D>(qr, x + 1));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = (kt < qt || 4 * g + r <= c) ? p[r] * p[r] : 0.f;
            den += p[r];
        }
        pf[kt] = IO<T>::to_frag(p);
    }
    return den;
}

// ---- chunk loading ------------------------------------------------------------
// The producer wavefront: chunk j is loaded into register slot j % PF, PF
// chunks ahead, and staged into LDS buffer j % 2 just before the barrier that
// ends the consumers' work on chunk j - 1.  One barrier per chunk, like the
// consumers.
template <typename T, int D, int M, bool WITH_Q, int TT, int PF>
__device__ __forceinline__ void produce_chunks(const T *Q, const T *K, const T *V, int64_t t_begin, int64_t t_end,
                                               int m0, PolyShared<T, D, M, TT, WITH_Q> &sm) {
    constexpr int CH = 16 * TT;
    const int lane = threadIdx.x & 63;   // (the lane-id builtin here crashes this compiler)
    const int64_t nch = (t_end - t_begin + CH - 1) / CH;
    PolyLines<T, D, M, WITH_Q, 64, TT> ld[PF];
#pragma unroll
    for (int p = 0; p < PF; ++p)
        if (p < nch) ld[p].load(Q, K, V, t_begin + p * CH, t_end, m0, lane);
    ld[0].stage(sm, 0, t_begin, t_end, lane);
    if (PF < nch) ld[0].load(Q, K, V, t_begin + PF * CH, t_end, m0, lane);
    __syncthreads();
    for (int64_t c0 = 0; c0 < nch; c0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int64_t c = c0 + u;
            if (c >= nch) break;
            if (c + 1 < nch) {
                ld[(u + 1) % PF].stage(sm, int((c + 1) & 1), t_begin + (c + 1) * CH, t_end, lane);
                if (c + 1 + PF < nch) ld[(u + 1) % PF].load(Q, K, V, t_begin + (c + 1 + PF) * CH, t_end, m0, lane);
            }
            __syncthreads();
        }
    }
}

// ---- kernels ------------------------------------------------------------------
// Calls f(std::integral_constant<int, w>) for the wavefront index w < N (each
// wavefront runs the code of its own feature tiles).
template <int N, int I = 0, typename F> __device__ __forceinline__ void poly_dispatch(int w, F &&f) {
    if constexpr (I < N) {
        if (w == I)
            f(std::integral_constant<int, I>());
        else
            poly_dispatch<N, I + 1>(w, f);
    }
}

template <typename T, int D, int M, int WI>
__device__ __forceinline__ void segment_state_wave(const T *K, const T *V, float *rec, int64_t t_begin,
                                                   int64_t t_end, int mb,
                                                   PolyShared<T, D, M, PolyCfg<T, D, M>::TT1, false> &sm) {
    typedef PolyCfg<T, D, M> C;
    constexpr int TT = C::TT1, CH = 16 * TT;
    const int tid = threadIdx.x;
    PolyWave<T, D, M, WI, 1> w;
    w.load_state(nullptr, mb);
    PolyLines<T, D, M, false, 64 * C::W, TT> ld;
    if constexpr (!C::PROD) {
        ld.load(nullptr, K, V, t_begin, t_end, mb * C::MB, tid);
        ld.stage(sm, 0, t_begin, t_end, tid);
    }
    __syncthreads();
    int buf = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += CH, buf ^= 1) {
        const bool more = t0 + CH < t_end;
        if (!C::PROD && more) ld.load(nullptr, K, V, t0 + CH, t_end, mb * C::MB, tid);
        w.template update_lds<TT>(sm, buf);
        if (!C::PROD && more) ld.stage(sm, buf ^ 1, t0 + CH, t_end, tid);
        __syncthreads();
    }
    w.store_state(rec, mb);
}

template <typename T, int D, int M>
__global__ __launch_bounds__((64 * PolyCfg<T, D, M>::NWAVE)) void k_poly_segment_state(const T *__restrict__ k,
                                                                                      const T *__restrict__ v,
                                                                                      float *__restrict__ ws,
                                                                                      int64_t N, int64_t nseg,
                                                                                      int64_t seg_tokens) {
    typedef PolyCfg<T, D, M> C;
    __shared__ PolyShared<T, D, M, C::TT1, false> sm;
    const int mb = blockIdx.x % C::NMB;
    const int64_t seg = (blockIdx.x / C::NMB) % nseg, bh = blockIdx.x / C::NMB / nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    float *rec = ws + (bh * nseg + seg) * C::REC;
    const int wave = threadIdx.x >> 6;
    if (C::PROD && wave == C::W) {
        produce_chunks<T, D, M, false, C::TT1, C::PF1>(nullptr, K, V, t_begin, t_end, mb * C::MB, sm);
        return;
    }
    poly_dispatch<C::W>(wave, [&](auto wi) { segment_state_wave<T, D, M, decltype(wi)::value>(K, V, rec, t_begin, t_end, mb, sm); });
}

// CAUSAL false: the non-causal form, every token read out from the (b, h)
// total in rec, with neither the intra-chunk part nor state updates.  fin:
// where to store the state after the segment's last token (or null).
template <typename T, int D, int M, int WI, bool CAUSAL>
__device__ __forceinline__ void output_wave(const T *Q, const T *K, const T *V, T *O, const float *rec, float *fin,
                                            int64_t t_begin, int64_t t_end, int mb,
                                            PolyShared<T, D, M, PolyCfg<T, D, M>::TT, true> &sm) {
    typedef PolyCfg<T, D, M> C;
    typedef PolyShared<T, D, M, C::TT, true> SM;
    typedef PolyWave<T, D, M, WI, 2> PW;
    typedef typename IO<T>::frag Fr;
    constexpr int MT = C::MT, W = C::W, TT = C::TT, CH = C::CH;
    constexpr PolyOwn OWN = poly_own<TT, MT, W>(WI);
    const int tid = threadIdx.x, lane = lane_id(), c = lane & 15, g = lane >> 4;
    const bool glo = g < 2;
    const int m0 = mb * C::MB;
    PW w;
    w.load_state(rec, mb);
    PolyLines<T, D, M, true, 64 * W, TT> ld;
    if constexpr (!C::PROD) {
        ld.load(Q, K, V, t_begin, t_end, m0, tid);
        ld.stage(sm, 0, t_begin, t_end, tid);
    }
    __syncthreads();
    int buf = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += CH, buf ^= 1) {
        const bool more = t0 + CH < t_end;
        if (!C::PROD && more) ld.load(Q, K, V, t0 + CH, t_end, m0, tid);
        Fr vf[TT][MT];
        w.read_v(sm, buf, vf);

        // 1. readout from the prefix state, the Z part of the denominators,
        //    and the intra-chunk part of the owned output tiles
        f32x4 acc[MT][TT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int tt = 0; tt < TT; ++tt) acc[mt][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float dpart[TT], pden[TT] = {};
        f32x4 intra[OWN.n > 0 ? OWN.n : 1];
#pragma unroll
        for (int u = 0; u < OWN.n; ++u) intra[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        Fr sb[PW::NF][MT];   // filled only when the state fragments are kept
        if constexpr (C::SB_CACHE) w.state_frags(sb);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
            float qr[D];
            load_qr<D, SM::QS, poly_qr_groups<C::NL>(PW::F0, PW::F1)>(qr, sm.q[buf], tt);
            w.template readout_tt<0, C::SB_CACHE, TT>(acc, sb, qr, tt, glo);
            dpart[tt] = w.den_part(qr);
            Fr pf[TT];
            bool have = false;
#pragma unroll
            for (int u = 0; u < OWN.n; ++u) {
                if (!CAUSAL || OWN.tt[u] != tt) continue;
                if (!have) {
                    pden[tt] = intra_p<T, D, TT>(pf, sm, buf, qr, tt);
                    have = true;
                }
                const int mt = OWN.mt[u];
                intra[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kt = 0; kt <= tt; kt += 2) {
                    if (kt + 1 <= tt)
                        mma2(intra[u], vf[kt][mt], vf[kt + 1][mt], pf[kt], pf[kt + 1]);
                    else
                        mma1(intra[u], vf[kt][mt], pf[kt]);
                }
            }
        }

        // 2. state update
        if constexpr (CAUSAL) {
            Fr kt[TT][C::NL];
            f32x4 own[TT][C::NL];
            w.read_k(sm, buf, kt, own);
            w.update(kt, own, vf);
        }

        // 3. post partials for the owners
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                if (poly_owner<TT, MT, W>(tt, mt) != WI) sm.part[buf][tt * MT + mt][WI][lane] = acc[mt][tt];
            sm.den[buf][WI][tt][lane] = dpart[tt];
        }
        if (!C::PROD && more) ld.stage(sm, buf ^ 1, t0 + CH, t_end, tid);
        __syncthreads();

#pragma unroll
        for (int u = 0; u < OWN.n; ++u) {
            const int tt = OWN.tt[u], mt = OWN.mt[u], o = tt * MT + mt;
            f32x4 s = acc[mt][tt];
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2)
                if (w2 != WI) s += sm.part[buf][o][w2][lane];
            const f32x4 num = 2.f * s + intra[u];
            float d = pden[tt];
#pragma unroll
            for (int w2 = 0; w2 < W; ++w2) d += sm.den[buf][w2][tt][lane];
            d += __shfl_xor(d, 16);
            d += __shfl_xor(d, 32);
            const int64_t t = t0 + 16 * tt + c;
            if (t < t_end)
                store4<T>(O + t * M + m0 + 16 * mt + 4 * g, IO<T>::from_f32(num * __builtin_amdgcn_rcpf(d)));
        }
    }
    if (fin) w.store_state(fin, mb);
}

template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__((64 * PolyCfg<T, D, M>::NWAVE)) void k_poly_output(const T *__restrict__ q,
                                                                               const T *__restrict__ k,
                                                                               const T *__restrict__ v,
                                                                               T *__restrict__ out,
                                                                               const float *__restrict__ ws,
                                                                               float *__restrict__ fin, int64_t N,
                                                                               int64_t nseg, int64_t seg_tokens) {
    typedef PolyCfg<T, D, M> C;
    __shared__ PolyShared<T, D, M, C::TT, true> sm;
    const int mb = blockIdx.x % C::NMB;
    const int64_t seg = (blockIdx.x / C::NMB) % nseg, bh = blockIdx.x / C::NMB / nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    T *O = out + bh * N * M;
    // causal: the segment's exclusive prefix (none: zero); non-causal: the
    // (b, h) total, in its first record
    const float *rec = CAUSAL ? (ws ? ws + (bh * nseg + seg) * C::REC : nullptr) : ws + bh * nseg * C::REC;
    float *f = (CAUSAL && fin && seg == nseg - 1) ? fin + bh * C::REC : nullptr;
    const int wave = threadIdx.x >> 6;
    if (C::PROD && wave == C::W) {
        produce_chunks<T, D, M, true, C::TT, C::PF>(Q, K, V, t_begin, t_end, mb * C::MB, sm);
        return;
    }
    poly_dispatch<C::W>(wave, [&](auto wi) {
        output_wave<T, D, M, decltype(wi)::value, CAUSAL>(Q, K, V, O, rec, f, t_begin, t_end, mb, sm);
    });
}

struct PolyPlan {
    int64_t nseg = 1, seg_tokens = 0, rec = 0, nmb = 1;
    size_t ws_bytes = 256;
};

// Enough (segment, column block) workgroups to give every CU one: a
// workgroup fills a CU (its wavefronts hold the state in registers).
// Segments are whole chunks of the kernels' chunk length.  The causal form
// needs records only with several segments; the non-causal one always keeps
// the (b, h) total.
inline PolyPlan make_poly_plan(int64_t BH, int64_t N, int64_t D, int64_t M, int cus, bool causal) {
    PolyPlan p;
    const int64_t NL = D / 16, FT = NL * (NL + 1) / 2 + 15 * NL * NL / 2;
    const int64_t chunk = 128;   // a multiple of both kernels' chunk lengths
    p.nmb = D == 32 ? 1 : M / 16;
    p.rec = (FT * (M / 16) + NL * NL) * 256;
    const int64_t nch = ceil_div(N, chunk);
    int64_t nseg = ceil_div(cus, BH * p.nmb);
    nseg = std::max<int64_t>(1, std::min<int64_t>({nseg, nch, kMaxSegPerHead}));
    p.seg_tokens = ceil_div(nch, nseg) * chunk;
    p.nseg = ceil_div(N, p.seg_tokens);
    if (p.nseg > 1 || !causal) p.ws_bytes = align256(size_t(BH * p.nseg * p.rec) * sizeof(float));
    return p;
}

template <typename T, int D, int M>
static hipError_t run_poly(bool causal, const void *q, const void *k, const void *v, void *out, float *fin,
                           int64_t BH, int64_t N, float *ws, hipStream_t s) {
    typedef PolyCfg<T, D, M> C;
    const PolyPlan p = make_poly_plan(BH, N, D, M, device_cus(), causal);
    if (p.seg_tokens % C::CH != 0 || p.seg_tokens % (16 * C::TT1) != 0) return hipErrorInvalidValue;
    const dim3 grid(unsigned(BH * p.nseg * C::NMB)), block(64 * C::NWAVE);
    hipError_t e;
    if (p.nseg > 1 || !causal) {
        hipLaunchKernelGGL((k_poly_segment_state<T, D, M>), grid, block, 0, s, (const T *)k, (const T *)v, ws, N,
                           p.nseg, p.seg_tokens);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (p.nseg > 1 && (e = launch_scan(ws, BH, p.nseg, p.rec, causal ? 0 : 1, s)) != hipSuccess) return e;
    }
    if (causal)
        hipLaunchKernelGGL((k_poly_output<T, D, M, true>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, p.nseg > 1 ? (const float *)ws : nullptr, fin, N, p.nseg,
                           p.seg_tokens);
    else
        hipLaunchKernelGGL((k_poly_output<T, D, M, false>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, (const float *)ws, (float *)nullptr, N, p.nseg, p.seg_tokens);
    return hipGetLastError();
}

// ---- decode -------------------------------------------------------------------
// One step for B*H independent streams, one workgroup of four wavefronts per
// stream, the state in the record layout (feature tiles, then the Z tiles;
// each tile 64 lanes x 4 floats in the accumulator order of the kernels
// above):  S_f += phi(k)_f v^T and Z += k k^T, then, read after the update,
//   out = 2 phi'(q) . S / q^T Z q,
// phi' being phi with the diagonal features halved (the count of each
// unordered pair, as in the forwards).  The step reads and writes the state
// once: it is bound by memory bandwidth, plain fp32 FMAs on the VALU.
constexpr int kPolyDecodeWaves = 4;

template <typename T, int D> __device__ __forceinline__ void load_rot(float (&xr)[D], const T *x) {
    const int g = lane_id() >> 4;
#pragma unroll
    for (int i = 0; i < D / 16; ++i)
#pragma unroll
        for (int x0 = 0; x0 < 16; x0 += 4) {
            const f32x4 y = IO<T>::to_f32(load4<T>(x + 16 * i + 4 * ((g + x0 / 4) & 3)));
#pragma unroll
            for (int e = 0; e < 4; ++e) xr[16 * i + x0 + e] = y[e];
        }
}

template <typename T, int D, int M, int F>
__device__ __forceinline__ void decode_tiles(float *st, const float (&kr)[D], const float (&qr)[D],
                                             const float (&vm)[M / 16], float (&num)[M / 16], int wave, bool glo) {
    constexpr int NL = D / 16, FT = poly_tiles<NL>(), MT = M / 16;
    if constexpr (F < FT) {
        if (F % kPolyDecodeWaves == wave) {
            const f32x4 pk = phi_q<NL, F, false>(kr, glo), pq = phi_q<NL, F, true>(qr, glo);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 *p = reinterpret_cast<f32x4 *>(st + int64_t(F * MT + mt) * 256) + lane_id();
                f32x4 x = *p;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    x[r] += pk[r] * vm[mt];
                    num[mt] += pq[r] * x[r];
                }
                *p = x;
            }
        }
        decode_tiles<T, D, M, F + 1>(st, kr, qr, vm, num, wave, glo);
    }
}

template <typename T, int D, int M>
__global__ __launch_bounds__(64 * kPolyDecodeWaves) void k_poly_decode(const T *__restrict__ q,
                                                                       const T *__restrict__ k,
                                                                       const T *__restrict__ v,
                                                                       float *__restrict__ state,
                                                                       T *__restrict__ out) {
    constexpr int NL = D / 16, FT = poly_tiles<NL>(), MT = M / 16, NZ = NL * NL;
    constexpr int64_t REC = int64_t(FT * MT + NZ) * 256;
    const int64_t s = blockIdx.x;
    const int wave = threadIdx.x >> 6, lane = lane_id(), c = lane & 15, g = lane >> 4;
    float *st = state + s * REC;
    const T *qs = q + s * D, *ks = k + s * D;
    float qr[D], kr[D];
    load_rot<T, D>(qr, qs);
    load_rot<T, D>(kr, ks);
    float vm[MT], num[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        vm[mt] = (float)v[s * M + 16 * mt + c];
        num[mt] = 0.f;
    }
    decode_tiles<T, D, M, 0>(st, kr, qr, vm, num, wave, g < 2);

    // Z tiles: lane (c, g) element r of tile (x, y) is Z[16x + 4g + r][16y + c]
    float den = 0.f;
#pragma unroll
    for (int z = 0; z < NZ; ++z) {
        if (z % kPolyDecodeWaves != wave) continue;
        const int x = z % NL, y = z / NL;
        const float ky = (float)ks[16 * y + c], qy = (float)qs[16 * y + c];
        f32x4 *p = reinterpret_cast<f32x4 *>(st + int64_t(FT * MT + z) * 256) + lane;
        f32x4 t = *p;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            t[r] += kr[16 * x + r] * ky;
            den += t[r] * qr[16 * x + r] * qy;
        }
        *p = t;
    }

    // numerators: lanes (c, 0..3) share column c; denominator: every lane
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        num[mt] += __shfl_xor(num[mt], 16);
        num[mt] += __shfl_xor(num[mt], 32);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) den += __shfl_xor(den, off);
    __shared__ float part[kPolyDecodeWaves][M + 1];
    if (g == 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) part[wave][16 * mt + c] = num[mt];
    }
    if (lane == 0) part[wave][M] = den;
    __syncthreads();
    if (wave == 0 && lane < M) {
        float n = 0.f, d = 0.f;
#pragma unroll
        for (int w = 0; w < kPolyDecodeWaves; ++w) {
            n += part[w][lane];
            d += part[w][M];
        }
        out[s * M + lane] = (T)(2.f * n * __builtin_amdgcn_rcpf(d));
    }
}

template <typename T, int D>
static hipError_t run_poly_m(bool causal, const void *q, const void *k, const void *v, void *out, float *fin,
                             int64_t BH, int64_t N, int64_t M, float *ws, hipStream_t s) {
    if (M == 32) return run_poly<T, D, 32>(causal, q, k, v, out, fin, BH, N, ws, s);
    if (M == 64) return run_poly<T, D, 64>(causal, q, k, v, out, fin, BH, N, ws, s);
    return hipErrorInvalidValue;
}

template <typename T, int D, int M>
static hipError_t decode_poly(const void *q, const void *k, const void *v, float *state, void *out, int64_t BH,
                              hipStream_t s) {
    hipLaunchKernelGGL((k_poly_decode<T, D, M>), dim3(unsigned(BH)), dim3(64 * kPolyDecodeWaves), 0, s,
                       (const T *)q, (const T *)k, (const T *)v, state, (T *)out);
    return hipGetLastError();
}

template <typename T>
static hipError_t decode_poly_dm(const void *q, const void *k, const void *v, float *state, void *out, int64_t BH,
                                 int64_t D, int64_t M, hipStream_t s) {
    if (D == 32) return M == 32 ? decode_poly<T, 32, 32>(q, k, v, state, out, BH, s)
                                : decode_poly<T, 32, 64>(q, k, v, state, out, BH, s);
    return M == 32 ? decode_poly<T, 64, 32>(q, k, v, state, out, BH, s)
                   : decode_poly<T, 64, 64>(q, k, v, state, out, BH, s);
}

} // namespace

bool poly_head_sizes(int64_t D, int64_t M) { return (D == 32 || D == 64) && (M == 32 || M == 64); }

int64_t poly_state_floats(int64_t D, int64_t M) {
    if (!poly_head_sizes(D, M)) return 0;
    const int64_t NL = D / 16, FT = NL * (NL + 1) / 2 + 15 * NL * NL / 2;
    return (FT * (M / 16) + NL * NL) * 256;
}

size_t poly_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M, bool causal) {
    return make_poly_plan(BH, N, D, M, device_cus(), causal).ws_bytes;
}

hipError_t launch_poly_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out,
                               float *state_final, int64_t BH, int64_t N, int64_t D, int64_t M, float *ws,
                               hipStream_t s) {
    if (!poly_head_sizes(D, M)) return hipErrorInvalidValue;
    if (dt == 0)
        return D == 32 ? run_poly_m<float, 32>(causal, q, k, v, out, state_final, BH, N, M, ws, s)
                       : run_poly_m<float, 64>(causal, q, k, v, out, state_final, BH, N, M, ws, s);
    return D == 32 ? run_poly_m<bf16, 32>(causal, q, k, v, out, state_final, BH, N, M, ws, s)
                   : run_poly_m<bf16, 64>(causal, q, k, v, out, state_final, BH, N, M, ws, s);
}

hipError_t launch_poly_decode(int dt, const void *q, const void *k, const void *v, float *state, void *out,
                              int64_t BH, int64_t D, int64_t M, hipStream_t s) {
    if (!poly_head_sizes(D, M)) return hipErrorInvalidValue;
    if (dt == 0) return decode_poly_dm<float>(q, k, v, state, out, BH, D, M, s);
    return decode_poly_dm<bf16>(q, k, v, state, out, BH, D, M, s);
}

} // namespace la
