// la_generic.hip -- causal and non-causal forward for every head size D, M in
// {16, 32, ..., 128} (the fused kernels of la_forward.hip take D, M in
// {32, 64}).
//
// Method: as la_forward.hip ([deck] = zhengyuhong.cn "Transformers are RNNs
// ... 解读", slides 3-4; [summary] = paperlayer.ai summary, 3.2-3.3.2):
//   out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i, S_i = sum_{j<=i} phi(K_j) V_j^T,
//   Z_i = sum_{j<=i} phi(K_j) (non-causal: sums over all tokens),
// in 16-token chunks with an exact intra-chunk term, fp32 state.
//
// Output columns are independent given the feature maps, so the work is cut
// by 16-column groups of V (and out): one wavefront owns a (segment, column
// group) pair and carries only its D x 16 slice of S plus the normalizer
// block (2 D / 16 accumulator tiles, 32 fp32 registers per 16 rows of D),
// which fits every D up to 128.  The chunk's Q and K rows are loaded by the
// segment's wavefronts together, mapped through phi once and staged in LDS,
// from which every wavefront reads the operands of its chunk's D-deep
// products (fp32 rows as split bf16 parts for the bf16 matrix instruction).
// Three launches: per-segment sums of
// phi(K) [V, 1]^T into row-major records (each wavefront its columns), the
// scan of la_forward.hip over segments (with the optional start state and
// final state), then the outputs.
//
// The backward for the same head sizes (the two-state kernels of
// la_backward.hip take D, M in {32, 64}) splits the same way: a workgroup
// walks one segment with one wavefront per 16-column group of V and dout.
// With g_i = dout_i / d_i, h_i = -(dout_i . out_i) / d_i ([summary] 3.3.1
// and appendix A, denominator terms written out as in la_backward.hip),
//   dL/dphi(q_i) = sum_{j<=i} (g_i . v_j + h_i) phi(k_j) = S_i g_i + Z_i h_i,
//   dL/dphi(k_j) = sum_{i>=j} (g_i . v_j + h_i) phi(q_i) = R_j v_j + u_j,
//   dV_j         = sum_{i>=j} (phi(q_i) . phi(k_j)) g_i  = R_j^T phi(k_j),
// every term is a sum over column groups (S_i g_i over the groups' columns
// of S and g, R_j v_j likewise) plus the h part, which the first group
// adds; dV is per group.  So each wavefront carries the D x 16 slices of S
// (with Z) and of R (with u on the first group), and the only values that
// need all groups -- dout . out for h, and the dQ and dK sums -- are added
// through LDS in group order, a fixed order, so results do not vary from run
// to run.  Launches: the per-segment sums above and the scan (forward
// states), the dQ pass (also 1/d and h per token and the segment's reverse
// sums), the scan in reverse, the dK/dV pass.
#include <type_traits>

#include "la_chunk.h"
#include "la_internal.h"
#include "la_split.h"

namespace la {

namespace {

constexpr int GCH = 16;   // tokens per chunk
// 16 rows x 16 columns [col0, col0 + 16) of a row-major [.][ld] tensor as a
// natural fragment: lane (c, g) holds row t0 + c, columns col0 + 4g .. + 3.
// Rows at or beyond t_end read row t_end - 1.
template <typename T>
__device__ __forceinline__ typename IO<T>::vec4 load_col_tile(const T *__restrict__ base, int64_t ld, int64_t col0,
                                                              int64_t t0, int64_t t_end) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const int64_t t = imin64(t0 + c, t_end - 1);
    return load4<T>(base + t * ld + col0 + 4 * g);
}

// ---- the chunk's Q and K rows shared by the column groups -----------------------
// The wavefronts of a workgroup (one per 16-column group) all need phi of
// the same 16 rows of Q and K.  They load those rows together, as 16-byte
// pieces of whole rows (piece p = 64 (w + ng i) + lane of the 16 F sizeof(T)
// / 16 pieces of 16 rows of F features), apply phi once per element, and
// stage them in one LDS area that every wavefront reads its fragments from;
// the feature map is not repeated per group.  bf16 rows are staged as they
// are; fp32 rows as two bf16 areas, the hi and lo parts of each value (the
// split operands of la_device.h), so the products run on the bf16 matrix
// instruction as in the fused fp32 forward.
template <typename T> constexpr int coop_pieces(int F) { return F * int(sizeof(T)); }   // per 16 rows
template <typename T, int F> constexpr int coop_np() { return (coop_pieces<T>(F) + 63) / 64; }
// CoopFrag<T>: the operand fragment of staged rows (bf16x4, or split4 for fp32).
template <typename T> using CoopFrag = typename std::conditional<sizeof(T) == 4, split4, bf16x4>::type;
// NPW: the most pieces one lane moves, coop_np<T, F>() when one wavefront
// does all; the host passes fewer when the workgroup's w wavefronts cover the
// pieces with that many each (64 w NPW >= the piece count), which saves
// registers.
template <int F, int NPW> struct CoopRows {
    static constexpr int NP = NPW;
    dwordx4 x[NP];
};
template <typename T, int F, int NPW>
__device__ __forceinline__ void coop_load(CoopRows<F, NPW> &r, const T *__restrict__ base, int64_t t0,
                                          int64_t t_end, int w, int ng) {
    constexpr int EPP = 16 / int(sizeof(T));   // elements per piece
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int p = 64 * (w + ng * i) + l;
        if (p < coop_pieces<T>(F)) {
            const int e = EPP * p, row = e / F, col = e % F;
            const int64_t t = imin64(t0 + row, t_end - 1);   // rows past the end read the last row
            r.x[i] = *reinterpret_cast<const dwordx4 *>(base + t * F + col);
        }
    }
}
// LDS elements of one staged chunk: rows of F + kStagePad elements, twice
// for fp32 (hi area, then lo area).
template <int F> constexpr int coop_rows_elems() { return 16 * (F + kStagePad); }
template <typename T, int F> constexpr int coop_stage_elems() { return (sizeof(T) == 4 ? 2 : 1) * coop_rows_elems<F>(); }
// PHI applies the feature map, MASK zeroes rows at or beyond t_end.
template <typename T, int F, bool PHI, bool MASK, int NPW>
__device__ __forceinline__ void coop_stage(lds_bf16 *stage, const CoopRows<F, NPW> &r, int64_t t0, int64_t t_end,
                                           int w, int ng) {
    constexpr int EPP = 16 / int(sizeof(T));
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < NPW; ++i) {
        const int p = 64 * (w + ng * i) + l;
        if (p < coop_pieces<T>(F)) {
            const int e = EPP * p, row = e / F, col = e % F;
            const bool zero = MASK && t0 + row >= t_end;
            if constexpr (sizeof(T) == 2) {
                dwordx4 y = r.x[i];
                if (PHI) y = phi8(y);
                if (zero) y = dwordx4{0u, 0u, 0u, 0u};
                *reinterpret_cast<lds_dwordx4 *>(stage + row * (F + kStagePad) + col) = y;
            } else {
                f32x4 y = __builtin_bit_cast(f32x4, r.x[i]);
                if (PHI) y = phi4(y);
                if (zero) y = f32x4{0.f, 0.f, 0.f, 0.f};
                const split4 sp = split_f32(y);
                *reinterpret_cast<lds_bf16x4 *>(stage + row * (F + kStagePad) + col) = split_hi(sp);
                *reinterpret_cast<lds_bf16x4 *>(stage + coop_rows_elems<F>() + row * (F + kStagePad) + col) =
                    split_lo(sp);
            }
        }
    }
}
// Natural and token-contiguous fragments of staged rows.
template <int F>
__device__ __forceinline__ void coop_natural(bf16x4 (&y)[1][F / 16], const lds_bf16 *stage) {
    natural_frags_lds<F, 1>(y, stage);
}
template <int F>
__device__ __forceinline__ void coop_natural(split4 (&y)[1][F / 16], const lds_bf16 *stage) {
    bf16x4 h[1][F / 16], l[1][F / 16];
    natural_frags_lds<F, 1>(h, stage);
    natural_frags_lds<F, 1>(l, stage + coop_rows_elems<F>());
#pragma unroll
    for (int f = 0; f < F / 16; ++f) y[0][f] = split_join(h[0][f], l[0][f]);
}
template <int F>
__device__ __forceinline__ void coop_transposed(bf16x4 (&y)[1][F / 16], const lds_bf16 *stage) {
    transposed_frags_lds<F, 1>(y, stage);
}
template <int F>
__device__ __forceinline__ void coop_transposed(split4 (&y)[1][F / 16], const lds_bf16 *stage) {
    bf16x4 h[1][F / 16], l[1][F / 16];
    transposed_frags_lds<F, 1>(h, stage);
    transposed_frags_lds<F, 1>(l, stage + coop_rows_elems<F>());
#pragma unroll
    for (int f = 0; f < F / 16; ++f) y[0][f] = split_join(h[0][f], l[0][f]);
}

// phi'(x) = min(phi(x), 1) of tile ft of rows staged by coop_stage<F, true, .>
// (phi(x) <= 1 exactly where x <= 0, where phi' = phi = exp(x)), in the
// natural layout: lane (c, g) gets row c, features 16 ft + 4g .. + 3.  Read at
// the point of use, so no wavefront holds phi' of every tile through a chunk.
template <int F>
__device__ __forceinline__ f32x4 dphi_staged(const lds_bf16 *stage, int ft) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const f32x4 ph = IO<bf16>::to_f32(*reinterpret_cast<const lds_bf16x4 *>(stage + c * (F + kStagePad) + 16 * ft + 4 * g));
    return f32x4{__builtin_fminf(ph[0], 1.f), __builtin_fminf(ph[1], 1.f), __builtin_fminf(ph[2], 1.f),
                 __builtin_fminf(ph[3], 1.f)};
}

}  // namespace

// ---- per-segment sums ---------------------------------------------------------
// Record of segment `seg` (row-major S [D][M], then Z [D]): wavefront cg of the
// segment's workgroup writes columns [16 cg, 16 cg + 16) of S, wavefront 0 Z.
// The chunk's K rows arrive as whole 16-byte pieces loaded by all the
// segment's wavefronts together (see coop_load), phi is applied once per
// element, and the staging is double buffered: the wavefronts stage chunk c
// into buffer c % 2, meet at one barrier, and read their fragments from it, so
// a wavefront that stages chunk c + 2 has passed the barrier of chunk c + 1,
// which every wavefront reaches only after its reads of chunk c.
template <typename T, int DT, bool PHI, int NPW, bool HELP>
__global__ __launch_bounds__(512) void k_gen_segstate_coop(const T *__restrict__ k, const T *__restrict__ v,
                                                           float *__restrict__ ws, int64_t N, int64_t M, int64_t nseg,
                                                           int64_t seg_tokens) {
    constexpr int D = 16 * DT;
    typedef CoopFrag<T> Fr;
    __shared__ __align__(16) bf16 shk[2][coop_stage_elems<T, D>()];
    __shared__ __align__(16) bf16 sv_mem[8][transpose_stage_elems<Fr, 1, 1>()];
    const int ng = int(M / 16), nw = int(blockDim.x >> 6);   // column groups; wavefronts (nw >= ng)
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // HELP: wavefronts past the column groups only load and stage rows
    const bool active = !HELP || cg < ng;
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    lds_bf16 *sv = (lds_bf16 *)sv_mem[cg];

    f32x4 St[DT][2];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) St[dt][0] = St[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // chunks loaded two ahead of the one being summed; chunk parity b picks
    // the register set and the LDS buffer
    CoopRows<D, NPW> rk[2];
    typename IO<T>::vec4 rv[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        coop_load<T, D>(rk[b], K, t_begin + b * GCH, t_end, cg, nw);
        if (active) rv[b] = load_col_tile<T>(V, M, 16 * cg, t_begin + b * GCH, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += 2 * GCH) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int64_t t0 = t00 + b * GCH;
            if (t0 >= t_end) break;   // uniform over the workgroup
            lds_bf16 *sk = (lds_bf16 *)shk[b];
            coop_stage<T, D, PHI, true>(sk, rk[b], t0, t_end, cg, nw);   // rows past t_end are zero
            Fr Vn[1][1];
            if (active) {
                const typename IO<T>::vec4 one[1][1] = {{rv[b]}};
                raw_frags<T, 16, 1>(Vn, one, t0, t_end);
            }
            coop_load<T, D>(rk[b], K, t0 + 2 * GCH, t_end, cg, nw);
            if (active) rv[b] = load_col_tile<T>(V, M, 16 * cg, t0 + 2 * GCH, t_end);
            lds_barrier();
            if (active) {
                Fr KT[1][DT], VT[1][1];
                coop_transposed<D>(KT, sk);
                transpose_frags<1, 1>(VT, Vn, sv);
                state_accumulate<Fr, D, 16, 1, false>(St, KT, VT);
            }
        }
    }
    if (!active) return;
    float *rec = ws + (bh * nseg + seg) * (int64_t(D) * M + D);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) rec[(16 * dt + 4 * g + r) * M + 16 * cg + c] = St[dt][0][r];
        if (cg == 0 && c == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[int64_t(D) * M + 16 * dt + 4 * g + r] = St[dt][1][r];
        }
    }
}

// ---- outputs --------------------------------------------------------------------
// Wavefront cg walks the segment's chunks from the state of everything before
// it (causal: the segment's exclusive prefix; non-causal: the total in record
// 0), writing columns [16 cg, 16 cg + 16) of out; Q and K rows staged as in
// the segment sums.  No row masks (as in the fused forward's output pass):
// rows past the end are copies of the last valid row, their outputs are not
// stored, the causal mask keeps them out of every stored output, and the state
// is not used after the last chunk.
template <typename T, int DT, bool CAUSAL, bool PHI, int NPW, bool HELP>
__global__ __launch_bounds__(512) void k_gen_output_coop(const T *__restrict__ q, const T *__restrict__ k,
                                                         const T *__restrict__ v, T *__restrict__ out,
                                                         const float *__restrict__ ws, int64_t N, int64_t M,
                                                         int64_t nseg, int64_t seg_tokens) {
    constexpr int D = 16 * DT;
    typedef CoopFrag<T> Fr;
    __shared__ __align__(16) bf16 shq[2][coop_stage_elems<T, D>()];
    __shared__ __align__(16) bf16 shk[CAUSAL ? 2 : 1][CAUSAL ? coop_stage_elems<T, D>() : 8];
    __shared__ __align__(16) bf16 sv_mem[8][transpose_stage_elems<Fr, 1, 1>()];
    const int ng = int(M / 16), nw = int(blockDim.x >> 6);   // column groups; wavefronts (nw >= ng)
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // HELP: wavefronts past the column groups only load and stage rows
    const bool active = !HELP || cg < ng;
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    T *O = out + bh * N * M;
    lds_bf16 *sv = (lds_bf16 *)sv_mem[cg];

    f32x4 St[DT][2];
    if (active) {
        const float *rec = ws + (bh * nseg + (CAUSAL ? seg : 0)) * (int64_t(D) * M + D);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                St[dt][0][r] = rec[(16 * dt + 4 * g + r) * M + 16 * cg + c];
                St[dt][1][r] = rec[int64_t(D) * M + 16 * dt + 4 * g + r];
            }
    }
    const Fr ones = frag_ones<Fr>();

    // chunks loaded two ahead of the one being computed; chunk parity b
    // picks the register set and the LDS buffer
    CoopRows<D, NPW> rq[2], rk[2];
    typename IO<T>::vec4 rv[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        coop_load<T, D>(rq[b], Q, t_begin + b * GCH, t_end, cg, nw);
        if (CAUSAL) {
            coop_load<T, D>(rk[b], K, t_begin + b * GCH, t_end, cg, nw);
            if (active) rv[b] = load_col_tile<T>(V, M, 16 * cg, t_begin + b * GCH, t_end);
        }
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += 2 * GCH) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int64_t t0 = t00 + b * GCH;
        if (t0 >= t_end) break;   // uniform over the workgroup
        lds_bf16 *sq = (lds_bf16 *)shq[b];
        lds_bf16 *sk = (lds_bf16 *)shk[CAUSAL ? b : 0];
        coop_stage<T, D, PHI, false>(sq, rq[b], t0, t_end, cg, nw);
        Fr Vn[1][1];
        if (CAUSAL) {
            coop_stage<T, D, PHI, false>(sk, rk[b], t0, t_end, cg, nw);
            if (active) value_frags_unmasked(Vn[0][0], rv[b]);
        }
        coop_load<T, D>(rq[b], Q, t0 + 2 * GCH, t_end, cg, nw);
        if (CAUSAL) {
            coop_load<T, D>(rk[b], K, t0 + 2 * GCH, t_end, cg, nw);
            if (active) rv[b] = load_col_tile<T>(V, M, 16 * cg, t0 + 2 * GCH, t_end);
        }
        lds_barrier();
        if (!active) continue;   // uniform: the load-only wavefronts go on to the next chunk
        Fr Qn[1][DT];
        coop_natural<D>(Qn, sq);

        f32x4 Ot[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            Fr SF[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) SF[dt] = frag_from<Fr>(St[dt][mt]);
            mma_tiles<Fr, DT>(Ot[mt], SF, Qn[0]);
        }
        if (CAUSAL) {
            Fr Kn[1][DT], KT[1][DT], VT[1][1];
            coop_natural<D>(Kn, sk);
            coop_transposed<D>(KT, sk);
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            mma_tiles<Fr, DT>(p, Kn[0], Qn[0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
            const Fr PT = frag_from<Fr>(p);
            transpose_frags<1, 1>(VT, Vn, sv);
            mma1(Ot[0], VT[0][0], PT);
            mma1(Ot[1], ones, PT);
            state_accumulate<Fr, D, 16, 1, true>(St, KT, VT);
        }
        const float inv = __builtin_amdgcn_rcpf(Ot[1][0]);
        const int64_t t = t0 + c;
        if (t < t_end) store4<T>(O + t * M + 16 * cg + 4 * g, IO<T>::from_f32(Ot[0] * inv));
    }
    }
}

// ---- backward ----------------------------------------------------------------------
// Token-contiguous copies in the column-group backward: bf16 through the
// wavefront's LDS area; fp32 operands, split (split4) or not, by identity
// products on the matrix cores, exact, since the groups' partial sums leave
// no LDS for the two-area copies of split operands.
template <int NF, int TT>
__device__ __forceinline__ void gtrans(bf16x4 (&yt)[TT][NF], const bf16x4 (&y)[TT][NF], lds_bf16 *stage) {
    transpose_frags<NF, TT>(yt, y, stage);
}
template <int NF, int TT>
__device__ __forceinline__ void gtrans(f32x4 (&yt)[TT][NF], const f32x4 (&y)[TT][NF], lds_bf16 *stage) {
    transpose_frags<NF, TT>(yt, y, stage);   // identity products on the fp32 instruction
}
template <int NF, int TT>
__device__ __forceinline__ void gtrans(split4 (&yt)[TT][NF], const split4 (&y)[TT][NF], lds_bf16 *) {
    const split4 ident = frag_identity<split4>();
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NF; ++f) yt[tt][f] = transpose_frag(y[tt][f], ident);
}
// LDS per wavefront for the token-contiguous copies (bf16: the D x 32 state
// slice, or one chunk of phi(Q) and the two g columns tiles); fp32 copies go
// through identity products.
template <typename T, int DT>
constexpr int gbwd_stage_elems() {
    return sizeof(T) == 4 ? 8
                          : (stage_elems<DT, 2>() > stage_elems<DT, 1>() + stage_elems<2, 1>()
                                 ? stage_elems<DT, 2>()
                                 : stage_elems<DT, 1>() + stage_elems<2, 1>());
}

// Partial sums of the wavefronts (one per column group) in LDS: part[cg][dt]
// holds wavefront cg's D-row tile dt, 64 lanes x 4 floats.  reduce_rows
// returns the sum over groups 0 .. ng - 1 of tile dt for this lane.
template <int DT>
__device__ __forceinline__ f32x4 reduce_rows(const f32x4 (*part)[DT][64], int ng, int dt) {
    const int lane = lane_id();
    f32x4 s = part[0][dt][lane];
    for (int w = 1; w < ng; ++w) s += part[w][dt][lane];
    return s;
}

// Forward direction.  Wavefront cg: S and Z slice St (Z replicated, as in
// k_gen_output_coop), this segment's reverse sums Ra = sum_i phi(q_i) [g_i, h_i]^T
// restricted to its columns (u, in column 0 of the second tile, on group 0).
// bf16 keeps the register count within two wavefronts per SIMD for every D:
// the state's bf16 copy goes to LDS as soon as it is formed, and the operand
// tiles of the dQ products (S^T, phi(K)^T) are read back from LDS one tile at
// a time where they are used.
template <typename T, int DT, bool CAUSAL, int NPW>
__global__ __launch_bounds__(512) void k_gbwd_dq(const T *__restrict__ q, const T *__restrict__ k,
                                                 const T *__restrict__ v, const T *__restrict__ dout,
                                                 T *__restrict__ dq, const float *__restrict__ wsS,
                                                 float *__restrict__ wsR, float *__restrict__ ibuf,
                                                 float *__restrict__ hbuf, int64_t N, int64_t M, int64_t nseg,
                                                 int64_t seg_tokens) {
    constexpr int D = 16 * DT;
    // fp32: split operands up to D = 64; beyond, their conversions and
    // identity-product copies cost more registers than the loops have, and
    // the fp32 instruction is faster there
    typedef typename std::conditional<(sizeof(T) == 4 && DT > 4), f32x4, CoopFrag<T>>::type Fr;
    typedef typename IO<T>::vec4 V4;
    // bf16 (SHARED): phi(Q) and phi(K) rows staged once per chunk for every
    // group, double-buffered (see k_gen_output_coop); phi'(x) = min(phi(x), 1)
    // is read off the staged phi
    constexpr bool SHARED = sizeof(T) == 2;
    constexpr int SR = SHARED ? coop_rows_elems<D>() : 8;
    constexpr int SS = D + kStagePad;   // row stride of the staged rows and of the state copy
    __shared__ __align__(16) bf16 stage_mem[8][gbwd_stage_elems<T, DT>()];
    __shared__ __align__(16) f32x4 part[8][DT][64];
    __shared__ float hpart[8][16];
    __shared__ __align__(16) bf16 shq[SHARED ? 2 : 1][SR], shk[SHARED && CAUSAL ? 2 : 1][SR];
    const int ng = int(M / 16);
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const int64_t rec = int64_t(D) * M + D;
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    const T *G = dout + bh * N * M;
    T *DQ = dq + bh * N * D;
    lds_bf16 *stage = (lds_bf16 *)stage_mem[cg];

    f32x4 St[DT][2], Ra[DT][2];
    {
        const float *r0 = wsS + (bh * nseg + (CAUSAL ? seg : 0)) * rec;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                St[dt][0][r] = r0[(16 * dt + 4 * g + r) * M + 16 * cg + c];
                St[dt][1][r] = r0[int64_t(D) * M + 16 * dt + 4 * g + r];
            }
            Ra[dt][0] = Ra[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    const Fr ones = frag_ones<Fr>();
    const Fr k0ones = frag_k0_ones<Fr>();

    // a chunk's inputs in registers; bf16 loads them two chunks ahead (chunk
    // parity b picks the set and the LDS buffer)
    constexpr int PF = SHARED ? 2 : 1;
    struct In {
        V4 rq[1][SHARED ? 1 : DT], rk[1][SHARED ? 1 : DT], rv, rg;
        CoopRows<D, SHARED ? NPW : 1> cq, ck;
    } in[PF];
    auto load_all = [&](In &x, int64_t t0) {
        if constexpr (SHARED) {
            coop_load<bf16, D>(x.cq, (const bf16 *)Q, t0, t_end, cg, ng);
            if (CAUSAL) coop_load<bf16, D>(x.ck, (const bf16 *)K, t0, t_end, cg, ng);
        } else {
            load_chunk<T, D, 1>(x.rq, Q, t0, t_end);
            if (CAUSAL) load_chunk<T, D, 1>(x.rk, K, t0, t_end);
        }
        if (CAUSAL) x.rv = load_col_tile<T>(V, M, 16 * cg, t0, t_end);
        x.rg = load_col_tile<T>(G, M, 16 * cg, t0, t_end);
    };
#pragma unroll
    for (int b = 0; b < PF; ++b) load_all(in[b], t_begin + b * GCH);   // rows past t_end read row t_end - 1
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * GCH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + b * GCH;
        if (t0 >= t_end) break;   // uniform over the workgroup
        In &cur = in[b];
        Fr Qn[1][DT], Kn[1][DT], Vn[1][1];
        f32x4 dphq[SHARED ? 1 : DT];   // fp32: phi'(Q) of this lane's (token, 4 features) per tile
        lds_bf16 *sq = (lds_bf16 *)shq[SHARED ? b : 0];
        lds_bf16 *sk = (lds_bf16 *)shk[SHARED && CAUSAL ? b : 0];
        if (CAUSAL) {
            const V4 one[1][1] = {{cur.rv}};
            raw_frags<T, 16, 1>(Vn, one, t0, t_end);
        }
        const f32x4 graw = IO<T>::to_f32(cur.rg);
        if constexpr (SHARED) {
            coop_stage<bf16, D, true, true>(sq, cur.cq, t0, t_end, cg, ng);   // rows past t_end are zero
            if (CAUSAL) coop_stage<bf16, D, true, true>(sk, cur.ck, t0, t_end, cg, ng);
            load_all(cur, t0 + PF * GCH);   // rows past t_end read row t_end - 1
            lds_barrier();
            natural_frags_lds<D, 1>(Qn, sq);
            if (CAUSAL) natural_frags_lds<D, 1>(Kn, sk);
        } else {
            phi_frags<T, D, 1>(Qn, cur.rq, t0, t_end);
            if (CAUSAL) phi_frags<T, D, 1>(Kn, cur.rk, t0, t_end);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) dphq[dt] = dphi4(IO<T>::to_f32(cur.rq[0][dt]));
            load_all(cur, t0 + PF * GCH);   // rows past t_end read row t_end - 1
        }
        const int64_t t = t0 + c;   // this lane's query token
        const bool valid = t < t_end;

        // V^T before the state copy takes the staging area (bf16: the
        // transposing write and read use the area the copy overwrites next)
        Fr VT[1][1];
        if (CAUSAL) gtrans<1, 1>(VT, Vn, stage + stage_elems<DT, 1>());

        // intra-chunk scores P^T[j][i] = phi(k_j) . phi(q_i), j <= i (first, so
        // that phi(K) is no longer held while the state is read out)
        Fr PT = frag_zero<Fr>();
        Fr KT[1][SHARED ? 1 : DT];
        if (CAUSAL) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
            mma_tiles<Fr, DT>(p, Kn[0], Qn[0]);
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
            PT = frag_from<Fr>(p);
            if constexpr (!SHARED) gtrans<DT, 1>(KT, Kn, stage);
        }

        // out^T of this group's columns (Ot[0]) and den (every row of Ot[1]);
        // fp32 keeps the state's operand copy SF for the dQ products, bf16
        // writes it to LDS (tile row mt, feature tile dt) as it goes
        f32x4 Ot[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        Fr SF[2][SHARED ? 1 : DT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            Fr sf[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                sf[dt] = frag_from<Fr>(St[dt][mt]);
                if constexpr (SHARED)
                    *reinterpret_cast<lds_bf16x4 *>(stage + (16 * mt + c) * SS + 16 * dt + 4 * g) = sf[dt];
                else
                    SF[mt][dt] = sf[dt];
            }
            mma_tiles<Fr, DT>(Ot[mt], sf, Qn[0]);
        }
        if (CAUSAL) {
            mma1(Ot[0], VT[0][0], PT);
            mma1(Ot[1], ones, PT);
        }
        const float inv = valid ? __builtin_amdgcn_rcpf(Ot[1][0]) : 0.f;

        // h = -(dout . out) / d: this group's share, then the sum over groups
        const f32x4 o = Ot[0] * inv;
        float go = graw[0] * o[0] + graw[1] * o[1] + graw[2] * o[2] + graw[3] * o[3];
        go += __shfl_xor(go, 16);
        go += __shfl_xor(go, 32);
        if (g == 0) hpart[cg][c] = go;
        lds_barrier();
        float gsum = hpart[0][c];
        for (int w = 1; w < ng; ++w) gsum += hpart[w][c];
        const float h = -gsum * inv;
        if (CAUSAL && cg == 0 && valid && g == 0) {
            ibuf[bh * N + t] = inv;
            hbuf[bh * N + t] = h;
        }
        const Fr Gn = frag_from<Fr>(graw * inv);                           // rows past t_end: inv = 0
        const Fr Gh = frag_from<Fr>(f32x4{g == 0 ? h : 0.f, 0.f, 0.f, 0.f});   // h in column 0

        // dA^T[j][i] = v_j . g_i over this group's columns (group 0 adds h_i), j <= i
        Fr dAT = frag_zero<Fr>();
        if (CAUSAL) {
            f32x4 da = {0.f, 0.f, 0.f, 0.f};
            mma1(da, Vn[0][0], Gn);
            if (cg == 0) mma1(da, k0ones, Gh);
#pragma unroll
            for (int r = 0; r < 4; ++r) da[r] = (4 * g + r <= c) ? da[r] : 0.f;
            dAT = frag_from<Fr>(da);
        }

        // this group's part of dL/dphi(q)^T[d][i]: sum_j phi(k_j)[d] dA^T[j][i]
        // + S[d][its columns] g_i (+ Z[d] h_i on group 0)
        if constexpr (SHARED) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (CAUSAL) mma1(acc, transposed_tile_lds(sk, SS, 0, dt), dAT);
                mma1(acc, transposed_tile_lds(stage, SS, 0, dt), Gn);
                if (cg == 0) mma1(acc, transposed_tile_lds(stage, SS, 1, dt), Gh);
                part[cg][dt][lane] = acc;
            }
        } else {
            Fr SFT[2][DT];
            gtrans<DT, 2>(SFT, SF, stage);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (CAUSAL) mma1(acc, KT[0][dt], dAT);
                mma1(acc, SFT[0][dt], Gn);
                if (cg == 0) mma1(acc, SFT[1][dt], Gh);
                part[cg][dt][lane] = acc;
            }
        }
        lds_barrier();
        for (int dt = cg; dt < DT; dt += ng) {   // the groups' sum, tiles dealt out over the wavefronts
            f32x4 dph;
            if constexpr (SHARED)
                dph = dphi_staged<D>(sq, dt);
            else
                dph = dphq[dt];
            const f32x4 dqv = reduce_rows<DT>(part, ng, dt) * dph;
            if (valid) store4<T>(DQ + t * D + 16 * dt + 4 * g, IO<T>::from_f32(dqv));
        }

        // this segment's reverse sums: Ra += phi(Q)^T [g | h] (its columns)
        Fr QT[1][DT], GT[1][2];
        if constexpr (SHARED)
            transposed_frags_lds<D, 1>(QT, sq);
        else
            gtrans<DT, 1>(QT, Qn, stage);
        {
            const Fr gg[1][2] = {{Gn, Gh}};
            gtrans<2, 1>(GT, gg, stage + stage_elems<DT, 1>());
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            mma1(Ra[dt][0], QT[0][dt], GT[0][0]);
            if (cg == 0) mma1(Ra[dt][1], QT[0][dt], GT[0][1]);
        }

        if (CAUSAL) {
            if constexpr (SHARED) {
                Fr KTs[1][DT];
                transposed_frags_lds<D, 1>(KTs, sk);
                state_accumulate<Fr, D, 16, 1, true>(St, KTs, VT);
            } else {
                state_accumulate<Fr, D, 16, 1, true>(St, KT, VT);
            }
        }
    }
    }
    float *r1 = wsR + (bh * nseg + seg) * rec;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
        for (int r = 0; r < 4; ++r) r1[(16 * dt + 4 * g + r) * M + 16 * cg + c] = Ra[dt][0][r];
        if (cg == 0 && c == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) r1[int64_t(D) * M + 16 * dt + 4 * g + r] = Ra[dt][1][r];
        }
    }
}

// Reverse direction.  Wavefront cg carries R[:, its columns] and (group 0)
// u, walking the chunks last to first; writes dV of its columns and, with
// the other groups, dK.  bf16 holds the state's operand copy in LDS and reads
// the transposed tiles (R^T, phi(Q)^T) where they are used, as k_gbwd_dq does.
template <typename T, int DT, bool CAUSAL, int NPW>
__global__ __launch_bounds__(512) void k_gbwd_dkdv(const T *__restrict__ q, const T *__restrict__ k,
                                                   const T *__restrict__ v, const T *__restrict__ dout,
                                                   const float *__restrict__ ibuf, const float *__restrict__ hbuf,
                                                   T *__restrict__ dk, T *__restrict__ dv,
                                                   const float *__restrict__ wsR, int64_t N, int64_t M,
                                                   int64_t nseg, int64_t seg_tokens) {
    constexpr int D = 16 * DT;
    // fp32: split operands up to D = 64; beyond, their conversions and
    // identity-product copies cost more registers than the loops have, and
    // the fp32 instruction is faster there
    typedef typename std::conditional<(sizeof(T) == 4 && DT > 4), f32x4, CoopFrag<T>>::type Fr;
    typedef typename IO<T>::vec4 V4;
    constexpr bool SHARED = sizeof(T) == 2;   // as in k_gbwd_dq
    constexpr int SR = SHARED ? coop_rows_elems<D>() : 8;
    constexpr int SS = D + kStagePad;
    __shared__ __align__(16) bf16 stage_mem[8][gbwd_stage_elems<T, DT>()];
    __shared__ __align__(16) f32x4 part[8][DT][64];
    __shared__ __align__(16) bf16 shq[SHARED && CAUSAL ? 2 : 1][SR], shk[SHARED ? 2 : 1][SR];
    const int ng = int(M / 16);
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const int64_t rec = int64_t(D) * M + D;
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    const T *G = dout + bh * N * M;
    T *DK = dk + bh * N * D;
    T *DV = dv + bh * N * M;
    lds_bf16 *stage = (lds_bf16 *)stage_mem[cg];

    f32x4 Rr[DT][2];   // R[:, its columns]; u in column 0 of the second tile (group 0 only)
    {
        const float *r0 = wsR + (bh * nseg + (CAUSAL ? seg : 0)) * rec;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Rr[dt][0][r] = r0[(16 * dt + 4 * g + r) * M + 16 * cg + c];
                Rr[dt][1][r] = (cg == 0 && c == 0) ? r0[int64_t(D) * M + 16 * dt + 4 * g + r] : 0.f;
            }
    }
    const Fr k0ones = frag_k0_ones<Fr>();

    const int64_t nch = (t_end - t_begin + GCH - 1) / GCH;
    // a chunk's inputs in registers; bf16 loads them two chunks ahead (step s
    // visits chunk nch - 1 - s from set and LDS buffer s % 2)
    constexpr int PF = SHARED ? 2 : 1;
    struct In {
        V4 rq[1][SHARED ? 1 : DT], rk[1][SHARED ? 1 : DT], rv, rg;
        CoopRows<D, SHARED ? NPW : 1> cq, ck;
        float rh, ri;
    } in[PF];
    auto load_all = [&](In &x, int64_t t0) {
        if constexpr (SHARED) {
            if (CAUSAL) coop_load<bf16, D>(x.cq, (const bf16 *)Q, t0, t_end, cg, ng);
            coop_load<bf16, D>(x.ck, (const bf16 *)K, t0, t_end, cg, ng);
        } else {
            if (CAUSAL) load_chunk<T, D, 1>(x.rq, Q, t0, t_end);
            load_chunk<T, D, 1>(x.rk, K, t0, t_end);
        }
        x.rv = load_col_tile<T>(V, M, 16 * cg, t0, t_end);
        if (CAUSAL) {
            x.rg = load_col_tile<T>(G, M, 16 * cg, t0, t_end);
            x.rh = (t0 + c < t_end) ? hbuf[bh * N + t0 + c] : 0.f;
            x.ri = (t0 + c < t_end) ? ibuf[bh * N + t0 + c] : 0.f;
        }
    };
#pragma unroll
    for (int b = 0; b < PF; ++b) load_all(in[b], t_begin + imax64(nch - 1 - b, 0) * GCH);
    for (int64_t s0 = 0; s0 < nch; s0 += PF) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t ci = nch - 1 - (s0 + b);
        if (ci < 0) break;   // uniform over the workgroup
        const int64_t t0 = t_begin + ci * GCH;
        In &cur = in[b];
        Fr Qn[1][DT], Kn[1][DT], Vn[1][1];
        Fr Gn = frag_zero<Fr>(), Gh = frag_zero<Fr>();
        f32x4 dphk[SHARED ? 1 : DT];   // fp32: phi'(K) of this lane's (token, 4 features) per tile
        lds_bf16 *sq = (lds_bf16 *)shq[SHARED && CAUSAL ? b : 0];
        lds_bf16 *sk = (lds_bf16 *)shk[SHARED ? b : 0];
        if constexpr (SHARED) {
            if (CAUSAL) coop_stage<bf16, D, true, true>(sq, cur.cq, t0, t_end, cg, ng);   // rows past t_end are zero
            coop_stage<bf16, D, true, true>(sk, cur.ck, t0, t_end, cg, ng);
        } else {
            if (CAUSAL) phi_frags<T, D, 1>(Qn, cur.rq, t0, t_end);
            phi_frags<T, D, 1>(Kn, cur.rk, t0, t_end);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) dphk[dt] = dphi4(IO<T>::to_f32(cur.rk[0][dt]));
        }
        {
            const V4 one[1][1] = {{cur.rv}};
            raw_frags<T, 16, 1>(Vn, one, t0, t_end);
        }
        if (CAUSAL) {   // g = dout / d as in the forward-direction pass; rows past t_end are 0 (ri = 0)
            Gn = frag_from<Fr>(IO<T>::to_f32(cur.rg) * cur.ri);
            Gh = frag_from<Fr>(f32x4{g == 0 ? cur.rh : 0.f, 0.f, 0.f, 0.f});
        }
        if (ci >= PF) load_all(cur, t0 - PF * GCH);
        if constexpr (SHARED) {
            lds_barrier();
            if (CAUSAL) natural_frags_lds<D, 1>(Qn, sq);
            natural_frags_lds<D, 1>(Kn, sk);
        }
        const int64_t t = t0 + c;   // this lane's key token
        const bool valid = t < t_end;

        // [g | h]^T before the state copy takes the staging area (bf16: the
        // transposing write and read use the area the copy overwrites next)
        Fr GT[1][2];
        if (CAUSAL) {
            const Fr gg[1][2] = {{Gn, Gh}};
            gtrans<2, 1>(GT, gg, stage + stage_elems<DT, 1>());
        }

        // P[i][j] = phi(q_i) . phi(k_j); dA[i][j] = g_i . v_j over this group's columns
        // (group 0 adds h_i); both masked to i >= j
        Fr Pf = frag_zero<Fr>(), dAf = frag_zero<Fr>();
        if (CAUSAL) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f}, da = {0.f, 0.f, 0.f, 0.f};
            mma_tiles<Fr, DT>(p, Qn[0], Kn[0]);
            mma1(da, Gn, Vn[0][0]);
            if (cg == 0) mma1(da, Gh, k0ones);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool keep = 4 * g + r >= c;
                p[r] = keep ? p[r] : 0.f;
                da[r] = keep ? da[r] : 0.f;
            }
            Pf = frag_from<Fr>(p);
            dAf = frag_from<Fr>(da);
        }

        // dV^T[m][j] (its columns) = sum_i g[i][m] P[i][j] + sum_d R[d][m] phi(k_j)[d];
        // the state's operand copy RF is formed here (bf16: written to LDS,
        // tile row mt, feature tile dt, for the transposed reads below)
        Fr RF[2][SHARED ? 1 : DT];
        {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (CAUSAL) mma1(acc, GT[0][0], Pf);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                Fr rf[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    rf[dt] = frag_from<Fr>(Rr[dt][mt]);
                    if constexpr (SHARED)
                        *reinterpret_cast<lds_bf16x4 *>(stage + (16 * mt + c) * SS + 16 * dt + 4 * g) = rf[dt];
                    else
                        RF[mt][dt] = rf[dt];
                }
                if (mt == 0) mma_tiles<Fr, DT>(acc, rf, Kn[0]);
            }
            if (valid) store4<T>(DV + t * M + 16 * cg + 4 * g, IO<T>::from_f32(acc));
        }

        // this group's part of dL/dphi(k)^T[d][j]: sum_i phi(q_i)[d] dA[i][j]
        // + R[d][its columns] v_j (+ u[d] on group 0)
        Fr QT[1][SHARED ? 1 : DT];
        if constexpr (SHARED) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (CAUSAL) mma1(acc, transposed_tile_lds(sq, SS, 0, dt), dAf);
                mma1(acc, transposed_tile_lds(stage, SS, 0, dt), Vn[0][0]);
                if (cg == 0) mma1(acc, transposed_tile_lds(stage, SS, 1, dt), k0ones);
                part[cg][dt][lane] = acc;
            }
        } else {
            Fr RFT[2][DT];
            gtrans<DT, 2>(RFT, RF, stage);
            if (CAUSAL) gtrans<DT, 1>(QT, Qn, stage);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (CAUSAL) mma1(acc, QT[0][dt], dAf);
                mma1(acc, RFT[0][dt], Vn[0][0]);
                if (cg == 0) mma1(acc, RFT[1][dt], k0ones);
                part[cg][dt][lane] = acc;
            }
        }
        lds_barrier();
        for (int dt = cg; dt < DT; dt += ng) {
            f32x4 dph;
            if constexpr (SHARED)
                dph = dphi_staged<D>(sk, dt);
            else
                dph = dphk[dt];
            const f32x4 dkv = reduce_rows<DT>(part, ng, dt) * dph;
            if (valid) store4<T>(DK + t * D + 16 * dt + 4 * g, IO<T>::from_f32(dkv));
        }
        // carry R (and u) towards earlier tokens
        if (CAUSAL) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                Fr qt;
                if constexpr (SHARED)
                    qt = transposed_tile_lds(sq, SS, 0, dt);
                else
                    qt = QT[0][dt];
                mma1(Rr[dt][0], qt, GT[0][0]);
                if (cg == 0) mma1(Rr[dt][1], qt, GT[0][1]);
            }
        }
        // every group has read `part` before the next chunk writes it: with
        // shared staging (bf16) the next chunk's staging barrier, which comes
        // before those writes, already ensures it
        if constexpr (!SHARED) lds_barrier();
    }
    }
}

// ---- host side -------------------------------------------------------------------
// The workspace starts with the same 256-byte header as the fused forwards'
// (its error word stays as the caller left it: nothing here waits), then one
// record per segment.
constexpr size_t kGenHeader = 256;
size_t generic_workspace_bytes(int64_t BH, int64_t N, int64_t D, int64_t M) {
    const SegPlan p = make_plan(BH, N, D, M);
    return kGenHeader + align256(size_t(BH * p.nseg * p.rec) * sizeof(float));
}

// Whether each lane moves at most one piece of a chunk's shared Q or K rows
// (CoopRows NPW = 1): the segment's M / 16 wavefronts cover the 2 D
// sixteen-byte pieces once, 64 (M / 16) >= 2 D.
// Whether each lane moves at most one piece of a chunk's shared Q or K rows
// (CoopRows NPW = 1): the segment's M / 16 wavefronts cover the pieces once.
// Wavefronts of a forward workgroup: one per column group, and at least
// enough that each lane moves at most two pieces of a chunk's shared Q or K
// rows (the extra wavefronts only load and stage rows).
template <typename T, int DT> static int gen_waves(int64_t M) {
    const int need = int((coop_pieces<T>(16 * DT) + 127) / 128);
    return int(M / 16) > need ? int(M / 16) : need;
}
// Pieces per lane (NPW) of a forward launch with nw wavefronts: 1 or 2.
template <typename T, int DT> static int gen_npw(int nw) { return 64 * nw >= coop_pieces<T>(16 * DT) ? 1 : 2; }
// Whether each lane of the backward's M / 16 wavefronts moves one piece (bf16).
template <typename T, int DT> static bool gen_one_piece(int64_t M) {
    return coop_np<T, 16 * DT>() == 1 || 64 * (M / 16) >= coop_pieces<T>(16 * DT);
}

// Per-segment sums of phi(K) [V, 1]^T (the block is 64 gen_waves(M) threads).
template <typename T, int DT>
static void launch_gen_segstate(bool phi, dim3 grid, const void *k, const void *v, float *ws, int64_t N, int64_t M,
                                const SegPlan &p, hipStream_t s) {
    const int nw = gen_waves<T, DT>(M);
    const dim3 block(unsigned(64 * nw));
#define LA_GEN_SEG(W, H)                                                                                          \
    do {                                                                                                          \
        if (phi)                                                                                                  \
            hipLaunchKernelGGL((k_gen_segstate_coop<T, DT, true, W, H>), grid, block, 0, s, (const T *)k,          \
                               (const T *)v, ws, N, M, p.nseg, p.seg_tokens);                                     \
        else                                                                                                      \
            hipLaunchKernelGGL((k_gen_segstate_coop<T, DT, false, W, H>), grid, block, 0, s, (const T *)k,         \
                               (const T *)v, ws, N, M, p.nseg, p.seg_tokens);                                     \
    } while (0)
    if (gen_npw<T, DT>(nw) == 1)
        LA_GEN_SEG(1, false);
    else if (nw == M / 16)
        LA_GEN_SEG(2, false);
    else if constexpr (coop_pieces<T>(16 * DT) > 128)
        LA_GEN_SEG(2, true);
#undef LA_GEN_SEG
}

template <typename T, int DT>
static hipError_t run_generic(bool causal, bool phi, const void *q, const void *k, const void *v, void *out,
                              int64_t BH, int64_t N, int64_t M, float *ws, StateIO sio, hipStream_t s) {
    constexpr int D = 16 * DT;
    const SegPlan p = make_plan(BH, N, D, M);
    const dim3 grid(unsigned(BH * p.nseg));
    ws = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + kGenHeader);
    launch_gen_segstate<T, DT>(phi, grid, k, v, ws, N, M, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanIO io;
    io.s0 = sio.s0;
    io.z0 = sio.z0;
    io.s1 = sio.s1;
    io.z1 = sio.z1;
    io.srec = int64_t(D) * M;
    if ((e = launch_scan(ws, BH, p.nseg, p.rec, causal ? 0 : 1, s, io)) != hipSuccess) return e;
    const int nw = gen_waves<T, DT>(M);
    const dim3 block(unsigned(64 * nw));
    const int npw = gen_npw<T, DT>(nw);
#define LA_GEN_OUT_K(C, P, W, H)                                                                                  \
    hipLaunchKernelGGL((k_gen_output_coop<T, DT, C, P, W, H>), grid, block, 0, s, (const T *)q, (const T *)k,       \
                       (const T *)v, (T *)out, (const float *)ws, N, M, p.nseg, p.seg_tokens)
#define LA_GEN_OUT(C, P)                                                                                          \
    do {                                                                                                          \
        if (npw == 1)                                                                                             \
            LA_GEN_OUT_K(C, P, 1, false);                                                                         \
        else if (nw == M / 16)                                                                                    \
            LA_GEN_OUT_K(C, P, 2, false);                                                                         \
        else if constexpr (coop_pieces<T>(D) > 128)                                                               \
            LA_GEN_OUT_K(C, P, 2, true);                                                                          \
    } while (0)
    if (!causal) {
        LA_GEN_OUT(false, true);
    } else if (phi) {
        LA_GEN_OUT(true, true);
    } else {
        LA_GEN_OUT(true, false);
    }
#undef LA_GEN_OUT
#undef LA_GEN_OUT_K
    return hipGetLastError();
}

template <typename T>
static hipError_t run_generic_t(bool causal, bool phi, const void *q, const void *k, const void *v, void *out,
                                int64_t BH, int64_t N, int64_t D, int64_t M, float *ws, StateIO sio, hipStream_t s) {
    switch (D) {
    case 16: return run_generic<T, 1>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 32: return run_generic<T, 2>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 48: return run_generic<T, 3>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 64: return run_generic<T, 4>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 80: return run_generic<T, 5>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 96: return run_generic<T, 6>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 112: return run_generic<T, 7>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    case 128: return run_generic<T, 8>(causal, phi, q, k, v, out, BH, N, M, ws, sio, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_forward_generic(bool causal, int dt, const void *q, const void *k, const void *v, void *out,
                                  int64_t BH, int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s,
                                  StateIO sio) {
    if (M % 16 != 0 || M < 16 || M > 128 || (!causal && (sio.s0 || sio.s1 || sio.features_given)))
        return hipErrorInvalidValue;
    const bool phi = !sio.features_given;
    if (dt == 0) return run_generic_t<float>(causal, phi, q, k, v, out, BH, N, D, M, ws, sio, s);
    return run_generic_t<bf16>(causal, phi, q, k, v, out, BH, N, D, M, ws, sio, s);
}


// The dQ pass, the reverse scan and the dK/dV pass, with NPW pieces of each
// chunk's Q and K rows per lane (bf16; unused for fp32).
template <typename T, int DT, int NPW>
static hipError_t run_gbwd_passes(bool causal, dim3 grid, dim3 block, const void *q, const void *k, const void *v,
                                  const void *dout, void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t M,
                                  const SegPlan &p, float *wsS, float *wsR, float *ibuf, float *hbuf,
                                  hipStream_t s) {
    if (causal)
        hipLaunchKernelGGL((k_gbwd_dq<T, DT, true, NPW>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (T *)dq, (const float *)wsS, wsR, ibuf, hbuf, N, M, p.nseg,
                           p.seg_tokens);
    else
        hipLaunchKernelGGL((k_gbwd_dq<T, DT, false, NPW>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (T *)dq, (const float *)wsS, wsR, ibuf, hbuf, N, M, p.nseg,
                           p.seg_tokens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_scan(wsR, BH, p.nseg, p.rec, causal ? 2 : 1, s)) != hipSuccess) return e;
    if (causal)
        hipLaunchKernelGGL((k_gbwd_dkdv<T, DT, true, NPW>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (const float *)ibuf, (const float *)hbuf, (T *)dk,
                           (T *)dv, (const float *)wsR, N, M, p.nseg, p.seg_tokens);
    else
        hipLaunchKernelGGL((k_gbwd_dkdv<T, DT, false, NPW>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (const T *)dout, (const float *)ibuf, (const float *)hbuf, (T *)dk,
                           (T *)dv, (const float *)wsR, N, M, p.nseg, p.seg_tokens);
    return hipGetLastError();
}

template <typename T, int DT>
static hipError_t run_generic_backward(bool causal, const void *q, const void *k, const void *v, const void *dout,
                                       void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t M, float *ws,
                                       hipStream_t s) {
    constexpr int D = 16 * DT;
    const SegPlan p = make_plan(BH, N, D, M);
    const BwdLayout L = backward_layout(BH, N, D, M, sizeof(T));
    float *wsS = ws;
    float *wsR = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.states);
    float *ibuf = causal ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.inv_off) : nullptr;
    float *hbuf = causal ? reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + L.h_off) : nullptr;
    const dim3 grid(unsigned(BH * p.nseg)), block(unsigned(64 * (M / 16)));
    launch_gen_segstate<T, DT>(true, grid, k, v, wsS, N, M, p, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = launch_scan(wsS, BH, p.nseg, p.rec, causal ? 0 : 1, s)) != hipSuccess) return e;
    constexpr int NP = coop_np<bf16, D>();
    if (sizeof(T) == 4 || gen_one_piece<bf16, DT>(M))
        return run_gbwd_passes<T, DT, 1>(causal, grid, block, q, k, v, dout, dq, dk, dv, BH, N, M, p, wsS, wsR, ibuf,
                                         hbuf, s);
    if constexpr (sizeof(T) == 2 && NP > 1)
        return run_gbwd_passes<T, DT, NP>(causal, grid, block, q, k, v, dout, dq, dk, dv, BH, N, M, p, wsS, wsR,
                                          ibuf, hbuf, s);
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t run_generic_backward_t(bool causal, const void *q, const void *k, const void *v,
                                         const void *dout, void *dq, void *dk, void *dv, int64_t BH, int64_t N,
                                         int64_t D, int64_t M, float *ws, hipStream_t s) {
    switch (D) {
    case 16: return run_generic_backward<T, 1>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 32: return run_generic_backward<T, 2>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 48: return run_generic_backward<T, 3>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 64: return run_generic_backward<T, 4>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 80: return run_generic_backward<T, 5>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 96: return run_generic_backward<T, 6>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 112: return run_generic_backward<T, 7>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    case 128: return run_generic_backward<T, 8>(causal, q, k, v, dout, dq, dk, dv, BH, N, M, ws, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_backward_generic(bool causal, int dt, const void *q, const void *k, const void *v,
                                   const void *dout, void *dq, void *dk, void *dv, int64_t BH, int64_t N, int64_t D,
                                   int64_t M, float *ws, hipStream_t s) {
    if (M % 16 != 0 || M < 16 || M > 128) return hipErrorInvalidValue;
    if (dt == 0) return run_generic_backward_t<float>(causal, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
    return run_generic_backward_t<bf16>(causal, q, k, v, dout, dq, dk, dv, BH, N, D, M, ws, s);
}

}  // namespace la
