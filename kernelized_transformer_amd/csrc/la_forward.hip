// la_forward.hip -- chunked causal and non-causal forward on gfx950.
//
// Method ([deck] = zhengyuhong.cn "Transformers are RNNs ... 解读", slides
// 3-4; [summary] = paperlayer.ai summary, sections 3.2-3.3.2):
//   causal:     out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i, with the inclusive
//               prefix states S_i = sum_{j<=i} phi(K_j) V_j^T, Z_i = sum_{j<=i} phi(K_j);
//   non-causal: the same with S, Z summed over all tokens.
// The training-time form is evaluated in parallel over the sequence
// ([summary] 3.3.2): the sequence is cut into chunks of 16 tokens, and a
// chunk's outputs are
//   num_c = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) S_prev,
//   den_c = tril(phi(Q_c) phi(K_c)^T) 1   + phi(Q_c) Z_prev,
// an exact regrouping of the prefix sums.  All products run on the matrix
// cores with fp32 accumulation, in transposed form (out^T = V^T P^T + S^T Q^T)
// so that every operand is either a plain row-major load or an accumulator
// tile reused in place (see la_device.h).
//
// Sequence parallelism.  Each wavefront owns a sub-segment of whole chunks
// and walks it twice: first summing phi(K_t) [V_t, 1]^T into a local fp32
// state, then (after learning the state of everything before it) producing
// the outputs chunk by chunk while carrying (S, Z) in registers.
//   causal (one launch, k_fwd_fused): eight wavefronts (two per SIMD) form a block; their
//     local states are combined in LDS, and the blocks of one (b, h) form
//     their prefix states together through the workspace (see the comment
//     at the kernel);
//   non-causal (three launches): per-segment states, their sum per (b, h),
//     then the readout.
#include <atomic>
#include <type_traits>
#include <chrono>

#include "la_chunk.h"
#include "la_internal.h"
#include "la_split.h"

namespace la {

constexpr int TT = 1;        // token tiles per chunk in the forward kernels
constexpr int CH = 16 * TT;  // = kChunk
static_assert(CH == kChunk, "forward chunk");
constexpr int kPrefetch = 2; // chunks in flight ahead of the one being computed
// fp32 operands at D = M = 64 take twice the registers: one chunk ahead there
template <typename T, int D, int M> constexpr int fwd_prefetch() {
    return (sizeof(T) == 4 && D == 64 && M == 64) ? 1 : kPrefetch;
}

// ---- chunk loops ------------------------------------------------------------

// St += sum over tokens [t_begin, t_end) of phi(K_t) [V_t, 1]^T.
// PF chunks are kept in flight: the loop is unrolled by PF so that chunk i
// always lives in buffer i % PF (a register copy between buffers would force
// a wait on the loads in flight).
// PHI: apply the feature map to K (otherwise K holds the features already).
// Fr: the operand fragment type (split4 runs fp32 data on the bf16 matrix
// instruction; the staging areas then hold two bf16 tiles each).
template <typename T, int D, int M, int PF, bool PHI = true, typename Fr = typename IO<T>::frag>
__device__ __forceinline__ void seg_aggregate(const T *__restrict__ K, const T *__restrict__ V, int64_t t_begin,
                                              int64_t t_end, f32x4 (&St)[D / 16][M / 16 + 1], lds_bf16 *stage_k,
                                              lds_bf16 *stage_v) {
    typedef typename IO<T>::vec4 V4;
    V4 rk[PF][TT][D / 16], rv[PF][TT][M / 16];
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        load_chunk<T, D, TT>(rk[b], K, t_begin + b * CH, t_end);
        load_chunk<T, M, TT>(rv[b], V, t_begin + b * CH, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * CH) {
#pragma unroll
        for (int b = 0; b < PF; ++b) {
            const int64_t t0 = t00 + b * CH;   // may lie past t_end: fully masked, no stores
            Fr Kn[TT][D / 16], Vn[TT][M / 16];
            feat_frags<T, D, TT, PHI>(Kn, rk[b], t0, t_end);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int f = 0; f < M / 16; ++f) value_frags_unmasked(Vn[tt][f], rv[b][tt][f]);
            load_chunk<T, D, TT>(rk[b], K, t0 + PF * CH, t_end);
            load_chunk<T, M, TT>(rv[b], V, t0 + PF * CH, t_end);
            // keep the prefetch where it is: the scheduler would otherwise sink
            // the loads next to their use two chunks later
            __builtin_amdgcn_sched_barrier(0);
            Fr KT[TT][D / 16], VT[TT][M / 16];
            transpose_frags<D / 16>(KT, Kn, stage_k);
            transpose_frags<M / 16>(VT, Vn, stage_v);
            state_accumulate<Fr, D, M, TT, true>(St, KT, VT);
        }
    }
}

// Outputs for tokens [t_begin, t_end), starting from the state St of all
// earlier tokens (updated as the walk proceeds when CAUSAL).  Per chunk,
// with Acc tiles Ot[mt][it] = out^T (rows m plus the normalizer row block,
// cols = queries):
//   readout:  Ot[mt][it] += S^T[m][d] phi(Q)[i][d]      (S from St, as is)
//   intra:    Ot[mt][it] += V^T[m][j] P^T[j][i], P^T[j][i] = phi(K_j).phi(Q_i), j <= i
//   update:   St += phi(K)^T [V, 1]
// The normalizer row block of Ot gets den_i in row 0.
// The first PF chunks of seg_output, loaded ahead (the fused forward issues
// them before its cross-workgroup hand-off, while the memory system is idle).
template <typename T, int D, int M, int PF> struct ChunkAhead {
    typename IO<T>::vec4 rq[PF][TT][D / 16], rk[PF][TT][D / 16], rv[PF][TT][M / 16];
    template <bool CAUSAL>
    __device__ __forceinline__ void load(const T *Q, const T *K, const T *V, int64_t t_begin, int64_t t_end) {
#pragma unroll
        for (int b = 0; b < PF; ++b) {
            load_chunk<T, D, TT>(rq[b], Q, t_begin + b * CH, t_end);
            if (CAUSAL) {
                load_chunk<T, D, TT>(rk[b], K, t_begin + b * CH, t_end);
                load_chunk<T, M, TT>(rv[b], V, t_begin + b * CH, t_end);
            }
        }
    }
};

template <typename T, int D, int M, bool CAUSAL, int PF, bool PHI = true, typename Fr = typename IO<T>::frag>
__device__ __forceinline__ void seg_output(const T *__restrict__ Q, const T *__restrict__ K,
                                           const T *__restrict__ V, T *__restrict__ O, int64_t t_begin,
                                           int64_t t_end, f32x4 (&St)[D / 16][M / 16 + 1], lds_bf16 *stage_k,
                                           lds_bf16 *stage_v, ChunkAhead<T, D, M, PF> &ahead) {
    constexpr int DT = D / 16, MT = M / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const Fr ones = frag_ones<Fr>();
    const Fr zero = frag_zero<Fr>();
    auto &rq = ahead.rq;
    auto &rk = ahead.rk;
    auto &rv = ahead.rv;
    for (int64_t t00 = t_begin; t00 < t_end; t00 += PF * CH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int64_t t0 = t00 + b * CH;   // may lie past t_end: fully masked, no stores
        // no row masks (as in seg_output_bf16): rows past the end hold copies of
        // the last valid row (finite whenever the data is), their outputs are
        // not stored, the causal mask keeps them out of every stored output,
        // and the state is not used after the last chunk
        Fr Qn[TT][DT], Kn[TT][DT], Vn[TT][MT];
        feat_frags<T, D, TT, PHI, false>(Qn, rq[b], t0, t_end);
        if (CAUSAL) {
            feat_frags<T, D, TT, PHI, false>(Kn, rk[b], t0, t_end);
#pragma unroll
            for (int tt = 0; tt < TT; ++tt)
#pragma unroll
                for (int f = 0; f < MT; ++f) value_frags_unmasked(Vn[tt][f], rv[b][tt][f]);
        }
        load_chunk<T, D, TT>(rq[b], Q, t0 + PF * CH, t_end);
        if (CAUSAL) {
            load_chunk<T, D, TT>(rk[b], K, t0 + PF * CH, t_end);
            load_chunk<T, M, TT>(rv[b], V, t0 + PF * CH, t_end);
        }
        __builtin_amdgcn_sched_barrier(0);

        f32x4 Ot[MT + 1][TT];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int it = 0; it < TT; ++it) Ot[mt][it] = f32x4{0.f, 0.f, 0.f, 0.f};

        // readout against the state carried in from earlier tokens
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) {
            Fr SF[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) SF[dt] = frag_from<Fr>(St[dt][mt]);
#pragma unroll
            for (int it = 0; it < TT; ++it)
#pragma unroll
                for (int dt = 0; dt < DT; dt += 2) mma2(Ot[mt][it], SF[dt], SF[dt + 1], Qn[it][dt], Qn[it][dt + 1]);
        }

        if (CAUSAL) {
            // P^T tiles (keys x queries), causal mask inside the diagonal tiles
            Fr PT[TT][TT];
#pragma unroll
            for (int it = 0; it < TT; ++it)
#pragma unroll
                for (int jt = 0; jt < TT; ++jt) {
                    if (jt > it) {
                        PT[jt][it] = zero;
                        continue;
                    }
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int dt = 0; dt < DT; dt += 2) mma2(p, Kn[jt][dt], Kn[jt][dt + 1], Qn[it][dt], Qn[it][dt + 1]);
                    if (jt == it) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
                    }
                    PT[jt][it] = frag_from<Fr>(p);
                }
            Fr KT[TT][DT], VT[TT][MT];
            transpose_frags<DT>(KT, Kn, stage_k);
            transpose_frags<MT>(VT, Vn, stage_v);
            // intra-chunk term; the ones block sums P^T into den (every row)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
                for (int it = 0; it < TT; ++it) {
                    Fr a[TT], b[TT];
#pragma unroll
                    for (int jt = 0; jt < TT; ++jt) {
                        a[jt] = (mt < MT) ? VT[jt][mt] : ones;
                        b[jt] = PT[jt][it];
                    }
                    mma_tiles<Fr, TT>(Ot[mt][it], a, b);
                }
            state_accumulate<Fr, D, M, TT, true>(St, KT, VT);
        }

        // normalize and store: every row of the normalizer block holds den,
        // so element 0 of lane (c, g) is the denominator of token c
#pragma unroll
        for (int it = 0; it < TT; ++it) {
            const float den = Ot[MT][it][0];
            const float inv = __builtin_amdgcn_rcpf(den);
            const int64_t t = t0 + 16 * it + c;
            if (t < t_end) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) store4<T>(O + t * M + 16 * mt + 4 * g, IO<T>::from_f32(Ot[mt][it] * inv));
            }
        }
    }
    }
}

// ---- chunk loops, bf16: contiguous loads + LDS staging ---------------------------

// Normalizes one 16-token output tile (Ot[mt] = out^T tiles, every row of
// the normalizer block Ot[M/16] holding the tokens' denominators) and stores
// it through the wavefront's LDS tile `so` (16 rows of M + kStagePad), so
// that each store instruction writes 1 KB of whole rows.  O points at the
// wavefront's first token; t0 and n count tokens from there.
template <int M>
__device__ __forceinline__ void store_tile_bf16(bf16 *__restrict__ O, int t0, int n, const f32x4 (&Ot)[M / 16 + 1],
                                                lds_bf16 *so) {
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const float inv = __builtin_amdgcn_rcpf(Ot[M / 16][0]);
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt)
        *reinterpret_cast<lds_bf16x4 *>(so + c * (M + kStagePad) + 16 * mt + 4 * g) = IO<bf16>::from_f32(Ot[mt] * inv);
#pragma unroll
    for (int i = 0; i < M / 32; ++i) {
        const int e = (64 * i + lane) * 8, row = e / M, col = e % M;
        const dwordx4 y = *reinterpret_cast<const lds_dwordx4 *>(so + row * (M + kStagePad) + col);
        const uint32_t t = uint32_t(t0 + row);
        if (t < uint32_t(n))
            *reinterpret_cast<dwordx4 *>(reinterpret_cast<char *>(O) + (t * uint32_t(2 * M) + uint32_t(2 * col))) = y;
    }
}

// Same products as above; the chunk's rows are fetched with contiguous
// 16-byte loads, the feature map is applied in registers, and the rows are
// staged in the wavefront's LDS area, from which the natural and the
// token-contiguous fragments are read.  Global addresses are 32-bit element
// offsets from the wavefront's first token (a sub-segment spans far fewer
// than 2^31 / 64 tokens), so each load or store costs one address add.

template <int D, int M, int PF, bool PHI = true>
__device__ __forceinline__ void seg_aggregate_bf16(const bf16 *__restrict__ K, const bf16 *__restrict__ V,
                                                   int64_t t_begin, int64_t t_end, f32x4 (&St)[D / 16][M / 16 + 1],
                                                   lds_bf16 *sk, lds_bf16 *sv) {
    // The chunks are visited last to first, so that the wavefront's first
    // chunks are the most recently read when its output pass starts with them
    // (and are often still in L2).  Step s visits chunk nch - 1 - s; steps
    // past the first chunk (s >= nch) re-read chunk 0 and add nothing.
    static_assert(TT == 1, "16-row chunks");
    constexpr int NK = Lines<D, TT>::n, NV = Lines<M, TT>::n;
    // loads are relative to row tb and clamped to its n rows; an empty range
    // (t_begin == t_end) keeps a valid row to load and has no chunks
    const int64_t tb = imin64(t_begin, t_end - 1);
    const bf16 *Kw = K + tb * D, *Vw = V + tb * M;
    const int n = int(t_end - tb), nch = int((t_end - t_begin + CH - 1) / CH);
    auto chunk = [&](int step) { return max(nch - 1 - step, 0) * CH; };
    dwordx4 rk[PF][NK], rv[PF][NV];
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        load_rows32<D>(rk[b], Kw, chunk(b), n);
        load_rows32<M>(rv[b], Vw, chunk(b), n);
    }
    for (int s0 = 0; s0 < nch; s0 += PF) {
#pragma unroll
        for (int b = 0; b < PF; ++b) {
            const int step = s0 + b, t0 = chunk(step);
            if (step < nch) {   // uniform
                stage_lines<D, TT, PHI, true>(sk, rk[b], t0, n);   // rows past the end masked
                stage_lines<M, TT, false>(sv, rv[b], t0, n);
            }
            load_rows32<D>(rk[b], Kw, chunk(step + PF), n);
            load_rows32<M>(rv[b], Vw, chunk(step + PF), n);
            __builtin_amdgcn_sched_barrier(0);
            if (step < nch) {
                bf16x4 KT[TT][D / 16], VT[TT][M / 16];
                transposed_frags_lds<D, TT>(KT, sk);
                transposed_frags_lds<M, TT>(VT, sv);
                state_accumulate<bf16x4, D, M, TT, true>(St, KT, VT);
            }
        }
    }
}

// The rows of the first PF chunks of seg_output_bf16, loaded ahead (the
// causal forward issues them before its cross-workgroup hand-off, while the
// memory system is idle).
template <int D, int M, int PF> struct OutAhead {
    dwordx4 rq[PF][Lines<D, TT>::n], rk[PF][Lines<D, TT>::n], rv[PF][Lines<M, TT>::n];
    template <bool CAUSAL>
    __device__ __forceinline__ void load(const bf16 *Q, const bf16 *K, const bf16 *V, int64_t t_begin,
                                         int64_t t_end) {
        const int64_t tb = imin64(t_begin, t_end - 1);   // an empty range loads a valid row
        const int n = int(t_end - tb);
#pragma unroll
        for (int b = 0; b < PF; ++b) {
            load_rows32<D>(rq[b], Q + tb * D, b * CH, n);
            if (CAUSAL) {
                load_rows32<D>(rk[b], K + tb * D, b * CH, n);
                load_rows32<M>(rv[b], V + tb * M, b * CH, n);
            }
        }
    }
};

template <int D, int M, bool CAUSAL, int PF, bool PHI = true>
__device__ __forceinline__ void seg_output_bf16(const bf16 *__restrict__ Q, const bf16 *__restrict__ K,
                                                const bf16 *__restrict__ V, bf16 *__restrict__ O, int64_t t_begin,
                                                int64_t t_end, f32x4 (&St)[D / 16][M / 16 + 1], lds_bf16 *sq,
                                                lds_bf16 *sk, lds_bf16 *sv, lds_bf16 *so, OutAhead<D, M, PF> &ahead) {
    typedef bf16x4 Fr;
    constexpr int DT = D / 16, MT = M / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const Fr ones = frag_ones<Fr>();
    const Fr zero = frag_zero<Fr>();

    static_assert(TT == 1, "16-row chunks");
    auto &rq = ahead.rq;
    auto &rk = ahead.rk;
    auto &rv = ahead.rv;
    // as in seg_aggregate_bf16: rows relative to tb (an empty range has no chunks)
    const int64_t tb = imin64(t_begin, t_end - 1);
    const bf16 *Qw = Q + tb * D, *Kw = K + tb * D, *Vw = V + tb * M;
    bf16 *Ow = O + tb * M;
    const int n = int(t_end - tb), len = int(t_end - t_begin);
    for (int t00 = 0; t00 < len; t00 += PF * CH) {
#pragma unroll
    for (int b = 0; b < PF; ++b) {
        const int t0 = t00 + b * CH;   // may lie past the end: fully masked, no stores
        // no row masks: rows past the end hold copies of the last valid row (finite),
        // their outputs are not stored, the causal mask keeps them out of every
        // stored output, and the state is not used after the last chunk
        stage_lines<D, TT, PHI, false>(sq, rq[b], t0, n);
        if (CAUSAL) {
            stage_lines<D, TT, PHI, false>(sk, rk[b], t0, n);
            stage_lines<M, TT, false, false>(sv, rv[b], t0, n);
        }
        load_rows32<D>(rq[b], Qw, t0 + PF * CH, n);
        if (CAUSAL) {
            load_rows32<D>(rk[b], Kw, t0 + PF * CH, n);
            load_rows32<M>(rv[b], Vw, t0 + PF * CH, n);
        }
        __builtin_amdgcn_sched_barrier(0);
        Fr Qn[TT][DT];
        natural_frags_lds<D, TT>(Qn, sq);

        f32x4 Ot[MT + 1][TT];
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
            for (int it = 0; it < TT; ++it) Ot[mt][it] = f32x4{0.f, 0.f, 0.f, 0.f};

        // readout against the state carried in from earlier tokens
#pragma unroll
        for (int mt = 0; mt <= MT; ++mt) {
            Fr SF[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) SF[dt] = IO<bf16>::to_frag(St[dt][mt]);
#pragma unroll
            for (int it = 0; it < TT; ++it)
#pragma unroll
                for (int dt = 0; dt < DT; dt += 2) mma2(Ot[mt][it], SF[dt], SF[dt + 1], Qn[it][dt], Qn[it][dt + 1]);
        }

        if (CAUSAL) {
            Fr Kn[TT][DT], KT[TT][DT], VT[TT][MT];
            natural_frags_lds<D, TT>(Kn, sk);
            transposed_frags_lds<D, TT>(KT, sk);
            transposed_frags_lds<M, TT>(VT, sv);
            // P^T tiles (keys x queries), causal mask inside the diagonal tiles
            Fr PT[TT][TT];
#pragma unroll
            for (int it = 0; it < TT; ++it)
#pragma unroll
                for (int jt = 0; jt < TT; ++jt) {
                    if (jt > it) {
                        PT[jt][it] = zero;
                        continue;
                    }
                    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int dt = 0; dt < DT; dt += 2) mma2(p, Kn[jt][dt], Kn[jt][dt + 1], Qn[it][dt], Qn[it][dt + 1]);
                    if (jt == it) {
#pragma unroll
                        for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
                    }
                    PT[jt][it] = IO<bf16>::to_frag(p);
                }
            // intra-chunk term; the ones block sums P^T into den (every row)
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
                for (int it = 0; it < TT; ++it) {
                    Fr a[TT], b[TT];
#pragma unroll
                    for (int jt = 0; jt < TT; ++jt) {
                        a[jt] = (mt < MT) ? VT[jt][mt] : ones;
                        b[jt] = PT[jt][it];
                    }
                    mma_tiles<Fr, TT>(Ot[mt][it], a, b);
                }
            state_accumulate<Fr, D, M, TT, true>(St, KT, VT);
        }

        // normalize and store (every row of the normalizer block holds den)
#pragma unroll
        for (int it = 0; it < TT; ++it) {
            f32x4 tile[MT + 1];
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt) tile[mt] = Ot[mt][it];
            store_tile_bf16<M>(Ow, t0 + 16 * it, n, tile, so);
        }
    }
    }
}

// ---- per-segment kernel (the backward's forward-direction states) -----------
// Record of segment `seg`: sum over its tokens of phi(K_t) [V_t, 1]^T,
// written with state_store.  kSegWaves wavefronts share a segment: wave w
// sums the w-th run of whole chunks, then the partial states are added
// through LDS in wavefront order (a fixed order: results do not vary from
// run to run), so that two wavefronts per SIMD keep K and V streaming.
// The kernel holds no output tiles, so bf16 chunks are loaded four ahead of
// the one being summed (two ahead in the forward's passes).
constexpr int kSegWaves = 2;
constexpr int kSegPrefetch = 4;
template <typename T, int D, int M>
__global__ __launch_bounds__(64 * kSegWaves) void k_segment_state(const T *__restrict__ k, const T *__restrict__ v,
                                                                  float *__restrict__ ws, int64_t N, int64_t nseg,
                                                                  int64_t seg_tokens, int64_t rec) {
    static_assert(kSegWaves == 2, "the partial states are combined pairwise");
    // fp32 runs on split operands (split4), whose transposes take two LDS areas
    typedef typename std::conditional<sizeof(T) == 4, split4, typename IO<T>::frag>::type Fr;
    constexpr int SK = transpose_stage_elems<Fr, D / 16, TT>(), SV = transpose_stage_elems<Fr, M / 16, TT>();
    constexpr int STG = SK + SV;   // bf16 per wavefront
    constexpr int NTILE = (D / 16) * (M / 16 + 1);
    constexpr int STAGE_BYTES = kSegWaves * STG * int(sizeof(bf16));
    constexpr int SLOT_BYTES = NTILE * 64 * int(sizeof(f32x4));   // one wavefront's St, lane-major
    __shared__ __align__(16) unsigned char lds_raw[STAGE_BYTES > SLOT_BYTES ? STAGE_BYTES : SLOT_BYTES];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = lane_id();
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t s_begin = seg * seg_tokens, s_end = imin64(N, s_begin + seg_tokens);
    const int64_t nch = (s_end - s_begin + kChunk - 1) / kChunk;
    const int64_t cpw = (nch + kSegWaves - 1) / kSegWaves;   // chunks per wavefront
    const int64_t t_begin = imin64(s_end, s_begin + wave * cpw * kChunk);
    const int64_t t_end = imin64(s_end, t_begin + cpw * kChunk);
    lds_bf16 *sk = (lds_bf16 *)(reinterpret_cast<bf16 *>(lds_raw) + wave * STG);
    lds_bf16 *sv = sk + SK;
    f32x4 St[D / 16][M / 16 + 1];
    state_zero<D, M>(St);
    if (t_begin < t_end) {   // uniform; a short segment can leave wavefront 1 without chunks
        if constexpr (sizeof(T) == 2)
            seg_aggregate_bf16<D, M, kSegPrefetch>(k + bh * N * D, v + bh * N * M, t_begin, t_end, St, sk, sv);
        else
            seg_aggregate<T, D, M, fwd_prefetch<T, D, M>(), true, Fr>(k + bh * N * D, v + bh * N * M, t_begin, t_end,
                                                                    St, sk, sv);
    }
    __syncthreads();   // the staging areas are free
    f32x4 *slot = reinterpret_cast<f32x4 *>(lds_raw);
    if (wave == 1) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int mt = 0; mt <= M / 16; ++mt) slot[(dt * (M / 16 + 1) + mt) * 64 + lane] = St[dt][mt];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
            for (int mt = 0; mt <= M / 16; ++mt) St[dt][mt] += slot[(dt * (M / 16 + 1) + mt) * 64 + lane];
        state_store<D, M>(ws + (bh * nseg + seg) * rec, St);
    }
}

// ---- scan over segments ---------------------------------------------------
// Block = kScanCols float4 columns of the records x kScanG groups of
// consecutive segments (256 threads).  Each thread loads its group's values
// (all loads in flight at once: rows past the end read a valid record and are
// zeroed), sums them, the group sums are combined in LDS in group order, and
// the prefixes are written back.  The summation order depends only on nseg.
constexpr int kScanG = 8;
constexpr int kScanCols = 32;
constexpr int kScanRows = int(kMaxSegPerHead / kScanG);

// ROWS >= the rows of a group (per = ceil(nseg / kScanG)); the host picks the
// smallest power of two, so no thread issues loads for rows it does not have
// and the register count follows the segment count.
template <int ROWS>
__global__ __launch_bounds__(256) void k_state_scan(float *__restrict__ ws, int64_t nseg, int64_t rec, int mode,
                                                    ScanIO io) {
    // mode 0: exclusive prefix in place; 1: total into record 0 (non-causal);
    // 2: exclusive suffix in place (scan from the last segment backwards).
    // io: an optional start state added to every prefix (mode 0) and the
    // final state (start + total), each as S [srec] and Z [rec - srec].
    __shared__ f32x4 part[kScanG][kScanCols];
    const int cl = threadIdx.x % kScanCols, grp = threadIdx.x / kScanCols;
    const int64_t rec4 = rec / 4, s4 = io.srec / 4;
    const int64_t nblk_c = (rec4 + kScanCols - 1) / kScanCols;
    const int64_t bh = blockIdx.x / nblk_c;
    const int64_t c4 = (blockIdx.x % nblk_c) * kScanCols + cl;
    const bool ok = c4 < rec4;
    const bool rev = mode == 2;
    const int per = int((nseg + kScanG - 1) / kScanG);
    const int s0 = grp * per;                        // position in scan order
    const int nrow = max(0, min(per, int(nseg) - s0));   // rows this group has
    f32x4 *base = reinterpret_cast<f32x4 *>(ws + bh * nseg * rec) + (ok ? c4 : 0);
    // row j of the group is record (rev ? nseg - 1 - (s0 + j) : s0 + j): a
    // fixed step of +-rec4 float4s from the group's first record (a group
    // without rows, s0 >= nseg, points at the last valid one and stores nothing)
    const int sc = min(s0, int(nseg) - 1);
    f32x4 *first = base + (rev ? nseg - 1 - sc : sc) * rec4;
    const int64_t step = rev ? -rec4 : rec4;

    // the start state is read before any thread writes the final state (they
    // may be the same memory)
    f32x4 init = {0.f, 0.f, 0.f, 0.f};
    if (ok && io.s0)
        init = c4 < s4 ? reinterpret_cast<const f32x4 *>(io.s0 + bh * io.srec)[c4]
                       : reinterpret_cast<const f32x4 *>(io.z0 + bh * (rec - io.srec))[c4 - s4];
    f32x4 x[ROWS];
#pragma unroll
    for (int j = 0; j < ROWS; ++j)   // all loads in flight first; rows past the group's end read its last row
        x[j] = first[int64_t(min(j, max(nrow - 1, 0))) * step];
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < ROWS; ++j) {
        if (j >= nrow) x[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        sum += x[j];
    }
    part[grp][cl] = sum;
    __syncthreads();
    f32x4 run = init;
    f32x4 total = run;
    for (int p = 0; p < kScanG; ++p) {
        if (p < grp) run += part[p][cl];
        total += part[p][cl];
    }
    if (!ok) return;
    if (mode != 1) {
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            if (j < nrow) {
                first[int64_t(j) * step] = run;
                run += x[j];
            }
        }
    } else if (grp == 0) {
        base[0] = total;
    }
    if (io.s1 && grp == 0) {
        if (c4 < s4) reinterpret_cast<f32x4 *>(io.s1 + bh * io.srec)[c4] = total;
        else reinterpret_cast<f32x4 *>(io.z1 + bh * (rec - io.srec))[c4 - s4] = total;
    }
}

hipError_t launch_scan(float *ws, int64_t BH, int64_t nseg, int64_t rec, int mode, hipStream_t s, ScanIO io) {
    if (rec % 4 != 0 || io.srec % 4 != 0 || nseg > kMaxSegPerHead) return hipErrorInvalidValue;
    const int64_t nblk = BH * ((rec / 4 + kScanCols - 1) / kScanCols);
    const int64_t per = (nseg + kScanG - 1) / kScanG;
    const dim3 grid{unsigned(nblk)}, block{256};
    if (per <= 1) hipLaunchKernelGGL(k_state_scan<1>, grid, block, 0, s, ws, nseg, rec, mode, io);
    else if (per <= 2) hipLaunchKernelGGL(k_state_scan<2>, grid, block, 0, s, ws, nseg, rec, mode, io);
    else if (per <= 4) hipLaunchKernelGGL(k_state_scan<4>, grid, block, 0, s, ws, nseg, rec, mode, io);
    else if (per <= 8) hipLaunchKernelGGL(k_state_scan<8>, grid, block, 0, s, ws, nseg, rec, mode, io);
    else if (per <= 16) hipLaunchKernelGGL(k_state_scan<16>, grid, block, 0, s, ws, nseg, rec, mode, io);
    else hipLaunchKernelGGL(k_state_scan<kScanRows>, grid, block, 0, s, ws, nseg, rec, mode, io);
    return hipGetLastError();
}

// ---- fused causal forward ---------------------------------------------------
//
// Workgroup = kFusedWaves wavefronts = one block of consecutive sub-segments
// of one (b, h); workgroup i is block i % nb of head i / nb.
//   1. each wavefront sums phi(K) [V, 1]^T over its sub-segment (fp32);
//   2. hand-off between the nb blocks of a head, through the workspace:
//      a. block s publishes its total A_s = A_w0 + A_w1 + ... (the last block
//         of the head publishes none: nobody needs it);
//      b. the record is cut into nb slices and block s owns slice s: once all
//         totals are out it forms, for its slice, the exclusive prefixes
//         P_t = A_0 + A_1 + ... + A_{t-1} of every block t (one running sum in
//         block order per element) and publishes them;
//      c. once every slice is out, block s reads its P_s.
//      Each element of each P_t is summed by one thread in a fixed order, so
//      results do not depend on timing.  A block moves 3 records and waits
//      twice, however many blocks precede it;
//   3. wavefront w starts from P_s + A_w0 + ... + A_{w-1} and writes its
//      outputs, re-reading its K, V (mostly from the memory-side cache).
// Records and flags move with device-coherent (agent-scope, sc1) loads and
// stores, which bypass the per-XCD caches that are not kept coherent with
// each other; a flag is stored only after the wavefront's record stores have
// completed (vmcnt 0), and records are loaded only after the flag has been
// seen.  No cache-wide write-back or invalidate is needed, so the hand-off
// does not disturb the other blocks' cached K, V.  Only wavefront 0 of a block
// stores records.  Every wait is bounded: a block that waited too long sets
// the error word and carries on, so every wavefront always exits.  All blocks
// of a head must be able to run at the same time (at most kMaxBlkPerHead
// blocks of kFusedWaves wavefronts); the chip holds hundreds.
constexpr int kWaitVmcnt0 = 0x0f70;   // s_waitcnt vmcnt(0), other counters untouched

__device__ __forceinline__ void dev_store(f32x4 *p, f32x4 x) {
    unsigned long long *u = reinterpret_cast<unsigned long long *>(p);
    __hip_atomic_store(u, __builtin_bit_cast(unsigned long long, f32x2{x[0], x[1]}), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(u + 1, __builtin_bit_cast(unsigned long long, f32x2{x[2], x[3]}), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x4 dev_load(const f32x4 *p) {
    const unsigned long long *u = reinterpret_cast<const unsigned long long *>(p);
    const f32x2 a = __builtin_bit_cast(f32x2, __hip_atomic_load(u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    const f32x2 b = __builtin_bit_cast(f32x2, __hip_atomic_load(u + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    return f32x4{a[0], a[1], b[0], b[1]};
}

// Flags are 64-bit words: a flag is set for this call when it holds the
// call's tag, a value the host draws fresh for every call (never 0), so the
// flags need no clearing between calls and stale or uninitialized words do
// not read as set.

// Whole workgroup: every thread's earlier stores complete, then one thread
// stores the tag into *flag.
__device__ __forceinline__ void block_publish(unsigned long long *flag, unsigned long long tag) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");   // the compiler keeps the stores above
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);                  // the hardware completes them
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(flag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wavefront-wide wait until flags[0 .. count) all hold tag (count <= 64).
// At most `limit` polls: a wait that gives up or-s 1 into *err (the results
// are then wrong, and the error word says so) and lets the block carry on,
// so every wavefront always exits; limit 0 gives up at once.
__device__ __forceinline__ void wait_flags(const unsigned long long *flags, int count, unsigned long long tag,
                                           int *err, int64_t limit) {
    const int lane = lane_id();
    if (count > 0) {
        for (int64_t iter = 0;; ++iter) {
            if (iter >= limit) {
                if (lane == 0) atomicOr(err, 1);
                break;
            }
            const bool set = (lane >= count) ||
                             __hip_atomic_load(&flags[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag;
            if (__ballot(!set) == 0) break;
            __builtin_amdgcn_s_sleep(2);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // later loads stay below (compiler)
}

// Zeroes the hand-off flags of a call that is being captured into a graph:
// its tag is fixed at capture, so the flags a replay waits for must not
// still hold it from the replay before.  A kernel rather than a memset node.
__global__ __launch_bounds__(256) void k_clear_flags(unsigned long long *__restrict__ flags, int64_t n) {
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) flags[i] = 0;
}

// PHI = false: q and k hold the features already (no feature map applied).
// CAUSAL = false: the non-causal forward -- every block publishes its total,
// the slice owners form the head's full sum (one record), and every
// wavefront reads its queries out against it.
template <typename T, int D, int M, bool PHI, bool CAUSAL = true>
__global__ __launch_bounds__(64 * kFusedWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_fwd_fused(const T *__restrict__ q, const T *__restrict__ k,
                                                                const T *__restrict__ v, T *__restrict__ out,
                                                                int *__restrict__ header,
                                                                unsigned long long *__restrict__ flags,
                                                                unsigned long long tag,
                                                                float *__restrict__ recs, int64_t N, int64_t nblk,
                                                                int64_t sub_tokens, int64_t limit, StateIO sio) {
    constexpr int REC = D * M + D, REC4 = REC / 4;
    static_assert(REC % 4 == 0, "records move as f32x4");
    constexpr int NT = 64 * kFusedWaves;
    // LDS: per-wavefront staging (q, k, v chunks) during the two passes; during
    // the hand-off the same bytes hold one slot per wavefront: slot w >= 1 the
    // partial sum A_w0 + ... + A_{w-1}, slot 0 the block total, then the
    // group sums of the prefix slice being formed, then the block's own
    // prefix P_s.
    constexpr int SK = stage_elems<D / 16, TT>(), SV = stage_elems<M / 16, TT>(), SO = 16 * (M + kStagePad);
    constexpr int SW = 2 * SK + SV + SO;   // per wavefront: q, k, v chunks and one output tile
    constexpr int STAGE_BYTES = kFusedWaves * SW * int(sizeof(bf16));
    constexpr int SLOT4 = REC4 + int(kMaxBlkPerHead);
    constexpr int SLOT_BYTES = kFusedWaves * SLOT4 * int(sizeof(f32x4));
    __shared__ __align__(16) unsigned char lds_raw[STAGE_BYTES > SLOT_BYTES ? STAGE_BYTES : SLOT_BYTES];
    bf16 *lds_stage = reinterpret_cast<bf16 *>(lds_raw);
    f32x4 *slot4 = reinterpret_cast<f32x4 *>(lds_raw);
    auto slot = [&](int w) { return reinterpret_cast<float *>(slot4 + w * SLOT4); };
    float *pbuf = slot(0);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar loop control

    const int64_t bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
    const int nb = int(nblk), sb = int(blk);
    const int64_t t_begin = min(N, (blk * kFusedWaves + wave) * sub_tokens);
    const int64_t t_end = min(N, t_begin + sub_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    unsigned long long *flag_tot = flags + bh * 2 * nblk;   // [nblk]: total published
    unsigned long long *flag_pre = flag_tot + nblk;         // [nblk]: prefix slice published
    float *head_recs = recs + bh * nblk * 2 * REC;   // per block: total, exclusive prefix

    // 1. local totals
    f32x4 St[D / 16][M / 16 + 1];
    state_zero<D, M>(St);
    lds_bf16 *stage_q = (lds_bf16 *)(lds_stage + wave * SW);
    lds_bf16 *stage_k = stage_q + SK;
    lds_bf16 *stage_v = stage_k + SK;
    // fp32 I/O (split into bf16 parts): the same area holds the two K tiles
    // from stage_q on, then the two V tiles
    static_assert(2 * SK + 2 * SV <= SW, "split fp32 tiles fit the wavefront's staging area");
    lds_bf16 *stage_f32v = stage_q + 2 * SK;
    if constexpr (sizeof(T) == 2)
        seg_aggregate_bf16<D, M, kPrefetch, PHI>(K, V, t_begin, t_end, St, stage_k, stage_v);
    else
        seg_aggregate<T, D, M, fwd_prefetch<T, D, M>(), PHI, split4>(K, V, t_begin, t_end, St, stage_q, stage_f32v);
    __syncthreads();   // every wavefront is done with its staging area
    state_store_frag<D, M>(slot(wave), St);
    __syncthreads();

    // pass 2's first chunks, loaded while the workgroups exchange their state
    typename std::conditional<sizeof(T) == 2, OutAhead<D, M, kPrefetch>,
                              ChunkAhead<T, D, M, fwd_prefetch<T, D, M>()>>::type ahead;
    ahead.template load<CAUSAL>(Q, K, V, t_begin, t_end);

    // Initial state (zero unless given), this thread's record elements.  Read
    // here, before the block publishes anything: the last block of the head
    // writes the final state only after every block has published, so the
    // two may share memory.
    constexpr int NJ4 = (REC4 + NT - 1) / NT;
    f32x4 init[NJ4];
#pragma unroll
    for (int j = 0; j < NJ4; ++j) {
        const int i4 = tid + NT * j;
        init[j] = (sio.s0 && i4 < REC4) ? record_frag4_load<D, M>(sio.s0 + bh * D * M, sio.z0 + bh * D, i4)
                                        : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // 2a. in place: slot w = A_w0 + ... + A_{w-1} for w >= 1, slot 0 = the
    // block total A_s (wavefront 0's partial sum is zero)
#pragma unroll
    for (int j = 0; j < NJ4; ++j) {   // as f32x4: four elements per LDS access
        const int e = tid + NT * j;
        if (e < REC4) {
            f32x4 run = slot4[e];
#pragma unroll
            for (int w = 1; w < kFusedWaves; ++w) {
                const f32x4 x = slot4[w * SLOT4 + e];
                if (CAUSAL) slot4[w * SLOT4 + e] = run;
                run += x;
            }
            slot4[e] = run;
        }
    }
    __syncthreads();
    // the last block keeps its total for the final state (the slice scan
    // below reuses slot 0 as scratch)
    const bool last = sio.s1 != nullptr && sb == nb - 1;
    f32x4 tot[NJ4];
#pragma unroll
    for (int j = 0; j < NJ4; ++j)
        tot[j] = (last && tid + NT * j < REC4) ? slot4[tid + NT * j] : f32x4{0.f, 0.f, 0.f, 0.f};
    if (nb > 1 && (!CAUSAL || sb < nb - 1)) {   // every thread stores a share of the total
        f32x4 *dst = reinterpret_cast<f32x4 *>(head_recs + blk * 2 * REC);
#pragma unroll
        for (int j = 0; j < (REC4 + NT - 1) / NT; ++j)
            if (tid + NT * j < REC4) dev_store(dst + tid + NT * j, slot4[tid + NT * j]);
        block_publish(&flag_tot[blk], tag);
    }
    // With few blocks per head each block sums the totals it needs itself (one
    // exchange); otherwise the slices below form the prefixes (two exchanges,
    // but a block reads 3 records however many precede it).
    const bool direct = nb <= kFusedDirectBlocks;
    if (wave == 0 && nb > 1) wait_flags(flag_tot, CAUSAL ? (direct ? sb : nb - 1) : nb, tag, &header[1], limit);
    __syncthreads();

    if (nb > 1 && !direct) {
        // 2b. this block's slice [c0, c0 + ncol) of every prefix P_1 .. P_{nb-1}.
        // Work unit (column cc, row group g): rows g R .. g R + R - 1 of the
        // nr = nb - 1 totals; a unit sums its rows, the group sums go through
        // LDS, and each row's prefix is (sum of the earlier groups) + (running
        // sum within the group) -- a fixed order for every element.
        const int nr = CAUSAL ? nb - 1 : nb;   // non-causal: every total, summed into one record
        const int per = (REC4 + nb - 1) / nb;
        const int c0 = min(REC4, sb * per), ncol = min(REC4, c0 + per) - c0;
        const int G = ncol > 0 ? max(1, min(nr, NT / max(ncol, 1))) : 1;
        const int R = (nr + G - 1) / G;
        constexpr int RMAX = kFusedSliceRows;   // R <= RMAX (checked on the host)
        f32x4 *gsum = slot4;      // [G][ncol] group sums, in slot 0
        f32x4 run[RMAX];
        for (int u0 = 0; u0 < ncol * G; u0 += NT) {   // one pass unless ncol > NT
            const int u = u0 + tid;
            const bool on = u < ncol * G;
            const int g = on ? u / ncol : 0, cc = on ? u - g * ncol : 0;
            const int r0 = g * R;
            const f32x4 *col = reinterpret_cast<const f32x4 *>(head_recs) + c0 + cc;
#pragma unroll
            for (int k = 0; k < RMAX; ++k)   // all loads in flight first
                run[k] = (on && k < R && r0 + k < nr) ? dev_load(col + int64_t(r0 + k) * 2 * REC4)
                                                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 1; k < RMAX; ++k) run[k] += run[k - 1];
            if (on) gsum[g * ncol + cc] = run[RMAX - 1];
            __syncthreads();
            if (!CAUSAL) {   // the head's total, at block 0's prefix slot
                if (on && g == 0) {
                    f32x4 tot4 = gsum[cc];
                    for (int h = 1; h < G; ++h) tot4 += gsum[h * ncol + cc];
                    dev_store(reinterpret_cast<f32x4 *>(head_recs + REC) + c0 + cc, tot4);
                }
            } else if (on) {
                f32x4 off = {0.f, 0.f, 0.f, 0.f};
                for (int h = 0; h < g; ++h) off += gsum[h * ncol + cc];
                f32x4 *dst = reinterpret_cast<f32x4 *>(head_recs + 3 * REC) + c0 + cc;   // prefix of block r + 1
#pragma unroll
                for (int k = 0; k < RMAX; ++k)
                    if (k < R && r0 + k < nr) dev_store(dst + int64_t(r0 + k) * 2 * REC4, (g > 0 ? off + run[k] : run[k]));
            }
            __syncthreads();
        }
        block_publish(&flag_pre[blk], tag);
        if (wave == 0 && (sb > 0 || !CAUSAL)) wait_flags(flag_pre, nb, tag, &header[1], limit);
        __syncthreads();
    }
    // 2c. P_s = initial state + the earlier blocks' totals into LDS; the last
    // block also forms the final state P_s + A_s
    {
        // causal: P_s (zero for the first block); non-causal: the head's total
        // (a single block already holds it in slot 0)
        const f32x4 *src = reinterpret_cast<const f32x4 *>(head_recs + (CAUSAL ? blk * 2 + 1 : 1) * REC);
        const bool fetch = CAUSAL ? sb > 0 : nb > 1;
        f32x4 buf[NJ4];
        if (direct && fetch) {
            // the totals of blocks 0 .. sb - 1 (non-causal: all nb), summed in block order
            const int nsum = CAUSAL ? sb : nb;
            const f32x4 *tot0 = reinterpret_cast<const f32x4 *>(head_recs);
            // in batches of 4 totals, all loads of a batch in flight first; the
            // second batch only for blocks with more than 4 predecessors (uniform)
            static_assert(kFusedDirectBlocks % 4 == 0, "batches of 4 totals");
#pragma unroll
            for (int r0 = 0; r0 < kFusedDirectBlocks; r0 += 4) {
                if (r0 > 0 && nsum <= r0) break;
#pragma unroll
                for (int j = 0; j < NJ4; ++j) {
                    f32x4 x[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        x[r] = (r0 + r < nsum && tid + NT * j < REC4)
                                   ? dev_load(tot0 + int64_t(r0 + r) * 2 * REC4 + tid + NT * j)
                                   : f32x4{0.f, 0.f, 0.f, 0.f};
                    if (r0 == 0) buf[j] = x[0];
                    else buf[j] += x[0];
#pragma unroll
                    for (int r = 1; r < 4; ++r) buf[j] += x[r];
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NJ4; ++j)
                buf[j] = fetch ? (tid + NT * j < REC4 ? dev_load(src + tid + NT * j) : f32x4{0.f, 0.f, 0.f, 0.f})
                               : (CAUSAL || tid + NT * j >= REC4 ? f32x4{0.f, 0.f, 0.f, 0.f} : slot4[tid + NT * j]);
        }
#pragma unroll
        for (int j = 0; j < NJ4; ++j) {
            const int i4 = tid + NT * j;
            if (i4 < REC4) {
                const f32x4 p = buf[j] + init[j];
                if (last) buf[j] = p + tot[j];
                reinterpret_cast<f32x4 *>(pbuf)[i4] = p;
            }
        }
        if (last) {
#pragma unroll
            for (int j = 0; j < NJ4; ++j)
                if (tid + NT * j < REC4) record_frag4_store<D, M>(sio.s1 + bh * D * M, sio.z1 + bh * D, tid + NT * j, buf[j]);
        }
    }
    __syncthreads();

    // 3. outputs, starting from P_s + the totals of the earlier wavefronts
    // (non-causal: from the head's total)
    state_load_frag2<D, M>(St, pbuf, (CAUSAL && wave > 0) ? slot(wave) : nullptr);
    __syncthreads();   // the prefix is read: the staging area is free again
    if constexpr (sizeof(T) == 2)
        seg_output_bf16<D, M, CAUSAL, kPrefetch, PHI>(Q, K, V, out + bh * N * M, t_begin, t_end, St, stage_q,
                                                      stage_k, stage_v, stage_v + SV, ahead);
    else
        seg_output<T, D, M, CAUSAL, fwd_prefetch<T, D, M>(), PHI, split4>(Q, K, V, out + bh * N * M, t_begin, t_end,
                                                                        St, stage_q, stage_f32v, ahead);
}

// ---- host side ---------------------------------------------------------------
uint64_t next_call_tag() {
    static const uint64_t seed =
        uint64_t(std::chrono::steady_clock::now().time_since_epoch().count()) ^ uint64_t(uintptr_t(&seed));
    static std::atomic<uint64_t> count{0};
    uint64_t z = seed + 0x9E3779B97F4A7C15ull * (count.fetch_add(1, std::memory_order_relaxed) + 1);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;   // splitmix64 finalizer: a bijection
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return z ? z : 1;
}

constexpr int64_t kDefaultWaitLimit = int64_t(1) << 20;   // about a second of polling
static std::atomic<int64_t> g_wait_limit{kDefaultWaitLimit};
int64_t wait_limit() { return g_wait_limit.load(std::memory_order_relaxed); }
int64_t set_wait_limit(int64_t polls) {
    return g_wait_limit.exchange(polls < 0 ? kDefaultWaitLimit : polls, std::memory_order_relaxed);
}

// Scratch of la_forward_causal_noalloc: the workspace of its causal forward
// (header, hand-off flags, state records), owned by the library, one copy per
// GPU, held until the process ends.  The flags are tagged per call and never
// need clearing; calls that overlap on one GPU share it and race.  In host
// code `scratch` is only a stand-in for the symbol: its device address on the
// current device comes from hipGetSymbolAddress (cached per device) and is
// the only thing ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

void *noalloc_scratch() {
    constexpr int kMaxDevices = 64;
    static std::atomic<void *> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (p != nullptr) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    cache[dev].store(p, std::memory_order_release);
    return p;
}

int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// A plan the fused kernel cannot run (too many record rows for one thread to
// sum while forming a prefix slice, or a wavefront's rows past 32-bit byte
// offsets) -- a limit of this implementation, checked before any launch.
bool forward_plan_supported(int64_t BH, int64_t N, int64_t D, int64_t M, size_t esize) {
    const FusedPlan p = make_fused_plan(BH, N, D, M);
    for (int causal = 0; causal < 2; ++causal)
        if (fused_slice_rows(p.nblk, causal ? p.nblk - 1 : p.nblk, (D * M + D) / 4, 64 * kFusedWaves) >
            kFusedSliceRows)
            return false;
    // the bf16 chunk loops address a wavefront's rows by 32-bit byte offsets
    // (far from binding: a wavefront's share of any problem that fits in memory
    // spans well under 1 GB)
    return (p.sub_tokens + 2 * kChunk) * std::max(D, M) * int64_t(esize) <= int64_t(UINT32_MAX);
}

template <typename T, int D, int M>
static hipError_t run_forward(bool causal, const void *q, const void *k, const void *v, void *out, int64_t BH,
                              int64_t N, float *ws, StateIO sio, hipStream_t s) {
    const FusedPlan p = make_fused_plan(BH, N, D, M);
    if (!forward_plan_supported(BH, N, D, M, sizeof(T))) return hipErrorInvalidValue;
    char *base = reinterpret_cast<char *>(ws);
    int *header = reinterpret_cast<int *>(base);
    unsigned long long *flags = reinterpret_cast<unsigned long long *>(base + p.flags_off);
    float *recs = reinterpret_cast<float *>(base + p.recs_off);
    // Under graph capture the tag below is fixed for every replay: the flags
    // are cleared by a kernel node first, so no replay sees its predecessor's.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) == hipSuccess && cap == hipStreamCaptureStatusActive) {
        const int64_t nflags = 2 * BH * p.nblk;
        const unsigned blocks = unsigned(std::min<int64_t>(1024, ceil_div(nflags, 256)));
        hipLaunchKernelGGL(k_clear_flags, dim3(blocks), dim3(256), 0, s, flags, nflags);
    }
    const unsigned long long tag = next_call_tag();
    const int64_t limit = wait_limit();
    const dim3 grid(unsigned(BH * p.nblk)), block(64 * kFusedWaves);
    if (!causal)
        hipLaunchKernelGGL((k_fwd_fused<T, D, M, true, false>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, header, flags, tag, recs, N, p.nblk, p.sub_tokens, limit, sio);
    else if (sio.features_given)
        hipLaunchKernelGGL((k_fwd_fused<T, D, M, false>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, header, flags, tag, recs, N, p.nblk, p.sub_tokens, limit, sio);
    else
        hipLaunchKernelGGL((k_fwd_fused<T, D, M, true>), grid, block, 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, header, flags, tag, recs, N, p.nblk, p.sub_tokens, limit, sio);
    return hipGetLastError();
}

template <typename T>
static hipError_t run_forward_t(bool causal, const void *q, const void *k, const void *v, void *out, int64_t BH,
                                int64_t N, int64_t D, int64_t M, float *ws, StateIO sio, hipStream_t s) {
    if (D == 32 && M == 32) return run_forward<T, 32, 32>(causal, q, k, v, out, BH, N, ws, sio, s);
    if (D == 32 && M == 64) return run_forward<T, 32, 64>(causal, q, k, v, out, BH, N, ws, sio, s);
    if (D == 64 && M == 32) return run_forward<T, 64, 32>(causal, q, k, v, out, BH, N, ws, sio, s);
    if (D == 64 && M == 64) return run_forward<T, 64, 64>(causal, q, k, v, out, BH, N, ws, sio, s);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out, int64_t BH,
                          int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s, StateIO sio) {
    if (!causal && (sio.s0 || sio.s1 || sio.features_given)) return hipErrorInvalidValue;
    if (dt == 0) return run_forward_t<float>(causal, q, k, v, out, BH, N, D, M, ws, sio, s);
    return run_forward_t<bf16>(causal, q, k, v, out, BH, N, D, M, ws, sio, s);
}

template <typename T>
static hipError_t run_segment_state_t(const void *k, const void *v, float *ws, int64_t BH, int64_t N, int64_t D,
                                      int64_t M, hipStream_t s) {
    const SegPlan p = make_plan(BH, N, D, M);
    const dim3 grid(unsigned(BH * p.nseg));
#define LA_SEGSTATE_CASE(DD, MM)                                                                                 \
    if (D == DD && M == MM) {                                                                                    \
        hipLaunchKernelGGL((k_segment_state<T, DD, MM>), grid, dim3(64 * kSegWaves), 0, s, (const T *)k,         \
                           (const T *)v, ws, N, p.nseg, p.seg_tokens, p.rec);                                    \
        return hipGetLastError();                                                                                \
    }
    LA_SEGSTATE_CASE(32, 32)
    LA_SEGSTATE_CASE(32, 64)
    LA_SEGSTATE_CASE(64, 32)
    LA_SEGSTATE_CASE(64, 64)
#undef LA_SEGSTATE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_segment_state(int dt, const void *k, const void *v, float *ws, int64_t BH, int64_t N, int64_t D,
                                int64_t M, hipStream_t s) {
    if (dt == 0) return run_segment_state_t<float>(k, v, ws, BH, N, D, M, s);
    return run_segment_state_t<bf16>(k, v, ws, BH, N, D, M, s);
}

} // namespace la
