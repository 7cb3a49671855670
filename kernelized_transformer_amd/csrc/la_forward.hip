// la_forward.hip -- chunked causal and non-causal forward on gfx950.
//
// Method ([deck] = zhengyuhong.cn "Transformers are RNNs ... 解读", slides
// 3-4; [summary] = paperlayer.ai summary, sections 3.2-3.3.2):
//   causal:     out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i, with the inclusive
//               prefix states S_i = sum_{j<=i} phi(K_j) V_j^T, Z_i = sum_{j<=i} phi(K_j);
//   non-causal: the same with S, Z summed over all tokens.
// The training-time form is evaluated in parallel over the sequence
// ([summary] 3.3.2): the sequence is cut into chunks of 32 tokens, and a
// chunk's outputs are
//   num_c = tril(phi(Q_c) phi(K_c)^T) V_c + phi(Q_c) S_prev,
//   den_c = tril(phi(Q_c) phi(K_c)^T) 1   + phi(Q_c) Z_prev,
// an exact regrouping of the prefix sums.  All products run on the matrix
// cores with fp32 accumulation, in transposed form (out^T = V^T P^T + S^T Q^T)
// so that every operand is either a plain row-major load or an accumulator
// tile reused in place (see la_device.h).
//
// Sequence parallelism: each (b, h) is cut into segments of whole chunks,
// one wavefront per segment.  Three launches:
//   1. k_segment_state: per segment, sum_t phi(K_t) [V_t, 1]^T  (fp32),
//   2. k_state_scan:    exclusive prefix of those records over segments,
//   3. k_segment_output: per segment, start from its prefix and walk the
//      chunks, writing out and carrying (S, Z) in fp32 registers.
#include "la_chunk.h"
#include "la_internal.h"

namespace la {

constexpr int TT = 2;        // token tiles per chunk in the forward kernels
constexpr int CH = 16 * TT;  // = kChunk
static_assert(CH == kChunk, "forward chunk");

// ---- 1. per-segment state ------------------------------------------------
template <typename T, int D, int M>
__global__ __launch_bounds__(64) void k_segment_state(const T *__restrict__ k, const T *__restrict__ v,
                                                      float *__restrict__ ws, int64_t N, int64_t nseg,
                                                      int64_t seg_tokens, int64_t rec) {
    typedef typename IO<T>::frag Fr;
    typedef typename IO<T>::vec4 V4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;

    f32x4 St[D / 16][M / 16 + 1];
    state_zero<D, M>(St);

    V4 rk[TT][D / 16], rv[TT][M / 16];
    load_chunk<T, D, TT>(rk, K, t_begin, t_end);
    load_chunk<T, M, TT>(rv, V, t_begin, t_end);
    for (int64_t t0 = t_begin; t0 < t_end; t0 += CH) {
        Fr Kn[TT][D / 16], Vn[TT][M / 16];
        phi_frags<T, D, TT>(Kn, rk, t0, t_end);
        raw_frags<T, M, TT>(Vn, rv);
        if (t0 + CH < t_end) {
            load_chunk<T, D, TT>(rk, K, t0 + CH, t_end);
            load_chunk<T, M, TT>(rv, V, t0 + CH, t_end);
        }
        Fr KT[TT][D / 16], VT[TT][M / 16];
        transpose_frags<Fr, D / 16, TT>(KT, Kn);
        transpose_frags<Fr, M / 16, TT>(VT, Vn);
        state_accumulate<Fr, D, M, TT>(St, KT, VT);
    }
    state_store<D, M>(ws + (bh * nseg + seg) * rec, St);
}

// ---- 2. scan over segments ----------------------------------------------
// Block = 64 record elements x 4 segment quarters (256 threads).  Each thread
// keeps its quarter's values in registers, the quarters' totals are combined
// in LDS, then the prefixes are written back.
constexpr int kScanQ = 4;
constexpr int kScanPerQ = int(kMaxSegPerHead / kScanQ);

__global__ __launch_bounds__(256) void k_state_scan(float *__restrict__ ws, int64_t nseg, int64_t rec, int mode,
                                                    const float *__restrict__ init, float *__restrict__ fin) {
    // mode 0: exclusive prefix in place; 1: total into record 0 (non-causal);
    // 2: exclusive suffix in place (scan from the last segment backwards).
    __shared__ float part[kScanQ][64];
    const int e_local = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t nblk_e = (rec + 63) / 64;
    const int64_t bh = blockIdx.x / nblk_e;
    const int64_t e = (blockIdx.x % nblk_e) * 64 + e_local;
    const bool ok = e < rec;
    const bool rev = mode == 2;
    const int64_t per_q = (nseg + kScanQ - 1) / kScanQ;
    const int64_t s0 = q * per_q;   // position in scan order
    float *base = ws + bh * nseg * rec + e;

    float x[kScanPerQ];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kScanPerQ; ++j) {
        const int64_t s = s0 + j;
        const int64_t seg = rev ? nseg - 1 - s : s;
        x[j] = (ok && j < per_q && s < nseg) ? base[seg * rec] : 0.f;
        sum += x[j];
    }
    part[q][e_local] = sum;
    __syncthreads();
    float run = (ok && init) ? init[bh * rec + e] : 0.f;
    float total = run;
    for (int p = 0; p < kScanQ; ++p) {
        if (p < q) run += part[p][e_local];
        total += part[p][e_local];
    }
    if (!ok) return;
    if (mode != 1) {
#pragma unroll
        for (int j = 0; j < kScanPerQ; ++j) {
            const int64_t s = s0 + j;
            const int64_t seg = rev ? nseg - 1 - s : s;
            if (j < per_q && s < nseg) {
                base[seg * rec] = run;
                run += x[j];
            }
        }
    } else if (q == 0) {
        base[0] = total;
    }
    if (fin && q == 0) fin[bh * rec + e] = total;
}

hipError_t launch_scan(float *ws, int64_t BH, int64_t nseg, int64_t rec, int mode, const float *init, float *fin,
                       hipStream_t s) {
    const int64_t nblk = BH * ((rec + 63) / 64);
    hipLaunchKernelGGL(k_state_scan, dim3(unsigned(nblk)), dim3(256), 0, s, ws, nseg, rec, mode, init, fin);
    return hipGetLastError();
}

// ---- 3. per-segment output -------------------------------------------------
// Per chunk (32 tokens = query tiles it, key tiles jt), with Acc tiles
// Ot[mt][it] = out^T (rows m, plus the normalizer row block), cols = queries:
//   readout:  Ot[mt][it] += S^T[m][d] phi(Q)[i][d]      (S from St, as is)
//   intra:    Ot[mt][it] += V^T[m][j] P^T[j][i], P^T[j][i] = phi(K_j).phi(Q_i), j <= i
//   update:   St += phi(K)^T [V, 1]
// The normalizer row block of Ot gets den_i in row 0.
template <typename T, int D, int M, bool CAUSAL>
__global__ __launch_bounds__(64) void k_segment_output(const T *__restrict__ q, const T *__restrict__ k,
                                                       const T *__restrict__ v, T *__restrict__ out,
                                                       const float *__restrict__ ws, int64_t N, int64_t nseg,
                                                       int64_t seg_tokens, int64_t rec) {
    typedef typename IO<T>::frag Fr;
    typedef typename IO<T>::vec4 V4;
    constexpr int DT = D / 16, MT = M / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens;
    const int64_t t_end = min(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    T *O = out + bh * N * M;

    f32x4 St[DT][MT + 1];
    state_load<D, M>(St, ws + (bh * nseg + (CAUSAL ? seg : 0)) * rec);

    const Fr ones = frag_row0_ones<Fr>();
    const Fr zero = frag_zero<Fr>();

    V4 rq[TT][DT], rk[TT][DT], rv[TT][MT];
    load_chunk<T, D, TT>(rq, Q, t_begin, t_end);
    if (CAUSAL) {
        load_chunk<T, D, TT>(rk, K, t_begin, t_end);
        load_chunk<T, M, TT>(rv, V, t_begin, t_end);
    }
    for (int64_t t0 = t_begin; t0 < t_end; t0 += CH) {
        Fr Qn[TT][DT], Kn[TT][DT], Vn[TT][MT];
        phi_frags<T, D, TT>(Qn, rq, t0, t_end);
        if (CAUSAL) {
            phi_frags<T, D, TT>(Kn, rk, t0, t_end);
            raw_frags<T, M, TT>(Vn, rv);
        }
        if (t0 + CH < t_end) {
            load_chunk<T, D, TT>(rq, Q, t0 + CH, t_end);
            if (CAUSAL) {
                load_chunk<T, D, TT>(rk, K, t0 + CH, t_end);
                load_chunk<T, M, TT>(rv, V, t0 + CH, t_end);
            }
        }

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
            for (int dt = 0; dt < DT; ++dt) SF[dt] = IO<T>::to_frag(St[dt][mt]);
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
                    PT[jt][it] = IO<T>::to_frag(p);
                }
            Fr KT[TT][DT], VT[TT][MT];
            transpose_frags<Fr, DT, TT>(KT, Kn);
            transpose_frags<Fr, MT, TT>(VT, Vn);
            // intra-chunk term; the ones row block sums P^T into den
#pragma unroll
            for (int mt = 0; mt <= MT; ++mt)
#pragma unroll
                for (int it = 0; it < TT; ++it) {
                    const Fr a0 = (mt < MT) ? VT[0][mt] : ones;
                    const Fr a1 = (mt < MT) ? VT[1][mt] : ones;
                    mma2(Ot[mt][it], a0, a1, PT[0][it], PT[1][it]);
                }
            state_accumulate<Fr, D, M, TT>(St, KT, VT);
        }

        // normalize and store: den_i sits in row 0 of the normalizer block,
        // i.e. element 0 of lane c (g = 0)
#pragma unroll
        for (int it = 0; it < TT; ++it) {
            const float den = __shfl(Ot[MT][it][0], c);
            const float inv = __builtin_amdgcn_rcpf(den);
            const int64_t t = t0 + 16 * it + c;
            if (t < t_end) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) store4<T>(O + t * M + 16 * mt + 4 * g, IO<T>::from_f32(Ot[mt][it] * inv));
            }
        }
    }
}

template <typename T, int D, int M>
static hipError_t run_forward(bool causal, const void *q, const void *k, const void *v, void *out, int64_t BH,
                              int64_t N, float *ws, hipStream_t s) {
    const SegPlan p = make_plan(BH, N, D, M);
    const dim3 grid(unsigned(BH * p.nseg));
    hipLaunchKernelGGL((k_segment_state<T, D, M>), grid, dim3(64), 0, s, (const T *)k, (const T *)v, ws, N, p.nseg,
                       p.seg_tokens, p.rec);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_scan(ws, BH, p.nseg, p.rec, causal ? 0 : 1, nullptr, nullptr, s);
    if (e != hipSuccess) return e;
    if (causal)
        hipLaunchKernelGGL((k_segment_output<T, D, M, true>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, (const float *)ws, N, p.nseg, p.seg_tokens, p.rec);
    else
        hipLaunchKernelGGL((k_segment_output<T, D, M, false>), grid, dim3(64), 0, s, (const T *)q, (const T *)k,
                           (const T *)v, (T *)out, (const float *)ws, N, p.nseg, p.seg_tokens, p.rec);
    return hipGetLastError();
}

template <typename T>
static hipError_t run_forward_t(bool causal, const void *q, const void *k, const void *v, void *out, int64_t BH,
                                int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s) {
    if (D == 32 && M == 32) return run_forward<T, 32, 32>(causal, q, k, v, out, BH, N, ws, s);
    if (D == 32 && M == 64) return run_forward<T, 32, 64>(causal, q, k, v, out, BH, N, ws, s);
    if (D == 64 && M == 32) return run_forward<T, 64, 32>(causal, q, k, v, out, BH, N, ws, s);
    if (D == 64 && M == 64) return run_forward<T, 64, 64>(causal, q, k, v, out, BH, N, ws, s);
    return hipErrorInvalidValue;
}

hipError_t launch_forward(bool causal, int dt, const void *q, const void *k, const void *v, void *out, int64_t BH,
                          int64_t N, int64_t D, int64_t M, float *ws, hipStream_t s) {
    if (dt == 0) return run_forward_t<float>(causal, q, k, v, out, BH, N, D, M, ws, s);
    return run_forward_t<bf16>(causal, q, k, v, out, BH, N, D, M, ws, s);
}

template <typename T>
static hipError_t run_segment_state_t(const void *k, const void *v, float *ws, int64_t BH, int64_t N, int64_t D,
                                      int64_t M, hipStream_t s) {
    const SegPlan p = make_plan(BH, N, D, M);
    const dim3 grid(unsigned(BH * p.nseg));
#define LA_SEGSTATE_CASE(DD, MM)                                                                                 \
    if (D == DD && M == MM) {                                                                                    \
        hipLaunchKernelGGL((k_segment_state<T, DD, MM>), grid, dim3(64), 0, s, (const T *)k, (const T *)v, ws, N, \
                           p.nseg, p.seg_tokens, p.rec);                                                         \
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
