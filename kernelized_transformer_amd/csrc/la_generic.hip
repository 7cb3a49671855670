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
// which fits every D up to 128.  Each wavefront applies the feature map to
// the whole of Q and K for its chunks and forms the chunk's D-deep products
// itself; the M / 16 wavefronts of a segment read the same Q, K rows (from
// the caches after the first).  Three launches: per-segment sums of
// phi(K) [V, 1]^T into row-major records (each wavefront its columns), the
// scan of la_forward.hip over segments (with the optional start state and
// final state), then the outputs.
#include <type_traits>

#include "la_chunk.h"
#include "la_internal.h"

namespace la {

namespace {

constexpr int GCH = 16;   // tokens per chunk
// chunks in flight ahead of the one being computed (one for fp32 at D > 64,
// whose Q and K chunks take twice the registers)
template <typename T, int DT> constexpr int gen_prefetch() { return (sizeof(T) == 4 && DT > 4) ? 1 : 2; }

// acc += A * B^T over NT contraction tiles (pairs on bf16, a lone last tile padded).
template <typename Fr, int NT>
__device__ __forceinline__ void mma_run(f32x4 &acc, const Fr (&a)[NT], const Fr (&b)[NT]) {
#pragma unroll
    for (int t = 0; t + 1 < NT; t += 2) mma2(acc, a[t], a[t + 1], b[t], b[t + 1]);
    if (NT & 1) mma1(acc, a[NT - 1], b[NT - 1]);
}

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

// Per-wavefront LDS staging for the token-contiguous copies (bf16 only).
template <int DT> constexpr int gen_stage_elems() { return stage_elems<DT, 1>() + stage_elems<1, 1>(); }

}  // namespace

// ---- per-segment sums ---------------------------------------------------------
// Record of segment `seg` (row-major S [D][M], then Z [D]): wavefront cg of the
// segment's workgroup writes columns [16 cg, 16 cg + 16) of S, wavefront 0 Z.
template <typename T, int DT, bool PHI>
__global__ __launch_bounds__(512) void k_gen_segstate(const T *__restrict__ k, const T *__restrict__ v,
                                                      float *__restrict__ ws, int64_t N, int64_t M, int64_t nseg,
                                                      int64_t seg_tokens) {
    constexpr int D = 16 * DT, GPF = gen_prefetch<T, DT>();
    typedef typename IO<T>::frag Fr;
    typedef typename IO<T>::vec4 V4;
    __shared__ __align__(16) bf16 stage_mem[8][gen_stage_elems<DT>()];
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    lds_bf16 *sk = (lds_bf16 *)stage_mem[cg];
    lds_bf16 *sv = sk + stage_elems<DT, 1>();

    f32x4 St[DT][2];   // S[:, 16 cg .. + 16] and (column 0) Z
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) St[dt][0] = St[dt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    V4 rk[GPF][1][DT], rv[GPF];
#pragma unroll
    for (int b = 0; b < GPF; ++b) {
        load_chunk<T, D, 1>(rk[b], K, t_begin + b * GCH, t_end);
        rv[b] = load_col_tile<T>(V, M, 16 * cg, t_begin + b * GCH, t_end);
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += GPF * GCH) {
#pragma unroll
        for (int b = 0; b < GPF; ++b) {
            const int64_t t0 = t00 + b * GCH;   // may lie past t_end: all rows masked, nothing added
            Fr Kn[1][DT], Vn[1][1];
            feat_frags<T, D, 1, PHI>(Kn, rk[b], t0, t_end);   // rows past t_end are zero
            {
                const V4 one[1][1] = {{rv[b]}};
                raw_frags<T, 16, 1>(Vn, one, t0, t_end);
            }
            load_chunk<T, D, 1>(rk[b], K, t0 + GPF * GCH, t_end);
            rv[b] = load_col_tile<T>(V, M, 16 * cg, t0 + GPF * GCH, t_end);
            __builtin_amdgcn_sched_barrier(0);
            Fr KT[1][DT], VT[1][1];
            transpose_frags<DT, 1>(KT, Kn, sk);
            transpose_frags<1, 1>(VT, Vn, sv);
            state_accumulate<Fr, D, 16, 1, false>(St, KT, VT);
        }
    }
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
// 0), writing columns [16 cg, 16 cg + 16) of out.
template <typename T, int DT, bool CAUSAL, bool PHI>
__global__ __launch_bounds__(512) void k_gen_output(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v, T *__restrict__ out,
                                                    const float *__restrict__ ws, int64_t N, int64_t M, int64_t nseg,
                                                    int64_t seg_tokens) {
    constexpr int D = 16 * DT, GPF = gen_prefetch<T, DT>();
    typedef typename IO<T>::frag Fr;
    typedef typename IO<T>::vec4 V4;
    __shared__ __align__(16) bf16 stage_mem[8][gen_stage_elems<DT>()];
    const int cg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane_id() & 15, g = lane_id() >> 4;
    const int64_t bh = blockIdx.x / nseg, seg = blockIdx.x % nseg;
    const int64_t t_begin = seg * seg_tokens, t_end = imin64(N, t_begin + seg_tokens);
    const T *Q = q + bh * N * D;
    const T *K = k + bh * N * D;
    const T *V = v + bh * N * M;
    T *O = out + bh * N * M;
    lds_bf16 *sk = (lds_bf16 *)stage_mem[cg];
    lds_bf16 *sv = sk + stage_elems<DT, 1>();

    // St[dt][0]: S rows 16 dt.., columns 16 cg..; St[dt][1]: Z replicated in every column
    f32x4 St[DT][2];
    {
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

    V4 rq[GPF][1][DT], rk[GPF][1][DT], rv[GPF];
#pragma unroll
    for (int b = 0; b < GPF; ++b) {
        load_chunk<T, D, 1>(rq[b], Q, t_begin + b * GCH, t_end);
        if (CAUSAL) {
            load_chunk<T, D, 1>(rk[b], K, t_begin + b * GCH, t_end);
            rv[b] = load_col_tile<T>(V, M, 16 * cg, t_begin + b * GCH, t_end);
        }
    }
    for (int64_t t00 = t_begin; t00 < t_end; t00 += GPF * GCH) {
#pragma unroll
        for (int b = 0; b < GPF; ++b) {
            const int64_t t0 = t00 + b * GCH;   // may lie past t_end: nothing stored
            Fr Qn[1][DT], Kn[1][DT], Vn[1][1];
            feat_frags<T, D, 1, PHI>(Qn, rq[b], t0, t_end);
            if (CAUSAL) {
                feat_frags<T, D, 1, PHI>(Kn, rk[b], t0, t_end);
                const V4 one[1][1] = {{rv[b]}};
                raw_frags<T, 16, 1>(Vn, one, t0, t_end);
            }
            load_chunk<T, D, 1>(rq[b], Q, t0 + GPF * GCH, t_end);
            if (CAUSAL) {
                load_chunk<T, D, 1>(rk[b], K, t0 + GPF * GCH, t_end);
                rv[b] = load_col_tile<T>(V, M, 16 * cg, t0 + GPF * GCH, t_end);
            }
            __builtin_amdgcn_sched_barrier(0);

            // out^T (16 columns, then the normalizer rows) against the carried state
            f32x4 Ot[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                Fr SF[DT];
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) SF[dt] = IO<T>::to_frag(St[dt][mt]);
                mma_run<Fr, DT>(Ot[mt], SF, Qn[0]);
            }
            if (CAUSAL) {
                // P^T[j][i] = phi(K_j) . phi(Q_i), j <= i
                f32x4 p = {0.f, 0.f, 0.f, 0.f};
                mma_run<Fr, DT>(p, Kn[0], Qn[0]);
#pragma unroll
                for (int r = 0; r < 4; ++r) p[r] = (4 * g + r <= c) ? p[r] : 0.f;
                const Fr PT = IO<T>::to_frag(p);
                Fr KT[1][DT], VT[1][1];
                transpose_frags<DT, 1>(KT, Kn, sk);
                transpose_frags<1, 1>(VT, Vn, sv);
                mma1(Ot[0], VT[0][0], PT);
                mma1(Ot[1], ones, PT);
                state_accumulate<Fr, D, 16, 1, true>(St, KT, VT);
            }
            // every row of the normalizer tile holds den: lane (c, g) element 0 is token c's
            const float inv = __builtin_amdgcn_rcpf(Ot[1][0]);
            const int64_t t = t0 + c;
            if (t < t_end) store4<T>(O + t * M + 16 * cg + 4 * g, IO<T>::from_f32(Ot[0] * inv));
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

template <typename T, int DT>
static hipError_t run_generic(bool causal, bool phi, const void *q, const void *k, const void *v, void *out,
                              int64_t BH, int64_t N, int64_t M, float *ws, StateIO sio, hipStream_t s) {
    constexpr int D = 16 * DT;
    const SegPlan p = make_plan(BH, N, D, M);
    const dim3 grid(unsigned(BH * p.nseg)), block(unsigned(64 * (M / 16)));
    ws = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + kGenHeader);
    if (phi)
        hipLaunchKernelGGL((k_gen_segstate<T, DT, true>), grid, block, 0, s, (const T *)k, (const T *)v, ws, N, M,
                           p.nseg, p.seg_tokens);
    else
        hipLaunchKernelGGL((k_gen_segstate<T, DT, false>), grid, block, 0, s, (const T *)k, (const T *)v, ws, N, M,
                           p.nseg, p.seg_tokens);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ScanIO io;
    io.s0 = sio.s0;
    io.z0 = sio.z0;
    io.s1 = sio.s1;
    io.z1 = sio.z1;
    io.srec = int64_t(D) * M;
    if ((e = launch_scan(ws, BH, p.nseg, p.rec, causal ? 0 : 1, s, io)) != hipSuccess) return e;
#define LA_GEN_OUT(C, P)                                                                                          \
    hipLaunchKernelGGL((k_gen_output<T, DT, C, P>), grid, block, 0, s, (const T *)q, (const T *)k, (const T *)v,   \
                       (T *)out, (const float *)ws, N, M, p.nseg, p.seg_tokens)
    if (!causal) LA_GEN_OUT(false, true);
    else if (phi) LA_GEN_OUT(true, true);
    else LA_GEN_OUT(true, false);
#undef LA_GEN_OUT
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

}  // namespace la
