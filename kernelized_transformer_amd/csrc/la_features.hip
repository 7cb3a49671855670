// la_features.hip -- random Fourier features on gfx950.
//
// [summary] section 5 names random Fourier features, approximating the RBF
// kernel, as a feature map for reusing softmax-pretrained models; the map is
// the standard one: phi_r(x) = sqrt(2/R) cos(sum_d x_d omega[d][r] + b_r)
// with omega [D][R] and b [R] drawn by the caller, so that phi(q) . phi(k)
// estimates exp(-|q - k|^2 / (2 sigma^2)) for omega ~ N(0, 1/sigma^2) and
// b ~ U[0, 2 pi).
//
// One wavefront per run of 16-row tiles.  The projection x omega is a
// product on the matrix cores computed transposed (features as output rows,
// rows of x as output columns), so each lane ends with 4 consecutive
// features of one row.  bf16 inputs are exact in bf16; omega (fp32) is split
// into bf16 hi + lo parts and both are applied in one 32-deep product, which
// keeps the angle accurate to about 2^-16 relative.  fp32 inputs use the fp32
// matrix instruction.  Angles, cosines and scaling are fp32; outputs are
// rounded once to the I/O type.
#include "la_chunk.h"
#include "la_internal.h"
#include "la_split.h"

namespace la {

constexpr int kFeatRowsPerWave = 256;   // 16 tiles of 16 rows
constexpr int kFeatAhead = 4;           // tiles of rows in flight
constexpr int kFeatWavesPerBlock = 4;

template <typename T, int D, int R>
__global__ __launch_bounds__(64 * kFeatWavesPerBlock) void k_rff_features(const T *__restrict__ x,
                                                                          const float *__restrict__ omega,
                                                                          const float *__restrict__ bias,
                                                                          T *__restrict__ out, int64_t rows) {
    constexpr int DT = D / 16, RT = R / 16;
    const int lane = lane_id(), c = lane & 15, g = lane >> 4;
    const int wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t(blockIdx.x) * kFeatWavesPerBlock + wave) * kFeatRowsPerWave;
    if (r0 >= rows) return;   // whole wavefront: no barrier below
    const int64_t r_end = min(rows, r0 + kFeatRowsPerWave);

    // omega^T tiles as A operands: lane (c, g) of tile (rt, dt) holds
    // omega[16 dt + 4g + j][16 rt + c], j = 0..3
    typename IO<T>::frag ohi[RT][DT], olo[RT][DT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            f32x4 w;
#pragma unroll
            for (int j = 0; j < 4; ++j) w[j] = omega[(16 * dt + 4 * g + j) * R + 16 * rt + c];
            if constexpr (sizeof(T) == 2) {
                const bf16x4 hi = IO<bf16>::from_f32(w);
                ohi[rt][dt] = hi;
                olo[rt][dt] = IO<bf16>::from_f32(w - IO<bf16>::to_f32(hi));
            } else {
                ohi[rt][dt] = w;
            }
        }
    f32x4 bv[RT];   // b of this lane's 4 features per tile
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) bv[rt] = *reinterpret_cast<const f32x4 *>(bias + 16 * rt + 4 * g);
    const float scale = __builtin_sqrtf(2.f / float(R));

    __shared__ bf16 tiles[kFeatWavesPerBlock][16 * (R + kStagePad)];
    lds_bf16 *otile = (lds_bf16 *)tiles[wave];
    // bf16 rows arrive as 16-byte pieces of whole rows (1 KB per load
    // instruction) and are staged here, from which the fragments are read
    __shared__ bf16 xstage[kFeatWavesPerBlock][16 * (D + kStagePad)];
    lds_bf16 *xtile = (lds_bf16 *)xstage[wave];

    // rows past the end read a valid row and are not stored; kFeatAhead tiles
    // of rows are in flight (tile i lives in slot i % kFeatAhead)
    constexpr int NL = Lines<D, 1>::n;
    typename IO<T>::frag xr[kFeatAhead][DT];
    dwordx4 xl[kFeatAhead][NL];
    const bf16 *xw = reinterpret_cast<const bf16 *>(x) + r0 * D;   // bf16: this wavefront's first row
    const int nrows = int(r_end - r0);
#pragma unroll
    for (int a = 0; a < kFeatAhead; ++a) {
        if constexpr (sizeof(T) == 2) {
            load_rows32<D>(xl[a], xw, 16 * a, nrows);
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                xr[a][dt] = load4<T>(x + min(r0 + 16 * a + c, r_end - 1) * D + 16 * dt + 4 * g);
        }
    }
    for (int64_t t00 = r0; t00 < r_end; t00 += 16 * kFeatAhead) {
#pragma unroll
    for (int a = 0; a < kFeatAhead; ++a) {
        const int64_t t0 = t00 + 16 * a;   // may lie past r_end: computed, not stored
        typename IO<T>::frag xf[DT];
        if constexpr (sizeof(T) == 2) {
            stage_lines<D, 1, false, false>(xtile, xl[a], 0, 16);
            bf16x4 xn[1][DT];
            natural_frags_lds<D, 1>(xn, xtile);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) xf[dt] = xn[0][dt];
            load_rows32<D>(xl[a], xw, int(t0 - r0) + 16 * kFeatAhead, nrows);
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) xf[dt] = xr[a][dt];
            const int64_t tn = min(t0 + 16 * kFeatAhead + c, r_end - 1);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) xr[a][dt] = load4<T>(x + tn * D + 16 * dt + 4 * g);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if constexpr (sizeof(T) == 2)
                    mma2(acc, ohi[rt][dt], olo[rt][dt], xf[dt], xf[dt]);
                else
                    mma1(acc, ohi[rt][dt], xf[dt]);
            }
            f32x4 y;
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = scale * __cosf(acc[j] + bv[rt][j]);
            if constexpr (sizeof(T) == 2)
                tile_put_bf16<R>(otile, rt, IO<bf16>::from_f32(y));
            else if (t0 + c < r_end)
                store4<T>(out + (t0 + c) * R + 16 * rt + 4 * g, y);
        }
        if constexpr (sizeof(T) == 2) tile_flush_bf16<R>((bf16 *)out, t0, r_end, otile);
    }
    }
}

template <typename T>
static hipError_t run_rff(const void *x, const float *omega, const float *bias, void *out, int64_t rows, int64_t D,
                          int64_t R, hipStream_t s) {
    const int64_t waves = ceil_div(rows, kFeatRowsPerWave);
    const dim3 grid(unsigned(ceil_div(waves, kFeatWavesPerBlock))), block(64 * kFeatWavesPerBlock);
#define LA_RFF_CASE(DD, RR)                                                                                        \
    if (D == DD && R == RR) {                                                                                      \
        hipLaunchKernelGGL((k_rff_features<T, DD, RR>), grid, block, 0, s, (const T *)x, omega, bias, (T *)out,   \
                           rows);                                                                                  \
        return hipGetLastError();                                                                                  \
    }
    LA_RFF_CASE(32, 32)
    LA_RFF_CASE(32, 64)
    LA_RFF_CASE(64, 32)
    LA_RFF_CASE(64, 64)
#undef LA_RFF_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_rff_features(int dt, const void *x, const float *omega, const float *bias, void *out, int64_t rows,
                               int64_t D, int64_t R, hipStream_t s) {
    if (dt == 0) return run_rff<float>(x, omega, bias, out, rows, D, R, s);
    return run_rff<bf16>(x, omega, bias, out, rows, D, R, s);
}

} // namespace la
