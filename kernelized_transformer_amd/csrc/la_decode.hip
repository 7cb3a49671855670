// la_decode.hip -- one RNN-style decode step for many independent streams.
//
// Method ([review] = nubint.ai "[Paper Review] Transformers are RNNs",
// "Proposed method": attention memory s and normalizer memory z with a
// two-step update; [summary] = paperlayer.ai summary, 3.3.2 and 3.4; [deck] =
// zhengyuhong.cn "... 解读", slide 4):
//   S += phi(k) v^T;  Z += phi(k);  out = S^T phi(q) / phi(q)^T Z.
// Updating first makes a run of steps equal the inclusive causal forward.
//
// The step is a pure stream over the fp32 state (4*D*M + 4*D bytes read and
// written per stream against 4*D*M flops), so it is bound by memory
// bandwidth, not arithmetic: plain fp32 FMAs on the vector ALUs, no matrix
// cores.  One wavefront per stream; each lane owns float4 quads of S laid
// out so that every load/store instruction of the wavefront touches one
// contiguous 1 KB (D = M = 64) block.
#include "la_device.h"
#include "la_internal.h"

namespace la {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
    return x;
}

// Lane layout: each row d of S is M/4 float4 quads, handled by a power-of-two
// group of QPRP >= M/4 lanes (lanes past M/4 idle when M/4 is not a power of
// two), RPI = 64/QPRP rows per wavefront instruction, NJ instructions cover
// the D rows.  Lane l holds phi(k_d), phi(q_d), Z_d for d = l and d = l + 64.
template <typename T, int D, int M>
__global__ __launch_bounds__(256) void k_decode_step(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, float *__restrict__ S,
                                                     float *__restrict__ Z, T *__restrict__ out, int64_t BH) {
    constexpr int QPR = M / 4;            // float4 quads per row of S
    constexpr int QPRP = QPR <= 4 ? 4 : QPR <= 8 ? 8 : QPR <= 16 ? 16 : 32;
    constexpr int RPI = 64 / QPRP;        // rows covered by one wavefront instruction
    constexpr int NJ = (D + RPI - 1) / RPI;
    constexpr int DH = (D + 63) / 64;     // d values per lane
    static_assert(M % 16 == 0 && M <= 128 && D % 16 == 0 && D <= 128, "head sizes");
    const int lane = threadIdx.x & 63;
    const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (s >= BH) return;
    const int quad = lane % QPRP, r0 = lane / QPRP;
    const bool qok = quad < QPR;

    float *Sp = S + s * D * M;
    f32x4 x[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int d = RPI * j + r0;
        x[j] = (qok && d < D) ? *reinterpret_cast<const f32x4 *>(Sp + d * M + 4 * quad) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    float kh[DH], qh[DH], z[DH];
#pragma unroll
    for (int h = 0; h < DH; ++h) {
        const int d = lane + 64 * h;
        kh[h] = qh[h] = z[h] = 0.f;
        if (d < D) {
            kh[h] = phi((float)k[s * D + d]);
            qh[h] = phi((float)q[s * D + d]);
            z[h] = Z[s * D + d] + kh[h];
            Z[s * D + d] = z[h];
        }
    }
    const f32x4 vq = qok ? IO<T>::to_f32(load4<T>(v + s * M + 4 * quad)) : f32x4{0.f, 0.f, 0.f, 0.f};

    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int d = RPI * j + r0;
        const int hsel = (RPI * j) / 64;   // rows of one instruction never straddle d = 64
        const float kd = __shfl(kh[hsel], d & 63), qd = __shfl(qh[hsel], d & 63);
        if (qok && d < D) {
            x[j] += kd * vq;
            *reinterpret_cast<f32x4 *>(Sp + d * M + 4 * quad) = x[j];
            num += qd * x[j];
        }
    }
    float dz = 0.f;
#pragma unroll
    for (int h = 0; h < DH; ++h) dz += qh[h] * z[h];
    const float den = wave_sum(dz);
#pragma unroll
    for (int off = QPRP; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) num[r] += __shfl_xor(num[r], off);
    }
    if (lane < QPR) store4<T>(out + s * M + 4 * lane, IO<T>::from_f32(num * __builtin_amdgcn_rcpf(den)));
}

template <typename T, int D, int M>
static hipError_t decode_one(const void *q, const void *k, const void *v, float *S, float *Z, void *out, int64_t BH,
                             hipStream_t st) {
    const dim3 grid(unsigned((BH + 3) / 4)), block(256);
    hipLaunchKernelGGL((k_decode_step<T, D, M>), grid, block, 0, st, (const T *)q, (const T *)k, (const T *)v, S, Z,
                       (T *)out, BH);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t decode_m(const void *q, const void *k, const void *v, float *S, float *Z, void *out, int64_t BH,
                           int64_t M, hipStream_t st) {
    switch (M) {
    case 16: return decode_one<T, D, 16>(q, k, v, S, Z, out, BH, st);
    case 32: return decode_one<T, D, 32>(q, k, v, S, Z, out, BH, st);
    case 48: return decode_one<T, D, 48>(q, k, v, S, Z, out, BH, st);
    case 64: return decode_one<T, D, 64>(q, k, v, S, Z, out, BH, st);
    case 80: return decode_one<T, D, 80>(q, k, v, S, Z, out, BH, st);
    case 96: return decode_one<T, D, 96>(q, k, v, S, Z, out, BH, st);
    case 112: return decode_one<T, D, 112>(q, k, v, S, Z, out, BH, st);
    case 128: return decode_one<T, D, 128>(q, k, v, S, Z, out, BH, st);
    }
    return hipErrorInvalidValue;
}

template <typename T>
static hipError_t run_decode(const void *q, const void *k, const void *v, float *S, float *Z, void *out, int64_t BH,
                             int64_t D, int64_t M, hipStream_t st) {
    switch (D) {
    case 16: return decode_m<T, 16>(q, k, v, S, Z, out, BH, M, st);
    case 32: return decode_m<T, 32>(q, k, v, S, Z, out, BH, M, st);
    case 48: return decode_m<T, 48>(q, k, v, S, Z, out, BH, M, st);
    case 64: return decode_m<T, 64>(q, k, v, S, Z, out, BH, M, st);
    case 80: return decode_m<T, 80>(q, k, v, S, Z, out, BH, M, st);
    case 96: return decode_m<T, 96>(q, k, v, S, Z, out, BH, M, st);
    case 112: return decode_m<T, 112>(q, k, v, S, Z, out, BH, M, st);
    case 128: return decode_m<T, 128>(q, k, v, S, Z, out, BH, M, st);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(int dt, const void *q, const void *k, const void *v, float *S, float *Z, void *out,
                         int64_t BH, int64_t D, int64_t M, hipStream_t st) {
    if (dt == 0) return run_decode<float>(q, k, v, S, Z, out, BH, D, M, st);
    return run_decode<bf16>(q, k, v, S, Z, out, BH, D, M, st);
}

} // namespace la
