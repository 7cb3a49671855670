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

template <typename T, int D, int M>
__global__ __launch_bounds__(256) void k_decode_step(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, float *__restrict__ S,
                                                     float *__restrict__ Z, T *__restrict__ out, int64_t BH) {
    constexpr int QPR = M / 4;            // float4 quads per row of S
    constexpr int RPI = 64 / QPR;         // rows covered by one wavefront instruction
    constexpr int NJ = D * M / 4 / 64;    // quads per lane
    static_assert(NJ * RPI == D, "layout");
    const int lane = threadIdx.x & 63;
    const int64_t s = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (s >= BH) return;
    const int quad = lane % QPR, r0 = lane / QPR;

    float *Sp = S + s * D * M;
    f32x4 x[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) x[j] = *reinterpret_cast<const f32x4 *>(Sp + (RPI * j + r0) * M + 4 * quad);

    // lane d < D holds phi(k_d), phi(q_d) and Z_d
    float kh = 0.f, qh = 0.f, z = 0.f;
    if (lane < D) {
        kh = phi((float)k[s * D + lane]);
        qh = phi((float)q[s * D + lane]);
        z = Z[s * D + lane] + kh;
        Z[s * D + lane] = z;
    }
    const f32x4 vq = IO<T>::to_f32(load4<T>(v + s * M + 4 * quad));

    f32x4 num = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int d = RPI * j + r0;
        const float kd = __shfl(kh, d), qd = __shfl(qh, d);
        x[j] += kd * vq;
        *reinterpret_cast<f32x4 *>(Sp + d * M + 4 * quad) = x[j];
        num += qd * x[j];
    }
    const float den = wave_sum(qh * z);
#pragma unroll
    for (int off = QPR; off < 64; off <<= 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) num[r] += __shfl_xor(num[r], off);
    }
    if (lane < QPR) store4<T>(out + s * M + 4 * lane, IO<T>::from_f32(num * __builtin_amdgcn_rcpf(den)));
}

template <typename T>
static hipError_t run_decode(const void *q, const void *k, const void *v, float *S, float *Z, void *out, int64_t BH,
                             int64_t D, int64_t M, hipStream_t st) {
    const dim3 grid(unsigned((BH + 3) / 4)), block(256);
#define LA_DECODE_CASE(DD, MM)                                                                                   \
    if (D == DD && M == MM) {                                                                                    \
        hipLaunchKernelGGL((k_decode_step<T, DD, MM>), grid, block, 0, st, (const T *)q, (const T *)k,            \
                           (const T *)v, S, Z, (T *)out, BH);                                                    \
        return hipGetLastError();                                                                                \
    }
    LA_DECODE_CASE(32, 32)
    LA_DECODE_CASE(32, 64)
    LA_DECODE_CASE(64, 32)
    LA_DECODE_CASE(64, 64)
#undef LA_DECODE_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(int dt, const void *q, const void *k, const void *v, float *S, float *Z, void *out,
                         int64_t BH, int64_t D, int64_t M, hipStream_t st) {
    if (dt == 0) return run_decode<float>(q, k, v, S, Z, out, BH, D, M, st);
    return run_decode<bf16>(q, k, v, S, Z, out, BH, D, M, st);
}

} // namespace la
