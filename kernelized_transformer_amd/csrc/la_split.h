// la_split.h -- helpers for the kernels that walk one segment with two
// wavefronts (bf16, D = 64), each owning half of the feature rows d.
#pragma once

#include "la_chunk.h"

namespace la {

// A segment's states are split by feature row d between two wavefronts:
// wavefront w owns rows [32 w, 32 w + 32) and loads only its 32 columns of
// the d-indexed inputs.  Helpers for those kernels; their global accesses
// use 32-bit offsets from a per-head base pointer (callers check that a
// head's bytes fit), computed in bytes so that the compiler adds them to the
// scalar base in the load or store itself.
constexpr int kW2Half = 32;   // feature columns per wavefront

// 16 rows x 32 bf16 columns of a row-major tensor with row stride S (base
// already offset to the first column): lane l moves row l / 4, columns
// 8 (l % 4) .. + 7.  Rows at or beyond t_end read row t_end - 1.
template <int S>
__device__ __forceinline__ dwordx4 load_cols32(const bf16 *__restrict__ base, int64_t t0, int64_t t_end) {
    // 32-bit byte offsets from the (uniform) per-head base: the load adds them to the scalar base
    const int l = lane_id();
    const uint32_t t = min(uint32_t(t0) + uint32_t(l >> 2), uint32_t(t_end - 1));
    return *reinterpret_cast<const dwordx4 *>(reinterpret_cast<const char *>(base) +
                                              (t * uint32_t(2 * S) + uint32_t(16 * (l & 3))));
}
// 16 whole rows of F bf16 features (as load_lines, 32-bit offsets).
template <int F>
__device__ __forceinline__ void load_rows32(dwordx4 (&x)[F / 32], const bf16 *__restrict__ base, int64_t t0,
                                            int64_t t_end) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < F / 32; ++i) {
        const int e = (64 * i + l) * 8;
        const uint32_t t = min(uint32_t(t0) + uint32_t(e / F), uint32_t(t_end - 1));
        x[i] = *reinterpret_cast<const dwordx4 *>(reinterpret_cast<const char *>(base) +
                                                   (t * uint32_t(2 * F) + uint32_t(2 * (e % F))));
    }
}
// 16 whole rows loaded by load_rows32<F>, each scaled by its token's factor
// (lane c < 16 holds the factor of row c in `scale_c`) and rounded to bf16,
// into staging rows of F + kStagePad; rows at or beyond t_end become 0.
template <int F>
__device__ __forceinline__ void stage_rows_scaled(lds_bf16 *stage, const dwordx4 (&x)[F / 32], float scale_c,
                                                  int64_t t0, int64_t t_end) {
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < F / 32; ++i) {
        const int e = (64 * i + l) * 8, row = e / F, col = e % F;
        const float sc = __shfl(scale_c, row);
        dwordx4 y;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float lo = __builtin_bit_cast(float, x[i][w] << 16);
            const float hi = __builtin_bit_cast(float, x[i][w] & 0xffff0000u);
            const bf16x2 p = {(bf16)(lo * sc), (bf16)(hi * sc)};
            y[w] = __builtin_bit_cast(unsigned int, p);
        }
        if (t0 + row >= t_end) y = dwordx4{0u, 0u, 0u, 0u};
        *reinterpret_cast<lds_dwordx4 *>(stage + row * (F + kStagePad) + col) = y;
    }
}
// ... into staging rows of 32 + kStagePad, phi applied (no row masks: the
// callers keep rows past t_end out of every stored result themselves).
__device__ __forceinline__ void stage_cols32_phi(lds_bf16 *stage, dwordx4 x) {
    const int l = lane_id();
    *reinterpret_cast<lds_dwordx4 *>(stage + (l >> 2) * (kW2Half + kStagePad) + 8 * (l & 3)) = phi8(x);
}
// Rows [r0, r0 + NR) of a 16-row LDS tile (row stride F + kStagePad, F
// columns) to rows t0 + r of a tensor with row stride S (dst already offset
// to the first column); rows at or beyond t_end are not written.
template <int F, int S, int NR>
__device__ __forceinline__ void flush_rows(bf16 *__restrict__ dst, int64_t t0, int64_t t_end, const lds_bf16 *tile,
                                           int r0) {
    constexpr int PR = F / 8, NP = NR * PR;   // 16-byte pieces per row, in all
    const int l = lane_id();
#pragma unroll
    for (int i = 0; i < (NP + 63) / 64; ++i) {
        const int p = 64 * i + l;
        if (NP % 64 == 0 || p < NP) {
            const int row = r0 + p / PR, col = 8 * (p % PR);
            const dwordx4 y = *reinterpret_cast<const lds_dwordx4 *>(tile + row * (F + kStagePad) + col);
            const uint32_t t = uint32_t(t0) + uint32_t(row);
            if (t < uint32_t(t_end))
                *reinterpret_cast<dwordx4 *>(reinterpret_cast<char *>(dst) + (t * uint32_t(2 * S) + uint32_t(2 * col))) = y;
        }
    }
}
// Both wavefronts of the workgroup have finished their LDS accesses so far
// (global loads in flight are not waited for).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Rows [d0, d0 + 16 DTH) of a row-major record, as Acc tiles (the layout of
// state_load: REP puts Z in every column of the normalizer tile, otherwise
// in column 0).
template <int D, int M, int DTH, bool REP>
__device__ __forceinline__ void rows_load(f32x4 (&St)[DTH][M / 16 + 1], const float *__restrict__ rec, int d0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < DTH; ++dt) {
        const int d = d0 + 16 * dt + 4 * g;
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) St[dt][mt][r] = rec[(d + r) * M + 16 * mt + c];
#pragma unroll
        for (int r = 0; r < 4; ++r) St[dt][M / 16][r] = (REP || c == 0) ? rec[D * M + d + r] : 0.f;
    }
}
template <int D, int M, int DTH>
__device__ __forceinline__ void rows_store(float *__restrict__ rec, const f32x4 (&St)[DTH][M / 16 + 1], int d0) {
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int dt = 0; dt < DTH; ++dt) {
        const int d = d0 + 16 * dt + 4 * g;
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[(d + r) * M + 16 * mt + c] = St[dt][mt][r];
        if (c == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rec[D * M + d + r] = St[dt][M / 16][r];
        }
    }
}

// Natural fragments y[tt][ft] written row-major into LDS (row stride
// 16 NF + kStagePad), to be read back transposed by transposed_frags_lds
// (the two halves of transpose_frags_lds, split so that other work can
// run in between).
template <int NF, int TT>
__device__ __forceinline__ void put_frags_lds(lds_bf16 *stage, const bf16x4 (&y)[TT][NF]) {
    constexpr int S = 16 * NF + kStagePad;
    const int c = lane_id() & 15, g = lane_id() >> 4;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int ft = 0; ft < NF; ++ft)
            *reinterpret_cast<lds_bf16x4 *>(stage + (16 * tt + c) * S + 16 * ft + 4 * g) = y[tt][ft];
}

} // namespace la
