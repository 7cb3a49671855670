// la_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// Tile algebra.  Every matrix product in the kernels is built from 16x16
// tiles on the CDNA matrix cores (one 64-lane wavefront per tile product):
//
//   * Acc  (f32x4): a 16x16 fp32 accumulator tile C in the MFMA output
//     layout: lane l = 16*g + c (c = l & 15, g = l >> 4) holds
//     C[4g + r][c] for r = 0..3.
//   * Frag (bf16x4 or f32x4): a 16x16 operand tile X, seen as
//     "row index" x "contraction index": lane (c, g) holds X[c][4g + r],
//     r = 0..3.  The same registers serve as the A operand (rows = output
//     rows) or the B operand (rows = output columns) of a product.
//
// A product C += A * B^T over a 16-wide contraction pairs element r of lane
// (c, g) of A with element r of lane (c', g) of B, so any consistent choice of
// which contraction index sits in (g, r) gives the same sum.  Two facts make
// the kernels work without any LDS transposes:
//   1. an Acc tile whose rows run along a contraction axis is, lane for
//      lane, already a Frag for a product contracting over that axis
//      (lane (c, g) holds C[4g + r][c]); only a conversion to bf16 is needed;
//   2. a Frag loaded from row-major memory (4 consecutive features of one
//      token per lane) contracts over features; to contract over tokens it is
//      pushed once through a product with the 16x16 identity, which returns
//      it as an Acc with tokens as rows (exact: x * 1 + 0).
//
// bf16 operands use v_mfma_f32_16x16x32_bf16 (two tiles per instruction);
// fp32 operands use four v_mfma_f32_16x16x4_f32, or are split into bf16
// parts (split4) for the bf16 instruction.
// Accumulation is always fp32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Integer min / max for 64-bit indices (plain selects: the templated
// min / max of the device math headers convert through double).
__device__ __forceinline__ int64_t imax64(int64_t a, int64_t b) { return a > b ? a : b; }
__device__ __forceinline__ int64_t imin64(int64_t a, int64_t b) { return a < b ? a : b; }

// phi(x) = elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (positive).
// Evaluated as max(exp(-|x|), x + 1) -- for x <= 0, exp(x) >= x + 1; for
// x > 0, exp(-x) < 1 < x + 1 -- which costs one exponential and no select.
constexpr float kLog2e = 1.44269504088896341f;
__device__ __forceinline__ float phi(float x) {
    return __builtin_fmaxf(__builtin_amdgcn_exp2f(-__builtin_fabsf(x * kLog2e)), x + 1.f);
}
// phi'(x): 1 for x > 0, exp(x) otherwise, i.e. min(exp(x), 1).
__device__ __forceinline__ float dphi(float x) { return __builtin_fminf(__builtin_amdgcn_exp2f(x * kLog2e), 1.f); }

// ---- element type traits ------------------------------------------------
template <typename T> struct IO;
template <> struct IO<float> {
    typedef f32x4 frag;                    // operand fragment type
    typedef f32x4 vec4;                    // 4 consecutive elements in memory
    static __device__ __forceinline__ f32x4 to_f32(vec4 x) { return x; }
    static __device__ __forceinline__ vec4 from_f32(f32x4 x) { return x; }
    static __device__ __forceinline__ frag to_frag(f32x4 x) { return x; }
};
template <> struct IO<bf16> {
    typedef bf16x4 frag;
    typedef bf16x4 vec4;
    static __device__ __forceinline__ f32x4 to_f32(vec4 x) {
        return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    }
    static __device__ __forceinline__ vec4 from_f32(f32x4 x) {
        return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    }
    static __device__ __forceinline__ frag to_frag(f32x4 x) { return from_f32(x); }
};

// ---- tile products ------------------------------------------------------
// acc += A * B^T over one 16-wide contraction tile.
// All bf16 products use the single opcode v_mfma_f32_16x16x32_bf16 (a lone
// tile is padded with zeros): the compiler inserts no wait states when an
// accumulator written by one bf16 MFMA opcode is read as the SrcC of the
// other, which gave wrong, run-to-run varying results in dependent chains.
__device__ __forceinline__ void mma1(f32x4 &acc, bf16x4 a, bf16x4 b) {
    const bf16x4 z = IO<bf16>::from_f32(f32x4{0.f, 0.f, 0.f, 0.f});
    bf16x8 a8 = __builtin_shufflevector(a, z, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b8 = __builtin_shufflevector(b, z, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, b8, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma1(f32x4 &acc, f32x4 a, f32x4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], acc, 0, 0, 0);
}
// acc += A0 * B0^T + A1 * B1^T (two contraction tiles).
__device__ __forceinline__ void mma2(f32x4 &acc, bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1) {
    bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma2(f32x4 &acc, f32x4 a0, f32x4 a1, f32x4 b0, f32x4 b1) {
    mma1(acc, a0, b0);
    mma1(acc, a1, b1);
}

// An fp32 operand carried as two bf16 parts, x = hi + lo: hi is x rounded
// to bf16 (RNE, 8 significant bits), lo the exact remainder x - hi rounded
// to bf16, so that |x - hi - lo| <= 2^-16 |x|.  The parts sit in one 8-wide
// operand [hi, lo], and a 16-deep tile product is two 32-deep bf16
// instructions: [hi, lo] . [hi, lo] + [hi, lo] . [lo, hi] = (a_hi + a_lo)
// (b_hi + b_lo), the product of the split values with no term dropped, so
// each product is within about 2 * 2^-16 of |a||b| (errors of random sign,
// which average out in the sums), at 32 cycles per 16-deep tile against 128
// for four 4-deep fp32 instructions.  Only the swapped copy of the second
// operand is ever moved between registers; no operand is zero-padded.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
struct split4 {
    bf16x8 hl;   // elements 0-3: hi, 4-7: lo
};
__device__ __forceinline__ split4 split_f32(f32x4 a) {
    // each pair rounded once (one v_cvt_pk_bf16_f32); the fp32 values of the
    // rounded halves are the packed word shifted / masked.  The empty asm
    // (no instruction) keeps the compiler from re-deriving the low half with a
    // second, single-value conversion.
    unsigned h01 = __builtin_bit_cast(unsigned, bf16x2{(bf16)a[0], (bf16)a[1]});
    unsigned h23 = __builtin_bit_cast(unsigned, bf16x2{(bf16)a[2], (bf16)a[3]});
    __asm__("" : "+v"(h01), "+v"(h23));
    const f32x4 hf = {__builtin_bit_cast(float, h01 << 16), __builtin_bit_cast(float, h01 & 0xffff0000u),
                      __builtin_bit_cast(float, h23 << 16), __builtin_bit_cast(float, h23 & 0xffff0000u)};
    const f32x4 r = a - hf;
    const unsigned l01 = __builtin_bit_cast(unsigned, bf16x2{(bf16)r[0], (bf16)r[1]});
    const unsigned l23 = __builtin_bit_cast(unsigned, bf16x2{(bf16)r[2], (bf16)r[3]});
    return split4{__builtin_bit_cast(bf16x8, u32x4{h01, h23, l01, l23})};
}
__device__ __forceinline__ bf16x4 split_hi(split4 x) { return __builtin_shufflevector(x.hl, x.hl, 0, 1, 2, 3); }
__device__ __forceinline__ bf16x4 split_lo(split4 x) { return __builtin_shufflevector(x.hl, x.hl, 4, 5, 6, 7); }
__device__ __forceinline__ split4 split_join(bf16x4 hi, bf16x4 lo) {
    return split4{__builtin_shufflevector(hi, lo, 0, 1, 2, 3, 4, 5, 6, 7)};
}
__device__ __forceinline__ void mma1(f32x4 &acc, split4 a, split4 b) {
    const bf16x8 bs = __builtin_shufflevector(b.hl, b.hl, 4, 5, 6, 7, 0, 1, 2, 3);   // [lo, hi]
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hl, b.hl, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.hl, bs, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma2(f32x4 &acc, split4 a0, split4 a1, split4 b0, split4 b1) {
    mma1(acc, a0, b0);
    mma1(acc, a1, b1);
}

__device__ __forceinline__ bf16x4 acc_to_frag(f32x4 a, bf16x4) { return IO<bf16>::to_frag(a); }
__device__ __forceinline__ f32x4 acc_to_frag(f32x4 a, f32x4) { return a; }
__device__ __forceinline__ split4 acc_to_frag(f32x4 a, split4) { return split_f32(a); }
template <typename F> __device__ __forceinline__ F frag_from(f32x4 x) { return acc_to_frag(x, F{}); }

template <typename F> __device__ __forceinline__ F frag_zero() { return frag_from<F>(f32x4{0.f, 0.f, 0.f, 0.f}); }

// Frag whose row 0 is all ones and other rows zero: as an A operand it sums
// the B operand over the contraction (a normalizer row); as a B operand it
// adds a column of ones.
template <typename F> __device__ __forceinline__ F frag_row0_ones() {
    const float o = ((lane_id() & 15) == 0) ? 1.f : 0.f;
    return frag_from<F>(f32x4{o, o, o, o});
}

// Frag of all ones: as an A operand every output row is the sum of the B
// operand over the contraction; as a B operand every output column is the
// sum of the A operand (the normalizer replicated across the tile).
template <typename F> __device__ __forceinline__ F frag_ones() { return frag_from<F>(f32x4{1.f, 1.f, 1.f, 1.f}); }

// 16x16 identity as a Frag: lane (c, g) element r is [4g + r == c].
template <typename F> __device__ __forceinline__ F frag_identity() {
    const int c = lane_id() & 15, g4 = (lane_id() >> 4) * 4;
    return frag_from<F>(f32x4{(g4 + 0 == c) ? 1.f : 0.f, (g4 + 1 == c) ? 1.f : 0.f, (g4 + 2 == c) ? 1.f : 0.f,
                              (g4 + 3 == c) ? 1.f : 0.f});
}

// Re-lay a Frag so that it contracts over its former row index: returns
// Y with lane (c, g) holding X[4g + r][c] (exact).

template <typename F> __device__ __forceinline__ F transpose_frag(F x, F ident) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    mma1(acc, x, ident);
    return acc_to_frag(acc, x);
}

// ---- memory helpers -----------------------------------------------------
template <typename T>
__device__ __forceinline__ typename IO<T>::vec4 load4(const T *p) {
    return *reinterpret_cast<const typename IO<T>::vec4 *>(p);
}
template <typename T>
__device__ __forceinline__ void store4(T *p, typename IO<T>::vec4 x) {
    *reinterpret_cast<typename IO<T>::vec4 *>(p) = x;
}

__device__ __forceinline__ f32x4 phi4(f32x4 x) { return f32x4{phi(x[0]), phi(x[1]), phi(x[2]), phi(x[3])}; }
__device__ __forceinline__ f32x4 dphi4(f32x4 x) { return f32x4{dphi(x[0]), dphi(x[1]), dphi(x[2]), dphi(x[3])}; }

} // namespace la
