// common.hpp -- small device helpers shared by the gfx950 kernels.
//
// Element types: bf16 inputs are handled as raw 16-bit patterns (uint16_t);
// widening to fp32 is exact (shift into the high half).  Narrowing uses the
// hardware round-to-nearest-even conversion (v_cvt_pk_bf16_f32 on gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace based {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Taylor feature count for feature dim d: 1 + d + d*d.
constexpr int kDFeat = 16;
constexpr int kNumFeat = 1 + kDFeat + kDFeat * kDFeat;  // 273
// d'^(-1/4) for d' = 16 is exactly 1/2.
constexpr float kPreScale = 0.5f;
constexpr float kInvSqrt2 = 0.70710678118654752440f;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Widening loads from either element type.
__device__ __forceinline__ float load_elem(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_elem(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

// Round two floats to a packed bf16 pair (RNE), as raw bits (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    bf16x2 r = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Value of the low / high bf16 of a packed pair, widened to fp32 (exact).
__device__ __forceinline__ float bf16lo_f32(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi_f32(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }

// The lo half of a hi/lo bf16 split of two floats: given the hi pair
// hp = pack_bf16x2(x0, x1), the bf16 pair of the remainders x - hi, so that
// x ~= hi + lo to about 16 mantissa bits.  Each x - hi is one
// v_dot2_f32_bf16 of the packed pair against (-1, -0) or (-0, -1) plus x:
// the products are exact and x - hi is representable, so its one rounding
// changes nothing.  (The selectors keep a -0 in the other half: the pair
// (-1, +0) has the bit pattern of a small integer that the assembler would
// emit as an inline float constant.)
__device__ __forceinline__ uint32_t lo_pair_of(uint32_t hp, float x0, float x1) {
    const bf16x2 sel0 = __builtin_bit_cast(bf16x2, 0x8000bf80u);
    const bf16x2 sel1 = __builtin_bit_cast(bf16x2, 0xbf808000u);
    const bf16x2 hb = __builtin_bit_cast(bf16x2, hp);
    return pack_bf16x2(__builtin_amdgcn_fdot2_f32_bf16(hb, sel0, x0, false),
                       __builtin_amdgcn_fdot2_f32_bf16(hb, sel1, x1, false));
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Feature geometry for feature dim D: F = 1 + D + D*D rows, pre-scale
// D^(-1/4) (exactly 1/2 for D = 16; rounded to fp32 otherwise).
template <int D>
struct Feat {
    static_assert(D == 8 || D == 16 || D == 24 || D == 32, "feature dims 8, 16, 24, 32");
    static constexpr int kF = 1 + D + D * D;
    static constexpr float kPre = D == 8 ? 0.5946035575013605f
                                 : D == 16 ? 0.5f
                                 : D == 24 ? 0.45180100180492244f
                                           : 0.42044820762685725f;
};

// Taylor feature f (0..F-1) of a pre-scaled vector xs[D], feature order:
// 0 -> 1; 1+a -> xs[a]; 1+D+a*D+b -> xs[a]*xs[b]/sqrt2.
template <int D>
__device__ __forceinline__ float taylor_feature(const float* xs, int f) {
    if (f == 0) return 1.0f;
    if (f <= D) return xs[f - 1];
    const int r = f - 1 - D;
    return xs[r / D] * xs[r % D] * kInvSqrt2;
}

}  // namespace based
