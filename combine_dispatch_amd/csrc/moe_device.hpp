// moe_device.hpp -- device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }

// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    typedef float f2 __attribute__((ext_vector_type(2)));
    f2 v = {lo, hi};
    bf2 r = __builtin_convertvector(v, bf2);
    return __builtin_bit_cast(uint32_t, r);
}

// fp32 -> bf16 -> fp32 (the rounding the GEMM epilogue applies).
__device__ __forceinline__ float round_bf16(float v) {
    return __uint_as_float(pack_bf16x2(v, 0.f) << 16);
}

// UE8M0 scale byte for an e4m3 group: the smallest b with
// amax <= 448 * 2^(b-127), from the fp32 fields of amax: exponent field
// minus 8, plus one when the significand exceeds 1.75 (448 = 1.75 * 2^8).
__device__ __forceinline__ uint32_t ue8m0_e4m3(float amax) {
    const uint32_t bits = __float_as_uint(amax);
    int b = (int)((bits >> 23) & 0xFFu) - 8 + ((bits & 0x7FFFFFu) > 0x600000u ? 1 : 0);
    b = b < 0 ? 0 : (b > 254 ? 254 : b);
    return (uint32_t)b;
}

// Same from the bits of a non-negative finite amax, in three integer ops:
// adding 0x1FFFFF carries into the exponent field exactly when the
// significand field exceeds 0x600000, and the 8 << 23 taken off first makes
// the (arithmetic) shift give the exponent minus 8 directly.
__device__ __forceinline__ uint32_t ue8m0_e4m3_bits(uint32_t bits) {
    const int b = (int)(bits + 0x1FFFFFu - (8u << 23)) >> 23;
    return (uint32_t)(b < 0 ? 0 : (b > 254 ? 254 : b));
}

// Bytes (0, 1, 2, 3) -> (0, 2, 1, 3): the order of k-blocks inside a packed
// scale word.
__device__ __forceinline__ uint32_t swap_bytes12(uint32_t v) {
    return (v & 0xFF0000FFu) | ((v >> 8) & 0x0000FF00u) | ((v << 8) & 0x00FF0000u);
}

// e4m3 bytes of v * 2^(127-s) for a UE8M0 scale byte s, the scaling done by
// the conversion itself (v_cvt_scalef32_pk_fp8_f32 divides by its scale
// operand; an fp32 whose exponent field is s is 2^(s-127), s = 0 included).
// Measured on gfx950: the same bytes as v_ldexp_f32 by 127-s followed by
// v_cvt_pk_fp8_f32, on 2^21 pairs of exact codes, ties, e4m3 subnormals and
// other values, over scale bytes 0..254.
typedef short short2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_fp8x2_scaled(float a, float b, uint32_t s) {
    const short2_t z = {0, 0};
    const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, __uint_as_float(s << 23), false);
    return (uint32_t)(uint16_t)r.x;
}
__device__ __forceinline__ uint32_t pack_fp8x4_scaled(float a, float b, float c, float d, uint32_t s) {
    const float sc = __uint_as_float(s << 23);
    const short2_t z = {0, 0};
    const short2_t lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, a, b, sc, false);
    const short2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, c, d, sc, true);
    return (uint32_t)(uint16_t)r.x | ((uint32_t)(uint16_t)r.y << 16);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// DPP lane permutations (gfx9 encodings of the dpp_ctrl field).
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Max over the 4 lanes of an aligned quad (all lanes get it).
__device__ __forceinline__ float quad_max(float v) {
    v = fmaxf(v, dpp<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp<kDppQuadSwap2>(v));
    return v;
}

// Max over each aligned group of 8 lanes of four non-negative values held as
// float bits (unsigned order = float order), all lanes get them: mirror
// inside the 8, then the two quad swaps; the four chains interleave.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ void group8_max_u32x4(uint32_t (&m)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = max(m[q], dpp_u32<kDppRowHalfMirror>(m[q]));
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = max(m[q], dpp_u32<kDppQuadSwap1>(m[q]));
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = max(m[q], dpp_u32<kDppQuadSwap2>(m[q]));
}

// Max over each aligned group of 32 lanes of four non-negative values held as
// float bits: the 8-lane max, then lane i <-> 15-i inside each 16 (DPP row
// mirror), then the two 16-lane halves of each 32 (ds_swizzle, xor 16).
constexpr int kDppRowMirror = 0x140;
constexpr int kSwizzleXor16 = 0x401F;  // bit-mask mode: and 0x1F, or 0, xor 0x10
__device__ __forceinline__ void group32_max_u32x4(uint32_t (&m)[4]) {
    group8_max_u32x4(m);
#pragma unroll
    for (int q = 0; q < 4; ++q) m[q] = max(m[q], dpp_u32<kDppRowMirror>(m[q]));
#pragma unroll
    for (int q = 0; q < 4; ++q)
        m[q] = max(m[q], (uint32_t)__builtin_amdgcn_ds_swizzle((int)m[q], kSwizzleXor16));
}

// Max over each aligned group of 8 lanes (all lanes get it): mirror inside
// the 8, then the two quad swaps.
__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp<kDppQuadSwap2>(v));
    return v;
}

}  // namespace moe
