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

// Two fp32 -> two e4m3 bytes in the low half (v_cvt_pk_fp8_f32, OCP e4m3fn,
// round to nearest even).
__device__ __forceinline__ uint32_t pack_fp8x2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four fp32 -> four e4m3 bytes.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
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

// v * 2^(127-b): exact (v_ldexp_f32).
__device__ __forceinline__ float unscale(float v, uint32_t b) {
    return __builtin_amdgcn_ldexpf(v, 127 - (int)b);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// DPP lane permutations (gfx9 encodings of the dpp_ctrl field).
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each 16 lanes

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

// Max over each aligned group of 32 lanes (all lanes get it): four DPP steps
// reduce each row of 16 lanes, one ds_swizzle (lane ^ 16 inside 32) joins the
// two rows.
__device__ __forceinline__ float half_wave_max(float v) {
    v = fmaxf(v, dpp<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp<kDppRowMirror>(v));
    // swizzle bitmask mode: and 0x1F, or 0, xor 0x10
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F)));
    return v;
}

// 4x4 transposes inside each quad of lanes.  Lane t of a quad holds element
// (t, q) of a 4x4 block in part q of its register(s); afterwards it holds
// element (q, t) in part q.  Two DPP exchanges (lane ^ 1, lane ^ 2) and
// v_perm_b32 byte selects; t is the lane's position in its quad.
__device__ __forceinline__ uint32_t quad_transpose_b8(uint32_t x, int t) {
    const uint32_t y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppQuadSwap1, 0xF, 0xF, false);
    const uint32_t r = __builtin_amdgcn_perm(y, x, (t & 1) ? 0x03070105u : 0x06020400u);
    const uint32_t z = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)r, kDppQuadSwap2, 0xF, 0xF, false);
    return __builtin_amdgcn_perm(z, r, (t & 2) ? 0x03020706u : 0x05040100u);
}

// Same for 16-bit elements: x0 = parts (0, 1), x1 = parts (2, 3).
__device__ __forceinline__ void quad_transpose_b16(uint32_t& x0, uint32_t& x1, int t) {
    // exchange 1: even lanes send their high halves, odd lanes their low halves
    const uint32_t send = __builtin_amdgcn_perm(x1, x0, (t & 1) ? 0x05040100u : 0x07060302u);
    const uint32_t recv = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send, kDppQuadSwap1, 0xF, 0xF, false);
    const uint32_t n0 = __builtin_amdgcn_perm(recv, x0, (t & 1) ? 0x03020504u : 0x05040100u);
    const uint32_t n1 = __builtin_amdgcn_perm(recv, x1, (t & 1) ? 0x03020706u : 0x07060100u);
    // exchange 2: lanes 0,1 send n1, lanes 2,3 send n0
    const uint32_t send2 = (t & 2) ? n0 : n1;
    const uint32_t recv2 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)send2, kDppQuadSwap2, 0xF, 0xF, false);
    x0 = (t & 2) ? recv2 : n0;
    x1 = (t & 2) ? n1 : recv2;
}

}  // namespace moe
