// bsq_device.h -- device-side format codecs and wavefront helpers for gfx950 (CDNA4).
//
// Every conversion here is integer/bit arithmetic or a single IEEE binary32 operation, so
// the results do not depend on any hardware conversion instruction.  The build disables
// FMA contraction (-ffp-contract=off); binary32 denormals are kept (the default denormal
// mode of HIP device code on gfx950), which the MXFP8 path relies on for BF16 subnormal
// inputs.
//
// Formats (page "Towards Blackwell-native 8-bit and 4-bit RL", section "Format
// background"): E4M3 = OCP E4M3FN, E8M0 = unsigned power of two, E2M1 = {0 .. 6}.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsq {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------------------- BF16

// Widen the low / high BF16 of a packed pair to binary32 bits (exact).
__device__ __forceinline__ uint32_t bf16_lo_bits(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t bf16_hi_bits(uint32_t w) { return w & 0xFFFF0000u; }

// Packed running maximum of BF16 magnitudes.  For finite BF16 the magnitude order is the
// unsigned order of (bits & 0x7FFF), so one packed u16 max per two elements suffices.
__device__ __forceinline__ uint32_t absmax2(uint32_t acc, uint32_t w) {
    u16x2 a = __builtin_bit_cast(u16x2, acc);
    u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

// Larger of the two halves of a packed magnitude pair.
__device__ __forceinline__ uint32_t fold2(uint32_t acc) {
    return max(acc & 0xFFFFu, acc >> 16);
}

// Round binary32 bits to BF16 (nearest, ties to even); finite values and infinities.
__device__ __forceinline__ uint32_t rne_bf16(uint32_t u) {
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ----------------------------------------------------------------------------- E8M0

// E8M0 code of a block from the BF16 magnitude bits of its amax: the smallest e >= -127
// with amax <= 448 * 2^e, as e + 127; zero gives 0.  With amax = (1 + m/128) * 2^(E-127)
// (E the BF16 exponent field) the condition holds for e = E - 135 exactly when
// 1 + m/128 <= 1.75, i.e. m <= 0x60; otherwise one more.  Subnormal or zero amax: 0.
__device__ __forceinline__ uint32_t e8m0_code_from_bf16_mag(uint32_t amax_bits) {
    int c = (int)(amax_bits >> 7) - 8 + ((amax_bits & 0x7Fu) > 0x60u ? 1 : 0);
    return (uint32_t)max(c, 0);
}

// binary32 value 2^(127 - c): the multiplier that maps a block into the E4M3 range.
// c <= 247 for finite BF16, so the exponent field 254 - c stays in 7..254 (normal).
__device__ __forceinline__ float e8m0_inverse(uint32_t c) {
    return __uint_as_float((254u - c) << 23);
}

// binary32 value 2^(c - 127) (c == 0 gives the subnormal 2^-127); c == 255 is NaN.
__device__ __forceinline__ float e8m0_decode(uint32_t c) {
    uint32_t bits = (c == 0u) ? 0x00400000u : (c << 23);
    return (c == 255u) ? __uint_as_float(0x7FC00000u) : __uint_as_float(bits);
}

// ----------------------------------------------------------------------------- E4M3

// E4M3 magnitude code of a >= 0 (binary32, not NaN): nearest finite value, ties to the
// even code, saturating at 448 (0x7E).
//  * a >= 2^-6 (normal E4M3): round the 23-bit mantissa to 3 bits on the bit pattern;
//    the biased E4M3 exponent is the binary32 one minus 120, carries propagate.
//  * a <  2^-6 (subnormal E4M3, step 2^-9): adding 2^14, whose binary32 ulp is 2^-9,
//    rounds a to a multiple of 2^-9 with round-to-nearest-even; the multiple is the code.
__device__ __forceinline__ uint32_t e4m3_code(float a) {
    uint32_t u = __float_as_uint(a);
    uint32_t cn = ((u + 0x7FFFFu + ((u >> 20) & 1u)) >> 20) - (120u << 3);
    uint32_t cs = __float_as_uint(a + 16384.0f) - 0x46800000u;
    uint32_t c = (a < 0.015625f) ? cs : cn;
    return min(c, 0x7Eu);
}

// binary32 value of an E4M3 magnitude code 0..0x7E (exact).
__device__ __forceinline__ float e4m3_decode_mag(uint32_t m) {
    uint32_t e = m >> 3, f = m & 7u;
    float sub = (float)f * 0.001953125f;                 // f * 2^-9, exact
    float nrm = __uint_as_float(((e + 120u) << 23) | (f << 20));
    return (e == 0u) ? sub : nrm;
}

// ----------------------------------------------------------------------------- E2M1

// E2M1 magnitude code of a >= 0 (binary32, not NaN): nearest of {0,.5,1,1.5,2,3,4,6},
// ties to the even code, saturating at 6 (code 7).
//  * a >= 1: round the mantissa to 1 bit on the bit pattern; code = (biased exponent -
//    126) * 2 + mantissa bit, i.e. (bits >> 22) - 252 after rounding.
//  * a < 1 (step 0.5): adding 2^22, whose binary32 ulp is 0.5, rounds a to a multiple of
//    0.5 with round-to-nearest-even; the multiple (0, 1 or 2) is the code.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
    uint32_t u = __float_as_uint(a);
    uint32_t cn = ((u + 0x1FFFFFu + ((u >> 22) & 1u)) >> 22) - 252u;
    uint32_t cs = __float_as_uint(a + 4194304.0f) - 0x4A800000u;
    uint32_t c = (a < 1.0f) ? cs : cn;
    return min(c, 7u);
}

// binary32 value of an E2M1 magnitude code 0..7 (exact).
__device__ __forceinline__ float e2m1_decode_mag(uint32_t m) {
    // codes >= 2 are normal: exponent field (m >> 1) + 126, mantissa bit m & 1 at bit 22,
    // which is (m + 252) << 22; code 1 is 0.5 and code 0 is 0.
    float nrm = __uint_as_float((m + 252u) << 22);
    return (m >= 2u) ? nrm : (m == 1u ? 0.5f : 0.0f);
}

// ----------------------------------------------------------------------------- lanes

// DPP quad permutations: value of the lane (i ^ 1) and (i ^ 2) within each quad.
#define BSQ_DPP_QUAD_XOR1 0xB1  // quad_perm [1,0,3,2]
#define BSQ_DPP_QUAD_XOR2 0x4E  // quad_perm [2,3,0,1]

__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, BSQ_DPP_QUAD_XOR1, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, BSQ_DPP_QUAD_XOR2, 0xF, 0xF, true);
}

// Max over each aligned group of 4 lanes (all lanes of the group receive it).
__device__ __forceinline__ uint32_t quad_max(uint32_t v) {
    v = max(v, dpp_xor1(v));
    return max(v, dpp_xor2(v));
}

// Max over each aligned pair of lanes.
__device__ __forceinline__ uint32_t pair_max(uint32_t v) {
    return max(v, dpp_xor1(v));
}

// Max over aligned groups of `width` lanes (power of two, <= 64) via lane shuffles.
template <int width>
__device__ __forceinline__ uint32_t group_max(uint32_t v) {
    v = max(v, dpp_xor1(v));
    v = max(v, dpp_xor2(v));
#pragma unroll
    for (int o = 4; o < width; o <<= 1)
        v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

}  // namespace bsq
