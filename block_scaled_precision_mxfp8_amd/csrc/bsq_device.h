// bsq_device.h -- device-side format codecs and wavefront helpers for gfx950 (CDNA4).
//
// Scale arithmetic is integer/bit manipulation or single IEEE binary32 operations; the
// per-element conversions use the gfx950 conversion instructions wrapped below, in the
// one way each of them matches the contract bit for bit.  The build disables FMA
// contraction (-ffp-contract=off) and keeps binary32 denormals (the default denormal mode
// of HIP device code on gfx950; subnormal scales and BF16 subnormal inputs rely on it).
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

// ----------------------------------------------------------------------------- gfx950 converts
//
// The scaled conversion instructions of gfx950 compute, with round-to-nearest-even,
//   to FP8/FP4:   ENC(x / 2^floor(log2 scale))   (FP8: NaN beyond 448; FP4: saturates at 6)
//   from FP8/FP4: DEC(code) * 2^floor(log2 scale)
// The kernels only use them where that is exactly the contract: MXFP8 encode (scale is
// the E8M0 power of two and |x / scale| <= 448 by construction), NVFP4 element encode
// (scale 1.0 on the already multiplied binary32 value), MXFP8 decode to BF16, NVFP4
// decode to binary32 (scale 1.0), and binary32 -> BF16.  The tests sweep each use
// exhaustively against the CPU oracle: every BF16 input at every E8M0 scale through the
// MXFP8 kernels, all 256 x 256 MXFP8 (code, scale) pairs through dequantization, and all
// 2^32 binary32 inputs for the FP4 encode and the BF16 rounding helpers below.

typedef short short2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

// Four E4M3 codes (little-endian bytes) of the BF16 pairs w0 = (x0, x1), w1 = (x2, x3)
// divided by `scale` (a power of two 2^(c-127); 2^-127 is the subnormal 0x00400000).
__device__ __forceinline__ uint32_t cvt_e4m3x4_bf16(uint32_t w0, uint32_t w1, float scale) {
    short2_t r = {0, 0};
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w0), scale, false);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, w1), scale, true);
    return __builtin_bit_cast(uint32_t, r);
}

// Byte `sel` of `old` replaced by the two E2M1 codes of a (low nibble) and b (high
// nibble): nearest, ties to the even code, sign kept, saturating at 6.
template <int sel>
__device__ __forceinline__ uint32_t cvt_e2m1x2_f32(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, sel);
}

// The two BF16 values (packed) of E4M3 codes in bytes 2*hi, 2*hi+1 of w times `scale`
// (a power of two), rounded to nearest-even.  NaN codes come out as 0xFFC0.
template <bool hi>
__device__ __forceinline__ uint32_t cvt_bf16x2_e4m3(uint32_t w, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, hi));
}

// The two binary32 values of the E2M1 codes in byte `sel` of w (exact).
template <int sel>
__device__ __forceinline__ float2_t cvt_f32x2_e2m1(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, sel);
}

// BF16 pair of two binary32 values, round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_bf16x2_f32(float a, float b) {
    float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ----------------------------------------------------------------------------- division

// Exact n / d for every 32-bit n and 1 <= d < 2^32 by one multiply-high: with
// c = ceil(2^64 / d), floor(n * c / 2^64) == floor(n / d) because c * d - 2^64 < d makes the
// error term n * (c - 2^64/d) / 2^64 < 2^32 / 2^64 < 1 / d.  The 96-bit product's top
// bits are m_hi * n + mulhi(m_lo, n), shifted by 32.  d == 1 is passed through.
struct FastDiv {
    uint32_t m_lo, m_hi, d;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    const uint64_t c = (d <= 1u) ? 0u : (UINT64_MAX / d + 1u);
    f.m_lo = (uint32_t)c;
    f.m_hi = (uint32_t)(c >> 32);
    return f;
}

__device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
    if (f.d == 1u) return n;
    const uint64_t t = (uint64_t)f.m_hi * n + (uint64_t)__umulhi(f.m_lo, n);
    return (uint32_t)(t >> 32);
}

// ----------------------------------------------------------------------------- launch limits

// Whether one launch of `workgroups` x `threads` can be dispatched: the x dimension of a
// grid holds at most 2^31 - 1 workgroups, and the dispatch packet counts the grid's
// work-items in 32 bits.  Each launcher states its grid through a *_launch_fits function
// that the C ABI calls before launching anything.
inline bool dispatch_fits(int64_t workgroups, int64_t threads) {
    return workgroups >= 0 && workgroups < (int64_t(1) << 31) && workgroups * threads < (int64_t(1) << 32);
}

// ----------------------------------------------------------------------------- streaming access

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Loads of inputs and stores of outputs that a kernel touches exactly once.  NT selects
// the non-temporal form (the caches do not keep the line for reuse); each kernel family
// picks its policy from measurements.
template <bool NT>
__device__ __forceinline__ void st_stream(uint32_t* p, uint32_t v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p); else *p = v;
}
template <bool NT>
__device__ __forceinline__ void st_stream(uint2* p, uint2 v) {
    if constexpr (NT) __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t*>(p));
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
    if constexpr (NT)
        __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
    else *p = v;
}
template <bool NT>
__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
    if constexpr (NT) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *p;
}
template <bool NT>
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
    if constexpr (NT) {
        const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        return make_uint2(v.x, v.y);
    }
    return *p;
}
template <bool NT>
__device__ __forceinline__ uint32_t ld_stream(const uint32_t* p) {
    if constexpr (NT) return __builtin_nontemporal_load(p);
    return *p;
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

// Max over the whole wave, returned uniform: quad max by DPP, then the half-row mirror
// (lane i <-> 7-i) and the row mirror (lane i <-> 15-i) give every lane its 16-lane row's
// max, and the four row results are read into scalars.
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
    v = quad_max(v);
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));  // row_half_mirror
    v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));  // row_mirror
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
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
