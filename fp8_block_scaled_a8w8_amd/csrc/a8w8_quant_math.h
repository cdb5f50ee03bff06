// a8w8_quant_math.h -- the per-1x128 activation quantisation arithmetic,
// shared by the standalone quantisation kernel (a8w8_quant.hip) and the
// decode kernel's fused bf16-activation mode (a8w8_kernels.hip), so that both
// produce the same codes and scales bit for bit.
//
// Per group: s = fp32(amax / 448); each value becomes the e4m3fn code nearest
// to clamp(fp32(x / s), -448, 448), ties to the even code, sign bit from the
// fp32 quotient; a group with amax 0 gets s = 0 and zero codes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace a8w8 {
namespace kern {

// e4m3fn bytes of finite fp32 values, rounded to nearest with ties to even,
// magnitudes above 448 saturating to 448: clamp to [-448, 448] (one med3) and
// convert with gfx950's v_cvt_pk_fp8_f32, two values per instruction.  On
// [-448, 448] the conversion is exactly the e4m3fn round-to-nearest-even
// encoding (bias 7, 3 mantissa bits, multiples of 2^-9 below 2^-6, sign of
// -0 kept): a device check compared it with a bit-level software encoder for
// every fp32 value in [0, 448] and its negative, with no difference.
__device__ __forceinline__ uint32_t e4m3fn_pack4(float q0, float q1, float q2, float q3)
{
    const float c0 = __builtin_amdgcn_fmed3f(q0, -448.0f, 448.0f), c1 = __builtin_amdgcn_fmed3f(q1, -448.0f, 448.0f);
    const float c2 = __builtin_amdgcn_fmed3f(q2, -448.0f, 448.0f), c3 = __builtin_amdgcn_fmed3f(q3, -448.0f, 448.0f);
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, lo, true);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 x / s rounded to nearest even, given r = RN(1/s) for a normal s > 0:
// q = RN(x r) is within one ulp of x/s, the residual x - q s is exact with an
// FMA, and one correction q + (x - q s) r rounded once gives RN(x/s)
// (Markstein's theorem for FMA division: reciprocal correctly rounded,
// first quotient within one ulp, no overflow; the quotients here stay
// within 448 in magnitude).  The sign is copied from x so that x = -0 gives
// -0, as the division does (the FMAs would return +0).  Four instructions
// instead of a full division.
__device__ __forceinline__ float div_rn(float x, float s, float r)
{
    const float q = x * r;
    const float e = __builtin_fmaf(-q, s, x);
    return __builtin_copysignf(__builtin_fmaf(e, r, q), x);
}

__device__ __forceinline__ uint32_t pack4(const float *x, float s, float r)
{
    return e4m3fn_pack4(div_rn(x[0], s, r), div_rn(x[1], s, r), div_rn(x[2], s, r), div_rn(x[3], s, r));
}

__device__ __forceinline__ uint32_t pack4_ieee(const float *x, float s)
{
    return e4m3fn_pack4(x[0] / s, x[1] / s, x[2] / s, x[3] / s);
}

// One step of a max-butterfly over lanes: each lane takes the larger of its
// value and that of lane l ^ MASK.  Within a row of 16 lanes the partner comes
// through DPP: quad_perm for 1 and 2, then the half-row mirror for 4 and the
// row mirror for 8 (lane i of 8 reads lane 7 - i, of 16 lane 15 - i), which
// give the same maxima as l ^ 4 and l ^ 8 once the smaller steps are done, as
// every lane of a 4- or 8-lane group then holds one value.  16 and 32 cross
// rows: ds_bpermute.
template <int MASK>
__device__ __forceinline__ float amax_step(float m)
{
    const int v = __float_as_int(m);
    int o;
    if constexpr (MASK == 1)
        o = __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);    // quad_perm [1,0,3,2]
    else if constexpr (MASK == 2)
        o = __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);    // quad_perm [2,3,0,1]
    else if constexpr (MASK == 4)
        o = __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);   // row_half_mirror
    else if constexpr (MASK == 8)
        o = __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);   // row_mirror
    else
        o = __shfl_xor(v, MASK);
    return fmaxf(m, __int_as_float(o));
}

// Largest |x| over this lane's bf16 values (two per word, any subset of a
// group): finite bf16 magnitudes order as their low 15 bits read as integers,
// so the maximum is taken on the bits (no conversions kept live).  Non-finite
// inputs give an unspecified result.
template <int W>
__device__ __forceinline__ float bf16_absmax(const uint32_t (&w)[W])
{
    uint32_t mb = 0u;
#pragma unroll
    for (int i = 0; i < W; ++i) {
        const uint32_t a = w[i] & 0x7fff7fffu;
        mb = max(mb, max(a & 0xffffu, a >> 16));
    }
    return __uint_as_float(mb << 16);
}

// The codes and scale of one group, given this lane's bf16 values of it (W
// words, two values each, the lower K in the low half) and the group's amax
// already reduced over its lanes: codes[i] packs the values of words 2i and
// 2i+1, lowest K in the low byte (W = 1: the low two bytes of codes[0]).
// Returns s.
template <int W>
__device__ __forceinline__ float quant_bf16(const uint32_t (&w)[W], float amax, uint32_t (&codes)[(W + 1) / 2])
{
    const float s = amax / 448.0f;
#pragma unroll
    for (int i = 0; i < (W + 1) / 2; ++i)
        codes[i] = 0u;
    if (s >= 0x1p-126f) {
        const float r = 1.0f / s;
#pragma unroll
        for (int i = 0; i < (W + 1) / 2; ++i) {
            const uint32_t w1 = 2 * i + 1 < W ? w[2 * i + 1] : 0u;
            const float x[4] = {bf16_lo(w[2 * i]), bf16_hi(w[2 * i]), bf16_lo(w1), bf16_hi(w1)};
            codes[i] = pack4(x, s, r);
        }
    } else if (s > 0.0f) {
        // A subnormal scale (amax below 448 * 2^-126): full IEEE divisions.
#pragma unroll
        for (int i = 0; i < (W + 1) / 2; ++i) {
            const uint32_t w1 = 2 * i + 1 < W ? w[2 * i + 1] : 0u;
            const float x[4] = {bf16_lo(w[2 * i]), bf16_hi(w[2 * i]), bf16_lo(w1), bf16_hi(w1)};
            codes[i] = pack4_ieee(x, s);
        }
    }
    return s;
}

}  // namespace kern
}  // namespace a8w8
