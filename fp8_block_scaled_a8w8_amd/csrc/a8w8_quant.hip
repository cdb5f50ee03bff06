// a8w8_quant.hip -- gfx950 kernel of the per-1x128 activation quantisation,
// the step upstream of the a8w8 block-scale GEMM: bf16 activations [M, K] ->
// e4m3fn codes [M, K] + one fp32 scale per 1 x 128 group.
//
// Per group: s = fp32(amax / 448); each value becomes the e4m3fn code nearest
// to clamp(fp32(x / s), -448, 448), ties to the even code, sign bit from the
// fp32 quotient; a group with amax 0 gets s = 0 and zero codes.  This is the
// reading of the activation operand that the GEMM's inputs are generated
// with (the pages name the operand "FP8" with per-group scales and stop
// there).  The quotient decides an integer code, so it is the correctly
// rounded fp32 quotient (see div_rn below).
//
// The kernel is HBM-bound: it reads 2 bytes and writes 1 + 4/128 bytes per
// element.  X, A and a_scale are walked as flat arrays of groups (row-major
// [M, K] with K a multiple of 128 puts group (m, g) at index m * K/128 + g),
// so every wave instruction moves whole 16-byte chunks of contiguous memory.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "a8w8_internal.h"

namespace a8w8 {
namespace kern {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

// One lane converts 8 consecutive values (16 bytes) of a group; the 16 lanes
// of a group take its amax with a butterfly over the lanes, then each forms s
// and its 8 codes; lane 0 of the group stores s.  Grid-stride over groups,
// four groups per lane and trip, their loads issued together so that enough
// bytes are in flight per CU; the 16 lanes of a group always agree on
// whether a group index is in range.
constexpr int kGroupsPerTrip = 4;

__device__ __forceinline__ void quant_group(u32x4 v, uint8_t *A, float *S, int64_t gi, int sub)
{
    float x[8] = {bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1]),
                  bf16_lo(v[2]), bf16_hi(v[2]), bf16_lo(v[3]), bf16_hi(v[3])};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, __shfl_xor(m, 8, 16));
    m = fmaxf(m, __shfl_xor(m, 4, 16));
    m = fmaxf(m, __shfl_xor(m, 2, 16));
    m = fmaxf(m, __shfl_xor(m, 1, 16));
    const float s = m / 448.0f;
    u32x2 codes = {0u, 0u};
    if (s >= 0x1p-126f) {
        const float r = 1.0f / s;
        codes[0] = pack4(x, s, r);
        codes[1] = pack4(x + 4, s, r);
    } else if (s > 0.0f) {
        // A subnormal scale (amax below 448 * 2^-126): full IEEE divisions.
        codes[0] = pack4_ieee(x, s);
        codes[1] = pack4_ieee(x + 4, s);
    }
    __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(A + gi * 128) + sub);
    if (sub == 0)
        S[gi] = s;
}

__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t *X, uint8_t *A, float *S, int64_t groups)
{
    const int sub = threadIdx.x & 15;
    const int64_t step = (int64_t)gridDim.x * (blockDim.x >> 4);
    for (int64_t g0 = (int64_t)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4); g0 < groups;
         g0 += kGroupsPerTrip * step) {
        u32x4 v[kGroupsPerTrip];
#pragma unroll
        for (int u = 0; u < kGroupsPerTrip; ++u) {
            const int64_t gi = g0 + u * step;
            if (gi < groups)
                v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X + gi * 128) + sub);
        }
#pragma unroll
        for (int u = 0; u < kGroupsPerTrip; ++u) {
            const int64_t gi = g0 + u * step;
            if (gi < groups)
                quant_group(v[u], A, S, gi, sub);
        }
    }
}

}  // namespace kern

hipError_t launch_quant_1x128(const void *X, void *A, float *a_scale, int64_t groups, int cus, hipStream_t stream)
{
    // Small problems: one group per lane group (more workgroups in flight);
    // large ones: a capped grid walks kGroupsPerTrip groups per trip.  The cap
    // grows with the problem -- 8, 16 or 32 workgroups per CU below 16, 64
    // and above 64 workgroups' worth of groups per CU -- the fastest of the
    // three measured at M = 1024 .. 16384 (K = 5120) and M = 8192, K = 7168.
    const int64_t wgs = (groups + 15) / 16;
    const int64_t c = cus > 0 ? cus : 256;
    const int64_t cap = c * (wgs >= 64 * c ? 32 : wgs >= 16 * c ? 16 : 8);
    const unsigned grid = (unsigned)(wgs < cap ? wgs : cap);
    hipLaunchKernelGGL(kern::quant_1x128_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(X), static_cast<uint8_t *>(A), a_scale, groups);
    return hipGetLastError();
}

}  // namespace a8w8
