// a8w8_quant.hip -- gfx950 kernel of the per-1x128 activation quantisation,
// the step upstream of the a8w8 block-scale GEMM: bf16 activations [M, K] ->
// e4m3fn codes [M, K] + one fp32 scale per 1 x 128 group.
//
// Per group: s = fp32(amax / 448); each value becomes the e4m3fn code nearest
// to clamp(fp32(x / s), -448, 448), ties to the even code, sign bit from the
// fp32 quotient; a group with amax 0 gets s = 0 and zero codes.  This is the
// reading of the activation operand that the GEMM's inputs are generated
// with (the pages name the operand "FP8" with per-group scales and stop
// there).  The quotient uses IEEE division (hipcc's correctly rounded
// default), because it decides an integer code.
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

// e4m3fn byte of a finite fp32 value inside [-448, 448]: round to nearest,
// ties to even.  Bias 7, 3 mantissa bits; below 2^-6 the values are the
// multiples of 2^-9 (codes 0..7, and 8 = 2^-6 is the smallest normal); the
// largest finite value 448 is code 0x7E.
__device__ __forceinline__ uint32_t e4m3fn_rne(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t code;
    if (a < 0x3c800000u) {                             // |y| < 2^-6
        code = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);   // exact product, ties to even
    } else {
        const uint32_t e = (a >> 23) - 120u;           // biased e4m3 exponent: (e8 - 127) + 7
        uint32_t r = (a >> 20) & 7u;                   // top three fp32 mantissa bits
        const uint32_t rest = a & 0xfffffu;            // the 20 bits rounded away
        r += (rest > 0x80000u || (rest == 0x80000u && (r & 1u))) ? 1u : 0u;
        code = (e << 3) + r;                           // r == 8 carries into the exponent
    }
    return sign | code;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack4(const float *x, float s)
{
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        c |= e4m3fn_rne(fminf(fmaxf(x[i] / s, -448.0f), 448.0f)) << (8 * i);
    return c;
}

// One lane converts 8 consecutive values (16 bytes) of a group; the 16 lanes
// of a group take its amax with a butterfly over the lanes, then each forms s
// and its 8 codes; lane 0 of the group stores s.  Grid-stride over groups:
// the 16 lanes of a group always take the same loop trip count.
__global__ __launch_bounds__(256) void quant_1x128_kernel(const uint16_t *X, uint8_t *A, float *S, int64_t groups)
{
    const int sub = threadIdx.x & 15;
    const int64_t step = (int64_t)gridDim.x * (blockDim.x >> 4);
    for (int64_t gi = (int64_t)blockIdx.x * (blockDim.x >> 4) + (threadIdx.x >> 4); gi < groups; gi += step) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(X + gi * 128) + sub);
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
        if (s > 0.0f) {
            codes[0] = pack4(x, s);
            codes[1] = pack4(x + 4, s);
        }
        __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(A + gi * 128) + sub);
        if (sub == 0)
            S[gi] = s;
    }
}

}  // namespace kern

hipError_t launch_quant_1x128(const void *X, void *A, float *a_scale, int64_t groups, int cus, hipStream_t stream)
{
    const int64_t wgs = (groups + 15) / 16;              // 16 groups per 256-thread workgroup
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * 8;
    const unsigned grid = (unsigned)(wgs < cap ? wgs : cap);
    hipLaunchKernelGGL(kern::quant_1x128_kernel, dim3(grid), dim3(256), 0, stream,
                       static_cast<const uint16_t *>(X), static_cast<uint8_t *>(A), a_scale, groups);
    return hipGetLastError();
}

}  // namespace a8w8
