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
#include "a8w8_quant_math.h"

namespace a8w8 {
namespace kern {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// One lane converts 8 consecutive values (16 bytes) of a group; the 16 lanes
// of a group take its amax with a DPP butterfly over the lanes (2.2 against
// 2.4 us at M = 16, K = 5120 with lane shuffles), then each forms s
// and its 8 codes; lane 0 of the group stores s.  Grid-stride over groups,
// four groups per lane and trip, their loads issued together so that enough
// bytes are in flight per CU; the 16 lanes of a group always agree on
// whether a group index is in range.
constexpr int kGroupsPerTrip = 4;

__device__ __forceinline__ void quant_group(u32x4 v, uint8_t *A, float *S, int64_t gi, int sub)
{
    const uint32_t w[4] = {v[0], v[1], v[2], v[3]};
    // the group's 16 lanes are one 16-lane row: DPP steps, smallest first
    float m = bf16_absmax(w);
    m = amax_step<1>(m);
    m = amax_step<2>(m);
    m = amax_step<4>(m);
    m = amax_step<8>(m);
    uint32_t c[2];
    const float s = quant_bf16(w, m, c);
    const u32x2 codes = {c[0], c[1]};
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
