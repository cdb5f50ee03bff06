// mfma_ceiling.hip -- the sustained fp8 MFMA rate of the part, the measured
// compute ceiling the large-M GEMM is compared with (a measurement aid for the
// benchmark, not part of the GEMM library).
//
// Every wave loads two operand fragments of real fp8 data (the benchmark passes
// weight bytes), then issues `iters` rounds of CHAINS independent
// v_mfma_f32_16x16x128_f8f6f4 instructions, each accumulating in place into
// its own 16 x 16 fp32 tile; the operands rotate between rounds so no round is
// a repeat of the last.  With two waves per SIMD and CHAINS independent
// accumulators per wave the matrix core always has an instruction ready, so
// the time is the MFMA issue rate at whatever clock the part sustains under
// this load with realistic (not zero) operands.  The accumulators are folded
// and stored only when the result equals a fixed constant, so nothing is
// dropped and nearly nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int CHAINS = 8;

__global__ __launch_bounds__(256) void mfma_ceiling_kernel(const v8i *src, int64_t nfrag, int iters, float *sink)
{
    // fragment pair of this wave: 2w and 2w + 1, w < nfrag / 2 (nfrag >= 2)
    const int64_t w = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) % (nfrag / 2);
    const int lane = threadIdx.x & 63;
    v8i a = src[(2 * w) * 64 + lane];
    v8i b = src[(2 * w + 1) * 64 + lane];
    v4f acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
        acc[c] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < CHAINS; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
        // rotate the operand words (cheap, keeps the data realistic and changing)
        const v8i t = a;
        a = __builtin_shufflevector(b, b, 1, 2, 3, 4, 5, 6, 7, 0);
        b = t;
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
        s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    if (s == 1.2345678e30f)
        sink[blockIdx.x] = s;
}

}  // namespace

// Flops one launch performs: grid workgroups x 4 waves x iters x CHAINS x 16*16*128*2.
extern "C" double a8w8_mfma_ceiling_flops(int grid, int iters)
{
    return (double)grid * 4.0 * (double)iters * CHAINS * 16.0 * 16.0 * 128.0 * 2.0;
}

// Launch `grid` workgroups of 4 waves; `src` holds `nfrag` 2 KB operand fragments
// (nfrag >= 2), `sink` grid floats.  Returns 0 or the HIP error of the launch.
extern "C" int a8w8_mfma_ceiling_launch(const void *src, int64_t nfrag, void *sink, int grid, int iters,
                                        void *stream)
{
    if (src == nullptr || sink == nullptr || nfrag < 2 || grid < 1 || iters < 1)
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const v8i *>(src), nfrag, iters, static_cast<float *>(sink));
    return (int)hipGetLastError();
}
