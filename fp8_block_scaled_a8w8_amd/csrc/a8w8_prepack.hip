// a8w8_prepack.hip -- offline weight layout for gfx950: row-major e4m3fn W
// [N, K] -> the packed (fragment-order) layout the GEMM kernels can read.
//
// Packed layout: rows padded with zeros to N' = 16 * ceil(N / 16); for every
// 16-row tile t and 128-wide K block kb, 2048 bytes at offset
// (t * K/128 + kb) * 2048, ordered [h][lane][16 bytes] with lane l (0..63)
// holding row 16 t + l % 16, bytes 16 (l / 16) + 64 h .. + 16 of the block.
// That is the operand layout of v_mfma_f32_16x16x128_f8f6f4 in the
// instruction's own K order (lane l: row l % 16, 16-byte K chunks l / 16 and
// l / 16 + 4), split into two contiguous kilobytes, so a wave loads a whole
// fragment with two contiguous 16-byte-per-lane loads and no lane exchange --
// the "pre-shuffled weights" idea, laid out for this MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "a8w8_internal.h"

namespace a8w8 {
namespace kern {

typedef uint32_t u32x4p __attribute__((ext_vector_type(4)));

// One thread writes one 16-byte piece of the packed matrix (grid-stride).
__global__ __launch_bounds__(256) void prepack_kernel(const uint8_t *W, uint8_t *Wp, int N, int K, int64_t pieces)
{
    const int KB = K >> 7;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < pieces; o += step) {
        const int64_t blk = o >> 7;                    // 128 pieces per 2 KB block
        const int within = (int)(o & 127);
        const int h = within >> 6, lane = within & 63;
        const int64_t tile = blk / KB;
        const int kb = (int)(blk - tile * KB);
        const int64_t row = tile * 16 + (lane & 15);
        const int col = kb * 128 + 16 * (lane >> 4) + 64 * h;
        u32x4p v = {0u, 0u, 0u, 0u};
        if (row < N)
            v = *reinterpret_cast<const u32x4p *>(W + row * K + col);
        *reinterpret_cast<u32x4p *>(Wp + o * 16) = v;
    }
}

}  // namespace kern

hipError_t launch_prepack(const void *W, void *Wp, int64_t N, int64_t K, int cus, hipStream_t stream)
{
    const int64_t pieces = ((N + 15) / 16) * 16 * K / 16;
    const int64_t wgs = (pieces + 255) / 256;
    const int64_t cap = (int64_t)(cus > 0 ? cus : 256) * 16;
    hipLaunchKernelGGL(kern::prepack_kernel, dim3((unsigned)(wgs < cap ? wgs : cap)), dim3(256), 0, stream,
                       static_cast<const uint8_t *>(W), static_cast<uint8_t *>(Wp), (int)N, (int)K, pieces);
    return hipGetLastError();
}

}  // namespace a8w8
