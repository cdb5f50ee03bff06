// read_ceiling.hip -- a plain streaming read, the measured ceiling the decode
// kernels are compared with (a measurement aid for the benchmark, not part of
// the GEMM library).
//
// Workgroup i (256 lanes) reads the i-th of `grid` contiguous slices of the
// buffer with 16-byte non-temporal loads, U loads per lane in flight, and
// folds them into an XOR.  The XOR is stored (to sink[i]) only when it equals
// a fixed constant, so the loads cannot be dropped and nearly nothing is
// written.  The benchmark times it on rotated copies of the decode's byte
// count with the same HIP-graph method as the GEMM and keeps the best of a
// few grids.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4r __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void read_kernel(const u32x4r *p, int64_t n16, int64_t per_wg, uint32_t *sink)
{
    const int64_t lo = (int64_t)blockIdx.x * per_wg;
    const int64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
    uint32_t x = 0;
    for (int64_t base = lo; base < hi; base += 256 * U) {
        u32x4r v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = i < hi ? __builtin_nontemporal_load(p + i) : (u32x4r){0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    if (x == 0x9e3779b9u)
        sink[blockIdx.x] = x;
}

}  // namespace

// Read `bytes` (a multiple of 16) at `buf` once; `sink` holds `grid` words.
// unroll is 8 or 16.  Returns 0 or the HIP error of the launch.
extern "C" int a8w8_read_ceiling_launch(const void *buf, int64_t bytes, void *sink, int grid, int unroll,
                                        void *stream)
{
    if (buf == nullptr || sink == nullptr || bytes <= 0 || (bytes & 15) || grid < 1 || (unroll != 8 && unroll != 16))
        return (int)hipErrorInvalidValue;
    const int64_t n16 = bytes / 16;
    const int64_t per_wg = (n16 + grid - 1) / grid;
    const u32x4r *p = static_cast<const u32x4r *>(buf);
    uint32_t *s = static_cast<uint32_t *>(sink);
    if (unroll == 8)
        hipLaunchKernelGGL(read_kernel<8>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), p, n16, per_wg, s);
    else
        hipLaunchKernelGGL(read_kernel<16>, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), p, n16, per_wg, s);
    return (int)hipGetLastError();
}
