// cu_capacity.hip -- what one compute unit moves per clock through the three
// data paths the tile kernels are built on (a measurement aid for the
// benchmark, not part of the GEMM library):
//
//   lds_read   16-byte LDS reads into registers (the MFMA fragment reads),
//   vmem_load  16-byte vector-memory loads into registers from an L2-resident
//              buffer (the skinny kernels' path),
//   lds_dma    16-byte direct-to-LDS copies from the same buffer (the tile
//              kernels' copy path: buffer_load_dwordx4 ... lds).
//
// Every workgroup has 16 waves and asks for 96 KB of LDS, more than half of a
// CU's 160 KB, so no two workgroups share a CU.  After a barrier the group
// reads the shader-clock counter (s_memtime) and the 100 MHz real-time counter
// (s_memrealtime), runs a fixed loop, waits for everything it issued, meets at
// a barrier again and reads both counters once more; wave 0 stores the two
// differences.  Bytes moved per workgroup are fixed by the arguments, so the
// host gets bytes per clock per CU, and the clock the part ran at, from these
// two counts alone.
//
// Loaded values are handed to an empty asm statement, which keeps every load
// without adding VALU work that could become the limit.  Every address is in
// bounds: LDS offsets are masked into the workgroup's allocation, and the
// vector-memory loads go through a buffer descriptor sized to the buffer
// (anything past it would read zeros).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int NW = 16;                   // waves per workgroup
constexpr int LDS_BYTES = 96 * 1024;     // per workgroup: one workgroup per CU
constexpr int READ_SPAN = 64 * 1024;     // LDS bytes the read loop walks over

__device__ __forceinline__ void keep(v4i v)
{
    asm volatile("" : : "v"(v));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void stamp(uint64_t &c, uint64_t &r)
{
    c = __builtin_amdgcn_s_memtime();
    r = __builtin_amdgcn_s_memrealtime();
}

// out[2 b] = shader-clock cycles, out[2 b + 1] = real-time ticks of workgroup b's loop.
__device__ __forceinline__ void finish(uint64_t c0, uint64_t r0, uint64_t *out)
{
    __syncthreads();
    uint64_t c1, r1;
    stamp(c1, r1);
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = c1 - c0;
        out[2 * blockIdx.x + 1] = r1 - r0;
    }
}

// Read u of a step of lane l, wave w: 16 bytes at
// ((w * 1024 + step * 9216) mod 32 KB) + 4096 u + 16 l, below 61 KB: each
// instruction covers one contiguous kilobyte (no bank conflicts), the eight
// reads of a step take one address and eight immediate offsets, and
// consecutive steps move to other kilobytes.
__global__ __launch_bounds__(NW * 64) void lds_read_kernel(int iters, uint64_t *out)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    for (int i = threadIdx.x; i < READ_SPAN / 16; i += NW * 64)
        reinterpret_cast<v4i *>(smem)[i] = (v4i){i, 3 * i, 5 * i, 7 * i};
    __syncthreads();
    uint64_t c0, r0;
    stamp(c0, r0);
    const uint32_t base = (threadIdx.x >> 6) * 1024u + (threadIdx.x & 63) * 16u;
    for (int it = 0; it < iters; ++it) {
        v4i v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t off = ((base + (uint32_t)it * 9216u) & 0x7FFFu) + 4096u * u;
            v[u] = *reinterpret_cast<const v4i *>(smem + off);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            keep(v[u]);
    }
    finish(c0, r0, out);
}

// Lane l of wave w of workgroup b loads 16 bytes at byte
// ((b * NW + w) * 8 + u + 8 * NW * it) * 1024 + 16 l, wrapped to the buffer (a
// power of two), 8 loads in flight per wave.
__global__ __launch_bounds__(NW * 64) void vmem_load_kernel(const void *src, uint32_t bytes, int iters, uint64_t *out)
{
    const __amdgpu_buffer_rsrc_t r = rsrc(src, bytes);
    const uint32_t mask = bytes - 1u;
    const uint32_t w = blockIdx.x * NW + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    __syncthreads();
    uint64_t c0, r0;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
        v4i v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t kb = w * 8u + (uint32_t)u + 8u * NW * (uint32_t)it;
            v[u] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(((kb * 1024u) & mask) + lane * 16u), 0, 0);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            keep(v[u]);
    }
    finish(c0, r0, out);
}

// The same source addresses as vmem_load_kernel, copied straight into LDS: copy
// u of a step goes to kilobyte (w * 4 + u % 4) of the workgroup's allocation
// (16 waves x 4 KB = 64 KB < 96 KB).  The LDS address goes through m0, which
// needs one wait state before the copy reads it; a scalar register written by
// a VALU instruction (readfirstlane) needs five before a vector-memory
// instruction reads it: s_nop 4 covers both.  At most 16 copies are left in
// flight per wave at each step's end (the counter holds 63).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(r)
                 : "memory", "m0");
}

__global__ __launch_bounds__(NW * 64) void lds_dma_kernel(const void *src, uint32_t bytes, int iters, uint64_t *out)
{
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const __amdgpu_buffer_rsrc_t r = rsrc(src, bytes);
    const uint32_t mask = bytes - 1u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t w = blockIdx.x * NW + wave, lane = threadIdx.x & 63;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)smem;
    __syncthreads();
    uint64_t c0, r0;
    stamp(c0, r0);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t kb = w * 8u + (uint32_t)u + 8u * NW * (uint32_t)it;
            dma16(r, ((kb * 1024u) & mask) + lane * 16u, lds0 + (wave * 4u + (uint32_t)(u & 3)) * 1024u);
        }
        asm volatile("s_waitcnt vmcnt(16)" : : : "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
    finish(c0, r0, out);
}

}  // namespace

// Which: 0 = LDS reads, 1 = vector-memory loads, 2 = direct-to-LDS copies.
// `grid` workgroups of 16 waves, `iters` steps of 8 16-byte operations per
// lane; src (kinds 1, 2) holds `bytes` bytes, a power of two from 64 KB to
// 256 MB; out holds 2 * grid words.  Bytes moved per workgroup:
// a8w8_cu_capacity_bytes(iters).  Returns 0 or a HIP error code.
extern "C" double a8w8_cu_capacity_bytes(int iters)
{
    return (double)NW * 64.0 * 16.0 * 8.0 * (double)iters;
}

extern "C" int a8w8_cu_capacity_launch(int which, const void *src, int64_t bytes, void *out, int grid, int iters,
                                       void *stream)
{
    if (out == nullptr || grid < 1 || iters < 1 || which < 0 || which > 2)
        return (int)hipErrorInvalidValue;
    if (which > 0 && (src == nullptr || bytes < 65536 || bytes > ((int64_t)1 << 28) || (bytes & (bytes - 1)) != 0))
        return (int)hipErrorInvalidValue;
    // 96 KB of dynamic LDS is above the launch default: allow it once per kernel.
    static const hipError_t attr = [] {
        for (const void *fn : {reinterpret_cast<const void *>(&lds_read_kernel),
                               reinterpret_cast<const void *>(&vmem_load_kernel),
                               reinterpret_cast<const void *>(&lds_dma_kernel)}) {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }();
    if (attr != hipSuccess)
        return (int)attr;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    uint64_t *o = static_cast<uint64_t *>(out);
    const uint32_t b = (uint32_t)bytes;
    if (which == 0)
        hipLaunchKernelGGL(lds_read_kernel, dim3(grid), dim3(NW * 64), LDS_BYTES, s, iters, o);
    else if (which == 1)
        hipLaunchKernelGGL(vmem_load_kernel, dim3(grid), dim3(NW * 64), LDS_BYTES, s, src, b, iters, o);
    else
        hipLaunchKernelGGL(lds_dma_kernel, dim3(grid), dim3(NW * 64), LDS_BYTES, s, src, b, iters, o);
    return (int)hipGetLastError();
}
