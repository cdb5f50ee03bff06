// a8w8_kernels.hip -- gfx950 kernels of the a8w8 block-scale GEMM.
//
// Y[m,n] = bf16( sum_kb (sum_{k in kb} A[m,k] W[n,k]) * a_scale[m,kb] * w_scale[n/128,kb] )
// with A, W OCP fp8 E4M3 (row-major, K contiguous) and 128-wide K blocks, the
// operation the "[Perf] Retune gfx942 Qwen3.8-27B a8w8 blockscale decode rows
// for cold weights" page tunes (Kernel section).
//
// Both kernels are built on v_mfma_f32_16x16x128_f8f6f4: one instruction takes
// a 16 x 128 fp8 W slice and a 16 x 128 fp8 A slice, i.e. exactly one
// 128-wide scale block, and returns the 16 x 16 block dot in fp32.  The block
// scale is then applied with one FMA per output into an fp32 accumulator, so
// no second ("per block") accumulator set is ever held in registers.
//
// Operand roles: the MFMA "A" operand is W (rows n), the "B" operand is the
// activation (columns m).  Lane l of a wave holds, for both operands, row
// (l % 16) of its 16-row slice and the 32 K bytes [32*(l/16), 32*(l/16)+32) of
// the block; its 4 results are D[n = 4*(l/16)+i][m = l%16], i = 0..3.  So one
// lane's outputs share one activation row, and a single a_scale value per
// (lane, block) suffices.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "a8w8_internal.h"
#include "gemm_a8w8_blockscale.h"

namespace a8w8 {
namespace kern {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

__device__ __forceinline__ v4f mfma_block(v8i w, v8i a)
{
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    // Format codes 0/0: both operands fp8 E4M3; zero scale operands select the
    // unscaled instruction.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, z, 0, 0, 0, 0, 0, 0);
}

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0, 32-bit data
// format word of the CDNA buffer resource).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ v8i cat(v4i lo, v4i hi)
{
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ v4f fma4(v4f d, float s, v4f acc)
{
    acc[0] = __builtin_fmaf(d[0], s, acc[0]);
    acc[1] = __builtin_fmaf(d[1], s, acc[1]);
    acc[2] = __builtin_fmaf(d[2], s, acc[2]);
    acc[3] = __builtin_fmaf(d[3], s, acc[3]);
    return acc;
}

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return 0x7fc0u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Store the 4 consecutive columns n..n+3 of row m (n < N checked per element
// unless the vector path is allowed and all four exist).
__device__ __forceinline__ void store4(uint16_t *Y, int64_t row_off, int n, int N, bool vec, v4f v)
{
    const uint32_t b0 = bf16_rne(v[0]), b1 = bf16_rne(v[1]);
    const uint32_t b2 = bf16_rne(v[2]), b3 = bf16_rne(v[3]);
    if (vec && n + 3 < N) {
        uint2 pk;
        pk.x = b0 | (b1 << 16);
        pk.y = b2 | (b3 << 16);
        *reinterpret_cast<uint2 *>(Y + row_off + n) = pk;
    } else {
        if (n < N) Y[row_off + n] = (uint16_t)b0;
        if (n + 1 < N) Y[row_off + n + 1] = (uint16_t)b1;
        if (n + 2 < N) Y[row_off + n + 2] = (uint16_t)b2;
        if (n + 3 < N) Y[row_off + n + 3] = (uint16_t)b3;
    }
}

// ---------------------------------------------------------------------------
// Skinny kernel, M <= 16 (decode): stream every byte of W from HBM exactly
// once with as many bytes in flight as possible.
//
// A workgroup owns RG = 16*TPW rows of W (TPW 16-row tiles) and all of K; its
// NW waves split the K blocks into contiguous runs of D blocks (more passes
// if NW*D < K/128).  A wave issues all loads of a pass at once -- per block one
// activation fragment and TPW weight fragments -- and one activation fragment
// feeds TPW MFMAs.  Per block: one MFMA per tile, then one FMA per output with
// a_scale * w_scale.  The NW wave partials of each tile are summed through LDS
// in wave order (fixed order: bitwise deterministic), rounded once to bf16.
//
// Weight loads cover whole 128-byte lines: load 0 of a block takes rows 0-7 of
// the 16-row tile and load 1 rows 8-15, lane (rho = l/16, p = l%16) reading
// chunk 2 rho + (p >= 8) of row (p & 7) (+8).  A row_ror:8 DPP exchange between
// lanes p and p+8 of each 16-lane row then leaves lane l with row l%16, bytes
// [32 rho, 32 rho + 32) of the block -- the MFMA operand layout.  Streaming
// whole lines per instruction is what lets the loads run at the HBM ceiling;
// the half-line pattern of a direct MFMA-layout load measured ~35% slower.
__device__ __forceinline__ v8i fix_row_layout(v4i v0, v4i v1)
{
    // lanes 8-15 of each row take v1 from lane p-8; lanes 0-7 take v0 from lane p+8
    v4i a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __builtin_amdgcn_update_dpp(v0[i], v1[i], 0x128, 0xF, 0xC, false);
        b[i] = __builtin_amdgcn_update_dpp(v1[i], v0[i], 0x128, 0xF, 0x3, false);
    }
    return cat(a, b);
}

template <int TPW, int D, int NW>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(Args p, int vec_store)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int n0 = (int)blockIdx.x * (16 * TPW);
    const int r16 = lane & 15, g = lane >> 4;
    const bool mval = r16 < M;

    // Whole-line load addressing (see fix_row_layout): load h of a block takes
    // row 8h + (r16 & 7), 16-byte chunk 2g + (r16 >> 3).  Loads go through
    // buffer descriptors: a 32-bit per-lane offset (the host keeps N*K and
    // M*K below 2^32) plus the wave-uniform block offset kb*128.
    const int lrow = r16 & 7;
    const uint32_t lcol = (uint32_t)(2 * g + (r16 >> 3)) * 16;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.W, (uint32_t)N * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)K);
    uint32_t woff[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[t][h] = (uint32_t)min(n0 + 16 * t + 8 * h + lrow, N - 1) * (uint32_t)K + lcol;
    // Activation rows past M load row 0: they only feed output columns that are never stored.
    uint32_t aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int m = 8 * h + lrow;
        aoff[h] = (uint32_t)(m < M ? m : 0) * (uint32_t)K + lcol;
    }
    const float *asp = p.a_scale + (size_t)(mval ? r16 : 0) * KB;
    // RG divides 128, so the row group lies in one 128-row weight block.
    const float *wsp = p.w_scale + (size_t)(n0 >> 7) * KB;

    v4f acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};

    for (int kb_begin = wave * D; kb_begin < KB; kb_begin += NW * D) {
        v4i ar[D][2];
        v4i wr[D][TPW][2];
        float sa[D], sw[D];
        // Issue every load of the pass before consuming any of them.
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = min(kb_begin + j, KB - 1);   // blocks past the end load a valid block, skipped below
            const int koff = kb * 128;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wr[j][t][h] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woff[t][h], koff, 2 /* nt */);
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ar[j][h] = __builtin_amdgcn_raw_buffer_load_b128(ares, (int)aoff[h], koff, 0);
            sa[j] = asp[kb];
            sw[j] = wsp[kb];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (kb_begin + j < KB) {
                const v8i af = fix_row_layout(ar[j][0], ar[j][1]);
                const float sc = sa[j] * sw[j];
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    acc[t] = fma4(mfma_block(fix_row_layout(wr[j][t][0], wr[j][t][1]), af), sc, acc[t]);
            }
        }
    }

    const bool vec = vec_store != 0;
    if constexpr (NW > 1) {
        __shared__ v4f red[NW][TPW][64];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            red[wave][t][lane] = acc[t];
        __syncthreads();
        for (int t = wave; t < TPW; t += NW) {
            v4f v = red[0][t][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const v4f o = red[w][t][lane];
                v[0] += o[0];
                v[1] += o[1];
                v[2] += o[2];
                v[3] += o[3];
            }
            if (mval)
                store4(p.Y, (int64_t)r16 * N, n0 + 16 * t + 4 * g, N, vec, v);
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            if (mval)
                store4(p.Y, (int64_t)r16 * N, n0 + 16 * t + 4 * g, N, vec, acc[t]);
    }
}

// Copy block kb of the A and W tiles into LDS stage `base` with direct-to-LDS
// 16-byte loads: each wave instruction writes 1 KB (8 rows x 128 bytes) at
// consecutive LDS addresses, lane i at byte 16 i.
template <int A_LOADS, int W_LOADS>
__device__ __forceinline__ void issue_tile_loads(const uint8_t *const (&a_src)[A_LOADS],
                                                 const uint8_t *const (&w_src)[W_LOADS], int kb,
                                                 uint8_t *base, int a_bytes, int wave)
{
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
        __builtin_amdgcn_global_load_lds(a_src[i] + (size_t)kb * 128,
                                         (lds_ptr_t)(base + (wave * A_LOADS + i) * 1024), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i)
        __builtin_amdgcn_global_load_lds(w_src[i] + (size_t)kb * 128,
                                         (lds_ptr_t)(base + a_bytes + (wave * W_LOADS + i) * 1024), 16, 0, 0);
}

// MFMA operand of this lane: logical chunks 2g and 2g+1 (K bytes 32g..32g+31)
// of tile row `row`, undoing the chunk ^ (row & 7) placement.
__device__ __forceinline__ v8i lds_fragment(const uint8_t *tile, int row, int g)
{
    const uint8_t *rp = tile + row * 128;
    const int x = row & 7;
    const v4i lo = *reinterpret_cast<const v4i *>(rp + (((2 * g) ^ x) << 4));
    const v4i hi = *reinterpret_cast<const v4i *>(rp + (((2 * g + 1) ^ x) << 4));
    return cat(lo, hi);
}

// ---------------------------------------------------------------------------
// Tile kernel.  A workgroup of 4 waves (2 x 2) owns a BM x BN output tile and
// walks K one 128-wide block at a time.  The A [BM x 128] and W [BN x 128]
// fp8 tiles of block kb+1 are copied global -> LDS with direct-to-LDS 16-byte
// loads (no VGPR staging) while block kb is multiplied from the other LDS
// buffer.  Each wave owns a (BM/2) x (BN/2) sub-tile: per block it reads its W
// and A fragments from LDS, takes one MFMA per 16 x 16 output, and folds the
// result into the fp32 accumulator with the block's a_scale * w_scale.
//
// LDS layout of one tile: row-major 128-byte rows; the 16-byte chunk c of row
// r is stored at chunk position c ^ (r & 7), so the 8 rows that a direct load
// writes, and the 16 rows a fragment read touches, spread over the banks.
template <int BM, int BN>
__global__ __launch_bounds__(256) void tile_kernel(Args p, int vec_store)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128, STAGE = A_BYTES + W_BYTES;
    constexpr int A_LOADS = BM / 32, W_LOADS = BN / 32;   // 1 KB direct loads per wave per stage
    static_assert(BM % 32 == 0 && BN % 32 == 0, "tile dims must be multiples of 32");
    static_assert(WN <= 128, "a wave's columns must lie in one 128-row weight block");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (int)(blockIdx.x / tiles_n) * BM;
    const int n0 = (int)(blockIdx.x % tiles_n) * BN;
    const int r16 = lane & 15, g = lane >> 4;

    // Direct-load sources: lane covers row (lane >> 3) of an 8-row group and
    // physical chunk (lane & 7), which holds logical chunk (lane & 7) ^ row.
    const int lrow = lane >> 3, pch = lane & 7;
    const uint8_t *a_src[A_LOADS];
    const uint8_t *w_src[W_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const int row = (wave * A_LOADS + i) * 8 + lrow;
        const int grow = min(m0 + row, M - 1);
        a_src[i] = p.A + (size_t)grow * K + ((pch ^ lrow) << 4);
    }
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i) {
        const int row = (wave * W_LOADS + i) * 8 + lrow;
        const int grow = min(n0 + row, N - 1);
        w_src[i] = p.W + (size_t)grow * K + ((pch ^ lrow) << 4);
    }

    // Scales: one activation row per lane per 16-row slice; one weight block per wave.
    int a_off[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
        a_off[t] = min(m0 + wm * WM + 16 * t + r16, M - 1) * KB;
    const int NB = (N + 127) >> 7;
    const float *wsp = p.w_scale + (size_t)min((n0 + wn * WN) >> 7, NB - 1) * KB;

    v4f acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    float sa[TM];
    float ws;
    issue_tile_loads<A_LOADS, W_LOADS>(a_src, w_src, 0, smem, A_BYTES, wave);
#pragma unroll
    for (int t = 0; t < TM; ++t)
        sa[t] = p.a_scale[a_off[t]];
    ws = wsp[0];

    for (int kb = 0; kb < KB; ++kb) {
        float sc[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t)
            sc[t] = sa[t] * ws;
        __builtin_amdgcn_s_waitcnt(0);    // this wave's copies of block kb have landed
        __syncthreads();                  // ... and every wave's; buffer (kb+1)&1 is free
        // Prefetch block kb+1 (the last iteration re-fetches block KB-1 into the
        // idle buffer, which keeps the loop body branch-free).
        const int kn = min(kb + 1, KB - 1);
        issue_tile_loads<A_LOADS, W_LOADS>(a_src, w_src, kn, smem + ((kb + 1) & 1) * STAGE, A_BYTES, wave);
#pragma unroll
        for (int t = 0; t < TM; ++t)
            sa[t] = p.a_scale[a_off[t] + kn];
        ws = wsp[kn];

        const uint8_t *sA = smem + (kb & 1) * STAGE;
        const uint8_t *sW = sA + A_BYTES;
        v8i wf[TN];
#pragma unroll
        for (int u = 0; u < TN; ++u)
            wf[u] = lds_fragment(sW, wn * WN + 16 * u + r16, g);
        // Software pipeline over the 16-row activation slices: the MFMAs of
        // slice t+1 are issued before the scale FMAs of slice t consume the
        // results of slice t, so the matrix core never waits on the VALU.
        v4f d[2][TN];
        {
            const v8i af = lds_fragment(sA, wm * WM + r16, g);
#pragma unroll
            for (int u = 0; u < TN; ++u)
                d[0][u] = mfma_block(wf[u], af);
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t + 1 < TM) {
                const v8i af = lds_fragment(sA, wm * WM + 16 * (t + 1) + r16, g);
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    d[(t + 1) & 1][u] = mfma_block(wf[u], af);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u)
                acc[t][u] = fma4(d[t & 1][u], sc[t], acc[t][u]);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);        // no copy into LDS may outlive the workgroup

#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int m = m0 + wm * WM + 16 * t + r16;
        if (m < M) {
#pragma unroll
            for (int u = 0; u < TN; ++u)
                store4(p.Y, (int64_t)m * N, n0 + wn * WN + 16 * u + 4 * g, N, vec_store != 0, acc[t][u]);
        }
    }
}

// Explicit instantiations (emit the host-side launch stubs).
#define A8W8_TILE_INST(BM, BN) template __global__ void tile_kernel<BM, BN>(Args, int);
A8W8_TILE_INST(256, 128)
A8W8_TILE_INST(128, 128)
A8W8_TILE_INST(128, 64)
A8W8_TILE_INST(64, 128)
A8W8_TILE_INST(64, 64)
A8W8_TILE_INST(256, 32)
A8W8_TILE_INST(128, 32)
A8W8_TILE_INST(32, 128)
A8W8_TILE_INST(32, 64)
A8W8_TILE_INST(64, 32)
A8W8_TILE_INST(32, 32)
#undef A8W8_TILE_INST

}  // namespace kern

namespace {

using namespace kern;

// ---------------------------------------------------------------------------
// Instance table.

struct Entry {
    Variant v;
    const void *fn;
    int lds_bytes;
};

#define SKINNY(TPW, D, NW) {{A8W8_KERNEL_SKINNY, 16, 16 * TPW, NW, D, 16, "skinny_r" #TPW "_d" #D "_w" #NW}, \
                            reinterpret_cast<const void *>(&skinny_kernel<TPW, D, NW>), 0}
#define TILE(BM, BN) {{A8W8_KERNEL_TILE, BM, BN, 4, 1, 0, "tile_" #BM "x" #BN}, \
                       reinterpret_cast<const void *>(&tile_kernel<BM, BN>), 2 * (BM + BN) * 128}

const Entry kEntries[] = {
    SKINNY(1, 5, 8), SKINNY(2, 5, 8), SKINNY(4, 5, 8), SKINNY(1, 6, 8), SKINNY(2, 6, 8),
    SKINNY(1, 3, 16), SKINNY(2, 3, 16), SKINNY(1, 10, 4), SKINNY(1, 12, 4), SKINNY(1, 2, 4),
    TILE(256, 128), TILE(128, 128), TILE(128, 64), TILE(64, 128), TILE(64, 64),
    TILE(256, 32), TILE(128, 32), TILE(32, 128), TILE(32, 64), TILE(64, 32), TILE(32, 32),
};
constexpr int kNumEntries = sizeof(kEntries) / sizeof(kEntries[0]);

}  // namespace

int num_variants() { return kNumEntries; }

const Variant &variant(int id) { return kEntries[id].v; }

int64_t variant_grid(int id, int64_t M, int64_t N, int64_t K)
{
    (void)K;
    const Variant &v = kEntries[id].v;
    if (v.kernel == A8W8_KERNEL_SKINNY)
        return (N + v.bn - 1) / v.bn;
    return ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
}

int64_t variant_passes(int id, int64_t K)
{
    const Variant &v = kEntries[id].v;
    if (v.kernel != A8W8_KERNEL_SKINNY)
        return K / 128;
    const int64_t per_pass = (int64_t)v.waves * v.kblocks;
    return (K / 128 + per_pass - 1) / per_pass;
}

hipError_t set_kernel_attributes()
{
    for (int i = 0; i < kNumEntries; ++i) {
        if (kEntries[i].lds_bytes > 0) {
            hipError_t e = hipFuncSetAttribute(kEntries[i].fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               kEntries[i].lds_bytes);
            if (e != hipSuccess)
                return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_variant(int id, const Args &a, hipStream_t stream)
{
    const Entry &e = kEntries[id];
    const int64_t grid = variant_grid(id, a.M, a.N, a.K);
    int vec = ((reinterpret_cast<uintptr_t>(a.Y) & 7) == 0 && (a.N & 3) == 0) ? 1 : 0;
    Args args = a;
    void *params[] = {&args, &vec};
    return hipLaunchKernel(e.fn, dim3((unsigned)grid), dim3(e.v.waves * 64), params,
                           (size_t)e.lds_bytes, stream);
}

}  // namespace a8w8
