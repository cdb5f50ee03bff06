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
// Read-only global data read through the constant address space: wave-uniform
// loads from it become scalar loads.
typedef const __attribute__((address_space(4))) float const_f32;

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

// Copy block kb into one LDS stage with direct-to-LDS loads: A_LOADS + W_LOADS
// 16-byte loads (each wave instruction writes 1 KB = 8 rows x 128 bytes at
// consecutive LDS addresses, lane i at byte 16 i), then one 4-byte load of 64
// activation-scale values (lane i -> float i).  Every wave issues exactly
// A_LOADS + W_LOADS + 1 vector-memory instructions per block, which is what the
// counted waits in the main loop rely on.
//
// The copies are written as inline asm on purpose: the compiler treats every
// LDS read as possibly aliasing every copy still in flight and would wait for
// all of them before the first fragment read, collapsing the ring to depth 1.
// The asm has no register outputs (only the address and the LDS base, which
// the hardware reads at issue), and the kernel's own counted waits below are
// what order the copies against the reads.
__device__ __forceinline__ void lds_copy16(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ void lds_copy4(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off" : : "s"(m0), "v"(src) : "memory", "m0");
}

template <int A_LOADS, int W_LOADS>
__device__ __forceinline__ void issue_tile_loads(const uint8_t *const (&a_src)[A_LOADS],
                                                 const uint8_t *const (&w_src)[W_LOADS], const float *as_src,
                                                 int kb, uint8_t *stage, int a_bytes, int w_bytes, int wave)
{
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
        lds_copy16(a_src[i] + (size_t)kb * 128, stage + (wave * A_LOADS + i) * 1024);
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i)
        lds_copy16(w_src[i] + (size_t)kb * 128, stage + a_bytes + (wave * W_LOADS + i) * 1024);
    lds_copy4(as_src + kb, stage + a_bytes + w_bytes + wave * 256);
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    // s_waitcnt immediate (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// LDS tiles are row-major 128-byte rows whose 16-byte chunk c sits at chunk
// position c ^ chunk_swizzle(row).  A fragment read has lane (g = l/16,
// p = l%16) read chunk 2g (then 2g+1) of row r0 + p; with this swizzle those
// 16-byte reads are free of LDS bank conflicts (measured with the LDS bank
// conflict counter over candidate placements: plain r & 7 still costs 1.33
// extra cycles per read).  Rows are 16-aligned in every read, so the pattern
// only needs to be a bijection on each row.
__device__ __forceinline__ int chunk_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// MFMA operand of this lane: logical chunks 2g and 2g+1 (K bytes 32g..32g+31)
// of tile row `row`.
__device__ __forceinline__ v8i lds_fragment(const uint8_t *tile, int row, int g)
{
    const uint8_t *rp = tile + row * 128;
    const int x = chunk_swizzle(row);
    const v4i lo = *reinterpret_cast<const v4i *>(rp + (((2 * g) ^ x) << 4));
    const v4i hi = *reinterpret_cast<const v4i *>(rp + (((2 * g + 1) ^ x) << 4));
    return cat(lo, hi);
}

// Tile index of workgroup `b` among T tiles: workgroups are dispatched to the
// 8 XCDs round-robin (b % 8), so each XCD is given a contiguous range of tile
// ids; inside it, tiles run in groups of G tile-rows, column by column, so the
// workgroups that are resident together on one XCD share A rows and W rows in
// that XCD's L2.  A bijection on [0, T): results do not depend on it.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, int G, int &tm, int &tn)
{
    const int T = tiles_m * tiles_n;
    const int xcd = b & 7, local = b >> 3;
    const int q = T >> 3, r = T & 7;
    const int t = xcd * q + min(xcd, r) + local;
    const int per_group = G * tiles_n;
    const int group = t / per_group;
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// ---------------------------------------------------------------------------
// Tile kernel.  A workgroup of WGM x WGN waves owns a BM x BN output tile and
// walks K one 128-wide scale block at a time through a STAGES-deep ring of LDS
// buffers: block kb+STAGES-1 is copied global -> LDS (direct-to-LDS loads, no
// VGPR staging) while block kb is multiplied.  Each wave owns a
// (BM/WGM) x (BN/WGN) sub-tile: per block it reads its W and A fragments from
// LDS, takes one MFMA per 16 x 16 output, and folds the result into the fp32
// accumulator with the block's a_scale * w_scale.  The MFMAs of 16-row slice
// t+1 are issued before the scale FMAs of slice t consume slice t's results,
// so the matrix core and the VALU work overlap.
//
// LDS stage: A tile [BM][128] | W tile [BN][128] | activation scales
// [64 * waves] floats, tiles swizzled as described at chunk_swizzle().
template <int BM, int BN, int WGM, int WGN, int STAGES>
__global__ __launch_bounds__(WGM * WGN * 64) void tile_kernel(Args p, int vec_store)
{
    constexpr int NWAVES = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
    constexpr int STAGE = A_BYTES + W_BYTES + NWAVES * 256;
    constexpr int A_LOADS = BM / (8 * NWAVES), W_LOADS = BN / (8 * NWAVES);   // 1 KB loads per wave per block
    constexpr int PER_BLOCK = A_LOADS + W_LOADS + 1;                         // vector-memory ops per block
    static_assert(A_LOADS >= 1 && W_LOADS >= 1 && BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0,
                  "each wave copies whole 8-row groups of both tiles");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile is made of 16 x 16 MFMA outputs");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-row weight block");
    static_assert(STAGES >= 2 && (STAGES - 2) * PER_BLOCK < 64, "ring depth");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
    int tmi, tni;
    tile_coords((int)blockIdx.x, tiles_m, tiles_n, BM >= 256 ? 2 : 4, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int r16 = lane & 15, g = lane >> 4;

    // Direct-load sources: lane covers row (lane >> 3) of an 8-row group and
    // physical chunk (lane & 7), which holds logical chunk (lane & 7) ^ swizzle(row).
    const int lrow = lane >> 3, pch = lane & 7;
    const uint8_t *a_src[A_LOADS];
    const uint8_t *w_src[W_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const int row = (wave * A_LOADS + i) * 8 + lrow;
        a_src[i] = p.A + (size_t)min(m0 + row, M - 1) * K + ((pch ^ chunk_swizzle(row)) << 4);
    }
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i) {
        const int row = (wave * W_LOADS + i) * 8 + lrow;
        w_src[i] = p.W + (size_t)min(n0 + row, N - 1) * K + ((pch ^ chunk_swizzle(row)) << 4);
    }
    // Activation scales: wave w copies tile rows 64w + lane (rows past the tile
    // or past M repeat a valid row and are never read).
    const float *as_src = p.a_scale + (size_t)min(m0 + min(wave * 64 + lane, BM - 1), M - 1) * KB;
    const int NB = (N + 127) >> 7;
    const_f32 *wsp = (const_f32 *)(p.w_scale + (size_t)min((n0 + wn * WN) >> 7, NB - 1) * KB);

    v4f acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    // Prologue: blocks 0 .. STAGES-2 in flight (indices past the end repeat the last block).
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
        issue_tile_loads<A_LOADS, W_LOADS>(a_src, w_src, as_src, min(s, KB - 1), smem + s * STAGE, A_BYTES,
                                           W_BYTES, wave);
    float ws_next = wsp[0];

    for (int kb = 0; kb < KB; ++kb) {
        const float ws = ws_next;
        wait_vmcnt<(STAGES - 2) * PER_BLOCK>();   // this wave's copies of block kb have landed
        __syncthreads();                          // ... every wave's, and stage (kb-1) % STAGES is free
        const int kn = min(kb + STAGES - 1, KB - 1);
        issue_tile_loads<A_LOADS, W_LOADS>(a_src, w_src, as_src, kn, smem + ((kb + STAGES - 1) % STAGES) * STAGE,
                                           A_BYTES, W_BYTES, wave);
        ws_next = wsp[min(kb + 1, KB - 1)];

        const uint8_t *sA = smem + (kb % STAGES) * STAGE;
        const uint8_t *sW = sA + A_BYTES;
        const float *sS = reinterpret_cast<const float *>(sW + W_BYTES);
        float sc[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t)
            sc[t] = sS[wm * WM + 16 * t + r16] * ws;
        v8i wf[TN];
#pragma unroll
        for (int u = 0; u < TN; ++u)
            wf[u] = lds_fragment(sW, wn * WN + 16 * u + r16, g);
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
    wait_vmcnt<0>();                      // no copy into LDS may outlive the workgroup

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
#define A8W8_TILE_INST(BM, BN, WGM, WGN, S) template __global__ void tile_kernel<BM, BN, WGM, WGN, S>(Args, int);
A8W8_TILE_INST(256, 256, 2, 4, 2)
A8W8_TILE_INST(256, 128, 2, 4, 3)
A8W8_TILE_INST(128, 256, 2, 4, 3)
A8W8_TILE_INST(128, 128, 2, 2, 2)
A8W8_TILE_INST(128, 128, 2, 2, 4)
A8W8_TILE_INST(128, 64, 2, 2, 3)
A8W8_TILE_INST(64, 128, 2, 2, 3)
A8W8_TILE_INST(64, 64, 2, 2, 3)
A8W8_TILE_INST(256, 32, 4, 1, 3)
A8W8_TILE_INST(128, 32, 4, 1, 3)
A8W8_TILE_INST(32, 128, 1, 4, 3)
A8W8_TILE_INST(32, 64, 2, 2, 3)
A8W8_TILE_INST(64, 32, 2, 2, 3)
A8W8_TILE_INST(32, 32, 2, 2, 3)
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
#define TILE(BM, BN, WGM, WGN, S) {{A8W8_KERNEL_TILE, BM, BN, WGM * WGN, S, 0, \
                                    "tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_s" #S}, \
                                   reinterpret_cast<const void *>(&tile_kernel<BM, BN, WGM, WGN, S>), \
                                   S * ((BM + BN) * 128 + WGM * WGN * 256)}

const Entry kEntries[] = {
    SKINNY(1, 5, 8), SKINNY(2, 5, 8), SKINNY(4, 5, 8), SKINNY(1, 6, 8), SKINNY(2, 6, 8),
    SKINNY(1, 3, 16), SKINNY(2, 3, 16), SKINNY(1, 10, 4), SKINNY(1, 12, 4), SKINNY(1, 2, 4),
    TILE(256, 256, 2, 4, 2), TILE(256, 128, 2, 4, 3), TILE(128, 256, 2, 4, 3), TILE(128, 128, 2, 2, 2),
    TILE(128, 128, 2, 2, 4), TILE(128, 64, 2, 2, 3), TILE(64, 128, 2, 2, 3), TILE(64, 64, 2, 2, 3),
    TILE(256, 32, 4, 1, 3), TILE(128, 32, 4, 1, 3), TILE(32, 128, 1, 4, 3), TILE(32, 64, 2, 2, 3),
    TILE(64, 32, 2, 2, 3), TILE(32, 32, 2, 2, 3),
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
