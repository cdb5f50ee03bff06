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
// (l % 16) of its 16-row slice and two 16-byte K chunks of the block: chunk
// g = l/16 (K bytes 16g..16g+15) in its first four registers and chunk g + 4
// (K bytes 64+16g..) in the last four -- the K order the instruction itself
// uses (measured: a byte's position selects its 32-wide scale group exactly
// so).  Its 4 results are D[n = 4*(l/16)+i][m = l%16], i = 0..3.  So one
// lane's outputs share one activation row, and a single a_scale value per
// (lane, block) suffices.
//
// MX-scaled variant (compile-time MX): the mxfp8 GEMM with 32 x 32
// weight-scale blocks of the gfx1250 BF16 and MX32 tuned-rows page (ROCm/aiter
// #7247, Motivation and Technical Details), read with OCP MX scales: one E8M0
// byte (2^(e-127)) per activation row and 32-wide K group and per 32 x 32
// weight block.  A row of such scales holds K/32 bytes = K/128 32-bit words,
// word kb packing the four groups of K block kb (lowest K in the low byte), so
// every kernel fetches MX scale words exactly where it fetches fp32 block
// scales (weight rows counted per 32 instead of per 128).  The instruction
// takes the scale of its K group q (K bytes 32q..32q+31 in its own K order,
// which the operand layout below follows) from lane 16q + row, so lane l hands
// byte l/16 of its words to the scaled MFMA, which applies both operands'
// 2^(e-127) itself and accumulates in place: no per-block scale FMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "a8w8_internal.h"
#include "a8w8_quant_math.h"
#include "gemm_a8w8_blockscale.h"

// Timeline build (-DA8W8_TIMELINE, a separate library that diagnostics load):
// the row-range skinny kernel stamps the 100 MHz real-time counter at five
// points of every wave -- entry, first pass issued, last data consumed, after
// the reduction barrier, after its store -- and its hardware id, into the
// call's workspace ([workgroup][wave][6] 64-bit words from ws on) when one is
// given.  The product library compiles none of it.
#ifdef A8W8_TIMELINE
#define A8W8_TL(...) __VA_ARGS__
#else
#define A8W8_TL(...)
#endif

namespace a8w8 {
namespace kern {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
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

// MX block step: acc += the block's 16 x 16 dot with every operand group
// scaled by its E8M0 value.  w_word / a_word are the 32-bit scale words (in
// float registers, never used as numbers) of the lane's weight row and
// activation row; byte g = l/16 is the lane's K group.  Scale operand "a"
// belongs to the first MFMA operand (W), "b" to the second (activations).
__device__ __forceinline__ v4f mfma_mx(v8i w, v8i a, v4f acc, float w_word, float a_word, int g)
{
    const int ws = (int)(__float_as_uint(w_word) >> (8 * g));
    const int as = (int)(__float_as_uint(a_word) >> (8 * g));
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, acc, 0, 0, 0, ws, 0, as);
}

// Scale kinds (compile-time SM of every kernel):
//   SM_BLOCK   fp32 scales per 1 x 128 activation group and 128 x 128 weight block;
//   SM_MX      E8M0 scales per 1 x 32 activation group and 32 x 32 weight block;
//   SM_ROWWISE fp32 scale per activation row and per weight row (output
//              channel): the MFMAs accumulate the unscaled dot over all of K
//              and the epilogue multiplies by a_scale[m] * w_scale[n].
constexpr int SM_BLOCK = 0, SM_MX = 1, SM_ROWWISE = 2;

// One K block into the accumulator: block scale (the fp32 product of the two
// scales, one FMA per output), MX (E8M0 scales inside the MFMA) or row-wise
// (unscaled, in place).
template <int SM>
__device__ __forceinline__ v4f block_step(v4f acc, v8i w, v8i a, float sw, float sa, int g)
{
    if constexpr (SM == SM_MX) {
        return mfma_mx(w, a, acc, sw, sa, g);
    } else if constexpr (SM == SM_ROWWISE) {
        // zero scale operands select the unscaled instruction
        return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, acc, 0, 0, 0, 0, 0, 0);
    } else {
        return fma4(mfma_block(w, a), sa * sw, acc);
    }
}

// Weight rows covered by one per-block scale row: 128 (block scale) or 32 (MX).
template <int SM>
constexpr int wscale_shift() { return SM == SM_MX ? 5 : 7; }

// Row-wise kind: a lane's outputs for row m, columns n..n+3 times
// a_scale[m] * w_scale[n + i] (as (v * a) * w), before rounding.  m < M.
template <int SM>
__device__ __forceinline__ v4f rowwise_scale(v4f v, const Args &p, int m, int n)
{
    if constexpr (SM == SM_ROWWISE) {
        const float sa = p.a_scale[m];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < p.N)
                v[i] = (v[i] * sa) * p.w_scale[n + i];
    }
    return v;
}

// The same scales fetched ahead of time (the weight-streaming kernels load
// them before their K loop, so the epilogue waits for no memory): row m's
// a_scale (0 past M) and w_scale of columns n..n+3 (0 past N).
struct RowScales {
    float a, w[4];
};
template <int SM>
__device__ __forceinline__ RowScales rowwise_fetch(const Args &p, int m, int n)
{
    RowScales r = {0.f, {0.f, 0.f, 0.f, 0.f}};
    if constexpr (SM == SM_ROWWISE) {
        if (m < p.M)
            r.a = p.a_scale[m];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (n + i < p.N)
                r.w[i] = p.w_scale[n + i];
    }
    return r;
}
template <int SM>
__device__ __forceinline__ v4f rowwise_apply(v4f v, const RowScales &r)
{
    if constexpr (SM == SM_ROWWISE) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            v[i] = (v[i] * r.a) * r.w[i];
    }
    return v;
}

// Batched launches: batch blockIdx.y works on its own slice of every array.
__device__ __forceinline__ void select_batch(Args &p)
{
    const int64_t z = (int64_t)blockIdx.y;
    p.A += z * p.bs_a;
    p.a_scale += z * p.bs_as;
    p.W += z * p.bs_w;
    p.w_scale += z * p.bs_ws;
    p.Y += z * p.bs_y;
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
// Split instances (SK) give each of S workgroups per row group 1/S of K and
// combine their sums through the workspace in split order before rounding.
//
// Weight loads cover whole 128-byte lines: load 0 of a block takes rows 0-7 of
// the 16-row tile and load 1 rows 8-15, lane (rho = l/16, p = l%16) reading
// chunk rho + 4 (p >= 8) of row (p & 7) (+8).  A row_ror:8 DPP exchange between
// lanes p and p+8 of each 16-lane row then leaves lane l with row l%16, chunks
// rho and rho + 4 of the block -- the MFMA operand layout.  Streaming
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

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    // s_waitcnt immediate (gfx9): vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] << 14
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Packed weights (the optional offline layout a8w8_prepack_weights writes):
// rows padded with zeros to a multiple of 16; for every 16-row tile t and K
// block kb, 2 KB in MFMA operand order, [h][lane][16 bytes], lane l holding
// row 16t + l%16, 16-byte chunk l/16 + 4h of the block.  A wave then reads
// each half of a fragment (1 KB) with one contiguous load and needs no lane
// exchange.  Byte offset of tile t, block kb:
__device__ __forceinline__ uint32_t packed_block(uint32_t tile, uint32_t kb, uint32_t KB)
{
    return (tile * KB + kb) << 11;
}
// Weight fragment from its two 16-byte loads (row layout needs the lane exchange).
__device__ __forceinline__ v8i w_fragment(v4i w0, v4i w1, bool pk)
{
    return pk ? cat(w0, w1) : fix_row_layout(w0, w1);
}
// Weight rows the buffer holds: padded to a multiple of 16 when packed.
template <bool PK>
__device__ __forceinline__ uint32_t w_rows(const Args &p)
{
    return PK ? (uint32_t)((p.N + 15) & ~15) : (uint32_t)p.N;
}

template <int TPW, int D, int NW, bool SK, bool PK, int SM>
__global__ __launch_bounds__(NW * 64) void skinny_kernel(Args p, int vec_store)
{
    select_batch(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    // Split K (SK instances, p.splits = S > 1): workgroup i takes row group
    // i / S and the K blocks [s KB / S, (s + 1) KB / S) of split s = i % S; the
    // partial sums meet in the fixed-order reduction at the end.  Other
    // instances fold S = 1 at compile time.
    const int S = SK ? p.splits : 1;
    const int tile = (int)blockIdx.x / S, split = (int)blockIdx.x - tile * S;
    const int kb_lo = split * KB / S, kb_hi = (split + 1) * KB / S;
    const int n0 = tile * (16 * TPW);
    const int r16 = lane & 15, g = lane >> 4;
    const bool mval = r16 < M;

    // Whole-line load addressing (see fix_row_layout): load h of a block takes
    // row 8h + (r16 & 7), 16-byte chunk g + 4 (r16 >> 3).  Loads go through
    // buffer descriptors: a 32-bit per-lane offset (the host keeps N*K and
    // M*K below 2^32) plus the wave-uniform block offset kb*128.
    const int lrow = r16 & 7;
    const uint32_t lcol = (uint32_t)(g + 4 * (r16 >> 3)) * 16;
    constexpr bool pk = PK;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.W, w_rows<PK>(p) * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)K);
    // Row layout: per-lane row offsets, block offset kb * 128.  Packed: lane l
    // reads bytes 16 l (+1024 for the second half) of the tile's block.
    const int last_tile = ((N + 15) >> 4) - 1;
    uint32_t woff[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[t][h] = pk ? (uint32_t)(lane * 16 + h * 1024)
                            : (uint32_t)min(n0 + 16 * t + 8 * h + lrow, N - 1) * (uint32_t)K + lcol;
    // Activation rows past M load row 0: they only feed output columns that are never stored.
    uint32_t aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int m = 8 * h + lrow;
        aoff[h] = (uint32_t)(m < M ? m : 0) * (uint32_t)K + lcol;
    }
    const float *asp = p.a_scale + (size_t)(mval ? r16 : 0) * KB;
    // Weight scale rows.  Block scale: RG divides 128, so the row group lies in
    // one 128-row block.  MX: tiles 2i and 2i+1 lie in one 32-row block (RG is
    // 16 or a multiple of 32); tiles past N read the last block.  Row-wise: no
    // per-block scales.
    constexpr bool MX = SM == SM_MX, PER_BLOCK_SCALES = SM != SM_ROWWISE;
    constexpr int WS = MX ? (TPW + 1) / 2 : 1;
    const float *wsp[WS];
#pragma unroll
    for (int i = 0; i < WS; ++i)
        wsp[i] = p.w_scale + (size_t)(MX ? min((n0 >> 5) + i, (N - 1) >> 5) : (n0 >> 7)) * KB;

    v4f acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};

    // Row-wise: the scales of the outputs this lane stores (wave t stores tile t).
    static_assert(NW == 1 || TPW <= NW, "each wave stores at most one tile");
    constexpr int RS = NW > 1 ? 1 : TPW;
    RowScales rs[RS];
#pragma unroll
    for (int i = 0; i < RS; ++i)
        rs[i] = rowwise_fetch<SM>(p, r16, n0 + 16 * (NW > 1 ? wave : i) + 4 * g);

    for (int kb_begin = kb_lo + wave * D; kb_begin < kb_hi; kb_begin += NW * D) {
        v4i ar[D][2];
        v4i wr[D][TPW][2];
        float sa[D] = {}, sw[D][WS] = {};
        // Issue every load of the pass before consuming any of them.
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = min(kb_begin + j, kb_hi - 1);   // blocks past the range load a valid block, skipped below
            const int koff = kb * 128;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                const int wso = pk ? (int)packed_block(min((n0 >> 4) + t, last_tile), kb, KB) : koff;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wr[j][t][h] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woff[t][h], wso, 2 /* nt */);
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ar[j][h] = __builtin_amdgcn_raw_buffer_load_b128(ares, (int)aoff[h], koff, 0);
            if constexpr (PER_BLOCK_SCALES) {
                sa[j] = asp[kb];
#pragma unroll
                for (int i = 0; i < WS; ++i)
                    sw[j][i] = wsp[i][kb];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (kb_begin + j < kb_hi) {
                const v8i af = fix_row_layout(ar[j][0], ar[j][1]);
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    acc[t] = block_step<SM>(acc[t], w_fragment(wr[j][t][0], wr[j][t][1], pk), af,
                                            sw[j][MX ? t >> 1 : 0], sa[j], g);
            }
        }
    }

    // Each wave's share of the output: with several waves, wave t (t < TPW) sums
    // tile t over the waves in wave order; a single wave holds every tile.
    constexpr int NV = NW > 1 ? 1 : TPW;
    const bool own = NW == 1 || wave < TPW;
    v4f out[NV];
    if constexpr (NW > 1) {
        __shared__ v4f red[NW][TPW][64];
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            red[wave][t][lane] = acc[t];
        __syncthreads();
        if (own) {
            out[0] = red[0][wave][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const v4f o = red[w][wave][lane];
                out[0][0] += o[0];
                out[0][1] += o[1];
                out[0][2] += o[2];
                out[0][3] += o[3];
            }
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            out[t] = acc[t];
    }

    if (S > 1) {
        // Partial row group of split s: [group][s][tile][component][lane] fp32 in
        // this batch's workspace, written and read with device-scope accesses;
        // the last split to count itself sums the S partials in split order and
        // stores the result (the protocol of the split tile kernel below).
        constexpr int GROUP_F = 256 * TPW;
        const size_t group_g = (size_t)blockIdx.y * (gridDim.x / S) + tile;
        float *part = p.ws + group_g * S * GROUP_F + lane;
        if (own) {
#pragma unroll
            for (int i = 0; i < NV; ++i)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    __hip_atomic_store(part + (size_t)split * GROUP_F + ((NW > 1 ? wave : i) * 4 + c) * 64,
                                       out[i][c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __shared__ int last;
        wait_vmcnt<0>();                                     // this wave's partial stores are complete
        __syncthreads();                                     // ... and every wave's
        if (threadIdx.x == 0)
            last = __hip_atomic_fetch_add(p.cnt + group_g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!last)
            return;
        if (own) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const float *q = part + ((NW > 1 ? wave : i) * 4) * 64;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    out[i][c] = __hip_atomic_load(q + c * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int s2 = 1; s2 < S; ++s2)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        out[i][c] += __hip_atomic_load(q + (size_t)s2 * GROUP_F + c * 64, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(p.cnt + group_g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    const bool vec = vec_store != 0;
    if (own && mval) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int t = NW > 1 ? wave : i;
            store4(p.Y, (int64_t)r16 * N, n0 + 16 * t + 4 * g, N, vec, rowwise_apply<SM>(out[i], rs[i]));
        }
    }
}

// ---------------------------------------------------------------------------
// Persistent skinny kernel, M <= 16, for tall weights.  The skinny kernel
// above gives a workgroup RG rows and all of K; when N is many times 16 x the
// CU count that leaves either a partly filled last wave of workgroups (wide
// row groups) or every workgroup fetching the whole M x K activation again
// (16-row groups).  Here about one workgroup per CU walks the 16-row tiles
// b, b + G, b + 2G, ... of W (G = grid size): each wave loads its activation
// fragments once and keeps them in registers, and the weight loads of the
// next tile are in flight while the current tile is multiplied.
//
// Wave w owns the K blocks [D w, D w + D) (the instance needs NW * D >= K/128).
// Its weight loads run P - 1 tiles ahead of the tile it multiplies.  Per
// tile it loads its blocks of the 16 weight rows with the whole-line
// pattern of the skinny kernel (plus each block's w_scale, through the same
// vector-memory queue so that one counter orders them), takes one MFMA and
// one scale FMA per block, and writes its partial sum to one of two LDS
// slots.  After one barrier the wave whose turn it is adds the NW partials in
// wave order (fixed order: bitwise deterministic) and stores the 16 x 16
// bf16 tile.  Loads for tiles past the workgroup's share go through a
// descriptor of zero records, which returns zeros without touching memory.
template <int D, int NW, int P, bool PK, int SM>
__global__ __launch_bounds__(NW * 64) void pskinny_kernel(Args p, int vec_store)
{
    select_batch(p);
    __shared__ v4f red[2][NW][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int r16 = lane & 15, g = lane >> 4;
    const bool mval = r16 < M;
    const int ntiles = (N + 15) >> 4;
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int mine = b < ntiles ? (ntiles - 1 - b) / G + 1 : 0;
    const int kb0 = wave * D;
    const bool vec = vec_store != 0;

    const int lrow = r16 & 7;
    const uint32_t lcol = (uint32_t)(g + 4 * (r16 >> 3)) * 16;
    constexpr bool pk = PK;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.W, w_rows<PK>(p) * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t none = buffer_rsrc(p.W, 0u);
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)K);
    // Weight scale rows: one per 128 rows (block scale) or per 32 (MX); a
    // 16-row tile lies in one.
    constexpr int SH = wscale_shift<SM>();
    constexpr bool PER_BLOCK_SCALES = SM != SM_ROWWISE;
    const __amdgpu_buffer_rsrc_t sres =
        buffer_rsrc(p.w_scale, (uint32_t)((N + (1 << SH) - 1) >> SH) * (uint32_t)KB * 4u);

    // This wave's activation blocks and scales, held for the whole kernel
    // (put into the MFMA layout once the first weight loads are issued).
    v4i araw[D][2];
    v8i af[D];
    float sa[D] = {};
    {
        const float *asp = p.a_scale + (size_t)(mval ? r16 : 0) * KB;
        uint32_t aoff[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 8 * h + lrow;
            aoff[h] = (uint32_t)(m < M ? m : 0) * (uint32_t)K + lcol;   // rows past M: row 0, never stored
        }
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = min(kb0 + j, KB - 1);   // blocks past K load a valid block, skipped below
#pragma unroll
            for (int h = 0; h < 2; ++h)
                araw[j][h] = __builtin_amdgcn_raw_buffer_load_b128(ares, (int)aoff[h], kb * 128, 0);
            if constexpr (PER_BLOCK_SCALES)
                sa[j] = asp[kb];
        }
    }

    // Row-wise: this lane's a_scale once, the w_scale of its four columns with each tile.
    const RowScales rs_a = rowwise_fetch<SM>(p, r16, N);
    const __amdgpu_buffer_rsrc_t rwres = buffer_rsrc(p.w_scale, SM == SM_ROWWISE ? (uint32_t)N * 4u : 0u);

    // Issue the weight and w_scale loads of this workgroup's tile i.
    auto load_tile = [&](int i, v4i (&wr)[D][2], float (&sw)[D], RowScales &rw) {
        const bool live = i < mine;
        const int n0 = (b + (live ? i : 0) * G) * 16;
        const __amdgpu_buffer_rsrc_t r = live ? wres : none;
        uint32_t woff[2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[h] = pk ? (uint32_t)(lane * 16 + h * 1024)
                         : (uint32_t)min(n0 + 8 * h + lrow, N - 1) * (uint32_t)K + lcol;
        const int srow = (n0 >> SH) * KB;
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = min(kb0 + j, KB - 1);
            const int wso = pk ? (int)packed_block((uint32_t)(n0 >> 4), kb, KB) : kb * 128;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wr[j][h] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)woff[h], wso, 2 /* nt */);
            if constexpr (PER_BLOCK_SCALES)
                sw[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sres, 0, (srow + kb) * 4, 0));
            else
                sw[j] = 0.f;
        }
        if constexpr (SM == SM_ROWWISE) {
            // columns past N (and tiles past the share) read zeros through the descriptors
            const __amdgpu_buffer_rsrc_t sr = live ? rwres : none;
            rw.a = rs_a.a;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                rw.w[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, (n0 + 4 * g + e) * 4, 0, 0));
        }
    };
    // Multiply tile i, reduce it over the waves and store it.
    auto finish_tile = [&](int i, const v4i (&wr)[D][2], const float (&sw)[D], const RowScales &rw) {
        v4f acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < D; ++j)
            if (kb0 + j < KB)
                acc = block_step<SM>(acc, w_fragment(wr[j][0], wr[j][1], pk), af[j], sw[j], sa[j], g);
        red[i & 1][wave][lane] = acc;
        __syncthreads();
        if (wave == i % NW) {
            v4f v = red[i & 1][0][lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) {
                const v4f o = red[i & 1][w][lane];
                v[0] += o[0];
                v[1] += o[1];
                v[2] += o[2];
                v[3] += o[3];
            }
            if (mval)
                store4(p.Y, (int64_t)r16 * N, (b + i * G) * 16 + 4 * g, N, vec, rowwise_apply<SM>(v, rw));
        }
    };

    // P register sets: the loads of tiles i+1 .. i+P-1 are in flight while
    // tile i is finished.
    v4i wr[P][D][2];
    float sw[P][D];
    RowScales rsw[P];
#pragma unroll
    for (int q = 0; q + 1 < P; ++q)
        load_tile(q, wr[q], sw[q], rsw[q]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < D; ++j)
        af[j] = fix_row_layout(araw[j][0], araw[j][1]);
    // The grid never exceeds the tile count: every workgroup has a tile.
    int i = 0;
    do {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            load_tile(i + q + P - 1, wr[(q + P - 1) % P], sw[(q + P - 1) % P], rsw[(q + P - 1) % P]);
            if (i + q < mine)
                finish_tile(i + q, wr[q], sw[q], rsw[q]);
        }
        i += P;
    } while (i < mine);
}

// ---------------------------------------------------------------------------
// Row-range skinny kernel ("rskinny"), M <= 16 (decode): every compute unit
// streams an equal share of the weight rows.  The row-group kernel above gives
// each workgroup whole 16-row tiles, so the tile count per workgroup is an
// integer and N = 14336 (896 tiles) either leaves CUs idle (224 workgroups of
// four tiles) or loads some CUs more than others; N = 5120 (320 tiles) had
// 160 workgroups of two tiles.  Here workgroup b of G (about one per CU) owns
// the rows [r0, r1) of a split of N into G nearly equal runs of RG-row units
// (RG = 4 for row-major weights: 56 rows per CU at N = 14336 and 20 at
// N = 5120; 16 for packed weights, whose tiles are 16-row aligned).  T 16-row
// tiles cover the run, the last one partly: lanes on rows at or past r1 load
// through an out-of-range offset, which returns zeros without touching memory,
// and their outputs are never stored.
//
// Scales: each wave fetches the activation scales of its pass (M rows x D
// blocks) with one word per lane and shares them through its own LDS slot (a
// per-lane load of a_scale[m][kb] in every block touched sixteen cache lines
// for 64 bytes at M = 16, which measured ~0.9 us on N = 14336); block-scale
// weight scales come through scalar loads of the two scale rows the run can
// span, so a tile may straddle a 128-row boundary: each output row takes its
// own row's scale (MX: each lane passes its own row's 32-row scale word to the
// scaled MFMA).  Otherwise as the row-group kernel: NW waves split K into runs
// of D blocks (passes if NW * D < K/128), whole-line weight loads with the
// DPP fix (packed: two contiguous kilobytes), one activation fragment per
// block feeding T MFMAs, and the wave partials summed through LDS in wave
// order (bitwise reproducible), rounded once to bf16.
//
// Fused quantisation (QX, block scales only): A is bf16 [M, K] and the kernel
// quantises it per 1 x 128 group itself, with the arithmetic of the
// standalone quantisation kernel, so the codes and scales are the ones that
// kernel writes, bit for bit, and the result equals quantise-then-GEMM with
// the same instance bitwise.  Every workgroup quantises all of A (each wave
// its own blocks), so the work per block is spread over the wave to scale
// with M: the block's MQ rows (MQ = 1, 2, 4, 8 or 16, the first power of two
// >= M) take 64 / MQ lanes each, 2 MQ values per lane; the lanes of a row
// combine their amax with a butterfly, and each lane forms the group scale
// and its codes.  MQ = 16: the lane's values are exactly those its MFMA
// operand holds (row l % 16, K 16g..16g+15 and 64+16g..64+16g+15 of the
// block, g = l / 16), so the codes go straight into the operand and the scale
// is the lane's own row scale.  MQ < 16: the codes and scales go through the
// wave's own LDS slot ([block][row][128] bytes) and come back in operand
// order; lanes of rows >= MQ take zero codes.  MQ = 16 takes the LDS route
// too where the pass's codes would not fit in registers beside its weights.
// A pass's activations are loaded before its weights and quantised as soon
// as they arrive, while the weights stream; where the registers do not hold
// both, only the first QE blocks' weights go out with the activations.
// Rows [r0, r1) of workgroup b of G: RG-row units split as evenly as integers allow.
template <bool PK>
__device__ __forceinline__ void rsk_rows(int b, int G, int N, int &r0, int &r1)
{
    constexpr int RG = PK ? 16 : 4;
    const int units = (N + RG - 1) / RG;
    r0 = RG * (int)((int64_t)b * units / G);
    r1 = min(N, RG * (int)((int64_t)(b + 1) * units / G));
}

// The amax of each of D 1 x 128 groups over the lanes that hold it: MQ = 16,
// lanes l, l^16, l^32, l^48 (the MFMA operand layout); otherwise 64 / MQ
// consecutive lanes, reduced smallest step first (the mirrors need that).
// Each step runs over all D groups before the next, so their exchanges overlap.
template <int MQ, int D>
__device__ __forceinline__ void group_amax(float (&m)[D])
{
    constexpr int LR = 64 / MQ;
    if constexpr (MQ == 16) {
#pragma unroll
        for (int j = 0; j < D; ++j)
            m[j] = amax_step<16>(m[j]);
#pragma unroll
        for (int j = 0; j < D; ++j)
            m[j] = amax_step<32>(m[j]);
    } else {
#pragma unroll
        for (int j = 0; j < D; ++j)
            m[j] = amax_step<1>(m[j]);
        if constexpr (LR > 2) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                m[j] = amax_step<2>(m[j]);
        }
        if constexpr (LR > 4) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                m[j] = amax_step<4>(m[j]);
        }
        if constexpr (LR > 8) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                m[j] = amax_step<8>(m[j]);
        }
        if constexpr (LR > 16) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                m[j] = amax_step<16>(m[j]);
        }
        if constexpr (LR > 32) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                m[j] = amax_step<32>(m[j]);
        }
    }
}

// QX: bf16 activations quantised in the kernel, MQ rows per block, the first
// QE blocks' weights issued with the activations (see issue).
template <int T, int D, int NW, bool PK, int SM, bool QX = false, int QE = D, int MQ = 16>
__global__ __launch_bounds__(NW * 64) void rskinny_kernel(Args p, int vec_store)
{
    static_assert(!QX || SM == SM_BLOCK, "fused quantisation makes 1 x 128 fp32 block scales");
    static_assert(QE >= 1 && QE <= D, "at least one block of weights goes out with the activations");
    static_assert(MQ == 1 || MQ == 2 || MQ == 4 || MQ == 8 || MQ == 16, "rows per block: a power of two");
    constexpr int LR = 64 / MQ, XW = MQ;                        // QX: lanes per row, bf16 words per lane
    // Codes through LDS: MQ < 16, and at MQ = 16 where the pass's codes would
    // not fit in registers beside its weights (t4_d5: 205 VGPRs, spilled).
    constexpr bool QLDS = QX && (MQ < 16 || 8 * T * D + 9 * D > 200);
    select_batch(p);
    constexpr bool MX = SM == SM_MX, PER_BLOCK_SCALES = SM != SM_ROWWISE;
    constexpr bool STAGE_AS = PER_BLOCK_SCALES && !QX;     // a_scale read from memory
    constexpr int SH = wscale_shift<SM>();
    constexpr int AS32 = (16 * D + 63) / 64;                  // a_scale words per lane per pass
    static_assert(T <= NW, "wave t sums and stores tile t");
    __shared__ float s_as[NW][16 * D];                         // this wave's a_scale [m][block of the pass]
    __shared__ v4f red[NW][T][64];
    __shared__ __align__(16) uint8_t q_lds[QLDS ? NW * D * MQ * 128 : 16];   // [wave][block][row][128]
    __shared__ float s_lds[QLDS ? NW * D * MQ : 1];                          // [wave][block][row]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    int r0, r1;
    rsk_rows<PK>((int)blockIdx.x, (int)gridDim.x, N, r0, r1);
    const int r16 = lane & 15, g = lane >> 4, lrow = r16 & 7;
    const uint32_t lcol = (uint32_t)(g + 4 * (r16 >> 3)) * 16;
    constexpr uint32_t OOB = 0x7ffff000u;                     // beyond any buffer: loads return zeros
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.W, w_rows<PK>(p) * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)K * (QX ? 2u : 1u));
    const __amdgpu_buffer_rsrc_t none = buffer_rsrc(p.W, 0u);   // zero records: every load returns zeros
    const __amdgpu_buffer_rsrc_t sares = buffer_rsrc(p.a_scale, STAGE_AS ? (uint32_t)(M * KB) * 4u : 0u);
    const int NB = (N + (1 << SH) - 1) >> SH;
    const int sb0 = min(r0, N - 1) >> SH;
    // Block scale: the run's rows lie in weight-scale rows sb0 and sb0 + 1 (scalar loads).
    const_f32 *wsp0 = (const_f32 *)(p.w_scale + (size_t)sb0 * KB);
    const_f32 *wsp1 = (const_f32 *)(p.w_scale + (size_t)min(sb0 + 1, NB - 1) * KB);
    // Row-wise: the scales of the tile this wave stores.
    const RowScales rs = rowwise_fetch<SM>(p, r16, min(r0 + 16 * wave + 4 * g, N - 1));

    // Per-lane load offsets.  Row layout: load h of a tile takes row 8h + (r16 & 7),
    // chunk g + 4 (r16 >> 3) (whole lines, DPP fix below); packed: lane l reads
    // bytes 16 l (+1024) of the tile's block.  Rows at or past r1, M: out of range.
    uint32_t woff[T][2];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (PK) {
                woff[t][h] = r0 + 16 * t < r1 ? (uint32_t)(lane * 16 + h * 1024) : OOB;
            } else {
                const int row = r0 + 16 * t + 8 * h + lrow;
                woff[t][h] = row < r1 ? (uint32_t)row * (uint32_t)K + lcol : OOB;
            }
        }
    uint32_t aoff[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int m = 8 * h + lrow;
        aoff[h] = m < M ? (uint32_t)m * (uint32_t)K + lcol : OOB;
    }
    // QX, MQ = 16: bf16 row r16, bytes 32 g (+16) and 128 + 32 g (+16) of each block;
    // MQ < 16: row qrow = l / LR, bytes 4 MQ qcol (qcol = l % LR) onward.
    const int qrow = MQ == 16 ? r16 : lane / LR, qcol = MQ == 16 ? g : lane % LR;
    const uint32_t xoff = qrow < M ? (uint32_t)qrow * (uint32_t)K * 2u +
                                         (MQ == 16 ? 32u * (uint32_t)g : 4u * MQ * (uint32_t)qcol)
                                   : OOB;
    // Block scale: output rows n = r0 + 16 t + 4 g + i take scale row sb0 or sb0 + 1.
    bool second[T][4];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            second[t][i] = ((r0 + 16 * t + 4 * g + i) >> SH) > sb0;
    // MX: the scale-row offset (words) of this lane's own weight row in tile t.
    uint32_t mxoff[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        mxoff[t] = (uint32_t)(min(r0 + 16 * t + r16, N - 1) >> SH) * (uint32_t)KB * 4u;
    const __amdgpu_buffer_rsrc_t swres = buffer_rsrc(p.w_scale, MX ? (uint32_t)NB * (uint32_t)KB * 4u : 0u);

    v4f acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t)
        acc[t] = (v4f){0.f, 0.f, 0.f, 0.f};

    v4i ar[D][2];
    uint32_t xw[QX ? D : 1][XW];
    v4i wr[D][T][2];
    float asv[AS32];
    float mxw[D][T];
    v8i afq[QX && !QLDS ? D : 1];
    float saq[QX && !QLDS ? D : 1];
    // The weight loads of block kb_begin + j (blocks past K read through the
    // zero-record descriptor: no traffic).
    auto issue_w = [&](int kb_begin, int j) __attribute__((always_inline)) {
        const int kb = kb_begin + j;
        const bool live = kb < KB;
        const int koff = (live ? kb : 0) * 128;
        const __amdgpu_buffer_rsrc_t rw = live ? wres : none;
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int so = PK ? (int)packed_block((uint32_t)((r0 >> 4) + t), (uint32_t)(live ? kb : 0),
                                                  (uint32_t)KB) : koff;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                wr[j][t][h] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)woff[t][h], so, 2 /* nt */);
            if constexpr (MX)
                mxw[j][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                          live ? swres : none, (int)mxoff[t], (live ? kb : 0) * 4, 0));
        }
    };
    // The activation loads of block kb_begin + j (QX: this lane's XW bf16 words).
    auto issue_a = [&](int kb_begin, int j) __attribute__((always_inline)) {
        const int kb = kb_begin + j;
        const bool live = kb < KB;
        const int koff = (live ? kb : 0) * 128;
        const __amdgpu_buffer_rsrc_t ra = live ? ares : none;
        if constexpr (QX) {
            if constexpr (MQ >= 4) {
#pragma unroll
                for (int c = 0; c < XW / 4; ++c) {
                    const uint32_t at = MQ == 16 ? 16u * (c & 1) + 128u * (c >> 1) : 16u * c;
                    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)(xoff + at), 2 * koff, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xw[j][4 * c + i] = (uint32_t)v[i];
                }
            } else if constexpr (MQ == 2) {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(ra, (int)xoff, 2 * koff, 0);
                xw[j][0] = v[0];
                xw[j][1] = v[1];
            } else {
                xw[j][0] = __builtin_amdgcn_raw_buffer_load_b32(ra, (int)xoff, 2 * koff, 0);
            }
        } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ar[j][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)aoff[h], koff, 0);
        }
    };
    // Issue the loads of the pass starting at block kb_begin: first this wave's
    // activation scales (one word per lane: rows m < M, blocks of the pass, in
    // consecutive words of each row), then per block the weights and the
    // activations.  QX: the pass's bf16 activations first, then the
    // weights of its first QE blocks only (the rest follow once the
    // activations are quantised and their registers free).
    auto issue = [&](int kb_begin) {
        if constexpr (STAGE_AS) {
#pragma unroll
            for (int u = 0; u < AS32; ++u) {
                const int i = lane + 64 * u, m = i / D, j = i - m * D;
                const bool ok = m < M && kb_begin + j < KB;
                asv[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                       sares, ok ? (m * KB + kb_begin + j) * 4 : (int)OOB, 0, 0));
            }
        }
        if constexpr (QX) {
#pragma unroll
            for (int j = 0; j < D; ++j)
                issue_a(kb_begin, j);
#pragma unroll
            for (int j = 0; j < QE; ++j)
                issue_w(kb_begin, j);
        } else {
            // (written out rather than through issue_w / issue_a: with those the
            // scheduler moved block 0's loads behind the others, so that the first
            // MFMA waited for nearly the whole pass -- 9% slower on qkv at M = 8)
#pragma unroll
            for (int j = 0; j < D; ++j) {
                const int kb = kb_begin + j;
                const bool live = kb < KB;
                const int koff = (live ? kb : 0) * 128;
                const __amdgpu_buffer_rsrc_t rw = live ? wres : none, ra = live ? ares : none;
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const int so = PK ? (int)packed_block((uint32_t)((r0 >> 4) + t), (uint32_t)(live ? kb : 0),
                                                          (uint32_t)KB) : koff;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        wr[j][t][h] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)woff[t][h], so, 2 /* nt */);
                    if constexpr (MX)
                        mxw[j][t] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                  live ? swres : none, (int)mxoff[t], (live ? kb : 0) * 4, 0));
                }
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    ar[j][h] = __builtin_amdgcn_raw_buffer_load_b128(ra, (int)aoff[h], koff, 0);
            }
        }
    };
    // QX: quantise the pass's activations (into the operand registers, or the
    // wave's LDS slot), then issue its remaining weights.
    auto quantise_early = [&](int kb_begin) __attribute__((always_inline)) {
        if constexpr (QX) {
            float am[D];
#pragma unroll
            for (int j = 0; j < D; ++j)
                am[j] = bf16_absmax(xw[j]);
            group_amax<MQ>(am);
#pragma unroll
            for (int j = 0; j < D; ++j) {
                if (kb_begin + j < KB) {
                    uint32_t c[(XW + 1) / 2];
                    const float sq = quant_bf16(xw[j], am[j], c);
                    if constexpr (!QLDS) {
                        afq[j] = (v8i){(int)c[0], (int)c[1], (int)c[2], (int)c[3],
                                       (int)c[4], (int)c[5], (int)c[6], (int)c[7]};
                        saq[j] = sq;
                    } else {
                        uint8_t *q = q_lds + ((wave * D + j) * MQ + qrow) * 128 + (MQ == 16 ? 16 : 2 * MQ) * qcol;
                        if constexpr (MQ == 16) {
                            *reinterpret_cast<v4i *>(q) = (v4i){(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
                            *reinterpret_cast<v4i *>(q + 64) = (v4i){(int)c[4], (int)c[5], (int)c[6], (int)c[7]};
                        } else if constexpr (MQ == 8)
                            *reinterpret_cast<v4i *>(q) = (v4i){(int)c[0], (int)c[1], (int)c[2], (int)c[3]};
                        else if constexpr (MQ == 4)
                            *reinterpret_cast<v2u *>(q) = (v2u){c[0], c[1]};
                        else if constexpr (MQ == 2)
                            *reinterpret_cast<uint32_t *>(q) = c[0];
                        else
                            *reinterpret_cast<uint16_t *>(q) = (uint16_t)c[0];
                        if (qcol == 0)
                            s_lds[(wave * D + j) * MQ + qrow] = sq;
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = QE; j < D; ++j)
                issue_w(kb_begin, j);
        }
    };
    // Multiply the pass starting at kb_begin.
    auto consume = [&](int kb_begin) {
        if constexpr (STAGE_AS) {
            // this wave's scales into its own LDS slot (read back by other lanes of the wave)
#pragma unroll
            for (int u = 0; u < AS32; ++u)
                if (lane + 64 * u < 16 * D)
                    s_as[wave][lane + 64 * u] = asv[u];
            __builtin_amdgcn_s_waitcnt(0xc07f);    // lgkmcnt(0): the wave's LDS writes are done
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = kb_begin + j;
            if (kb < KB) {
                v8i af;
                float sa = 0.f;
                if constexpr (QX && !QLDS) {
                    af = afq[j];
                    sa = saq[j];
                } else if constexpr (QLDS) {
                    // rows >= MQ: zero codes (and scale)
                    const int row = r16 < MQ ? r16 : 0;
                    const uint8_t *q = q_lds + ((wave * D + j) * MQ + row) * 128 + 16 * g;
                    const v4i lo = *reinterpret_cast<const v4i *>(q), hi = *reinterpret_cast<const v4i *>(q + 64);
                    af = r16 < MQ ? cat(lo, hi) : (v8i){0, 0, 0, 0, 0, 0, 0, 0};
                    sa = r16 < MQ ? s_lds[(wave * D + j) * MQ + row] : 0.f;
                } else {
                    af = fix_row_layout(ar[j][0], ar[j][1]);
                    if constexpr (PER_BLOCK_SCALES)
                        sa = s_as[wave][min(r16, M - 1) * D + j];
                }
                float sc0 = 0.f, sc1 = 0.f;
                if constexpr (SM == SM_BLOCK) {
                    sc0 = sa * wsp0[kb];
                    sc1 = sa * wsp1[kb];
                }
#pragma unroll
                for (int t = 0; t < T; ++t) {
                    const v8i wf = w_fragment(wr[j][t][0], wr[j][t][1], PK);
                    if constexpr (SM == SM_BLOCK) {
                        const v4f d = mfma_block(wf, af);
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            acc[t][i] = __builtin_fmaf(d[i], second[t][i] ? sc1 : sc0, acc[t][i]);
                    } else {
                        acc[t] = block_step<SM>(acc[t], wf, af, MX ? mxw[j][t] : 0.f, sa, g);
                    }
                }
            }
        }
        if constexpr (STAGE_AS)
            __builtin_amdgcn_wave_barrier();       // the slot is rewritten by the next pass
    };

    A8W8_TL(uint64_t tl[5] = {__builtin_amdgcn_s_memrealtime(), 0, 0, 0, 0};)
    for (int kb_begin = wave * D; kb_begin < KB; kb_begin += NW * D) {
        issue(kb_begin);
        __builtin_amdgcn_sched_barrier(0);
        A8W8_TL(if (tl[1] == 0) tl[1] = __builtin_amdgcn_s_memrealtime();)
        if constexpr (QX) {
            quantise_early(kb_begin);
            __builtin_amdgcn_sched_barrier(0);
        }
        consume(kb_begin);
    }
    A8W8_TL(__builtin_amdgcn_s_waitcnt(0); tl[2] = __builtin_amdgcn_s_memrealtime();)

    // Wave t sums tile t over the waves in wave order and stores it.
#pragma unroll
    for (int t = 0; t < T; ++t)
        red[wave][t][lane] = acc[t];
    __syncthreads();
    A8W8_TL(tl[3] = __builtin_amdgcn_s_memrealtime();)
    if (wave < T) {
        v4f v = red[0][wave][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const v4f o = red[w][wave][lane];
            v[0] += o[0];
            v[1] += o[1];
            v[2] += o[2];
            v[3] += o[3];
        }
        const int n = r0 + 16 * wave + 4 * g;
        if (r16 < M && n < r1)
            store4(p.Y, (int64_t)r16 * N, n, N, vec_store != 0, rowwise_apply<SM>(v, rs));
    }
    A8W8_TL(__builtin_amdgcn_s_waitcnt(0); tl[4] = __builtin_amdgcn_s_memrealtime();
            if (p.ws != nullptr && lane == 0) {
                uint64_t *rec = reinterpret_cast<uint64_t *>(p.ws) + ((int)blockIdx.x * NW + wave) * 6;
                for (int i = 0; i < 5; ++i)
                    rec[i] = tl[i];
                rec[5] = __smid();
            })
}

// ---------------------------------------------------------------------------
// Tall kernel, N <= 16 * NT (a few weight rows, many activation rows): the
// skinny kernel with the roles of the two dimensions exchanged.  Here the
// activations are the stream read once from HBM and the small weight matrix
// is re-read from L2.  A workgroup owns 16 * TPW activation rows and all N;
// its NW waves split K into runs of D blocks exactly as in the skinny kernel
// (same whole-line loads and DPP fix, same operand roles: W is the MFMA "A"
// operand, so a lane's four outputs are four consecutive columns of one
// output row and take one a_scale per block).  Per block: TPW * NT MFMAs,
// each followed by one scale FMA per output; the wave partials are summed
// through LDS in wave order and rounded once.
template <int TPW, int NT, int D, int NW, bool PK, int SM>
__global__ __launch_bounds__(NW * 64) void tall_kernel(Args p, int vec_store)
{
    static_assert(16 * NT <= (SM == SM_MX ? 32 : 128), "every weight row lies in weight-scale row 0");
    constexpr bool PER_BLOCK_SCALES = SM != SM_ROWWISE;
    select_batch(p);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int m0 = (int)blockIdx.x * (16 * TPW);
    const int r16 = lane & 15, g = lane >> 4;
    const int lrow = r16 & 7;
    const uint32_t lcol = (uint32_t)(g + 4 * (r16 >> 3)) * 16;
    constexpr bool pk = PK;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(p.W, w_rows<PK>(p) * (uint32_t)K);
    const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(p.A, (uint32_t)M * (uint32_t)K);
    // Rows past N or M load the last row (packed: the last tile): they only
    // feed outputs that are never stored.
    const int last_tile = ((N + 15) >> 4) - 1;
    uint32_t woff[NT][2], aoff[TPW][2];
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            woff[u][h] = pk ? (uint32_t)(lane * 16 + h * 1024)
                            : (uint32_t)min(16 * u + 8 * h + lrow, N - 1) * (uint32_t)K + lcol;
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h)
            aoff[t][h] = (uint32_t)min(m0 + 16 * t + 8 * h + lrow, M - 1) * (uint32_t)K + lcol;
    const float *asp[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
        asp[t] = p.a_scale + (size_t)min(m0 + 16 * t + r16, M - 1) * KB;
    // 16 * NT rows: all in weight-scale row 0 (block scale and MX).
    const float *wsp = p.w_scale;

    v4f acc[TPW][NT];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u)
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    // Row-wise: the scales of the output tile this wave stores (tile i = wave).
    static_assert(TPW * NT <= NW, "each wave stores at most one output tile");
    const RowScales rs = rowwise_fetch<SM>(p, m0 + 16 * (wave / NT) + r16, 16 * (wave % NT) + 4 * g);

    for (int kb_begin = wave * D; kb_begin < KB; kb_begin += NW * D) {
        v4i wr[D][NT][2], ar[D][TPW][2];
        float sa[D][TPW] = {}, sw[D] = {};
#pragma unroll
        for (int j = 0; j < D; ++j) {
            const int kb = min(kb_begin + j, KB - 1);   // blocks past the end load a valid block, skipped below
            const int koff = kb * 128;
#pragma unroll
            for (int t = 0; t < TPW; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    ar[j][t][h] = __builtin_amdgcn_raw_buffer_load_b128(ares, (int)aoff[t][h], koff, 2 /* nt */);
#pragma unroll
            for (int u = 0; u < NT; ++u) {
                const int wso = pk ? (int)packed_block((uint32_t)min(u, last_tile), kb, KB) : koff;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    wr[j][u][h] = __builtin_amdgcn_raw_buffer_load_b128(wres, (int)woff[u][h], wso, 0);
            }
            if constexpr (PER_BLOCK_SCALES) {
#pragma unroll
                for (int t = 0; t < TPW; ++t)
                    sa[j][t] = asp[t][kb];
                sw[j] = wsp[kb];
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < D; ++j) {
            if (kb_begin + j < KB) {
                v8i wf[NT];
#pragma unroll
                for (int u = 0; u < NT; ++u)
                    wf[u] = w_fragment(wr[j][u][0], wr[j][u][1], pk);
#pragma unroll
                for (int t = 0; t < TPW; ++t) {
                    const v8i af = fix_row_layout(ar[j][t][0], ar[j][t][1]);
#pragma unroll
                    for (int u = 0; u < NT; ++u)
                        acc[t][u] = block_step<SM>(acc[t][u], wf[u], af, sw[j], sa[j][t], g);
                }
            }
        }
    }

    __shared__ v4f red[NW][TPW * NT][64];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int u = 0; u < NT; ++u)
            red[wave][t * NT + u][lane] = acc[t][u];
    __syncthreads();
    for (int i = wave; i < TPW * NT; i += NW) {
        v4f v = red[0][i][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) {
            const v4f o = red[w][i][lane];
            v[0] += o[0];
            v[1] += o[1];
            v[2] += o[2];
            v[3] += o[3];
        }
        const int m = m0 + 16 * (i / NT) + r16;
        if (m < M)
            store4(p.Y, (int64_t)m * N, 16 * (i % NT) + 4 * g, N, vec_store != 0, rowwise_apply<SM>(v, rs));
    }
}

// Direct global -> LDS copies.  Each wave instruction moves one value per lane
// and writes them to consecutive LDS addresses starting at the wave-uniform
// address in m0 (lane i at byte 16 i for the 16-byte form, 4 i for the 4-byte
// form), so one 16-byte copy fills 1 KB of LDS = 8 tile rows of 128 bytes.
//
// The copies are written as inline asm on purpose: the compiler treats every
// LDS read as possibly aliasing every copy still in flight and would wait for
// all of them before the first fragment read, collapsing the ring to depth 1.
// The asm has no register outputs (only the addresses, which the hardware reads
// at issue), and the kernel's own counted waits order the copies against the
// reads.  The compiler resolves hazards only for instructions it generates,
// not inside these strings, so the asm pads its own: a scalar write of m0
// needs one wait state before an LDS-DMA load reads it (without it the load
// can take a stale m0 as its LDS destination), and an SGPR written by a VALU
// instruction needs five before a vector-memory instruction reads it; s_nop 4
// covers both.
//
// The 16-byte form reads through a buffer descriptor (see tile_rsrc) at a
// 32-bit per-lane offset: lanes past the descriptor's range fetch zeros
// instead of faulting, which is how rows past M or N are handled.
__device__ __forceinline__ void lds_copy16(v4i rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_addr), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

__device__ __forceinline__ void lds_copy4(const float *src, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dword %1, off" : : "s"(lds_addr), "v"(src) : "memory", "m0");
}

// Raw buffer descriptor (stride 0, 32-bit data format) over `bytes` bytes at
// `base`, built in scalar registers.
__device__ __forceinline__ v4i tile_rsrc(const uint8_t *base, uint32_t bytes)
{
    const uint64_t v = (uint64_t)(uintptr_t)base;
    v4i r;
    r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)v);
    r[1] = (int)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32) & 0xFFFFu);
    r[2] = (int)__builtin_amdgcn_readfirstlane(bytes);
    r[3] = 0x00020000;
    return r;
}

// Issue the copies of one K block into the LDS stage at byte address `stage`:
// A_LOADS 16-byte copies of activation rows, W_LOADS of weight rows (ra and rw
// describe the block's tile rows, see tile_kernel), and one 4-byte copy of
// scale values (SC: kinds with per-block scales).  Every wave issues exactly
// A_LOADS + W_LOADS + SC vector-memory instructions per block, which is what
// the counted waits in the main loop rely on.
template <int A_LOADS, int W_LOADS, int A_BYTES, int W_BYTES, bool SC>
__device__ __forceinline__ void issue_tile_loads(v4i ra, v4i rw, const uint32_t (&a_off)[A_LOADS],
                                                 const uint32_t (&w_off)[W_LOADS], const float *s_src, int kb,
                                                 uint32_t stage, int wave)
{
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
        lds_copy16(ra, a_off[i], stage + (uint32_t)(wave * A_LOADS + i) * 1024u);
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i)
        lds_copy16(rw, w_off[i], stage + (uint32_t)(A_BYTES + (wave * W_LOADS + i) * 1024));
    if constexpr (SC)
        lds_copy4(s_src + kb, stage + (uint32_t)(A_BYTES + W_BYTES + wave * 256));
}

// Copy number j (0 <= j < A_LOADS + W_LOADS + SC) of one block, in the order
// issue_tile_loads uses.
template <int A_LOADS, int W_LOADS, int A_BYTES, int W_BYTES, bool SC>
__device__ __forceinline__ void issue_one(int j, v4i ra, v4i rw, const uint32_t (&a_off)[A_LOADS],
                                          const uint32_t (&w_off)[W_LOADS], const float *s_src, int kb,
                                          uint32_t stage, int wave)
{
    if (j < A_LOADS)
        lds_copy16(ra, a_off[j], stage + (uint32_t)(wave * A_LOADS + j) * 1024u);
    else if (j < A_LOADS + W_LOADS)
        lds_copy16(rw, w_off[j - A_LOADS], stage + (uint32_t)(A_BYTES + (wave * W_LOADS + j - A_LOADS) * 1024));
    else if constexpr (SC)
        lds_copy4(s_src + kb, stage + (uint32_t)(A_BYTES + W_BYTES + wave * 256));
}

// LDS tiles are row-major 128-byte rows whose 16-byte chunk c sits at chunk
// position c ^ chunk_swizzle(row).  A fragment read has lane (g = l/16,
// p = l%16) read chunk g (then g + 4) of row r0 + p.  The swizzle XORs the
// chunk index with a linear function of the row's low four bits (bits 0, 1,
// 2, 3 contribute 4, 1, 2, 4): the three low bits rotated, then bit 3 into
// the top.  It was chosen offline as one that leaves these reads free of
// bank conflicts under every lane-to-pass grouping and bank count (32, 64,
// 128 four-byte banks) for which the earlier chunk order (2g, 2g+1 with
// swizzle (r & 7) ^ (r >> 3 & 1)) measured zero conflicts; the LDS bank
// conflict counter confirms zero for it on gfx950.  Rows are 16-aligned in
// every read, so the pattern only needs to be a bijection on each row.
__device__ __forceinline__ int chunk_swizzle(int row)
{
    return (((row & 1) << 2) | ((row >> 1) & 3)) ^ ((row >> 1) & 4);
}

// Byte offsets, from the first row of a 16-row group, of this lane's two
// fragment chunks: row l%16, logical chunks g and g + 4 (K bytes 16g..16g+15
// and 64+16g..64+16g+15).  Computed once per lane, so every read adds only
// its 16-aligned row base (an immediate offset).
struct FragOff {
    uint32_t lo, hi;
};
__device__ __forceinline__ FragOff frag_offsets(int lane)
{
    const int r = lane & 15, g = lane >> 4, x = chunk_swizzle(r);
    return {(uint32_t)(r * 128 + ((g ^ x) << 4)), (uint32_t)(r * 128 + (((g + 4) ^ x) << 4))};
}

// MFMA operand of this lane from the 16-row group starting at tile row row0.
__device__ __forceinline__ v8i lds_fragment(const uint8_t *tile, int row0, FragOff f)
{
    const uint8_t *rp = tile + row0 * 128;
    const v4i lo = *reinterpret_cast<const v4i *>(rp + f.lo);
    const v4i hi = *reinterpret_cast<const v4i *>(rp + f.hi);
    return cat(lo, hi);
}

// Weight stages hold either row-layout rows (as above) or, for packed weights,
// each 16-row tile's 2 KB exactly as stored in memory (operand order): the
// copies then move whole contiguous kilobytes, and lane l reads bytes 16 l of
// each half of the tile that starts at row0.
template <bool PK>
__device__ __forceinline__ v8i lds_w_fragment(const uint8_t *sW, int row0, FragOff f, int lane)
{
    if constexpr (PK) {
        const uint8_t *tp = sW + (row0 >> 4) * 2048 + lane * 16;
        return cat(*reinterpret_cast<const v4i *>(tp), *reinterpret_cast<const v4i *>(tp + 1024));
    } else {
        return lds_fragment(sW, row0, f);
    }
}

// ---------------------------------------------------------------------------
// Persistent tile kernel ("ptile").  Workgroup b takes output tiles rank(b),
// rank(b) + G, rank(b) + 2G, ... of the T = ceil(M/BM) * ceil(N/BN) tiles
// (G = gridDim.x, launched at about one workgroup per free CU slot), so the
// prologue and epilogue of one tile overlap the neighbouring tiles' work.
// A workgroup of WGM x WGN waves walks K one 128-wide scale block at a time
// through a STAGES-deep ring of LDS buffers filled by direct global -> LDS
// copies (no VGPR staging); the copy stream runs AHEAD blocks ahead (see the
// copy schedule below) and continues straight into the next tile.  Each wave
// owns a (BM/WGM) x (BN/WGN) sub-tile: TM 16-row activation slices times TN
// 16-row weight fragments, one MFMA each per block.
//
// Per block and wave, slice t does: issue its share of the block's copies,
// read the activation fragment of slice t+1, issue the TN MFMAs of slice t,
// and apply a_scale * w_scale to the results of slice t-1 with one FMA per
// output.  The results of a block's last slice are scaled at the start of the
// next block (or before the tile's stores).
//
// The one workgroup barrier per block sits at the start of the last slice.
// Before it every wave waits for its own copies of the next block; after it
// those copies are visible to all waves, and every wave has finished reading
// the current block's stage (its last fragment read happens before the
// barrier).  Right after the barrier each wave issues the last slice's MFMAs
// from registers and then reads the next block's weight fragments, first
// activation fragment and scales, so the LDS latency at a block boundary hides
// under that slice's work.
//
// LDS stage: A tile [BM][128] | W tile [BN][128] | scales [64 * waves] floats.
// Scale slot s < BM holds a_scale of tile row s; slot BM + j holds w_scale of
// the tile's j-th weight-scale row (128 weight rows each; MX: 32, and the
// block's MFMAs take the scale words instead of the FMAs, accumulating in
// place).  Tiles are swizzled as described at
// chunk_swizzle().
constexpr int cmin(int a, int b) { return a < b ? a : b; }

// Tile (tm, tn) of linear tile id L: tiles are numbered in groups of G tile
// rows, column by column inside a group.  Workgroups of one XCD hold
// consecutive ids (see tile_kernel), so the tiles resident together on an XCD
// form a compact G-row block that shares A rows and W rows in its L2.
__device__ __forceinline__ void linear_tile(int L, int tiles_m, int tiles_n, int G, int &tm, int &tn)
{
    const int per_group = G * tiles_n;
    const int group = L / per_group;
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in_group = L - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

template <int BM, int BN, int WGM, int WGN, int STAGES, bool SKM, bool PK, int SM>
__global__ __launch_bounds__(WGM * WGN * 64) void ptile_kernel(Args p, int vec_store)
{
    select_batch(p);
    constexpr int NWAVES = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
    constexpr int STAGE = A_BYTES + W_BYTES + NWAVES * 256;
    constexpr int A_LOADS = BM / (8 * NWAVES), W_LOADS = BN / (8 * NWAVES);   // 1 KB copies per wave per block
    constexpr bool MX = SM == SM_MX, SC = SM != SM_ROWWISE;                  // SC: per-block scale copies
    constexpr int PER_BLOCK = A_LOADS + W_LOADS + (SC ? 1 : 0);              // vector-memory ops per block
    constexpr int SH = wscale_shift<SM>();
    constexpr int NBW = (BN + (1 << SH) - 1) >> SH;                          // weight-scale rows a tile spans
    constexpr int WSN = MX ? TN : 1;                                         // weight-scale words per wave
    // Copy schedule.  Wave tiles of three or more slices spread a block's
    // copies, CPS per slice, over its first SPREAD slices; those copies run
    // before the block's barrier, so they can only refill the stage freed by
    // the previous barrier and fetch the block STAGES-1 steps ahead (with two
    // stages they must all precede the barrier).  Wave tiles of one or two
    // slices issue all copies right after the barrier ("late"), which has
    // just freed the current block's stage (its fragments are in registers),
    // and fetch the block STAGES steps ahead: a full ring of lookahead.
    constexpr bool LATE = TM <= 2;
    constexpr int AHEAD = LATE ? STAGES : STAGES - 1;
    constexpr int SPREAD = LATE ? 1 : STAGES == 2 ? cmin(TM - 1, 4) : cmin(TM, 4);
    constexpr int CPS = LATE ? PER_BLOCK : (PER_BLOCK + SPREAD - 1) / SPREAD;
    constexpr int C_BEFORE = LATE ? 0 : cmin(PER_BLOCK, cmin(SPREAD, TM - 1) * CPS);   // issued before the barrier
    // Copies a wave may still have in flight at a block's barrier: all of
    // those issued after the next block's.  (Vector memory operations complete
    // in issue order; the stores of a finished tile only make this wait
    // stricter.)
    constexpr int VM_AT_BARRIER = (AHEAD - 2) * PER_BLOCK + C_BEFORE;
    // VALU instructions issued after each MFMA (a slice's 4 * TN scale FMAs
    // and its scale product go behind the first MFMAs).
    constexpr int FMA_GROUP = 6;
    static_assert(A_LOADS >= 1 && W_LOADS >= 1 && BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0,
                  "each wave copies whole 8-row groups of both tiles");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile is made of 16 x 16 MFMA outputs");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-row weight block");
    static_assert(BN <= 128 ? 128 % BN == 0 : BN % 128 == 0, "tiles start on weight-block boundaries");
    static_assert(!MX || BN % 32 == 0, "MX: tiles start on 32-row weight-scale boundaries");
    static_assert(BM + NBW <= NWAVES * 64, "scale slots");
    static_assert(STAGES >= 2 && SPREAD >= 1 && SPREAD * CPS >= PER_BLOCK, "copy schedule");
    static_assert(LATE || STAGES > 2 || C_BEFORE == PER_BLOCK, "two stages: next block's copies precede the barrier");
    static_assert(VM_AT_BARRIER >= 0 && VM_AT_BARRIER < 64 && (AHEAD - 1) * PER_BLOCK < 64, "vmcnt range");
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    __shared__ int sk_last;                       // stream-K fixup: this workgroup arrived last

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const int M = p.M, N = p.N, K = p.K, KB = K >> 7;
    const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN, T = tiles_m * tiles_n;
    // Workgroup b runs on XCD b % 8; with the grid a multiple of 8, rank puts
    // the workgroups of one XCD on consecutive tile ids.
    const int grid = (int)gridDim.x, b = (int)blockIdx.x;
    const int rank = (grid & 7) == 0 ? (b & 7) * (grid >> 3) + (b >> 3) : b;
    // Stream-K instances (SKM): when T is not a multiple of the grid, the
    // tiles of the last one or two waves (sk_tiles of them, the last ids of
    // the tile order) are not dealt out whole.  Their T_sk x KB blocks form one
    // stream cut into `grid` nearly equal runs, run r = steps [B(r), B(r+1))
    // with B(r) = r * S / grid, so every workgroup does the same number of
    // blocks; a tile cut between runs is finished by the fixed-order fixup
    // after the K loop.  The other tiles go round-robin as below.
    //
    // With at most half as many tiles as workgroups the host launches
    // grid = S x T (S >= 2) and every tile is cut at the same S - 1 points
    // ("aligned"): workgroup rank takes piece j = rank / T of tile rank % T,
    // blocks [j KB / S, (j + 1) KB / S).  The workgroups that run together then
    // work at the same K position, so the tiles that share A rows or W rows
    // read the same slice of them at the same time, as whole tiles do.
    int dp_tiles = T, sk_tiles = 0;
    const bool aligned = SKM && 2 * T <= grid;
    const int S_al = aligned ? grid / T : 1;
    if constexpr (SKM) {
        const int full = T / grid, rem = T - full * grid;
        if (rem != 0) {
            dp_tiles = full >= 1 ? (full - 1) * grid : 0;
            sk_tiles = T - dp_tiles;
        }
    }
    // stream-K steps (the host keeps S_sk >= grid; sk_tiles < 2 grid, so S_sk fits 31 bits)
    const int64_t S_sk = (int64_t)sk_tiles * KB;
    int64_t sk_lo = (int64_t)rank * S_sk / grid, sk_hi = (int64_t)(rank + 1) * S_sk / grid;
    const int al_tile = rank % T, al_piece = rank / T;
    if (aligned) {
        sk_lo = (int64_t)al_tile * KB + (int64_t)al_piece * KB / S_al;
        sk_hi = (int64_t)al_tile * KB + (int64_t)(al_piece + 1) * KB / S_al;
    }
    if (rank >= T && S_sk == 0)
        return;
    const int ntiles = rank < dp_tiles && !aligned ? (dp_tiles - 1 - rank) / grid + 1 : 0;   // whole tiles
    int G = 1;
    while (4 * G * G <= (grid >> 3) && G < tiles_m)   // about sqrt(grid / 8) tile rows per group
        G *= 2;
    const int r16 = lane & 15, g = lane >> 4;
    const int lrow = lane >> 3, pch = lane & 7;
    const int NB = (N + (1 << SH) - 1) >> SH;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
    // Scale slot of weight fragment u (block scale: one for the wave's columns;
    // tiles start on weight-scale row boundaries).
    int ws_slot[WSN];
#pragma unroll
    for (int u = 0; u < WSN; ++u)
        ws_slot[u] = BM + ((wn * WN + 16 * u) >> SH);
    const int arow = wm * WM + r16;             // this lane's activation row (scale slots)
    const int arow0 = wm * WM, wrow0 = wn * WN;  // 16-aligned fragment rows
    const FragOff fo = frag_offsets(lane);

    // Copies.  Lane covers row (lane >> 3) of an 8-row group and physical
    // chunk (lane & 7), which holds logical chunk (lane & 7) ^ swizzle(row);
    // its offset from the block's first byte in the tile's first row is the
    // same for every tile (it fits in 32 bits because the host keeps 256 * K
    // below 2^31).  The per-block buffer descriptors end at the last row of
    // the matrix, so rows past M or N read zeros (their outputs are never
    // stored).  The scale copy reads per-lane pointers: lane slot s < BM takes
    // a_scale of tile row s (the last row past M), the lanes above take w_scale
    // of the tile's weight blocks.
    uint32_t a_off[A_LOADS], w_off[W_LOADS];
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) {
        const int row = (wave * A_LOADS + j) * 8 + lrow;
        a_off[j] = (uint32_t)row * (uint32_t)K + (uint32_t)((pch ^ chunk_swizzle(row)) << 4);
    }
#pragma unroll
    for (int j = 0; j < W_LOADS; ++j) {
        const int row = (wave * W_LOADS + j) * 8 + lrow;
        const uint32_t q = (uint32_t)(pch ^ chunk_swizzle(row));
        // packed: copy j moves kilobyte (wave * W_LOADS + j) of the tile's stage unchanged
        const uint32_t half = (uint32_t)(wave * W_LOADS + j);
        w_off[j] = PK ? ((((half >> 1) * (uint32_t)KB) << 11) + ((half & 1u) << 10) + (uint32_t)lane * 16u)
                      : (uint32_t)row * (uint32_t)K + (q << 4);
    }
    const int slot = wave * 64 + lane;
    struct CopyTile {
        int m0, n0;
        const float *s_src;
    };
    // Tile of linear id L (see linear_tile).
    auto copy_at = [&](int L) __attribute__((always_inline)) {
        int tm, tn;
        linear_tile(L, tiles_m, tiles_n, G, tm, tn);
        CopyTile c;
        c.m0 = tm * BM;
        c.n0 = tn * BN;
        // Lanes past the needed slots repeat the last needed address: one
        // cache line, not one per lane.
        c.s_src = !SC         ? p.a_scale
                  : slot < BM ? p.a_scale + (size_t)min(c.m0 + slot, M - 1) * KB
                              : p.w_scale + (size_t)min((c.n0 >> SH) + min(slot - BM, NBW - 1), NB - 1) * KB;
        return c;
    };
    // The i-th whole tile of this workgroup.
    auto copy_tile = [&](int i) __attribute__((always_inline)) { return copy_at(rank + i * grid); };
    // Position v of this workgroup's block stream: its whole tiles, then (SKM)
    // its stream-K run.  Returns the tile's linear id in L and the block in kb.
    const int dp_steps = ntiles * KB;
    auto step_pos = [&](int v, int &L, int &kb) __attribute__((always_inline)) {
        if (v < dp_steps) {
            const int i = v / KB;
            L = rank + i * grid;
            kb = v - i * KB;
        } else {
            const int s = (int)sk_lo + (v - dp_steps);        // < S_sk, which fits 31 bits
            const int t = s / KB;
            L = dp_tiles + t;
            kb = s - t * KB;
        }
    };
    // Descriptors of K block kb of a tile: the rows that exist, minus the
    // bytes before the block in the first row.
    auto rsrc_a = [&](int m0, int kb) __attribute__((always_inline)) {
        return tile_rsrc(p.A + (size_t)m0 * K + (size_t)kb * 128,
                         (uint32_t)min(M - m0, BM) * (uint32_t)K - (uint32_t)kb * 128u);
    };
    // Packed weights: the tile's 16-row tiles from block kb of its first one
    // to the end of its last one that exists.
    auto rsrc_w = [&](int n0, int kb) __attribute__((always_inline)) {
        if (PK) {
            const int t0 = n0 >> 4, tiles = min(((N + 15) >> 4) - t0, BN / 16);
            return tile_rsrc(p.W + (((size_t)t0 * KB + kb) << 11),
                             ((uint32_t)tiles * (uint32_t)KB - (uint32_t)kb) << 11);
        }
        return tile_rsrc(p.W + (size_t)n0 * K + (size_t)kb * 128,
                         (uint32_t)min(N - n0, BN) * (uint32_t)K - (uint32_t)kb * 128u);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    // Prologue: the first AHEAD blocks of the copy stream in flight, then the
    // fragments of block 0.  (Stream position q is block q % KB of this
    // workgroup's tile q / KB; past the end it repeats the last block, into
    // stages nobody reads again.)
    const int steps = dp_steps + (int)(sk_hi - sk_lo);
#pragma unroll
    for (int s = 0; s < AHEAD; ++s) {
        const int q = min(s, steps - 1);
        int cL, ckb;
        step_pos(q, cL, ckb);
        const CopyTile c = copy_at(cL);
        issue_tile_loads<A_LOADS, W_LOADS, A_BYTES, W_BYTES, SC>(rsrc_a(c.m0, ckb), rsrc_w(c.n0, ckb), a_off, w_off,
                                                            c.s_src, ckb, lds0 + (uint32_t)(s * STAGE), wave);
    }
    wait_vmcnt<(AHEAD - 1) * PER_BLOCK>();
    __syncthreads();
    v8i wf[TN], af;
    float sa[TM] = {}, ws[WSN] = {};
    {
        const uint8_t *sA = smem, *sW = smem + A_BYTES;
        const float *sS = reinterpret_cast<const float *>(sW + W_BYTES);
        wf[0] = lds_w_fragment<PK>(sW, wrow0, fo, lane);
        af = lds_fragment(sA, arow0, fo);
#pragma unroll
        for (int u = 1; u < TN; ++u)
            wf[u] = lds_w_fragment<PK>(sW, wrow0 + 16 * u, fo, lane);
        if constexpr (SC) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
                sa[t] = sS[arow + 16 * t];
#pragma unroll
            for (int u = 0; u < WSN; ++u)
                ws[u] = sS[ws_slot[u]];
        }
    }

    // Last slice of the previous block, scaled at the start of the next one
    // (zero before a tile's first block: adds exactly +0).
    v4f d_last[TN];
#pragma unroll
    for (int u = 0; u < TN; ++u)
        d_last[u] = (v4f){0.f, 0.f, 0.f, 0.f};
    float s_last = 0.f;

    // One K block at stream position `step`; its copies fetch block ckb of the
    // copy tile described by ra, rw and s_src.
    auto block = [&](int step, v4i ra, v4i rw, const float *s_src, int ckb) __attribute__((always_inline)) {
        const uint8_t *sA = smem + (step % STAGES) * STAGE;
        const uint32_t cstage = lds0 + (uint32_t)(((step + AHEAD) % STAGES) * STAGE);

        // Slice t multiplies activation slice t and scales the MFMA results of
        // slice t-1 (slice 0: the previous block's last slice).  Scales are
        // formed where they are used, so no wave waits for the scale reads of
        // the previous block before its barrier.
        v4f d[TN];
        float s_cur = 0.f;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const float sc_prev = t > 0 ? sa[t - 1] * ws[0] : s_last;
            if (t == TM - 1) {
                wait_vmcnt<VM_AT_BARRIER>();   // this wave's copies of the next block have landed
                __syncthreads();               // ... every wave's; this block's stage is read out
            }
            if (!LATE && t < SPREAD) {
#pragma unroll
                for (int j = t * CPS; j < (t + 1) * CPS && j < PER_BLOCK; ++j)
                    issue_one<A_LOADS, W_LOADS, A_BYTES, W_BYTES, SC>(j, ra, rw, a_off, w_off, s_src, ckb, cstage, wave);
            }
            v8i af_next = af;
            if (t + 1 < TM)
                af_next = lds_fragment(sA, arow0 + 16 * (t + 1), fo);
            v4f dn[TN];
            // Raised wave priority while this slice's MFMAs issue: the matrix
            // core is fed first when both waves of a SIMD have work.
            __builtin_amdgcn_s_setprio(1);
            if constexpr (SM != SM_BLOCK) {
                // MX: the block's scales go into the MFMA; row-wise: no per-block
                // scale.  Either way the MFMA accumulates in place.
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    acc[t][u] = block_step<SM>(acc[t][u], wf[u], af, ws[WSN > 1 ? u : 0], sa[t], g);
            } else {
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    dn[u] = mfma_block(wf[u], af);
            }
            if (t == TM - 1) {
                // The next block: its stage is complete (barrier above).  Weight
                // fragment u is read right after MFMA u has taken the old one.
                // After the last block these read a stale stage, unused.
                s_cur = sa[TM - 1] * ws[0];
                const uint8_t *nA = smem + ((step + 1) % STAGES) * STAGE, *nW = nA + A_BYTES;
                const float *nS = reinterpret_cast<const float *>(nW + W_BYTES);
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    wf[u] = lds_w_fragment<PK>(nW, wrow0 + 16 * u, fo, lane);
                af_next = lds_fragment(nA, arow0, fo);
                if constexpr (SC) {
#pragma unroll
                    for (int s = 0; s < TM; ++s)
                        sa[s] = nS[arow + 16 * s];
#pragma unroll
                    for (int u = 0; u < WSN; ++u)
                        ws[u] = nS[ws_slot[u]];
                }
            }
            if constexpr (SM == SM_BLOCK) {
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    if (t > 0)
                        acc[t - 1][u] = fma4(d[u], sc_prev, acc[t - 1][u]);
                    else
                        acc[TM - 1][u] = fma4(d_last[u], sc_prev, acc[TM - 1][u]);
                }
            }
            // Issue order: the next slice's activation fragment reads first
            // (most time to land), then each MFMA followed by a share of the
            // scale FMAs, which run on the vector ALU while the matrix core
            // works (in the last slice also the next block's weight fragment).
            if (t + 1 < TM)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (t == TM - 1)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, FMA_GROUP, 0);
            }
            __builtin_amdgcn_s_setprio(0);
            if (LATE && t == TM - 1) {
#pragma unroll
                for (int j = 0; j < PER_BLOCK; ++j)
                    issue_one<A_LOADS, W_LOADS, A_BYTES, W_BYTES, SC>(j, ra, rw, a_off, w_off, s_src, ckb, cstage, wave);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u)
                d[u] = dn[u];
            af = af_next;
            __builtin_amdgcn_sched_barrier(0);   // keep each slice's work together
        }
#pragma unroll
        for (int u = 0; u < TN; ++u)
            d_last[u] = d[u];
        s_last = s_cur;
    };

    // A tile's blocks are done: fold in the last slice (block scale).
    auto fold_last = [&]() __attribute__((always_inline)) {
        if constexpr (SM == SM_BLOCK) {
#pragma unroll
            for (int u = 0; u < TN; ++u)
                acc[TM - 1][u] = fma4(d_last[u], s_last, acc[TM - 1][u]);
        }
    };
    // Round the tile to bf16 and store it.
    auto store_tile = [&](const CopyTile &cur) __attribute__((always_inline)) {
        const int n_base = cur.n0 + wn * WN + 4 * g;
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int m = cur.m0 + wm * WM + 16 * t + r16;
            if (m < M) {
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    store4(p.Y, (int64_t)m * N, n_base + 16 * u, N, vec_store != 0,
                           rowwise_scale<SM>(acc[t][u], p, m, n_base + 16 * u));
            }
        }
    };
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < TN; ++u)
            d_last[u] = (v4f){0.f, 0.f, 0.f, 0.f};
        s_last = 0.f;
    };

    if constexpr (!SKM) {
        // Per tile: the blocks whose copies stay inside the tile, then the last
        // AHEAD blocks, whose copies already fetch the next tile, then the stores.
        const int main_blocks = KB - AHEAD > 0 ? KB - AHEAD : 0;
        int step = 0;
        for (int tile = 0; tile < ntiles; ++tile) {
            const CopyTile cur = copy_tile(tile);
            for (int kb = 0; kb < main_blocks; ++kb, ++step)
                block(step, rsrc_a(cur.m0, kb + AHEAD), rsrc_w(cur.n0, kb + AHEAD), cur.s_src, kb + AHEAD);
            for (int kb = main_blocks; kb < KB; ++kb, ++step) {
                const int q = min(step + AHEAD, steps - 1);
                const CopyTile c = copy_tile(q / KB);
                const int ckb = q % KB;
                block(step, rsrc_a(c.m0, ckb), rsrc_w(c.n0, ckb), c.s_src, ckb);
            }
            fold_last();
            store_tile(cur);
            reset();
        }
    } else {
        // Pieces of the block stream: each lies in one tile, a whole tile (the
        // round-robin ones and some of the stream-K run) or a cut piece of a
        // stream-K tile.  As in the loop above, the blocks whose copies stay
        // inside the piece take kb + AHEAD, the last AHEAD look the copy target
        // up in the stream.
        //
        // Fixup of stream-K tile tp, cut between runs r_lo..r_hi (the runs
        // whose steps meet [tp KB, (tp + 1) KB)): every piece writes its fp32
        // partial tile to the call's workspace with device-coherent stores and
        // goes on with its run; at the end of the run the workgroup waits for
        // its stores and counts each of its pieces in that tile's counter.
        // The last piece of a tile to be counted sums the pieces in run order
        // r_lo, r_lo + 1, ... (a fixed order whatever the arrival order, so the
        // result is bitwise reproducible), stores the tile and resets the
        // counter to zero for the next call.  Nothing waits on another
        // workgroup.  A run holds at most two cut pieces: the one with its
        // first step goes to partial slot 2r, the one with its last to 2r + 1
        // (workspace: counters [batch][sk_tiles], then [batch][2 grid][BM * BN]
        // fp32 partials; a slot is [wave][t][u][lane][4]).
        constexpr int TILE_F = BM * BN, WAVE_F = TM * TN * 256;
        const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(p.ws + (size_t)blockIdx.y * 2 * grid * TILE_F,
                                                        (uint32_t)(2 * grid) * (uint32_t)TILE_F * 4u);
        const int lane_off = (wave * WAVE_F + lane * 4) * 4;              // bytes, + ((t TN + u) 64 * 4) * 4
        // Pieces of tile tp: the runs r_lo..r_hi (aligned: ranks tp, tp + T, ...,
        // one piece each), in the order they are summed.
        auto sk_range = [&](int tp, int &r_lo, int &r_hi) __attribute__((always_inline)) {
            if (aligned) {
                r_lo = 0;
                r_hi = S_al - 1;
                return;
            }
            const int64_t x0 = (int64_t)tp * KB;
            r_lo = (int)min((int64_t)grid - 1, ((x0 + 1) * grid - 1) / S_sk);
            r_hi = (int)min((int64_t)grid - 1, ((x0 + KB) * grid - 1) / S_sk);
        };
        auto piece_rank = [&](int tp, int j) __attribute__((always_inline)) { return aligned ? tp + j * T : j; };
        auto slot_of = [&](int r, int tp) __attribute__((always_inline)) {
            if (aligned)
                return 2 * r;
            return 2 * r + ((int64_t)r * S_sk / grid >= (int64_t)tp * KB ? 0 : 1);
        };
        auto write_partial = [&](int tp) __attribute__((always_inline)) {
            const int soff = slot_of(rank, tp) * TILE_F * 4;
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[t][u]), pres,
                                                           lane_off + (t * TN + u) * 1024, soff, 16 /* sc1 */);
        };
        // Count this workgroup's piece of tile tp; the last one sums and stores the tile.
        auto finish_piece = [&](int tp) __attribute__((always_inline)) {
            int r_lo, r_hi;
            sk_range(tp, r_lo, r_hi);
            int32_t *cnt = p.cnt + (size_t)blockIdx.y * sk_tiles + tp;
            __syncthreads();                                     // sk_last of the previous piece is read out
            if (threadIdx.x == 0)
                sk_last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == r_hi - r_lo;
            __syncthreads();
            if (!sk_last)
                return;
            // Every other piece was counted after its stores completed.
            for (int j = r_lo; j <= r_hi; ++j) {
                const int r = piece_rank(tp, j);
                const int soff = slot_of(r, tp) * TILE_F * 4;
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int u = 0; u < TN; ++u) {
                        const v4f x = __builtin_bit_cast(
                            v4f, __builtin_amdgcn_raw_buffer_load_b128(pres, lane_off + (t * TN + u) * 1024, soff,
                                                                       16 /* sc1 */));
                        if (j == r_lo) {
                            acc[t][u] = x;
                        } else {
                            acc[t][u][0] += x[0];
                            acc[t][u][1] += x[1];
                            acc[t][u][2] += x[2];
                            acc[t][u][3] += x[3];
                        }
                    }
            }
            store_tile(copy_at(dp_tiles + tp));
            if (threadIdx.x == 0)
                __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            reset();
        };
        int pend0 = -1, pend1 = -1;                              // cut pieces written, counted at the end
        int v = 0;
        while (v < steps) {
            int L, kb0;
            step_pos(v, L, kb0);
            const int len = min(KB - kb0, steps - v);
            const CopyTile cur = copy_at(L);
            const int inner = len - AHEAD > 0 ? len - AHEAD : 0;
            for (int j = 0; j < inner; ++j, ++v)
                block(v, rsrc_a(cur.m0, kb0 + j + AHEAD), rsrc_w(cur.n0, kb0 + j + AHEAD), cur.s_src, kb0 + j + AHEAD);
            for (int j = inner; j < len; ++j, ++v) {
                const int q = min(v + AHEAD, steps - 1);
                int cL, ckb;
                step_pos(q, cL, ckb);
                const CopyTile c = copy_at(cL);
                block(v, rsrc_a(c.m0, ckb), rsrc_w(c.n0, ckb), c.s_src, ckb);
            }
            fold_last();
            if (kb0 == 0 && len == KB) {
                store_tile(cur);
            } else {
                write_partial(L - dp_tiles);
                if (pend0 < 0)
                    pend0 = L - dp_tiles;
                else
                    pend1 = L - dp_tiles;
            }
            reset();
        }
        if (pend0 >= 0) {
            wait_vmcnt<0>();                                     // this wave's partial stores are complete
            finish_piece(pend0);                                 // (its first barrier: every wave's)
            if (pend1 >= 0)
                finish_piece(pend1);
        }
    }
    wait_vmcnt<0>();                      // no copy into LDS may outlive the workgroup
}

// Explicit instantiations (emit the host-side launch stubs).
#define A8W8_PTILE_INST1(BM, BN, WGM, WGN, S, SKM)                                             \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, false, 0>(Args, int);     \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, true, 0>(Args, int);      \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, false, 1>(Args, int);     \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, true, 1>(Args, int);      \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, false, 2>(Args, int);     \
    template __global__ void ptile_kernel<BM, BN, WGM, WGN, S, SKM, true, 2>(Args, int);
#define A8W8_PTILE_INST(BM, BN, WGM, WGN, S) A8W8_PTILE_INST1(BM, BN, WGM, WGN, S, false)
A8W8_PTILE_INST(256, 256, 2, 4, 2)
A8W8_PTILE_INST(256, 128, 2, 4, 3)
A8W8_PTILE_INST(128, 256, 2, 4, 3)
A8W8_PTILE_INST(128, 128, 2, 2, 2)
A8W8_PTILE_INST(128, 128, 2, 2, 4)
A8W8_PTILE_INST(64, 64, 2, 2, 4)
A8W8_PTILE_INST(32, 64, 2, 2, 6)
A8W8_PTILE_INST(32, 32, 2, 2, 4)
A8W8_PTILE_INST(32, 32, 2, 2, 8)
A8W8_PTILE_INST(128, 128, 2, 4, 4)
A8W8_PTILE_INST(128, 128, 2, 4, 2)
A8W8_PTILE_INST(128, 128, 4, 2, 3)
A8W8_PTILE_INST1(256, 256, 2, 4, 2, true)
A8W8_PTILE_INST1(256, 128, 2, 4, 3, true)
A8W8_PTILE_INST1(128, 256, 2, 4, 3, true)
A8W8_PTILE_INST1(128, 128, 2, 2, 2, true)
#undef A8W8_PTILE_INST
#undef A8W8_PTILE_INST1

// ---------------------------------------------------------------------------
// One-workgroup-per-tile kernel ("tile").  The same block scaling and LDS
// layout as ptile_kernel, with a simpler schedule: one barrier at the start of
// each block, after which every wave issues all copies of the block STAGES-1
// steps ahead and reads its fragments of the current block.  It keeps a
// shorter dependence chain per block, which wins where few, short blocks
// dominate (tiny N, latency-bound) and for some mid-size tiles; the tuner
// picks between the two per shape.  Copies address global memory with 64-bit
// per-lane pointers (rows past M or N repeat the last valid row) and the
// weight scales come through scalar loads.

__device__ __forceinline__ void dma16_at(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(m0), "v"(src) : "memory", "m0");
}

__device__ __forceinline__ void dma4_at(const void *src, const void *lds_dst)
{
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds_dst);
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 4\n\tglobal_load_lds_dword %1, off" : : "s"(m0), "v"(src) : "memory", "m0");
}

template <int A_LOADS, int W_LOADS, bool SC>
__device__ __forceinline__ void issue_block_copies(const uint8_t *const (&a_src)[A_LOADS],
                                                 const uint8_t *const (&w_src)[W_LOADS], const float *as_src,
                                                 int kb, uint8_t *stage, int a_bytes, int w_bytes, int wave,
                                                 int w_block_stride)
{
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i)
        dma16_at(a_src[i] + (size_t)kb * 128, stage + (wave * A_LOADS + i) * 1024);
#pragma unroll
    for (int i = 0; i < W_LOADS; ++i)
        dma16_at(w_src[i] + (size_t)kb * w_block_stride, stage + a_bytes + (wave * W_LOADS + i) * 1024);
    if constexpr (SC)
        dma4_at(as_src + kb, stage + a_bytes + w_bytes + wave * 256);
}


// Work item of workgroup `b` among T items (T = the grid): workgroups are
// dispatched to the 8 XCDs round-robin (b % 8), so each XCD is given a
// contiguous range of item ids.  group_tile then runs tiles in groups of G
// tile-rows, column by column, so the workgroups that are resident together
// on one XCD share A rows and W rows in that XCD's L2.  Both are bijections:
// results do not depend on them.
__device__ __forceinline__ int xcd_item(int b, int T)
{
    const int xcd = b & 7, local = b >> 3;
    const int q = T >> 3, r = T & 7;
    return xcd * q + min(xcd, r) + local;
}
__device__ __forceinline__ void group_tile(int t, int tiles_m, int tiles_n, int G, int &tm, int &tn)
{
    const int per_group = G * tiles_n;
    const int group = t / per_group;
    const int first_m = group * G;
    const int gsize = min(tiles_m - first_m, G);
    const int in_group = t - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}


// Split K (p.splits = S > 1, for shapes with too few output tiles to fill the
// chip): the grid holds S workgroups per tile -- work item t = S * tile + s,
// XCD-contiguous as above, so a tile's splits mostly share one L2 -- and split
// s walks K blocks [s KB / S, (s + 1) KB / S).  Each writes its fp32 partial
// tile to the call's workspace with device-scope stores, waits for them to
// complete and counts itself in the tile's counter;
// the last of the S to arrive sums the S partials in split order 0, 1, ...
// (a fixed order whatever the arrival order, so the result is bitwise
// reproducible), rounds and stores the tile, and resets the counter to zero
// for the next call.  Nothing waits on another workgroup.
//
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
template <int BM, int BN, int WGM, int WGN, int STAGES, bool PK, int SM>
__global__ __launch_bounds__(WGM * WGN * 64) void tile_kernel(Args p, int vec_store)
{
    select_batch(p);
    constexpr int NWAVES = WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int A_BYTES = BM * 128, W_BYTES = BN * 128;
    constexpr int STAGE = A_BYTES + W_BYTES + NWAVES * 256;
    constexpr int A_LOADS = BM / (8 * NWAVES), W_LOADS = BN / (8 * NWAVES);   // 1 KB loads per wave per block
    constexpr bool SC = SM != SM_ROWWISE;                                    // per-block scale copies
    constexpr int PER_BLOCK = A_LOADS + W_LOADS + (SC ? 1 : 0);              // vector-memory ops per block
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
    const int S = p.splits;                                  // 1 <= S <= KB
    const int item = xcd_item((int)blockIdx.x, tiles_m * tiles_n * S);
    const int tile_lin = item / S, split = item - tile_lin * S;
    int tmi, tni;
    group_tile(tile_lin, tiles_m, tiles_n, BM >= 256 ? 2 : 4, tmi, tni);
    const int m0 = tmi * BM, n0 = tni * BN;
    const int kb_lo = split * KB / S, nkb = (split + 1) * KB / S - kb_lo;   // this split's K blocks
    const int r16 = lane & 15, g = lane >> 4;
    const FragOff fo = frag_offsets(lane);

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
        // packed: copy i moves kilobyte (wave * W_LOADS + i) of the tile's stage unchanged
        const int half = wave * W_LOADS + i;
        const int tile = min((n0 >> 4) + (half >> 1), ((N + 15) >> 4) - 1);
        w_src[i] = PK ? p.W + (((size_t)tile * KB) << 11) + ((half & 1) << 10) + lane * 16
                      : p.W + (size_t)min(n0 + row, N - 1) * K + ((pch ^ chunk_swizzle(row)) << 4);
    }
    // Activation scales: wave w copies tile rows 64w + lane (rows past the tile
    // or past M repeat a valid row and are never read).
    const float *as_src = SC ? p.a_scale + (size_t)min(m0 + min(wave * 64 + lane, BM - 1), M - 1) * KB : p.a_scale;
    const int w_stride = PK ? 2048 : 128;   // bytes from one K block of a weight row to the next
    // Weight scales through scalar loads: one row for the wave's columns
    // (block scale), or the row of each 16-row fragment u (MX).
    constexpr int SH = wscale_shift<SM>();
    constexpr int WSN = SM == SM_MX ? TN : 1;
    const int NB = (N + (1 << SH) - 1) >> SH;
    const_f32 *wsp[WSN];
#pragma unroll
    for (int u = 0; u < WSN; ++u)
        wsp[u] = (const_f32 *)(p.w_scale + (size_t)min((n0 + wn * WN + 16 * u) >> SH, NB - 1) * KB);

    v4f acc[TM][TN];
#pragma unroll
    for (int t = 0; t < TM; ++t)
#pragma unroll
        for (int u = 0; u < TN; ++u)
            acc[t][u] = (v4f){0.f, 0.f, 0.f, 0.f};

    // Prologue: blocks 0 .. STAGES-2 of the split in flight (indices past its
    // end repeat its last block).
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        issue_block_copies<A_LOADS, W_LOADS, SC>(a_src, w_src, as_src, kb_lo + min(st, nkb - 1), smem + st * STAGE,
                                           A_BYTES, W_BYTES, wave, w_stride);
    float ws_next[WSN] = {};
    if constexpr (SC) {
#pragma unroll
        for (int u = 0; u < WSN; ++u)
            ws_next[u] = wsp[u][kb_lo];
    }

    for (int kb = 0; kb < nkb; ++kb) {
        float ws[WSN];
#pragma unroll
        for (int u = 0; u < WSN; ++u)
            ws[u] = ws_next[u];
        wait_vmcnt<(STAGES - 2) * PER_BLOCK>();   // this wave's copies of block kb have landed
        __syncthreads();                          // ... every wave's, and stage (kb-1) % STAGES is free
        const int kn = kb_lo + min(kb + STAGES - 1, nkb - 1);
        issue_block_copies<A_LOADS, W_LOADS, SC>(a_src, w_src, as_src, kn, smem + ((kb + STAGES - 1) % STAGES) * STAGE,
                                           A_BYTES, W_BYTES, wave, w_stride);
        if constexpr (SC) {
#pragma unroll
            for (int u = 0; u < WSN; ++u)
                ws_next[u] = wsp[u][kb_lo + min(kb + 1, nkb - 1)];
        }

        const uint8_t *sA = smem + (kb % STAGES) * STAGE;
        const uint8_t *sW = sA + A_BYTES;
        const float *sS = reinterpret_cast<const float *>(sW + W_BYTES);
        if constexpr (SM != SM_BLOCK) {
            // MX: scales inside the MFMA; row-wise: none per block.  The MFMA
            // accumulates in place.
            v8i wf[TN];
#pragma unroll
            for (int u = 0; u < TN; ++u)
                wf[u] = lds_w_fragment<PK>(sW, wn * WN + 16 * u, fo, lane);
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const float sa = SC ? sS[wm * WM + 16 * t + r16] : 0.f;
                const v8i af = lds_fragment(sA, wm * WM + 16 * t, fo);
#pragma unroll
                for (int u = 0; u < TN; ++u)
                    acc[t][u] = block_step<SM>(acc[t][u], wf[u], af, ws[WSN > 1 ? u : 0], sa, g);
            }
            continue;
        }
        float sc[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t)
            sc[t] = sS[wm * WM + 16 * t + r16] * ws[0];
        v8i wf[TN];
#pragma unroll
        for (int u = 0; u < TN; ++u)
            wf[u] = lds_w_fragment<PK>(sW, wn * WN + 16 * u, fo, lane);
        v4f d[2][TN];
        {
            const v8i af = lds_fragment(sA, wm * WM, fo);
#pragma unroll
            for (int u = 0; u < TN; ++u)
                d[0][u] = mfma_block(wf[u], af);
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            if (t + 1 < TM) {
                const v8i af = lds_fragment(sA, wm * WM + 16 * (t + 1), fo);
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

    if (S > 1) {
        // Partial tile of split s: [tile][s][wave][t][u][lane][4] fp32 in this batch's
        // workspace, written and read with 16-byte device-coherent (sc1) accesses,
        // which are coherent across the XCDs' L2s by themselves: no cache-wide
        // writeback or invalidate, which would cost every other tile its cached
        // operands.  Each instruction moves 1 KB contiguous per wave.
        constexpr int TILE_F = BM * BN, WAVE_F = TM * TN * 256;
        const size_t tile_g = (size_t)blockIdx.y * tiles_m * tiles_n + tile_lin;
        const __amdgpu_buffer_rsrc_t pres = buffer_rsrc(p.ws + tile_g * S * TILE_F, (uint32_t)S * TILE_F * 4u);
        const int lane_off = (wave * WAVE_F + lane * 4) * 4;              // bytes, + (t TN + u) * 1024
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int u = 0; u < TN; ++u)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, acc[t][u]), pres,
                                                       lane_off + (t * TN + u) * 1024, split * TILE_F * 4,
                                                       16 /* sc1 */);
        __shared__ int last;
        wait_vmcnt<0>();                                     // this wave's partial stores are complete
        __syncthreads();                                     // ... and every wave's
        if (threadIdx.x == 0)
            last = __hip_atomic_fetch_add(p.cnt + tile_g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        __syncthreads();
        if (!last)
            return;
        // The last split: every other split counted itself after its stores
        // completed.  Sum in split order 0, 1, ... (its own partial included).
        for (int s2 = 0; s2 < S; ++s2) {
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int u = 0; u < TN; ++u) {
                    const v4f x = __builtin_bit_cast(
                        v4f, __builtin_amdgcn_raw_buffer_load_b128(pres, lane_off + (t * TN + u) * 1024,
                                                                   s2 * TILE_F * 4, 16 /* sc1 */));
                    if (s2 == 0) {
                        acc[t][u] = x;
                    } else {
                        acc[t][u][0] += x[0];
                        acc[t][u][1] += x[1];
                        acc[t][u][2] += x[2];
                        acc[t][u][3] += x[3];
                    }
                }
        }
        if (threadIdx.x == 0)
            __hip_atomic_store(p.cnt + tile_g, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

#pragma unroll
    for (int t = 0; t < TM; ++t) {
        const int m = m0 + wm * WM + 16 * t + r16;
        if (m < M) {
#pragma unroll
            for (int u = 0; u < TN; ++u)
                store4(p.Y, (int64_t)m * N, n0 + wn * WN + 16 * u + 4 * g, N, vec_store != 0,
                       rowwise_scale<SM>(acc[t][u], p, m, n0 + wn * WN + 16 * u + 4 * g));
        }
    }
}


#define A8W8_TILE_INST(BM, BN, WGM, WGN, S)                                                   \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, false, 0>(Args, int);           \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, true, 0>(Args, int);            \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, false, 1>(Args, int);           \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, true, 1>(Args, int);            \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, false, 2>(Args, int);           \
    template __global__ void tile_kernel<BM, BN, WGM, WGN, S, true, 2>(Args, int);
A8W8_TILE_INST(256, 256, 2, 4, 2)
A8W8_TILE_INST(256, 128, 2, 4, 3)
A8W8_TILE_INST(128, 256, 2, 4, 3)
A8W8_TILE_INST(128, 128, 2, 2, 2)
A8W8_TILE_INST(128, 128, 2, 2, 4)
A8W8_TILE_INST(128, 64, 2, 2, 3)
A8W8_TILE_INST(64, 128, 2, 2, 3)
A8W8_TILE_INST(64, 64, 2, 2, 3)
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

// Each instance is compiled six times: fn[2 * sm + wpk], for each scale kind
// sm (SM_BLOCK, SM_MX, SM_ROWWISE) and row-layout (wpk 0) or packed (wpk 1)
// weights.
struct Entry {
    Variant v;
    const void *fn[6];
    int lds_bytes;
    // Row-range skinny instances: the fused-quantisation kernels [log2 MQ][packed W].
    const void *fq[5][2];
};

#define FN_ONE(PKV, SMV, ...) reinterpret_cast<const void *>(&__VA_ARGS__, PKV, SMV>)
#define FN6(...) {FN_ONE(false, 0, __VA_ARGS__), FN_ONE(true, 0, __VA_ARGS__), \
                  FN_ONE(false, 1, __VA_ARGS__), FN_ONE(true, 1, __VA_ARGS__), \
                  FN_ONE(false, 2, __VA_ARGS__), FN_ONE(true, 2, __VA_ARGS__)}
#define SKINNY(TPW, D, NW) {{A8W8_KERNEL_SKINNY, 16, 16 * TPW, NW, D, 16, 0, 1, "skinny_r" #TPW "_d" #D "_w" #NW}, \
                            FN6(skinny_kernel<TPW, D, NW, false), 0}
// The same kernel with K split over SPLIT workgroups per row group (name suffix _k<SPLIT>).
#define SKINNY_SK(TPW, D, NW, SPLIT) {{A8W8_KERNEL_SKINNY, 16, 16 * TPW, NW, D, 16, 0, SPLIT, \
                                       "skinny_r" #TPW "_d" #D "_w" #NW "_k" #SPLIT}, \
                                      FN6(skinny_kernel<TPW, D, NW, true), 0}
// Persistent tile grids are sized for WPC waves per CU: 8 (two per SIMD) for
// the instances above 128 VGPRs, 16 for the small ones, or fewer workgroups
// where their LDS does not fit.
constexpr int tile_per_cu(int lds_bytes, int waves, int wpc)
{
    return cmin(163840 / lds_bytes, wpc / waves) > 0 ? cmin(163840 / lds_bytes, wpc / waves) : 1;
}
#define TILE(BM, BN, WGM, WGN, S) {{A8W8_KERNEL_TILE, BM, BN, WGM * WGN, S, 0, 0, 1, \
                                    "tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_s" #S}, \
                                   FN6(tile_kernel<BM, BN, WGM, WGN, S), \
                                   S * ((BM + BN) * 128 + WGM * WGN * 256)}
// The same kernel with K split over SPLIT workgroups per tile (name suffix _k<SPLIT>).
#define TILE_SK(BM, BN, WGM, WGN, S, SPLIT) {{A8W8_KERNEL_TILE, BM, BN, WGM * WGN, S, 0, 0, SPLIT, \
                                    "tile_" #BM "x" #BN "_w" #WGM "x" #WGN "_s" #S "_k" #SPLIT}, \
                                   FN6(tile_kernel<BM, BN, WGM, WGN, S), \
                                   S * ((BM + BN) * 128 + WGM * WGN * 256)}
#define PTILE(BM, BN, WGM, WGN, S, WPC) {{A8W8_KERNEL_PTILE, BM, BN, WGM * WGN, S, 0, \
                                    tile_per_cu(S * ((BM + BN) * 128 + WGM * WGN * 256), WGM * WGN, WPC), 1, \
                                    "ptile_" #BM "x" #BN "_w" #WGM "x" #WGN "_s" #S}, \
                                   FN6(ptile_kernel<BM, BN, WGM, WGN, S, false), \
                                   S * ((BM + BN) * 128 + WGM * WGN * 256)}
// The persistent tile kernel in stream-K mode (see ptile_kernel): the last one
// or two waves of tiles are cut into equal runs of K blocks, one per workgroup.
#define SKTILE(BM, BN, WGM, WGN, S, WPC) {{A8W8_KERNEL_SKTILE, BM, BN, WGM * WGN, S, 0, \
                                    tile_per_cu(S * ((BM + BN) * 128 + WGM * WGN * 256), WGM * WGN, WPC), 1, \
                                    "sktile_" #BM "x" #BN "_w" #WGM "x" #WGN "_s" #S}, \
                                   FN6(ptile_kernel<BM, BN, WGM, WGN, S, true), \
                                   S * ((BM + BN) * 128 + WGM * WGN * 256)}

#define TALL(TPW, NT, D, NW) {{A8W8_KERNEL_TALL, 16 * TPW, 16 * NT, NW, D, 0, 0, 1, \
                               "tall_r" #TPW "_n" #NT "_d" #D "_w" #NW}, \
                              FN6(tall_kernel<TPW, NT, D, NW), 0}
#define PSKINNY(D, NW, P) {{A8W8_KERNEL_PSKINNY, 16, 16, NW, D, 16, 1, 1, "pskinny_d" #D "_w" #NW "_p" #P}, \
                           FN6(pskinny_kernel<D, NW, P), 0}
// Fused quantisation: the weight blocks issued with the bf16 activations, all
// of them where the registers allow, else as many as fit (at least one); the
// rest follow once the activations are codes.  A wave of an NW-wave workgroup
// has 2048 / NW VGPRs; the activations take 16 D (MQ = 16) or MQ D of them,
// each weight block 8 T, and addresses, accumulators, codes and temporaries
// about 48 + 8 D (MQ = 16) or 40 + 4 D (as the compiler allocated them).
constexpr int rsk_qe_fit(int T, int D, int NW, int MQ)
{
    return (2048 / NW - (MQ == 16 ? 16 * D + 48 + 8 * D : MQ * D + 40 + 4 * D)) / (8 * T);
}
constexpr int rsk_qe(int T, int D, int NW, int MQ)
{
    return rsk_qe_fit(T, D, NW, MQ) >= D ? D : rsk_qe_fit(T, D, NW, MQ) >= 1 ? rsk_qe_fit(T, D, NW, MQ) : 1;
}
#define FQ(T, D, NW, PK, MQ) \
    reinterpret_cast<const void *>(&rskinny_kernel<T, D, NW, PK, SM_BLOCK, true, rsk_qe(T, D, NW, MQ), MQ>)
#define FQ2(T, D, NW, MQ) {FQ(T, D, NW, false, MQ), FQ(T, D, NW, true, MQ)}
// Row-range skinny: T tiles per workgroup at most, about G = WPC workgroups per CU.
#define RSKINNY(T, D, NW, WPC) {{A8W8_KERNEL_RSKINNY, 16, 16 * T, NW, D, 16, WPC, 1, \
                                 "rskinny_t" #T "_d" #D "_w" #NW "_g" #WPC}, FN6(rskinny_kernel<T, D, NW), 0, \
                                {FQ2(T, D, NW, 1), FQ2(T, D, NW, 2), FQ2(T, D, NW, 4), FQ2(T, D, NW, 8), \
                                 FQ2(T, D, NW, 16)}}

const Entry kEntries[] = {
    SKINNY(1, 5, 8), SKINNY(2, 5, 8), SKINNY(4, 5, 8), SKINNY(1, 6, 8), SKINNY(2, 6, 8),
    SKINNY(1, 3, 16), SKINNY(2, 3, 16), SKINNY(1, 10, 4), SKINNY(1, 12, 4), SKINNY(1, 2, 4),
    TILE(256, 256, 2, 4, 2), TILE(256, 128, 2, 4, 3), TILE(128, 256, 2, 4, 3), TILE(128, 128, 2, 2, 2),
    TILE(128, 128, 2, 2, 4), TILE(128, 64, 2, 2, 3), TILE(64, 128, 2, 2, 3), TILE(64, 64, 2, 2, 3),
    TILE(128, 32, 4, 1, 3), TILE(32, 128, 1, 4, 3), TILE(32, 64, 2, 2, 3), TILE(64, 32, 2, 2, 3), TILE(32, 32, 2, 2, 3),
    PTILE(256, 256, 2, 4, 2, 8), PTILE(256, 128, 2, 4, 3, 8), PTILE(128, 256, 2, 4, 3, 8), PTILE(128, 128, 2, 2, 2, 8),
    PTILE(128, 128, 2, 2, 4, 8), PTILE(64, 64, 2, 2, 4, 16), PTILE(32, 64, 2, 2, 6, 16), PTILE(32, 32, 2, 2, 4, 16),
    PTILE(32, 32, 2, 2, 8, 16),
    PSKINNY(5, 8, 2), PSKINNY(4, 10, 3), PSKINNY(6, 8, 2),
    TALL(1, 2, 3, 8), TALL(2, 2, 3, 8), TALL(4, 2, 3, 8), TALL(2, 2, 6, 8), TALL(1, 2, 6, 8), TALL(1, 2, 3, 16),
    TALL(1, 1, 3, 8), TALL(2, 1, 3, 8), TALL(4, 1, 3, 8),
    TILE_SK(256, 256, 2, 4, 2, 2), TILE_SK(256, 128, 2, 4, 3, 2), TILE_SK(256, 128, 2, 4, 3, 4),
    TILE_SK(128, 256, 2, 4, 3, 2), TILE_SK(128, 256, 2, 4, 3, 4), TILE_SK(128, 128, 2, 2, 4, 2),
    TILE_SK(128, 128, 2, 2, 4, 4), TILE_SK(128, 128, 2, 2, 4, 8), TILE_SK(128, 64, 2, 2, 3, 2),
    TILE_SK(128, 64, 2, 2, 3, 4), TILE_SK(64, 128, 2, 2, 3, 2), TILE_SK(64, 128, 2, 2, 3, 4),
    TILE_SK(64, 128, 2, 2, 3, 8), TILE_SK(64, 64, 2, 2, 3, 2), TILE_SK(64, 64, 2, 2, 3, 4),
    TILE_SK(64, 64, 2, 2, 3, 8), TILE_SK(32, 128, 1, 4, 3, 4), TILE_SK(32, 128, 1, 4, 3, 8),
    TILE_SK(32, 64, 2, 2, 3, 4), TILE_SK(32, 64, 2, 2, 3, 8), TILE_SK(64, 32, 2, 2, 3, 4),
    TILE_SK(64, 32, 2, 2, 3, 8), TILE_SK(32, 32, 2, 2, 3, 4), TILE_SK(32, 32, 2, 2, 3, 8),
    SKINNY_SK(1, 3, 4, 4), SKINNY_SK(1, 3, 8, 2), SKINNY_SK(2, 3, 8, 2), SKINNY_SK(4, 3, 4, 4),
    SKINNY_SK(2, 5, 4, 2), SKINNY_SK(4, 5, 4, 2), SKINNY_SK(1, 5, 2, 4), SKINNY_SK(2, 4, 8, 2),
    RSKINNY(2, 3, 16, 1), RSKINNY(2, 6, 8, 1), RSKINNY(4, 5, 8, 1), RSKINNY(3, 5, 8, 1), RSKINNY(1, 5, 8, 2),
    RSKINNY(1, 3, 16, 2), RSKINNY(2, 5, 8, 1), RSKINNY(4, 3, 8, 1),
    SKTILE(256, 256, 2, 4, 2, 8), SKTILE(256, 128, 2, 4, 3, 8), SKTILE(128, 256, 2, 4, 3, 8),
    SKTILE(128, 128, 2, 2, 2, 8),
    // 128 x 128 tiles with 8 waves (two per SIMD), for shapes with few tiles
    PTILE(128, 128, 2, 4, 4, 8), PTILE(128, 128, 2, 4, 2, 16), PTILE(128, 128, 4, 2, 3, 8),
    // K split three ways: mid-M shapes whose tiles number about a third of the CUs
    // (5120 x 6144 at M = 256: 80 tiles of 128 x 128).  (Six- and sixteen-way splits were
    // tuned too and won no key.)
    TILE_SK(128, 128, 2, 2, 4, 3), TILE_SK(128, 64, 2, 2, 3, 3), TILE_SK(64, 128, 2, 2, 3, 3),
    TILE_SK(64, 64, 2, 2, 3, 3), TILE_SK(128, 256, 2, 4, 3, 3),
    // A two-stage 128 x 128 instance split three ways: 66 KB of LDS, two workgroups per
    // CU (5120 x 6144 at M = 453..512: 3-4% faster; two- and six-way splits won no key).
    TILE_SK(128, 128, 2, 2, 2, 3),
};
constexpr int kNumEntries = sizeof(kEntries) / sizeof(kEntries[0]);

}  // namespace

int num_variants() { return kNumEntries; }

const Variant &variant(int id) { return kEntries[id].v; }

int64_t rskinny_grid(int id, int64_t N, int cus, bool packed)
{
    const Variant &v = kEntries[id].v;
    const int64_t units = packed ? (N + 15) / 16 : (N + 3) / 4;
    const int64_t slots = (int64_t)(cus > 0 ? cus : 256) * v.per_cu;
    return units < slots ? units : slots;
}

bool rskinny_rows_fit(int id, int64_t N, int cus)
{
    const Variant &v = kEntries[id].v;
    for (int packed = 0; packed < 2; ++packed) {
        const int64_t rg = packed ? 16 : 4, units = (N + rg - 1) / rg, G = rskinny_grid(id, N, cus, packed != 0);
        if (rg * ((units + G - 1) / G) > v.bn)
            return false;
    }
    return true;
}

int64_t variant_grid(int id, int64_t M, int64_t N, int64_t K, int cus)
{
    (void)K;
    const Variant &v = kEntries[id].v;
    if (v.kernel == A8W8_KERNEL_SKINNY)
        return (N + v.bn - 1) / v.bn * v.splits;
    if (v.kernel == A8W8_KERNEL_RSKINNY)
        return rskinny_grid(id, N, cus, false);
    if (v.kernel == A8W8_KERNEL_TALL)
        return (M + v.bm - 1) / v.bm;
    if (v.kernel == A8W8_KERNEL_PSKINNY) {
        // As few workgroups as still give each the fewest tiles the slots
        // allow, so that all but the last few take exactly that many.
        const int64_t tiles16 = (N + 15) / 16, slots = (int64_t)(cus > 0 ? cus : 1) * v.per_cu;
        const int64_t each = (tiles16 + slots - 1) / slots;
        return (tiles16 + each - 1) / each;
    }
    const int64_t tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
    if (v.kernel == A8W8_KERNEL_TILE)
        return tiles * v.splits;
    const int64_t slots = (int64_t)(cus > 0 ? cus : 1) * v.per_cu;
    if (v.kernel == A8W8_KERNEL_SKTILE) {
        // At most half as many tiles as slots: S = slots / tiles aligned pieces per
        // tile (at most one per K block), one workgroup each.  Otherwise every
        // slot, unless the whole problem has fewer K blocks than slots.
        const int64_t KB = K / 128;
        if (2 * tiles <= slots) {
            const int64_t S = slots / tiles < KB ? slots / tiles : KB;
            if (S >= 2)
                return S * tiles;
        }
        const int64_t steps = tiles * KB;
        return steps < slots ? steps : slots;
    }
    return tiles < slots ? tiles : slots;
}

// Stream-K tiles of a stream-K instance on `grid` workgroups (the kernel's own rule).
static int64_t sk_tiles_of(int64_t tiles, int64_t grid)
{
    const int64_t full = tiles / grid, rem = tiles % grid;
    if (rem == 0)
        return 0;
    return full >= 1 ? grid + rem : tiles;
}

int64_t variant_passes(int id, int64_t K)
{
    const Variant &v = kEntries[id].v;
    if (v.kernel == A8W8_KERNEL_PSKINNY)
        return 1;
    if (v.kernel != A8W8_KERNEL_SKINNY && v.kernel != A8W8_KERNEL_TALL && v.kernel != A8W8_KERNEL_RSKINNY)
        return (K / 128 + v.splits - 1) / v.splits;
    const int64_t per_pass = (int64_t)v.waves * v.kblocks, per_split = (K / 128 + v.splits - 1) / v.splits;
    return (per_split + per_pass - 1) / per_pass;
}

int64_t variant_workspace_bytes(int id, int64_t M, int64_t N, int64_t K, int cus)
{
    const Variant &v = kEntries[id].v;
    const int64_t tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
    if (v.kernel == A8W8_KERNEL_SKTILE) {
        // two partial slots per workgroup, when any tile is cut
        const int64_t grid = variant_grid(id, M, N, K, cus);
        return sk_tiles_of(tiles, grid) > 0 ? 2 * grid * v.bm * v.bn * 4 : 0;
    }
    if (v.splits <= 1)
        return 0;
    return tiles * v.splits * v.bm * v.bn * 4;
}

int64_t variant_counters(int id, int64_t M, int64_t N, int64_t K, int cus)
{
    const Variant &v = kEntries[id].v;
    const int64_t tiles = ((M + v.bm - 1) / v.bm) * ((N + v.bn - 1) / v.bn);
    if (v.kernel == A8W8_KERNEL_SKTILE)
        return sk_tiles_of(tiles, variant_grid(id, M, N, K, cus));
    if (v.splits <= 1)
        return 0;
    return tiles;
}

hipError_t set_kernel_attributes()
{
    for (int i = 0; i < kNumEntries; ++i) {
        if (kEntries[i].lds_bytes > 0) {
            for (const void *fn : kEntries[i].fn) {
                hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                                   kEntries[i].lds_bytes);
                if (e != hipSuccess)
                    return e;
            }
        }
    }
    return hipSuccess;
}

bool variant_fuses_quant(int id) { return id >= 0 && id < kNumEntries && kEntries[id].fq[0][0] != nullptr; }

hipError_t launch_quant_fused(int id, const Args &a, int cus, hipStream_t stream)
{
    if (!variant_fuses_quant(id) || a.sm != 0 || !rskinny_rows_fit(id, a.N, cus))
        return hipErrorInvalidConfiguration;
    const int mq = a.M <= 1 ? 0 : a.M <= 2 ? 1 : a.M <= 4 ? 2 : a.M <= 8 ? 3 : 4;
    const Entry &e = kEntries[id];
    const int64_t grid = rskinny_grid(id, a.N, cus, a.wpk != 0);
    int vec = ((reinterpret_cast<uintptr_t>(a.Y) & 7) == 0 && (a.N & 3) == 0) ? 1 : 0;
    Args args = a;
    void *params[] = {&args, &vec};
    return hipLaunchKernel(e.fq[mq][a.wpk ? 1 : 0], dim3((unsigned)grid, 1u), dim3(e.v.waves * 64), params, 0,
                           stream);
}

hipError_t launch_variant(int id, const Args &a, int batch, int cus, hipStream_t stream)
{
    const Entry &e = kEntries[id];
    // A split instance always runs with its own split count (the host gives it
    // the workspace that needs); the kernels read the count from a.splits.
    if (a.splits != e.v.splits)
        return hipErrorInvalidValue;
    int64_t grid = variant_grid(id, a.M, a.N, a.K, cus);
    // The kernels number workgroups and tiles in 32 bits (and the x dimension of a
    // grid is limited to 2^31 - 1): refuse, never truncate, a larger grid.
    if (grid < 1 || grid > 0x7fffffff)
        return hipErrorInvalidConfiguration;
    if (e.v.kernel == A8W8_KERNEL_RSKINNY) {
        // packed weights split rows in 16-row units (the layout's tiles)
        if (!rskinny_rows_fit(id, a.N, cus))
            return hipErrorInvalidConfiguration;
        grid = rskinny_grid(id, a.N, cus, a.wpk != 0);
    }
    // 8-byte stores need every row (and, batched, every batch) 8-byte aligned.
    int vec = ((reinterpret_cast<uintptr_t>(a.Y) & 7) == 0 && (a.N & 3) == 0) ? 1 : 0;
    Args args = a;
    void *params[] = {&args, &vec};
    return hipLaunchKernel(e.fn[2 * a.sm + (a.wpk ? 1 : 0)], dim3((unsigned)grid, (unsigned)batch),
                           dim3(e.v.waves * 64), params, (size_t)e.lds_bytes, stream);
}

}  // namespace a8w8
