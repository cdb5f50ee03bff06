/*
 * gemm_a8w8_blockscale.h -- C ABI of libgemm_a8w8.so, the a8w8 block-scale
 * GEMM for AMD Instinct MI355X (gfx950).
 *
 * The operation ("gemm_a8w8_blockscale", the op that the "[Perf] Retune gfx942
 * Qwen3.8-27B a8w8 blockscale decode rows for cold weights" page retunes in its
 * Kernel section, and that dense projections of a checkpoint quantised with
 * "weight_block_size: [128,128]" take, per "Why aiter#5069's measured -25%
 * kernel win moved serving throughput by 0.0%"):
 *
 *   Y[m,n] = bf16( sum over 128-wide K blocks kb of
 *                  (sum_{k in kb} e4m3(A[m,k]) * e4m3(W[n,k]))
 *                  * a_scale[m,kb] * w_scale[n/128,kb] )
 *
 * i.e. Y = A . W^T with fp8 e4m3 operands, fp32 scales per 1x128 activation
 * group and per 128x128 weight block, fp32 accumulation, and one
 * round-to-nearest-even to bf16 at the end.  The pages name the op but print no
 * formula; this scale granularity and the e4m3 variant (OCP "e4m3fn", largest
 * finite 448, no infinities) are this library's reading.
 *
 * Buffers (all device memory, row-major, owned by the caller; the library
 * never frees or keeps a pointer after the call returns):
 *   A        uint8 e4m3fn [M, K]                         16-byte aligned
 *   a_scale  float32      [M, K/128]                      4-byte aligned
 *   W        uint8 e4m3fn [N, K]                         16-byte aligned
 *   w_scale  float32      [ceil(N/128), K/128]            4-byte aligned
 *   Y        bf16 (uint16 bit patterns) [M, N]            2-byte aligned; overwritten
 * Y must not overlap any input.
 *
 * Threading / asynchrony: calls only enqueue one kernel on `stream` (a
 * hipStream_t of the current device; NULL = the null stream) and return.
 * Plans that split K over several workgroups per output tile (shapes with
 * few tiles; plan.splits > 1) use a workspace the library keeps per (device,
 * stream) for the life of the process: the first such call on a stream
 * allocates it (32 to 128 MB, plus a zero fill of its counters on that
 * stream), a later one that needs more allocates a larger one (the old one
 * stays allocated, for graphs captured with it); none is allocated while
 * the stream is capturing a graph -- a split plan without a large enough
 * workspace then runs unsplit.  A captured graph uses the workspace of the
 * stream it was captured on: do not run it concurrently with other work
 * captured or enqueued on that stream.  Otherwise calls never synchronise
 * the host, allocate device memory or issue memsets, so they may be captured
 * into a HIP graph (run one call eagerly on the stream first to keep the
 * split plan).  Each output
 * element is reduced in a fixed order (split partials in split order), so
 * results are bitwise reproducible.  The first call on a device reads its
 * properties (architecture, compute units) once.  Calls are re-entrant; the
 * selector table is immutable.
 */
#ifndef GEMM_A8W8_BLOCKSCALE_H
#define GEMM_A8W8_BLOCKSCALE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  Nothing is thrown across this ABI. */
enum {
    A8W8_OK = 0,
    A8W8_ERR_NULL = 1,    /* a required pointer is NULL                          */
    A8W8_ERR_SHAPE = 2,   /* M < 0, N < 1, K < 1, K % 128 != 0, M or N > 2^30, K > 2^22, batch out of [0, 65535] */
    A8W8_ERR_ALIGN = 3,   /* A or W not 16-byte aligned, a scale or Y not 4-byte aligned */
    A8W8_ERR_ARCH = 4,    /* the current device is not gfx950                    */
    A8W8_ERR_HIP = 5,     /* a HIP runtime call or kernel launch failed          */
    A8W8_ERR_PLAN = 6     /* a plan passed to gemm_a8w8_blockscale_run_plan is invalid for the shape */
};

/* Kernels behind the selector. */
enum {
    A8W8_KERNEL_SKINNY = 1,  /* M <= 16: streams W once, K split over the waves of a workgroup */
    A8W8_KERNEL_TILE = 2,    /* fp8-MFMA output tiles, one workgroup per tile, LDS ring       */
    A8W8_KERNEL_PTILE = 3,   /* fp8-MFMA output tiles, persistent workgroups, LDS ring        */
    A8W8_KERNEL_PSKINNY = 4, /* M <= 16, tall W: about one workgroup per CU walks 16-row tiles */
    A8W8_KERNEL_TALL = 5     /* N <= 32: streams A once, K split over the waves of a workgroup */
};

/*
 * A launch plan.  `variant` identifies a compiled kernel instance; the other
 * fields describe it (and the launch for the given shape) for logging and tests.
 */
typedef struct {
    int32_t kernel;     /* A8W8_KERNEL_*                                                  */
    int32_t variant;    /* index in [0, gemm_a8w8_num_variants())                         */
    int32_t bm, bn;     /* output tile of one workgroup: rows of Y (M) x columns (N)      */
    int32_t waves;      /* waves (64 lanes) per workgroup                                 */
    int32_t kblocks;    /* 128-wide K blocks one wave loads at once (skinny, pskinny, tall); LDS ring depth (tile) */
    int32_t kpasses;    /* passes over K per wave (skinny, tall), K/128 steps per tile (tile) */
    int32_t fallback;   /* 1: (N,K) has no tuned table, a heuristic plan was chosen       */
    int64_t grid;       /* workgroups launched for this shape (tile: persistent, at most  */
                        /* a few per CU, each looping over its share of the output tiles) */
    int64_t key_m;      /* selector table key this M maps to (M <= key_m <= 1.25 M), or M */
    int32_t splits;     /* tile, skinny: workgroups per output tile, each taking 1/splits of K (1: none) */
    int32_t reserved;
} a8w8_plan;

/*
 * Y = A . W^T with block scales (see top of file).  M == 0 is a no-op
 * returning A8W8_OK.  Errors are reported before anything is enqueued.
 */
int gemm_a8w8_blockscale(const void *A, const float *a_scale,
                         const void *W, const float *w_scale,
                         void *Y, int64_t M, int64_t N, int64_t K,
                         void *stream);

/*
 * The plan gemm_a8w8_blockscale would launch for (M, N, K) on a gfx950
 * device with `cu_count` compute units (0 = 256).  Host only; needs no GPU.
 */
int gemm_a8w8_blockscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count,
                              a8w8_plan *out);

/* Number of compiled kernel instances, and the description of one of them
   (grid, for a 256-CU device, and key_m are filled for (M, N, K); M may be 0
   for a bare description). */
int gemm_a8w8_num_variants(void);
int gemm_a8w8_describe_variant(int32_t variant, int64_t M, int64_t N, int64_t K,
                               a8w8_plan *out);

/*
 * Run a specific instance (for tuning).  Same contract as gemm_a8w8_blockscale;
 * returns A8W8_ERR_PLAN if the instance cannot handle the shape (the skinny
 * kernels need M <= 16, a pskinny instance also K/128 <= waves * kblocks; a
 * tall instance needs N <= its bn; a split instance needs K/128 >= 2 * splits
 * and at most 128 MB of fp32 partials).
 */
int gemm_a8w8_blockscale_run_variant(int32_t variant,
                                     const void *A, const float *a_scale,
                                     const void *W, const float *w_scale,
                                     void *Y, int64_t M, int64_t N, int64_t K,
                                     void *stream);

/*
 * Packed weights (optional offline layout; the pre-shuffled-weight idea of
 * the pages' "bpreshuffle" kernels, laid out for this library's MFMA):
 * W [N, K] row-major -> Wp of 16 * ceil(N/16) * K bytes.  For every 16-row
 * tile t and 128-wide K block kb, the 2048 bytes at (t * K/128 + kb) * 2048
 * hold, in order h = 0, 1 and lane l = 0..63, the 16 bytes of row 16 t + l%16
 * at columns 128 kb + 16 (l/16) + 64 h .. + 16; rows past N are zero.  Every
 * kernel then reads a weight fragment as two contiguous 1 KB loads.
 *
 * a8w8_prepack_weights enqueues the conversion (W and Wp device memory,
 * 16-byte aligned, not overlapping; K % 128 == 0).  gemm_a8w8_blockscale_packed
 * computes exactly what gemm_a8w8_blockscale computes from the same W (the
 * same kernels and instances, bitwise identical Y) reading Wp instead; N is
 * the real row count.  Same contract otherwise.
 */
int a8w8_prepack_weights(const void *W, void *Wp, int64_t N, int64_t K, void *stream);
int gemm_a8w8_blockscale_packed(const void *A, const float *a_scale,
                                const void *Wp, const float *w_scale,
                                void *Y, int64_t M, int64_t N, int64_t K,
                                void *stream);
int gemm_a8w8_blockscale_packed_run_variant(int32_t variant,
                                            const void *A, const float *a_scale,
                                            const void *Wp, const float *w_scale,
                                            void *Y, int64_t M, int64_t N, int64_t K,
                                            void *stream);

/*
 * MX-scaled variant: the mxfp8 GEMM with "32x32" weight-scale blocks (dense,
 * and batched with b = 8, N = 1024, K = 4096) that the gfx1250 BF16 and MX32
 * tuned-rows page (ROCm/aiter #7247, Motivation and Technical Details) tunes.
 * That page gives the block shape and the element type only; the scales are
 * read as OCP Microscaling (MX) scales, one E8M0 byte each (value
 * 2^(e - 127); 0xFF is NaN):
 *
 *   Y[m,n] = bf16( sum_k e4m3(A[m,k]) * 2^(a_scale[m, k/32] - 127)
 *                        * e4m3(W[n,k]) * 2^(w_scale[n/32, k/32] - 127) )
 *
 * fp32 accumulation (the scaled MFMA applies the powers of two exactly),
 * one round-to-nearest-even to bf16.  Same kernels, threading and error
 * rules as gemm_a8w8_blockscale; the exact-M selector has its own tables for
 * this variant (the page's shapes), other (N, K) get the heuristic plan
 * (fallback = 1).  K % 128 == 0 (whole 128-wide K blocks), and
 * ceil(N/32) * K/128 * 4 < 2^31.
 *
 * Buffers (device memory, row-major, caller-owned):
 *   A        uint8 e4m3fn [batch, M, K]              16-byte aligned
 *   a_scale  uint8 E8M0   [batch, M, K/32]            4-byte aligned
 *   W        uint8 e4m3fn [batch, N, K]              16-byte aligned
 *            (packed entries: batch consecutive a8w8_prepack_weights images
 *            of 16 * ceil(N/16) * K bytes each)
 *   w_scale  uint8 E8M0   [batch, ceil(N/32), K/32]   4-byte aligned
 *   Y        bf16 [batch, M, N]                       2-byte aligned; overwritten
 * The unbatched entries take batch = 1.  batch == 0 or M == 0 is a no-op;
 * batch <= 65535.  Batches are independent problems of one shape.
 */
int gemm_a8w8_mxscale(const void *A, const void *a_scale,
                      const void *W, const void *w_scale,
                      void *Y, int64_t M, int64_t N, int64_t K, void *stream);
int gemm_a8w8_mxscale_packed(const void *A, const void *a_scale,
                             const void *Wp, const void *w_scale,
                             void *Y, int64_t M, int64_t N, int64_t K, void *stream);
int batched_gemm_a8w8_mxscale(const void *A, const void *a_scale,
                              const void *W, const void *w_scale, void *Y,
                              int64_t batch, int64_t M, int64_t N, int64_t K, void *stream);
int batched_gemm_a8w8_mxscale_packed(const void *A, const void *a_scale,
                                     const void *Wp, const void *w_scale, void *Y,
                                     int64_t batch, int64_t M, int64_t N, int64_t K,
                                     void *stream);
/* The plan the MX entries launch for (M, N, K) (per batch; host only). */
int gemm_a8w8_mxscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out);
/* Run a specific instance on MX operands (for tuning and tests); w_packed
   selects the packed weight layout.  Returns A8W8_ERR_PLAN as
   gemm_a8w8_blockscale_run_variant does. */
int gemm_a8w8_mxscale_run_variant(int32_t variant, const void *A, const void *a_scale,
                                  const void *W, const void *w_scale, void *Y,
                                  int64_t batch, int64_t M, int64_t N, int64_t K,
                                  int32_t w_packed, void *stream);

/*
 * Row-wise ("per-token") variant: one fp32 scale per activation row (token)
 * and one per weight row (output channel) -- the non-block-scale a8w8 path
 * that the "Why aiter#5069's measured -25% kernel win moved serving
 * throughput by 0.0%" page describes as fed by a per-token fp8 setting
 * (its unreachable-half paragraph).  The pages give no formula; the reading
 * here is the plain row-wise scaled product
 *
 *   Y[m,n] = bf16( (sum_k e4m3(A[m,k]) * e4m3(W[n,k])) * a_scale[m] * w_scale[n] )
 *
 * with the dot accumulated in fp32 over all of K and the two scales applied
 * once, in that order, before the round to nearest even.  Buffers as for
 * gemm_a8w8_blockscale except a_scale float32 [M] and w_scale float32 [N]
 * (4-byte aligned).  The _packed form reads a8w8_prepack_weights output.  Same
 * kernels and selection tables as the block-scale entries, same threading and
 * error rules; bitwise reproducible.
 */
int gemm_a8w8_rowwise(const void *A, const float *a_scale,
                      const void *W, const float *w_scale,
                      void *Y, int64_t M, int64_t N, int64_t K, void *stream);
int gemm_a8w8_rowwise_packed(const void *A, const float *a_scale,
                             const void *Wp, const float *w_scale,
                             void *Y, int64_t M, int64_t N, int64_t K, void *stream);
/* Run a specific instance on row-wise operands (tuning and tests); w_packed
   selects the packed weight layout. */
int gemm_a8w8_rowwise_run_variant(int32_t variant, const void *A, const float *a_scale,
                                  const void *W, const float *w_scale, void *Y,
                                  int64_t M, int64_t N, int64_t K, int32_t w_packed,
                                  void *stream);

/* Static name of a compiled instance, e.g. "tile_256x128" (NULL if out of range). */
const char *gemm_a8w8_variant_name(int32_t variant);

/* Static, human-readable text for a status code. */
const char *gemm_a8w8_status_string(int status);

/* Hash of the compiled selector table (identifies the tuning that is deployed). */
uint64_t gemm_a8w8_table_hash(void);

/*
 * Per-1x128 activation quantisation: the step upstream of the GEMM, which
 * produces its A and a_scale operands from bf16 activations.  For each row m
 * and 128-wide group g along K:
 *
 *   a_scale[m,g] = fp32(amax over the group of |X| / 448)
 *   A[m,k]       = e4m3fn code nearest to clamp(fp32(X[m,k] / a_scale[m,g]), -448, 448)
 *
 * (IEEE fp32 division; ties to the even code; the sign bit follows the fp32
 * quotient).  A group whose amax is 0 gets a_scale 0 and zero codes.  The
 * pages describe the activation operand only as FP8 with per-group scales;
 * this is the library's reading, the one its GEMM inputs are generated with.
 *
 * Buffers (device memory, row-major, owned by the caller):
 *   X        bf16 (uint16 bit patterns) [M, K]   16-byte aligned, finite values
 *                                                (non-finite inputs give unspecified
 *                                                codes and scales in their group)
 *   A        uint8 e4m3fn [M, K]                 8-byte aligned; overwritten
 *   a_scale  float32 [M, K/128]                  4-byte aligned; overwritten
 * Outputs must not overlap X.  K % 128 == 0, K <= 2^22, M <= 2^30; M == 0 is a
 * no-op.  Same asynchrony and error rules as gemm_a8w8_blockscale: one kernel
 * enqueued on `stream`, no allocation, no memset, no host synchronisation;
 * errors are returned before anything is enqueued.
 */
int a8w8_quantize_1x128(const void *X, void *A, float *a_scale, int64_t M, int64_t K, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_A8W8_BLOCKSCALE_H */
