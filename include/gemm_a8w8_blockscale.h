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
 * Threading / asynchrony: every call only enqueues work on `stream` (a
 * hipStream_t of the current device; NULL = the null stream) and returns.  No
 * call allocates device memory, issues a memset or synchronises the host, and
 * the library keeps no per-stream state, so every call may be captured into a
 * HIP graph and replays it exactly (the pages' split-K check replays a
 * captured call against eager, "[Perf] Retune gfx942 Qwen3.8-27B a8w8
 * blockscale decode rows for cold weights", Kernel section).  The first call
 * on a device reads its properties (architecture, compute units) once.  Calls
 * are re-entrant; the selector table is immutable.  Each output element is
 * reduced in a fixed order, so results are bitwise reproducible.
 *
 * Split K across workgroups.  For shapes with few output tiles the fastest
 * plan can split K over several workgroups per tile (split-K), or cut the
 * last waves of tiles into equal runs of K blocks, one per workgroup
 * (stream-K); the pieces of a tile meet in a workspace: device memory the
 * CALLER owns and passes through gemm_a8w8_ex (see a8w8_gemm_desc).  The plain entries (gemm_a8w8_blockscale and the
 * other fixed-signature ones) bring no workspace: they always run the fastest
 * plan that splits no K across workgroups (gemm_a8w8_blockscale_plan reports
 * it), which needs nothing beyond the operands.
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
    A8W8_ERR_ALIGN = 3,   /* A or W not 16-byte aligned, a scale not 4, Y not 2, a workspace not 256 */
    A8W8_ERR_ARCH = 4,    /* the current device is not gfx950                    */
    A8W8_ERR_HIP = 5,     /* a HIP runtime call or kernel launch failed          */
    A8W8_ERR_PLAN = 6,    /* a forced kernel instance cannot serve the shape         */
    A8W8_ERR_WORKSPACE = 7 /* a forced split-K instance lacks workspace, or a workspace  */
                          /* argument is inconsistent (NULL with a size, size < 0)      */
};

/* Scale kinds of gemm_a8w8_ex (a8w8_gemm_desc.scale_kind). */
enum {
    A8W8_SCALE_BLOCK = 0,   /* fp32 per 1x128 activation group and 128x128 weight block */
    A8W8_SCALE_MX = 1,      /* E8M0 per 1x32 activation group and 32x32 weight block    */
    A8W8_SCALE_ROWWISE = 2  /* fp32 per activation row and per weight row               */
};

/* Kernels behind the selector. */
enum {
    A8W8_KERNEL_SKINNY = 1,  /* M <= 16: streams W once, K split over the waves of a workgroup */
    A8W8_KERNEL_TILE = 2,    /* fp8-MFMA output tiles, one workgroup per tile, LDS ring       */
    A8W8_KERNEL_PTILE = 3,   /* fp8-MFMA output tiles, persistent workgroups, LDS ring        */
    A8W8_KERNEL_PSKINNY = 4, /* M <= 16, tall W: about one workgroup per CU walks 16-row tiles */
    A8W8_KERNEL_TALL = 5,    /* N <= 32: streams A once, K split over the waves of a workgroup */
    A8W8_KERNEL_RSKINNY = 6, /* M <= 16: about one workgroup per CU, each an equal run of W rows  */
    A8W8_KERNEL_SKTILE = 7   /* persistent tiles, last waves cut into equal K runs (stream-K)     */
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
    int32_t splits;     /* tile, skinny: workgroups per output tile, each taking 1/splits of K (1: none; stream-K: 1) */
    int32_t reserved;
    int64_t workspace;  /* bytes of split-K / stream-K workspace this launch uses (0: none);
                           stream-K: depends on cu_count (two partial tiles per workgroup) */
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
 * The plan gemm_a8w8_blockscale launches for (M, N, K) on a gfx950 device with
 * `cu_count` compute units (0 = 256): exactly the instance, tile, grid and
 * table key of that call (never a split-K plan, workspace = 0).  Host only;
 * needs no GPU.  The pages decide from lookup logs which tuned row each
 * served shape hit ("Why aiter#5069's measured -25% kernel win moved serving
 * throughput by 0.0%", its census-tool section); this query is the library's
 * way of giving that answer without running the kernel (a project reading:
 * the pages print no such call).
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
 * and at most 128 MB of fp32 partials) and A8W8_ERR_WORKSPACE for a split
 * instance (these entries bring no workspace: run those through gemm_a8w8_ex).
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
 * computes what gemm_a8w8_blockscale computes from the same W, reading Wp
 * instead; N is the real row count.  Every instance gives bitwise the same Y
 * on Wp as on W (_run_variant); the packed entry's plan comes from its own
 * decode table where one is tuned (M <= 16 on the tuned decode shapes: the
 * contiguous loads favour other instances there) and from the block-scale
 * table otherwise (gemm_a8w8_ex_plan with w_packed = 1 reports it).  Same
 * contract otherwise.
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
 * kernels as the block-scale entries; plans from the row-wise decode tables
 * (M <= 16 on the tuned decode shapes, either weight layout) and the
 * block-scale tables otherwise; same threading and error rules; bitwise
 * reproducible.
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

/* Static, human-readable text for a status code (a project reading: the pages
   say only that a lookup miss should fall back rather than fail, "Rounds
   40-41: the CK int8 GEMM ...", Gate 1; errors the call cannot recover from
   are returned as these codes, never thrown or printed). */
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

/*
 * Quantise-and-multiply in one kernel, for decode (M <= 16): X bf16 [M, K] is
 * quantised per 1x128 group inside the GEMM kernel exactly as
 * a8w8_quantize_1x128 does it, then multiplied by the block-scaled W:
 *
 *   Y = gemm_a8w8_blockscale(quantize_1x128(X), W, w_scale)
 *
 * bitwise equal to those two calls in sequence when the GEMM runs the
 * instance this entry's plan reports (gemm_a8w8_blockscale_run_variant with
 * plan.variant).  The activation quantisation otherwise runs as a kernel of
 * its own before every decode GEMM (the "CK int8 GEMM ... gfx90a" page's
 * decode kernel table, section 3, lists the quantising kernel beside the
 * GEMM); fusing it saves that launch and the codes' round trip through memory.
 * The kernels are the row-range skinny ones (A8W8_KERNEL_RSKINNY); each
 * wave quantises the blocks it multiplies, its lanes spread over the M rows.
 *
 * Buffers (device memory, row-major, caller-owned):
 *   X        bf16 (uint16 bit patterns) [M, K]   16-byte aligned, finite values
 *   W        uint8 e4m3fn [N, K]                 16-byte aligned (w_packed = 1:
 *                                                a8w8_prepack_weights layout)
 *   w_scale  float32 [ceil(N/128), K/128]        4-byte aligned
 *   Y        bf16 [M, N]                         2-byte aligned; overwritten
 *   variant  -1: the plan below; else a row-range skinny instance (tuning, tests)
 * Plan (variant = -1; no tuned table): of the row-range skinny instances that
 * take (M, N, K), the one with the fewest passes over K, then the most waves,
 * then the most 16-row tiles per workgroup.  0 <= M <= 16 (A8W8_ERR_SHAPE
 * otherwise; M == 0 is a no-op); A8W8_ERR_PLAN when no row-range skinny
 * instance takes (N, K) (they cover N up to 64 rows per CU, e.g. not
 * N = 34816 on 256 CUs) or a forced instance is not one.  Same threading and
 * error rules as gemm_a8w8_blockscale: one kernel enqueued, no allocation, no
 * memset.  Every workgroup quantises all of X, so that work grows with M:
 * measured on MI355X against the two calls (both in HIP graphs, cold weights),
 * the fused call takes 18-23% less time at M = 1..4 on a 5120 x 6144 weight
 * and 3-5% less on 14336 x 5120 (M = 1..8), but up to 19% more at M = 16;
 * above M = 8, quantise-then-GEMM is generally the faster path.
 */
int gemm_a8w8_blockscale_fused_quant(const void *X, const void *W, const float *w_scale, void *Y,
                                     int64_t M, int64_t N, int64_t K, int32_t w_packed, int32_t variant,
                                     void *stream);
/* The plan gemm_a8w8_blockscale_fused_quant launches (host only; cu_count 0 = 256). */
int gemm_a8w8_blockscale_fused_quant_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, int32_t variant,
                                          a8w8_plan *out);

/*
 * One call of any scale kind and weight layout, with an optional caller-owned
 * split-K workspace and an optional forced instance.  The plain entries above
 * are this call with workspace = NULL, workspace_bytes = 0, variant = -1.
 *
 *   A, a_scale, W, w_scale, Y  as for the entry of that scale kind (device
 *                              memory, row-major; W packed when w_packed = 1)
 *   batch        >= 0 consecutive problems of one shape (every operand has a
 *                leading batch dimension; 1 for plain 2-D operands)
 *   scale_kind   A8W8_SCALE_BLOCK, A8W8_SCALE_MX or A8W8_SCALE_ROWWISE
 *   variant      -1: the selector's plan; else a compiled instance (tuning, tests)
 *   workspace    NULL, or a split-K / stream-K workspace: caller-owned device memory,
 *                256-byte aligned, of workspace_bytes bytes, zero-filled once
 *                by gemm_a8w8_workspace_init before its first use.  Its first
 *                A8W8_WORKSPACE_COUNTER_BYTES hold the per-tile counters of a
 *                split or stream-K call (the same area for every call), the
 *                rest the fp32 partial tiles.  Every call leaves the counters zero
 *                again, so one workspace serves any number of calls, of any
 *                shapes, IN STREAM ORDER; calls (or graph replays) that may
 *                overlap in time need workspaces of their own.  The library
 *                keeps no pointer to it.
 *
 * Plan rule (variant = -1): the table row's fastest instance if its
 * workspace (gemm_a8w8_ex_plan with workspace_bytes large: plan.workspace)
 * fits in workspace_bytes, else the row's fastest instance that cuts no K
 * across workgroups.  A forced split or stream-K instance without enough
 * workspace for this device returns A8W8_ERR_WORKSPACE before anything is
 * enqueued.
 */
#define A8W8_WORKSPACE_COUNTER_BYTES 65536

typedef struct {
    const void *A;
    const void *a_scale;
    const void *W;
    const void *w_scale;
    void *Y;
    int64_t batch;
    int64_t M, N, K;
    int32_t scale_kind;
    int32_t w_packed;
    int32_t variant;
    int32_t reserved;
    void *workspace;
    int64_t workspace_bytes;
} a8w8_gemm_desc;

int gemm_a8w8_ex(const a8w8_gemm_desc *desc, void *stream);
/* The plan gemm_a8w8_ex launches for `desc` (host only; pointers are not
   read, workspace_bytes is): plan.workspace is the workspace it uses. */
int gemm_a8w8_ex_plan(const a8w8_gemm_desc *desc, int32_t cu_count, a8w8_plan *out);
/* Enqueue the zero fill of a split-K workspace (one kernel of the library on
   `stream`, no memset, so it may be captured too). */
int gemm_a8w8_workspace_init(void *workspace, int64_t bytes, void *stream);

/*
 * Allocation-free entry: for callers that cannot allocate device memory
 * (code under HIP-graph capture, tight serving loops, harnesses that forbid
 * hipMalloc) yet want the split-K plans, which need a workspace.  Same
 * arguments and result as gemm_a8w8_blockscale, but it runs the plan
 * gemm_a8w8_ex runs with a workspace of A8W8_NOALLOC_SCRATCH_BYTES -- the
 * table row's fastest plan when its split-K / stream-K workspace fits that
 * size, else the row's fastest plan that cuts no K (gemm_a8w8_ex_plan with
 * that workspace_bytes reports it) -- and takes the workspace from a static
 * device array of that size per GPU, which the library holds until the
 * process ends.  It allocates nothing, issues
 * no memset and does not synchronise.  Every call on a GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, concurrent
 * graph replays) race and give wrong results; calls in stream order are safe.
 */
#define A8W8_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
int gemm_a8w8_blockscale_noalloc(const void *A, const float *a_scale,
                                 const void *W, const float *w_scale,
                                 void *Y, int64_t M, int64_t N, int64_t K,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_A8W8_BLOCKSCALE_H */
