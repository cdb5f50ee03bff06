// a8w8_internal.h -- declarations shared by the host API and the kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace a8w8 {

// One compiled kernel instance.
struct Variant {
    int32_t kernel;    // A8W8_KERNEL_*
    int32_t bm, bn;    // output tile per workgroup (skinny: 16 x 16 * tiles per wave)
    int32_t waves;     // waves per workgroup
    int32_t kblocks;   // K blocks each wave loads (skinny, pskinny), LDS ring depth (tile)
    int32_t max_m;     // largest M the instance accepts (skinny, pskinny: 16), 0 = any
    int32_t per_cu;    // ptile, pskinny, rskinny: workgroups per CU the grid is sized for
    int32_t splits;    // tile: workgroups per output tile, each taking 1/splits of K (1: no split;
                       // stream-K instances cut tiles by their own rule and keep 1 here)
    const char *name;
};


struct Args {
    const uint8_t *A;
    const float *a_scale;
    const uint8_t *W;
    const float *w_scale;
    uint16_t *Y;
    int32_t M, N, K;
    int32_t wpk;       // 1: W is in the packed (fragment-order) layout, see packed_block
    int32_t sm;        // scale kind: 0 fp32 per 1 x 128 / 128 x 128 blocks; 1 MX (E8M0 bytes per
                       // 1 x 32 / 32 x 32); 2 row-wise (fp32 per activation row, per weight row)
    // Batched calls: gridDim.y batches; batch z reads A + z * bs_a, a_scale + z * bs_as,
    // W + z * bs_w, w_scale + z * bs_ws and writes Y + z * bs_y (elements of each array).
    int64_t bs_a, bs_as, bs_w, bs_ws, bs_y;
    // Split K (split instances): splits per tile; the call's workspace for the
    // fp32 partial tiles [batch][tile][split][BM * BN] and one zeroed counter per
    // [batch][tile] (the last split of a tile resets it).  Stream-K instances:
    // partials [batch][2 * grid][BM * BN], counters [batch][stream-K tile].
    int32_t splits;
    float *ws;
    int32_t *cnt;
};

int num_variants();
const Variant &variant(int id);
// Workspace a split-K or stream-K instance needs per batch on a device with
// `cus` compute units: fp32 partial bytes and counters (0 and 0: none).
int64_t variant_workspace_bytes(int id, int64_t M, int64_t N, int64_t K, int cus);
int64_t variant_counters(int id, int64_t M, int64_t N, int64_t K, int cus);
// Workgroups the instance launches for (M, N, K) on a device with `cus`
// compute units (ptile, pskinny: min(tiles, cus * per_cu), each workgroup
// looping over its share of the tiles), and the passes over K one wave makes
// (skinny: ceil(K/128 / (waves * kblocks)); pskinny: 1; tile: K/128 blocks per tile).
int64_t variant_grid(int id, int64_t M, int64_t N, int64_t K, int cus);
int64_t variant_passes(int id, int64_t K);
// Row-range skinny instances: their grid (row-major or packed weights) and whether
// every workgroup's run of rows fits the instance's tiles on a device with `cus` CUs.
int64_t rskinny_grid(int id, int64_t N, int cus, bool packed);
bool rskinny_rows_fit(int id, int64_t N, int cus);
// Row-range skinny instances also come with fused-quantisation kernels: A is
// then bf16 [M, K] (a.A; a.a_scale unused) quantised per 1 x 128 group inside
// the kernel, block scales only (a.sm == 0), one problem.
bool variant_fuses_quant(int id);
hipError_t launch_quant_fused(int id, const Args &a, int cus, hipStream_t stream);
// Raise the dynamic-LDS limit of the instances that need more than 64 KB
// (once per device, with that device current).
hipError_t set_kernel_attributes();
// Enqueue the instance for `batch` batches (grid y); returns hipSuccess or the launch error.
hipError_t launch_variant(int id, const Args &a, int batch, int cus, hipStream_t stream);
// Enqueue the conversion of row-major W [N, K] to the packed layout.
hipError_t launch_prepack(const void *W, void *Wp, int64_t N, int64_t K, int cus, hipStream_t stream);
// Enqueue the per-1x128 activation quantisation of `groups` groups.
hipError_t launch_quant_1x128(const void *X, void *A, float *a_scale, int64_t groups, int cus, hipStream_t stream);

}  // namespace a8w8
