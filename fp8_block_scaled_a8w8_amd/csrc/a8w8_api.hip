// a8w8_api.hip -- C ABI of libgemm_a8w8.so: argument checks, the exact-M
// selector, per-device set-up and the launch on the caller's stream.
//
// Selection.  For each registered (N, K) the tuned table holds ascending keys
// key_m[0] < key_m[1] < ... and the instance picked for each key.  A request
// M is served by the instance of the smallest key >= M.  The generator that
// writes the table keeps consecutive keys close enough that the key is never
// above 1.25 M (and equals M for M <= 16), so no M runs an instance that was
// tuned for a much larger problem -- unlike a lookup that pads M to the next
// power of two and makes M = 6016 use the row tuned for 8192, the failure the
// "Why aiter#5069's measured -25% kernel win moved serving throughput by 0.0%"
// page describes (its "Two amplifiers" section).  An (N, K) with no table gets
// a heuristic plan of the same kernels and is flagged, never refused: a lookup
// gap falls back to a default kernel, as the "CK int8 GEMM ... gfx90a" page
// recommends after its build-time lookup raised instead (its Gate 1).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <tuple>
#include <utility>

#include "a8w8_internal.h"
#include "a8w8_selector_table.h"
#include "gemm_a8w8_blockscale.h"

using a8w8::Args;
using a8w8::Variant;

namespace {

constexpr int kMaxDevices = 64;
constexpr int64_t kMaxDim = (int64_t)1 << 30;
// The tile kernel addresses a tile's rows with 32-bit offsets: 256 * K < 2^31.
constexpr int64_t kMaxK = (int64_t)1 << 22;
// Batches are the grid's y dimension.
constexpr int64_t kMaxBatch = 65535;
// Largest split-K workspace (fp32 partial tiles) one stream may hold.
constexpr int64_t kMaxWorkspace = (int64_t)128 << 20;

// Per-device state: 0 = not yet checked, 1 = gfx950 ready, 2 = unsupported.
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];
std::mutex g_init_mutex;

int device_ready(int *cus)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return A8W8_ERR_HIP;
    int st = g_dev_state[dev].load(std::memory_order_acquire);
    if (st == 0) {
        std::lock_guard<std::mutex> lock(g_init_mutex);
        st = g_dev_state[dev].load(std::memory_order_acquire);
        if (st == 0) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
                return A8W8_ERR_HIP;
            if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
                st = 2;
            } else {
                if (a8w8::set_kernel_attributes() != hipSuccess)
                    return A8W8_ERR_HIP;
                g_dev_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
                st = 1;
            }
            g_dev_state[dev].store(st, std::memory_order_release);
        }
    }
    if (st != 1)
        return A8W8_ERR_ARCH;
    *cus = g_dev_cus[dev].load(std::memory_order_relaxed);
    return A8W8_OK;
}

int check_shape(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 1 || K < 1 || (K % 128) != 0)
        return A8W8_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxK)
        return A8W8_ERR_SHAPE;
    // Row offsets into the scale arrays are 32-bit inside the kernels.
    if (M * (K / 128) >= ((int64_t)1 << 31) || ((N + 127) / 128) * (K / 128) >= ((int64_t)1 << 31))
        return A8W8_ERR_SHAPE;
    return A8W8_OK;
}

int check_pointers(const void *A, const void *a_scale, const void *W, const void *w_scale, const void *Y)
{
    if (!A || !a_scale || !W || !w_scale || !Y)
        return A8W8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(W) & 15))
        return A8W8_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(a_scale) & 3) || (reinterpret_cast<uintptr_t>(w_scale) & 3))
        return A8W8_ERR_ALIGN;
    if (reinterpret_cast<uintptr_t>(Y) & 1)
        return A8W8_ERR_ALIGN;
    return A8W8_OK;
}

// The skinny and tall kernels address A and W with 32-bit per-lane offsets
// (W rows counted padded to a multiple of 16, as the packed layout stores them).
bool skinny_fits(int64_t N, int64_t K)
{
    return ((N + 15) & ~(int64_t)15) * K < ((int64_t)1 << 32) && 16 * K < ((int64_t)1 << 32);
}

bool variant_accepts(int id, int64_t M, int64_t N, int64_t K)
{
    const Variant &v = a8w8::variant(id);
    // Split K: at least two K blocks per split, and a workspace within the cap.
    if (v.splits > 1 && (K / 128 < 2 * (int64_t)v.splits || a8w8::variant_workspace_bytes(id, M, N) > kMaxWorkspace))
        return false;
    if (v.kernel == A8W8_KERNEL_SKINNY)
        return M <= v.max_m && skinny_fits(N, K);
    if (v.kernel == A8W8_KERNEL_PSKINNY)
        return M <= v.max_m && skinny_fits(N, K) && K / 128 <= (int64_t)v.waves * v.kblocks;
    if (v.kernel == A8W8_KERNEL_TALL)
        return N <= v.bn && skinny_fits(N, K) && skinny_fits(M, K);
    return true;
}

int find_variant(int kernel, int bm, int bn, int waves, int kblocks, int splits = 1)
{
    for (int i = 0; i < a8w8::num_variants(); ++i) {
        const Variant &v = a8w8::variant(i);
        if (v.kernel == kernel && v.bm == bm && v.bn == bn && (waves == 0 || v.waves == waves) &&
            (kblocks == 0 || v.kblocks == kblocks) && v.splits == splits)
            return i;
    }
    return -1;
}

// Split-K workspace of one (device, stream): fp32 partial tiles and the
// per-tile counters, which start at zero and are reset by the last split of
// each tile.  One per stream, so calls on different streams never share one;
// calls on one stream run in order.
struct Workspace {
    float *buf = nullptr;
    int64_t bytes = 0;
    int32_t *cnt = nullptr;
    int64_t counters = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

// The calling stream's workspace with room for `bytes` and `counters`,
// allocated (or replaced by a larger one) here -- only while the stream is not
// capturing a graph.  A replaced workspace is retired, never freed: graphs
// captured earlier keep using it.  Returns false when no suitable workspace
// can be had; the caller then runs the unsplit instance.
bool stream_workspace(int dev, hipStream_t stream, int64_t bytes, int64_t counters, float **ws, int32_t **cnt)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace &w = g_ws[std::make_pair(dev, reinterpret_cast<uintptr_t>(stream))];
    if (w.bytes < bytes || w.counters < counters) {
        hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &st) != hipSuccess || st != hipStreamCaptureStatusNone)
            return false;
        const int64_t nb = std::max<int64_t>(std::max<int64_t>(bytes, 2 * w.bytes), (int64_t)32 << 20);
        const int64_t nc = std::max<int64_t>(std::max<int64_t>(counters, 2 * w.counters), (int64_t)1 << 15);
        void *b = nullptr, *c = nullptr;
        if (hipMalloc(&b, (size_t)std::min(nb, kMaxWorkspace)) != hipSuccess || hipMalloc(&c, (size_t)nc * 4) != hipSuccess ||
            hipMemsetAsync(c, 0, (size_t)nc * 4, stream) != hipSuccess) {
            (void)hipGetLastError();
            (void)hipFree(b);
            (void)hipFree(c);
            return false;
        }
        w.buf = static_cast<float *>(b);          // the previous buffers (if any) stay allocated
        w.bytes = std::min(nb, kMaxWorkspace);
        w.cnt = static_cast<int32_t *>(c);
        w.counters = nc;
    }
    *ws = w.buf;
    *cnt = w.cnt;
    return true;
}

// Plan for shapes with no tuned table.  Up to M = 16: the skinny instance
// with the widest row group that still yields at least ~200 workgroups (wider
// groups share each activation fragment across more weight tiles), covering
// K in the fewest passes with the most blocks per pass (8 waves x 6 blocks
// measured fastest at K = 2048..8192); with fewer than 32 row groups, K split
// four ways over 16-row groups (measured 1.3-1.6x faster at N = 32..256,
// slower from ~64 groups up).  Above, for N <= 32: the
// tall kernel (16-row activation groups, 16 waves; 32-row groups from
// M = 4096).  Otherwise the largest tile that still gives every compute unit
// at least two workgroups, else the smallest, with K split when even that
// leaves compute units idle.
int heuristic_variant(int64_t M, int64_t N, int64_t K, int cus)
{
    if (M <= 16 && skinny_fits(N, K)) {
        int best = -1;
        int64_t best_key = 0;
        for (int i = 0; i < a8w8::num_variants(); ++i) {
            const Variant &v = a8w8::variant(i);
            if (v.kernel != A8W8_KERNEL_SKINNY || v.splits > 1)
                continue;
            const int64_t groups = (N + v.bn - 1) / v.bn;
            const int64_t passes = std::min<int64_t>(a8w8::variant_passes(i, K), 99);
            // rank: enough workgroups, then fewer passes, then wider rows, then more blocks per pass
            const int64_t key = (groups >= 200 || v.bn == 16 ? 1 : 0) * 100000000 - passes * 1000000 +
                                v.bn * 1000 + v.waves * v.kblocks;
            if (best < 0 || key > best_key) {
                best = i;
                best_key = key;
            }
        }
        if (best >= 0 && (N + 15) / 16 < 32) {
            const int sid = find_variant(A8W8_KERNEL_SKINNY, 16, 16, 4, 3, 4);
            if (sid >= 0 && variant_accepts(sid, M, N, K))
                return sid;
        }
        if (best >= 0)
            return best;
    }
    if (N <= 32 && skinny_fits(N, K) && skinny_fits(M, K)) {
        const int bn = N <= 16 ? 16 : 32;
        const int id = M < 4096 ? find_variant(A8W8_KERNEL_TALL, 16, bn, bn == 32 ? 16 : 8, 3)
                                : find_variant(A8W8_KERNEL_TALL, 32, bn, 8, bn == 32 ? 6 : 3);
        if (id >= 0)
            return id;
    }
    static const int kTiles[][2] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}, {64, 64}, {32, 64}, {32, 32}};
    const int nt = (int)(sizeof(kTiles) / sizeof(kTiles[0]));
    for (int i = 0; i < nt; ++i) {
        const int bm = kTiles[i][0], bn = kTiles[i][1];
        if (N <= 32 && bn > 32)
            continue;
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        if (tiles >= 2 * (int64_t)cus)
            return find_variant(A8W8_KERNEL_TILE, bm, bn, 0, 0);
    }
    // Fewer tiles than two per CU even at 32 x 32: split K over S workgroups per tile,
    // the smallest S (2, 4, 8) that gives every CU a workgroup, keeping >= 4 K blocks
    // per split (the tuned tables pick split plans in this regime).
    const int base = find_variant(A8W8_KERNEL_TILE, 32, 32, 0, 0);
    const Variant &bv = a8w8::variant(base);
    const int64_t tiles = ((M + 31) / 32) * ((N + 31) / 32);
    int best = base;
    for (int s : {2, 4, 8}) {
        if (K / 128 < 4 * (int64_t)s)
            break;
        const int sid = find_variant(A8W8_KERNEL_TILE, 32, 32, bv.waves, bv.kblocks, s);
        if (sid < 0 || !variant_accepts(sid, M, N, K))
            continue;
        best = sid;
        if (tiles * s >= cus)
            break;
    }
    return best;
}

struct Choice {
    int variant;
    int64_t key_m;
    int fallback;
};

Choice select_variant(int64_t M, int64_t N, int64_t K, int cus, int mx)
{
    using namespace a8w8_table;
    for (int t = 0; t < kNumShapes; ++t) {
        const ShapeTable &s = kShapes[t];
        if (s.n != N || s.k != K || s.mx != mx)
            continue;
        // smallest key >= M (binary search over the ascending keys)
        int lo = 0, hi = s.count;
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (s.key_m[mid] < M)
                lo = mid + 1;
            else
                hi = mid;
        }
        if (lo < s.count) {
            const int v = find_variant(s.kernel[lo], s.bm[lo], s.bn[lo], s.waves[lo], s.kblocks[lo], s.splits[lo]);
            if (v >= 0 && variant_accepts(v, M, N, K))
                return {v, s.key_m[lo], 0};
        }
        break;
    }
    return {heuristic_variant(M, N, K, cus), M, 1};
}

void fill_plan(int id, int64_t M, int64_t N, int64_t K, int cus, int64_t key_m, int fallback, a8w8_plan *out)
{
    const Variant &v = a8w8::variant(id);
    std::memset(out, 0, sizeof(*out));
    out->kernel = v.kernel;
    out->variant = id;
    out->bm = v.bm;
    out->bn = v.bn;
    out->waves = v.waves;
    out->kblocks = v.kblocks;
    out->kpasses = (int32_t)a8w8::variant_passes(id, K);
    out->grid = M > 0 ? a8w8::variant_grid(id, M, N, K, cus) : 0;
    out->key_m = key_m;
    out->fallback = fallback;
    out->splits = v.splits;
}

// GEMM_A8W8_LOG=1: one stderr line per distinct (M, N, K) with the plan used.
void log_plan(int64_t M, int64_t N, int64_t K, int id, int64_t key_m, int fallback)
{
    static const bool enabled = [] {
        const char *e = std::getenv("GEMM_A8W8_LOG");
        return e && e[0] && std::strcmp(e, "0") != 0;
    }();
    if (!enabled)
        return;
    static std::mutex mu;
    static std::set<std::tuple<int64_t, int64_t, int64_t>> seen;
    std::lock_guard<std::mutex> lock(mu);
    if (!seen.insert(std::make_tuple(M, N, K)).second)
        return;
    std::fprintf(stderr, "gemm_a8w8: M=%lld N=%lld K=%lld -> %s key_m=%lld%s\n", (long long)M, (long long)N,
                 (long long)K, a8w8::variant(id).name, (long long)key_m, fallback ? " fallback" : "");
}

// Operand set of one call: `batch` consecutive problems of one shape.
struct Operands {
    const void *A;
    const void *a_scale;
    const void *W;
    const void *w_scale;
    void *Y;
    int64_t batch;
    int wpk;   // W in the packed layout
    int sm;    // scale kind: 0 fp32 block scales, 1 MX (E8M0), 2 row-wise fp32
};

// Elements of each array per batch (scale arrays in 32-bit words: an MX row of
// K/32 bytes is K/128 words, the same count as a row of fp32 block scales;
// row-wise scales are one word per row).
void batch_strides(const Operands &o, int64_t M, int64_t N, int64_t K, Args &a)
{
    const int64_t KB = K / 128;
    const int64_t w_rows = o.wpk ? (N + 15) / 16 * 16 : N;
    const int64_t s_rows = o.sm == 1 ? (N + 31) / 32 : (N + 127) / 128;
    a.bs_a = M * K;
    a.bs_as = o.sm == 2 ? M : M * KB;
    a.bs_w = w_rows * K;
    a.bs_ws = o.sm == 2 ? N : s_rows * KB;
    a.bs_y = M * N;
}

int launch(int id, const Operands &o, int64_t M, int64_t N, int64_t K, int cus, void *stream)
{
    Args a;
    a.splits = 1;
    a.ws = nullptr;
    a.cnt = nullptr;
    if (a8w8::variant(id).splits > 1) {
        int dev = 0;
        const int64_t bytes = o.batch * a8w8::variant_workspace_bytes(id, M, N);
        const int64_t counters = o.batch * a8w8::variant_counters(id, M, N);
        if (hipGetDevice(&dev) == hipSuccess && bytes <= kMaxWorkspace &&
            stream_workspace(dev, static_cast<hipStream_t>(stream), bytes, counters, &a.ws, &a.cnt))
            a.splits = a8w8::variant(id).splits;
        // else the instance runs unsplit: one workgroup per tile, no workspace.
    }
    a.A = static_cast<const uint8_t *>(o.A);
    a.a_scale = static_cast<const float *>(o.a_scale);
    a.W = static_cast<const uint8_t *>(o.W);
    a.w_scale = static_cast<const float *>(o.w_scale);
    a.Y = static_cast<uint16_t *>(o.Y);
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.wpk = o.wpk;
    a.sm = o.sm;
    batch_strides(o, M, N, K, a);
    if (a8w8::launch_variant(id, a, (int)o.batch, cus, static_cast<hipStream_t>(stream)) != hipSuccess)
        return A8W8_ERR_HIP;
    return A8W8_OK;
}

// Shape checks common to every call, plus the batched and MX limits.
int check_call(const Operands &o, int64_t M, int64_t N, int64_t K)
{
    int rc = check_shape(M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (o.batch < 0 || o.batch > kMaxBatch)
        return A8W8_ERR_SHAPE;
    // MX weight-scale rows (one per 32 weight rows): the pskinny kernel's
    // descriptor spans them in 32 bits, the kernels index them in 31.
    if (o.sm == 1 && (N + 31) / 32 * (K / 128) * 4 >= ((int64_t)1 << 31))
        return A8W8_ERR_SHAPE;
    return A8W8_OK;
}

int gemm_impl(const Operands &o, int64_t M, int64_t N, int64_t K, void *stream)
{
    int rc = check_call(o, M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (M == 0 || o.batch == 0)
        return A8W8_OK;
    rc = check_pointers(o.A, o.a_scale, o.W, o.w_scale, o.Y);
    if (rc != A8W8_OK)
        return rc;
    int cus = 0;
    rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    // Row-wise calls use the block-scale tables: same kernels and loads, less
    // scale work per block.
    const Choice c = select_variant(M, N, K, cus, o.sm == 1 ? 1 : 0);
    log_plan(M, N, K, c.variant, c.key_m, c.fallback);
    return launch(c.variant, o, M, N, K, cus, stream);
}

int run_variant_impl(int32_t variant, const Operands &o, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (variant < 0 || variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    int rc = check_call(o, M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (M == 0 || o.batch == 0)
        return A8W8_OK;
    if (!variant_accepts(variant, M, N, K))
        return A8W8_ERR_PLAN;
    rc = check_pointers(o.A, o.a_scale, o.W, o.w_scale, o.Y);
    if (rc != A8W8_OK)
        return rc;
    int cus = 0;
    rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    return launch(variant, o, M, N, K, cus, stream);
}

}  // namespace

extern "C" {

int gemm_a8w8_blockscale(const void *A, const float *a_scale, const void *W, const float *w_scale, void *Y,
                         int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, W, w_scale, Y, 1, 0, 0}, M, N, K, stream);
}

int gemm_a8w8_blockscale_packed(const void *A, const float *a_scale, const void *Wp, const float *w_scale, void *Y,
                                int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, Wp, w_scale, Y, 1, 1, 0}, M, N, K, stream);
}

int gemm_a8w8_mxscale(const void *A, const void *a_scale, const void *W, const void *w_scale, void *Y, int64_t M,
                      int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, W, w_scale, Y, 1, 0, 1}, M, N, K, stream);
}

int gemm_a8w8_mxscale_packed(const void *A, const void *a_scale, const void *Wp, const void *w_scale, void *Y,
                             int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, Wp, w_scale, Y, 1, 1, 1}, M, N, K, stream);
}

int batched_gemm_a8w8_mxscale(const void *A, const void *a_scale, const void *W, const void *w_scale, void *Y,
                              int64_t batch, int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, W, w_scale, Y, batch, 0, 1}, M, N, K, stream);
}

int batched_gemm_a8w8_mxscale_packed(const void *A, const void *a_scale, const void *Wp, const void *w_scale,
                                     void *Y, int64_t batch, int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, Wp, w_scale, Y, batch, 1, 1}, M, N, K, stream);
}

int gemm_a8w8_mxscale_run_variant(int32_t variant, const void *A, const void *a_scale, const void *W,
                                  const void *w_scale, void *Y, int64_t batch, int64_t M, int64_t N, int64_t K,
                                  int32_t w_packed, void *stream)
{
    return run_variant_impl(variant, {A, a_scale, W, w_scale, Y, batch, w_packed ? 1 : 0, 1}, M, N, K, stream);
}

int gemm_a8w8_rowwise(const void *A, const float *a_scale, const void *W, const float *w_scale, void *Y,
                      int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, W, w_scale, Y, 1, 0, 2}, M, N, K, stream);
}

int gemm_a8w8_rowwise_packed(const void *A, const float *a_scale, const void *Wp, const float *w_scale, void *Y,
                             int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl({A, a_scale, Wp, w_scale, Y, 1, 1, 2}, M, N, K, stream);
}

int gemm_a8w8_rowwise_run_variant(int32_t variant, const void *A, const float *a_scale, const void *W,
                                  const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K, int32_t w_packed,
                                  void *stream)
{
    return run_variant_impl(variant, {A, a_scale, W, w_scale, Y, 1, w_packed ? 1 : 0, 2}, M, N, K, stream);
}

int gemm_a8w8_mxscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out)
{
    if (!out)
        return A8W8_ERR_NULL;
    const int rc = check_call({nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1}, M, N, K);
    if (rc != A8W8_OK)
        return rc;
    const int cus = cu_count > 0 ? cu_count : 256;
    const Choice c = select_variant(M > 0 ? M : 1, N, K, cus, 1);
    fill_plan(c.variant, M, N, K, cus, c.key_m, c.fallback, out);
    return A8W8_OK;
}

int gemm_a8w8_blockscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out)
{
    if (!out)
        return A8W8_ERR_NULL;
    const int rc = check_shape(M, N, K);
    if (rc != A8W8_OK)
        return rc;
    const int cus = cu_count > 0 ? cu_count : 256;
    const Choice c = select_variant(M > 0 ? M : 1, N, K, cus, 0);
    fill_plan(c.variant, M, N, K, cus, c.key_m, c.fallback, out);
    return A8W8_OK;
}

int gemm_a8w8_num_variants(void) { return a8w8::num_variants(); }

int gemm_a8w8_describe_variant(int32_t variant, int64_t M, int64_t N, int64_t K, a8w8_plan *out)
{
    if (!out)
        return A8W8_ERR_NULL;
    if (variant < 0 || variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    if (M < 0 || N < 1 || K < 1)
        return A8W8_ERR_SHAPE;
    fill_plan(variant, M, N, K, 256, M, 0, out);
    return A8W8_OK;
}

int gemm_a8w8_blockscale_run_variant(int32_t variant, const void *A, const float *a_scale, const void *W,
                                     const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K,
                                     void *stream)
{
    return run_variant_impl(variant, {A, a_scale, W, w_scale, Y, 1, 0, 0}, M, N, K, stream);
}

int gemm_a8w8_blockscale_packed_run_variant(int32_t variant, const void *A, const float *a_scale, const void *Wp,
                                            const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K,
                                            void *stream)
{
    return run_variant_impl(variant, {A, a_scale, Wp, w_scale, Y, 1, 1, 0}, M, N, K, stream);
}

int a8w8_prepack_weights(const void *W, void *Wp, int64_t N, int64_t K, void *stream)
{
    if (N < 1 || K < 1 || (K % 128) != 0 || N > kMaxDim || K > kMaxK)
        return A8W8_ERR_SHAPE;
    if (!W || !Wp)
        return A8W8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(W) & 15) || (reinterpret_cast<uintptr_t>(Wp) & 15))
        return A8W8_ERR_ALIGN;
    int cus = 0;
    const int rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    if (a8w8::launch_prepack(W, Wp, N, K, cus, static_cast<hipStream_t>(stream)) != hipSuccess)
        return A8W8_ERR_HIP;
    return A8W8_OK;
}

const char *gemm_a8w8_variant_name(int32_t variant)
{
    if (variant < 0 || variant >= a8w8::num_variants())
        return nullptr;
    return a8w8::variant(variant).name;
}

const char *gemm_a8w8_status_string(int status)
{
    switch (status) {
    case A8W8_OK: return "ok";
    case A8W8_ERR_NULL: return "a required pointer is NULL";
    case A8W8_ERR_SHAPE: return "invalid shape (need M >= 0, N >= 1, K >= 1, K % 128 == 0, M, N <= 2^30, K <= 2^22, 0 <= batch <= 65535)";
    case A8W8_ERR_ALIGN: return "misaligned buffer (A and W need 16 bytes, scales 4, Y 2)";
    case A8W8_ERR_ARCH: return "the current device is not gfx950 (MI355X)";
    case A8W8_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case A8W8_ERR_PLAN: return "invalid kernel instance for this shape";
    default: return "unknown status";
    }
}

uint64_t gemm_a8w8_table_hash(void) { return a8w8_table::kTableHash; }

int a8w8_quantize_1x128(const void *X, void *A, float *a_scale, int64_t M, int64_t K, void *stream)
{
    if (M < 0 || K < 1 || (K % 128) != 0 || M > kMaxDim || K > kMaxK)
        return A8W8_ERR_SHAPE;
    if (M == 0)
        return A8W8_OK;
    if (!X || !A || !a_scale)
        return A8W8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(X) & 15) || (reinterpret_cast<uintptr_t>(A) & 7) ||
        (reinterpret_cast<uintptr_t>(a_scale) & 3))
        return A8W8_ERR_ALIGN;
    int cus = 0;
    const int rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    if (a8w8::launch_quant_1x128(X, A, a_scale, M * (K / 128), cus, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return A8W8_ERR_HIP;
    return A8W8_OK;
}

}  // extern "C"
