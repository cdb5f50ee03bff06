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
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <cstring>
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
// Largest fp32 partial-tile area one split-K launch may use (per batch).
constexpr int64_t kMaxWorkspace = (int64_t)128 << 20;

// Per-device state: 0 = not yet checked, 1 = gfx950 ready, 2 = unsupported.
std::atomic<int> g_dev_state[kMaxDevices];
std::atomic<int> g_dev_cus[kMaxDevices];
std::mutex g_init_mutex;

}  // namespace

// Scratch of the allocation-free entry point (gemm_a8w8_blockscale_noalloc): a
// split-K workspace in static device memory, one copy per GPU (each at its own
// address), held until the process ends.  Its counter area starts zeroed and
// every call leaves it zeroed.  In host code this name stands for the host-side
// symbol, not the device copy: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device (scratch_address below).
static __device__ __align__(256) uint8_t scratch[A8W8_NOALLOC_SCRATCH_BYTES];

namespace {

// Device address of `scratch` per device (0: not looked up yet), and whether
// its counter area has been cleared by an eager (not captured) call.
std::atomic<uintptr_t> g_scratch[kMaxDevices];
std::atomic<int> g_scratch_clean[kMaxDevices];

int device_ready(int *cus, int *device = nullptr)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return A8W8_ERR_HIP;
    if (device)
        *device = dev;
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

// `cus`: compute units of the device (0: not known yet; the row-range skinny
// instances, whose grid depends on it, are then checked again at launch).
bool variant_accepts(int id, int64_t M, int64_t N, int64_t K, int cus)
{
    const Variant &v = a8w8::variant(id);
    if (v.kernel == A8W8_KERNEL_RSKINNY)
        return M <= v.max_m && skinny_fits(N, K) && (cus <= 0 || a8w8::rskinny_rows_fit(id, N, cus));
    // Split K: at least two K blocks per split, and a workspace within the cap
    // (stream-K: its partial slots on this device; 256 CUs while not known).
    if (v.splits > 1 && K / 128 < 2 * (int64_t)v.splits)
        return false;
    if ((v.splits > 1 || v.kernel == A8W8_KERNEL_SKTILE) &&
        a8w8::variant_workspace_bytes(id, M, N, K, cus > 0 ? cus : 256) > kMaxWorkspace)
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

// Split-K workspace.  A split instance runs S workgroups per output tile;
// they meet through caller-owned device memory laid out as
//   [counters: kCounterBytes, one int32 per (batch, tile) from the start][fp32 partials]
// (partials [batch][tile][split][BM * BN]).  The counter area has the same
// size and place for every call, so calls of different shapes and plans can
// share a workspace: every counter is zero when a call starts, and every split
// call leaves the counters it used zero again (the last split of a tile resets
// its counter), so a workspace cleared once with gemm_a8w8_workspace_init
// serves any number of calls in stream order.  Partials need no clearing.
constexpr int64_t kCounterBytes = A8W8_WORKSPACE_COUNTER_BYTES;

// Workspace bytes instance `id` needs for `batch` problems of (M, N, K) on a
// device with `cus` compute units: 0 when it cuts no K; INT64_MAX when its
// counters do not fit the counter area.  A stream-K instance's need depends on
// the device (its grid): with `cus` <= 0 (not known yet) this returns the
// counter area alone, a lower bound, and the caller checks again once it is.
int64_t workspace_need(int id, int64_t M, int64_t N, int64_t K, int64_t batch, int cus)
{
    if (a8w8::variant(id).kernel == A8W8_KERNEL_SKTILE && cus <= 0)
        return kCounterBytes;
    const int64_t counters = a8w8::variant_counters(id, M, N, K, cus);
    if (counters == 0)
        return 0;
    if (batch * counters * 4 > kCounterBytes)
        return INT64_MAX;
    return kCounterBytes + batch * a8w8::variant_workspace_bytes(id, M, N, K, cus);
}

// Ranking of the row-range skinny instances that take a shape: the fewest
// passes over K, then the most waves, then the most 16-row tiles per
// workgroup, then the fewest K blocks per pass.  Measured on the seven untuned
// decode shapes of 20 MiB and more among ten (N x K from 4608 x 5120 to
// 16384 x 2048, M = 1, 8, 16), the instance it ranks first is within 7% of the
// fastest row-range instance (within 2% on all but one of the 21 points).
// Returns -1 when none takes (M, N, K).
int best_rskinny(int64_t M, int64_t N, int64_t K, int cus, bool need_fused)
{
    int best = -1;
    int64_t best_key = 0;
    for (int i = 0; i < a8w8::num_variants(); ++i) {
        const Variant &v = a8w8::variant(i);
        if (v.kernel != A8W8_KERNEL_RSKINNY || (need_fused && !a8w8::variant_fuses_quant(i)) ||
            !variant_accepts(i, M, N, K, cus))
            continue;
        const int64_t key = -std::min<int64_t>(a8w8::variant_passes(i, K), 99) * 100000000 +
                            (int64_t)v.waves * 100000 + (int64_t)v.bn * 100 - v.waves * v.kblocks;
        if (best < 0 || key > best_key) {
            best = i;
            best_key = key;
        }
    }
    return best;
}

// Plan for shapes with no tuned table.  Up to M = 16: for weights of 20 MiB
// and more (fp32 block or row-wise scales), the row-range skinny instance ranked first above (measured 2-41%
// less time than the skinny rule below on those seven shapes: 5120 x 17408 at
// M = 16 in 23.9 against 40.2 us; on the three smaller ones, 15-17 MB, the
// skinny rule took up to 15% less time at M = 1); below, the skinny instance
// with the widest row group that still yields at least ~200 workgroups (wider
// groups share each activation fragment across more weight tiles), covering
// K in the fewest passes with the most blocks per pass (8 waves x 6 blocks
// measured fastest at K = 2048..8192); with fewer than 32 row groups and a
// split-K workspace, K split four ways over 16-row groups (measured 1.3-1.6x
// faster at N = 32..256, slower from ~64 groups up).  Above, for N <= 32: the
// tall kernel (16-row activation groups, 16 waves; 32-row groups from
// M = 4096).  Otherwise the largest tile that still gives every compute unit
// at least two workgroups, else the smallest, with K split (given a
// workspace) when even that leaves compute units idle.  Returns the plan with
// split K allowed in *split and the one without in *unsplit.
void heuristic_variants(int64_t M, int64_t N, int64_t K, int cus, int mx, int *split, int *unsplit)
{
    if (M <= 16 && !mx && N * K >= ((int64_t)20 << 20)) {
        const int r = best_rskinny(M, N, K, cus, false);
        if (r >= 0) {
            *split = *unsplit = r;
            return;
        }
    }
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
        if (best >= 0) {
            *split = *unsplit = best;
            if ((N + 15) / 16 < 32) {
                const int sid = find_variant(A8W8_KERNEL_SKINNY, 16, 16, 4, 3, 4);
                if (sid >= 0 && variant_accepts(sid, M, N, K, cus))
                    *split = sid;
            }
            return;
        }
    }
    if (N <= 32 && skinny_fits(N, K) && skinny_fits(M, K)) {
        const int bn = N <= 16 ? 16 : 32;
        const int id = M < 4096 ? find_variant(A8W8_KERNEL_TALL, 16, bn, bn == 32 ? 16 : 8, 3)
                                : find_variant(A8W8_KERNEL_TALL, 32, bn, 8, bn == 32 ? 6 : 3);
        if (id >= 0) {
            *split = *unsplit = id;
            return;
        }
    }
    static const int kTiles[][2] = {{256, 256}, {256, 128}, {128, 128}, {128, 64}, {64, 64}, {32, 64}, {32, 32}};
    const int nt = (int)(sizeof(kTiles) / sizeof(kTiles[0]));
    for (int i = 0; i < nt; ++i) {
        const int bm = kTiles[i][0], bn = kTiles[i][1];
        if (N <= 32 && bn > 32)
            continue;
        const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
        if (tiles >= 2 * (int64_t)cus) {
            *split = *unsplit = find_variant(A8W8_KERNEL_TILE, bm, bn, 0, 0);
            return;
        }
    }
    // Fewer tiles than two per CU even at 32 x 32: split K over S workgroups per tile,
    // the smallest S (2, 4, 8) that gives every CU a workgroup, keeping >= 4 K blocks
    // per split (the tuned tables pick split plans in this regime).
    const int base = find_variant(A8W8_KERNEL_TILE, 32, 32, 0, 0);
    const Variant &bv = a8w8::variant(base);
    const int64_t tiles = ((M + 31) / 32) * ((N + 31) / 32);
    *unsplit = *split = base;
    for (int s : {2, 4, 8}) {
        if (K / 128 < 4 * (int64_t)s)
            break;
        const int sid = find_variant(A8W8_KERNEL_TILE, 32, 32, bv.waves, bv.kblocks, s);
        if (sid < 0 || !variant_accepts(sid, M, N, K, cus))
            continue;
        *split = sid;
        if (tiles * s >= cus)
            break;
    }
}

struct Choice {
    int variant;
    int64_t key_m;
    int fallback;
};

// Table forms (the generated table's `form` field): fp32 block scales with
// row-major weights, MX, fp32 block scales with prepacked weights, row-wise.
// The packed and row-wise tables are decode tables (keys 1..16).
constexpr int FORM_BLOCK = 0, FORM_MX = 1, FORM_PACKED = 2, FORM_ROWWISE = 3;

int call_form(int sm, int wpk)
{
    return sm == 1 ? FORM_MX : sm == 2 ? FORM_ROWWISE : wpk ? FORM_PACKED : FORM_BLOCK;
}

// The row of the (N, K) table of `form` that serves M, if the table has one:
// its fastest instance, or -- when the call brings less workspace than that
// instance needs for `batch` problems -- the fastest one that splits no K.
Choice table_variant(int64_t M, int64_t N, int64_t K, int cus, int form, int64_t batch, int64_t ws_bytes)
{
    using namespace a8w8_table;
    for (int t = 0; t < kNumShapes; ++t) {
        const ShapeTable &s = kShapes[t];
        if (s.n != N || s.k != K || s.form != form)
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
            if (v >= 0 && variant_accepts(v, M, N, K, cus) && workspace_need(v, M, N, K, batch, cus) <= ws_bytes)
                return {v, s.key_m[lo], 0};
            const int u = find_variant(s.u_kernel[lo], s.u_bm[lo], s.u_bn[lo], s.u_waves[lo], s.u_kblocks[lo], 1);
            if (u >= 0 && variant_accepts(u, M, N, K, cus))
                return {u, s.key_m[lo], 0};
        }
        break;
    }
    return {-1, M, 1};
}

// The instance serving (M, N, K) for a call of `form`: the row of that form's
// table, else (packed and row-wise calls above their decode tables, or without
// one) the row of the block-scale table -- the MX table for MX calls -- else the
// heuristic plan (fallback = 1).
Choice select_variant(int64_t M, int64_t N, int64_t K, int cus, int form, int64_t batch, int64_t ws_bytes)
{
    Choice c = table_variant(M, N, K, cus, form, batch, ws_bytes);
    const int base = form == FORM_MX ? FORM_MX : FORM_BLOCK;
    if (c.variant < 0 && form != base)
        c = table_variant(M, N, K, cus, base, batch, ws_bytes);
    if (c.variant >= 0)
        return c;
    int split = -1, unsplit = -1;
    heuristic_variants(M, N, K, cus, form == FORM_MX ? 1 : 0, &split, &unsplit);
    return {workspace_need(split, M, N, K, batch, cus) <= ws_bytes ? split : unsplit, M, 1};
}

void fill_plan(int id, int64_t M, int64_t N, int64_t K, int64_t batch, int cus, int64_t key_m, int fallback,
               a8w8_plan *out)
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
    out->workspace = M > 0 ? workspace_need(id, M, N, K, batch > 0 ? batch : 1, cus) : 0;
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

// Operand set of one call: `batch` consecutive problems of one shape, and the
// split-K workspace it brings (NULL / 0: none).
struct Operands {
    const void *A;
    const void *a_scale;
    const void *W;
    const void *w_scale;
    void *Y;
    int64_t batch;
    int wpk;   // W in the packed layout
    int sm;    // scale kind: 0 fp32 block scales, 1 MX (E8M0), 2 row-wise fp32
    void *ws;
    int64_t ws_bytes;
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

// Enqueue instance `id` exactly as planned: a split instance takes its
// counters and partials from the call's workspace (the caller checked that it
// is large enough).
int launch(int id, const Operands &o, int64_t M, int64_t N, int64_t K, int cus, void *stream)
{
    Args a;
    a.splits = a8w8::variant(id).splits;
    a.ws = nullptr;
    a.cnt = nullptr;
    if (o.ws != nullptr) {
        uint8_t *base = static_cast<uint8_t *>(o.ws);
        a.cnt = reinterpret_cast<int32_t *>(base);
        a.ws = reinterpret_cast<float *>(base + kCounterBytes);
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
    if (o.sm < 0 || o.sm > 2 || o.wpk < 0 || o.wpk > 1)
        return A8W8_ERR_SHAPE;
    // MX weight-scale rows (one per 32 weight rows): the pskinny kernel's
    // descriptor spans them in 32 bits, the kernels index them in 31.
    if (o.sm == 1 && (N + 31) / 32 * (K / 128) * 4 >= ((int64_t)1 << 31))
        return A8W8_ERR_SHAPE;
    if (o.ws_bytes < 0)
        return A8W8_ERR_WORKSPACE;
    return A8W8_OK;
}

// The workspace argument of a call (planning looks at its size only).
int check_workspace(const Operands &o)
{
    if (o.ws_bytes > 0 && o.ws == nullptr)
        return A8W8_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(o.ws) & 255)
        return A8W8_ERR_ALIGN;
    return A8W8_OK;
}

// `variant` < 0: the selector's plan; otherwise that instance, which must
// accept the shape and find the workspace it needs.
int gemm_impl(int32_t variant, const Operands &o, int64_t M, int64_t N, int64_t K, void *stream)
{
    if (variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    int rc = check_call(o, M, N, K);
    if (rc == A8W8_OK)
        rc = check_workspace(o);
    if (rc != A8W8_OK)
        return rc;
    if (M == 0 || o.batch == 0)
        return A8W8_OK;
    if (variant >= 0 && !variant_accepts(variant, M, N, K, 0))
        return A8W8_ERR_PLAN;
    // A forced split instance's need is known here; a stream-K instance's depends on the
    // device's CU count (it may cut no tile at all) and is checked once that is known.
    if (variant >= 0 && a8w8::variant(variant).kernel != A8W8_KERNEL_SKTILE &&
        workspace_need(variant, M, N, K, o.batch, 0) > o.ws_bytes)
        return A8W8_ERR_WORKSPACE;
    rc = check_pointers(o.A, o.a_scale, o.W, o.w_scale, o.Y);
    if (rc != A8W8_OK)
        return rc;
    int cus = 0;
    rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    if (variant >= 0 && !variant_accepts(variant, M, N, K, cus))
        return A8W8_ERR_PLAN;
    int id = variant;
    if (id < 0) {
        // Packed and row-wise calls take their own decode tables where tuned and
        // the block-scale table otherwise: the same kernels serve every form.
        const Choice c = select_variant(M, N, K, cus, call_form(o.sm, o.wpk), o.batch, o.ws_bytes);
        log_plan(M, N, K, c.variant, c.key_m, c.fallback);
        id = c.variant;
    }
    if (workspace_need(id, M, N, K, o.batch, cus) > o.ws_bytes)
        return A8W8_ERR_WORKSPACE;
    return launch(id, o, M, N, K, cus, stream);
}

int plan_impl(int32_t variant, const Operands &o, int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out)
{
    if (!out)
        return A8W8_ERR_NULL;
    if (variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    int rc = check_call(o, M, N, K);
    if (rc != A8W8_OK)
        return rc;
    const int cus = cu_count > 0 ? cu_count : 256;
    const int64_t Mp = M > 0 ? M : 1, batch = o.batch > 0 ? o.batch : 1;
    if (variant >= 0) {
        if (!variant_accepts(variant, Mp, N, K, cus))
            return A8W8_ERR_PLAN;
        if (workspace_need(variant, Mp, N, K, batch, cus) > o.ws_bytes)
            return A8W8_ERR_WORKSPACE;
        fill_plan(variant, M, N, K, batch, cus, M, 0, out);
        return A8W8_OK;
    }
    const Choice c = select_variant(Mp, N, K, cus, call_form(o.sm, o.wpk), batch, o.ws_bytes);
    fill_plan(c.variant, M, N, K, batch, cus, c.key_m, c.fallback, out);
    return A8W8_OK;
}

Operands from_desc(const a8w8_gemm_desc &d)
{
    return {d.A, d.a_scale, d.W, d.w_scale, d.Y, d.batch, d.w_packed, d.scale_kind, d.workspace, d.workspace_bytes};
}

// The instance the fused-quantisation entry runs: a forced one must be a
// row-range skinny instance that takes the shape; otherwise the one
// best_rskinny ranks first (on out_proj, qkv and down_proj at M = 1..16 within
// 3% of the fastest fused instance).  -1: none.
int fused_variant(int32_t variant, int64_t M, int64_t N, int64_t K, int cus)
{
    if (variant >= 0)
        return a8w8::variant_fuses_quant(variant) && variant_accepts(variant, M, N, K, cus) ? variant : -1;
    return best_rskinny(M, N, K, cus, true);
}

int fused_check(const void *X, const void *W, const float *w_scale, const void *Y, int64_t M, int64_t N, int64_t K,
                int32_t w_packed)
{
    int rc = check_shape(M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (M > 16 || w_packed < 0 || w_packed > 1)
        return A8W8_ERR_SHAPE;
    if (M == 0)
        return A8W8_OK;
    if (!X || !W || !w_scale || !Y)
        return A8W8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(X) & 15) || (reinterpret_cast<uintptr_t>(W) & 15) ||
        (reinterpret_cast<uintptr_t>(w_scale) & 3) || (reinterpret_cast<uintptr_t>(Y) & 1))
        return A8W8_ERR_ALIGN;
    return A8W8_OK;
}

__global__ void workspace_clear_kernel(uint4 *p, int64_t n16)
{
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

int gemm_a8w8_blockscale(const void *A, const float *a_scale, const void *W, const float *w_scale, void *Y,
                         int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, W, w_scale, Y, 1, 0, 0, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_blockscale_packed(const void *A, const float *a_scale, const void *Wp, const float *w_scale, void *Y,
                                int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, Wp, w_scale, Y, 1, 1, 0, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_mxscale(const void *A, const void *a_scale, const void *W, const void *w_scale, void *Y, int64_t M,
                      int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, W, w_scale, Y, 1, 0, 1, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_mxscale_packed(const void *A, const void *a_scale, const void *Wp, const void *w_scale, void *Y,
                             int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, Wp, w_scale, Y, 1, 1, 1, nullptr, 0}, M, N, K, stream);
}

int batched_gemm_a8w8_mxscale(const void *A, const void *a_scale, const void *W, const void *w_scale, void *Y,
                              int64_t batch, int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, W, w_scale, Y, batch, 0, 1, nullptr, 0}, M, N, K, stream);
}

int batched_gemm_a8w8_mxscale_packed(const void *A, const void *a_scale, const void *Wp, const void *w_scale,
                                     void *Y, int64_t batch, int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, Wp, w_scale, Y, batch, 1, 1, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_mxscale_run_variant(int32_t variant, const void *A, const void *a_scale, const void *W,
                                  const void *w_scale, void *Y, int64_t batch, int64_t M, int64_t N, int64_t K,
                                  int32_t w_packed, void *stream)
{
    if (variant < 0)
        return A8W8_ERR_PLAN;
    return gemm_impl(variant, {A, a_scale, W, w_scale, Y, batch, w_packed ? 1 : 0, 1, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_rowwise(const void *A, const float *a_scale, const void *W, const float *w_scale, void *Y,
                      int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, W, w_scale, Y, 1, 0, 2, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_rowwise_packed(const void *A, const float *a_scale, const void *Wp, const float *w_scale, void *Y,
                             int64_t M, int64_t N, int64_t K, void *stream)
{
    return gemm_impl(-1, {A, a_scale, Wp, w_scale, Y, 1, 1, 2, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_rowwise_run_variant(int32_t variant, const void *A, const float *a_scale, const void *W,
                                  const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K, int32_t w_packed,
                                  void *stream)
{
    if (variant < 0)
        return A8W8_ERR_PLAN;
    return gemm_impl(variant, {A, a_scale, W, w_scale, Y, 1, w_packed ? 1 : 0, 2, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_ex(const a8w8_gemm_desc *desc, void *stream)
{
    if (!desc)
        return A8W8_ERR_NULL;
    return gemm_impl(desc->variant < 0 ? -1 : desc->variant, from_desc(*desc), desc->M, desc->N, desc->K, stream);
}

int gemm_a8w8_ex_plan(const a8w8_gemm_desc *desc, int32_t cu_count, a8w8_plan *out)
{
    if (!desc)
        return A8W8_ERR_NULL;
    const Operands o = from_desc(*desc);   // planning looks at the workspace size only
    return plan_impl(desc->variant < 0 ? -1 : desc->variant, o, desc->M, desc->N, desc->K, cu_count, out);
}

int gemm_a8w8_workspace_init(void *workspace, int64_t bytes, void *stream)
{
    if (bytes < 0)
        return A8W8_ERR_SHAPE;
    if (bytes == 0)
        return A8W8_OK;
    if (!workspace)
        return A8W8_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255) || (bytes & 255))
        return A8W8_ERR_ALIGN;
    int cus = 0;
    const int rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    const int64_t n16 = bytes / 16;
    const int64_t blocks = std::min<int64_t>((n16 + 255) / 256, (int64_t)cus * 8);
    hipLaunchKernelGGL(workspace_clear_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<uint4 *>(workspace), n16);
    return hipGetLastError() == hipSuccess ? A8W8_OK : A8W8_ERR_HIP;
}

int gemm_a8w8_blockscale_noalloc(const void *A, const float *a_scale, const void *W, const float *w_scale, void *Y,
                                 int64_t M, int64_t N, int64_t K, void *stream)
{
    Operands o = {A, a_scale, W, w_scale, Y, 1, 0, 0, nullptr, 0};
    int rc = check_call(o, M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (M == 0)
        return A8W8_OK;
    rc = check_pointers(A, a_scale, W, w_scale, Y);
    if (rc != A8W8_OK)
        return rc;
    int cus = 0, dev = 0;
    rc = device_ready(&cus, &dev);
    if (rc != A8W8_OK)
        return rc;
    // The table's fastest plan when its workspace fits the array, else the
    // fastest one that cuts no K (the selector's rule for a call's workspace).
    const Choice c = select_variant(M, N, K, cus, FORM_BLOCK, 1, (int64_t)A8W8_NOALLOC_SCRATCH_BYTES);
    if (workspace_need(c.variant, M, N, K, 1, cus) > (int64_t)A8W8_NOALLOC_SCRATCH_BYTES)
        return A8W8_ERR_WORKSPACE;
    // Set-up, once per device with that device current: the device address of
    // this GPU's copy of the array.
    uintptr_t addr = g_scratch[dev].load(std::memory_order_acquire);
    if (addr == 0) {
        std::lock_guard<std::mutex> lock(g_init_mutex);
        addr = g_scratch[dev].load(std::memory_order_acquire);
        if (addr == 0) {
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
                return A8W8_ERR_HIP;
            addr = reinterpret_cast<uintptr_t>(ptr);
            g_scratch[dev].store(addr, std::memory_order_release);
        }
    }
    // Static device memory starts zero-filled; until an eager call has cleared
    // the counter area with the library's fill kernel (stream-ordered before
    // this call's GEMM), every call enqueues that clear first -- inside a
    // captured graph too, where it is part of each replay.
    if (g_scratch_clean[dev].load(std::memory_order_acquire) == 0) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs) != hipSuccess)
            return A8W8_ERR_HIP;
        hipLaunchKernelGGL(workspace_clear_kernel, dim3(16), dim3(256), 0, static_cast<hipStream_t>(stream),
                           reinterpret_cast<uint4 *>(addr), (int64_t)(kCounterBytes / 16));
        if (hipGetLastError() != hipSuccess)
            return A8W8_ERR_HIP;
        if (cs == hipStreamCaptureStatusNone)
            g_scratch_clean[dev].store(1, std::memory_order_release);
    }
    o.ws = reinterpret_cast<void *>(addr);
    o.ws_bytes = A8W8_NOALLOC_SCRATCH_BYTES;
    log_plan(M, N, K, c.variant, c.key_m, c.fallback);
    return launch(c.variant, o, M, N, K, cus, stream);
}

int gemm_a8w8_mxscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out)
{
    return plan_impl(-1, {nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 1, nullptr, 0}, M, N, K, cu_count, out);
}

int gemm_a8w8_blockscale_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, a8w8_plan *out)
{
    return plan_impl(-1, {nullptr, nullptr, nullptr, nullptr, nullptr, 1, 0, 0, nullptr, 0}, M, N, K, cu_count, out);
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
    fill_plan(variant, M, N, K, 1, 256, M, 0, out);
    return A8W8_OK;
}

int gemm_a8w8_blockscale_run_variant(int32_t variant, const void *A, const float *a_scale, const void *W,
                                     const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K,
                                     void *stream)
{
    if (variant < 0)
        return A8W8_ERR_PLAN;
    return gemm_impl(variant, {A, a_scale, W, w_scale, Y, 1, 0, 0, nullptr, 0}, M, N, K, stream);
}

int gemm_a8w8_blockscale_packed_run_variant(int32_t variant, const void *A, const float *a_scale, const void *Wp,
                                            const float *w_scale, void *Y, int64_t M, int64_t N, int64_t K,
                                            void *stream)
{
    if (variant < 0)
        return A8W8_ERR_PLAN;
    return gemm_impl(variant, {A, a_scale, Wp, w_scale, Y, 1, 1, 0, nullptr, 0}, M, N, K, stream);
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
    case A8W8_ERR_ALIGN: return "misaligned buffer (A and W need 16 bytes, scales 4, Y 2, a split-K workspace 256)";
    case A8W8_ERR_ARCH: return "the current device is not gfx950 (MI355X)";
    case A8W8_ERR_HIP: return "HIP runtime call or kernel launch failed";
    case A8W8_ERR_PLAN: return "invalid kernel instance for this shape";
    case A8W8_ERR_WORKSPACE: return "the kernel instance splits K and the call's workspace is missing or too small";
    default: return "unknown status";
    }
}

uint64_t gemm_a8w8_table_hash(void) { return a8w8_table::kTableHash; }

int gemm_a8w8_blockscale_fused_quant(const void *X, const void *W, const float *w_scale, void *Y, int64_t M,
                                     int64_t N, int64_t K, int32_t w_packed, int32_t variant, void *stream)
{
    if (variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    int rc = fused_check(X, W, w_scale, Y, M, N, K, w_packed);
    if (rc != A8W8_OK || M == 0)
        return rc;
    if (variant >= 0 && (!a8w8::variant_fuses_quant(variant) || !variant_accepts(variant, M, N, K, 0)))
        return A8W8_ERR_PLAN;
    int cus = 0;
    rc = device_ready(&cus);
    if (rc != A8W8_OK)
        return rc;
    const int id = fused_variant(variant, M, N, K, cus);
    if (id < 0)
        return A8W8_ERR_PLAN;
    Args a;
    std::memset(&a, 0, sizeof(a));
    a.A = static_cast<const uint8_t *>(X);
    a.W = static_cast<const uint8_t *>(W);
    a.w_scale = w_scale;
    a.Y = static_cast<uint16_t *>(Y);
    a.M = (int32_t)M;
    a.N = (int32_t)N;
    a.K = (int32_t)K;
    a.wpk = w_packed;
    a.sm = 0;
    a.splits = 1;
    if (a8w8::launch_quant_fused(id, a, cus, static_cast<hipStream_t>(stream)) != hipSuccess)
        return A8W8_ERR_HIP;
    return A8W8_OK;
}

int gemm_a8w8_blockscale_fused_quant_plan(int64_t M, int64_t N, int64_t K, int32_t cu_count, int32_t variant,
                                          a8w8_plan *out)
{
    if (!out)
        return A8W8_ERR_NULL;
    if (variant >= a8w8::num_variants())
        return A8W8_ERR_PLAN;
    int rc = check_shape(M, N, K);
    if (rc != A8W8_OK)
        return rc;
    if (M > 16)
        return A8W8_ERR_SHAPE;
    const int cus = cu_count > 0 ? cu_count : 256;
    const int id = fused_variant(variant, M > 0 ? M : 1, N, K, cus);
    if (id < 0)
        return A8W8_ERR_PLAN;
    fill_plan(id, M, N, K, 1, cus, M, 0, out);
    return A8W8_OK;
}

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
