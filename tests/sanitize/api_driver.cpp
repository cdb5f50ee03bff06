// Sanitizer driver for the library's host side (built with AddressSanitizer
// and UndefinedBehaviorSanitizer on the host code only, by
// tests/test_sanitizers.py).  It exercises everything that runs without a
// GPU: the selector (every M = 1..8192 of every tuned (N, K), block and MX,
// several workspace sizes, batches and CU counts), the heuristic plans of
// untuned shapes, the instance descriptions, the status strings, the argument
// checks of every entry point (errors are reported before any device call)
// and the workspace-size arithmetic of split and stream-K instances.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "gemm_a8w8_blockscale.h"

static int fails = 0;
#define CHECK(c, ...)                     \
    do {                                  \
        if (!(c)) {                       \
            fprintf(stderr, __VA_ARGS__); \
            fprintf(stderr, "\n");        \
            ++fails;                      \
        }                                 \
    } while (0)

static a8w8_gemm_desc desc(int64_t M, int64_t N, int64_t K, int kind, int64_t batch, int variant, int64_t ws)
{
    a8w8_gemm_desc d;
    memset(&d, 0, sizeof(d));
    d.batch = batch;
    d.M = M;
    d.N = N;
    d.K = K;
    d.scale_kind = kind;
    d.variant = variant;
    d.workspace_bytes = ws;
    return d;
}

int main()
{
    const int64_t nk[][2] = {{14336, 5120}, {5120, 6144}, {16384, 5120}, {34816, 5120}, {256, 6144}, {32, 6144},
                             {1792, 5120}, {1000, 3072}, {128, 8192}, {100, 8192}, {3000, 384}, {77, 128}};
    const int64_t wss[] = {0, 1 << 20, (int64_t)129 << 20, (int64_t)1 << 40};
    a8w8_plan p;
    long plans = 0;
    for (const auto &s : nk)
        for (int64_t M = 1; M <= 8192; M += (M < 64 ? 1 : M / 16)) {
            CHECK(gemm_a8w8_blockscale_plan(M, s[0], s[1], 0, &p) == A8W8_OK, "plan %lld", (long long)M);
            CHECK(p.workspace == 0 && p.variant >= 0 && p.variant < gemm_a8w8_num_variants(), "plain plan");
            CHECK(gemm_a8w8_mxscale_plan(M, s[0], s[1], 256, &p) == A8W8_OK, "mx plan");
            for (int64_t ws : wss)
                for (int kind = 0; kind < 3; ++kind)
                    for (int cus : {0, 80, 256, 304}) {
                        a8w8_gemm_desc d = desc(M, s[0], s[1], kind, kind == 1 ? 3 : 1, -1, ws);
                        CHECK(gemm_a8w8_ex_plan(&d, cus, &p) == A8W8_OK, "ex plan");
                        CHECK(p.workspace <= ws, "plan workspace %lld > %lld", (long long)p.workspace,
                              (long long)ws);
                        ++plans;
                    }
        }
    const int nv = gemm_a8w8_num_variants();
    for (int v = -2; v < nv + 2; ++v) {
        const char *name = gemm_a8w8_variant_name(v);
        CHECK((v >= 0 && v < nv) == (name != nullptr), "variant name %d", v);
        for (int64_t M : {0, 1, 7, 16, 17, 300, 4097})
            for (int64_t N : {1, 32, 300, 14336})
                for (int64_t K : {128, 640, 5120}) {
                    const int rc = gemm_a8w8_describe_variant(v, M, N, K, &p);
                    CHECK((v >= 0 && v < nv) == (rc == A8W8_OK), "describe %d", v);
                    for (int64_t ws : wss) {
                        a8w8_gemm_desc d = desc(M > 0 ? M : 1, N, K, 0, 1, v, ws);
                        const int r2 = gemm_a8w8_ex_plan(&d, 256, &p);
                        CHECK(r2 == A8W8_OK || r2 == A8W8_ERR_PLAN || r2 == A8W8_ERR_WORKSPACE, "forced plan rc %d",
                              r2);
                        if (r2 == A8W8_OK)
                            CHECK(p.workspace <= ws && (v < 0 || p.variant == v), "forced plan %d", v);
                    }
                }
    }
    for (int st = -3; st < 12; ++st)
        CHECK(gemm_a8w8_status_string(st) != nullptr && strlen(gemm_a8w8_status_string(st)) > 0, "status %d", st);
    // argument checks: every one returns before a device call
    alignas(256) static uint8_t buf[1 << 16];
    uint8_t *b = buf;
    CHECK(gemm_a8w8_blockscale(nullptr, (float *)b, b, (float *)b, b, 4, 16, 128, nullptr) == A8W8_ERR_NULL, "null A");
    CHECK(gemm_a8w8_blockscale(b, (float *)b, b, (float *)b, b, 4, 16, 100, nullptr) == A8W8_ERR_SHAPE, "K not a multiple of 128");
    CHECK(gemm_a8w8_blockscale(b, (float *)b, b, (float *)b, b, -1, 16, 128, nullptr) == A8W8_ERR_SHAPE, "M < 0");
    CHECK(gemm_a8w8_blockscale(b + 1, (float *)(b + 2), b, (float *)b, b, 4, 16, 128, nullptr) == A8W8_ERR_ALIGN,
          "misaligned a_scale");
    CHECK(gemm_a8w8_blockscale(b, (float *)b, b, (float *)b, b, 0, 16, 128, nullptr) == A8W8_OK, "M = 0 no-op");
    a8w8_gemm_desc d = desc(4, 16, 128, 0, 1, -1, 256);
    d.A = b; d.a_scale = b; d.W = b; d.w_scale = b; d.Y = b;
    d.workspace = nullptr;
    CHECK(gemm_a8w8_ex(&d, nullptr) == A8W8_ERR_WORKSPACE, "workspace size without pointer");
    d.workspace = b + 64;
    CHECK(gemm_a8w8_ex(&d, nullptr) == A8W8_ERR_ALIGN, "misaligned workspace");
    d.workspace = b; d.workspace_bytes = -1;
    CHECK(gemm_a8w8_ex(&d, nullptr) == A8W8_ERR_WORKSPACE, "negative workspace");
    d.workspace_bytes = 0; d.scale_kind = 7;
    CHECK(gemm_a8w8_ex(&d, nullptr) == A8W8_ERR_SHAPE, "bad scale kind");
    d.scale_kind = 0; d.variant = 1 << 20;
    CHECK(gemm_a8w8_ex(&d, nullptr) == A8W8_ERR_PLAN, "bad variant");
    CHECK(gemm_a8w8_ex(nullptr, nullptr) == A8W8_ERR_NULL, "null desc");
    CHECK(gemm_a8w8_ex_plan(nullptr, 0, &p) == A8W8_ERR_NULL, "null desc plan");
    CHECK(gemm_a8w8_workspace_init(nullptr, 256, nullptr) != A8W8_OK, "null workspace init");
    CHECK(gemm_a8w8_table_hash() != 0, "table hash");
    if (fails)
        fprintf(stderr, "%d failures\n", fails);
    else
        printf("api sanitizer driver: ok (%ld plans)\n", plans);
    return fails ? 1 : 0;
}
