"""Host-side checks of libgemm_a8w8.so: exports, argument errors, selector table.

Nothing here launches a kernel: argument errors are reported before the
library touches the HIP runtime, and planning is host-only.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import fp8_block_scaled_a8w8_amd as g
from fp8_block_scaled_a8w8_amd import gen_selector_table as gst

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_a8w8_blockscale.h")

# the (N, K) pairs the tuned table must cover, M = 1..8192
REGISTERED = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144), (512, 1024)]


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:batched_)?(?:gemm_)?a8w8_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(g.LIB_PATH)
    declared = _declared_functions()
    assert len(declared) >= 8
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(g.EXPORTED) == declared


def _call(A=16, a_s=16, W=16, w_s=16, Y=16, M=4, N=512, K=1024):
    return g.lib().gemm_a8w8_blockscale(A, a_s, W, w_s, Y, M, N, K, None)


@pytest.mark.parametrize("M,N,K", [(-1, 512, 1024), (4, 0, 1024), (4, 512, 0), (4, 512, 1000),
                                   (4, 512, 127), (1 << 31, 512, 1024), (4, 512, (1 << 22) + 128)])
def test_bad_shapes(M, N, K):
    assert _call(M=M, N=N, K=K) == g.A8W8_ERR_SHAPE
    p = g.Plan()
    assert g.lib().gemm_a8w8_blockscale_plan(M, N, K, 0, ctypes.byref(p)) == g.A8W8_ERR_SHAPE


def test_m_zero_is_a_no_op_even_with_null_pointers():
    assert g.lib().gemm_a8w8_blockscale(None, None, None, None, None, 0, 512, 1024, None) == g.A8W8_OK
    assert g.lib().a8w8_quantize_1x128(None, None, None, 0, 1024, None) == g.A8W8_OK


@pytest.mark.parametrize("M,K", [(-1, 1024), (4, 0), (4, 1000), (4, 127), (1 << 31, 1024), (4, (1 << 22) + 128)])
def test_quantize_bad_shapes(M, K):
    assert g.lib().a8w8_quantize_1x128(16, 16, 16, M, K, None) == g.A8W8_ERR_SHAPE


def test_packed_entry_points_check_arguments():
    L = g.lib()
    assert L.a8w8_prepack_weights(16, 16, 0, 1024, None) == g.A8W8_ERR_SHAPE
    assert L.a8w8_prepack_weights(16, 16, 64, 1000, None) == g.A8W8_ERR_SHAPE
    assert L.a8w8_prepack_weights(None, 16, 64, 1024, None) == g.A8W8_ERR_NULL
    assert L.a8w8_prepack_weights(16, 24, 64, 1024, None) == g.A8W8_ERR_ALIGN
    assert L.gemm_a8w8_blockscale_packed(16, 16, 16, 16, 16, 4, 512, 1000, None) == g.A8W8_ERR_SHAPE
    assert L.gemm_a8w8_blockscale_packed(16, 16, None, 16, 16, 4, 512, 1024, None) == g.A8W8_ERR_NULL
    assert L.gemm_a8w8_blockscale_packed(None, None, None, None, None, 0, 512, 1024, None) == g.A8W8_OK
    skinny = [v["variant"] for v in g.variants() if v["kernel_name"] == "skinny"][0]
    assert L.gemm_a8w8_blockscale_packed_run_variant(skinny, 16, 16, 16, 16, 16, 17, 512, 1024, None) == g.A8W8_ERR_PLAN


def test_quantize_null_and_misaligned_pointers():
    q = g.lib().a8w8_quantize_1x128
    assert q(None, 16, 16, 4, 1024, None) == g.A8W8_ERR_NULL
    assert q(16, None, 16, 4, 1024, None) == g.A8W8_ERR_NULL
    assert q(16, 16, None, 4, 1024, None) == g.A8W8_ERR_NULL
    assert q(24, 16, 16, 4, 1024, None) == g.A8W8_ERR_ALIGN      # X needs 16 bytes
    assert q(16, 20, 16, 4, 1024, None) == g.A8W8_ERR_ALIGN      # A needs 8
    assert q(16, 16, 18, 4, 1024, None) == g.A8W8_ERR_ALIGN      # a_scale needs 4


@pytest.mark.parametrize("which", ["A", "a_s", "W", "w_s", "Y"])
def test_null_pointers(which):
    assert _call(**{which: None}) == g.A8W8_ERR_NULL


@pytest.mark.parametrize("kw", [{"A": 24}, {"W": 8}, {"a_s": 18}, {"w_s": 2}, {"Y": 17}])
def test_misaligned_pointers(kw):
    assert _call(**kw) == g.A8W8_ERR_ALIGN


def test_status_strings_and_variant_names():
    for s in range(8):
        assert g.gemm_a8w8_status_string(s) != "unknown status"
    assert g.gemm_a8w8_status_string(99) == "unknown status"
    n = g.gemm_a8w8_num_variants()
    names = [g.gemm_a8w8_variant_name(i) for i in range(n)]
    assert len(set(names)) == n and all(names)
    assert g.gemm_a8w8_variant_name(n) is None
    assert g.lib().gemm_a8w8_describe_variant(n, 1, 1, 128, ctypes.byref(g.Plan())) == g.A8W8_ERR_PLAN


def test_run_variant_rejects_skinny_above_16_rows():
    skinny = [v["variant"] for v in g.variants() if v["kernel_name"] == "skinny"]
    assert skinny
    rc = g.lib().gemm_a8w8_blockscale_run_variant(skinny[0], 16, 16, 16, 16, 16, 17, 512, 1024, None)
    assert rc == g.A8W8_ERR_PLAN


def test_run_variant_rejects_persistent_skinny_beyond_its_k():
    ps = [v for v in g.variants() if v["kernel_name"] == "pskinny"]
    assert ps
    for v in ps:
        kb = v["waves"] * v["kblocks"]
        lib = g.lib()
        assert lib.gemm_a8w8_blockscale_run_variant(v["variant"], 16, 16, 16, 16, 16, 17, 512, 128 * kb,
                                                    None) == g.A8W8_ERR_PLAN
        assert lib.gemm_a8w8_blockscale_run_variant(v["variant"], 16, 16, 16, 16, 16, 4, 512, 128 * (kb + 1),
                                                    None) == g.A8W8_ERR_PLAN


def test_variant_shapes_are_launchable():
    for v in g.variants():
        if v["kernel_name"] in ("tile", "ptile", "sktile"):
            assert v["bm"] % 32 == 0 and v["bn"] % 32 == 0 and v["bn"] // 2 <= 128
            assert 128 % (v["bn"] // 2) == 0, v          # a wave's columns stay in one weight block
            assert 2 * (v["bm"] + v["bn"]) * 128 <= 160 * 1024
        elif v["kernel_name"] == "tall":
            assert v["bn"] in (16, 32) and v["bm"] in (16, 32, 64), v     # all weight rows in weight block 0
        elif v["kernel_name"] == "rskinny":
            assert v["bm"] == 16 and v["bn"] % 16 == 0 and v["bn"] <= 128, v   # at most two weight-scale rows
            assert v["bn"] // 16 <= v["waves"], v                          # wave t stores tile t
        else:
            assert v["bm"] == 16 and v["bn"] in (16, 32, 64, 128), v   # row group inside one weight block
            assert v["waves"] >= 1 and v["kblocks"] >= 1


# ---------------------------------------------------------------- selector table

def test_generated_header_matches_table():
    assert gst.main(["--check"]) == 0


def test_table_validation_rejects_bad_tables():
    good = {"shapes": [{"n": 64, "k": 128, "rows":
                        [{"key_m": m, "kernel": "skinny", "bm": 16, "bn": 16, "waves": 4} for m in range(1, 17)] +
                        [{"key_m": 20, "kernel": "tile", "bm": 32, "bn": 32, "waves": 4},
                         {"key_m": 8192, "kernel": "tile", "bm": 32, "bn": 32, "waves": 4}]}]}
    with pytest.raises(ValueError):
        gst.validate(good)                                   # 8192 serves M = 21 (> 1.25x)
    rows = good["shapes"][0]["rows"][:-1]
    m = 20
    while m < 8192:
        m = min(8192, int(m * 1.25))
        rows.append({"key_m": m, "kernel": "tile", "bm": 32, "bn": 32, "waves": 4})
    ok = {"shapes": [{"n": 64, "k": 128, "rows": rows}]}
    gst.validate(ok)
    dup = {"shapes": ok["shapes"] * 2}
    with pytest.raises(ValueError):
        gst.validate(dup)
    bad = {"shapes": [{"n": 64, "k": 128, "rows": rows[:3] + [dict(rows[3], key_m=3)] + rows[4:]}]}
    with pytest.raises(ValueError):
        gst.validate(bad)


def _table_shapes(mx=False, form=None):
    want = form or ("mx" if mx else "block")
    return [(int(s["n"]), int(s["k"])) for s in gst.load()["shapes"] if gst.form_of(s) == want]


@pytest.mark.parametrize("N,K", REGISTERED)
def test_every_m_has_a_tuned_plan_within_125_percent(N, K):
    if (N, K) not in _table_shapes():
        pytest.skip(f"({N},{K}) has no tuned table yet")
    for M in range(1, 8193):
        p = g.gemm_a8w8_blockscale_plan(M, N, K)
        assert p["fallback"] == 0, (M, p)
        assert M <= p["key_m"] <= 1.25 * M, (M, p)
        if M <= 16:
            assert p["key_m"] == M
        if p["kernel_name"] == "skinny":
            assert M <= 16


BIG_WS = 1 << 40


def test_heuristic_skinny_rule():
    # Up to M = 16 on an unregistered (N, K): fewest passes over K, then the deepest
    # pass (8 waves x 6 blocks); fewer than 32 sixteen-row groups split K four ways
    # when the call brings a workspace.
    for M, N, K in ((1, 1000, 3072), (16, 640, 4096), (1, 2000, 2048), (16, 3000, 5120), (1, 4096, 4096)):
        p = g.gemm_a8w8_blockscale_plan(M, N, K)
        assert p["fallback"] == 1 and p["name"] == "skinny_r1_d6_w8" and p["kpasses"] == 1, (M, N, K, p)
    for M, N, K in ((8, 128, 8192), (5, 100, 1024), (16, 496, 4096), (1, 32, 3072)):
        p = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=BIG_WS)
        assert p["fallback"] == 1 and p["name"] == "skinny_r1_d3_w4_k4", (M, N, K, p)
        assert p["grid"] == -(-N // 16) * 4 and p["workspace"] > 0
        u = g.gemm_a8w8_blockscale_plan(M, N, K)                   # no workspace: unsplit
        assert u["fallback"] == 1 and u["splits"] == 1 and u["workspace"] == 0 and u["kernel_name"] == "skinny"
        assert g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=p["workspace"] - 256)["name"] == u["name"]
        assert g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=p["workspace"])["name"] == p["name"]
    # too few K blocks for four splits (K/128 < 8): unsplit
    p = g.gemm_a8w8_ex_plan(5, 100, 896, workspace_bytes=BIG_WS)
    assert p["fallback"] == 1 and p["splits"] == 1 and p["kernel_name"] == "skinny"


def test_heuristic_row_range_rule_for_large_weights():
    # Up to M = 16 on an unregistered (N, K) with at least 20 MiB of weights: the
    # row-range skinny instance with the fewest passes over K, then the most waves,
    # then the widest, then the shortest pass; below 20 MiB the skinny rule.
    cases = {(8, 6144, 4096): "rskinny_t2_d3_w16_g1", (1, 5120, 17408): "rskinny_t2_d3_w16_g1",
             (16, 12288, 4096): "rskinny_t4_d5_w8_g1", (1, 16384, 2048): "rskinny_t4_d3_w8_g1",
             (8, 10240, 3072): "rskinny_t4_d3_w8_g1", (16, 4608, 5120): "rskinny_t2_d3_w16_g1"}
    for (M, N, K), name in cases.items():
        p = g.gemm_a8w8_blockscale_plan(M, N, K, cu_count=256)
        assert p["fallback"] == 1 and p["name"] == name, (M, N, K, p)
        assert g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=BIG_WS, cu_count=256)["name"] == name
    for M, N, K in ((1, 4096, 4096), (16, 7168, 2048), (8, 2048, 8192)):
        assert g.gemm_a8w8_blockscale_plan(M, N, K, cu_count=256)["kernel_name"] == "skinny", (M, N, K)
    # rows beyond the largest row-range instance (64 per CU): the skinny rule
    assert g.gemm_a8w8_blockscale_plan(4, 20480, 2048, cu_count=256)["kernel_name"] == "skinny"
    # MX scales keep the skinny rule
    assert g.gemm_a8w8_mxscale_plan(8, 6144, 4096, cu_count=256)["kernel_name"] != "rskinny"


def test_unregistered_shape_falls_back_not_fails():
    p = g.gemm_a8w8_blockscale_plan(3, 1000, 384)
    assert p["fallback"] == 1 and p["kernel_name"] == "skinny"
    p = g.gemm_a8w8_blockscale_plan(5000, 1000, 384)
    assert p["fallback"] == 1 and p["kernel_name"] == "tile"
    tiles = ((5000 + p["bm"] - 1) // p["bm"]) * ((1000 + p["bn"] - 1) // p["bn"])
    assert min(tiles, 256) <= p["grid"] <= tiles          # persistent: at most one workgroup per tile
    for n, m in ((8, 100), (17, 100), (32, 5000), (12, 9000)):
        p = g.gemm_a8w8_blockscale_plan(m, n, 384)
        assert p["fallback"] == 1 and p["kernel_name"] == "tall" and n <= p["bn"], (n, m, p)
        assert p["grid"] == (m + p["bm"] - 1) // p["bm"]


# ---------------------------------------------------------------- MX-scaled entries

def _mx(name="gemm_a8w8_mxscale", A=16, a_s=16, W=16, w_s=16, Y=16, batch=None, M=4, N=512, K=1024):
    f = getattr(g.lib(), name)
    if batch is None:
        return f(A, a_s, W, w_s, Y, M, N, K, None)
    return f(A, a_s, W, w_s, Y, batch, M, N, K, None)


@pytest.mark.parametrize("name", ["gemm_a8w8_mxscale", "gemm_a8w8_mxscale_packed"])
def test_mx_entries_check_arguments(name):
    assert _mx(name, K=96) == g.A8W8_ERR_SHAPE                   # whole 128-wide K blocks only
    assert _mx(name, M=-1) == g.A8W8_ERR_SHAPE
    assert _mx(name, N=0) == g.A8W8_ERR_SHAPE
    assert _mx(name, A=None) == g.A8W8_ERR_NULL
    assert _mx(name, w_s=None) == g.A8W8_ERR_NULL
    assert _mx(name, W=24) == g.A8W8_ERR_ALIGN
    assert _mx(name, a_s=18) == g.A8W8_ERR_ALIGN
    assert _mx(name, M=0, A=None, W=None) == g.A8W8_OK


@pytest.mark.parametrize("name", ["batched_gemm_a8w8_mxscale", "batched_gemm_a8w8_mxscale_packed"])
def test_mx_batched_entries_check_arguments(name):
    assert _mx(name, batch=-1) == g.A8W8_ERR_SHAPE
    assert _mx(name, batch=65536) == g.A8W8_ERR_SHAPE
    assert _mx(name, batch=0, A=None, W=None) == g.A8W8_OK     # empty batch: no-op
    assert _mx(name, batch=8, M=0, A=None) == g.A8W8_OK
    assert _mx(name, batch=8, K=200) == g.A8W8_ERR_SHAPE
    assert _mx(name, batch=8, Y=None) == g.A8W8_ERR_NULL


def test_mx_weight_scale_rows_limit():
    # ceil(N/32) * K/128 * 4 must stay below 2^31 (32-bit scale descriptors).
    assert _mx(N=1 << 30, K=1 << 14) == g.A8W8_ERR_SHAPE
    assert g.lib().gemm_a8w8_mxscale_plan(16, 1 << 30, 1 << 14, 0, ctypes.byref(g.Plan())) == g.A8W8_ERR_SHAPE


def test_mx_run_variant_rejects_like_block_scale():
    skinny = next(i for i in range(g.gemm_a8w8_num_variants())
                  if g.gemm_a8w8_describe_variant(i)["kernel_name"] == "skinny")
    rc = g.lib().gemm_a8w8_mxscale_run_variant(skinny, 16, 16, 16, 16, 16, 1, 17, 512, 1024, 0, None)
    assert rc == g.A8W8_ERR_PLAN
    assert g.lib().gemm_a8w8_mxscale_run_variant(-1, 16, 16, 16, 16, 16, 1, 4, 512, 1024, 0, None) == g.A8W8_ERR_PLAN


# The page's MX shapes (dense, and the batched N=1024, K=4096 one).
REGISTERED_MX = [(1792, 5120), (4608, 5120), (5120, 2304), (5120, 8192), (32768, 1280), (1024, 4096)]


@pytest.mark.parametrize("N,K", REGISTERED_MX)
def test_mx_every_m_has_a_tuned_plan_within_125_percent(N, K):
    assert (N, K) in _table_shapes(mx=True)
    for M in range(1, 8193):
        p = g.gemm_a8w8_mxscale_plan(M, N, K)
        assert p["fallback"] == 0, (M, p)
        assert M <= p["key_m"] <= 1.25 * M, (M, p)
        if M <= 16:
            assert p["key_m"] == M
        if p["kernel_name"] in ("skinny", "pskinny", "rskinny"):
            assert M <= 16


def test_mx_and_block_scale_tables_are_separate():
    # A block-scale table does not serve the MX variant (and the reverse).
    for N, K in _table_shapes(mx=False):
        if (N, K) not in REGISTERED_MX:
            assert g.gemm_a8w8_mxscale_plan(100, N, K)["fallback"] == 1
    for N, K in REGISTERED_MX:
        if (N, K) not in _table_shapes(mx=False):
            assert g.gemm_a8w8_blockscale_plan(100, N, K)["fallback"] == 1


@pytest.mark.parametrize("M,N,K", [(48, 1000, 5120), (3000, 5000, 2304), (100, 20, 4096), (7, 640, 1024)])
def test_mx_unregistered_shape_gets_a_valid_heuristic_plan(M, N, K):
    p = g.gemm_a8w8_mxscale_plan(M, N, K)
    assert p["fallback"] == 1 and p["key_m"] == M
    assert 0 <= p["variant"] < g.gemm_a8w8_num_variants()
    if p["kernel_name"] in ("skinny", "pskinny", "rskinny"):
        assert M <= 16
    if p["kernel_name"] == "tall":
        assert N <= p["bn"]


# ---------------------------------------------------------------- row-wise entries

def _rw(name="gemm_a8w8_rowwise", A=16, a_s=16, W=16, w_s=16, Y=16, M=4, N=512, K=1024):
    return getattr(g.lib(), name)(A, a_s, W, w_s, Y, M, N, K, None)


@pytest.mark.parametrize("name", ["gemm_a8w8_rowwise", "gemm_a8w8_rowwise_packed"])
def test_rowwise_entries_check_arguments(name):
    assert _rw(name, K=100) == g.A8W8_ERR_SHAPE
    assert _rw(name, N=0) == g.A8W8_ERR_SHAPE
    assert _rw(name, M=-3) == g.A8W8_ERR_SHAPE
    assert _rw(name, a_s=None) == g.A8W8_ERR_NULL
    assert _rw(name, Y=None) == g.A8W8_ERR_NULL
    assert _rw(name, A=8) == g.A8W8_ERR_ALIGN
    assert _rw(name, w_s=6) == g.A8W8_ERR_ALIGN
    assert _rw(name, M=0, A=None, a_s=None) == g.A8W8_OK


def test_rowwise_run_variant_rejects_like_block_scale():
    skinny = next(i for i in range(g.gemm_a8w8_num_variants())
                  if g.gemm_a8w8_describe_variant(i)["kernel_name"] == "skinny")
    L = g.lib()
    assert L.gemm_a8w8_rowwise_run_variant(skinny, 16, 16, 16, 16, 16, 17, 512, 1024, 0, None) == g.A8W8_ERR_PLAN
    assert L.gemm_a8w8_rowwise_run_variant(10 ** 6, 16, 16, 16, 16, 16, 4, 512, 1024, 0, None) == g.A8W8_ERR_PLAN


# ---------------------------------------------------------------- split-K instances

def test_split_instances_need_two_k_blocks_per_split():
    L = g.lib()
    for v in g.variants():
        if v["splits"] > 1:
            small_k = 128 * (2 * v["splits"] - 1)
            M = 16 if v["kernel_name"] == "skinny" else 64
            assert L.gemm_a8w8_blockscale_run_variant(v["variant"], 16, 16, 16, 16, 16, M, 512, small_k,
                                                      None) == g.A8W8_ERR_PLAN, v["name"]
            d = g.gemm_a8w8_describe_variant(v["variant"], M, 1000, 128 * 4 * v["splits"])
            per_pass = v["waves"] * v["kblocks"] if v["kernel_name"] == "skinny" else 1
            assert d["kpasses"] == -(-4 // per_pass), v["name"]
            assert d["grid"] == -(-M // v["bm"]) * -(-1000 // v["bn"]) * v["splits"], v["name"]


def test_split_instances_beyond_the_workspace_cap_are_rejected():
    v = next(v for v in g.variants() if v["splits"] == 8)
    # 8 splits x (M x N) fp32 partials far above 128 MB
    rc = g.lib().gemm_a8w8_blockscale_run_variant(v["variant"], 16, 16, 16, 16, 16, 8192, 8192, 4096, None)
    assert rc == g.A8W8_ERR_PLAN


def test_rskinny_instances_split_rows_evenly_or_refuse():
    """Row-range skinny instances take a shape only when every workgroup's run of rows fits their
    tiles (row-major runs of 4-row units, packed runs of 16-row tiles), at the device's CU count."""
    rs = [v for v in g.variants() if v["kernel_name"] == "rskinny"]
    assert rs
    for v in rs:
        T = v["bn"] // 16
        wpc = g.gemm_a8w8_describe_variant(v["variant"], 1, 1 << 20, 1024)["grid"] // 256
        for N in (64, 300, 5120, 5122, 14336, 16384, 34816):
            for cus in (256, 80):
                G4 = min(-(-N // 4), cus * wpc)
                G16 = min(-(-N // 16), cus * wpc)
                fits = 4 * -(-(-(-N // 4)) // G4) <= 16 * T and 16 * -(-(-(-N // 16)) // G16) <= 16 * T
                p = g.Plan()
                d = g.GemmDesc(None, None, None, None, None, 1, 8, N, 1024, 0, 0, v["variant"], 0, None, 0)
                rc = g.lib().gemm_a8w8_ex_plan(ctypes.byref(d), cus, ctypes.byref(p))
                assert (rc == g.A8W8_OK) == fits, (v["name"], N, cus, rc)
                if fits:
                    assert p.grid == G4
        assert g.lib().gemm_a8w8_ex_plan(ctypes.byref(g.GemmDesc(None, None, None, None, None, 1, 17, 5120, 1024,
                                                                  0, 0, v["variant"], 0, None, 0)), 0,
                                         ctypes.byref(g.Plan())) == g.A8W8_ERR_PLAN     # M > 16


def test_plans_report_splits():
    for M, N, K in ((1, 14336, 5120), (8192, 14336, 5120)):
        assert g.gemm_a8w8_blockscale_plan(M, N, K)["splits"] >= 1


@pytest.mark.parametrize("N,K", REGISTERED)
def test_plain_entry_never_splits_and_ex_follows_the_table(N, K):
    """The plain entry's plan never needs a workspace: it runs the row's instance when that needs
    none at this M (a stream-K row whose grid cuts no tile), else the row's unsplit instance;
    gemm_a8w8_ex with room for the workspace runs the row's instance, with less room the unsplit
    one."""
    rows = {int(r["key_m"]): r for s in gst.load()["shapes"]
            if (int(s["n"]), int(s["k"])) == (N, K) and gst.form_of(s) == "block" for r in s["rows"]}
    keys = sorted(rows)
    for M in list(range(1, 200)) + list(range(200, 8193, 37)):
        key = next(k for k in keys if k >= M)
        r = rows[key]
        u = gst.unsplit_of(r)
        p = g.gemm_a8w8_blockscale_plan(M, N, K)
        e = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=BIG_WS)
        want = r["name"] if e["workspace"] == 0 else u["name"]
        assert p["splits"] == 1 and p["workspace"] == 0 and p["name"] == want, (M, p["name"], want)
        assert e["name"] == r["name"] and e["key_m"] == key, (M, e["name"], r["name"])
        # a split row always needs its workspace; a stream-K row needs one when it cuts a tile at this M
        if int(r.get("splits", 1)) > 1:
            assert e["workspace"] > 0
        if e["workspace"] > 0:
            assert gst.cuts_k(r), (M, r["name"])
        if e["workspace"] > 0:
            assert g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=e["workspace"] - 1)["name"] == u["name"]


@pytest.mark.parametrize("form", ["packed", "rowwise"])
def test_decode_form_tables_serve_m_up_to_16_and_block_table_above(form):
    """Packed-weight and row-wise calls take their own decode table (exact keys 1..16) where one
    is tuned, and the block-scale table's plan for every other M."""
    shapes = _table_shapes(form=form)
    if not shapes:
        pytest.skip(f"no {form} tables")
    kind = "rowwise" if form == "rowwise" else "block"
    packed = form == "packed"
    for N, K in shapes:
        rows = {int(r["key_m"]): r for s in gst.load()["shapes"]
                if (int(s["n"]), int(s["k"])) == (N, K) and gst.form_of(s) == form for r in s["rows"]}
        assert sorted(rows) == list(range(1, 17))
        for M in range(1, 17):
            e = g.gemm_a8w8_ex_plan(M, N, K, scale_kind=kind, packed=packed, workspace_bytes=BIG_WS)
            assert e["fallback"] == 0 and e["key_m"] == M and e["name"] == rows[M]["name"], (N, K, M, e["name"])
        for M in list(range(17, 300, 7)) + [1024, 4097, 8192]:
            e = g.gemm_a8w8_ex_plan(M, N, K, scale_kind=kind, packed=packed, workspace_bytes=BIG_WS)
            b = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=BIG_WS)
            assert (e["name"], e["key_m"], e["fallback"]) == (b["name"], b["key_m"], 0), (N, K, M)
    # a row-wise call with packed weights takes the row-wise table; MX calls never take these tables
    for N, K in shapes:
        if form == "rowwise":
            assert g.gemm_a8w8_ex_plan(3, N, K, scale_kind="rowwise", packed=True)["name"] == \
                g.gemm_a8w8_ex_plan(3, N, K, scale_kind="rowwise")["name"]


def test_table_validation_of_decode_forms():
    rows = [{"key_m": m, "kernel": "skinny", "bm": 16, "bn": 16, "waves": 4} for m in range(1, 17)]
    gst.validate({"shapes": [{"n": 64, "k": 128, "form": "packed", "rows": rows}]})
    with pytest.raises(ValueError):                           # a decode table stops at 16
        gst.validate({"shapes": [{"n": 64, "k": 128, "form": "packed",
                                  "rows": rows + [{"key_m": 20, "kernel": "tile", "bm": 32, "bn": 32, "waves": 4}]}]})
    with pytest.raises(ValueError):                           # ... and covers every M up to 16
        gst.validate({"shapes": [{"n": 64, "k": 128, "form": "rowwise", "rows": rows[:8]}]})
    with pytest.raises(ValueError):
        gst.validate({"shapes": [{"n": 64, "k": 128, "form": "other", "rows": rows}]})


def _desc(**kw):
    d = dict(A=16, a_scale=16, W=16, w_scale=16, Y=16, batch=1, M=64, N=512, K=1024, scale_kind=0,
             w_packed=0, variant=-1, reserved=0, workspace=None, workspace_bytes=0)
    d.update(kw)
    return g.GemmDesc(*(d[f] for f, _ in g.GemmDesc._fields_))


def test_ex_entry_checks_arguments():
    L = g.lib()
    ex = lambda **kw: L.gemm_a8w8_ex(ctypes.byref(_desc(**kw)), None)
    assert L.gemm_a8w8_ex(None, None) == g.A8W8_ERR_NULL
    assert L.gemm_a8w8_ex_plan(None, 0, ctypes.byref(g.Plan())) == g.A8W8_ERR_NULL
    assert ex(K=1000) == g.A8W8_ERR_SHAPE
    assert ex(batch=-1) == g.A8W8_ERR_SHAPE
    assert ex(scale_kind=3) == g.A8W8_ERR_SHAPE
    assert ex(w_packed=2) == g.A8W8_ERR_SHAPE
    assert ex(workspace_bytes=4096) == g.A8W8_ERR_WORKSPACE       # a size without memory
    assert ex(workspace=256, workspace_bytes=-256) == g.A8W8_ERR_WORKSPACE
    assert ex(workspace=272, workspace_bytes=4096) == g.A8W8_ERR_ALIGN
    assert ex(A=None) == g.A8W8_ERR_NULL
    assert ex(M=0, A=None, Y=None) == g.A8W8_OK
    assert ex(batch=0, A=None) == g.A8W8_OK
    assert ex(variant=10 ** 6) == g.A8W8_ERR_PLAN
    split = next(v for v in g.variants() if v["splits"] > 1 and v["kernel_name"] == "tile")
    need = g.gemm_a8w8_describe_variant(split["variant"], 64, 512, 1024)["workspace"]
    assert need > 0
    # a forced split instance without enough workspace is refused before any device call
    assert ex(variant=split["variant"]) == g.A8W8_ERR_WORKSPACE
    assert ex(variant=split["variant"], workspace=256, workspace_bytes=need - 256) == g.A8W8_ERR_WORKSPACE
    assert L.gemm_a8w8_blockscale_run_variant(split["variant"], 16, 16, 16, 16, 16, 64, 512, 1024,
                                              None) == g.A8W8_ERR_WORKSPACE
    p = g.Plan()
    assert L.gemm_a8w8_ex_plan(ctypes.byref(_desc(variant=split["variant"])), 0, ctypes.byref(p)) == \
        g.A8W8_ERR_WORKSPACE
    assert L.gemm_a8w8_ex_plan(ctypes.byref(_desc(variant=split["variant"], workspace_bytes=need)), 0,
                               ctypes.byref(p)) == g.A8W8_OK
    assert p.workspace == need and p.variant == split["variant"]


def test_workspace_init_checks_arguments():
    L = g.lib()
    assert L.gemm_a8w8_workspace_init(None, 0, None) == g.A8W8_OK
    assert L.gemm_a8w8_workspace_init(256, -256, None) == g.A8W8_ERR_SHAPE
    assert L.gemm_a8w8_workspace_init(None, 256, None) == g.A8W8_ERR_NULL
    assert L.gemm_a8w8_workspace_init(272, 256, None) == g.A8W8_ERR_ALIGN
    assert L.gemm_a8w8_workspace_init(256, 300, None) == g.A8W8_ERR_ALIGN


def test_workspace_size_covers_counters_and_partials():
    for v in g.variants():
        if v["splits"] > 1:
            for M, N in ((64, 512), (300, 1000), (16, 32)):
                d = g.gemm_a8w8_describe_variant(v["variant"], M, N, 4096)
                tiles = -(-M // v["bm"]) * -(-N // v["bn"])
                assert d["workspace"] == 65536 + tiles * v["splits"] * v["bm"] * v["bn"] * 4


# ---------------------------------------------------------------- benchmark read-ceiling kernel

def test_ceilings_library_builds_and_checks_arguments():
    # The benchmark's streaming-read and MFMA kernels live in a library of their own; bad
    # arguments are refused before anything is launched.
    import ctypes
    import os
    from fp8_block_scaled_a8w8_amd import build as libbuild
    if not os.path.exists(libbuild.CEILINGS_LIB):
        libbuild.build_ceilings()
    lib = ctypes.CDLL(libbuild.CEILINGS_LIB)
    mf = lib.a8w8_mfma_ceiling_launch
    mf.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    mf.restype = ctypes.c_int
    for args in ((None, 4, 16, 8, 10), (16, 1, 16, 8, 10), (16, 4, None, 8, 10), (16, 4, 16, 0, 10),
                 (16, 4, 16, 8, 0)):
        assert mf(*args, None) != 0, args
    fl = lib.a8w8_mfma_ceiling_flops
    fl.argtypes = [ctypes.c_int, ctypes.c_int]
    fl.restype = ctypes.c_double
    assert fl(512, 1000) == 512 * 4 * 1000 * 8 * 16 * 16 * 128 * 2
    fn = lib.a8w8_read_ceiling_launch
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    for args in ((16, 1000, 16, 8, 8), (16, 1024, None, 8, 8), (None, 1024, 16, 8, 8), (16, 1024, 16, 0, 8),
                 (16, 1024, 16, 8, 4), (16, 0, 16, 8, 16)):
        assert fn(*args, None) != 0, args
    cap = lib.a8w8_cu_capacity_launch
    cap.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                    ctypes.c_void_p]
    cap.restype = ctypes.c_int
    for args in ((3, 16, 1 << 20, 16, 8, 8), (0, None, 0, None, 8, 8), (1, None, 1 << 20, 16, 8, 8),
                 (1, 16, 3 << 20, 16, 8, 8), (2, 16, 1 << 12, 16, 8, 8), (2, 16, 1 << 29, 16, 8, 8),
                 (1, 16, 1 << 20, 16, 0, 8), (0, None, 0, 16, 8, 0)):
        assert cap(*args, None) != 0, args
    nb = lib.a8w8_cu_capacity_bytes
    nb.argtypes = [ctypes.c_int]
    nb.restype = ctypes.c_double
    assert nb(10) == 16 * 64 * 16 * 8 * 10


def test_instance_parameters_identify_instances():
    """The selector table names an instance by (kernel, bm, bn, waves, kblocks, splits): no two
    compiled instances may share that key."""
    keys = {}
    for v in g.variants():
        k = (v["kernel"], v["bm"], v["bn"], v["waves"], v["kblocks"], v["splits"])
        assert k not in keys, (v["name"], keys.get(k))
        keys[k] = v["name"]
