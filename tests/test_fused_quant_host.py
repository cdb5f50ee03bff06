"""Host-side checks of the fused quantise-and-multiply entry (decode, M <= 16):
argument errors, and the plan rule over the row-range skinny instances.  Nothing
here launches a kernel."""
from __future__ import annotations

import ctypes

import pytest

import fp8_block_scaled_a8w8_amd as g

CUS = 256


def _fused(X=16, W=16, w_s=16, Y=16, M=4, N=512, K=1024, packed=0, variant=-1):
    return g.lib().gemm_a8w8_blockscale_fused_quant(X, W, w_s, Y, M, N, K, packed, variant, None)


def _plan(M, N, K, variant=-1, cus=CUS):
    p = g.Plan()
    rc = g.lib().gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cus, variant, ctypes.byref(p))
    return rc, p


def test_m_zero_is_a_no_op_and_shapes_are_checked():
    assert _fused(None, None, None, None, M=0) == g.A8W8_OK
    for M, N, K in ((17, 512, 1024), (-1, 512, 1024), (4, 0, 1024), (4, 512, 1000), (4, 512, (1 << 22) + 128)):
        assert _fused(M=M, N=N, K=K) == g.A8W8_ERR_SHAPE, (M, N, K)
        assert _plan(M, N, K)[0] == g.A8W8_ERR_SHAPE, (M, N, K)
    assert _fused(packed=2) == g.A8W8_ERR_SHAPE


@pytest.mark.parametrize("which", ["X", "W", "w_s", "Y"])
def test_null_pointers(which):
    assert _fused(**{which: None}) == g.A8W8_ERR_NULL


@pytest.mark.parametrize("kw", [{"X": 24}, {"W": 8}, {"w_s": 2}, {"Y": 17}])
def test_misaligned_pointers(kw):
    assert _fused(**kw) == g.A8W8_ERR_ALIGN


def test_forced_instance_must_be_row_range_skinny():
    other = [v["variant"] for v in g.variants() if v["kernel_name"] != "rskinny"]
    for vid in other[:5]:
        assert _fused(variant=vid) == g.A8W8_ERR_PLAN
        assert _plan(4, 512, 1024, variant=vid)[0] == g.A8W8_ERR_PLAN
    assert _fused(variant=g.gemm_a8w8_num_variants()) == g.A8W8_ERR_PLAN


def test_rows_beyond_the_row_range_instances_are_refused():
    # 34816 rows over 256 CUs: 136 rows per workgroup, past the largest instance's 64
    assert _plan(1, 34816, 5120)[0] == g.A8W8_ERR_PLAN


def _rskinny():
    return [v for v in g.variants() if v["kernel_name"] == "rskinny"]


@pytest.mark.parametrize("N,K", [(5120, 6144), (14336, 5120), (5120, 17408), (300, 1024), (130, 256)])
def test_plan_rule_fewest_passes_then_most_waves_then_widest(N, K):
    for M in (1, 2, 4, 8, 9, 16):
        rc, p = _plan(M, N, K)
        assert rc == g.A8W8_OK
        d = p.as_dict()
        assert d["kernel_name"] == "rskinny" and d["workspace"] == 0 and d["splits"] == 1
        cands = []
        for v in _rskinny():
            rcv, pv = _plan(M, N, K, variant=v["variant"])
            if rcv == g.A8W8_OK:
                cands.append((-pv.kpasses, v["waves"], v["bn"], v["variant"]))
        best = max(cands)
        assert (-d["kpasses"], d["waves"], d["bn"]) == best[:3], (M, N, K, d, cands)


def test_decode_plans():
    # the instances measured fastest among the fused ones (out_proj, qkv)
    name = lambda M, N, K: g.gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count=CUS)["name"]
    assert name(1, 5120, 6144) == "rskinny_t2_d3_w16_g1"
    assert name(16, 14336, 5120) == "rskinny_t4_d5_w8_g1"
