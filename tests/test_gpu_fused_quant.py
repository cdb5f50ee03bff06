"""GPU tests of the fused quantise-and-multiply entry (gemm_a8w8_blockscale_fused_quant, M <= 16).

Its result must equal a8w8_quantize_1x128 followed by the GEMM with the same instance bit for
bit: the codes are integers and the scales exact fp32 values decided by the same arithmetic, and
the GEMM then sums the same products in the same order.  It must also meet the parity bar against
the oracle, oracle.quantize_1x128 then oracle.gemm (both pinned in the oracle tests).  Covered:
every row-range skinny instance; every rows-per-block width the kernel quantises with (M = 1, 2,
3, 4, 5, 8, 9, 16 take MQ = 1, 2, 4, 4, 8, 8, 16, 16); both weight layouts; ragged N and several
passes over K; groups at the encoder's edge cases; the plan at every M on the decode shapes; and
graph replay.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, variant_names, variant_by_name, y_bits, y_host
from tests.parity_util import assert_parity
from tests.test_gpu_quant import _edge_rows

pytestmark = pytest.mark.gpu

RSKINNY = variant_names(kinds=("rskinny",))
MS = (1, 2, 3, 4, 5, 8, 9, 16)
_REF = {}


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _problem(N, K, seed):
    """16 activation rows (bf16, on the device), weights, and the oracle's Y for all 16 rows
    (row m of Y depends on row m of X only, so Y[:M] serves every M)."""
    key = (N, K, seed)
    if key not in _REF:
        x = inputgen.normal_bf16(16, K, 1.0, seed=seed)
        W, w_s = inputgen.make_weights(N, K, seed=seed + 1)
        A, a_s = oracle.quantize_1x128(x.numpy())
        ref = oracle.gemm(A, a_s, W, w_s)
        _REF[key] = (x.to(torch.bfloat16).to(DEV), torch.from_numpy(W).to(DEV), torch.from_numpy(w_s).to(DEV), ref)
    return _REF[key]


def _two_kernel(vid, X, dW, dw, packed_n=None):
    q, s = g.quantize_1x128(X)
    if packed_n is None:
        return g.gemm_a8w8_blockscale_run_variant(vid, q, s, dW, dw)
    return g.gemm_a8w8_blockscale_packed_run_variant(vid, q, s, dW, dw, packed_n)


def _accepts(vid, M, N, K):
    try:
        g.gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count=_cus(), variant=vid)
        return True
    except g.A8W8Error:
        return False


@pytest.mark.parametrize("name", RSKINNY)
def test_fused_instance_equals_quantise_then_gemm(name):
    vid = variant_by_name(name)["variant"]
    cus = _cus()
    ran = 0
    for (N, K) in ((20 * cus + 2, 640), (300, 1024), (5120, 6144), (14336, 5120), (130, 256), (20 * cus, 8192)):
        if not _accepts(vid, 16, N, K):
            continue
        X16, dW, dw, ref = _problem(N, K, seed=N + K)
        dWp = g.prepack_weights(dW)
        for M in MS:
            X = X16[:M]
            y = g.gemm_a8w8_blockscale_fused_quant(X, dW, dw, variant=vid)
            two = _two_kernel(vid, X, dW, dw)
            assert np.array_equal(y_bits(y), y_bits(two)), f"{name} N={N} K={K} M={M}: fused != quantise+gemm"
            assert_parity(y_host(y), ref[:M], f"{name} fused N={N} K={K} M={M}")
            yp = g.gemm_a8w8_blockscale_fused_quant(X, dWp, dw, packed_n=N, variant=vid)
            assert np.array_equal(y_bits(yp), y_bits(y)), f"{name} N={N} K={K} M={M}: packed differs"
        say(f"{name} N={N} K={K}: M in {MS} bitwise = quantise+gemm, oracle parity ok")
        ran += 1
    assert ran >= 2, f"{name}: too few shapes accepted"


@pytest.mark.parametrize("N,K", [(5120, 6144), (14336, 5120)])
def test_fused_plan_every_m_on_decode_shapes(N, K):
    X16, dW, dw, ref = _problem(N, K, seed=7)
    for M in range(1, 17):
        plan = g.gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count=_cus())
        y = g.gemm_a8w8_blockscale_fused_quant(X16[:M], dW, dw)
        two = _two_kernel(plan["variant"], X16[:M], dW, dw)
        assert np.array_equal(y_bits(y), y_bits(two)), f"plan {plan['name']} N={N} K={K} M={M}"
        assert_parity(y_host(y), ref[:M], f"fused plan N={N} K={K} M={M}")
    say(f"fused plan N={N} K={K}: M = 1..16 ok")


@pytest.mark.parametrize("K", [256, 1024])
def test_fused_edge_groups(K):
    """Zero groups, bf16 subnormals (subnormal scales: IEEE division path), a single large value,
    huge magnitudes, negative zeros, alternating +-448: alone (M = 1), as 8 rows, and under 8
    normal rows (M = 16)."""
    N = 200
    edge = _edge_rows(K, seed=K)
    W, w_s = inputgen.make_weights(N, K, seed=3)
    dW, dw = torch.from_numpy(W).to(DEV), torch.from_numpy(w_s).to(DEV)
    rows = torch.cat([edge, inputgen.normal_bf16(8, K, 1.0, seed=K + 1)])
    cases = [rows[i:i + 1] for i in range(8)] + [rows[:8], rows]
    for x in cases:
        M = x.shape[0]
        X = x.to(torch.bfloat16).to(DEV)
        plan = g.gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count=_cus())
        y = g.gemm_a8w8_blockscale_fused_quant(X, dW, dw)
        two = _two_kernel(plan["variant"], X, dW, dw)
        assert np.array_equal(y_bits(y), y_bits(two)), f"edge K={K} M={M}"
        A, a_s = oracle.quantize_1x128(x.numpy())
        ref = oracle.gemm(A, a_s, W, w_s)
        # The oracle bar holds where every a_scale * w_scale product is an fp32 normal
        # (or 0): the bf16-subnormal row's products lie below 2^-126, where fp32 keeps
        # only a few bits and the kernel's scale product rounds to a handful of ulps.
        # Those rows are held to the bitwise check above (and their codes to the
        # quantisation tests).
        normal = np.all((a_s == 0) | (a_s.astype(np.float64) * float(w_s.min()) >= 2.0 ** -126), axis=1)
        if normal.any():
            assert_parity(y_host(y)[normal], ref[normal], f"edge K={K} M={M}")
    say(f"fused edge groups K={K} ok")


def test_fused_graph_replay_matches_eager():
    cases = []
    for (M, N, K) in ((1, 5120, 6144), (6, 300, 1024), (16, 14336, 5120)):
        X16, dW, dw, _ = _problem(N, K, seed=11)
        X = X16[:M].clone()
        eager = y_bits(g.gemm_a8w8_blockscale_fused_quant(X, dW, dw))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        cases.append((X, dW, dw, out, eager))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for X, dW, dw, out, _ in cases:
            g.gemm_a8w8_blockscale_fused_quant(X, dW, dw, out=out, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        for X, dW, dw, out, _ in cases:
            g.gemm_a8w8_blockscale_fused_quant(X, dW, dw, out=out, stream=s)
    for rep in range(3):
        for *_, out, _ in cases:
            out.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for *_, out, eager in cases:
            assert np.array_equal(y_bits(out), eager), f"replay {rep}"


def test_fused_empty_and_refusals():
    X = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    W = torch.zeros((64, 256), dtype=torch.uint8, device=DEV)
    w = torch.ones((1, 2), dtype=torch.float32, device=DEV)
    assert g.gemm_a8w8_blockscale_fused_quant(X, W, w).shape == (0, 64)
    with pytest.raises(g.A8W8Error):
        g.gemm_a8w8_blockscale_fused_quant(torch.zeros((17, 256), dtype=torch.bfloat16, device=DEV), W, w)
