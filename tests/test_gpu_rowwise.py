"""GPU parity tests of the row-wise (per-token / per-channel) GEMM
(gemm_a8w8_rowwise and its packed form) against ``oracle.gemm_rowwise``.

Every compiled instance on ragged shapes (row-major and packed, bitwise
equal to each other), the selector path at the decode and prefill shapes on
sampled rows, an integer case bitwise, and zero scales.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, shared_workspace, variant_by_name, variant_names, y_bits, y_host
from tests.parity_util import assert_parity, bf16_round

pytestmark = pytest.mark.gpu


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


def _operands(M, N, K, seed):
    A, a = inputgen.make_rowwise_activations(M, K, seed=seed)
    W, w = inputgen.make_rowwise_weights(N, K, seed=seed + 1)
    return A, a, W, w


def _rows(M):
    return sorted({0, 1 % M, M // 3, M // 2, M - 1})


def _shape_for(v, cus):
    k = v["kernel_name"]
    if k == "skinny":
        return 9, 300
    if k == "rskinny":
        return 9, 20 * cus + 2
    if k == "pskinny":
        return 9, 16 * (2 * cus + 37) + 5
    if k == "tall":
        return 3 * v["bm"] + 5, v["bn"] - 3
    per_cu = g.gemm_a8w8_describe_variant(v["variant"], 1 << 24, 1 << 16, 640)["grid"] // 256
    N = 3 * v["bn"] + 40
    tiles_n = (N + v["bn"] - 1) // v["bn"]
    tiles_m = (2 * cus * max(per_cu, 1) + tiles_n - 1) // tiles_n + 1 if k in ("ptile", "sktile") else 3
    return tiles_m * v["bm"] - v["bm"] // 2 - 3, N


@pytest.mark.parametrize("name", variant_names())
def test_every_instance_rowwise(name):
    v = variant_by_name(name)
    variant = v["variant"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = max(640, 256 * v["splits"])   # split-K instances need >= 2 K blocks per split
    M, N = _shape_for(v, cus)
    A, a, W, w = _operands(M, N, K, seed=2000 + variant)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"rowwise {v['name']} M={M} N={N} K={K}")
    y = g.gemm_a8w8_rowwise_run_variant(variant, dA, da, dW, dw, workspace=shared_workspace())
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_rowwise(A, a, W, w, rows=rows), f"rowwise {v['name']}")
    yp = g.gemm_a8w8_rowwise_run_variant(variant, dA, da, g.prepack_weights(dW), dw, packed_n=N, workspace=shared_workspace())
    assert np.array_equal(y_bits(yp), y_bits(y)), f"rowwise packed {v['name']}"


@pytest.mark.parametrize("M,N,K", [(1, 14336, 5120), (16, 14336, 5120), (100, 14336, 5120), (2048, 14336, 5120),
                                   (9, 34816, 5120), (700, 5120, 6144), (3000, 32, 6144), (77, 256, 6144)])
def test_selector_shapes_rowwise(M, N, K):
    A, a, W, w = _operands(M, N, K, seed=M + N)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"rowwise selector M={M} N={N} K={K}")
    y = g.gemm_a8w8_rowwise(dA, da, dW, dw)
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_rowwise(A, a, W, w, rows=rows), f"rowwise M={M} N={N}")
    yp = g.gemm_a8w8_rowwise_packed(dA, da, g.prepack_weights(dW), dw, N)
    assert np.array_equal(y_bits(yp), y_bits(y))


def test_integer_case_bitwise():
    # Values in {-1, 0, +1} and power-of-two scales: the fp32 dot is exact and the
    # two scale products are exact, so every instance gives bf16(Y_ref) bit for bit.
    rng = np.random.default_rng(11)
    M, N, K = 41, 200, 512
    A = rng.choice(np.array([0x38, 0xB8, 0x00], np.uint8), size=(M, K))
    W = rng.choice(np.array([0x38, 0xB8, 0x00], np.uint8), size=(N, K))
    a = np.ldexp(np.float32(1), rng.integers(-5, 6, size=M)).astype(np.float32)
    w = np.ldexp(np.float32(1), rng.integers(-9, 2, size=N)).astype(np.float32)
    dA, da, dW, dw = _dev(A, a, W, w)
    ref = bf16_round(oracle.gemm_rowwise(A, a, W, w))
    for vid in range(g.gemm_a8w8_num_variants()):
        v = g.gemm_a8w8_describe_variant(vid)
        if v["kernel_name"] in ("skinny", "pskinny", "rskinny") or (v["kernel_name"] == "tall" and v["bn"] < N) \
                or K // 128 < 2 * v["splits"]:
            continue
        y = y_host(g.gemm_a8w8_rowwise_run_variant(vid, dA, da, dW, dw, workspace=shared_workspace()))
        assert np.array_equal(y, ref), v["name"]
    y = y_host(g.gemm_a8w8_rowwise(dA[:9].contiguous(), da[:9].contiguous(), dW, dw))
    assert np.array_equal(y, ref[:9])


def test_zero_scales_give_zero_rows_and_columns():
    M, N, K = 20, 300, 384
    A, a, W, w = _operands(M, N, K, seed=5)
    a[3] = 0
    w[17] = 0
    dA, da, dW, dw = _dev(A, a, W, w)
    for Ms in (M, 9):
        y = y_host(g.gemm_a8w8_rowwise(dA[:Ms].contiguous(), da[:Ms].contiguous(), dW, dw))
        assert np.all(y[3] == 0) and np.all(y[:, 17] == 0)
        ref = oracle.gemm_rowwise(A[:Ms], a[:Ms], W, w)
        assert_parity(y, ref, f"rowwise zero scales M={Ms}")


@pytest.mark.parametrize("M,N,K", [(5, 1000, 3072), (100, 1000, 3072), (1500, 640, 1024), (300, 24, 2048)])
def test_unregistered_shapes_use_the_heuristic_plan(M, N, K):
    assert g.gemm_a8w8_blockscale_plan(M, N, K)["fallback"] == 1
    A, a, W, w = _operands(M, N, K, seed=M + N)
    y = g.gemm_a8w8_rowwise(*_dev(A, a, W, w))
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_rowwise(A, a, W, w, rows=rows), "rowwise heuristic")
