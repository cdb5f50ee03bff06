"""GPU parity tests of the MX-scaled GEMM (gemm_a8w8_mxscale and its batched
and packed forms) against the fp64 oracle ``oracle.gemm_mx``.

The variant is the mxfp8 GEMM with 32 x 32 weight-scale blocks, dense and
batched (b = 8, N = 1024, K = 4096), of the gfx1250 BF16 and MX32 tuned-rows
page (ROCm/aiter #7247, Technical Details), read with OCP MX scales.  Every
compiled kernel instance is checked on ragged shapes with per-group scale
codes drawn over a wide range (a lane taking the wrong group's scale byte
would be off by powers of two); the selector path at the page's dense shapes
on sampled rows; the batched form in full; packed weights bitwise against
row-major; an integer case bitwise; NaN scale codes.
"""
from __future__ import annotations

import functools

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


def _wide_scales(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape, dtype=np.uint8)


def _mx_operands(M, N, K, seed, wide=True):
    A, a = inputgen.make_mx_activations(M, K, seed=seed)
    W, w = inputgen.make_mx_weights(N, K, seed=seed + 1)
    if wide:
        rng = np.random.default_rng(seed + 2)
        a = _wide_scales(rng, a.shape, 118, 136)
        w = _wide_scales(rng, w.shape, 112, 130)
    return A, a, W, w


def _rows(M, extra=()):
    return sorted({0, 1 % M, M // 3, M // 2, M - 2 if M > 1 else 0, M - 1, *extra})


def _shape_for(v, cus):
    k = v["kernel_name"]
    if k == "skinny":
        return 9, 300
    if k == "pskinny":
        return 9, 16 * (2 * cus + 37) + 5
    if k == "rskinny":
        return 9, 20 * cus + 2           # runs of 24 rows: tiles straddle 32-row scale blocks
    if k == "tall":
        return 3 * v["bm"] + 5, v["bn"] - 3
    per_cu = g.gemm_a8w8_describe_variant(v["variant"], 1 << 24, 1 << 16, 640)["grid"] // 256
    N = 3 * v["bn"] + 40
    tiles_n = (N + v["bn"] - 1) // v["bn"]
    tiles_m = (2 * cus * max(per_cu, 1) + tiles_n - 1) // tiles_n + 1 if k in ("ptile", "sktile") else 3
    return tiles_m * v["bm"] - v["bm"] // 2 - 3, N


@pytest.mark.parametrize("name", variant_names())
def test_every_instance_mx(name):
    v = variant_by_name(name)
    variant = v["variant"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = max(640, 256 * v["splits"])   # split-K instances need >= 2 K blocks per split
    M, N = _shape_for(v, cus)
    A, a, W, w = _mx_operands(M, N, K, seed=1000 + variant)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"mx {v['name']} M={M} N={N} K={K}")
    y = g.gemm_a8w8_mxscale_run_variant(variant, dA, da, dW, dw, workspace=shared_workspace())
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_mx(A, a, W, w, rows=rows), f"mx {v['name']}")
    yp = g.gemm_a8w8_mxscale_run_variant(variant, dA, da, g.prepack_weights(dW), dw, packed_n=N, workspace=shared_workspace())
    assert np.array_equal(y_bits(yp), y_bits(y)), f"mx packed {v['name']}"


@functools.lru_cache(maxsize=1)
def _page_weights(N, K):
    W, w = inputgen.make_mx_weights(N, K, seed=N + K)
    return W, w, _dev(W, w)


@pytest.mark.parametrize("N,K", [(1792, 5120), (4608, 5120), (5120, 2304), (5120, 8192), (32768, 1280)])
@pytest.mark.parametrize("M", [1, 16, 48, 300, 768])
def test_selector_page_dense_shapes(M, N, K):
    A, a = inputgen.make_mx_activations(M, K, seed=M)
    W, w, (dW, dw) = _page_weights(N, K)
    dA, da = _dev(A, a)
    plan = g.gemm_a8w8_mxscale_plan(M, N, K)
    say(f"mx selector M={M} N={N} K={K} -> {plan['name']}")
    y = g.gemm_a8w8_mxscale(dA, da, dW, dw)
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_mx(A, a, W, w, rows=rows), f"mx M={M} N={N} K={K}")
    yp = g.gemm_a8w8_mxscale_packed(dA, da, g.prepack_weights(dW), dw, N)
    assert np.array_equal(y_bits(yp), y_bits(y))


def _batched_operands(b, M, N, K, seed):
    parts = [_mx_operands(M, N, K, seed=seed + 10 * i, wide=False) for i in range(b)]
    return [np.stack([p[j] for p in parts]) for j in range(4)]


@pytest.mark.parametrize("M", [16, 48, 133])
def test_batched_page_shape_full(M):
    b, N, K = 8, 1024, 4096
    A, a, W, w = _batched_operands(b, M, N, K, seed=M)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"mx batched b={b} M={M} N={N} K={K}")
    y = g.batched_gemm_a8w8_mxscale(dA, da, dW, dw)
    ref = oracle.gemm_mx_batched(A, a, W, w)
    yh = y_host(y)
    for i in range(b):
        assert_parity(yh[i], ref[i], f"batch {i}")
    # every batch equals the unbatched call on its slice, bitwise
    for i in (0, b - 1):
        yi = g.gemm_a8w8_mxscale(dA[i], da[i], dW[i], dw[i])
        assert np.array_equal(y_bits(yi), y_bits(y[i]))
    # packed weights: each batch prepacked, bitwise equal
    dWp = torch.stack([g.prepack_weights(dW[i]) for i in range(b)])
    yp = g.batched_gemm_a8w8_mxscale_packed(dA, da, dWp, dw, N)
    assert np.array_equal(y_bits(yp), y_bits(y))


def test_batched_ragged_every_kernel_family():
    # One instance of each kernel family, batched over 3 problems of a ragged shape.
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    seen = set()
    for vid in range(g.gemm_a8w8_num_variants()):
        v = g.gemm_a8w8_describe_variant(vid)
        if v["kernel_name"] in seen:
            continue
        seen.add(v["kernel_name"])
        M, N = _shape_for(v, cus)
        if v["kernel_name"] in ("ptile", "sktile"):
            M = min(M, 3 * v["bm"] + 7)
        K = 384
        A, a, W, w = _batched_operands(3, M, N, K, seed=vid)
        dA, da, dW, dw = _dev(A, a, W, w)
        say(f"mx batched {v['name']} b=3 M={M} N={N} K={K}")
        y = g.gemm_a8w8_mxscale_run_variant(vid, dA, da, dW, dw, workspace=shared_workspace())
        yh = y_host(y)
        rows = _rows(M)
        for i in range(3):
            assert_parity(yh[i][rows], oracle.gemm_mx(A[i], a[i], W[i], w[i], rows=rows), f"{v['name']} batch {i}")
    assert seen == {"skinny", "pskinny", "tall", "tile", "ptile", "rskinny", "sktile"}


def test_integer_case_bitwise():
    # Values in {-1, 0, +1}, scale codes 125..129 (powers of two 1/4 .. 4): every
    # partial sum is a multiple of 2^-4 below 2^13, exact in fp32, so the GPU result
    # must be bf16(Y_ref) bit for bit.
    rng = np.random.default_rng(7)
    M, N, K = 37, 200, 512
    A = rng.choice(np.array([0x38, 0xB8, 0x00], np.uint8), size=(M, K))
    W = rng.choice(np.array([0x38, 0xB8, 0x00], np.uint8), size=(N, K))
    a = _wide_scales(rng, (M, K // 32), 125, 129)
    w = _wide_scales(rng, ((N + 31) // 32, K // 32), 125, 129)
    dA, da, dW, dw = _dev(A, a, W, w)
    ref = bf16_round(oracle.gemm_mx(A, a, W, w))
    for vid in range(g.gemm_a8w8_num_variants()):
        v = g.gemm_a8w8_describe_variant(vid)
        if v["kernel_name"] in ("skinny", "pskinny", "rskinny") or (v["kernel_name"] == "tall" and v["bn"] < N) \
                or K // 128 < 2 * v["splits"]:
            continue
        y = y_host(g.gemm_a8w8_mxscale_run_variant(vid, dA, da, dW, dw, workspace=shared_workspace()))
        assert np.array_equal(y, ref), v["name"]
    Ms = 9
    y = y_host(g.gemm_a8w8_mxscale(dA[:Ms].contiguous(), da[:Ms].contiguous(), dW, dw))
    assert np.array_equal(y, ref[:Ms])


def test_nan_scale_code_poisons_its_row():
    M, N, K = 20, 96, 256
    A, a, W, w = _mx_operands(M, N, K, seed=5, wide=False)
    a[4, 3] = 255
    dA, da, dW, dw = _dev(A, a, W, w)
    y = y_host(g.gemm_a8w8_mxscale(dA, da, dW, dw))
    assert np.all(np.isnan(y[4]))
    keep = [r for r in range(M) if r != 4]
    assert_parity(y[keep], oracle.gemm_mx(A, a, W, w, rows=keep), "rows without the NaN code")


def test_empty_calls_are_no_ops():
    K, N = 256, 64
    A, a, W, w = _mx_operands(4, N, K, seed=9, wide=False)
    dA, da, dW, dw = _dev(A, a, W, w)
    out = torch.full((0, 4, N), 1.0, dtype=torch.bfloat16, device=DEV)
    g.batched_gemm_a8w8_mxscale(dA[None][:0], da[None][:0], dW[None][:0], dw[None][:0], out=out)
    y = torch.full((0, N), 1.0, dtype=torch.bfloat16, device=DEV)
    g.gemm_a8w8_mxscale(dA[:0], da[:0], dW, dw, out=y)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(5, 1000, 3072), (100, 1000, 3072), (1500, 640, 1024), (300, 24, 2048)])
def test_unregistered_shapes_use_the_heuristic_plan(M, N, K):
    plan = g.gemm_a8w8_mxscale_plan(M, N, K)
    assert plan["fallback"] == 1
    A, a, W, w = _mx_operands(M, N, K, seed=M + N)
    y = g.gemm_a8w8_mxscale(*_dev(A, a, W, w))
    rows = _rows(M)
    assert_parity(y_host(y)[rows], oracle.gemm_mx(A, a, W, w, rows=rows), f"mx heuristic {plan['name']}")
