"""GPU tests of the packed weight layout (a8w8_prepack_weights, gemm_a8w8_blockscale_packed).

Every instance must compute on packed weights exactly what it computes on
row-major weights: the same kernels and accumulation order, so Y is compared
bitwise with the row-major run of the same instance, and against the oracle
to the parity bar.  The packed entry's own plan (its decode table on the
tuned decode shapes, the block-scale table elsewhere) is checked the same
way.  The layout itself
is checked byte for byte against a numpy permutation written from its
definition in include/gemm_a8w8_blockscale.h.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, shared_workspace, to_dev, variant_by_name, variant_names, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu


def _pack_reference(W: np.ndarray) -> np.ndarray:
    """The packed layout from its definition: per 16-row tile t and K block kb, [h][lane][16 bytes],
    lane l holding row 16t + l%16, columns 128kb + 16(l/16) + 64h .. +16; rows past N zero."""
    N, K = W.shape
    Np = (N + 15) // 16 * 16
    Wz = np.zeros((Np, K), np.uint8)
    Wz[:N] = W
    T, KB = Np // 16, K // 128
    # Wz[16t + r, 128kb + 64h + 16g + b] -> packed[t, kb, h, 16g + r, b]
    v = Wz.reshape(T, 16, KB, 2, 4, 16)                  # t, r, kb, h, g, b
    return np.ascontiguousarray(v.transpose(0, 2, 3, 4, 1, 5)).reshape(Np, K)


@pytest.mark.parametrize("N,K", [(16, 128), (300, 640), (5, 256), (14336, 5120)])
def test_prepack_layout_byte_exact(N, K):
    W, _ = inputgen.make_weights(N, K, seed=N)
    Wp = g.prepack_weights(torch.from_numpy(W).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(Wp.cpu().numpy(), _pack_reference(W))


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
def test_every_instance_packed_equals_row_major(name):
    v = variant_by_name(name)
    variant = v["variant"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = max(640, 256 * v["splits"])   # split-K instances need >= 2 K blocks per split
    M, N = _shape_for(v, cus)
    A, a_s = inputgen.make_activations(M, K, seed=M)
    W, w_s = inputgen.make_weights(N, K, seed=N)
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    y_row = g.gemm_a8w8_blockscale_run_variant(variant, dA, da, dW, dw, workspace=shared_workspace())
    y_pk = g.gemm_a8w8_blockscale_packed_run_variant(variant, dA, da, g.prepack_weights(dW), dw, N, workspace=shared_workspace())
    assert np.array_equal(y_bits(y_pk), y_bits(y_row)), f"{v['name']} M={M} N={N}"
    rows = sorted({0, M // 2, M - 1})
    assert_parity(y_host(y_pk)[rows], oracle.gemm(A, a_s, W, w_s, rows=rows), f"{v['name']} packed")
    say(f"packed {v['name']} M={M} N={N}: bitwise equal to row-major")


@pytest.mark.parametrize("N,K,Ms", [(14336, 5120, range(1, 17)), (34816, 5120, (2, 9, 16)), (32, 6144, (100, 3000)),
                                    (16384, 5120, (2048,)), (5120, 6144, (700, 6016))])
def test_selector_plan_packed_equals_row_major(N, K, Ms):
    Ms = list(Ms)
    A, a_s = inputgen.make_activations(max(Ms), K, seed=3)
    W, w_s = inputgen.make_weights(N, K, seed=4)
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    dWp = g.prepack_weights(dW)
    for M in Ms:
        plan = g.gemm_a8w8_ex_plan(M, N, K, packed=True)
        y_pk = g.gemm_a8w8_blockscale_packed(dA[:M], da[:M], dWp, dw, N)
        y_row = g.gemm_a8w8_blockscale_run_variant(plan["variant"], dA[:M], da[:M], dW, dw)
        assert np.array_equal(y_bits(y_pk), y_bits(y_row)), f"M={M} N={N} K={K} {plan['name']}"
        rows = sorted({0, M // 2, M - 1})
        assert_parity(y_host(y_pk)[rows], oracle.gemm(A[:M], a_s[:M], W, w_s, rows=rows), f"packed M={M} N={N}")
    say(f"packed selector path N={N} K={K}: {len(Ms)} M values bitwise equal")
