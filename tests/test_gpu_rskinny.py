"""GPU tests of the row-range skinny kernel (M <= 16): every workgroup owns a run
of weight rows that need not start on a 16-row tile, a 128-row block-scale row
or a 32-row MX scale row, so its tiles straddle scale rows and its last tile
is partial.

Checked against the oracle for every instance, the three scale kinds and both
weight layouts: runs of 24 rows (N = 20 x CUs + 2: a ragged last run and a
last row group of 2), several passes over K, tiny N (one 4-row unit per
workgroup), and the qkv shape.  Packed weights split rows in whole 16-row
tiles, yet every output element sums the same K runs in the same order, so the
packed result must equal the row-major one bitwise; repeats are bitwise equal.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, variant_by_name, variant_names, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu

RSKINNY = variant_names(kinds=("rskinny",))


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


def _shapes():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return [(16, 20 * cus + 2, 640), (5, 20 * cus, 8192), (1, 300, 1024), (13, 14336, 5120), (7, 130, 256)]


def _accepts(vid, M, N, K, kind):
    try:
        g.gemm_a8w8_ex_plan(M, N, K, scale_kind=kind, variant=vid,
                            cu_count=torch.cuda.get_device_properties(0).multi_processor_count)
        return True
    except g.A8W8Error:
        return False


@pytest.mark.parametrize("name", RSKINNY)
@pytest.mark.parametrize("kind", ["block", "mx", "rowwise"])
def test_rskinny_instance(name, kind):
    v = variant_by_name(name)
    vid = v["variant"]
    ran = 0
    for (M, N, K) in _shapes():
        if not _accepts(vid, M, N, K, kind):
            continue
        if kind == "block":
            A, a = inputgen.make_activations(M, K, seed=M + N)
            W, w = inputgen.make_weights(N, K, seed=N + K)
            ref = oracle.gemm(A, a, W, w)
        elif kind == "mx":
            A, a = inputgen.make_mx_activations(M, K, seed=M + N)
            W, w = inputgen.make_mx_weights(N, K, seed=N + K)
            ref = oracle.gemm_mx(A, a, W, w)
        else:
            A, a = inputgen.make_rowwise_activations(M, K, seed=M + N)
            W, w = inputgen.make_rowwise_weights(N, K, seed=N + K)
            ref = oracle.gemm_rowwise(A, a, W, w)
        dA, da, dW, dw = _dev(A, a, W, w)
        y = g.gemm_a8w8_ex(dA, da, dW, dw, scale_kind=kind, variant=vid)
        st = assert_parity(y_host(y), ref, f"{name} {kind} M={M} N={N} K={K}")
        y2 = g.gemm_a8w8_ex(dA, da, dW, dw, scale_kind=kind, variant=vid)
        assert np.array_equal(y_bits(y2), y_bits(y)), f"{name} {kind}: repeat differs"
        if _accepts(vid, M, N, K, kind):
            yp = g.gemm_a8w8_ex(dA, da, g.prepack_weights(dW), dw, scale_kind=kind, packed_n=N, variant=vid)
            assert np.array_equal(y_bits(yp), y_bits(y)), f"{name} {kind} M={M} N={N}: packed differs"
        say(f"{name} {kind} M={M} N={N} K={K}: rel_l2={st['rel_l2']:.3e}")
        ran += 1
    assert ran >= 2, f"{name}: too few shapes accepted"


def test_rskinny_every_m_on_out_proj_and_qkv():
    """The decode shapes at every M = 1..16 through the instances that take them."""
    for N, K in ((5120, 6144), (14336, 5120)):
        A, a = inputgen.make_activations(16, K, seed=3)
        W, w = inputgen.make_weights(N, K, seed=4)
        ref = oracle.gemm(A, a, W, w)
        dA, da, dW, dw = _dev(A, a, W, w)
        for name in RSKINNY:
            vid = variant_by_name(name)["variant"]
            if not _accepts(vid, 16, N, K, "block"):
                continue
            for M in range(1, 17):
                y = g.gemm_a8w8_blockscale_run_variant(vid, dA[:M], da[:M], dW, dw)
                assert_parity(y_host(y), ref[:M], f"{name} M={M} N={N} K={K}")
            say(f"{name} N={N} K={K}: M = 1..16 ok")
