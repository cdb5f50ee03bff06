"""GPU test of the allocation-free entry (gemm_a8w8_blockscale_noalloc), through the C ABI.

Its result must equal, bitwise, gemm_a8w8_ex with a caller-owned workspace and
the same plan (the table's fastest, split K included), on two calls in a row
per shape -- the second with a smaller input -- so that the scratch the calls
share must come back ready after each.  Shapes: split plans of the tile and
skinny kernels (N = 256 and N = 32 at K = 6144, out_proj-like and MX-free),
an unsplit decode plan and the tiny configuration; the first call of each is
also checked against the oracle.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu

# (N, K, first M, second smaller M)
CASES = [(256, 6144, 1500, 700), (32, 6144, 2000, 300), (256, 6144, 16, 3), (32, 6144, 9, 2),
         (5120, 6144, 40, 19), (14336, 5120, 16, 1), (512, 1024, 4, 2)]


def _noalloc(dA, da, dW, dw, out):
    M, K = dA.shape
    N = dW.shape[0]
    rc = g.lib().gemm_a8w8_blockscale_noalloc(dA.data_ptr(), da.data_ptr(), dW.data_ptr(), dw.data_ptr(),
                                             out.data_ptr(), M, N, K, torch.cuda.current_stream().cuda_stream)
    assert rc == g.A8W8_OK, g.gemm_a8w8_status_string(rc)
    return out


def test_noalloc_matches_workspace_entry_two_calls_in_a_row():
    ws = g.Workspace(64 << 20)
    split_seen = 0
    for N, K, M1, M2 in CASES:
        A, a = inputgen.make_activations(M1, K, seed=N + M1)
        W, w = inputgen.make_weights(N, K, seed=N + K)
        dA, da, dW, dw = (torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (A, a, W, w))
        for i, M in enumerate((M1, M2)):
            plan = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=1 << 62)
            assert plan["workspace"] <= ctypes.c_int64(32 << 20).value
            split_seen += plan["splits"] > 1
            out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
            y = _noalloc(dA[:M], da[:M], dW, dw, out)
            ref = g.gemm_a8w8_blockscale(dA[:M], da[:M], dW, dw, workspace=ws)
            assert np.array_equal(y_bits(y), y_bits(ref)), f"N={N} K={K} M={M} call {i}"
            say(f"noalloc N={N} K={K} M={M} call {i}: plan {plan['name']} bitwise equal")
            if i == 0:
                rows = sorted({0, M // 2, M - 1})
                assert_parity(y_host(y)[rows], oracle.gemm(A[:M], a[:M], W, w, rows=rows), f"noalloc N={N} M={M}")
    assert split_seen >= 4


def test_noalloc_rejects_bad_arguments_before_launch():
    L = g.lib()
    assert L.gemm_a8w8_blockscale_noalloc(16, 16, 16, 16, 16, 4, 512, 1000, None) == g.A8W8_ERR_SHAPE
    assert L.gemm_a8w8_blockscale_noalloc(None, 16, 16, 16, 16, 4, 512, 1024, None) == g.A8W8_ERR_NULL
    assert L.gemm_a8w8_blockscale_noalloc(None, None, None, None, None, 0, 512, 1024, None) == g.A8W8_OK
