"""Pins of the MX-scaled oracle (``oracle.gemm_mx``) to facts outside it.

The MX variant (E8M0 power-of-two scales, one per row per 32-wide K group of
the activations and one per 32 x 32 weight block; the mxfp8 GEMM that the
gfx1250 BF16 and MX32 tuned-rows page, ROCm/aiter #7247, tunes) is pinned by:
the E8M0 format definition; exact rational brute force on tiny inputs;
power-of-two changes of one activation group and of one weight block, which
must move exactly their own K range and rows (this catches a scale index
taken per 128 instead of per 32, or rows and columns swapped); permutation
weights; a unit-scale special case equal to a numpy float64 matmul; the
reduction to the (separately pinned) block-scale oracle when every 32-wide
scale inside a 128-wide block agrees; NaN propagation from the 0xFF code; and
the seeded generator's shared-exponent rule.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import inputgen
import oracle

U = 2.0 ** -53


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _mx_case(M=5, N=100, K=256, seed=61):
    A, a = inputgen.make_mx_activations(M, K, seed=seed)
    W, w = inputgen.make_mx_weights(N, K, seed=seed + 1)
    return A, a, W, w


# ---------------------------------------------------------------- E8M0 codec

def test_e8m0_against_format_definition():
    assert oracle.e8m0_value(127) == 1.0
    assert oracle.e8m0_value(128) == 2.0
    assert oracle.e8m0_value(126) == 0.5
    assert oracle.e8m0_value(0) == 2.0 ** -127
    assert oracle.e8m0_value(254) == 2.0 ** 127
    assert math.isnan(oracle.e8m0_value(255))
    vals = [oracle.e8m0_value(c) for c in range(255)]
    for c in range(1, 255):
        assert vals[c] == 2 * vals[c - 1]


# ---------------------------------------------------------------- exact brute force

def _exact_mx(A, a, W, w):
    dec = [Fraction(v) if np.isfinite(v) else None for v in oracle.e4m3fn_table()]
    M, K = A.shape
    N = W.shape[0]
    p2 = lambda e: Fraction(2) ** (int(e) - 127)
    out, absum = {}, {}
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            ab = Fraction(0)
            for k in range(K):
                t = dec[A[m, k]] * p2(a[m, k // 32]) * dec[W[n, k]] * p2(w[n // 32, k // 32])
                acc += t
                ab += abs(t)
            out[m, n], absum[m, n] = acc, ab
    return out, absum


@pytest.mark.parametrize("M,N,K,seed", [(2, 70, 128, 71), (1, 33, 96, 72), (3, 5, 64, 73)])
def test_mx_brute_force_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    a = rng.integers(100, 150, size=(M, K // 32), dtype=np.uint8)
    w = rng.integers(100, 150, size=((N + 31) // 32, K // 32), dtype=np.uint8)
    Y = oracle.gemm_mx(A, a, W, w)
    exact, absum = _exact_mx(A, a, W, w)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(Y[m, n]) - exact[m, n])
            assert err <= Fraction((K + 1) * U) * absum[m, n], (m, n, float(err))


def test_mx_row_subset_equals_full():
    A, a, W, w = _mx_case(M=7)
    full = oracle.gemm_mx(A, a, W, w)
    rows = [6, 0, 3, 3]
    assert np.array_equal(oracle.gemm_mx(A, a, W, w, rows=rows), full[rows])


# ---------------------------------------------------------------- one group, one block

def test_mx_one_activation_group_moves_only_its_k_range():
    A, a, W, w = _mx_case()
    m, j = 2, 5                                  # row 2, K range [160, 192)
    a2 = a.copy()
    a2[m, j] += 1                                # doubles that group
    Y = oracle.gemm_mx(A, a, W, w)
    Y2 = oracle.gemm_mx(A, a2, W, w)
    others = np.arange(A.shape[0]) != m
    assert np.array_equal(Y2[others], Y[others])
    # The change is the group's own contribution: A zeroed outside [32 j, 32 j + 32).
    Aj = np.zeros_like(A)
    Aj[:, 32 * j:32 * j + 32] = A[:, 32 * j:32 * j + 32]
    contrib = oracle.gemm_mx(Aj, a, W, w)[m]
    scale = np.abs(Y2[m]).max()
    assert np.allclose(Y2[m] - Y[m], contrib, rtol=0, atol=1e-13 * scale)
    assert np.any(contrib != 0)


def test_mx_one_weight_block_moves_only_its_rows_and_k_range():
    A, a, W, w = _mx_case()
    i, j = 1, 3                                  # weight rows [32, 64), K range [96, 128)
    w2 = w.copy()
    w2[i, j] += 1
    Y = oracle.gemm_mx(A, a, W, w)
    Y2 = oracle.gemm_mx(A, a, W, w2)
    cols = np.arange(W.shape[0]) // 32 == i
    assert np.array_equal(Y2[:, ~cols], Y[:, ~cols])
    Wj = np.zeros_like(W)
    Wj[:, 32 * j:32 * j + 32] = W[:, 32 * j:32 * j + 32]
    contrib = oracle.gemm_mx(A, a, Wj, w)[:, cols]
    scale = np.abs(Y2[:, cols]).max()
    assert np.allclose(Y2[:, cols] - Y[:, cols], contrib, rtol=0, atol=1e-13 * scale)
    assert np.any(contrib != 0)


def test_mx_permutation_weights_pin_indexing():
    M, K, N = 3, 256, 96
    A, a = inputgen.make_mx_activations(M, K, seed=81)
    perm = np.random.default_rng(82).permutation(K)[:N]
    W = np.zeros((N, K), dtype=np.uint8)
    W[np.arange(N), perm] = 0x38                 # one 1.0 per weight row
    w = np.random.default_rng(83).integers(120, 135, size=(N // 32, K // 32), dtype=np.uint8)
    Y = oracle.gemm_mx(A, a, W, w)
    dec = oracle.e4m3fn_table()
    n = np.arange(N)
    expect = dec[A[:, perm]] * np.ldexp(1.0, a[:, perm // 32].astype(np.int64) - 127) \
        * np.ldexp(1.0, w[n // 32, perm // 32].astype(np.int64) - 127)
    assert np.array_equal(Y, expect)


# ---------------------------------------------------------------- special cases

def test_mx_unit_scales_equal_numpy_matmul_exactly():
    # Code 127 is the scale 1: the oracle then computes dec(A) . dec(W)^T, exact in
    # fp64 for these sizes (see the block-scale pin of the same kind).
    rng = np.random.default_rng(91)
    M, N, K = 6, 70, 512
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    dec = oracle.e4m3fn_table()
    Y = oracle.gemm_mx(A, np.full((M, K // 32), 127, np.uint8), W, np.full((3, K // 32), 127, np.uint8))
    assert np.array_equal(Y, dec[A] @ dec[W].T)


def test_mx_reduces_to_block_scale_oracle():
    # When the four 32-wide scales of every 128-wide activation group agree, and
    # every 32 x 32 weight scale inside a 128 x 128 block agrees, the MX product
    # is the block-scale product with fp32 scales 2^(e - 127).
    rng = np.random.default_rng(101)
    M, N, K = 4, 300, 384
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    ea = rng.integers(110, 140, size=(M, K // 128), dtype=np.uint8)
    ew = rng.integers(110, 140, size=((N + 127) // 128, K // 128), dtype=np.uint8)
    a_mx = np.repeat(ea, 4, axis=1)
    w_mx = np.repeat(np.repeat(ew, 4, axis=0)[:(N + 31) // 32], 4, axis=1)
    Y_mx = oracle.gemm_mx(A, a_mx, W, w_mx)
    Y_bs = oracle.gemm(A, np.ldexp(np.float32(1), ea.astype(np.int32) - 127).astype(np.float32), W,
                       np.ldexp(np.float32(1), ew.astype(np.int32) - 127).astype(np.float32))
    assert np.array_equal(Y_mx, Y_bs)


def test_mx_nan_scale_code_poisons_only_its_row():
    A, a, W, w = _mx_case()
    a2 = a.copy()
    a2[1, 0] = 255
    Y = oracle.gemm_mx(A, a2, W, w)
    assert np.all(np.isnan(Y[1]))
    assert np.all(np.isfinite(np.delete(Y, 1, axis=0)))


def test_mx_batched_is_per_batch():
    parts = [_mx_case(M=3, N=40, K=128, seed=s) for s in (111, 113)]
    A = np.stack([p[0] for p in parts])
    a = np.stack([p[1] for p in parts])
    W = np.stack([p[2] for p in parts])
    w = np.stack([p[3] for p in parts])
    Y = oracle.gemm_mx_batched(A, a, W, w)
    for i, p in enumerate(parts):
        assert np.array_equal(Y[i], oracle.gemm_mx(*p))


# ---------------------------------------------------------------- the seeded MX generator

def test_mx_generator_shared_exponent_and_saturation():
    x = inputgen.normal_bf16(6, 256, 1.0, 121)
    q, e = inputgen.quantize_mx(x, 1)
    xs = x.double().numpy()
    dec = oracle.e4m3fn_table()
    for r in range(6):
        for j in range(8):
            g = xs[r, 32 * j:32 * j + 32]
            amax = float(np.abs(g).max())
            # floor(log2(amax)) from the binary exponent, independently of the generator
            assert int(e[r, j]) - 127 == math.frexp(amax)[1] - 1 - 8
            s = 2.0 ** (int(e[r, j]) - 127)
            vals = dec[q[r, 32 * j:32 * j + 32]]
            y = np.clip(g / s, -448.0, 448.0)
            # nearest representable: within half the e4m3 spacing (relative 2^-4) or the subnormal step
            assert np.all(np.abs(vals - y) <= np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10))
            assert 256.0 <= np.abs(vals).max() <= 448.0


def test_mx_generator_zero_block_and_partial_last_block():
    x = torch.zeros(40, 64)
    x[33, 5] = 3.0                               # only the partial second row-block is non-zero
    q, e = inputgen.quantize_mx(x, 32)
    assert e.shape == (2, 2)
    assert e[0, 0] == 127 and e[0, 1] == 127 and e[1, 1] == 127 and np.all(q[:32] == 0)
    assert int(e[1, 0]) - 127 == 1 - 8         # floor(log2 3) = 1
    assert oracle.e4m3fn_value(int(q[33, 5])) * 2.0 ** (int(e[1, 0]) - 127) == 3.0
