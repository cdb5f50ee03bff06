"""Pins of the row-wise oracle (``oracle.gemm_rowwise``: one fp32 scale per
activation row and one per weight row) to facts outside it.

Exact rational brute force on tiny inputs; exact doubling of one row's and one
column's scale (only that row / column changes, by exactly 2x: catches a scale
applied to the wrong axis); zero scales; a unit-scale special case equal to a
numpy float64 matmul; the reduction to the (separately pinned) block-scale
oracle when the per-channel scales are constant over each 128-row block and
every scale is a power of two (then both compute exactly); and the seeded
per-row generator's amax/448 rule.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import inputgen
import oracle

U = 2.0 ** -53


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E
    return c


def _case(M=6, N=150, K=384, seed=131):
    A, a = inputgen.make_rowwise_activations(M, K, seed=seed)
    W, w = inputgen.make_rowwise_weights(N, K, seed=seed + 1)
    return A, a, W, w


@pytest.mark.parametrize("M,N,K,seed", [(3, 40, 128, 141), (1, 7, 256, 142), (2, 33, 96, 143)])
def test_rowwise_brute_force_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    a = rng.uniform(0.01, 2.0, size=M).astype(np.float32)
    w = rng.uniform(0.001, 0.1, size=N).astype(np.float32)
    Y = oracle.gemm_rowwise(A, a, W, w)
    dec = [Fraction(v) if np.isfinite(v) else None for v in oracle.e4m3fn_table()]
    for m in range(M):
        for n in range(N):
            prods = [dec[A[m, k]] * dec[W[n, k]] for k in range(K)]
            exact = sum(prods, Fraction(0)) * Fraction(float(a[m])) * Fraction(float(w[n]))
            bound = Fraction((K + 3) * U) * sum((abs(p) for p in prods), Fraction(0)) \
                * Fraction(float(a[m])) * Fraction(float(w[n]))
            assert abs(Fraction(Y[m, n]) - exact) <= bound, (m, n)


def test_rowwise_row_subset_equals_full():
    A, a, W, w = _case()
    full = oracle.gemm_rowwise(A, a, W, w)
    rows = [5, 0, 2, 2]
    assert np.array_equal(oracle.gemm_rowwise(A, a, W, w, rows=rows), full[rows])


def test_rowwise_doubling_one_row_and_one_column():
    A, a, W, w = _case()
    Y = oracle.gemm_rowwise(A, a, W, w)
    a2 = a.copy()
    a2[3] *= 2
    Ya = oracle.gemm_rowwise(A, a2, W, w)
    assert np.array_equal(Ya[3], 2 * Y[3])
    assert np.array_equal(np.delete(Ya, 3, axis=0), np.delete(Y, 3, axis=0))
    w2 = w.copy()
    w2[77] *= 2
    Yw = oracle.gemm_rowwise(A, a, W, w2)
    assert np.array_equal(Yw[:, 77], 2 * Y[:, 77])
    assert np.array_equal(np.delete(Yw, 77, axis=1), np.delete(Y, 77, axis=1))


def test_rowwise_zero_scales():
    A, a, W, w = _case()
    a0 = a.copy()
    a0[1] = 0
    w0 = w.copy()
    w0[10] = 0
    Y = oracle.gemm_rowwise(A, a0, W, w0)
    assert np.all(Y[1] == 0) and np.all(Y[:, 10] == 0)
    assert np.any(Y[0] != 0)


def test_rowwise_unit_scales_equal_numpy_matmul_exactly():
    rng = np.random.default_rng(151)
    M, N, K = 7, 90, 1024
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    dec = oracle.e4m3fn_table()
    Y = oracle.gemm_rowwise(A, np.ones(M, np.float32), W, np.ones(N, np.float32))
    assert np.array_equal(Y, dec[A] @ dec[W].T)


def test_rowwise_reduces_to_block_scale_oracle_with_power_of_two_scales():
    rng = np.random.default_rng(161)
    M, N, K = 5, 300, 512
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    ea = rng.integers(-6, 7, size=M)
    ew = rng.integers(-9, 3, size=(N + 127) // 128)
    a = np.ldexp(np.float32(1), ea).astype(np.float32)
    w_blocks = np.ldexp(np.float32(1), ew).astype(np.float32)
    w = w_blocks[np.arange(N) // 128]
    Y_rw = oracle.gemm_rowwise(A, a, W, w)
    Y_bs = oracle.gemm(A, np.repeat(a[:, None], K // 128, axis=1), W,
                       np.repeat(w_blocks[:, None], K // 128, axis=1))
    assert np.array_equal(Y_rw, Y_bs)


def test_rowwise_generator_amax_rule():
    x = inputgen.normal_bf16(4, 640, 1.0, 171)
    q, s = inputgen.quantize_per_row(x)
    xs = x.double().numpy()
    dec = oracle.e4m3fn_table()
    for r in range(4):
        assert s[r] == np.float32(np.float32(np.abs(xs[r]).max()) / np.float32(448.0))
        vals = dec[q[r]]
        assert np.abs(vals).max() == 448.0
        assert np.all(np.abs(vals * float(s[r]) - xs[r]) <= np.abs(xs[r]) * 2.0 ** -4 + float(s[r]) * 2.0 ** -10)
