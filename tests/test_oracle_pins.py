"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test fixes a part of the oracle against something independent: the OCP
e4m3fn format definition and torch's own fp8 decode, exact rational
arithmetic, exact power-of-two scaling, deleted K blocks, identity and
permutation weights, a numpy float64 matmul special case, and the relative-L2
figures printed on the "[Perf] Retune gfx942 Qwen3.8-27B a8w8 blockscale
decode rows for cold weights" page (Kernel section).
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import inputgen
import oracle
from tests.parity_util import bf16_round

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_accuracy.txt")
U = 2.0 ** -53


def _golden():
    vals = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def _finite_codes(rng, shape, allow_all=True):
    """Random e4m3fn bytes excluding the two NaN codes."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = 0x7E
    return c


# ---------------------------------------------------------------- e4m3fn codec

def test_decode_against_format_definition():
    t = oracle.e4m3fn_table()
    assert t[0x38] == 1.0                       # S=0 E=0111 M=000
    assert t[0x7E] == 448.0                     # largest finite
    assert t[0xFE] == -448.0
    assert t[0x01] == 2.0 ** -9                 # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9             # largest subnormal
    assert t[0x08] == 2.0 ** -6                 # smallest normal
    assert t[0x00] == 0.0 and t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert int(np.isfinite(t).sum()) == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)             # monotone over the positive codes
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])


def test_decode_matches_torch_fp8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    t = oracle.e4m3fn_table()
    both_nan = np.isnan(ref) & np.isnan(t)
    assert np.all(both_nan | (ref == t))


# ---------------------------------------------------------------- exact brute force

def _exact_gemm(A, a_s, W, w_s):
    dec = [Fraction(v) if np.isfinite(v) else None for v in oracle.e4m3fn_table()]
    M, K = A.shape
    N = W.shape[0]
    out = [[Fraction(0)] * N for _ in range(M)]
    absum = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            ab = Fraction(0)
            for k in range(K):
                t = dec[A[m, k]] * Fraction(float(a_s[m, k // 128])) * \
                    dec[W[n, k]] * Fraction(float(w_s[n // 128, k // 128]))
                acc += t
                ab += abs(t)
            out[m][n] = acc
            absum[m][n] = ab
    return out, absum


@pytest.mark.parametrize("M,N,K,seed", [(3, 130, 256, 11), (2, 1, 128, 12), (1, 129, 384, 13)])
def test_brute_force_exact_rational(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    KB, NB = K // 128, (N + 127) // 128
    a_s = rng.uniform(0.01, 2.0, size=(M, KB)).astype(np.float32)
    w_s = rng.uniform(0.001, 0.1, size=(NB, KB)).astype(np.float32)
    Y = oracle.gemm(A, a_s, W, w_s)
    exact, absum = _exact_gemm(A, a_s, W, w_s)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(Y[m, n]) - exact[m][n])
            assert err <= Fraction((K + 1) * U) * absum[m][n], (m, n, float(err))


def test_row_subset_equals_full():
    rng = np.random.default_rng(3)
    A, a_s = inputgen.make_activations(7, 384, seed=4)
    W, w_s = inputgen.make_weights(200, 384, seed=5)
    full = oracle.gemm(A, a_s, W, w_s)
    rows = [6, 0, 3, 3]
    part = oracle.gemm(A, a_s, W, w_s, rows=rows)
    assert np.array_equal(part, full[rows])


# ---------------------------------------------------------------- scaling laws

def _small_case(M=5, N=260, K=512, seed=21):
    A, a_s = inputgen.make_activations(M, K, seed=seed)
    W, w_s = inputgen.make_weights(N, K, seed=seed + 1)
    return A, a_s, W, w_s


def test_exact_doubling_all_activation_scales():
    A, a_s, W, w_s = _small_case()
    Y = oracle.gemm(A, a_s, W, w_s)
    Y2 = oracle.gemm(A, a_s * np.float32(2), W, w_s)
    assert np.array_equal(Y2, 2.0 * Y)


def test_doubling_one_weight_block():
    A, a_s, W, w_s = _small_case()
    nb, kb = 1, 2
    w2 = w_s.copy()
    w2[nb, kb] *= 2
    Y = oracle.gemm(A, a_s, W, w_s)
    Y2 = oracle.gemm(A, a_s, W, w2)
    cols = np.arange(W.shape[0]) // 128 == nb
    assert np.array_equal(Y2[:, ~cols], Y[:, ~cols])
    # the change in block nb is exactly that K block's contribution (to fp64 rounding)
    only = np.zeros_like(w_s)
    only[nb, kb] = w_s[nb, kb]
    contrib = oracle.gemm(A, a_s, W, only)
    scale = np.abs(Y2[:, cols]).max()
    assert np.allclose(Y2[:, cols] - Y[:, cols], contrib[:, cols], rtol=0, atol=1e-13 * scale)


def test_zero_scale_block_equals_deleted_block():
    A, a_s, W, w_s = _small_case()
    kb = 1
    w0 = w_s.copy()
    w0[:, kb] = 0
    Y0 = oracle.gemm(A, a_s, W, w0)
    keep = np.r_[0:kb * 128, (kb + 1) * 128:A.shape[1]]
    kbs = [b for b in range(w_s.shape[1]) if b != kb]
    Yd = oracle.gemm(A[:, keep], a_s[:, kbs], W[:, keep], w_s[:, kbs])
    scale = np.abs(Yd).max()
    assert np.allclose(Y0, Yd, rtol=0, atol=1e-13 * scale)


def test_zero_scales_give_exact_zeros():
    A, a_s, W, w_s = _small_case()
    assert np.all(oracle.gemm(A, np.zeros_like(a_s), W, w_s) == 0)
    assert np.all(oracle.gemm(A, a_s, W, np.zeros_like(w_s)) == 0)
    a0 = a_s.copy()
    a0[2] = 0
    Y = oracle.gemm(A, a0, W, w_s)
    assert np.all(Y[2] == 0)
    assert np.any(Y[1] != 0)


# ---------------------------------------------------------------- identity-like weights

def test_identity_weights_select_activation_values():
    M, K = 4, 384
    N = 300
    A, a_s = inputgen.make_activations(M, K, seed=31)
    W = np.zeros((N, K), dtype=np.uint8)
    W[np.arange(N), np.arange(N)] = 0x38          # 1.0
    w_s = np.ones(((N + 127) // 128, K // 128), dtype=np.float32)
    Y = oracle.gemm(A, a_s, W, w_s)
    dec = oracle.e4m3fn_table()
    expect = dec[A[:, :N]] * a_s[:, np.arange(N) // 128].astype(np.float64)
    assert np.array_equal(Y, expect)


def test_permutation_weights_pin_column_indexing():
    M, K, N = 3, 256, 256
    A, a_s = inputgen.make_activations(M, K, seed=41)
    perm = np.random.default_rng(42).permutation(K)[:N]
    W = np.zeros((N, K), dtype=np.uint8)
    W[np.arange(N), perm] = 0x38
    w_s = np.array([[1.0, 2.0], [0.5, 4.0]], dtype=np.float32)   # [NB=2, KB=2]
    Y = oracle.gemm(A, a_s, W, w_s)
    dec = oracle.e4m3fn_table()
    n = np.arange(N)
    expect = dec[A[:, perm]] * a_s[:, perm // 128] * w_s[n // 128, perm // 128]
    assert np.array_equal(Y, expect)


# ---------------------------------------------------------------- textbook special case

def test_unit_scales_equal_numpy_matmul_exactly():
    # With all scales 1 every product dec*dec is a multiple of 2^-18 below 2^18 in
    # magnitude, and any sum of <= 1024 of them is exact in fp64, so the oracle and a
    # float64 BLAS matmul (any summation order) must agree bit for bit.
    rng = np.random.default_rng(51)
    M, N, K = 9, 140, 1024
    A = _finite_codes(rng, (M, K))
    W = _finite_codes(rng, (N, K))
    dec = oracle.e4m3fn_table()
    Y = oracle.gemm(A, np.ones((M, K // 128), np.float32), W, np.ones((2, K // 128), np.float32))
    ref = dec[A] @ dec[W].T
    assert np.array_equal(Y, ref)


# ---------------------------------------------------------------- the pages' accuracy figures

@pytest.fixture(scope="module")
def decode_like():
    # 16 activation rows x 1024 weight rows of the K=5120 decode recipe.
    A, a_s = inputgen.make_activations(16, 5120, seed=0)
    W, w_s = inputgen.make_weights(1024, 5120, seed=1)
    return A, a_s, W, w_s


def test_bf16_rounding_floor_matches_page(decode_like):
    A, a_s, W, w_s = decode_like
    Y = oracle.gemm(A, a_s, W, w_s)
    rel = np.linalg.norm(bf16_round(Y) - Y) / np.linalg.norm(Y)
    page = _golden()["rel_l2_no_split"]
    assert abs(rel - page) <= 0.15e-3, rel


def test_split_k_bf16_atomics_signature_matches_page(decode_like):
    # Two K halves, each rounded to bf16, then added into a bf16 output (one more
    # rounding): the split-K accumulation that the page measures at 2.5e-3.
    A, a_s, W, w_s = decode_like
    Y = oracle.gemm(A, a_s, W, w_s)
    h = A.shape[1] // 2
    kb = h // 128
    y0 = oracle.gemm(A[:, :h], a_s[:, :kb], W[:, :h], w_s[:, :kb])
    y1 = oracle.gemm(A[:, h:], a_s[:, kb:], W[:, h:], w_s[:, kb:])
    ys = bf16_round(bf16_round(y0) + bf16_round(y1))
    rel = np.linalg.norm(ys - Y) / np.linalg.norm(Y)
    page = _golden()["rel_l2_split_k_bf16_atomics"]
    assert abs(rel - page) <= 0.15e-3, rel


def test_dequantisation_direction_against_unquantised_product(decode_like):
    # Against the product of the unquantised bf16 values, the oracle differs only by
    # e4m3 quantisation noise (a few percent), never by a scale-sized factor.
    A, a_s, W, w_s = decode_like
    Y = oracle.gemm(A, a_s, W, w_s)
    xa = inputgen.normal_bf16(16, 5120, 1.0, 0).numpy().astype(np.float64)
    xw = inputgen.normal_bf16(1024, 5120, 0.02, 1).numpy().astype(np.float64)
    ref = xa @ xw.T
    rel = np.linalg.norm(Y - ref) / np.linalg.norm(ref)
    assert 2e-2 < rel < 5e-2, rel


# ---------------------------------------------------------------- activation quantisation

def _group_with(values, amax=448.0):
    """One 1 x 128 group: the given values, then zeros, with one element = amax (so s = amax/448)."""
    g = np.zeros(128, dtype=np.float32)
    g[0] = amax
    g[1:1 + len(values)] = np.asarray(values, dtype=np.float32)
    return g


def test_quantize_ties_and_boundaries_hand_derived():
    """amax = 448 gives s = 1 exactly, so each code is the e4m3fn rounding of the value itself.
    Expected bytes worked out by hand from the format (bias 7, 3 mantissa bits, subnormal
    step 2^-9, largest finite 448 = 0x7E), ties going to the even mantissa."""
    cases = [
        (2.0 ** -10, 0x00),            # half of the smallest subnormal: tie -> 0 (even)
        (1.5 * 2.0 ** -9, 0x02),       # between 1 and 2 subnormal steps: tie -> 2
        (7.5 * 2.0 ** -9, 0x08),       # between 7 * 2^-9 and 2^-6: tie -> 0x08 (smallest normal)
        (1.0625, 0x38),                # between 1.0 (0x38) and 1.125 (0x39): tie -> 0x38
        (1.1875, 0x3A),                # between 1.125 (0x39) and 1.25 (0x3A): tie -> 0x3A
        (432.0, 0x7E),                 # between 416 (0x7D) and 448 (0x7E): tie -> 0x7E
        (-3.0, 0xC4),                  # -1.5 * 2^1: sign 1, exponent field 8, mantissa 4
        (-(2.0 ** -12), 0x80),         # negative value rounding to zero keeps the sign bit
        (0.1, 0x1D),                   # 0.1 -> 1.625 * 2^-4 = 0.1015625 (nearest): 0x1D
    ]
    g = _group_with([v for v, _ in cases])
    q, s = oracle.quantize_1x128(g[None, :])
    assert s[0, 0] == np.float32(1.0)
    got = [int(c) for c in q[0, 1:1 + len(cases)]]
    assert got == [c for _, c in cases], [hex(c) for c in got]
    assert q[0, 0] == 0x7E and np.all(q[0, 1 + len(cases):] == 0)


def test_quantize_matches_torch_fp8_cast_of_the_same_quotient():
    """Library special case: torch's float8_e4m3fn cast (round to nearest even) of the same
    fp32 quotients gives the same bytes, and the scales are amax / 448 in fp32."""
    x = torch.randn(37, 1024, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).float()
    x[5, 128:256] = 0.0                                   # a zero group
    x[6, :128] *= 1e-30                                   # tiny values
    q, s = oracle.quantize_1x128(x.numpy())
    g = x.reshape(37, 8, 128)
    amax = g.abs().amax(-1)
    s_ref = (amax / 448.0).to(torch.float32)
    assert np.array_equal(s, s_ref.numpy())
    safe = torch.where(s_ref > 0, s_ref, torch.ones_like(s_ref))
    y = (g / safe[..., None]).clamp(-448.0, 448.0)
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(37, 1024).numpy()
    ref = np.where(np.repeat((s_ref > 0).numpy(), 128, axis=1), ref, 0)
    assert np.array_equal(q, ref)


def test_quantize_zero_group_max_element_and_error_bound():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 512)).astype(np.float32)
    x[2, 256:384] = 0.0
    q, s = oracle.quantize_1x128(x)
    assert s[2, 2] == 0 and np.all(q[2, 256:384] == 0)
    table = oracle.e4m3fn_table()
    for m in range(6):
        for gi in range(4):
            grp = x[m, 128 * gi:128 * gi + 128].astype(np.float64)
            if s[m, gi] == 0:
                continue
            k = int(np.argmax(np.abs(grp)))
            assert q[m, 128 * gi + k] in (0x7E, 0xFE)               # the group maximum maps to +-448
            deq = table[q[m, 128 * gi:128 * gi + 128]] * float(s[m, gi])
            # e4m3fn spacing at |v| is at most 2^(floor(log2|v|) - 3) (2^-9 below 2^-6)
            v = np.abs(grp) / float(s[m, gi])
            spacing = np.where(v >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(v, 1e-300))) - 3), 2.0 ** -9)
            assert np.all(np.abs(deq - grp) <= 0.5 * spacing * float(s[m, gi]) * (1 + 1e-6))
