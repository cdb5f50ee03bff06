"""GPU parity of the per-1x128 activation quantisation (a8w8_quantize_1x128).

The codes are integers decided by an fp32 quotient, so the bar is bit-exact:
codes and scales must equal the oracle's (``oracle.quantize_1x128``, pinned in
tests/test_oracle_pins.py) byte for byte.  Inputs are seeded N(0,1) bf16
activations at the decode and prefill widths, plus groups that hit the edge
cases: all zero, bf16 subnormals, values that quantise below 2^-6, negative
zero, very large magnitudes, a single non-zero value, ragged row counts.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, run, say, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu


def _edge_rows(K: int, seed: int) -> torch.Tensor:
    """bf16-valued fp32 rows whose groups exercise the encoder's edge cases."""
    x = inputgen.normal_bf16(8, K, 1.0, seed)
    x[0, :] = 0.0                                          # zero groups
    x[1, :] *= 2.0 ** -130                                 # bf16 subnormal range
    x[2, :] = x[2, :].sign() * 2.0 ** -20                  # equal magnitudes
    x[2, 0] = 1.0                                          # ... below one large value: codes near 2^-6 and 0
    x[3, :] *= 1e30                                        # huge magnitudes
    x[4, :] = -0.0                                         # negative zeros (amax 0)
    x[4, 3] = -5.0                                         # ... in one group with a single value
    x[5, ::7] = 0.0
    x[6, :] = torch.tensor([1.0, -1.0], dtype=torch.float32).repeat(K // 2) * 448.0
    x[7, :] = torch.arange(K, dtype=torch.float32) * 2.0 ** -14   # a ramp: every rounding position
    return x.to(torch.bfloat16).to(torch.float32)


def _check(xf: torch.Tensor, what: str):
    xb = xf.to(torch.bfloat16).to(DEV)
    q, s = g.quantize_1x128(xb)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_1x128(xf.numpy())
    qh = q.view(torch.uint8).cpu().numpy()
    sh = s.cpu().numpy()
    bad = np.flatnonzero(qh != q_ref)
    assert bad.size == 0, (f"{what}: {bad.size} codes differ, first at {np.unravel_index(bad[0], qh.shape)}: "
                           f"gpu {qh.flat[bad[0]]:#04x} oracle {q_ref.flat[bad[0]]:#04x}")
    assert np.array_equal(sh.view(np.uint32), s_ref.view(np.uint32)), f"{what}: scales differ"
    return q, s


@pytest.mark.parametrize("M,K", [(1, 128), (5, 640), (16, 5120), (300, 6144), (2049, 1024)])
def test_quantize_bit_exact_normal_inputs(M, K):
    _check(inputgen.normal_bf16(M, K, 1.0, seed=M + K), f"normal M={M} K={K}")
    say(f"quantize M={M} K={K}: bit-exact")


@pytest.mark.parametrize("K", [128, 1024])
def test_quantize_bit_exact_edge_groups(K):
    _check(_edge_rows(K, seed=K), f"edge K={K}")


def test_quantize_many_groups_per_lane_grid_stride():
    """201k groups: the capped grid walks several groups per workgroup."""
    M, K = 4096, 6144
    _check(inputgen.normal_bf16(M, K, 1.0, seed=4), f"grid-stride M={M} K={K}")


def test_quantize_matches_generated_gemm_inputs():
    """The kernel reproduces the generator's activation operand (same recipe)."""
    M, K = 33, 5120
    x = inputgen.normal_bf16(M, K, 1.0, seed=0)
    q, s = g.quantize_1x128(x.to(torch.bfloat16).to(DEV))
    A, a_s = inputgen.make_activations(M, K, seed=0)
    assert np.array_equal(q.view(torch.uint8).cpu().numpy(), A)
    assert np.array_equal(s.cpu().numpy(), a_s)


def test_quantize_then_gemm_end_to_end():
    M, N, K = 37, 14336, 5120
    x = inputgen.normal_bf16(M, K, 1.0, seed=21)
    q, s = g.quantize_1x128(x.to(torch.bfloat16).to(DEV))
    W, w_s = inputgen.make_weights(N, K, seed=1)
    dW, dw = torch.from_numpy(W).to(DEV), torch.from_numpy(w_s).to(DEV)
    y = run(q, s, dW, dw)
    A_ref, a_ref = oracle.quantize_1x128(x.numpy())
    assert_parity(y_host(y), oracle.gemm(A_ref, a_ref, W, w_s), "quantize -> gemm")


def test_quantize_guard_bands_and_empty():
    M, K = 19, 640
    x = inputgen.normal_bf16(M, K, 1.0, seed=8).to(torch.bfloat16).to(DEV)
    pad = 64
    qbuf = torch.full((pad + M * K + pad,), 0x5A, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((pad + M * (K // 128) + pad,), -7.0, dtype=torch.float32, device=DEV)
    q = qbuf[pad:pad + M * K].view(M, K)
    s = sbuf[pad:pad + M * (K // 128)].view(M, K // 128)
    g.quantize_1x128(x, out=q, scale_out=s)
    torch.cuda.synchronize()
    qb, sb = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(qb[:pad] == 0x5A) and np.all(qb[-pad:] == 0x5A)
    assert np.all(sb[:pad] == -7.0) and np.all(sb[-pad:] == -7.0)
    q0, s0 = g.quantize_1x128(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV))
    assert q0.shape == (0, 256) and s0.shape == (0, 2)


def test_quantize_every_bf16_value_under_many_scales():
    """The kernel forms x / s with a reciprocal and one FMA correction; this sweeps every finite
    bf16 value below each of 24 group maxima (7 of them not multiples of 7 times a power of two,
    so s = amax/448 is inexact) and compares every code with the oracle's IEEE division."""
    bits = np.arange(65536, dtype=np.uint32) << 16
    allv = bits.view(np.float32)
    allv = allv[np.isfinite(allv)]
    rng = np.random.default_rng(12)
    amaxes = [448.0, 1.0, 3.0, 5.0, 7.0, 1e-3, 2.0 ** -120, 1e30, 0.3, 11.0, 13.0, 100.0]
    amaxes += [float(np.float32(v)) for v in rng.lognormal(0.0, 8.0, 12)]
    rows = []
    for a in amaxes:
        a = float(torch.tensor([a]).to(torch.bfloat16).float())
        v = allv[np.abs(allv) <= a]
        n = (len(v) + 126) // 127
        v = np.concatenate([v, np.zeros(n * 127 - len(v), np.float32)]).reshape(n, 127)
        rows.append(np.concatenate([np.full((n, 1), a, np.float32), v], axis=1))
    groups = np.concatenate(rows)                                   # [G, 128]
    G = groups.shape[0]
    K = 1024
    M = (G + K // 128 - 1) // (K // 128)
    pad = M * (K // 128) - G
    groups = np.concatenate([groups, np.zeros((pad, 128), np.float32)])
    x = torch.from_numpy(groups.reshape(M, K).copy())
    _check(x, f"bf16 sweep ({G} groups)")
    say(f"quantize: every bf16 value under {len(amaxes)} maxima ({G} groups) bit-exact")
