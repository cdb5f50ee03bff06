"""Seeded synthetic inputs for the a8w8 block-scale GEMM.

This module produces the operands that both the GPU library and the CPU
oracle consume: fp8 E4M3 ("e4m3fn", OCP 8-bit floating point) bytes plus fp32
scales.  It contains input generation only -- no part of the GEMM itself.

Recipe (the one the workloads of this project are specified with):

* activations ``A[M, K]``: x ~ N(0, 1) in fp32, rounded to bf16 (RNE); for
  every 1 x 128 group along K, ``s = fp32(amax / 448)`` and
  ``q = e4m3fn_RNE(clamp(x / s, -448, 448))`` (division in fp32);
* weights ``W[N, K]``: x ~ N(0, 0.02) rounded to bf16, quantised the same way
  per 128 x 128 block (the last block along N covers only the rows that
  exist when N is not a multiple of 128);
* a group or block whose amax is 0 gets ``s = 0`` and all-zero codes.

The 128 x 128 weight block is the ``weight_block_size: [128,128]`` that the
"Why aiter#5069's measured -25% kernel win moved serving throughput by 0.0%"
page names for the block-quantised checkpoint; the activation group size, the
e4m3 variant and amax/448 are this project's reading of an operation the
pages name but do not define.

Layouts (all row-major, C-contiguous):
``A`` uint8 [M, K], ``a_scale`` float32 [M, K/128],
``W`` uint8 [N, K], ``w_scale`` float32 [ceil(N/128), K/128].
"""
from __future__ import annotations

import numpy as np
import torch

GROUP = 128          # K-extent of one activation group / weight block
FP8_MAX = 448.0      # largest finite e4m3fn magnitude

__all__ = [
    "GROUP", "FP8_MAX", "normal_bf16", "quantize_rows_1x128",
    "quantize_blocks_128x128", "make_activations", "make_weights",
    "sign_flip_copy", "random_m_values",
    "MX_GROUP", "E4M3_EMAX", "quantize_mx", "make_mx_activations", "make_mx_weights",
    "quantize_per_row", "make_rowwise_activations", "make_rowwise_weights",
]


def normal_bf16(rows: int, cols: int, std: float, seed: int) -> torch.Tensor:
    """fp32 tensor of N(0, std) samples rounded to bf16 (RNE), seeded by numpy's default_rng."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return torch.from_numpy(x).to(torch.bfloat16).to(torch.float32)


def _encode_e4m3fn(y: torch.Tensor) -> torch.Tensor:
    """Round fp32 values already inside [-448, 448] to e4m3fn bytes (torch's RNE cast)."""
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def quantize_rows_1x128(x: torch.Tensor) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 [R, K] with one scale per 1 x 128 group -> (uint8 [R, K], float32 [R, K/128])."""
    R, K = x.shape
    assert K % GROUP == 0, "K must be a multiple of 128"
    g = x.reshape(R, K // GROUP, GROUP)
    amax = g.abs().amax(dim=-1)                                # [R, KB]
    s = (amax / FP8_MAX).to(torch.float32)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    y = (g / safe.unsqueeze(-1)).clamp(-FP8_MAX, FP8_MAX)
    y = torch.where((s > 0).unsqueeze(-1), y, torch.zeros_like(y))
    q = _encode_e4m3fn(y).reshape(R, K)
    return q.numpy().copy(), s.numpy().copy()


def quantize_blocks_128x128(x: torch.Tensor) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 [N, K] with one scale per 128 x 128 block -> (uint8 [N, K], float32 [ceil(N/128), K/128])."""
    N, K = x.shape
    assert K % GROUP == 0, "K must be a multiple of 128"
    NB, KB = (N + GROUP - 1) // GROUP, K // GROUP
    pad = NB * GROUP - N
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x   # zero rows do not change amax
    b = xp.reshape(NB, GROUP, KB, GROUP)
    amax = b.abs().amax(dim=(1, 3))                            # [NB, KB]
    s = (amax / FP8_MAX).to(torch.float32)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    y = (b / safe[:, None, :, None]).clamp(-FP8_MAX, FP8_MAX)
    y = torch.where((s > 0)[:, None, :, None], y, torch.zeros_like(y))
    q = _encode_e4m3fn(y).reshape(NB * GROUP, K)[:N]
    return q.numpy().copy(), s.numpy().copy()


def make_activations(M: int, K: int, seed: int = 0, std: float = 1.0):
    """Activation operand: (A uint8 [M, K], a_scale float32 [M, K/128])."""
    return quantize_rows_1x128(normal_bf16(M, K, std, seed))


def make_weights(N: int, K: int, seed: int = 1, std: float = 0.02):
    """Weight operand: (W uint8 [N, K], w_scale float32 [ceil(N/128), K/128])."""
    return quantize_blocks_128x128(normal_bf16(N, K, std, seed))


def sign_flip_copy(W: np.ndarray, seed: int) -> np.ndarray:
    """A distinct copy of W with a seeded random subset of sign bits flipped.

    Flipping signs keeps |values| (hence every block's amax and its w_scale)
    and the distribution; the bytes differ, so each copy occupies its own
    memory.  Used to rotate weights so that each call reads them from HBM.
    """
    rng = np.random.default_rng(seed)
    mask = np.frombuffer(rng.bytes(W.size), dtype=np.uint8).reshape(W.shape) & np.uint8(0x80)
    return W ^ mask


def random_m_values(count: int, lo: int = 1, hi: int = 8192, seed: int = 2) -> list[int]:
    """`count` i.i.d. uniform integers in [lo, hi] (dense arbitrary M)."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.integers(lo, hi + 1, size=count)]


# ---------------------------------------------------------------------------
# MX-scaled operands (mxfp8 with 32 x 32 weight-scale blocks, the variant the
# gfx1250 BF16 and MX32 tuned-rows page, ROCm/aiter #7247, tunes).  The page
# gives the block shape only; the encoding is the OCP Microscaling one: a
# block of values shares one E8M0 byte e (value 2^(e - 127)) with
# e - 127 = floor(log2(amax)) - 8 (8 = the exponent of e4m3fn's largest
# normal), and each value becomes e4m3fn_RNE(clamp(x / 2^(e-127), -448, 448))
# -- the division is exact (a power of two), and the clamp saturates the top
# of the binade, [448, 512).  A block whose amax is 0 gets e = 127 and zero
# codes.  Activations: one scale per row per 32-wide K group,
# ``a_scale`` uint8 [M, K/32]; weights: one per 32 x 32 block,
# ``w_scale`` uint8 [ceil(N/32), K/32] (the last block along N covers the
# rows that exist).

MX_GROUP = 32
E4M3_EMAX = 8        # largest normal e4m3fn value is 1.75 * 2^8


def quantize_mx(x: torch.Tensor, rows_per_block: int) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 [R, K] with one E8M0 scale per rows_per_block x 32 block.

    Returns (codes uint8 [R, K], scales uint8 [ceil(R / rows_per_block), K / 32]).
    """
    R, K = x.shape
    assert K % MX_GROUP == 0, "K must be a multiple of 32"
    rb = rows_per_block
    RB, KG = (R + rb - 1) // rb, K // MX_GROUP
    pad = RB * rb - R
    xp = torch.nn.functional.pad(x, (0, 0, 0, pad)) if pad else x
    b = xp.reshape(RB, rb, KG, MX_GROUP)
    amax = b.abs().amax(dim=(1, 3))                            # [RB, KG]
    _, ex = torch.frexp(amax)                                  # amax = f * 2^ex, f in [0.5, 1)
    shared = (ex - 1 - E4M3_EMAX).clamp(-127, 127)             # floor(log2(amax)) - 8
    shared = torch.where(amax > 0, shared, torch.zeros_like(shared))
    code = (shared + 127).to(torch.uint8)
    y = torch.ldexp(b, -shared[:, None, :, None].to(torch.float32))
    y = y.clamp(-FP8_MAX, FP8_MAX)
    q = _encode_e4m3fn(y).reshape(RB * rb, K)[:R]
    return q.numpy().copy(), code.numpy().copy()


def make_mx_activations(M: int, K: int, seed: int = 0, std: float = 1.0):
    """MX activation operand: (A uint8 [M, K], a_scale uint8 E8M0 [M, K/32])."""
    return quantize_mx(normal_bf16(M, K, std, seed), 1)


def make_mx_weights(N: int, K: int, seed: int = 1, std: float = 0.02):
    """MX weight operand: (W uint8 [N, K], w_scale uint8 E8M0 [ceil(N/32), K/32])."""
    return quantize_mx(normal_bf16(N, K, std, seed), MX_GROUP)


# ---------------------------------------------------------------------------
# Row-wise operands (per-token activations, per-channel weights): one fp32
# scale per row over all of K, s = fp32(amax / 448), codes as for the block
# recipe (the reading of the per-token a8w8 path the pages name).

def quantize_per_row(x: torch.Tensor) -> tuple[np.ndarray, np.ndarray]:
    """Quantise fp32 [R, K] with one scale per row -> (uint8 [R, K], float32 [R])."""
    amax = x.abs().amax(dim=1)
    s = (amax / FP8_MAX).to(torch.float32)
    safe = torch.where(s > 0, s, torch.ones_like(s))
    y = (x / safe[:, None]).clamp(-FP8_MAX, FP8_MAX)
    y = torch.where((s > 0)[:, None], y, torch.zeros_like(y))
    return _encode_e4m3fn(y).numpy().copy(), s.numpy().copy()


def make_rowwise_activations(M: int, K: int, seed: int = 0, std: float = 1.0):
    """Per-token activation operand: (A uint8 [M, K], a_scale float32 [M])."""
    return quantize_per_row(normal_bf16(M, K, std, seed))


def make_rowwise_weights(N: int, K: int, seed: int = 1, std: float = 0.02):
    """Per-channel weight operand: (W uint8 [N, K], w_scale float32 [N])."""
    return quantize_per_row(normal_bf16(N, K, std, seed))
