"""Helpers shared by the GPU tests: upload seeded inputs, run through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fp8_block_scaled_a8w8_amd as g

DEV = "cuda:0"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(A, a_s, W, w_s):
    return (torch.from_numpy(np.ascontiguousarray(A)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(a_s)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(W)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(w_s)).to(DEV))


def run(dA, da, dW, dw, out=None, variant=None):
    if variant is None:
        y = g.gemm_a8w8_blockscale(dA, da, dW, dw, out=out)
    else:
        y = g.gemm_a8w8_blockscale_run_variant(variant, dA, da, dW, dw, out=out)
    return y


def y_host(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.to(torch.float32).cpu().numpy().astype(np.float64)


def y_bits(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy()
