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


_WS = []


def shared_workspace():
    """One split-K workspace for the forced-instance calls of a test session (calls run in
    stream order on the current stream)."""
    if not _WS:
        _WS.append(g.Workspace((128 << 20) + (1 << 20)))
    return _WS[0]


def run(dA, da, dW, dw, out=None, variant=None):
    if variant is None:
        y = g.gemm_a8w8_blockscale(dA, da, dW, dw, out=out)
    else:
        y = g.gemm_a8w8_blockscale_run_variant(variant, dA, da, dW, dw, out=out, workspace=shared_workspace())
    return y


def y_host(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.to(torch.float32).cpu().numpy().astype(np.float64)


def y_bits(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.view(torch.int16).cpu().numpy()


def _variants_or_empty():
    """Every compiled instance (host-only query, made at collection time); [] when the library
    is not built, so that collecting the GPU tests never needs it."""
    try:
        return g.variants()
    except (OSError, RuntimeError):
        return []


def split_variant_names():
    """Names of the instances that split K across workgroups."""
    return [v["name"] for v in _variants_or_empty() if v["splits"] > 1]


def variant_names(kinds=None, splits=None):
    """Names of the compiled instances, optionally of some kernel families / split counts."""
    out = []
    for v in _variants_or_empty():
        if kinds is not None and v["kernel_name"] not in kinds:
            continue
        if splits is not None and (v["splits"] > 1) != splits:
            continue
        out.append(v["name"])
    return out


def variant_by_name(name):
    return next(v for v in g.variants() if v["name"] == name)
