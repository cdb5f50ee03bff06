"""CPU fp64 oracle for the a8w8 block-scale GEMM -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the
two share no code: the oracle carries its own e4m3fn decoder and its own
loops (``a8w8_oracle.c``, plain C in fp64).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(exact rational brute force, exact doubling, zero scales, identity-like and
permutation weights, a numpy float64 matmul special case, the bf16 rounding
floor printed on the "Retune gfx942 ... a8w8 blockscale decode rows" page).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "a8w8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liba8w8_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp64, OpenMP, no fp contraction or fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.a8w8_oracle_e4m3fn_value.restype = ctypes.c_double
        lib.a8w8_oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
        lib.a8w8_oracle_threads.restype = ctypes.c_int
        lib.a8w8_oracle_gemm.restype = ctypes.c_int
        lib.a8w8_oracle_gemm.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + \
            [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        _lib = lib
    return _lib


def e4m3fn_value(code: int) -> float:
    """fp64 value of one e4m3fn byte (OCP 8-bit floating point, E4M3 without infinities)."""
    return _load().a8w8_oracle_e4m3fn_value(int(code) & 0xFF)


def e4m3fn_table() -> np.ndarray:
    """All 256 byte values as float64 (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else the host's cores)."""
    return _load().a8w8_oracle_threads()


def gemm(A: np.ndarray, a_scale: np.ndarray, W: np.ndarray, w_scale: np.ndarray,
         rows=None) -> np.ndarray:
    """Y (float64) = dequant(A) . dequant(W)^T for all rows, or only ``rows`` of Y.

    A uint8 [M,K]; a_scale float32 [M, ceil(K/128)]; W uint8 [N,K];
    w_scale float32 [ceil(N/128), ceil(K/128)].  Returns [len(rows) or M, N].
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError("A and W disagree on K")
    KB = (K + 127) // 128
    NB = (N + 127) // 128
    if a_scale.shape != (M, KB) or w_scale.shape != (NB, KB):
        raise ValueError("scale shapes must be [M, ceil(K/128)] and [ceil(N/128), ceil(K/128)]")
    if rows is None:
        rows_arr = None
        n_rows = M
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = rows_arr.size
        rows_ptr = rows_arr.ctypes.data
    Y = np.empty((n_rows, N), dtype=np.float64)
    rc = _load().a8w8_oracle_gemm(A.ctypes.data, a_scale.ctypes.data, W.ctypes.data,
                                  w_scale.ctypes.data, M, N, K, rows_ptr, n_rows,
                                  Y.ctypes.data)
    if rc != 0:
        raise RuntimeError("a8w8_oracle_gemm failed with code %d" % rc)
    return Y
