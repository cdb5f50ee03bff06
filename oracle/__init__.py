"""CPU fp64 oracle for the a8w8 block-scale GEMM, its MX-scaled and row-wise
(per-token / per-channel) variants and its activation quantisation step --
TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never does, and the
two share no code: the oracle carries its own e4m3fn decoder and its own
loops (``a8w8_oracle.c``, plain C in fp64).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
(exact rational brute force, exact doubling, zero scales, identity-like and
permutation weights, a numpy float64 matmul special case, the bf16 rounding
floor printed on the "Retune gfx942 ... a8w8 blockscale decode rows" page;
for ``quantize_1x128``: hand-derived codes at rounding ties, torch's fp8 cast
of the same quotients, zero groups, the group maximum, the half-spacing
error bound; for ``gemm_mx``: the E8M0 format definition, exact rational
brute force, one-group and one-block power-of-two changes that move exactly
their own K range and rows, a unit-scale numpy matmul special case, and the
reduction to ``gemm`` when every 32-wide scale of a 128-wide block agrees;
for ``gemm_rowwise``: exact rational brute force, exact power-of-two scaling
of one row and one column, zero scales, a unit-scale numpy matmul case and
the reduction to ``gemm`` with power-of-two scales).
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
        lib.a8w8_oracle_e8m0_value.restype = ctypes.c_double
        lib.a8w8_oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        lib.a8w8_oracle_gemm_rowwise.restype = ctypes.c_int
        lib.a8w8_oracle_gemm_rowwise.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + \
            [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.a8w8_oracle_gemm_mx.restype = ctypes.c_int
        lib.a8w8_oracle_gemm_mx.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + \
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


FP8_MAX = 448.0      # largest finite e4m3fn magnitude (code 0x7E)


def quantize_1x128(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per 1 x 128 activation quantisation, the step upstream of the GEMM.

    The pages name the activation operand of the op only as "FP8" with
    per-group scales; this is the project's reading (the one its inputs are
    generated with): for each row and 128-wide group along K,
    ``s = fp32(amax / 448)`` and each value becomes the e4m3fn code nearest
    to ``clamp(fp32(x / s), -448, 448)`` (ties to the even code; the sign bit
    follows the sign of the fp32 quotient, so a negative value that rounds to
    zero gives 0x80).  A group with amax 0 gets ``s = 0`` and all-zero codes.
    The quotient decides an integer, so it is formed in fp32 here exactly as
    the kernel forms it (IEEE division, round to nearest even); the encoding
    step is exact (a search over the oracle's own table of code values).

    x: float32 [M, K] (finite), K % 128 == 0.  Returns (codes uint8 [M, K],
    scales float32 [M, K/128]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    g = x.reshape(M, K // 128, 128)
    amax = np.abs(g).max(axis=-1)                                    # exact
    s = (amax / np.float32(FP8_MAX)).astype(np.float32)              # fp32 division
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        y = (g / safe[..., None]).astype(np.float32)                 # fp32 division
    y = np.clip(y, np.float32(-FP8_MAX), np.float32(FP8_MAX))
    # Non-negative finite codes 0x00..0x7E have strictly increasing values.
    vals = e4m3fn_table()[:0x7F]
    mag = np.abs(y.astype(np.float64)).ravel()
    hi = np.searchsorted(vals, mag, side="left")                     # vals[hi] >= mag
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - vals[lo]
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(mag == vals[hi], hi, code).astype(np.uint8)      # exact hits
    code = code | (np.signbit(y.ravel()).astype(np.uint8) << 7)
    code = code.reshape(M, K // 128, 128)
    code = np.where((s > 0)[..., None], code, np.uint8(0))
    return np.ascontiguousarray(code.reshape(M, K)), s


MX_GROUP = 32        # K-extent of one MX scale group; also the N-extent of a weight scale block


def e8m0_value(code: int) -> float:
    """fp64 value of one E8M0 scale byte (OCP MX: 2^(code - 127), 0xFF is NaN)."""
    return _load().a8w8_oracle_e8m0_value(int(code) & 0xFF)


def gemm_mx(A: np.ndarray, a_scale: np.ndarray, W: np.ndarray, w_scale: np.ndarray,
            rows=None) -> np.ndarray:
    """MX-scaled Y (float64) = dequant(A) . dequant(W)^T, all rows or only ``rows``.

    The mxfp8 GEMM with 32 x 32 weight-scale blocks that the gfx1250 BF16 and
    MX32 tuned-rows page (ROCm/aiter #7247) tunes, read with OCP MX scales:
    A uint8 e4m3fn [M,K]; a_scale uint8 E8M0 [M, ceil(K/32)] (one per row and
    32-wide K group); W uint8 e4m3fn [N,K]; w_scale uint8 E8M0
    [ceil(N/32), ceil(K/32)] (one per 32 x 32 block).  A value is
    e4m3fn(code) * 2^(scale - 127).  Returns [len(rows) or M, N].
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.uint8)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.uint8)
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError("A and W disagree on K")
    KG = (K + MX_GROUP - 1) // MX_GROUP
    NB = (N + MX_GROUP - 1) // MX_GROUP
    if a_scale.shape != (M, KG) or w_scale.shape != (NB, KG):
        raise ValueError("scale shapes must be [M, ceil(K/32)] and [ceil(N/32), ceil(K/32)]")
    if rows is None:
        n_rows, rows_ptr = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows, rows_ptr = rows_arr.size, rows_arr.ctypes.data
    Y = np.empty((n_rows, N), dtype=np.float64)
    rc = _load().a8w8_oracle_gemm_mx(A.ctypes.data, a_scale.ctypes.data, W.ctypes.data,
                                     w_scale.ctypes.data, M, N, K, rows_ptr, n_rows,
                                     Y.ctypes.data)
    if rc != 0:
        raise RuntimeError("a8w8_oracle_gemm_mx failed with code %d" % rc)
    return Y


def gemm_mx_batched(A, a_scale, W, w_scale, rows=None) -> np.ndarray:
    """The batched form (page: b = 8 batches of N = 1024, K = 4096): batch i is
    ``gemm_mx`` of the i-th slice of every operand.  Shapes carry a leading batch
    dimension; ``rows`` (optional) selects the same rows of every batch."""
    return np.stack([gemm_mx(A[i], a_scale[i], W[i], w_scale[i], rows=rows)
                     for i in range(A.shape[0])])


def gemm_rowwise(A: np.ndarray, a_scale: np.ndarray, W: np.ndarray, w_scale: np.ndarray,
                 rows=None) -> np.ndarray:
    """Row-wise scaled Y (float64) = a_scale[m] * w_scale[n] * (dec(A) . dec(W)^T)[m, n].

    The per-token a8w8 path (one fp32 scale per activation row, one per weight
    row / output channel), read as the plain row-wise scaled product.
    A uint8 [M,K]; a_scale float32 [M]; W uint8 [N,K]; w_scale float32 [N].
    """
    A = np.ascontiguousarray(A, dtype=np.uint8)
    W = np.ascontiguousarray(W, dtype=np.uint8)
    a_scale = np.ascontiguousarray(a_scale, dtype=np.float32).reshape(-1)
    w_scale = np.ascontiguousarray(w_scale, dtype=np.float32).reshape(-1)
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError("A and W disagree on K")
    if a_scale.size != M or w_scale.size != N:
        raise ValueError("row-wise scales must be [M] and [N]")
    if rows is None:
        n_rows, rows_ptr = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows, rows_ptr = rows_arr.size, rows_arr.ctypes.data
    Y = np.empty((n_rows, N), dtype=np.float64)
    rc = _load().a8w8_oracle_gemm_rowwise(A.ctypes.data, a_scale.ctypes.data, W.ctypes.data,
                                          w_scale.ctypes.data, M, N, K, rows_ptr, n_rows, Y.ctypes.data)
    if rc != 0:
        raise RuntimeError("a8w8_oracle_gemm_rowwise failed with code %d" % rc)
    return Y
