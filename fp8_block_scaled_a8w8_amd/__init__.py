"""Python binding of libgemm_a8w8.so, the a8w8 block-scale GEMM for MI355X (gfx950).

Argument marshalling only: every step of the GEMM runs in the HIP kernels of
the library.  torch supplies device memory and the stream.  The names mirror
the C ABI in ``include/gemm_a8w8_blockscale.h``.

    Y[m,n] = bf16( sum_kb (A_fp8 . W_fp8^T)_kb * a_scale[m,kb] * w_scale[n//128,kb] )

A ``float8_e4m3fn`` (or uint8 bytes) [M,K]; a_scale float32 [M,K/128];
W ``float8_e4m3fn`` (or uint8) [N,K]; w_scale float32 [ceil(N/128),K/128];
Y bfloat16 [M,N].

The MX-scaled variant (``gemm_a8w8_mxscale`` and its batched and packed
forms) takes E8M0 scale bytes instead: a_scale uint8 [M,K/32] (one per row
per 32-wide K group), w_scale uint8 [ceil(N/32),K/32] (one per 32x32 block),
value 2^(e-127).  The row-wise variant (``gemm_a8w8_rowwise``) takes one fp32
scale per activation row (a_scale [M]) and per weight row (w_scale [N]).

Split K across workgroups needs a caller-owned workspace (``Workspace``):
every GEMM function takes ``workspace=``; without one it runs the fastest
plan that splits no K (what the plain C entries run), with one the fastest
plan of the table row (``gemm_a8w8_ex`` in the C ABI).  A workspace serves
calls in stream order; calls that may overlap in time need one each.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgemm_a8w8.so")

A8W8_OK = 0
A8W8_ERR_NULL = 1
A8W8_ERR_SHAPE = 2
A8W8_ERR_ALIGN = 3
A8W8_ERR_ARCH = 4
A8W8_ERR_HIP = 5
A8W8_ERR_PLAN = 6
A8W8_ERR_WORKSPACE = 7
SCALE_KINDS = {"block": 0, "mx": 1, "rowwise": 2}
KERNEL_NAMES = {1: "skinny", 2: "tile", 3: "ptile", 4: "pskinny", 5: "tall", 6: "rskinny", 7: "sktile"}

EXPORTED = (
    "gemm_a8w8_blockscale",
    "gemm_a8w8_blockscale_plan",
    "gemm_a8w8_num_variants",
    "gemm_a8w8_describe_variant",
    "gemm_a8w8_blockscale_run_variant",
    "gemm_a8w8_variant_name",
    "gemm_a8w8_status_string",
    "gemm_a8w8_table_hash",
    "a8w8_quantize_1x128",
    "gemm_a8w8_blockscale_fused_quant",
    "gemm_a8w8_blockscale_fused_quant_plan",
    "a8w8_prepack_weights",
    "gemm_a8w8_blockscale_packed",
    "gemm_a8w8_blockscale_packed_run_variant",
    "gemm_a8w8_mxscale",
    "gemm_a8w8_mxscale_packed",
    "batched_gemm_a8w8_mxscale",
    "batched_gemm_a8w8_mxscale_packed",
    "gemm_a8w8_mxscale_plan",
    "gemm_a8w8_mxscale_run_variant",
    "gemm_a8w8_rowwise",
    "gemm_a8w8_rowwise_packed",
    "gemm_a8w8_rowwise_run_variant",
    "gemm_a8w8_ex",
    "gemm_a8w8_ex_plan",
    "gemm_a8w8_workspace_init",
    "gemm_a8w8_blockscale_noalloc",
)


class A8W8Error(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {gemm_a8w8_status_string(status)} (status {status})")


class Plan(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("bm", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("waves", ctypes.c_int32), ("kblocks", ctypes.c_int32),
                ("kpasses", ctypes.c_int32), ("fallback", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("key_m", ctypes.c_int64),
                ("splits", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace", ctypes.c_int64)]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}
        d["kernel_name"] = KERNEL_NAMES.get(self.kernel, "?")
        return d


class GemmDesc(ctypes.Structure):
    """a8w8_gemm_desc of the C ABI."""
    _fields_ = [("A", ctypes.c_void_p), ("a_scale", ctypes.c_void_p), ("W", ctypes.c_void_p),
                ("w_scale", ctypes.c_void_p), ("Y", ctypes.c_void_p),
                ("batch", ctypes.c_int64), ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("scale_kind", ctypes.c_int32), ("w_packed", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it was not built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m fp8_block_scaled_a8w8_amd.build or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.gemm_a8w8_blockscale.restype = ctypes.c_int
        L.gemm_a8w8_blockscale.argtypes = [vp] * 5 + [i64] * 3 + [vp]
        L.gemm_a8w8_blockscale_plan.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        L.gemm_a8w8_num_variants.restype = ctypes.c_int
        L.gemm_a8w8_num_variants.argtypes = []
        L.gemm_a8w8_describe_variant.restype = ctypes.c_int
        L.gemm_a8w8_describe_variant.argtypes = [i32, i64, i64, i64, ctypes.POINTER(Plan)]
        L.gemm_a8w8_blockscale_run_variant.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_run_variant.argtypes = [i32] + [vp] * 5 + [i64] * 3 + [vp]
        L.gemm_a8w8_variant_name.restype = ctypes.c_char_p
        L.gemm_a8w8_variant_name.argtypes = [i32]
        L.gemm_a8w8_status_string.restype = ctypes.c_char_p
        L.gemm_a8w8_status_string.argtypes = [ctypes.c_int]
        L.gemm_a8w8_table_hash.restype = ctypes.c_uint64
        L.gemm_a8w8_table_hash.argtypes = []
        L.a8w8_quantize_1x128.restype = ctypes.c_int
        L.a8w8_quantize_1x128.argtypes = [vp] * 3 + [i64] * 2 + [vp]
        L.a8w8_prepack_weights.restype = ctypes.c_int
        L.a8w8_prepack_weights.argtypes = [vp] * 2 + [i64] * 2 + [vp]
        L.gemm_a8w8_blockscale_packed.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_packed.argtypes = [vp] * 5 + [i64] * 3 + [vp]
        L.gemm_a8w8_blockscale_packed_run_variant.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_packed_run_variant.argtypes = [i32] + [vp] * 5 + [i64] * 3 + [vp]
        for name in ("gemm_a8w8_mxscale", "gemm_a8w8_mxscale_packed"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp] * 5 + [i64] * 3 + [vp]
        for name in ("batched_gemm_a8w8_mxscale", "batched_gemm_a8w8_mxscale_packed"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp] * 5 + [i64] * 4 + [vp]
        L.gemm_a8w8_mxscale_plan.restype = ctypes.c_int
        L.gemm_a8w8_mxscale_plan.argtypes = [i64, i64, i64, i32, ctypes.POINTER(Plan)]
        for name in ("gemm_a8w8_rowwise", "gemm_a8w8_rowwise_packed"):
            getattr(L, name).restype = ctypes.c_int
            getattr(L, name).argtypes = [vp] * 5 + [i64] * 3 + [vp]
        L.gemm_a8w8_rowwise_run_variant.restype = ctypes.c_int
        L.gemm_a8w8_rowwise_run_variant.argtypes = [i32] + [vp] * 5 + [i64] * 3 + [i32, vp]
        L.gemm_a8w8_mxscale_run_variant.restype = ctypes.c_int
        L.gemm_a8w8_mxscale_run_variant.argtypes = [i32] + [vp] * 5 + [i64] * 4 + [i32, vp]
        L.gemm_a8w8_ex.restype = ctypes.c_int
        L.gemm_a8w8_ex.argtypes = [ctypes.POINTER(GemmDesc), vp]
        L.gemm_a8w8_ex_plan.restype = ctypes.c_int
        L.gemm_a8w8_ex_plan.argtypes = [ctypes.POINTER(GemmDesc), i32, ctypes.POINTER(Plan)]
        L.gemm_a8w8_workspace_init.restype = ctypes.c_int
        L.gemm_a8w8_workspace_init.argtypes = [vp, i64, vp]
        L.gemm_a8w8_blockscale_noalloc.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_noalloc.argtypes = [vp] * 5 + [i64] * 3 + [vp]
        L.gemm_a8w8_blockscale_fused_quant.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_fused_quant.argtypes = [vp] * 4 + [i64] * 3 + [i32, i32, vp]
        L.gemm_a8w8_blockscale_fused_quant_plan.restype = ctypes.c_int
        L.gemm_a8w8_blockscale_fused_quant_plan.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(Plan)]
        _lib = L
    return _lib


def gemm_a8w8_status_string(status: int) -> str:
    return lib().gemm_a8w8_status_string(int(status)).decode()


def gemm_a8w8_variant_name(variant: int) -> str | None:
    r = lib().gemm_a8w8_variant_name(int(variant))
    return r.decode() if r is not None else None


def gemm_a8w8_table_hash() -> int:
    return int(lib().gemm_a8w8_table_hash())


def gemm_a8w8_num_variants() -> int:
    return int(lib().gemm_a8w8_num_variants())


def gemm_a8w8_blockscale_plan(M: int, N: int, K: int, cu_count: int = 0) -> dict:
    p = Plan()
    rc = lib().gemm_a8w8_blockscale_plan(M, N, K, cu_count, ctypes.byref(p))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale_plan")
    d = p.as_dict()
    d["name"] = gemm_a8w8_variant_name(d["variant"])
    return d


def gemm_a8w8_describe_variant(variant: int, M: int = 0, N: int = 1, K: int = 128) -> dict:
    p = Plan()
    rc = lib().gemm_a8w8_describe_variant(variant, M, N, K, ctypes.byref(p))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_describe_variant")
    d = p.as_dict()
    d["name"] = gemm_a8w8_variant_name(variant)
    return d


def _stream_handle(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check_device(named, device) -> None:
    """Every tensor contiguous, on the GPU, on `device`, which must be the current device (the
    library launches on the current device)."""
    for name, t in named:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, the other operands on {device}")
    if device.index is not None and device.index != torch.cuda.current_device():
        raise ValueError(f"operands are on {device} but the current device is cuda:{torch.cuda.current_device()}")


def _out(out, shape, device, what="out"):
    if out is None:
        return torch.empty(shape, dtype=torch.bfloat16, device=device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous bfloat16 {tuple(shape)} tensor")
    _check_device(((what, out),), device)
    return out


def _check(A, a_scale, W, w_scale, out):
    if A.dtype not in (torch.float8_e4m3fn, torch.uint8) or W.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError("A and W must be float8_e4m3fn (or raw uint8 bytes)")
    if a_scale.dtype != torch.float32 or w_scale.dtype != torch.float32:
        raise TypeError("scales must be float32")
    if A.dim() != 2 or W.dim() != 2:
        raise ValueError("A and W must be 2-D")
    M, K = A.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError(f"A is [M,{K}] but W is [N,{K2}]")
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    KB, NB = K // 128, (N + 127) // 128
    if tuple(a_scale.shape) != (M, KB) or tuple(w_scale.shape) != (NB, KB):
        raise ValueError(f"scale shapes must be [{M},{KB}] and [{NB},{KB}], got "
                         f"{tuple(a_scale.shape)} and {tuple(w_scale.shape)}")
    _check_device((("A", A), ("a_scale", a_scale), ("W", W), ("w_scale", w_scale)), A.device)
    out = _out(out, (M, N), A.device)
    return M, N, K, out


class Workspace:
    """Split-K workspace: caller-owned device memory that split plans use for their fp32 partial
    tiles and per-tile counters.  Allocated here by torch (device memory is torch's part) and
    zero-filled once by the library's own kernel (gemm_a8w8_workspace_init); every call leaves it
    ready for the next.  Calls using one workspace must run in stream order (one stream, or
    properly ordered streams); calls or graph replays that may overlap in time need one each."""

    def __init__(self, nbytes: int = 64 << 20, device=None, stream=None):
        nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device if device is not None else "cuda")
        self.nbytes = nbytes
        rc = lib().gemm_a8w8_workspace_init(self.buf.data_ptr(), nbytes, _stream_handle(stream))
        if rc != A8W8_OK:
            raise A8W8Error(rc, "gemm_a8w8_workspace_init")

    def ptr(self) -> int:
        return self.buf.data_ptr()


def _desc(A, a_scale, W, w_scale, out, batch, M, N, K, kind, w_packed, variant, workspace) -> GemmDesc:
    if workspace is not None and workspace.buf.device != A.device:
        raise ValueError(f"the workspace is on {workspace.buf.device}, the operands on {A.device}")
    return GemmDesc(A.data_ptr(), a_scale.data_ptr(), W.data_ptr(), w_scale.data_ptr(), out.data_ptr(),
                    batch, M, N, K, SCALE_KINDS[kind], 1 if w_packed else 0, -1 if variant is None else int(variant),
                    0, workspace.ptr() if workspace is not None else None,
                    workspace.nbytes if workspace is not None else 0)


def _ex_launch(desc: GemmDesc, stream, what: str) -> None:
    rc = lib().gemm_a8w8_ex(ctypes.byref(desc), _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, what)


def gemm_a8w8_blockscale(A: torch.Tensor, a_scale: torch.Tensor, W: torch.Tensor,
                         w_scale: torch.Tensor, out: torch.Tensor | None = None,
                         stream=None, workspace: Workspace | None = None) -> torch.Tensor:
    """Y = A . W^T with 1x128 activation / 128x128 weight fp32 block scales; returns bf16 [M,N].
    With a workspace the call may split K across workgroups (gemm_a8w8_ex)."""
    M, N, K, out = _check(A, a_scale, W, w_scale, out)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, 1, M, N, K, "block", False, None, workspace), stream,
                   "gemm_a8w8_ex")
        return out
    rc = lib().gemm_a8w8_blockscale(A.data_ptr(), a_scale.data_ptr(), W.data_ptr(),
                                    w_scale.data_ptr(), out.data_ptr(), M, N, K,
                                    _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale")
    return out


def gemm_a8w8_blockscale_noalloc(A, a_scale, W, w_scale, out=None, stream=None) -> torch.Tensor:
    """gemm_a8w8_blockscale_noalloc of the C ABI: the table's fastest plan (split K included) with
    the library's static scratch as workspace; the C call allocates nothing (``out`` may be given
    so that nothing is allocated here either).  Calls overlapping in time on one GPU race."""
    M, N, K, out = _check(A, a_scale, W, w_scale, out)
    rc = lib().gemm_a8w8_blockscale_noalloc(A.data_ptr(), a_scale.data_ptr(), W.data_ptr(), w_scale.data_ptr(),
                                            out.data_ptr(), M, N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale_noalloc")
    return out


def gemm_a8w8_blockscale_run_variant(variant: int, A, a_scale, W, w_scale, out=None, stream=None, workspace=None):
    """Same as gemm_a8w8_blockscale with a fixed kernel instance (tuning and tests); split
    instances need a workspace."""
    M, N, K, out = _check(A, a_scale, W, w_scale, out)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, 1, M, N, K, "block", False, variant, workspace), stream,
                   f"gemm_a8w8_ex(variant {variant})")
        return out
    rc = lib().gemm_a8w8_blockscale_run_variant(variant, A.data_ptr(), a_scale.data_ptr(),
                                                W.data_ptr(), w_scale.data_ptr(), out.data_ptr(),
                                                M, N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, f"gemm_a8w8_blockscale_run_variant({variant})")
    return out


def gemm_a8w8_ex(A, a_scale, W, w_scale, *, scale_kind: str = "block", packed_n: int | None = None,
                 variant: int | None = None, workspace: Workspace | None = None, out=None, stream=None):
    """gemm_a8w8_ex of the C ABI: any scale kind ("block", "mx", "rowwise"), row-major or packed W
    (packed_n = real row count), 2-D operands or batched 3-D MX operands, an optional forced
    instance and an optional workspace (split-K and stream-K plans)."""
    if scale_kind == "mx":
        batched = A.dim() == 3
        batch, M, N, K, out = _check_mx(A, a_scale, W, w_scale, out, batched, packed_n)
    elif scale_kind == "rowwise":
        M, N, K, out = _check_rowwise(A, a_scale, W, w_scale, out, packed_n)
        batch = 1
    elif scale_kind == "block":
        Wc = W if packed_n is None else _packed_view(W, packed_n)
        M, N, K, out = _check(A, a_scale, Wc, w_scale, out)
        batch = 1
    else:
        raise ValueError(f"scale_kind must be one of {sorted(SCALE_KINDS)}")
    _ex_launch(_desc(A, a_scale, W, w_scale, out, batch, M, N, K, scale_kind, packed_n is not None, variant,
                     workspace), stream, "gemm_a8w8_ex")
    return out


def gemm_a8w8_ex_plan(M: int, N: int, K: int, *, scale_kind: str = "block", batch: int = 1,
                      variant: int | None = None, workspace_bytes: int = 0, cu_count: int = 0,
                      packed: bool = False) -> dict:
    """The plan gemm_a8w8_ex launches for this shape with `workspace_bytes` of workspace
    (host only; packed: weights in the packed layout); plan["workspace"] is the workspace it uses."""
    d = GemmDesc(None, None, None, None, None, batch, M, N, K, SCALE_KINDS[scale_kind], 1 if packed else 0,
                 -1 if variant is None else int(variant), 0, None, int(workspace_bytes))
    p = Plan()
    rc = lib().gemm_a8w8_ex_plan(ctypes.byref(d), cu_count, ctypes.byref(p))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_ex_plan")
    r = p.as_dict()
    r["name"] = gemm_a8w8_variant_name(r["variant"])
    return r


def quantize_1x128(X: torch.Tensor, out: torch.Tensor | None = None, scale_out: torch.Tensor | None = None,
                   stream=None) -> tuple[torch.Tensor, torch.Tensor]:
    """bf16 activations [M,K] -> (e4m3fn codes [M,K], fp32 scales [M,K/128]), one scale per 1x128 group.

    The A / a_scale operands of gemm_a8w8_blockscale (see a8w8_quantize_1x128 in the C header)."""
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise ValueError("X must be a contiguous bfloat16 [M,K] GPU tensor")
    _check_device((("X", X),), X.device)
    M, K = X.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=X.device)
    elif out.dtype not in (torch.float8_e4m3fn, torch.uint8) or tuple(out.shape) != (M, K):
        raise ValueError("out must be a contiguous float8_e4m3fn (or uint8) [M,K] tensor")
    if scale_out is None:
        scale_out = torch.empty((M, K // 128), dtype=torch.float32, device=X.device)
    elif scale_out.dtype != torch.float32 or tuple(scale_out.shape) != (M, K // 128):
        raise ValueError("scale_out must be a contiguous float32 [M,K/128] tensor")
    _check_device((("out", out), ("scale_out", scale_out)), X.device)
    rc = lib().a8w8_quantize_1x128(X.data_ptr(), out.data_ptr(), scale_out.data_ptr(), M, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "a8w8_quantize_1x128")
    return out, scale_out


def gemm_a8w8_blockscale_fused_quant(X: torch.Tensor, W: torch.Tensor, w_scale: torch.Tensor,
                                     out: torch.Tensor | None = None, *, packed_n: int | None = None,
                                     variant: int | None = None, stream=None) -> torch.Tensor:
    """Decode (M <= 16): bf16 X [M,K] quantised per 1x128 group inside the GEMM kernel, times the
    block-scaled W; bitwise equal to quantize_1x128 then gemm_a8w8_blockscale_run_variant with the
    instance gemm_a8w8_blockscale_fused_quant_plan reports.  ``packed_n``: W is in the packed
    layout (prepack_weights) for N = packed_n rows."""
    if X.dtype != torch.bfloat16 or X.dim() != 2:
        raise ValueError("X must be a contiguous bfloat16 [M,K] GPU tensor")
    if W.dtype not in (torch.float8_e4m3fn, torch.uint8) or W.dim() != 2:
        raise TypeError("W must be a 2-D float8_e4m3fn (or raw uint8) tensor")
    if w_scale.dtype != torch.float32:
        raise TypeError("w_scale must be float32")
    Wv = W if packed_n is None else _packed_view(W, packed_n)
    M, K = X.shape
    N, K2 = Wv.shape
    if K2 != K or K % 128:
        raise ValueError(f"X is [M,{K}] and W is [N,{K2}]: K must agree and be a multiple of 128")
    if tuple(w_scale.shape) != ((N + 127) // 128, K // 128):
        raise ValueError(f"w_scale must be [{(N + 127) // 128},{K // 128}], got {tuple(w_scale.shape)}")
    _check_device((("X", X), ("W", W), ("w_scale", w_scale)), X.device)
    out = _out(out, (M, N), X.device)
    rc = lib().gemm_a8w8_blockscale_fused_quant(X.data_ptr(), W.data_ptr(), w_scale.data_ptr(), out.data_ptr(),
                                                M, N, K, 0 if packed_n is None else 1,
                                                -1 if variant is None else int(variant), _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale_fused_quant")
    return out


def gemm_a8w8_blockscale_fused_quant_plan(M: int, N: int, K: int, cu_count: int = 0,
                                          variant: int | None = None) -> dict:
    p = Plan()
    rc = lib().gemm_a8w8_blockscale_fused_quant_plan(M, N, K, cu_count, -1 if variant is None else int(variant),
                                                     ctypes.byref(p))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale_fused_quant_plan")
    d = p.as_dict()
    d["name"] = gemm_a8w8_variant_name(d["variant"])
    return d


def packed_rows(N: int) -> int:
    """Rows of the packed weight layout: N padded to a multiple of 16."""
    return (N + 15) // 16 * 16


def prepack_weights(W: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Row-major e4m3fn W [N,K] -> the packed layout (uint8 [16*ceil(N/16), K]); see the C header."""
    if W.dtype not in (torch.float8_e4m3fn, torch.uint8) or W.dim() != 2:
        raise ValueError("W must be a contiguous float8_e4m3fn (or uint8) [N,K] GPU tensor")
    _check_device((("W", W),), W.device)
    N, K = W.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    if out is None:
        out = torch.empty((packed_rows(N), K), dtype=torch.uint8, device=W.device)
    elif tuple(out.shape) != (packed_rows(N), K) or out.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"out must be a contiguous uint8 [{packed_rows(N)},{K}] tensor")
    _check_device((("out", out),), W.device)
    rc = lib().a8w8_prepack_weights(W.data_ptr(), out.data_ptr(), N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "a8w8_prepack_weights")
    return out


def _packed_view(Wp, N):
    if Wp.dtype not in (torch.float8_e4m3fn, torch.uint8) or Wp.dim() != 2:
        raise TypeError("Wp must be a 2-D uint8 (or float8_e4m3fn) tensor")
    if Wp.shape[0] != packed_rows(N):
        raise ValueError(f"packed weights for N={N} have {packed_rows(N)} rows, got {Wp.shape[0]}")
    if not Wp.is_contiguous():
        raise ValueError("Wp must be a contiguous GPU tensor")
    return Wp[:N]


def _check_packed(A, a_scale, Wp, w_scale, N, out):
    return _check(A, a_scale, _packed_view(Wp, N), w_scale, out)


def gemm_a8w8_blockscale_packed(A: torch.Tensor, a_scale: torch.Tensor, Wp: torch.Tensor, w_scale: torch.Tensor,
                                N: int, out: torch.Tensor | None = None, stream=None,
                                workspace: Workspace | None = None) -> torch.Tensor:
    """Same result as gemm_a8w8_blockscale, with W given in the packed layout (prepack_weights)."""
    M, N, K, out = _check_packed(A, a_scale, Wp, w_scale, N, out)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, Wp, w_scale, out, 1, M, N, K, "block", True, None, workspace), stream,
                   "gemm_a8w8_ex")
        return out
    rc = lib().gemm_a8w8_blockscale_packed(A.data_ptr(), a_scale.data_ptr(), Wp.data_ptr(), w_scale.data_ptr(),
                                           out.data_ptr(), M, N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_blockscale_packed")
    return out


def gemm_a8w8_blockscale_packed_run_variant(variant: int, A, a_scale, Wp, w_scale, N: int, out=None, stream=None,
                                            workspace=None):
    """gemm_a8w8_blockscale_packed with a fixed kernel instance (tuning and tests)."""
    M, N, K, out = _check_packed(A, a_scale, Wp, w_scale, N, out)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, Wp, w_scale, out, 1, M, N, K, "block", True, variant, workspace), stream,
                   f"gemm_a8w8_ex(variant {variant})")
        return out
    rc = lib().gemm_a8w8_blockscale_packed_run_variant(variant, A.data_ptr(), a_scale.data_ptr(), Wp.data_ptr(),
                                                       w_scale.data_ptr(), out.data_ptr(), M, N, K,
                                                       _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, f"gemm_a8w8_blockscale_packed_run_variant({variant})")
    return out


def variants() -> list[dict]:
    """Descriptions of every compiled kernel instance."""
    return [gemm_a8w8_describe_variant(i) for i in range(gemm_a8w8_num_variants())]


# ---------------------------------------------------------------------------
# MX-scaled variant (E8M0 scales: 1x32 activation groups, 32x32 weight blocks)

_E8M0_DTYPES = tuple(d for d in (torch.uint8, getattr(torch, "float8_e8m0fnu", None)) if d is not None)


def _check_mx(A, a_scale, W, w_scale, out, batched: bool, N: int | None = None):
    """Validate MX operands; W is row-major [.., N, K] or (N given) packed [.., 16*ceil(N/16), K]."""
    nd = 3 if batched else 2
    for name, t in (("A", A), ("W", W)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8) or t.dim() != nd:
            raise TypeError(f"{name} must be a {nd}-D float8_e4m3fn (or uint8) tensor")
    for name, t in (("a_scale", a_scale), ("w_scale", w_scale)):
        if t.dtype not in _E8M0_DTYPES or t.dim() != nd:
            raise TypeError(f"{name} must be a {nd}-D uint8 (E8M0 code) tensor")
    batch = A.shape[0] if batched else 1
    M, K = A.shape[-2:]
    rows, K2 = W.shape[-2:]
    if N is None:
        N = rows
    elif rows != packed_rows(N):
        raise ValueError(f"packed weights for N={N} have {packed_rows(N)} rows, got {rows}")
    if K2 != K:
        raise ValueError(f"A is [..,M,{K}] but W is [..,N,{K2}]")
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    lead = (batch,) if batched else ()
    if batched and (W.shape[0] != batch or a_scale.shape[0] != batch or w_scale.shape[0] != batch):
        raise ValueError("every operand needs the same batch count")
    if tuple(a_scale.shape) != lead + (M, K // 32) or tuple(w_scale.shape) != lead + ((N + 31) // 32, K // 32):
        raise ValueError(f"MX scale shapes must be {lead + (M, K // 32)} and {lead + ((N + 31) // 32, K // 32)}, "
                         f"got {tuple(a_scale.shape)} and {tuple(w_scale.shape)}")
    _check_device((("A", A), ("a_scale", a_scale), ("W", W), ("w_scale", w_scale)), A.device)
    out = _out(out, lead + (M, N), A.device)
    return batch, M, N, K, out


def _mx_call(name, A, a_scale, W, w_scale, out, batched, N, stream, workspace=None):
    packed = N is not None
    batch, M, N, K, out = _check_mx(A, a_scale, W, w_scale, out, batched, N)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, batch, M, N, K, "mx", packed, None, workspace), stream,
                   "gemm_a8w8_ex")
        return out
    args = [A.data_ptr(), a_scale.data_ptr(), W.data_ptr(), w_scale.data_ptr(), out.data_ptr()]
    args += [batch, M, N, K] if batched else [M, N, K]
    rc = getattr(lib(), name)(*args, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, name)
    return out


def gemm_a8w8_mxscale(A, a_scale, W, w_scale, out=None, stream=None, workspace=None) -> torch.Tensor:
    """MX-scaled Y = A . W^T (E8M0 scales per 1x32 activation group and 32x32 weight block); bf16 [M,N]."""
    return _mx_call("gemm_a8w8_mxscale", A, a_scale, W, w_scale, out, False, None, stream, workspace)


def gemm_a8w8_mxscale_packed(A, a_scale, Wp, w_scale, N: int, out=None, stream=None, workspace=None) -> torch.Tensor:
    """gemm_a8w8_mxscale with W in the packed layout (prepack_weights)."""
    return _mx_call("gemm_a8w8_mxscale_packed", A, a_scale, Wp, w_scale, out, False, N, stream, workspace)


def batched_gemm_a8w8_mxscale(A, a_scale, W, w_scale, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Batched MX GEMM: A [b,M,K], a_scale [b,M,K/32], W [b,N,K], w_scale [b,ceil(N/32),K/32] -> bf16 [b,M,N]."""
    return _mx_call("batched_gemm_a8w8_mxscale", A, a_scale, W, w_scale, out, True, None, stream, workspace)


def batched_gemm_a8w8_mxscale_packed(A, a_scale, Wp, w_scale, N: int, out=None, stream=None, workspace=None) -> torch.Tensor:
    """batched_gemm_a8w8_mxscale with each batch's W packed (Wp [b,16*ceil(N/16),K])."""
    return _mx_call("batched_gemm_a8w8_mxscale_packed", A, a_scale, Wp, w_scale, out, True, N, stream, workspace)


def gemm_a8w8_mxscale_plan(M: int, N: int, K: int, cu_count: int = 0) -> dict:
    p = Plan()
    rc = lib().gemm_a8w8_mxscale_plan(M, N, K, cu_count, ctypes.byref(p))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_mxscale_plan")
    d = p.as_dict()
    d["name"] = gemm_a8w8_variant_name(d["variant"])
    return d


def gemm_a8w8_mxscale_run_variant(variant: int, A, a_scale, W, w_scale, out=None, stream=None,
                                  packed_n: int | None = None, workspace=None) -> torch.Tensor:
    """MX GEMM with a fixed kernel instance; 2-D operands or 3-D (batched); packed W when packed_n is given."""
    batched = A.dim() == 3
    batch, M, N, K, out = _check_mx(A, a_scale, W, w_scale, out, batched, packed_n)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, batch, M, N, K, "mx", packed_n is not None, variant,
                         workspace), stream, f"gemm_a8w8_ex(variant {variant})")
        return out
    rc = lib().gemm_a8w8_mxscale_run_variant(variant, A.data_ptr(), a_scale.data_ptr(), W.data_ptr(),
                                             w_scale.data_ptr(), out.data_ptr(), batch, M, N, K,
                                             1 if packed_n is not None else 0, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, f"gemm_a8w8_mxscale_run_variant({variant})")
    return out


# ---------------------------------------------------------------------------
# Row-wise variant (fp32 scale per activation row and per weight row)

def _check_rowwise(A, a_scale, W, w_scale, out, N=None):
    for name, t in (("A", A), ("W", W)):
        if t.dtype not in (torch.float8_e4m3fn, torch.uint8) or t.dim() != 2:
            raise TypeError(f"{name} must be a 2-D float8_e4m3fn (or uint8) tensor")
    M, K = A.shape
    rows, K2 = W.shape
    if N is None:
        N = rows
    elif rows != packed_rows(N):
        raise ValueError(f"packed weights for N={N} have {packed_rows(N)} rows, got {rows}")
    if K2 != K or K % 128:
        raise ValueError("A and W must agree on K, a multiple of 128")
    if a_scale.dtype != torch.float32 or w_scale.dtype != torch.float32 or \
            tuple(a_scale.shape) != (M,) or tuple(w_scale.shape) != (N,):
        raise ValueError(f"row-wise scales must be float32 [{M}] and [{N}]")
    _check_device((("A", A), ("a_scale", a_scale), ("W", W), ("w_scale", w_scale)), A.device)
    out = _out(out, (M, N), A.device)
    return M, N, K, out


def gemm_a8w8_rowwise(A, a_scale, W, w_scale, out=None, stream=None, workspace=None) -> torch.Tensor:
    """Row-wise scaled Y = a_scale[m] * w_scale[n] * (A . W^T) (per-token / per-channel); bf16 [M,N]."""
    M, N, K, out = _check_rowwise(A, a_scale, W, w_scale, out)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, 1, M, N, K, "rowwise", False, None, workspace), stream,
                   "gemm_a8w8_ex")
        return out
    rc = lib().gemm_a8w8_rowwise(A.data_ptr(), a_scale.data_ptr(), W.data_ptr(), w_scale.data_ptr(),
                                 out.data_ptr(), M, N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_rowwise")
    return out


def gemm_a8w8_rowwise_packed(A, a_scale, Wp, w_scale, N: int, out=None, stream=None,
                             workspace=None) -> torch.Tensor:
    """gemm_a8w8_rowwise with W in the packed layout (prepack_weights)."""
    M, N, K, out = _check_rowwise(A, a_scale, Wp, w_scale, out, N)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, Wp, w_scale, out, 1, M, N, K, "rowwise", True, None, workspace), stream,
                   "gemm_a8w8_ex")
        return out
    rc = lib().gemm_a8w8_rowwise_packed(A.data_ptr(), a_scale.data_ptr(), Wp.data_ptr(), w_scale.data_ptr(),
                                        out.data_ptr(), M, N, K, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, "gemm_a8w8_rowwise_packed")
    return out


def gemm_a8w8_rowwise_run_variant(variant: int, A, a_scale, W, w_scale, out=None, stream=None,
                                  packed_n: int | None = None, workspace=None) -> torch.Tensor:
    """Row-wise GEMM with a fixed kernel instance; packed W when packed_n is given."""
    M, N, K, out = _check_rowwise(A, a_scale, W, w_scale, out, packed_n)
    if workspace is not None:
        _ex_launch(_desc(A, a_scale, W, w_scale, out, 1, M, N, K, "rowwise", packed_n is not None, variant,
                         workspace), stream, f"gemm_a8w8_ex(variant {variant})")
        return out
    rc = lib().gemm_a8w8_rowwise_run_variant(variant, A.data_ptr(), a_scale.data_ptr(), W.data_ptr(),
                                             w_scale.data_ptr(), out.data_ptr(), M, N, K,
                                             1 if packed_n is not None else 0, _stream_handle(stream))
    if rc != A8W8_OK:
        raise A8W8Error(rc, f"gemm_a8w8_rowwise_run_variant({variant})")
    return out
