"""GPU tests of the stream-K tile instances ("sktile"): the persistent tile kernel
with the last one or two waves of tiles cut into equal runs of K blocks, one
run per workgroup, and the cut tiles summed by the fixed-order fixup through
the call's workspace.

Shapes are chosen from the device's CU count so that every case of the
schedule occurs: fewer tiles than workgroups (every tile cut, several pieces
each), a tile count just above one and just above two waves (whole tiles
round-robin first, then the stream-K runs), a multiple of the grid (no cut:
the same arithmetic as the persistent kernel, bitwise) and one K block
(nothing to cut).  Each is compared with the oracle on full outputs or on
sampled rows that include rows of the last tiles; repeats are bitwise equal
(the counters are reset by every call); graph replays equal eager results;
the three scale kinds, packed weights and a batched call are covered.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, shared_workspace, variant_by_name, variant_names, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu

SK = variant_names(kinds=("sktile",))


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


def _grid(v, M, N, K):
    return g.gemm_a8w8_describe_variant(v["variant"], M, N, K)["grid"]


def _twin(v):
    """The persistent instance with the same tile and ring (no stream-K)."""
    name = v["name"].replace("sktile_", "ptile_")
    return variant_by_name(name)["variant"]


def _shapes(v, K):
    """(M, N, what) covering the schedule's cases for this instance on this device."""
    bm, bn = v["bm"], v["bn"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slots = g.gemm_a8w8_describe_variant(v["variant"], 1 << 20, 1 << 16, K)["grid"]   # cus x per-CU
    N = 3 * bn + 40                       # 4 tile columns, the last ragged
    tn = 4
    out = [(5 * bm - 7, 2 * bn - 9, "fewer tiles than workgroups")]
    for waves, extra in ((1, 37), (2, 5)):
        tiles = waves * slots + extra
        tm = -(-tiles // tn)
        out.append((tm * bm - bm // 2 - 3, N, f"{waves} wave(s) + {tm * tn - waves * slots} tiles"))
    tm = -(-slots // tn)
    out.append((tm * bm, tn * bn, "a multiple of the grid"))
    del cus
    return out


def _check(v, M, N, K, what, kind="block", packed=False):
    ws = shared_workspace()
    if kind == "block":
        A, a = inputgen.make_activations(M, K, seed=M % 97)
        W, w = inputgen.make_weights(N, K, seed=N % 89)
        ref_fn = oracle.gemm
    elif kind == "mx":
        A, a = inputgen.make_mx_activations(M, K, seed=M % 97)
        W, w = inputgen.make_mx_weights(N, K, seed=N % 89)
        ref_fn = oracle.gemm_mx
    else:
        A, a = inputgen.make_rowwise_activations(M, K, seed=M % 97)
        W, w = inputgen.make_rowwise_weights(N, K, seed=N % 89)
        ref_fn = oracle.gemm_rowwise
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"{v['name']} {kind}{' packed' if packed else ''} M={M} N={N} K={K} ({what}), grid {_grid(v, M, N, K)}")
    Wd = g.prepack_weights(dW) if packed else dW
    y = g.gemm_a8w8_ex(dA, da, Wd, dw, scale_kind=kind, packed_n=N if packed else None, variant=v["variant"],
                       workspace=ws)
    yb = y_bits(y).copy()
    for _ in range(2):                     # counters left at zero: repeats are identical
        y2 = g.gemm_a8w8_ex(dA, da, Wd, dw, scale_kind=kind, packed_n=N if packed else None, variant=v["variant"],
                            workspace=ws)
        assert np.array_equal(y_bits(y2), yb), f"{v['name']} M={M}: repeat differs"
    if M * N * K <= (1 << 33):
        assert_parity(y_host(y), ref_fn(A, a, W, w), f"{v['name']} {kind} M={M} N={N} K={K}")
    else:
        bm = v["bm"]
        rows = sorted({0, 1, bm - 1, bm, M // 2, M - 1, M - 2, M - bm, M - bm - 1, M - 2 * bm, M - 3 * bm + 5}
                      | set(np.random.default_rng(M).integers(0, M, 24).tolist()))
        rows = [r for r in rows if 0 <= r < M]
        assert_parity(y_host(y)[rows], ref_fn(A, a, W, w, rows=rows), f"{v['name']} {kind} M={M} N={N} K={K} rows")
    return dA, da, dW, dw, yb


@pytest.mark.parametrize("name", SK)
def test_stream_k_instance_every_schedule_case(name):
    v = variant_by_name(name)
    K = 640
    for (M, N, what) in _shapes(v, K):
        dA, da, dW, dw, yb = _check(v, M, N, K, what)
        if what == "a multiple of the grid":
            # no tile is cut: the persistent kernel's arithmetic, bitwise
            yp = g.gemm_a8w8_blockscale_run_variant(_twin(v), dA, da, dW, dw)
            assert np.array_equal(y_bits(yp), yb), f"{name}: uncut schedule differs from the persistent kernel"
    # one K block: nothing to cut whatever the tile count
    _check(v, 3 * v["bm"] + 1, 2 * v["bn"] + 3, 128, "one K block")


@pytest.mark.parametrize("kind", ["mx", "rowwise"])
def test_stream_k_other_scale_kinds_and_packed(kind):
    for name in SK:
        v = variant_by_name(name)
        M, N, what = _shapes(v, 1024)[1]
        _check(v, M, N, 1024, what, kind=kind)
        _check(v, M, N, 1024, what, kind="block", packed=True)


def test_stream_k_batched_mx():
    v = variant_by_name(SK[0])
    b, M, N, K = 2, 3 * v["bm"] + 11, 5 * v["bn"] - 7, 1280
    parts = [(inputgen.make_mx_activations(M, K, seed=60 + i), inputgen.make_mx_weights(N, K, seed=70 + i))
             for i in range(b)]
    A = np.stack([p[0][0] for p in parts])
    a = np.stack([p[0][1] for p in parts])
    W = np.stack([p[1][0] for p in parts])
    w = np.stack([p[1][1] for p in parts])
    need = g.gemm_a8w8_ex_plan(M, N, K, scale_kind="mx", batch=b, variant=v["variant"],
                               workspace_bytes=1 << 40)["workspace"]
    say(f"{v['name']} batched MX b={b} M={M} N={N} K={K}: workspace {need}")
    y = y_host(g.gemm_a8w8_mxscale_run_variant(v["variant"], *_dev(A, a, W, w), workspace=g.Workspace(need)))
    for i in range(b):
        assert_parity(y[i], oracle.gemm_mx(A[i], a[i], W[i], w[i]), f"stream-K batch {i}")


def test_stream_k_graph_replays_equal_eager():
    for name in SK:
        v = variant_by_name(name)
        M, N, _ = _shapes(v, 640)[1]
        A, a = inputgen.make_activations(M, 640, seed=5)
        W, w = inputgen.make_weights(N, 640, seed=6)
        dA, da, dW, dw = _dev(A, a, W, w)
        ws = shared_workspace()
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        call = lambda: g.gemm_a8w8_ex(dA, da, dW, dw, variant=v["variant"], workspace=ws, out=out)
        call()
        torch.cuda.synchronize()
        eager = y_bits(out).copy()
        s = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            call()
        for i in range(3):
            out.fill_(0)
            graph.replay()
            torch.cuda.synchronize()
            assert np.array_equal(y_bits(out), eager), f"{name}: replay {i} differs from eager"
            call()
            torch.cuda.synchronize()
        del graph
        say(f"{name} M={M} N={N}: graph == eager")


def test_stream_k_needs_its_workspace():
    v = variant_by_name(SK[0])
    M, N, _ = _shapes(v, 640)[0]
    A, a = inputgen.make_activations(M, 640, seed=1)
    W, w = inputgen.make_weights(N, 640, seed=2)
    dA, da, dW, dw = _dev(A, a, W, w)
    need = g.gemm_a8w8_ex_plan(M, N, 640, variant=v["variant"], workspace_bytes=1 << 40)["workspace"]
    assert need > 65536
    out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g.A8W8Error) as e:
        g.gemm_a8w8_ex(dA, da, dW, dw, variant=v["variant"], workspace=g.Workspace(need - 256), out=out)
    assert e.value.status == g.A8W8_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out.float() == 3.0).all()), "a refused call must not launch"
