"""GPU tests of split-K plans (tile and skinny kernels, several workgroups
per output tile, fp32 partials in the stream's workspace, the last split of a
tile sums them in split order and resets the tile's counter).

Checked: every split instance against the oracle and against its unsplit
twin where one is registered (both within tolerance), bitwise run-to-run
determinism over repeated calls (the counters must come back to zero), all
three scale kinds, batched calls, a captured HIP graph replayed between eager
calls, a call captured on a stream that has no workspace yet (it must run
unsplit: bitwise equal to the unsplit instance), and two streams running
split plans at once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


def _split_ids():
    return [v["variant"] for v in g.variants() if v["splits"] > 1]


def _twin(v):
    """The registered unsplit instance of the same kernel and shape, or None."""
    for u in g.variants():
        if (u["kernel_name"], u["bm"], u["bn"], u["waves"], u["kblocks"], u["splits"]) == \
                (v["kernel_name"], v["bm"], v["bn"], v["waves"], v["kblocks"], 1):
            return u["variant"]
    return None


def _split_shape(v, K_extra=384):
    """A ragged shape for a split instance: K blocks do not divide evenly over the splits."""
    K = 256 * v["splits"] + K_extra
    if v["kernel_name"] == "skinny":
        return 11, 2 * v["bn"] + 40, K
    return 2 * v["bm"] + 7, 2 * v["bn"] + 40, K


def test_split_instances_exist_and_describe_themselves():
    ids = _split_ids()
    kinds = [g.gemm_a8w8_describe_variant(i)["kernel_name"] for i in ids]
    assert kinds.count("tile") >= 20 and kinds.count("skinny") >= 6
    for vid in ids:
        M = 16 if g.gemm_a8w8_describe_variant(vid)["kernel_name"] == "skinny" else 300
        v = g.gemm_a8w8_describe_variant(vid, M, 500, 4096)
        assert v["name"].endswith(f"_k{v['splits']}")
        tiles = -(-M // v["bm"]) * -(-500 // v["bn"])
        assert v["grid"] == tiles * v["splits"]
    for v in g.variants():
        if v["splits"] > 1 and v["kernel_name"] == "tile":
            assert _twin(v) is not None, v["name"]


@pytest.mark.parametrize("vid_index", range(40))
def test_every_split_instance_block_scale(vid_index):
    ids = _split_ids()
    if vid_index >= len(ids):
        pytest.skip("no such split instance")
    vid = ids[vid_index]
    v = g.gemm_a8w8_describe_variant(vid)
    M, N, K = _split_shape(v)
    A, a = inputgen.make_activations(M, K, seed=vid)
    W, w = inputgen.make_weights(N, K, seed=vid + 1)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"split {v['name']} M={M} N={N} K={K}")
    y1 = g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw)
    y1b = y_bits(y1).copy()
    for _ in range(3):                               # counters reset: every repeat is identical
        y2 = g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw)
        assert np.array_equal(y_bits(y2), y1b), f"{v['name']} not reproducible"
    ref = oracle.gemm(A, a, W, w)
    assert_parity(y_host(y1), ref, f"{v['name']}")
    if _twin(v) is not None:
        yu = g.gemm_a8w8_blockscale_run_variant(_twin(v), dA, da, dW, dw)
        assert_parity(y_host(yu), ref, f"{v['name']} twin")


@pytest.mark.parametrize("kind", ["mx", "rowwise"])
def test_split_instances_other_scale_kinds(kind):
    ids = _split_ids()
    for vid in ids[::3] + [i for i in ids if g.gemm_a8w8_describe_variant(i)["kernel_name"] == "skinny"]:
        v = g.gemm_a8w8_describe_variant(vid)
        M, N, K = _split_shape(v, 128)
        if kind == "mx":
            A, a = inputgen.make_mx_activations(M, K, seed=vid)
            W, w = inputgen.make_mx_weights(N, K, seed=vid + 1)
            y = g.gemm_a8w8_mxscale_run_variant(vid, *_dev(A, a, W, w))
            ref = oracle.gemm_mx(A, a, W, w)
        else:
            A, a = inputgen.make_rowwise_activations(M, K, seed=vid)
            W, w = inputgen.make_rowwise_weights(N, K, seed=vid + 1)
            y = g.gemm_a8w8_rowwise_run_variant(vid, *_dev(A, a, W, w))
            ref = oracle.gemm_rowwise(A, a, W, w)
        assert_parity(y_host(y), ref, f"{kind} {v['name']}")
    say(f"split instances, {kind} scales: ok")


def _first_split(kernel, splits):
    return next(i for i in _split_ids() if (g.gemm_a8w8_describe_variant(i)["kernel_name"],
                                            g.gemm_a8w8_describe_variant(i)["splits"]) == (kernel, splits))


@pytest.mark.parametrize("kernel", ["tile", "skinny"])
def test_split_batched_mx(kernel):
    vid = _first_split(kernel, 4)
    v = g.gemm_a8w8_describe_variant(vid)
    b, M, N, K = 3, (v["bm"] + 5 if kernel == "tile" else 13), v["bn"] * 2 + 8, 2048
    parts = [(inputgen.make_mx_activations(M, K, seed=10 + i), inputgen.make_mx_weights(N, K, seed=20 + i))
             for i in range(b)]
    A = np.stack([p[0][0] for p in parts])
    a = np.stack([p[0][1] for p in parts])
    W = np.stack([p[1][0] for p in parts])
    w = np.stack([p[1][1] for p in parts])
    y = y_host(g.gemm_a8w8_mxscale_run_variant(vid, *_dev(A, a, W, w)))
    for i in range(b):
        assert_parity(y[i], oracle.gemm_mx(A[i], a[i], W[i], w[i]), f"batch {i}")


def _graph_case(kernel):
    vid = _first_split(kernel, 4)
    v = g.gemm_a8w8_describe_variant(vid)
    M, N, K = (2 * v["bm"] + 3 if kernel == "tile" else 7), 3 * v["bn"], 4096
    A, a = inputgen.make_activations(M, K, seed=3)
    W, w = inputgen.make_weights(N, K, seed=4)
    return vid, v, A, a, W, w


@pytest.mark.parametrize("kernel", ["tile", "skinny"])
def test_split_plan_in_a_captured_graph(kernel):
    vid, v, A, a, W, w = _graph_case(kernel)
    dA, da, dW, dw = _dev(A, a, W, w)
    s = torch.cuda.Stream()
    out = torch.empty((A.shape[0], W.shape[0]), dtype=torch.bfloat16, device=DEV)
    with torch.cuda.stream(s):
        g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, out=out)      # workspace for this stream
    torch.cuda.synchronize()
    eager = y_bits(out).copy()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, out=out)
    for _ in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(y_bits(out), eager)
        with torch.cuda.stream(s):                                            # eager work in between
            g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw)
        torch.cuda.synchronize()
    assert_parity(y_host(out), oracle.gemm(A, a, W, w), "graph replay")


@pytest.mark.parametrize("kernel", ["tile", "skinny"])
def test_capture_without_workspace_runs_unsplit(kernel):
    vid, v, A, a, W, w = _graph_case(kernel)
    dA, da, dW, dw = _dev(A, a, W, w)
    if _twin(v) is None:
        twin = None
    else:
        twin = g.gemm_a8w8_blockscale_run_variant(_twin(v), dA, da, dW, dw)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()                          # fresh stream: no workspace yet
    out = torch.empty((A.shape[0], W.shape[0]), dtype=torch.bfloat16, device=DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, out=out)
    graph.replay()
    torch.cuda.synchronize()
    if twin is not None:
        assert np.array_equal(y_bits(out), y_bits(twin))
    assert_parity(y_host(out), oracle.gemm(A, a, W, w), f"{v['name']} captured unsplit")


@pytest.mark.parametrize("kernel", ["tile", "skinny"])
def test_two_streams_run_split_plans_together(kernel):
    vid, v, A, a, W, w = _graph_case(kernel)
    dA, da, dW, dw = _dev(A, a, W, w)
    A2, a2 = inputgen.make_activations(A.shape[0], A.shape[1], seed=33)
    dA2, da2 = _dev(A2, a2)
    ref1 = y_bits(g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw)).copy()
    ref2 = y_bits(g.gemm_a8w8_blockscale_run_variant(vid, dA2, da2, dW, dw)).copy()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs1, outs2 = [], []
    for _ in range(6):
        with torch.cuda.stream(s1):
            outs1.append(g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw))
        with torch.cuda.stream(s2):
            outs2.append(g.gemm_a8w8_blockscale_run_variant(vid, dA2, da2, dW, dw))
    torch.cuda.synchronize()
    for o1, o2 in zip(outs1, outs2):
        assert np.array_equal(y_bits(o1), ref1) and np.array_equal(y_bits(o2), ref2)
