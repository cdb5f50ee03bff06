"""GPU tests of split-K plans (tile and skinny kernels, several workgroups
per output tile, fp32 partials in a caller-owned workspace, the last split of
a tile sums them in split order and resets the tile's counter).

Checked: every split instance against the oracle and against its unsplit
twin where one is registered (both within tolerance), bitwise run-to-run
determinism over repeated calls (the counters must come back to zero), all
three scale kinds, batched calls; a forced split instance without a
workspace is refused before launch; every split plan of the tuned tables,
captured into a HIP graph on a fresh stream, replays bitwise equal to the
same call made eagerly, and its plan query names what ran; the plain entry
(no workspace) runs the row's unsplit instance, eagerly and captured; two
streams with a workspace each run split plans at once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, split_variant_names, y_bits, y_host
from tests.parity_util import assert_parity

pytestmark = pytest.mark.gpu

SPLIT_NAMES = split_variant_names()


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


def _by_name(name):
    return next(v for v in g.variants() if v["name"] == name)


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


_WS = {}


def _ws(nbytes=64 << 20):
    if nbytes not in _WS:
        _WS[nbytes] = g.Workspace(nbytes)
    return _WS[nbytes]


def test_split_instances_exist_and_describe_themselves():
    kinds = [_by_name(n)["kernel_name"] for n in SPLIT_NAMES]
    assert kinds.count("tile") >= 20 and kinds.count("skinny") >= 6
    for name in SPLIT_NAMES:
        vid = _by_name(name)["variant"]
        M = 16 if _by_name(name)["kernel_name"] == "skinny" else 300
        v = g.gemm_a8w8_describe_variant(vid, M, 500, 4096)
        assert v["name"].endswith(f"_k{v['splits']}")
        tiles = -(-M // v["bm"]) * -(-500 // v["bn"])
        assert v["grid"] == tiles * v["splits"]
        assert v["workspace"] > 0
    for v in g.variants():
        if v["splits"] > 1 and v["kernel_name"] == "tile":
            assert _twin(v) is not None, v["name"]


@pytest.mark.parametrize("name", SPLIT_NAMES)
def test_every_split_instance_block_scale(name):
    v = _by_name(name)
    vid = v["variant"]
    M, N, K = _split_shape(v)
    A, a = inputgen.make_activations(M, K, seed=vid)
    W, w = inputgen.make_weights(N, K, seed=vid + 1)
    dA, da, dW, dw = _dev(A, a, W, w)
    say(f"split {name} M={M} N={N} K={K}")
    ws = _ws()
    y1 = g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, workspace=ws)
    y1b = y_bits(y1).copy()
    for _ in range(3):                               # counters reset: every repeat is identical
        y2 = g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, workspace=ws)
        assert np.array_equal(y_bits(y2), y1b), f"{name} not reproducible"
    ref = oracle.gemm(A, a, W, w)
    assert_parity(y_host(y1), ref, name)
    if _twin(v) is not None:
        yu = g.gemm_a8w8_blockscale_run_variant(_twin(v), dA, da, dW, dw)
        assert_parity(y_host(yu), ref, f"{name} twin")


def test_split_instance_without_workspace_is_refused():
    v = _by_name(SPLIT_NAMES[0])
    M, N, K = _split_shape(v)
    A, a = inputgen.make_activations(M, K, seed=5)
    W, w = inputgen.make_weights(N, K, seed=6)
    dA, da, dW, dw = _dev(A, a, W, w)
    out = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(g.A8W8Error) as e:
        g.gemm_a8w8_blockscale_run_variant(v["variant"], dA, da, dW, dw, out=out)
    assert e.value.status == g.A8W8_ERR_WORKSPACE
    tiny = g.Workspace(256)
    with pytest.raises(g.A8W8Error) as e:
        g.gemm_a8w8_blockscale_run_variant(v["variant"], dA, da, dW, dw, out=out, workspace=tiny)
    assert e.value.status == g.A8W8_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all()), "a refused call must not launch"


@pytest.mark.parametrize("kind", ["mx", "rowwise"])
def test_split_instances_other_scale_kinds(kind):
    ws = _ws()
    for name in SPLIT_NAMES:
        v = _by_name(name)
        vid = v["variant"]
        M, N, K = _split_shape(v, 128)
        if kind == "mx":
            A, a = inputgen.make_mx_activations(M, K, seed=vid)
            W, w = inputgen.make_mx_weights(N, K, seed=vid + 1)
            y = g.gemm_a8w8_mxscale_run_variant(vid, *_dev(A, a, W, w), workspace=ws)
            ref = oracle.gemm_mx(A, a, W, w)
        else:
            A, a = inputgen.make_rowwise_activations(M, K, seed=vid)
            W, w = inputgen.make_rowwise_weights(N, K, seed=vid + 1)
            y = g.gemm_a8w8_rowwise_run_variant(vid, *_dev(A, a, W, w), workspace=ws)
            ref = oracle.gemm_rowwise(A, a, W, w)
        assert_parity(y_host(y), ref, f"{kind} {name}")
    say(f"split instances, {kind} scales: ok")


def _first_split(kernel, splits):
    return next(_by_name(n)["variant"] for n in SPLIT_NAMES
                if (_by_name(n)["kernel_name"], _by_name(n)["splits"]) == (kernel, splits))


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
    y = y_host(g.gemm_a8w8_mxscale_run_variant(vid, *_dev(A, a, W, w), workspace=_ws()))
    for i in range(b):
        assert_parity(y[i], oracle.gemm_mx(A[i], a[i], W[i], w[i]), f"batch {i}")


def _tuned_split_rows():
    """(shape entry, row) for every row of the tuned tables whose instance cuts K across
    workgroups (split K or stream-K)."""
    import json
    import os
    path = os.path.join(os.path.dirname(g.__file__), "tuned_table.json")
    with open(path) as f:
        table = json.load(f)
    out = []
    for sh in table["shapes"]:
        if sh.get("form"):          # packed / row-wise decode tables: test_gpu_forms.py
            continue
        rows = [r for r in sh["rows"] if int(r.get("splits", 1)) > 1 or r["kernel"] == "sktile"]
        if rows:
            out.append((sh, rows))
    return out


def _replay_matches_eager(call, out, what):
    """Eager call, then the same call captured on a fresh stream and replayed three times with
    eager work in between: every replay bitwise equal to the eager result."""
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
        assert np.array_equal(y_bits(out), eager), f"{what}: replay {i} differs from eager"
        call()                                            # eager work between replays
        torch.cuda.synchronize()
    del graph
    return eager


@pytest.mark.parametrize("entry", range(len(_tuned_split_rows())),
                         ids=[f"{'mx' + str(sh.get('batch', 1)) + ':' if sh.get('mx') else ''}{sh['n']}:{sh['k']}"
                              for sh, _ in _tuned_split_rows()])
def test_every_tuned_split_plan_graph_equals_eager(entry):
    """Every split row of the tuned tables at its key M: the plan gemm_a8w8_ex reports is the split
    instance of the row and is what runs (bitwise equal to forcing it); a graph captured on a
    fresh stream replays bitwise equal to eager; the plain entry (no workspace) runs the row's
    unsplit instance (its own where that needs no workspace at M), captured or not."""
    sh, rows = _tuned_split_rows()[entry]
    N, K, mx, b = int(sh["n"]), int(sh["k"]), bool(sh.get("mx")), int(sh.get("batch", 1))
    kind = "mx" if mx else "block"
    Mmax = max(int(r["key_m"]) for r in rows)
    lead = (b,) if b > 1 else ()
    if mx:
        pa = [inputgen.make_mx_activations(Mmax, K, seed=40 + i) for i in range(b)]
        pw = [inputgen.make_mx_weights(N, K, seed=50 + i) for i in range(b)]
        st = (lambda xs: np.stack(xs)) if b > 1 else (lambda xs: xs[0])
        A, a = st([p[0] for p in pa]), st([p[1] for p in pa])
        W, w = st([p[0] for p in pw]), st([p[1] for p in pw])
    else:
        A, a = inputgen.make_activations(Mmax, K, seed=40)
        W, w = inputgen.make_weights(N, K, seed=50)
    dA, da, dW, dw = _dev(A, a, W, w)
    ws = _ws(max((128 << 20) + (1 << 20), b * (40 << 20)))
    say(f"tuned split rows {kind} N={N} K={K} batch={b}: {len(rows)} keys, M up to {Mmax}")
    for r in rows:
        M = int(r["key_m"])
        Am = (dA[:, :M] if b > 1 else dA[:M]).contiguous()
        am = (da[:, :M] if b > 1 else da[:M]).contiguous()
        plan = g.gemm_a8w8_ex_plan(M, N, K, scale_kind=kind, batch=b, workspace_bytes=ws.nbytes)
        assert plan["name"] == r["name"] and plan["splits"] == int(r["splits"]), (M, plan["name"], r["name"])
        assert plan["workspace"] <= ws.nbytes
        out = torch.empty(lead + (M, N), dtype=torch.bfloat16, device=DEV)
        eager = _replay_matches_eager(
            lambda: g.gemm_a8w8_ex(Am, am, dW, dw, scale_kind=kind, workspace=ws, out=out), out,
            f"{kind} N={N} K={K} M={M} {r['name']}")
        forced = g.gemm_a8w8_ex(Am, am, dW, dw, scale_kind=kind, variant=plan["variant"], workspace=ws)
        assert np.array_equal(y_bits(forced), eager), f"M={M}: the reported plan is not what ran"
        # the plain entry: no workspace, graph == eager; it runs the row's unsplit instance, or the
        # row's own instance where that cuts nothing at this M (a stream-K grid with whole waves)
        uplan = g.gemm_a8w8_blockscale_plan(M, N, K) if not mx else g.gemm_a8w8_mxscale_plan(M, N, K)
        want = r["name"] if plan["workspace"] == 0 else r["unsplit"]["name"]
        assert uplan["name"] == want and uplan["splits"] == 1 and uplan["workspace"] == 0, (M, uplan["name"], want)
        plain = (lambda: g.gemm_a8w8_blockscale(Am, am, dW, dw, out=out)) if not mx else \
            ((lambda: g.batched_gemm_a8w8_mxscale(Am, am, dW, dw, out=out)) if b > 1 else
             (lambda: g.gemm_a8w8_mxscale(Am, am, dW, dw, out=out)))
        ue = _replay_matches_eager(plain, out, f"{kind} N={N} K={K} M={M} plain")
        forced_u = g.gemm_a8w8_ex(Am, am, dW, dw, scale_kind=kind, variant=uplan["variant"])
        assert np.array_equal(y_bits(forced_u), ue), f"M={M}: the plain plan is not what ran"
        if M == Mmax or M == int(rows[0]["key_m"]):
            # parity of both plans on sampled rows (every batch)
            rws = sorted({0, M // 2, M - 1})
            for i in range(b):
                sl = (lambda x: x[i]) if b > 1 else (lambda x: x)
                if mx:
                    ref = oracle.gemm_mx(sl(A)[:M], sl(a)[:M], sl(W), sl(w), rows=rws)
                else:
                    ref = oracle.gemm(A[:M], a[:M], W, w, rows=rws)
                for what, bits in (("split", eager), ("unsplit", ue)):
                    yb = torch.from_numpy(sl(bits)[rws].copy()).view(torch.bfloat16).float().numpy()
                    assert_parity(yb.astype(np.float64), ref, f"{kind} N={N} K={K} M={M} {what} batch {i}")


@pytest.mark.parametrize("kernel", ["tile", "skinny"])
def test_two_streams_run_split_plans_together(kernel):
    vid = _first_split(kernel, 4)
    v = g.gemm_a8w8_describe_variant(vid)
    M, N, K = (2 * v["bm"] + 3 if kernel == "tile" else 7), 3 * v["bn"], 4096
    A, a = inputgen.make_activations(M, K, seed=3)
    W, w = inputgen.make_weights(N, K, seed=4)
    dA, da, dW, dw = _dev(A, a, W, w)
    A2, a2 = inputgen.make_activations(M, K, seed=33)
    dA2, da2 = _dev(A2, a2)
    ws1, ws2 = g.Workspace(16 << 20), g.Workspace(16 << 20)
    ref1 = y_bits(g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, workspace=ws1)).copy()
    ref2 = y_bits(g.gemm_a8w8_blockscale_run_variant(vid, dA2, da2, dW, dw, workspace=ws2)).copy()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs1, outs2 = [], []
    for _ in range(6):
        with torch.cuda.stream(s1):
            outs1.append(g.gemm_a8w8_blockscale_run_variant(vid, dA, da, dW, dw, workspace=ws1))
        with torch.cuda.stream(s2):
            outs2.append(g.gemm_a8w8_blockscale_run_variant(vid, dA2, da2, dW, dw, workspace=ws2))
    torch.cuda.synchronize()
    for o1, o2 in zip(outs1, outs2):
        assert np.array_equal(y_bits(o1), ref1) and np.array_equal(y_bits(o2), ref2)
    assert_parity(y_host(outs1[0]), oracle.gemm(A, a, W, w), "stream 1")


def test_one_workspace_serves_plans_of_different_sizes():
    """Regression: one workspace shared by split calls whose tile counts differ (a small call,
    a large one, the small one again) gives the results of fresh workspaces, bitwise.  The
    counters sit in the same area for every call, so a large call never reads a small call's
    partial sums as counters."""
    vid = next(_by_name(n)["variant"] for n in SPLIT_NAMES
               if _by_name(n)["kernel_name"] == "tile" and _by_name(n)["splits"] == 4 and _by_name(n)["bm"] == 64)
    N, K = 256, 6144
    A, a = inputgen.make_activations(2000, K, seed=8)
    W, w = inputgen.make_weights(N, K, seed=9)
    dA, da, dW, dw = _dev(A, a, W, w)
    fresh = {}
    for M in (100, 2000):
        fresh[M] = g.gemm_a8w8_blockscale_run_variant(vid, dA[:M], da[:M], dW, dw, workspace=g.Workspace(32 << 20))
    ws = g.Workspace(32 << 20)
    for M in (100, 2000, 100, 2000):
        y = g.gemm_a8w8_blockscale_run_variant(vid, dA[:M], da[:M], dW, dw, workspace=ws)
        assert np.array_equal(y_bits(y), y_bits(fresh[M])), f"M={M} with a shared workspace"
    rows = [0, 999, 1999]
    assert_parity(y_host(fresh[2000])[rows], oracle.gemm(A, a, W, w, rows=rows), "M=2000")
