"""GPU parity: libgemm_a8w8.so (through its C ABI) against the fp64 CPU oracle.

Bar: rel-L2 <= 3e-3 and per-element |err| <= 2e-2 rms(ref) unless the value is
one of the two bf16 neighbours of the exact result (tests/parity_util.py).
Workloads use the seeded recipe of inputgen (A ~ N(0,1) with 1x128 scales,
W ~ N(0,0.02) with 128x128 scales) at the shapes the pages time: decode
(N,K) in {(14336,5120), (5120,6144), (34816,5120)} at every M <= 16, prefill
M in {512, 2048, 6016, 8192}, and a dense sweep of 256 random M over six
(N,K).  Large outputs are checked on sampled rows (each row of Y depends only
on its row of A, so a sampled row is checked in full).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, run, say, shared_workspace, to_dev, variant_by_name, variant_names, y_bits, y_host
from tests.parity_util import assert_parity, bf16_round

pytestmark = pytest.mark.gpu


def _inputs(M, N, K, a_seed=0, w_seed=1):
    A, a_s = inputgen.make_activations(M, K, seed=a_seed)
    W, w_s = inputgen.make_weights(N, K, seed=w_seed)
    return A, a_s, W, w_s


def test_device_is_gfx950():
    assert torch.cuda.is_available()
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name


def test_tiny_config_full():
    M, N, K = 4, 512, 1024
    A, a_s, W, w_s = _inputs(M, N, K)
    y = run(*to_dev(A, a_s, W, w_s))
    st = assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), "tiny")
    say("tiny", st)


@pytest.mark.parametrize("N,K", [(14336, 5120), (5120, 6144), (34816, 5120)])
def test_decode_every_m_up_to_16(N, K):
    A, a_s, W, w_s = _inputs(16, N, K)
    ref = oracle.gemm(A, a_s, W, w_s)                 # row m of Y depends only on row m of A
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    for M in range(1, 17):
        y = run(dA[:M], da[:M], dW, dw)
        st = assert_parity(y_host(y), ref[:M], f"decode M={M} N={N} K={K}")
        say(f"decode M={M} N={N} K={K} plan={g.gemm_a8w8_blockscale_plan(M, N, K)['name']} "
            f"rel_l2={st['rel_l2']:.3e} err_ratio={st['error_ratio']:.2e}")


def _sample_rows(M, rng, extra=()):
    rows = {0, M - 1, M // 2, *[r for r in extra if 0 <= r < M]}
    for b in (32, 64, 128, 256):
        last = ((M - 1) // b) * b
        rows.update({last, max(0, last - 1)})
    rows.update(int(r) for r in rng.integers(0, M, size=6))
    return sorted(rows)


@pytest.mark.parametrize("N,K", [(14336, 5120), (16384, 5120)])
def test_prefill_sampled_rows(N, K):
    W, w_s = inputgen.make_weights(N, K, seed=1)
    dW = torch.from_numpy(W).to(DEV)
    dw = torch.from_numpy(w_s).to(DEV)
    A_all, a_all = inputgen.make_activations(8192, K, seed=0)
    rng = np.random.default_rng(5)
    for M in (512, 2048, 6016, 8192):
        A, a_s = A_all[:M], a_all[:M]
        y = run(torch.from_numpy(A).to(DEV), torch.from_numpy(a_s).to(DEV), dW, dw)
        rows = _sample_rows(M, rng)
        yh = y_host(y)[rows]
        st = assert_parity(yh, oracle.gemm(A, a_s, W, w_s, rows=rows), f"prefill M={M} N={N}")
        say(f"prefill M={M} N={N} K={K} plan={g.gemm_a8w8_blockscale_plan(M, N, K)['name']} "
            f"rows={len(rows)} rel_l2={st['rel_l2']:.3e}")
        del y


SWEEP_NK = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144)]


def sweep_rows(M, bm, pool, count=16):
    """Rows of an M-row output to check: 0, M - 1, the rows on each side of every third tile
    boundary of the plan's tile height bm (spread evenly when there are many), then rows of a
    fixed seeded pool, `count` in all when M has that many."""
    rows = {0, M - 1}
    bounds = [k * bm for k in range(3, -(-M // bm), 3)]
    if len(bounds) > 5:
        bounds = [bounds[int(i * (len(bounds) - 1) / 4)] for i in range(5)]
    for b in bounds:
        rows.update({b - 1, b})
    for r in pool:
        if len(rows) >= min(count, M):
            break
        if r < M:
            rows.add(int(r))
    r = 1
    while len(rows) < min(count, M):
        rows.add(r)
        r += 1
    return sorted(rows)


@pytest.mark.parametrize("N,K", SWEEP_NK)
def test_dense_m_sweep_sampled_rows(N, K):
    """256 seeded M in 1..8192 through the selector with a split-K workspace (the table's
    fastest plans), 16 checked rows per M including both sides of every third tile boundary;
    every fifth M also through the plain entry (the unsplit plans)."""
    Ms = inputgen.random_m_values(256, seed=2)
    A_all, a_all = inputgen.make_activations(8192, K, seed=0)
    W, w_s = inputgen.make_weights(N, K, seed=1)
    dA, da, dW, dw = to_dev(A_all, a_all, W, w_s)
    pool = np.random.default_rng(6).permutation(8192)[:64]
    ws = g.Workspace(64 << 20)
    picked = []          # (M, rows, gpu values of those rows)
    for i, M in enumerate(Ms):
        plan = g.gemm_a8w8_ex_plan(M, N, K, workspace_bytes=ws.nbytes)
        rows = sweep_rows(M, plan["bm"], pool)
        y = g.gemm_a8w8_blockscale(dA[:M], da[:M], dW, dw, workspace=ws)
        picked.append((M, rows, y[rows].to(torch.float32).cpu().numpy().astype(np.float64)))
        if i % 5 == 0:
            y = run(dA[:M], da[:M], dW, dw)
            picked.append((M, rows, y[rows].to(torch.float32).cpu().numpy().astype(np.float64)))
    union = sorted({r for _, rows, _ in picked for r in rows})
    ref = oracle.gemm(A_all, a_all, W, w_s, rows=union)
    pos = {r: i for i, r in enumerate(union)}
    ys = np.concatenate([v for _, _, v in picked])
    refs = np.concatenate([ref[[pos[r] for r in rows]] for _, rows, _ in picked])
    st = assert_parity(ys, refs, f"sweep N={N} K={K}")
    say(f"sweep N={N} K={K}: {len(Ms)} M values, {ys.shape[0]} rows, rel_l2={st['rel_l2']:.3e} "
        f"err_ratio={st['error_ratio']:.2e}")


# ---------------------------------------------------------------- every compiled instance

@pytest.mark.parametrize("name", variant_names())
def test_every_instance_on_ragged_shape(name):
    info = variant_by_name(name)
    variant = info["variant"]
    ws = shared_workspace()
    K = max(640, 256 * info["splits"])   # split-K instances need >= 2 K blocks per split
    if info["kernel_name"] in ("skinny", "pskinny", "rskinny"):
        shapes = [(1, 300), (7, 130), (16, 64)]
    elif info["kernel_name"] == "tall":
        shapes = [(300, info["bn"]), (1000, info["bn"] - 5), (77, 3), (5, info["bn"])]
    else:
        shapes = [(77, 300), (200, 520), (33, 32)]
    for (M, N) in shapes:
        A, a_s, W, w_s = _inputs(M, N, K, a_seed=10 + M, w_seed=20 + N)
        y = g.gemm_a8w8_blockscale_run_variant(variant, *to_dev(A, a_s, W, w_s), workspace=ws)
        assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), f"{info['name']} M={M} N={N}")
    say(f"instance {info['name']} ok")


def _persistent_instances():
    return [v for v in g.variants() if v["kernel_name"] == "ptile"]


@pytest.mark.parametrize("K", [128, 640])
def test_every_persistent_instance_loops_over_tiles(K):
    """Each workgroup of a persistent tile grid takes several tiles: ragged
    M and N with at least twice as many tiles as workgroups (K = 128: one
    K block, so the copies run several tiles ahead)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(11)
    for v in _persistent_instances():
        bm, bn = v["bm"], v["bn"]
        per_cu = g.gemm_a8w8_describe_variant(v["variant"], 1 << 24, 1 << 16, K)["grid"] // 256
        N = 3 * bn + 40
        tiles_n = (N + bn - 1) // bn
        tiles_m = (2 * cus * per_cu + tiles_n - 1) // tiles_n + 1
        M = tiles_m * bm - bm // 2 - 3
        A, a_s, W, w_s = _inputs(M, N, K, a_seed=30 + bm, w_seed=40 + bn)
        y = run(*to_dev(A, a_s, W, w_s), variant=v["variant"])
        rows = _sample_rows(M, rng, extra=[bm * i + j for i in (1, tiles_m // 2, tiles_m - 1) for j in (0, bm - 1)])
        st = assert_parity(y_host(y)[rows], oracle.gemm(A, a_s, W, w_s, rows=rows),
                           f"{v['name']} M={M} N={N} K={K}")
        say(f"instance {v['name']} M={M} N={N} K={K}: {tiles_m * tiles_n} tiles on "
            f"{min(tiles_m * tiles_n, cus * per_cu)} workgroups, rel_l2={st['rel_l2']:.3e}")
        del y


def _persistent_skinny_instances():
    return [v for v in g.variants() if v["kernel_name"] == "pskinny"]


def test_every_persistent_skinny_instance_loops_over_tiles():
    """Each workgroup of a persistent skinny grid walks two or three 16-row
    tiles (ragged last tile), at K = 128 (one block: most waves idle), at the
    largest K the instance takes, and at a K that leaves the last wave's run
    of blocks short."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N = 16 * (2 * cus + 37) + 5
    for v in _persistent_skinny_instances():
        kb_max = v["waves"] * v["kblocks"]
        for K, M in ((128, 16), (128 * kb_max, 9), (128 * (kb_max - v["kblocks"] // 2 - 1), 1)):
            A, a_s, W, w_s = _inputs(M, N, K, a_seed=50 + M, w_seed=60 + K // 128)
            y = run(*to_dev(A, a_s, W, w_s), variant=v["variant"])
            st = assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), f"{v['name']} M={M} N={N} K={K}")
            say(f"instance {v['name']} M={M} N={N} K={K}: rel_l2={st['rel_l2']:.3e}")
        del y


def test_every_tall_instance_several_k_passes():
    """K = 6144 takes two or more passes of the waves over K; ragged M and N."""
    K = 6144
    for v in [v for v in g.variants() if v["kernel_name"] == "tall"]:
        M = 3 * v["bm"] + 5
        for N in (v["bn"], v["bn"] - 3):
            A, a_s, W, w_s = _inputs(M, N, K, a_seed=70 + M, w_seed=80 + N)
            y = run(*to_dev(A, a_s, W, w_s), variant=v["variant"])
            st = assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), f"{v['name']} M={M} N={N} K={K}")
            say(f"instance {v['name']} M={M} N={N} K={K}: rel_l2={st['rel_l2']:.3e}")


# ---------------------------------------------------------------- bitwise invariants

def test_identity_weights_power_of_two_scales_exact():
    M, K, N = 21, 384, 300
    A, _ = inputgen.make_activations(M, K, seed=3)
    a_s = np.ldexp(np.ones((M, K // 128), np.float32),
                   np.random.default_rng(4).integers(-6, 3, size=(M, K // 128))).astype(np.float32)
    W = np.zeros((N, K), np.uint8)
    W[np.arange(N), np.arange(N)] = 0x38
    w_s = np.ones(((N + 127) // 128, K // 128), np.float32)
    ref = oracle.gemm(A, a_s, W, w_s)
    assert np.array_equal(bf16_round(ref), ref)          # every value is a bf16
    for Mx in (M, 5):
        y = run(*to_dev(A[:Mx], a_s[:Mx], W, w_s))
        assert np.array_equal(y_host(y), ref[:Mx])


def test_integer_valued_inputs_exact():
    rng = np.random.default_rng(8)
    for M, N, K in ((9, 200, 256), (70, 96, 128)):
        A = rng.choice(np.array([0xB8, 0x00, 0x38], np.uint8), size=(M, K))
        W = rng.choice(np.array([0xB8, 0x00, 0x38], np.uint8), size=(N, K))
        a_s = np.ones((M, K // 128), np.float32)
        w_s = np.ones(((N + 127) // 128, K // 128), np.float32)
        ref = oracle.gemm(A, a_s, W, w_s)
        y = run(*to_dev(A, a_s, W, w_s))
        assert np.array_equal(y_host(y), ref)


@pytest.mark.parametrize("M,N,K", [(8, 128, 8192), (5, 100, 1024), (16, 496, 4096), (1, 1000, 3072),
                                   (3, 2000, 2048), (5, 100, 896)])
def test_heuristic_skinny_plans(M, N, K):
    # Unregistered shapes at M <= 16: the heuristic's split and unsplit skinny plans,
    # full output against the oracle and bitwise repeatable.
    plan = g.gemm_a8w8_blockscale_plan(M, N, K)
    assert plan["fallback"] == 1 and plan["kernel_name"] == "skinny"
    A, a_s = inputgen.make_activations(M, K, seed=M + N)
    W, w_s = inputgen.make_weights(N, K, seed=K)
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    say(f"heuristic {plan['name']} M={M} N={N} K={K}")
    y = g.gemm_a8w8_blockscale(dA, da, dW, dw)
    first = y_bits(y).copy()
    assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), f"heuristic {plan['name']}")
    for _ in range(2):
        assert np.array_equal(y_bits(g.gemm_a8w8_blockscale(dA, da, dW, dw)), first)


@pytest.mark.parametrize("M,N,K", [(8, 6144, 4096), (1, 12288, 4096), (16, 16384, 2048), (13, 4608, 5120)])
def test_heuristic_row_range_plans(M, N, K):
    # Unregistered shapes with >= 20 MiB of weights at M <= 16: the heuristic's row-range
    # plan, full output against the oracle and bitwise repeatable.
    plan = g.gemm_a8w8_blockscale_plan(M, N, K)
    assert plan["fallback"] == 1 and plan["kernel_name"] == "rskinny"
    A, a_s = inputgen.make_activations(M, K, seed=M + N)
    W, w_s = inputgen.make_weights(N, K, seed=K)
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    say(f"heuristic {plan['name']} M={M} N={N} K={K}")
    y = g.gemm_a8w8_blockscale(dA, da, dW, dw)
    first = y_bits(y).copy()
    assert_parity(y_host(y), oracle.gemm(A, a_s, W, w_s), f"heuristic {plan['name']}")
    assert np.array_equal(y_bits(g.gemm_a8w8_blockscale(dA, da, dW, dw)), first)


@pytest.mark.parametrize("M,N,K", [(8, 5120, 6144), (300, 1000, 1024)])
def test_doubling_activation_scales_doubles_output(M, N, K):
    A, a_s, W, w_s = _inputs(M, N, K)
    dA, da, dW, dw = to_dev(A, a_s, W, w_s)
    y1 = y_host(run(dA, da, dW, dw))
    y2 = y_host(run(dA, da * 2, dW, dw))
    assert np.array_equal(y2, 2 * y1)


@pytest.mark.parametrize("M,N,K", [(4, 14336, 5120), (1000, 2048, 1024), (8, 34816, 5120), (300, 32, 6144)])
def test_repeat_calls_bitwise_identical(M, N, K):
    A, a_s, W, w_s = _inputs(M, N, K)
    d = to_dev(A, a_s, W, w_s)
    a = y_bits(run(*d))
    for _ in range(3):
        assert np.array_equal(y_bits(run(*d)), a)


def test_graph_replay_matches_eager():
    cases = []
    for (M, N, K) in ((2, 14336, 5120), (600, 1536, 1024), (5, 34816, 5120), (700, 32, 6144)):
        A, a_s, W, w_s = _inputs(M, N, K)
        d = to_dev(A, a_s, W, w_s)
        eager = y_bits(run(*d))
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        cases.append((d, out, eager))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for d, out, _ in cases:                  # warm-up on the capture stream
            run(*d, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        for d, out, _ in cases:
            g.gemm_a8w8_blockscale(*d, out=out, stream=s)
    for rep in range(4):
        for _, out, _ in cases:
            out.fill_(0)                         # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for _, out, eager in cases:
            assert np.array_equal(y_bits(out), eager), f"replay {rep}"


# ---------------------------------------------------------------- bounds

@pytest.mark.parametrize("M,N,K", [(1, 32, 6144), (5, 130, 256), (17, 32, 6144), (33, 300, 384),
                                   (255, 256, 6144), (257, 520, 640), (6016, 96, 256), (9, 34816, 5120),
                                   (100, 30, 640), (4100, 20, 256)])
def test_output_guard_bands_untouched(M, N, K):
    A, a_s, W, w_s = _inputs(M, N, K, a_seed=M, w_seed=N)
    pad = 64
    sentinel = torch.tensor([-12345.0], dtype=torch.bfloat16).view(torch.int16).item()
    buf = torch.full((pad + M * N + pad,), sentinel, dtype=torch.int16, device=DEV)
    out = buf[pad:pad + M * N].view(torch.bfloat16).view(M, N)
    run(*to_dev(A, a_s, W, w_s), out=out)
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert np.all(b[:pad] == sentinel) and np.all(b[-pad:] == sentinel)
    assert_parity(y_host(out), oracle.gemm(A, a_s, W, w_s), f"guard M={M} N={N}")


def test_error_paths_on_device():
    A, a_s, W, w_s = _inputs(17, 64, 256)
    d = to_dev(A, a_s, W, w_s)
    skinny = [v["variant"] for v in g.variants() if v["kernel_name"] == "skinny"][0]
    with pytest.raises(g.A8W8Error) as e:
        g.gemm_a8w8_blockscale_run_variant(skinny, *d)
    assert e.value.status == g.A8W8_ERR_PLAN
    out = torch.empty((17, 64), dtype=torch.bfloat16, device=DEV)
    rc = g.lib().gemm_a8w8_blockscale(d[0].data_ptr() + 1, d[1].data_ptr(), d[2].data_ptr(),
                                      d[3].data_ptr(), out.data_ptr(), 17, 64, 256, None)
    assert rc == g.A8W8_ERR_ALIGN
