"""Tune the exact-M selector table on one MI355X.

For every registered (N, K) and every key M -- each M from 1 to 16, then a
grid whose consecutive keys satisfy key_{i+1} <= 1.25 * (key_i + 1) up to
8192 -- every compiled kernel instance that accepts M is timed, and the
fastest one becomes the table row for that key.  A request M is later served
by the smallest key >= M, so no M runs an instance tuned for more than 1.25 M.

Timing follows the cold-weight method: each call reads its own copy of W
(copies totalling >= --rotate-gib, default 1 GiB, four times the 256 MB MALL;
copies are sign-flipped versions of one seeded W), R calls are captured in
one HIP graph, the graph is replayed, and the per-call time is the median of
--rounds interleaved rounds over all candidates (the pages' own tuner read
one resident weight copy, which mis-picked instances for decode).

Results are appended to tune_results.jsonl as they are measured (an
interrupted run resumes), and the table is written to tuned_table.json;
regenerate the header with gen_selector_table.py and rebuild afterwards.

Usage: python -m fp8_block_scaled_a8w8_amd.tune [--shapes N:K,...] [--rounds 3]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

import torch

from . import gemm_a8w8_blockscale_run_variant, variants
from . import gen_selector_table as gst

HERE = os.path.dirname(os.path.abspath(__file__))
RESULTS = os.path.join(HERE, "tune_results.jsonl")
REGISTERED = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144), (512, 1024)]


def key_grid(limit: int = 8192) -> list[int]:
    keys = list(range(1, 17))
    while keys[-1] < limit:
        keys.append(min(limit, int(math.floor(1.25 * (keys[-1] + 1)))))
    return keys


def candidates(M: int, N: int, K: int) -> list[dict]:
    out = []
    for v in variants():
        if v["kernel_name"] == "skinny":
            if M <= 16:
                out.append(v)
            continue
        if v["kernel_name"] == "pskinny":
            if M <= 16 and K // 128 <= v["waves"] * v["kblocks"]:
                out.append(v)
            continue
        if v["kernel_name"] == "tall":
            if N <= v["bn"] < 2 * max(N, 16):
                out.append(v)
            continue
        # tile instances: skip tiles far taller than M and tiles much wider than N
        if v["bm"] > max(32, 2 * M) or (N <= 32 and v["bn"] > 32) or v["bn"] > max(32, 2 * N):
            continue
        if M <= 16 and v["bm"] > 32:
            continue
        if M >= 1024 and N >= 1024 and v["bm"] * v["bn"] < 128 * 128:
            continue
        out.append(v)
    return out


def graph_for(calls):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps: int) -> float:
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    t0.record()
    for _ in range(reps):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / reps


def tune_shape(N: int, K: int, rounds: int, rotate_gib: float, done: dict, log) -> list[dict]:
    import inputgen
    dev = "cuda:0"
    A, a_s = inputgen.make_activations(8192, K, seed=0)
    W0, w_s = inputgen.make_weights(N, K, seed=1)
    dA = torch.from_numpy(A).to(dev)
    da = torch.from_numpy(a_s).to(dev)
    dw = torch.from_numpy(w_s).to(dev)
    R = max(2, math.ceil(rotate_gib * 2**30 / (W0.nbytes + w_s.nbytes)))
    copies = [torch.from_numpy(W0).to(dev)] + \
        [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
    rows = []
    for M in key_grid():
        key = f"{N}:{K}:{M}"
        if key in done:
            rows.append(done[key])
            continue
        cands = candidates(M, N, K)
        out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        graphs = {}
        for v in cands:
            calls = [(lambda r=r, vid=v["variant"]: gemm_a8w8_blockscale_run_variant(
                vid, dA[:M], da[:M], copies[r], dw, out=out)) for r in range(R)]
            graphs[v["variant"]] = graph_for(calls)
        # replays per measurement: about 4 ms of work, at least 2
        probe = time_graph(graphs[cands[0]["variant"]], 1)
        reps = max(2, min(50, int(4.0 / max(probe, 1e-3))))
        times = {v["variant"]: [] for v in cands}
        for _ in range(rounds):
            for v in cands:
                times[v["variant"]].append(time_graph(graphs[v["variant"]], reps) * 1000.0 / R)
        med = {vid: statistics.median(ts) for vid, ts in times.items()}
        best = min(cands, key=lambda v: med[v["variant"]])
        row = {"key_m": M, "kernel": best["kernel_name"], "bm": best["bm"], "bn": best["bn"],
               "waves": best["waves"], "kblocks": best["kblocks"], "name": best["name"],
               "us": round(med[best["variant"]], 3),
               "candidates": {v["name"]: round(med[v["variant"]], 3) for v in cands}}
        rows.append(row)
        done[key] = row
        with open(RESULTS, "a") as f:
            f.write(json.dumps({"key": key, "row": row}) + "\n")
        log(f"N={N} K={K} M={M:5d}: {best['name']:24s} {row['us']:9.2f} us  ({len(cands)} candidates)")
        del graphs, out
    del copies
    torch.cuda.empty_cache()
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default=",".join(f"{n}:{k}" for n, k in REGISTERED))
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--fresh", action="store_true", help="ignore earlier results")
    args = ap.parse_args(argv)
    root = os.path.dirname(HERE)
    if root not in sys.path:
        sys.path.insert(0, root)

    def log(msg):
        print(msg, flush=True)

    done = {}
    if os.path.exists(RESULTS) and not args.fresh:
        with open(RESULTS) as f:
            for line in f:
                rec = json.loads(line)
                done[rec["key"]] = rec["row"]
    table = gst.load()
    shapes = {(int(s["n"]), int(s["k"])): s for s in table["shapes"]}
    for item in args.shapes.split(","):
        N, K = (int(x) for x in item.split(":"))
        t = time.time()
        rows = tune_shape(N, K, args.rounds, args.rotate_gib, done, log)
        shapes[(N, K)] = {"n": N, "k": K, "rows": [
            {k: r[k] for k in ("key_m", "kernel", "bm", "bn", "waves", "kblocks", "name", "us")} for r in rows]}
        log(f"tuned N={N} K={K} in {time.time() - t:.1f}s")
        table = {"shapes": sorted(shapes.values(), key=lambda s: (s["n"], s["k"]))}
        gst.validate(table)
        with open(gst.TABLE_JSON, "w") as f:
            json.dump(table, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
