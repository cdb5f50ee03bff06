"""Tune the exact-M selector table on one MI355X.

For every registered (N, K) and every key M -- each M from 1 to 16, then a
grid whose consecutive keys satisfy key_{i+1} = floor(1.125 * (key_i + 1)) up
to 8192 (the selector allows 1.25) -- every compiled kernel instance that
accepts M is timed, and the
fastest one becomes the table row for that key.  A request M is later served
by the smallest key >= M, so no M runs an instance tuned for more than 1.25 M.

Timing follows the cold-weight method: each call reads its own copy of W
(copies totalling >= --rotate-gib, default 1 GiB, four times the 256 MB MALL,
at most --max-copies of them; copies are sign-flipped versions of one seeded
W), R calls are captured in
one HIP graph, the graph is replayed, and the per-call time is the median of
--rounds interleaved rounds over all candidates (the pages' own tuner read
one resident weight copy, which mis-picked instances for decode).

Results are appended to tune_results.jsonl as they are measured (an
interrupted run resumes), and the table is written to tuned_table.json;
regenerate the header with gen_selector_table.py and rebuild afterwards.

With --mx the MX-scaled variant is tuned instead (E8M0 scales, seeded MX
operands; --batch b times the batched form with b problems per call), and
the shapes are stored with "mx": true -- by default the page's MX shapes,
the dense (N, K) pairs and the batched b = 8, N = 1024, K = 4096 one.

Usage: python -m fp8_block_scaled_a8w8_amd.tune [--shapes N:K,...] [--rounds 3] [--mx [--batch b]]
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

from . import gemm_a8w8_blockscale_run_variant, gemm_a8w8_mxscale_run_variant, variants
from . import gen_selector_table as gst

HERE = os.path.dirname(os.path.abspath(__file__))
RESULTS = os.path.join(HERE, "tune_results.jsonl")
REGISTERED = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144), (512, 1024)]
# MX-scaled shapes of the gfx1250 BF16 and MX32 tuned-rows page (ROCm/aiter #7247,
# Technical Details): dense (N, K) pairs, and the batched one as N:K:batch.
REGISTERED_MX = ["1792:5120", "4608:5120", "5120:2304", "5120:8192", "32768:1280", "1024:4096:8"]


# The M values the MX page times (M = 16, 48, 768) get exact keys in the MX tables.
MX_EXTRA_KEYS = (48, 768)


# Above M = 16 consecutive keys grow by 1.125 (half the 1.25 the selector allows): the
# best instance can change sharply inside one 1.25x interval of the mid-M band
# (tile-count quantisation), so the finer grid serves every M with a row tuned closer to it.
KEY_RATIO = 1.125


def key_grid(limit: int = 8192, extra=()) -> list[int]:
    keys = list(range(1, 17))
    while keys[-1] < limit:
        keys.append(min(limit, int(math.floor(KEY_RATIO * (keys[-1] + 1)))))
    return sorted(set(keys) | set(extra))


def candidates(M: int, N: int, K: int) -> list[dict]:
    out = []
    for v in variants():
        if v["kernel_name"] == "skinny":
            groups = -(-N // v["bn"])
            # split K only where the unsplit row groups leave CUs idle, with >= 2 blocks per split
            if M <= 16 and (v["splits"] == 1 or (groups < 2 * 256 and K // 128 >= 2 * v["splits"]
                                                 and groups * v["splits"] <= 8 * 256)):
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
        if v["splits"] > 1:
            # split K only where the unsplit tiles leave CUs idle, with >= 2 blocks per split
            tiles = -(-M // v["bm"]) * -(-N // v["bn"])
            if tiles >= 2 * 256 or K // 128 < 2 * v["splits"] or tiles * v["splits"] > 8 * 256 or \
                    tiles * v["splits"] * v["bm"] * v["bn"] * 4 > (128 << 20):
                continue
        out.append(v)
    return out


_SIDE_STREAM = None


def graph_for(calls):
    # One side stream for every capture: split-K plans keep one workspace per stream.
    global _SIDE_STREAM
    if _SIDE_STREAM is None:
        _SIDE_STREAM = torch.cuda.Stream()
    s = _SIDE_STREAM
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


def _operands(N: int, K: int, mx: bool, batch: int):
    """Seeded operands on the device: activations for M up to 8192, one weight copy, scales."""
    import inputgen
    dev = "cuda:0"
    if not mx:
        A, a_s = inputgen.make_activations(8192, K, seed=0)
        W0, w_s = inputgen.make_weights(N, K, seed=1)
        return [torch.from_numpy(x).to(dev) for x in (A, a_s)], W0, torch.from_numpy(w_s).to(dev)
    parts_a = [inputgen.make_mx_activations(8192, K, seed=10 * i) for i in range(batch)]
    parts_w = [inputgen.make_mx_weights(N, K, seed=10 * i + 1) for i in range(batch)]
    import numpy as np
    A = np.stack([p[0] for p in parts_a]) if batch > 1 else parts_a[0][0]
    a_s = np.stack([p[1] for p in parts_a]) if batch > 1 else parts_a[0][1]
    W0 = np.stack([p[0] for p in parts_w]) if batch > 1 else parts_w[0][0]
    w_s = np.stack([p[1] for p in parts_w]) if batch > 1 else parts_w[0][1]
    return [torch.from_numpy(x).to(dev) for x in (A, a_s)], W0, torch.from_numpy(w_s).to(dev)


def tune_shape(N: int, K: int, rounds: int, rotate_gib: float, done: dict, log,
               mx: bool = False, batch: int = 1, results_path: str = RESULTS, max_copies: int = 256) -> list[dict]:
    import inputgen
    dev = "cuda:0"
    prefix = ("mx" + (str(batch) if batch > 1 else "") + ":") if mx else ""
    grid = key_grid(extra=MX_EXTRA_KEYS if mx else ())
    if all(f"{prefix}{N}:{K}:{M}" in done for M in grid):
        return [done[f"{prefix}{N}:{K}:{M}"] for M in grid]      # all measured: no GPU needed
    (dA, da), W0, dw = _operands(N, K, mx, batch)
    R = max(2, math.ceil(rotate_gib * 2**30 / (W0.nbytes + dw.numel() * dw.element_size())))
    R = min(R, max_copies)          # tiny weights: bounded graphs (the activations dominate the traffic there)
    copies = [torch.from_numpy(W0).to(dev)] + \
        [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
    rows = []
    for M in grid:
        key = f"{prefix}{N}:{K}:{M}"
        if key in done:
            rows.append(done[key])
            continue
        cands = candidates(M, N, K)
        if mx:
            lead = (batch,) if batch > 1 else ()
            Am = (dA[:, :M] if batch > 1 else dA[:M]).contiguous()
            am = (da[:, :M] if batch > 1 else da[:M]).contiguous()
            out = torch.empty(lead + (M, N), dtype=torch.bfloat16, device=dev)
        else:
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        graphs = {}
        for v in cands:
            if mx:
                calls = [(lambda r=r, vid=v["variant"]: gemm_a8w8_mxscale_run_variant(
                    vid, Am, am, copies[r], dw, out=out)) for r in range(R)]
            else:
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
               "waves": best["waves"], "kblocks": best["kblocks"], "splits": best["splits"], "name": best["name"],
               "us": round(med[best["variant"]], 3),
               "candidates": {v["name"]: round(med[v["variant"]], 3) for v in cands}}
        rows.append(row)
        done[key] = row
        with open(results_path, "a") as f:
            f.write(json.dumps({"key": key, "row": row}) + "\n")
        log(f"{prefix}N={N} K={K} M={M:5d}: {best['name']:24s} {row['us']:9.2f} us  ({len(cands)} candidates)")
        del graphs, out
    del copies
    torch.cuda.empty_cache()
    return rows


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default=None, help="N:K[,N:K...] (MX: N:K[:batch])")
    ap.add_argument("--mx", action="store_true", help="tune the MX-scaled variant")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--max-copies", type=int, default=256, help="at most this many weight copies per graph")
    ap.add_argument("--fresh", action="store_true", help="ignore earlier results")
    ap.add_argument("--results", default=RESULTS, help="measurement log to resume from and append to")
    args = ap.parse_args(argv)
    root = os.path.dirname(HERE)
    if root not in sys.path:
        sys.path.insert(0, root)

    def log(msg):
        print(msg, flush=True)

    done = {}
    if os.path.exists(args.results) and not args.fresh:
        with open(args.results) as f:
            for line in f:
                rec = json.loads(line)
                done[rec["key"]] = rec["row"]
    table = gst.load()
    shapes = {(int(s["n"]), int(s["k"]), bool(s.get("mx", False))): s for s in table["shapes"]}
    default = REGISTERED_MX if args.mx else [f"{n}:{k}" for n, k in REGISTERED]
    for item in (args.shapes.split(",") if args.shapes else default):
        f = [int(x) for x in item.split(":")]
        N, K = f[0], f[1]
        batch = f[2] if len(f) > 2 else 1
        t = time.time()
        rows = tune_shape(N, K, args.rounds, args.rotate_gib, done, log, mx=args.mx, batch=batch,
                          results_path=args.results, max_copies=args.max_copies)
        entry = {"n": N, "k": K, "rows": [
            {k: r.get(k, 1) for k in ("key_m", "kernel", "bm", "bn", "waves", "kblocks", "splits", "name", "us")}
            for r in rows]}
        if args.mx:
            entry = {"n": N, "k": K, "mx": True, "batch": batch, "rows": entry["rows"]}
        shapes[(N, K, args.mx)] = entry
        log(f"tuned {'MX ' if args.mx else ''}N={N} K={K} batch={batch} in {time.time() - t:.1f}s")
        table = {"shapes": sorted(shapes.values(), key=gst._order)}
        gst.validate(table)
        with open(gst.TABLE_JSON, "w") as f:
            json.dump(table, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
