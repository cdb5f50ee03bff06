"""Tune the exact-M selector table on one MI355X.

For every registered (N, K) and every key M -- each M from 1 to 16, then a
grid whose consecutive keys satisfy key_{i+1} = floor(1.125 * (key_i + 1)) up
to 8192 (the selector allows 1.25), plus the multiples of 128 up to 2048 and
of 256 up to 4096 -- every compiled kernel instance that
accepts M is timed, and the
fastest one becomes the table row for that key.  A request M is later served
by the smallest key >= M, so no M runs an instance tuned for more than 1.25 M.

Timing follows the cold-weight method: each call reads its own copy of W
(copies totalling >= --rotate-gib, default 2 GiB, eight times the 256 MB MALL,
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

With --form packed (fp32 block scales, weights prepacked by
a8w8_prepack_weights) or --form rowwise (per-row fp32 scales) the decode keys
M = 1..16 of that form are tuned, by default on the three decode shapes, and
stored with "form": "packed" / "rowwise"; calls of that form with M > 16 take
the block-scale table.

Usage: python -m fp8_block_scaled_a8w8_amd.tune [--shapes N:K,...] [--rounds 3] [--mx [--batch b]]
                                                [--form packed|rowwise]
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

from . import A8W8Error, Workspace, gemm_a8w8_ex, gemm_a8w8_ex_plan, variants
from . import gen_selector_table as gst

HERE = os.path.dirname(os.path.abspath(__file__))
RESULTS = os.path.join(HERE, "tune_results.jsonl")
REGISTERED = [(5120, 6144), (14336, 5120), (16384, 5120), (34816, 5120), (256, 6144), (32, 6144), (512, 1024)]
# MX-scaled shapes of the gfx1250 BF16 and MX32 tuned-rows page (ROCm/aiter #7247,
# Technical Details): dense (N, K) pairs, and the batched one as N:K:batch.
REGISTERED_MX = ["1792:5120", "4608:5120", "5120:2304", "5120:8192", "32768:1280", "1024:4096:8"]


# Decode shapes whose packed-weight and row-wise forms get decode tables of their own.
REGISTERED_DECODE = ["14336:5120", "5120:6144", "34816:5120"]
FORM_PREFIX = {"packed": "pk:", "rowwise": "rw:"}


# The M values the MX page times (M = 16, 48, 768) get exact keys in the MX tables.
MX_EXTRA_KEYS = (48, 768)


# Above M = 16 consecutive keys grow by 1.125 (half the 1.25 the selector allows): the
# best instance can change sharply inside one 1.25x interval of the mid-M band
# (tile-count quantisation), so the finer grid serves every M with a row tuned closer to it.
KEY_RATIO = 1.125
# Keys at the tile multiples of the mid-M band as well (every 128 up to 2048, every 256 up to
# 4096): a key's row is measured at the top of its interval, where the large tiles may need
# one more row of tiles than just below a multiple of their height -- M = 512 ran the row
# measured at 574, whose 256 x 256 tiles took 81 us where 128 x 256 takes 56 us at M <= 512.
TILE_KEYS = tuple(range(256, 2049, 128)) + tuple(range(2304, 4097, 256))

# An unsplit instance within this fraction of the fastest wins the row; a new pick must beat the
# production row by more than this in both re-measurements.
SPLIT_PREFERENCE = 0.02
REPLACE_MARGIN = 0.02
ROW_FIELDS = ("kernel", "bm", "bn", "waves", "kblocks", "splits", "name")


def cuts_k(v: dict) -> bool:
    """Whether the instance cuts K across workgroups (split K or stream-K): it needs a workspace."""
    return v["splits"] > 1 or v["kernel_name"] == "sktile"


def _instance(v: dict) -> dict:
    return {"kernel": v["kernel_name"], "bm": v["bm"], "bn": v["bn"], "waves": v["waves"],
            "kblocks": v["kblocks"], "splits": v["splits"], "name": v["name"]}


def pick_row(M: int, medians: dict, by_name: dict) -> dict:
    """Table row for key M from per-instance median times (us) keyed by instance name."""
    names = sorted(medians, key=lambda n: (medians[n], n))
    best = names[0]
    unsplit = [n for n in names if not cuts_k(by_name[n])]
    if cuts_k(by_name[best]) and unsplit and medians[unsplit[0]] <= (1 + SPLIT_PREFERENCE) * medians[best]:
        best = unsplit[0]
    row = {"key_m": M, **_instance(by_name[best]), "us": round(medians[best], 3)}
    others = [medians[n] for n in names if n != best]
    row["margin"] = round(min(others) / medians[best] - 1, 4) if others else None
    if cuts_k(by_name[best]):
        row["unsplit"] = {**_instance(by_name[unsplit[0]]), "us": round(medians[unsplit[0]], 3)}
    row["candidates"] = {n: round(medians[n], 3) for n in names}
    return row


def key_grid(limit: int = 8192, extra=()) -> list[int]:
    keys = list(range(1, 17))
    while keys[-1] < limit:
        keys.append(min(limit, int(math.floor(KEY_RATIO * (keys[-1] + 1)))))
    return sorted(set(keys) | set(extra))


def candidates(M: int, N: int, K: int, packed: bool = False) -> list[dict]:
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
        if v["kernel_name"] == "rskinny":
            # the instance must take the shape: each workgroup's run of rows within its tiles
            if M <= 16:
                try:
                    gemm_a8w8_ex_plan(M, N, K, variant=v["variant"], packed=packed)
                    out.append(v)
                except A8W8Error:
                    pass
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


def _operands(N: int, K: int, mx: bool, batch: int, form: str | None = None):
    """Seeded operands on the device: activations for M up to 8192, one weight copy, scales."""
    import inputgen
    dev = "cuda:0"
    if form == "rowwise":
        A, a_s = inputgen.make_rowwise_activations(8192, K, seed=0)
        W0, w_s = inputgen.make_rowwise_weights(N, K, seed=1)
        return [torch.from_numpy(x).to(dev) for x in (A, a_s)], W0, torch.from_numpy(w_s).to(dev)
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


def _measure(cands, make_calls, R: int, rounds: int) -> dict:
    """Median us per call of each candidate: one graph of R calls each, `rounds` interleaved rounds."""
    graphs = {v["name"]: graph_for(make_calls(v)) for v in cands}
    # replays per measurement: about 4 ms of work, at least 2
    probe = time_graph(graphs[cands[0]["name"]], 1)
    reps = max(2, min(50, int(4.0 / max(probe, 1e-3))))
    times = {v["name"]: [] for v in cands}
    for _ in range(rounds):
        for v in cands:
            times[v["name"]].append(time_graph(graphs[v["name"]], reps) * 1000.0 / R)
    del graphs
    return {n: statistics.median(ts) for n, ts in times.items()}


def tune_shape(N: int, K: int, rounds: int, rotate_gib: float, done: dict, log,
               mx: bool = False, batch: int = 1, results_path: str = RESULTS, max_copies: int = 256,
               production: dict | None = None, retune=(), form: str | None = None) -> list[dict]:
    import inputgen
    from . import prepack_weights
    dev = "cuda:0"
    prefix = ("mx" + (str(batch) if batch > 1 else "") + ":") if mx else FORM_PREFIX.get(form, "")
    grid = key_grid(limit=16) if form else key_grid(extra=MX_EXTRA_KEYS if mx else TILE_KEYS)
    done = {k: v for k, v in done.items() if not (k.startswith(f"{prefix}{N}:{K}:") and
                                                   int(k.rsplit(":", 1)[1]) in retune)}
    if all(f"{prefix}{N}:{K}:{M}" in done for M in grid):
        return [row_from_log(done[f"{prefix}{N}:{K}:{M}"]) for M in grid]   # all measured: no GPU needed
    (dA, da), W0, dw = _operands(N, K, mx, batch, form)
    R = max(2, math.ceil(rotate_gib * 2**30 / (W0.nbytes + dw.numel() * dw.element_size())))
    R = min(R, max_copies)          # tiny weights: bounded graphs (the activations dominate the traffic there)
    copies = [torch.from_numpy(W0).to(dev)] + \
        [torch.from_numpy(inputgen.sign_flip_copy(W0, seed=1000 + r)).to(dev) for r in range(1, R)]
    if form == "packed":
        copies = [prepack_weights(c) for c in copies]
    ws = Workspace(batch * (128 << 20) + (1 << 20))
    by_name = {v["name"]: v for v in variants()}
    prod_rows = {int(r["key_m"]): r for r in (production or {}).get("rows", [])}
    rows = []
    for M in grid:
        key = f"{prefix}{N}:{K}:{M}"
        if key in done:
            rows.append(row_from_log(done[key]))
            continue
        cands = candidates(M, N, K, packed=form == "packed")
        if mx:
            lead = (batch,) if batch > 1 else ()
            Am = (dA[:, :M] if batch > 1 else dA[:M]).contiguous()
            am = (da[:, :M] if batch > 1 else da[:M]).contiguous()
            out = torch.empty(lead + (M, N), dtype=torch.bfloat16, device=dev)
        else:
            Am, am = dA[:M], da[:M]
            out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

        def make_calls(v):
            kind = "mx" if mx else "rowwise" if form == "rowwise" else "block"
            pn = N if form == "packed" else None
            return [(lambda r=r, vid=v["variant"]: gemm_a8w8_ex(Am, am, copies[r], dw, scale_kind=kind, packed_n=pn,
                                                                variant=vid, workspace=ws, out=out))
                    for r in range(R)]

        med = _measure(cands, make_calls, R, rounds)
        row = pick_row(M, med, by_name)
        row["remeasure"] = None
        prod = prod_rows.get(M)
        if prod is not None and prod.get("name") != row["name"] and prod.get("name") in by_name and \
                any(v["name"] == prod["name"] for v in cands):
            # The new pick replaces production only if it wins by > 2% twice, each time in freshly captured graphs.
            pair = [by_name[row["name"]], by_name[prod["name"]]]
            trials = []
            for _ in range(2):
                m2 = _measure(pair, make_calls, R, rounds)
                trials.append({"new": round(m2[row["name"]], 3), "production": round(m2[prod["name"]], 3)})
            accepted = all(t["new"] * (1 + REPLACE_MARGIN) < t["production"] for t in trials)
            if not accepted:
                pn = prod["name"]
                keep = {"key_m": M, **_instance(by_name[pn]), "us": round(med[pn], 3)}
                others = [t for n, t in med.items() if n != pn]
                keep["margin"] = round(min(others) / med[pn] - 1, 4) if others else None
                if cuts_k(by_name[pn]):
                    u = min((n for n in med if not cuts_k(by_name[n])), key=lambda n: (med[n], n))
                    keep["unsplit"] = {**_instance(by_name[u]), "us": round(med[u], 3)}
                keep["candidates"] = row["candidates"]
                row = keep
            row["remeasure"] = trials
            row["replaced"] = accepted
        rows.append(row)
        done[key] = row
        with open(results_path, "a") as f:
            f.write(json.dumps({"key": key, "row": row}) + "\n")
        log(f"{prefix}N={N} K={K} M={M:5d}: {row['name']:24s} {row['us']:9.2f} us  ({len(cands)} candidates)")
        del out
    del copies, ws
    torch.cuda.empty_cache()
    return rows


def table_row(r: dict) -> dict:
    """The fields of a measured row that tuned_table.json keeps."""
    keep = ("key_m",) + ROW_FIELDS + ("us", "margin", "unsplit", "remeasure", "replaced")
    return {k: r[k] for k in keep if k in r}


def parse_instance(name: str) -> dict:
    """Instance parameters from a compiled instance's name (the names the library gives them)."""
    import re
    m = re.fullmatch(r"skinny_r(\d+)_d(\d+)_w(\d+)(?:_k(\d+))?", name)
    if m:
        tpw, d, nw, sk = m.groups()
        return {"name": name, "kernel_name": "skinny", "bm": 16, "bn": 16 * int(tpw), "waves": int(nw),
                "kblocks": int(d), "splits": int(sk or 1)}
    m = re.fullmatch(r"pskinny_d(\d+)_w(\d+)_p(\d+)", name)
    if m:
        d, nw, _ = m.groups()
        return {"name": name, "kernel_name": "pskinny", "bm": 16, "bn": 16, "waves": int(nw), "kblocks": int(d),
                "splits": 1}
    m = re.fullmatch(r"(p?tile|sktile)_(\d+)x(\d+)_w(\d+)x(\d+)_s(\d+)(?:_k(\d+))?", name)
    if m:
        kern, bm, bn, wm, wn, st, sk = m.groups()
        return {"name": name, "kernel_name": kern, "bm": int(bm), "bn": int(bn), "waves": int(wm) * int(wn),
                "kblocks": int(st), "splits": int(sk or 1)}
    m = re.fullmatch(r"rskinny_t(\d+)_d(\d+)_w(\d+)_g(\d+)", name)
    if m:
        t, d, nw, _ = m.groups()
        return {"name": name, "kernel_name": "rskinny", "bm": 16, "bn": 16 * int(t), "waves": int(nw),
                "kblocks": int(d), "splits": 1}
    m = re.fullmatch(r"tall_r(\d+)_n(\d+)_d(\d+)_w(\d+)", name)
    if m:
        tpw, nt, d, nw = m.groups()
        return {"name": name, "kernel_name": "tall", "bm": 16 * int(tpw), "bn": 16 * int(nt), "waves": int(nw),
                "kblocks": int(d), "splits": 1}
    raise ValueError(f"unknown instance name {name}")


def row_from_log(rec: dict) -> dict:
    """The table row for a logged measurement: a logged two-re-measurement decision stands as it
    is; otherwise the first rule picks from the logged candidate times."""
    if rec.get("remeasure") is not None or not rec.get("candidates"):
        return rec
    med = dict(rec["candidates"])
    row = pick_row(int(rec["key_m"]), med, {n: parse_instance(n) for n in med})
    row["remeasure"] = None
    return row


def rebuild(results_path: str = RESULTS) -> dict:
    """tuned_table.json rows from the measurement log alone (first rule applied; no re-measurement,
    no library needed: instance parameters come from the recorded names)."""
    done = {}
    with open(results_path) as f:
        for line in f:
            rec = json.loads(line)
            done[rec["key"]] = rec["row"]
    table = gst.load()
    out = []
    for sh in table["shapes"]:
        b = int(sh.get("batch", 1))
        prefix = ("mx" + (str(b) if b > 1 else "") + ":") if sh.get("mx") else FORM_PREFIX.get(sh.get("form"), "")
        rows = []
        for r in sh["rows"]:
            rec = done.get(f"{prefix}{sh['n']}:{sh['k']}:{r['key_m']}")
            if rec is None or not rec.get("candidates"):
                raise ValueError(f"no measurement for key {prefix}{sh['n']}:{sh['k']}:{r['key_m']}")
            rows.append(table_row(row_from_log(rec)))
        out.append({**{k: v for k, v in sh.items() if k != "rows"}, "rows": rows})
    return {"shapes": out}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default=None, help="N:K[,N:K...] (MX: N:K[:batch])")
    ap.add_argument("--mx", action="store_true", help="tune the MX-scaled variant")
    ap.add_argument("--form", choices=sorted(FORM_PREFIX), default=None,
                    help="tune the decode keys of the packed-weight or row-wise form")
    ap.add_argument("--rounds", type=int, default=3)
    ap.add_argument("--rotate-gib", type=float, default=2.0)
    ap.add_argument("--max-copies", type=int, default=256, help="at most this many weight copies per graph")
    ap.add_argument("--fresh", action="store_true", help="ignore earlier results")
    ap.add_argument("--results", default=RESULTS, help="measurement log to resume from and append to")
    ap.add_argument("--keys", default="",
                    help="key M values to measure again even if the log has them, e.g. 1-16 or 1,2,4")
    ap.add_argument("--rebuild", action="store_true",
                    help="rewrite tuned_table.json from the measurement log (no GPU), then exit")
    args = ap.parse_args(argv)
    if args.rebuild:
        table = rebuild(args.results)
        gst.validate(table)
        with open(gst.TABLE_JSON, "w") as f:
            json.dump(table, f, indent=1)
        return 0
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
    retune = set()
    for part in filter(None, args.keys.split(",")):
        lo, _, hi = part.partition("-")
        retune.update(range(int(lo), int(hi or lo) + 1))
    table = gst.load()
    if args.mx and args.form:
        ap.error("--mx and --form are exclusive")
    shapes = {(int(s["n"]), int(s["k"]), gst.form_of(s)): s for s in table["shapes"]}
    form = "mx" if args.mx else args.form or "block"
    default = REGISTERED_MX if args.mx else REGISTERED_DECODE if args.form else [f"{n}:{k}" for n, k in REGISTERED]
    for item in (args.shapes.split(",") if args.shapes else default):
        f = [int(x) for x in item.split(":")]
        N, K = f[0], f[1]
        batch = f[2] if len(f) > 2 else 1
        t = time.time()
        rows = tune_shape(N, K, args.rounds, args.rotate_gib, done, log, mx=args.mx, batch=batch,
                          results_path=args.results, max_copies=args.max_copies,
                          production=shapes.get((N, K, form)) or (shapes.get((N, K, "block")) if args.form else None),
                          retune=retune, form=args.form)
        entry = {"n": N, "k": K, "rows": [table_row(r) for r in rows]}
        if args.mx:
            entry = {"n": N, "k": K, "mx": True, "batch": batch, "rows": entry["rows"]}
        elif args.form:
            entry = {"n": N, "k": K, "form": args.form, "rows": entry["rows"]}
        shapes[(N, K, form)] = entry
        log(f"tuned {form} N={N} K={K} batch={batch} in {time.time() - t:.1f}s")
        table = {"shapes": sorted(shapes.values(), key=gst._order)}
        gst.validate(table)
        with open(gst.TABLE_JSON, "w") as f:
            json.dump(table, f, indent=1)
    return 0


if __name__ == "__main__":
    sys.exit(main())
