"""Host checks of the stream-K tile schedule (the persistent tile kernel's SKM mode).

The kernel deals whole tiles round-robin and, when the tile count T is not a
multiple of the grid G, cuts the last one or two waves of tiles into G equal
runs of K blocks.  This file restates that arithmetic (work split, run bounds,
the runs meeting a tile, the partial slot of each piece) and checks on the CPU,
for many (T, KB, G), that every block of every tile is done exactly once, that
the pieces of a cut tile are exactly the runs the fixup sums, that no two
pieces share a partial slot and that every slot and counter lies inside the
workspace the library asks for.  It also checks the library's plan and
workspace figures for the stream-K instances against the same rule.
"""
from __future__ import annotations

import pytest

import fp8_block_scaled_a8w8_amd as g


def split_work(T, G):
    full, rem = divmod(T, G)
    if rem == 0:
        return T, 0
    dp = (full - 1) * G if full >= 1 else 0
    return dp, T - dp


def schedule(T, KB, G):
    """Per workgroup rank: list of (tile, kb) steps, plus the fixup facts of each cut piece."""
    dp, sk = split_work(T, G)
    S = sk * KB
    assert S == 0 or S >= G, "the host keeps a stream-K grid no larger than the stream"
    B = lambda r: r * S // G
    work = {}
    pieces = {}          # stream-K tile -> list of (rank, first kb, count, slot)
    for rank in range(G):
        steps = []
        ntiles = (dp - 1 - rank) // G + 1 if rank < dp else 0
        for i in range(ntiles):
            steps += [(rank + i * G, kb) for kb in range(KB)]
        for s in range(B(rank), B(rank + 1)):
            steps.append((dp + s // KB, s % KB))
        work[rank] = steps
        # segments of this rank's stream-K run
        v = ntiles * KB
        while v < len(steps):
            L, kb0 = steps[v]
            n = min(KB - kb0, len(steps) - v)
            if not (kb0 == 0 and n == KB):
                tp = L - dp
                x0 = tp * KB
                r_lo = min(G - 1, ((x0 + 1) * G - 1) // S)
                r_hi = min(G - 1, ((x0 + KB) * G - 1) // S)
                slot = 2 * rank + (0 if B(rank) >= x0 else 1)
                pieces.setdefault(tp, []).append((rank, kb0, n, slot, r_lo, r_hi))
            v += n
    return dp, sk, work, pieces


CASES = [(T, KB, G) for T in (1, 7, 56, 168, 255, 256, 257, 300, 448, 511, 512, 513, 1344, 1792)
         for KB in (1, 2, 3, 40, 48) for G in (8, 64, 256, 512) if T * KB >= min(G, T * KB)]


@pytest.mark.parametrize("T,KB,G", CASES)
def test_every_block_once_and_fixup_pieces_consistent(T, KB, G):
    G = min(G, T * KB)                     # the host's grid rule: never more workgroups than blocks
    dp, sk, work, pieces = schedule(T, KB, G)
    seen = {}
    for rank, steps in work.items():
        for st in steps:
            assert st not in seen, (st, rank, seen.get(st))
            seen[st] = rank
    assert len(seen) == T * KB
    # balanced: stream-K runs differ by at most one block
    if sk:
        lens = [len(w) - ((dp - 1 - r) // G + 1 if r < dp else 0) * KB for r, w in work.items()]
        assert max(lens) - min(lens) <= 1
    used_slots = set()
    for tp, ps in pieces.items():
        assert 0 <= tp < sk
        ranks = sorted(p[0] for p in ps)
        r_lo, r_hi = ps[0][4], ps[0][5]
        assert all(p[4] == r_lo and p[5] == r_hi for p in ps)
        assert ranks == list(range(r_lo, r_hi + 1)), (tp, ranks, r_lo, r_hi)
        assert sum(p[2] for p in ps) == KB                     # the pieces cover the tile's K once
        for rank, kb0, n, slot, _, _ in ps:
            assert 0 <= slot < 2 * G
            assert slot // 2 == rank
            assert (rank, slot) not in used_slots
            used_slots.add((rank, slot))
    # a rank holds at most two pieces, in different slots
    per_rank = {}
    for ps in pieces.values():
        for rank, _, _, slot, _, _ in ps:
            per_rank.setdefault(rank, []).append(slot)
    assert all(len(v) <= 2 and len(set(v)) == len(v) for v in per_rank.values())


def _sk_variants():
    return [v for v in g.variants() if v["kernel_name"] == "sktile"]


def test_stream_k_instances_exist_and_plan_their_workspace():
    sks = _sk_variants()
    assert len(sks) >= 4
    cus = 256
    for v in sks:
        for M, N, K in ((574, 14336, 5120), (2048, 14336, 5120), (8192, 14336, 5120), (6016, 16384, 5120),
                        (300, 256, 1024)):
            plan = g.gemm_a8w8_ex_plan(M, N, K, variant=v["variant"], workspace_bytes=1 << 40, cu_count=cus)
            T = -(-M // v["bm"]) * -(-N // v["bn"])
            # one workgroup per CU (two for 128 x 128: its two-stage ring fits twice in the LDS),
            # never more than the problem's K blocks
            per_cu = 2 if (v["bm"], v["bn"]) == (128, 128) else 1
            G = plan["grid"]
            assert G == min(cus * per_cu, T * (K // 128)), (v["name"], G)
            dp, sk = split_work(T, G)
            want = 0 if sk == 0 else 65536 + 2 * G * v["bm"] * v["bn"] * 4
            assert plan["workspace"] == want, (v["name"], M, N, K, plan["workspace"], want)
            assert sk * 4 <= 65536


def test_plain_entry_never_runs_stream_k():
    for M in (300, 574, 700, 2048, 6016):
        plan = g.gemm_a8w8_blockscale_plan(M, 14336, 5120)
        assert plan["name"].split("_")[0] != "sktile", plan
