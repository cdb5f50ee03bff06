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


def host_grid(T, KB, slots):
    """The library's grid for a stream-K instance (T tiles, KB blocks each, `slots` workgroup slots)."""
    if 2 * T <= slots:
        S = min(slots // T, KB)
        if S >= 2:
            return S * T
    return min(slots, T * KB)


def split_work(T, G):
    full, rem = divmod(T, G)
    if rem == 0:
        return T, 0
    dp = (full - 1) * G if full >= 1 else 0
    return dp, T - dp


def schedule(T, KB, G):
    """Per workgroup rank: list of (tile, kb) steps, plus the fixup facts of each cut piece."""
    aligned = 2 * T <= G
    S_al = G // T if aligned else 1
    dp, sk = split_work(T, G)
    S = sk * KB
    assert S == 0 or S >= G, "the host keeps a stream-K grid no larger than the stream"
    B = lambda r: r * S // G
    work = {}
    pieces = {}          # stream-K tile -> list of (rank, first kb, count, slot, summed ranks in order)
    for rank in range(G):
        steps = []
        ntiles = (dp - 1 - rank) // G + 1 if rank < dp and not aligned else 0
        for i in range(ntiles):
            steps += [(rank + i * G, kb) for kb in range(KB)]
        if aligned:
            t, j = rank % T, rank // T
            lo, hi = t * KB + j * KB // S_al, t * KB + (j + 1) * KB // S_al
        else:
            lo, hi = B(rank), B(rank + 1)
        for s in range(lo, hi):
            steps.append((dp + s // KB, s % KB))
        work[rank] = steps
        # segments of this rank's stream-K run
        v = ntiles * KB
        while v < len(steps):
            L, kb0 = steps[v]
            n = min(KB - kb0, len(steps) - v)
            if not (kb0 == 0 and n == KB):
                tp = L - dp
                if aligned:
                    order = [tp + j * T for j in range(S_al)]
                    slot = 2 * rank
                else:
                    x0 = tp * KB
                    r_lo = min(G - 1, ((x0 + 1) * G - 1) // S)
                    r_hi = min(G - 1, ((x0 + KB) * G - 1) // S)
                    order = list(range(r_lo, r_hi + 1))
                    slot = 2 * rank + (0 if B(rank) >= x0 else 1)
                pieces.setdefault(tp, []).append((rank, kb0, n, slot, tuple(order)))
            v += n
    return dp, sk, work, pieces


CASES = [(T, KB, slots) for T in (1, 7, 56, 100, 128, 129, 168, 255, 256, 257, 300, 448, 511, 512, 513, 1344, 1792)
         for KB in (1, 2, 3, 40, 48) for slots in (8, 64, 256, 512)]


@pytest.mark.parametrize("T,KB,slots", CASES)
def test_every_block_once_and_fixup_pieces_consistent(T, KB, slots):
    G = host_grid(T, KB, slots)
    assert 1 <= G <= max(slots, 1)
    dp, sk, work, pieces = schedule(T, KB, G)
    seen = {}
    for rank, steps in work.items():
        for st in steps:
            assert st not in seen, (st, rank, seen.get(st))
            seen[st] = rank
    assert len(seen) == T * KB
    # balanced: stream-K runs differ by at most one block
    if sk:
        lens = [len(w) - ((dp - 1 - r) // G + 1 if r < dp and 2 * T > G else 0) * KB for r, w in work.items()]
        assert max(lens) - min(lens) <= 1, (min(lens), max(lens))
        assert min(lens) >= 1
    used_slots = set()
    for tp, ps in pieces.items():
        assert 0 <= tp < sk
        order = ps[0][4]
        assert all(p[4] == order for p in ps)
        assert sorted(p[0] for p in ps) == sorted(order), (tp, ps)        # the pieces are exactly the summed ranks
        assert sum(p[2] for p in ps) == KB                               # the pieces cover the tile's K once
        # summed in K order: each piece starts where the previous one ends
        by_rank = {p[0]: p for p in ps}
        starts = [by_rank[r][1] for r in order]
        assert starts == sorted(starts) and starts[0] == 0
        for rank, kb0, n, slot, _ in ps:
            assert 0 <= slot < 2 * G
            assert slot // 2 == rank
            assert (rank, slot) not in used_slots
            used_slots.add((rank, slot))
    # a rank holds at most two pieces, in different slots
    per_rank = {}
    for ps in pieces.values():
        for rank, _, _, slot, _ in ps:
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
            assert G == host_grid(T, K // 128, cus * per_cu), (v["name"], G)
            dp, sk = split_work(T, G)
            want = 0 if sk == 0 else 65536 + 2 * G * v["bm"] * v["bn"] * 4
            assert plan["workspace"] == want, (v["name"], M, N, K, plan["workspace"], want)
            assert sk * 4 <= 65536


def test_plain_entry_never_runs_stream_k():
    for M in (300, 574, 700, 2048, 6016):
        plan = g.gemm_a8w8_blockscale_plan(M, 14336, 5120)
        assert plan["name"].split("_")[0] != "sktile", plan
