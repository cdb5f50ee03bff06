"""GPU tests of the decode tables for prepacked weights and row-wise scales.

For every row (M = 1..16) of each packed-weight and row-wise decode table:
the plan the library reports is the table row's instance; the call captured
in a HIP graph on a fresh stream replays bitwise equal to the eager call
(three replays, eager work between them); the result is bitwise the result of
the same instance forced on the other weight layout; and every output row is
within the parity bar of the oracle (each row of Y depends only on its row of
A, so one oracle run of 16 rows serves every M).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

import fp8_block_scaled_a8w8_amd as g
import inputgen
import oracle
from tests.gpu_util import DEV, say, y_bits, y_host
from tests.parity_util import assert_parity
from tests.test_gpu_splitk import _replay_matches_eager

pytestmark = pytest.mark.gpu


def _form_tables():
    with open(os.path.join(os.path.dirname(g.__file__), "tuned_table.json")) as f:
        shapes = json.load(f)["shapes"]
    return [(sh["form"], int(sh["n"]), int(sh["k"]), sh["rows"]) for sh in shapes if sh.get("form")]


def _dev(*arrays):
    return tuple(torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays)


@pytest.mark.parametrize("entry", range(len(_form_tables())),
                         ids=[f"{f}:{n}:{k}" for f, n, k, _ in _form_tables()])
def test_decode_form_rows_plan_graph_and_parity(entry):
    form, N, K, rows = _form_tables()[entry]
    rowwise = form == "rowwise"
    if rowwise:
        A, a = inputgen.make_rowwise_activations(16, K, seed=70)
        W, w = inputgen.make_rowwise_weights(N, K, seed=71)
        ref = oracle.gemm_rowwise(A, a, W, w)
    else:
        A, a = inputgen.make_activations(16, K, seed=70)
        W, w = inputgen.make_weights(N, K, seed=71)
        ref = oracle.gemm(A, a, W, w)
    dA, da, dW, dw = _dev(A, a, W, w)
    dWp = g.prepack_weights(dW)
    kind = "rowwise" if rowwise else "block"
    say(f"{form} decode table N={N} K={K}: {len(rows)} rows")
    for r in rows:
        M = int(r["key_m"])
        plan = g.gemm_a8w8_ex_plan(M, N, K, scale_kind=kind, packed=not rowwise)
        assert plan["name"] == r["name"] and plan["key_m"] == M and plan["fallback"] == 0, (M, plan["name"])
        out = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        if rowwise:
            call = lambda: g.gemm_a8w8_rowwise(dA[:M], da[:M], dW, dw, out=out)
        else:
            call = lambda: g.gemm_a8w8_blockscale_packed(dA[:M], da[:M], dWp, dw, N, out=out)
        eager = _replay_matches_eager(call, out, f"{form} N={N} K={K} M={M} {r['name']}")
        if rowwise:
            other = g.gemm_a8w8_rowwise_run_variant(plan["variant"], dA[:M], da[:M], dWp, dw, packed_n=N)
        else:
            other = g.gemm_a8w8_blockscale_run_variant(plan["variant"], dA[:M], da[:M], dW, dw)
        assert np.array_equal(y_bits(other), eager), f"{form} M={M}: other layout differs"
        assert_parity(y_host(out), ref[:M], f"{form} N={N} K={K} M={M}")
