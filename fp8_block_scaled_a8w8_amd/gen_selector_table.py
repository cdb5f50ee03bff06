"""Write csrc/a8w8_selector_table.h from tuned_table.json.

tuned_table.json holds, per registered (N, K), ascending M keys and the
kernel instance the tuner picked for each key:

    {"shapes": [{"n": 14336, "k": 5120,
                 "rows": [{"key_m": 1, "kernel": "skinny", "bm": 16, "bn": 16,
                           "waves": 8, "us": 11.9}, ...]}, ...]}

A shape tuned for the MX-scaled variant carries ``"mx": true`` (and the
batch count it was timed with, ``"batch"``); the selector matches a call's
variant against it, so block-scale and MX tables for one (N, K) coexist.
A shape tuned for fp32 block scales with prepacked weights carries
``"form": "packed"``, one tuned for row-wise scales ``"form": "rowwise"``.
These two are decode tables (keys 1..16): a call of that form and M <= 16
takes its row, every other M the block-scale table's.

A row whose instance cuts K across workgroups (split K, "splits" > 1, or a
stream-K "sktile" instance) also names, under "unsplit", the fastest instance
without a cross-workgroup cut: calls that bring no workspace (or too small a
one) run that instance, so every key has a plan that needs no workspace.

A request M is served by the row with the smallest key_m >= M.  The checks
below make that safe: keys strictly ascending, every key <= 1.25 x the
smallest M it serves (exact keys for M <= 16), the skinny kernel only for
keys <= 16, the last key at least 8192 (exactly 16 for the packed and
row-wise decode tables), and an unsplit instance for every key.

Usage: python -m fp8_block_scaled_a8w8_amd.gen_selector_table [--check]
"""
from __future__ import annotations

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE_JSON = os.path.join(HERE, "tuned_table.json")
HEADER = os.path.join(HERE, "csrc", "a8w8_selector_table.h")
KERNELS = {"skinny": 1, "tile": 2, "ptile": 3, "pskinny": 4, "tall": 5, "rskinny": 6, "sktile": 7}
MAX_KEY_RATIO = 1.25
M_COVERED = 8192
# Table forms: the selector's code for each (0: fp32 block scales, row-major weights).
FORMS = {"block": 0, "mx": 1, "packed": 2, "rowwise": 3}
DECODE_FORMS = ("packed", "rowwise")     # tables of M <= 16 only


def form_of(sh: dict) -> str:
    if sh.get("mx"):
        return "mx"
    f = sh.get("form", "block")
    if f not in FORMS or f == "mx":
        raise ValueError(f"unknown table form {f!r}")
    return f


def load(path: str = TABLE_JSON) -> dict:
    if not os.path.exists(path):
        return {"shapes": []}
    with open(path) as f:
        return json.load(f)


def validate(table: dict) -> None:
    seen = set()
    for sh in table["shapes"]:
        form = form_of(sh)
        key = (int(sh["n"]), int(sh["k"]), form)
        if key in seen:
            raise ValueError(f"duplicate (N,K,form) {key}")
        seen.add(key)
        rows = sh["rows"]
        if not rows:
            raise ValueError(f"{key}: no rows")
        prev = 0
        for r in rows:
            km = int(r["key_m"])
            if km <= prev:
                raise ValueError(f"{key}: keys not strictly ascending at {km}")
            lowest_served = prev + 1
            if km > MAX_KEY_RATIO * lowest_served + 1e-9:
                raise ValueError(f"{key}: key {km} serves M={lowest_served} (> {MAX_KEY_RATIO}x)")
            if lowest_served <= 16 and km != lowest_served:
                raise ValueError(f"{key}: M <= 16 needs exact keys, got {km} for {lowest_served}")
            if r["kernel"] not in KERNELS:
                raise ValueError(f"{key}: unknown kernel {r['kernel']}")
            if r["kernel"] in ("skinny", "pskinny", "rskinny") and km > 16:
                raise ValueError(f"{key}: skinny kernel for key {km} > 16")
            u = unsplit_of(r)
            if u["kernel"] not in KERNELS or cuts_k(u):
                raise ValueError(f"{key}: key {km} has no unsplit instance")
            if u["kernel"] in ("skinny", "pskinny", "rskinny") and km > 16:
                raise ValueError(f"{key}: skinny kernel for key {km} > 16")
            prev = km
        covered = 16 if form in DECODE_FORMS else M_COVERED
        if prev < covered or (form in DECODE_FORMS and prev > 16):
            raise ValueError(f"{key}: table stops at M={prev}, needs {covered}")


def cuts_k(row: dict) -> bool:
    """Whether the row's instance cuts K across workgroups (and so needs a workspace)."""
    return int(row.get("splits", 1)) > 1 or row["kernel"] == "sktile"


def unsplit_of(row: dict) -> dict:
    """The instance a call without a workspace runs for this row."""
    if cuts_k(row):
        if "unsplit" not in row:
            raise ValueError(f"key {row['key_m']}: split row without an unsplit instance")
        return row["unsplit"]
    return row


def fnv1a64(data: bytes) -> int:
    h = 0xcbf29ce484222325
    for b in data:
        h ^= b
        h = (h * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def _order(sh: dict):
    return (FORMS[form_of(sh)], int(sh["n"]), int(sh["k"]))


def canonical(table: dict) -> bytes:
    rows = []
    for sh in sorted(table["shapes"], key=_order):
        for r in sh["rows"]:
            row = [sh["n"], sh["k"], r["key_m"], r["kernel"], r["bm"], r["bn"], r["waves"], r.get("kblocks", 1)]
            if form_of(sh) != "block":
                row.append(form_of(sh))
            if cuts_k(r):
                if int(r.get("splits", 1)) > 1:
                    row.append(f"k{int(r['splits'])}")
                u = unsplit_of(r)
                row += ["u", u["kernel"], u["bm"], u["bn"], u["waves"], u.get("kblocks", 1)]
            rows.append(row)
    return json.dumps(rows, separators=(",", ":")).encode()


def render(table: dict) -> str:
    out = []
    out.append("// a8w8_selector_table.h -- GENERATED by gen_selector_table.py from tuned_table.json.")
    out.append("// Do not edit by hand.")
    out.append("#pragma once")
    out.append("#include <stdint.h>")
    out.append("")
    out.append("namespace a8w8_table {")
    out.append("")
    out.append("struct ShapeTable {")
    out.append("    int64_t n, k;")
    out.append("    int32_t form;   // 0 fp32 block scales, 1 MX, 2 block scales + packed weights, 3 row-wise")
    out.append("    int count;")
    out.append("    const int64_t *key_m;")
    out.append("    const int32_t *kernel, *bm, *bn, *waves, *kblocks, *splits;   // fastest instance")
    out.append("    const int32_t *u_kernel, *u_bm, *u_bn, *u_waves, *u_kblocks;  // fastest without split K")
    out.append("};")
    out.append("")
    shapes = sorted(table["shapes"], key=_order)
    for i, sh in enumerate(shapes):
        rows = sh["rows"]
        def arr(ctype, name, vals):
            out.append(f"static const {ctype} s{i}_{name}[] = {{{', '.join(str(v) for v in vals)}}};")
        arr("int64_t", "key", [int(r["key_m"]) for r in rows])
        arr("int32_t", "kernel", [KERNELS[r["kernel"]] for r in rows])
        arr("int32_t", "bm", [int(r["bm"]) for r in rows])
        arr("int32_t", "bn", [int(r["bn"]) for r in rows])
        arr("int32_t", "waves", [int(r["waves"]) for r in rows])
        arr("int32_t", "kblocks", [int(r.get("kblocks", 1)) for r in rows])
        arr("int32_t", "splits", [int(r.get("splits", 1)) for r in rows])
        us = [unsplit_of(r) for r in rows]
        arr("int32_t", "u_kernel", [KERNELS[u["kernel"]] for u in us])
        arr("int32_t", "u_bm", [int(u["bm"]) for u in us])
        arr("int32_t", "u_bn", [int(u["bn"]) for u in us])
        arr("int32_t", "u_waves", [int(u["waves"]) for u in us])
        arr("int32_t", "u_kblocks", [int(u.get("kblocks", 1)) for u in us])
    out.append("")
    out.append(f"constexpr int kNumShapes = {len(shapes)};")
    if shapes:
        out.append("static const ShapeTable kShapes[] = {")
        for i, sh in enumerate(shapes):
            out.append(f"    {{{int(sh['n'])}, {int(sh['k'])}, {FORMS[form_of(sh)]}, {len(sh['rows'])}, "
                       f"s{i}_key, s{i}_kernel, "
                       f"s{i}_bm, s{i}_bn, s{i}_waves, s{i}_kblocks, s{i}_splits, "
                       f"s{i}_u_kernel, s{i}_u_bm, s{i}_u_bn, s{i}_u_waves, s{i}_u_kblocks}},")
        out.append("};")
    else:
        out.append("static const ShapeTable kShapes[1] = {{0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr}};")
    out.append(f"constexpr uint64_t kTableHash = 0x{fnv1a64(canonical(table)):016x}ull;")
    out.append("")
    out.append("}  // namespace a8w8_table")
    out.append("")
    return "\n".join(out)


def main(argv=None) -> int:
    argv = sys.argv[1:] if argv is None else argv
    table = load()
    validate(table)
    text = render(table)
    if "--check" in argv:
        with open(HEADER) as f:
            if f.read() != text:
                print("selector header is stale; regenerate it", file=sys.stderr)
                return 1
        return 0
    with open(HEADER, "w") as f:
        f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
