"""Parser for tests/golden/worked_blocks.txt (hand-worked Q4_K blocks)."""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _expand_hex(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.split("*")
            out += [int(v, 16)] * int(n)
        else:
            out.append(int(t, 16))
    return out


def _value(tok: str):
    """Return (Fraction value, sign) where sign is -1 for an explicit -0."""
    if tok in ("+0", "0"):
        return Fraction(0), 1
    if tok == "-0":
        return Fraction(0), -1
    if "/" in tok:
        a, b = tok.split("/")
        return Fraction(int(a), int(b)), 1
    return Fraction(tok), 1


def _expand_values(tokens):
    out = []
    for t in tokens:
        if "*" in t:
            v, n = t.rsplit("*", 1)
            out += [_value(v)] * int(n)
        else:
            out.append(_value(t))
    return out


def load_worked_blocks(path: str | None = None):
    path = path or os.path.join(GOLDEN, "worked_blocks.txt")
    entries = []
    cur = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = {"id": line[1:-1]}
                entries.append(cur)
                continue
            k, v = [p.strip() for p in line.split("=", 1)]
            cur[k] = v
    blocks = []
    for e in entries:
        d = int(e["d"], 16)
        dmin = int(e["dmin"], 16)
        s = _expand_hex(e["s"].split())
        assert len(s) == 12, e["id"]
        if e["qs"] == "E7pattern":
            qs = [(l & 15) | ((15 - (l & 15)) << 4) for g in range(4) for l in range(32)]
        else:
            qs = _expand_hex(e["qs"].split())
        assert len(qs) == 128, e["id"]
        blk = np.array([d & 0xFF, d >> 8, dmin & 0xFF, dmin >> 8] + s + qs, dtype=np.uint8)
        exp = _expand_values(e["expect"].split())
        assert len(exp) == 256, (e["id"], len(exp))
        item = {"id": e["id"], "block": blk, "expect": exp, "why": e.get("why", "")}
        if "sc" in e:
            item["sc"] = [int(t) for t in e["sc"].split()]
            item["m"] = [int(t) for t in e["m"].split()]
        blocks.append(item)
    return blocks
