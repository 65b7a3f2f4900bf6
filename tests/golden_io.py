"""Readers for the hand-written fixtures under tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


def _num(tok):
    return float.fromhex(tok) if "0x" in tok else float(tok)


def e2m1_table():
    """[(code, sign, exponent, mantissa, value)] from e2m1_table.txt."""
    rows = []
    for line in _lines("e2m1_table.txt"):
        c, s, e, m, v = line.split()
        rows.append((int(c), int(s), int(e), int(m), _num(v)))
    return rows


def mxfp4_blocks():
    """[(name, x[32], scale_code, packed[16])] from mxfp4_blocks.txt."""
    out, cur = [], None
    for line in _lines("mxfp4_blocks.txt"):
        key, _, rest = line.partition(" ")
        if key == "block":
            cur = {"name": rest}
            out.append(cur)
        elif key == "x":
            cur["x"] = [_num(t) for t in rest.split()]
        elif key == "scale":
            cur["scale"] = int(rest)
        elif key == "codes":
            cur["codes"] = [int(t, 16) for t in rest.split()]
    return [(b["name"], b["x"], b["scale"], b["codes"]) for b in out]
