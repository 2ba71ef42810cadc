"""Readers for the hand-derived fixtures in tests/golden/."""
import os

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(name):
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line.split()


def e2m1_table():
    """code -> value from e2m1_codes.txt (16 entries)."""
    out = {}
    for cols in _rows("e2m1_codes.txt"):
        out[int(cols[0], 16)] = float(cols[4])
    assert sorted(out) == list(range(16))
    return out


def packed_examples():
    return [(int(c[0], 16), float(c[1]), float(c[2])) for c in _rows("packed_bytes.txt")]


def scale_fp8_examples():
    return [(c[0], int(c[1], 0), float(c[2])) for c in _rows("ue8m0_e4m3_examples.txt")]


def bf16_examples():
    """(kind, x or code, expected) rows of bf16_round.txt; kind "round" or "decode"."""
    out = []
    for c in _rows("bf16_round.txt"):
        x = int(c[1], 16) if c[0] == "decode" else float(c[1])
        out.append((c[0], x, float(c[2])))
    return out
