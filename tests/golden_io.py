"""Readers for the hand-derived fixtures under tests/golden/."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line.split()


def pyval(expr):
    """Evaluate a fixture's numeric expression (literals, ** and float('inf') only)."""
    return float(eval(expr, {"__builtins__": {}}, {"float": float}))


def e2m1_table():
    return {int(r[0], 16): float(r[4]) for r in rows("e2m1_codes.txt")}


def e4m3_samples():
    return {int(r[0], 16): float(r[2]) for r in rows("e4m3_samples.txt")}
