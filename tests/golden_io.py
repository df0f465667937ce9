"""Readers for the hand-worked fixtures in tests/golden/ (test helpers)."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fields(name):
    """'key: rows separated by ;' lines -> {key: 2-D float array}."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or ":" not in line:
                continue
            key, val = line.split(":", 1)
            rows = [[float(t) for t in r.split()] for r in val.split(";")]
            out[key.strip()] = np.array(rows)
    return out


def read_rounding_cases():
    """[(fp64 value, expected fp16 bits)] from fp16_rounding.txt."""
    cases = []
    with open(os.path.join(GOLDEN, "fp16_rounding.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            expr, bits = line.rsplit(None, 1)
            cases.append((float(eval(expr, {"__builtins__": {}})), int(bits, 16)))
    return cases
