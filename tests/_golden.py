"""Reader for the small text fixtures under tests/golden (key = value lines, '#' comments).
Matrices are written as rows separated by ';'."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line or "=" not in line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out


def matrix(text):
    rows = [r.split() for r in text.split(";")]
    return np.array([[float(x) for x in r] for r in rows], dtype=np.float64)


def vector(text):
    return np.array([float(x) for x in text.split()], dtype=np.float64)


def mapping(text, key=int):
    out = {}
    for tok in text.split():
        k, v = tok.split(":")
        out[key(k, 0) if key is int else key(k)] = float(v)
    return out
