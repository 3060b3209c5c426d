"""Loader for the hand-derived fixtures under tests/golden/ (format in tests/golden/README.md)."""
from __future__ import annotations

import glob
import math
import os
import re
from fractions import Fraction

import numpy as np

from exact_arith import to_bits

GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _term(tok: str):
    m = re.fullmatch(r"(-?)(?:(\d+)\*)?2\^(-?\d+)", tok)
    if m:
        k = Fraction(int(m.group(2)) if m.group(2) else 1)
        v = k * Fraction(2) ** int(m.group(3))
        return -v if m.group(1) else v
    return Fraction(tok)


def parse_value(tok: str):
    """Exact value of a token: decimal, k*2^e, 2^e, a sum of those, inf, -inf; -0 -> 'neg0'."""
    if tok in ("inf", "-inf"):
        return math.inf if tok == "inf" else -math.inf
    if tok == "-0":
        return "neg0"
    parts = re.split(r"(?<=[^\^eE])\+", tok)
    return sum((_term(p) for p in parts), Fraction(0))


def encode(tok: str, dtype: str) -> int:
    v = parse_value(tok)
    if v == "neg0":
        return {"fp32": 1 << 31, "fp16": 0x8000, "bf16": 0x8000}[dtype]
    return to_bits(v, dtype)


def _storage(values, dtype, shape):
    bits = np.array([encode(t, dtype) for t in values], dtype=np.uint64).reshape(shape)
    if dtype == "fp32":
        return bits.astype(np.uint32).view(np.float32)
    return bits.astype(np.uint16)


def load(path: str) -> dict:
    kv = {}
    with open(path) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = line.split(":", 1)
            kv[k.strip()] = v.split()
    fx = {"name": os.path.basename(path), "pattern": kv["pattern"][0], "dtype": kv["dtype"][0]}
    W, M, H = int(kv["W"][0]), int(kv["M"][0]), int(kv["H"][0])
    dt = fx["dtype"]
    fx.update(W=W, M=M, H=H)

    def mat(prefix):
        return _storage([t for m in range(M) for t in kv["%s.row%d" % (prefix, m)]], dt, (M, H))

    fx["inputs"] = [mat("x%d" % r) for r in range(W)]
    if fx["pattern"] == "sum":
        fx["out"] = mat("out")
    else:
        fx["residual"] = mat("residual")
        fx["gamma"] = np.array([float(parse_value(t)) for t in kv["gamma"]], dtype=np.float32)
        fx["eps"] = float(kv["eps"][0])
        fx["residual_out"] = mat("residual_out")
        fx["norm_out"] = mat("norm_out")
    return fx


def all_fixtures():
    return [load(p) for p in sorted(glob.glob(os.path.join(GOLDEN_DIR, "*.txt")))]
