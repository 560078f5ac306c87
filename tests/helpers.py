"""Small helpers shared by the tests (fixture parsing, exact rounding, metrics)."""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> dict[str, dict[str, list[str]]]:
    """Parse a fixture: ``key: values`` lines, ``#`` comments, optional ``[section]``."""
    out: dict[str, dict[str, list[str]]] = {"": {}}
    cur = ""
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = line[1:-1]
                out[cur] = {}
                continue
            key, val = line.split(":", 1)
            out[cur][key.strip()] = val.split()
    return out


def ints(v: list[str]) -> np.ndarray:
    return np.array([int(s, 0) for s in v], dtype=np.int64)


def floats(v: list[str]) -> np.ndarray:
    return np.array([float(s) for s in v], dtype=np.float64)


def exact_round_bf16(q: Fraction) -> int:
    """bf16 bits of the nearest bf16 to the rational q (ties to even), by exact
    comparison with the two neighbouring bf16 values (normal range only)."""
    if q == 0:
        return 0
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    e = 0
    while a >= 2:
        a /= 2
        e += 1
    while a < 1:
        a *= 2
        e -= 1
    # a in [1, 2): significand with 7 fraction bits
    scaled = a * 128
    lo = int(scaled)  # floor
    frac = scaled - lo
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    if lo == 256:
        lo = 128
        e += 1
    exp_bits = e + 127
    assert 0 < exp_bits < 255
    return sign | (exp_bits << 7) | (lo - 128)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """Norm-wise relative error ||got - ref||_2 / ||ref||_2 in float64."""
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(r)
    num = np.linalg.norm(g - r)
    if den == 0:
        return float(num)
    return float(num / den)


def f32_from_bits_list(vals) -> np.ndarray:
    return np.array(vals, dtype=np.float32)
