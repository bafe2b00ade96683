"""Independent references used to pin the oracle (no numpy float arithmetic in
the rounding helpers: exact rationals and the standard library only)."""

import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def round_to_binary32(x):
    """Nearest binary32 value of the rational ``x`` (ties to even), as a Fraction."""
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                         # below: subnormal quantum 2^-149
    quantum = Fraction(2) ** (e - 23)
    n = round(a / quantum)                   # Fraction.__round__: half to even
    return sign * n * quantum


def fp16_bits_of(x):
    """IEEE half bits of the real ``x`` rounded to nearest even (struct 'e')."""
    return struct.unpack("<H", struct.pack("<e", float(x)))[0]


def parse_worked_examples():
    """Rows of tests/golden/codec_worked_examples.txt as
    (name, fmt, fp16 values[32], expected bytes)."""
    out = []
    with open(os.path.join(GOLDEN, "codec_worked_examples.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, fmt, vals, hexbytes = [p.strip() for p in line.split("|")]
            nbytes = 34 if fmt == "q8" else 18
            v = [float(t) for t in vals.split(",") if t.strip()] if vals else []
            v = v + [0.0] * (32 - len(v))
            b = [int(t, 16) for t in hexbytes.split()]
            b = b + [0] * (nbytes - len(b))
            x = np.array(v, dtype=np.float16)
            assert [float(t) for t in x] == v, f"{name}: value not fp16-exact"
            out.append((name, fmt, x, np.array(b, dtype=np.uint8)))
    return out


def parse_occupancy_table():
    rows = []
    with open(os.path.join(GOLDEN, "occupancy_table.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v, bpp, gb = [p.strip() for p in line.split("|")]
            rows.append((k, v, int(bpp), float(gb)))
    return rows
