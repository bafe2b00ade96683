"""Pins of the oracle's block codec against what the pages and IEEE arithmetic fix."""

import struct
from fractions import Fraction

import numpy as np
import pytest

from oracle import codec
from oracle_pins import (fp16_bits_of, parse_occupancy_table, parse_worked_examples,
                         round_to_binary32)


def test_block_sizes_from_modes_table():
    # MBufo page, section 2 modes table: 34 bytes (f16 scale + 32 x 8-bit), 18 bytes (4-bit).
    assert codec.block_bytes("q8") == 34
    assert codec.block_bytes("q4") == 18
    assert codec.qmax("q8") == 127 and codec.qmax("q4") == 7


@pytest.mark.parametrize("row", parse_occupancy_table(), ids=lambda r: f"{r[0]}-{r[1]}")
def test_occupancy_table(row):
    k, v, bpp, gb = row
    assert codec.bytes_per_position(4, 128, k, v) == bpp
    total = codec.session_bytes(262144, 12, 4, 128, k, v)
    assert round(total / 1e9, 2) == gb


def test_session_ratios_exact():
    # q8 stores 34 bytes per 32 values (17/32 of f16), K4V4 18 (9/32 of f16).
    f16 = codec.session_bytes(262144, 12, 4, 128, "f16", "f16")
    assert codec.session_bytes(262144, 12, 4, 128, "q8", "q8") * 32 == f16 * 17
    assert codec.session_bytes(262144, 12, 4, 128, "q4", "q4") * 32 == f16 * 9


@pytest.mark.parametrize("ex", parse_worked_examples(), ids=lambda e: e[0])
def test_worked_examples_encode(ex):
    name, fmt, x, expected = ex
    got = codec.encode_blocks(x[None, :], fmt)[0]
    assert got.tolist() == expected.tolist(), name


def test_worked_example_decoded_values():
    ex = {e[0]: e for e in parse_worked_examples()}
    _, fmt, _, b = ex["q8_unit_scale_ties"]
    want = [127, 64, 0, 2, 2, 0, -127] + [0] * 25
    assert codec.decode_blocks(b, fmt).tolist() == want
    _, fmt, _, b = ex["q4_unit_scale"]
    want = [7, -7, 4, 2, -4, 0, 2, -2] + [0] * 24
    assert codec.decode_blocks(b, fmt).tolist() == want
    _, fmt, _, b = ex["q8_subnormal_scale"]
    d = 129 * 2.0 ** -24
    assert codec.decode_blocks(b, fmt)[:2].tolist() == [127 * d, -64 * d]
    _, fmt, _, b = ex["q8_scale_underflows"]
    assert not codec.decode_blocks(b, fmt).any()


def test_nibble_decoding_by_hand():
    # 4-bit codes -8..7 as two's-complement nibbles, even element low.
    b = np.zeros(18, np.uint8)
    b[0:2] = [0x00, 0x3C]                        # d = 1.0
    b[2] = 0x8F                                  # low nibble F -> -1, high 8 -> -8
    b[3] = 0x70                                  # low 0 -> 0, high 7 -> 7
    vals = codec.decode_blocks(b, "q4")
    assert vals[:4].tolist() == [-1, -8, 0, 7]


def _random_blocks(rng, n):
    x = rng.standard_normal((n, 32)).astype(np.float32)
    kinds = rng.integers(0, 6, size=n)
    x[kinds == 1] *= 20.0                                          # outlier-scaled
    x[kinds == 2] *= np.float32(1e-4)                              # fp16 subnormal scales
    x[kinds == 3] *= np.float32(3e-7)                              # scales that underflow
    x[kinds == 4] = np.round(x[kinds == 4] * 8) / 2                # many exact ties
    sparse = kinds == 5
    x[sparse] *= (rng.random((int(sparse.sum()), 32)) < 0.1)       # mostly zero
    return x.astype(np.float16)


def test_binary32_divide_is_correctly_rounded():
    rng = np.random.default_rng(11)
    x = _random_blocks(rng, 400).reshape(-1)
    x = x[x != 0]
    den = np.abs(rng.choice(x, size=x.size)).astype(np.float32) / np.float32(127)
    num = x.astype(np.float32)
    q = np.divide(num, den, dtype=np.float32)
    for a, b, got in zip(num[:4000], den[:4000], q[:4000]):
        assert Fraction(float(got)) == round_to_binary32(Fraction(float(a)) / Fraction(float(b)))


def test_fp16_rounding_matches_ieee_half():
    rng = np.random.default_rng(12)
    s = (np.abs(rng.standard_normal(3000)) * 10.0 ** rng.uniform(-9, 2, 3000)).astype(np.float32)
    # exact midpoints between neighbouring fp16 values (normal and subnormal)
    h = np.arange(1, 2000, 7, dtype=np.uint16).view(np.float16).astype(np.float32)
    h2 = (np.arange(1, 2000, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float32)
    mids = ((h.astype(np.float64) + h2.astype(np.float64)) / 2).astype(np.float32)
    vals = np.concatenate([s, mids])
    got = vals.astype(np.float16).view(np.uint16)
    for v, g in zip(vals, got):
        assert int(g) == fp16_bits_of(float(v)), float(v)


def test_rint_is_half_to_even():
    v = (np.arange(-600, 601, dtype=np.float32) / np.float32(4))
    assert all(int(a) == round(float(b)) for a, b in zip(np.rint(v), v))


@pytest.mark.parametrize("fmt", ["q8", "q4"])
def test_codec_invariants(fmt):
    rng = np.random.default_rng(13 if fmt == "q8" else 14)
    x = _random_blocks(rng, 3000)
    b = codec.encode_blocks(x, fmt)
    d, q = codec.decode_codes(b, fmt)
    qm = codec.qmax(fmt)
    for i in range(0, len(x), 7):
        xi = [Fraction(float(t)) for t in x[i]]
        amax = max(abs(t) for t in xi)
        qi = q[i].astype(int).tolist()
        if amax == 0:
            assert b[i].tolist() == [0] * codec.block_bytes(fmt)
            continue
        s = round_to_binary32(amax / qm)                              # exact binary32 scale
        assert int(d[i].view(np.uint16)) == fp16_bits_of(s)             # stored scale = fp16(s)
        assert max(abs(t) for t in qi) == qm                            # the top code is hit
        for t, c in zip(xi, qi):
            assert abs(t / s - c) <= Fraction(1, 2) + Fraction(1, 2 ** 17)
        dd = Fraction(float(d[i]))
        xh = codec.decode_blocks(b[i], fmt)
        for t, c, h in zip(xi, qi, xh):
            assert Fraction(float(h)) == c * dd                         # exact product
            assert abs(t - c * dd) <= s / 2 + abs(c) * abs(s - dd) + s / 2 ** 17


def test_f16_block_is_the_little_endian_halves():
    # The unquantized mode: a block is its 32 values as IEEE halves (struct's
    # 'e' format is an independent encoder), 64 bytes, decoded exactly.
    assert codec.block_bytes("f16") == 64 and codec.qmax("f16") is None
    assert codec.bytes_per_position(4, 128, "f16", "f16") == 4 * 4 * codec.block_bytes("f16") * 2 == 2048
    rng = np.random.default_rng(21)
    x = _random_blocks(rng, 200)
    x[0, :4] = np.array([0.0, -0.0, 6.0e-8, -65504.0], dtype=np.float16)   # zeros, a subnormal, the limit
    b = codec.encode_blocks(x, "f16")
    assert b.shape == (200, 64)
    for i in range(len(x)):
        assert bytes(b[i]) == struct.pack("<32e", *[float(t) for t in x[i]])
    back = codec.decode_blocks(b, "f16")
    assert np.array_equal(back, x.astype(np.float64))
    assert np.array_equal(np.signbit(back[0, :2]), [False, True])


def test_encode_shape_and_dtype_contract():
    x = np.zeros((3, 5, 32), np.float16)
    assert codec.encode_blocks(x, "q8").shape == (3, 5, 34)
    assert codec.encode_blocks(x, "q4").shape == (3, 5, 18)
    with pytest.raises(AssertionError):
        codec.encode_blocks(np.zeros((2, 32), np.float32), "q8")
