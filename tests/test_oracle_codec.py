"""CPU pins of the oracle's OCP e4m3 codec and BF16 decode.

The pages name the cache format only as "FP8 e4m3" (aifeed.sk, section
"Dve odlišné úzke miesta v pamäti GPU"); the codec's values come from the
OCP FP8 specification (tests/golden/e4m3_ocp_table.txt). Pins here do not
retype the oracle's formulas: they check the spec's table, structural
properties of the value set, torch's independent float8_e4m3fn codec, and the
ties/saturation cases worked out by hand.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_table.txt")


def _golden_rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), val))
    return rows


def _parse(val: str) -> float:
    if val == "nan":
        return math.nan
    if val == "-0":
        return -0.0
    sign = -1.0 if val.startswith("-") else 1.0
    v = val.lstrip("-")
    if "*" in v:
        a, b = v.split("*")
        return sign * float(a) * 2.0 ** int(b.split("^")[1])
    if v.startswith("2^"):
        return sign * 2.0 ** int(v[2:])
    return sign * float(v)


def test_golden_ocp_table():
    for code, val in _golden_rows():
        got = oracle.e4m3_decode(code)
        want = _parse(val)
        if math.isnan(want):
            assert math.isnan(got), hex(code)
        else:
            assert got == want and math.copysign(1, got) == math.copysign(1, want), hex(code)


def test_p1_value_set_structure():
    v = oracle.e4m3_decode_all()
    nan = np.isnan(v)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert (~nan).sum() == 254
    pos = v[:0x7F]
    # strictly increasing over 0x00..0x7E, max 448 at 0x7E
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0
    # sign symmetry
    assert np.all(v[0x80:0xFF] == -v[0x00:0x7F])
    assert math.copysign(1.0, v[0x80]) == -1.0
    # equal spacing 2^-9 from 0 through the first normal binade [2^-6, 2^-5)
    assert np.all(np.diff(pos[:17]) == 2.0 ** -9)
    # every later binade [2^e, 2^(e+1)) holds 8 equally spaced values
    for e in range(-5, 9):
        b = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(b) == (7 if e == 8 else 8)
        assert b[0] == 2.0 ** e
        assert np.all(np.diff(b) == 2.0 ** (e - 3))


def test_p1_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    t = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    v = oracle.e4m3_decode_all()
    assert np.array_equal(np.isnan(t), np.isnan(v))
    ok = ~np.isnan(v)
    assert np.array_equal(t[ok], v[ok])
    assert np.array_equal(np.signbit(t[ok]), np.signbit(v[ok]))


def test_p2_round_trip():
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert oracle.e4m3_encode(np.float32(oracle.e4m3_decode(c))) == c, hex(c)


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),            # halfway 1 and 1.125 -> even mantissa (1.0)
    (1.1875, 0x3A),            # halfway 1.125 and 1.25 -> 1.25 (even)
    (2.0 ** -10, 0x00),        # halfway 0 and 2^-9 -> 0
    (3 * 2.0 ** -10, 0x02),    # halfway 2^-9 and 2^-8 -> 2^-8 (even code)
    (432.0, 0x7E),             # halfway 416 and 448 -> 448 (even code)
    (440.0, 0x7E),
    (448.0001, 0x7E),          # saturate
    (464.0, 0x7E),
    (1e6, 0x7E),
    (math.inf, 0x7E),
    (-448.0001, 0xFE),
    (-1e6, 0xFE),
    (-math.inf, 0xFE),
    (-1e-9, 0x80),             # negative underflow keeps its sign
    (-0.0, 0x80),
    (0.0, 0x00),
    (math.nan, 0x7F),
])
def test_p3_ties_and_saturation(x, code):
    assert oracle.e4m3_encode(x) == code
    assert oracle.e4m3_encode_brute(x) == code
    assert oracle.e4m3_encode_closed(x) == code


def _all_bf16_f32():
    return (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)


def test_p4_closed_form_equals_brute_force_all_bf16():
    xs = _all_bf16_f32()
    for x in xs:
        assert oracle.e4m3_encode(x) == oracle.e4m3_encode_closed(x), x


def test_bisection_equals_brute_force_all_bf16():
    """The encoder the oracle uses (bisection over the increasing code
    values) and the definition's scan over all 127 candidates agree on every
    bf16 pattern."""
    for x in _all_bf16_f32():
        assert oracle.e4m3_encode(x) == oracle.e4m3_encode_brute(x), x


def test_bisection_equals_brute_force_random_f32():
    """... and on fp32 quotients of every magnitude (kv_write encodes x /
    scale, which is rarely a bf16 value), including fp32 subnormals and
    values just below and above the saturation bound."""
    rng = np.random.default_rng(11)
    n = 60000
    xs = (rng.standard_normal(n) * np.exp2(rng.uniform(-150, 10, n))).astype(np.float32)
    xs = np.concatenate([xs, np.float32(448) * (1 + rng.uniform(-1e-3, 1e-3, 2000)).astype(
        np.float32), rng.integers(0, 1 << 23, 2000, dtype=np.uint32).view(np.float32)])
    for x in xs:
        assert oracle.e4m3_encode(x) == oracle.e4m3_encode_brute(x), x


def test_p4_midpoints_and_neighbours():
    v = oracle.e4m3_decode_all()[:0x7F]
    mids = (v[:-1] + v[1:]) / 2.0
    for m in mids:
        m32 = np.float32(m)
        assert float(m32) == m  # midpoints are exact in fp32
        for x in (np.nextafter(m32, np.float32(-1)), m32,
                  np.nextafter(m32, np.float32(1000))):
            for s in (x, -x):
                assert oracle.e4m3_encode(s) == oracle.e4m3_encode_closed(s)
                assert oracle.e4m3_encode(s) == oracle.e4m3_encode_brute(s)
        lo = int(np.searchsorted(v, m) - 1)
        even = lo if lo % 2 == 0 else lo + 1
        assert oracle.e4m3_encode(m32) == even
        assert oracle.e4m3_encode(np.nextafter(m32, np.float32(-1))) == lo
        assert oracle.e4m3_encode(np.nextafter(m32, np.float32(1000))) == lo + 1


def test_p4_matches_torch_below_464_all_bf16():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest-even and
    saturates below 464, so in that range it must agree exactly."""
    xs = _all_bf16_f32()
    finite = np.isfinite(xs) & (np.abs(xs) < 464.0)
    xs = xs[finite]
    t = torch.from_numpy(xs.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([oracle.e4m3_encode(x) for x in xs], dtype=np.uint8)
    assert np.array_equal(t, ours)


def test_encode_error_bound():
    """|decode(encode(x)) - x| <= half the code spacing at x (rounding
    bound), for a spread of magnitudes below 448."""
    rng = np.random.default_rng(7)
    xs = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000))).astype(np.float32)
    xs = xs[np.abs(xs) < 448]
    for x in xs:
        c = oracle.e4m3_encode(x)
        a = abs(float(x))
        spacing = 2.0 ** -9 if a < 2.0 ** -6 else 2.0 ** (math.floor(math.log2(a)) - 3)
        assert abs(oracle.e4m3_decode(c) - float(x)) <= spacing / 2


def test_bf16_decode_is_upper_half_of_fp32():
    for bits in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x7F80, 0x0001, 0x4049):
        want = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
        assert oracle.bf16_to_f32(bits) == want or (np.isnan(want))
    assert oracle.bf16_to_f32(0x3F80) == 1.0
    assert oracle.bf16_to_f32(0xC000) == -2.0
    assert oracle.bf16_to_f32(0x4049) == np.float32(3.140625)
