"""Pins for the oracle's FP8 E4M3 encode / decode (oracle/fp8.py): checks
against the OCP 8-bit floating point definition (values the format fixes),
against torch's float8_e4m3fn conversions (a library routine) where the two
conventions agree, and against the readings the FP8 variant states
(round-to-nearest-even, saturation at 448).  A planted mistake in either
function must trip at least one pin.

[mHC-cutile] = "mHC 算法分析 & cutile 高效实现"; its first benchmark runs with
every tensor in torch.float8_e4m3fn.
"""

import numpy as np
import pytest
import torch

import oracle.fp8 as FP8

pytestmark = pytest.mark.cpu


def _enc(m, v):
    return int(m.e4m3_encode(np.array([v], np.float64))[0])


def _dec(m, c):
    return float(m.e4m3_decode(np.array([c], np.uint8))[0])


def pin_named_values(m):
    """Codes and values the OCP E4M3 definition fixes."""
    table = [(0x00, 0.0), (0x38, 1.0), (0x40, 2.0), (0x3F, 1.875), (0x7E, 448.0),
             (0xFE, -448.0), (0x08, 2.0 ** -6), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
             (0x77, 240.0), (0xB8, -1.0), (0x30, 0.5)]
    for code, val in table:
        assert _dec(m, code) == val, hex(code)
        assert _enc(m, val) == code, hex(code)
    assert np.isnan(_dec(m, 0x7F)) and np.isnan(_dec(m, 0xFF))
    assert _enc(m, -0.0) == 0x80 and _enc(m, float("nan")) & 0x7F == 0x7F


def pin_decode_matches_torch(m):
    """All 256 codes decode as torch's float8_e4m3fn does."""
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = m.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def pin_encode_matches_torch_in_range(m):
    """Inside the range both round to nearest even; values are fp32 so torch's
    conversion rounds once."""
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.uniform(-447.0, 447.0, 20000),
        rng.standard_normal(20000),
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000),          # subnormal range
        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000),
    ]).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = m.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(got, ref)


def pin_ties_to_even(m):
    """Exact midpoints go to the code with the even mantissa."""
    assert _enc(m, 1.0625) == 0x38        # between 1.0 (m=0) and 1.125 (m=1)
    assert _enc(m, 1.1875) == 0x3A        # between 1.125 (m=1) and 1.25 (m=2)
    assert _enc(m, 1.9375) == 0x40        # between 1.875 (m=7) and 2.0 (next binade, m=0)
    assert _enc(m, 2.0 ** -10) == 0x00    # between 0 and the smallest subnormal
    assert _enc(m, 3 * 2.0 ** -10) == 0x02
    assert _enc(m, -1.0625) == 0xB8


def pin_saturation(m):
    """The variant's reading: finite magnitudes at or past 448 become +-448."""
    for v, c in ((448.0, 0x7E), (449.0, 0x7E), (464.0, 0x7E), (470.0, 0x7E), (1e30, 0x7E),
                 (-1e30, 0xFE), (-460.0, 0xFE), (float("inf"), 0x7E)):
        assert _enc(m, v) == c, v


def pin_roundtrip_and_order(m):
    """encode(decode(c)) = c for every finite code, and the positive codes are
    strictly increasing in value."""
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    back = m.e4m3_encode(m.e4m3_decode(codes))
    assert np.array_equal(back, codes)
    pos = m.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def pin_neighbor_rule(m):
    """The comparison rule: exact match away from midpoints, either neighbour
    at a midpoint."""
    exact = np.array([1.0, 1.0625, 1.3, 100.0 + 1e-9, 2.0 ** -10])
    enc = m.e4m3_encode(exact)
    assert m.e4m3_neighbors_ok(enc, exact).all()
    # one code off, away from a midpoint: rejected
    assert not m.e4m3_neighbors_ok(np.array([0x39], np.uint8), np.array([1.0])).any()
    assert not m.e4m3_neighbors_ok(np.array([0x3B], np.uint8), np.array([1.3])).any()
    # at a midpoint (within fp32 rounding of it): both neighbours accepted
    assert m.e4m3_neighbors_ok(np.array([0x38, 0x39], np.uint8), np.array([1.0625, 1.0625 + 1e-9])).all()


PINS = [pin_named_values, pin_decode_matches_torch, pin_encode_matches_torch_in_range,
        pin_ties_to_even, pin_saturation, pin_roundtrip_and_order, pin_neighbor_rule]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(FP8)


# ----------------------------------------------------------------------------
# planted mistakes (each must trip at least one pin)
# ----------------------------------------------------------------------------

_orig_decode, _orig_encode = FP8.e4m3_decode, FP8.e4m3_encode


def _mut_decode_bias8(codes):          # the FNUZ variant's bias
    return _orig_decode(codes) / 2.0


def _mut_decode_no_subnormals(codes):
    c = np.asarray(codes, np.uint8)
    out = _orig_decode(c)
    return np.where(((c >> 3) & 0xF) == 0, 0.0 * out, out)


def _mut_encode_half_up(values):
    v = np.asarray(values, np.float64)
    lo = _orig_encode(v)
    # where v is exactly a midpoint, pick the upper neighbour in magnitude
    a = np.abs(v)
    lo_v = np.abs(_orig_decode(lo))
    up = _orig_encode(np.nextafter(a, np.inf) * np.sign(np.where(v == 0, 1, v)))
    up_v = np.abs(_orig_decode(up))
    return np.where((lo_v != up_v) & (lo_v < a), up, lo)


def _mut_encode_truncate(values):
    v = np.asarray(values, np.float64)
    code = _orig_encode(v)
    val = _orig_decode(code)
    # step one code towards zero where rounding went up in magnitude
    down = np.where((np.abs(val) > np.abs(v)) & ((code & 0x7F) > 0), code - 1, code)
    return down.astype(np.uint8)


def _mut_encode_nan_past_range(values):
    v = np.asarray(values, np.float64)
    code = _orig_encode(v)
    return np.where(np.abs(v) > 448.0, (code | 0x7F), code).astype(np.uint8)


def _mut_encode_no_carry(values):
    v = np.asarray(values, np.float64)
    a = np.abs(v)
    f, k = np.frexp(a)
    q = np.rint((2.0 * f - 1.0) * 8.0)
    code = _orig_encode(v)
    # a mantissa that rounds to 8 wraps to 0 in the same binade
    wrapped = np.where((q == 8) & (a >= 2.0 ** -6) & (a < 448.0), code - 8, code)
    return wrapped.astype(np.uint8)


MUTATIONS = [
    ("e4m3_decode", _mut_decode_bias8),
    ("e4m3_decode", _mut_decode_no_subnormals),
    ("e4m3_encode", _mut_encode_half_up),
    ("e4m3_encode", _mut_encode_truncate),
    ("e4m3_encode", _mut_encode_nan_past_range),
    ("e4m3_encode", _mut_encode_no_carry),
]


@pytest.mark.parametrize("name,fn", MUTATIONS, ids=[f.__name__ for _, f in MUTATIONS])
def test_planted_mistake_is_caught(monkeypatch, name, fn):
    monkeypatch.setattr(FP8, name, fn)
    tripped = []
    for pin in PINS:
        try:
            pin(FP8)
        except AssertionError:
            tripped.append(pin.__name__)
    assert tripped, f"no pin catches {fn.__name__}"
