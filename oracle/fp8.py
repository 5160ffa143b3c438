"""FP8 E4M3 (the OCP "fn" variant) encode / decode for the FP8 residual-stream
variant of the forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (see the package docstring).

[mHC-cutile] (the page "mHC 算法分析 & cutile 高效实现") runs its first
benchmark, in its performance section before section 5, with every tensor in
torch.float8_e4m3fn and no scale factors.  That format is the E4M3 encoding of
the OCP 8-bit floating point specification (OFP8): 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 holds subnormals (mantissa x
2^-9); there are no infinities, and only S.1111.111 is NaN, so the largest
finite magnitude is 1.75 x 2^8 = 448.

Readings (the page gives no conversion rules of its own):
  * Values are stored unscaled (the page's benchmark passes no scales).
  * Narrowing rounds to nearest, ties to even, and saturates: every finite
    magnitude at or above 448 becomes +-448.  (torch's own cast returns NaN
    past the range instead; the kernels saturate, and so does this.)
  * The oracle computes in fp64 and encodes the exact fp64 value; the kernels
    encode their fp32 result.  The two can differ by one code where the exact
    value lies within fp32 rounding of a midpoint between two codes; the tests
    accept either neighbour exactly there and nowhere else.
"""

import numpy as np

E4M3_MAX = 448.0
_BIAS = 7


def e4m3_decode(codes):
    """Raw E4M3 codes (uint8) -> float64, exactly, by the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - _BIAS)
    sub = sign * (m / 8.0) * np.exp2(1.0 - _BIAS)
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def e4m3_encode(values):
    """float64 -> E4M3 codes: round to nearest even, saturate at +-448,
    NaN -> 0x7F.  Signed zeros keep their sign."""
    v = np.asarray(values, dtype=np.float64)
    a = np.abs(v)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.int64)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        # subnormal range |v| < 2^-6: code = round(|v| / 2^-9) (8 -> 2^-6, the
        # smallest normal, which is also code 8)
        q_sub = np.rint(a * 2.0 ** 9)
        # normal range: |v| = f * 2^k with f in [0.5, 1), so exponent k-1 and
        # mantissa (2f - 1) * 8 in [0, 8) before rounding
        f, k = np.frexp(a)
        q = np.rint((2.0 * f - 1.0) * 8.0)
        k = k - 1 + (q == 8)            # a mantissa that rounds up to 8 carries
        q = np.where(q == 8, 0.0, q)
        efield = k + _BIAS
        code_norm = (efield << 3) + q.astype(np.int64)
        code = np.where(a < 2.0 ** -6, q_sub.astype(np.int64), code_norm)
        code = np.where(a >= E4M3_MAX, 0x7E, code)   # saturate (448 is S.1111.110)
        code = np.where(np.isnan(v), 0x7F, code | sign)
    return code.astype(np.uint8)


def quantize(values):
    """The value E4M3 represents after encoding (float64)."""
    return e4m3_decode(e4m3_encode(values))


def e4m3_neighbors_ok(codes, exact, rel=1e-5, absolute=1e-12):
    """True where `codes` equals the encoding of `exact`, or where `exact` lies
    within rel*|exact| + absolute of a rounding midpoint and `codes` is the
    encoding of a value on either side of that midpoint."""
    codes = np.asarray(codes, dtype=np.uint8)
    exact = np.asarray(exact, dtype=np.float64)
    tol = rel * np.abs(exact) + absolute
    lo = e4m3_encode(exact - tol)
    hi = e4m3_encode(exact + tol)
    mid = e4m3_encode(exact)
    return (codes == mid) | (codes == lo) | (codes == hi)
