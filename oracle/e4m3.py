"""OCP 8-bit floating point, E4M3 variant (e4m3fn), decoded from its bit fields.

Oracle (test infrastructure only).  The pages use OCP E4M3 K/V caches whose
largest finite value is 448 ("Support paged FP8 Flash attention ..." overview
and the perf-matrix description).  The format: 1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals
m/8 * 2^-6; the all-ones exponent with all-ones mantissa (0x7F, 0xFF) is NaN;
there is no infinity.
"""
import numpy as np


def decode_e4m3(b) -> np.ndarray:
    """uint8 array of E4M3 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where((b >> 7) & 1, -1.0, 1.0)
    exp = (b >> 3) & 0xF
    man = (b & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(exp.astype(np.float64) - 7.0)
    sub = (man / 8.0) * np.exp2(-6.0)
    val = np.where(exp == 0, sub, normal)
    val = np.where((exp == 0xF) & ((b & 0x7) == 0x7), np.nan, val)
    return sign * val


E4M3_MAX = 448.0


def encode_e4m3(y) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8), rounding to nearest with ties to
    even and saturating: |y| >= 448 gives +-448 (the format has no infinity,
    and the code above 448 is NaN); NaN gives 0x7F with the sign of y.

    Written from the format: a value a >= 2^-6 is (1 + m/8) 2^e with
    e = floor(log2 a), so its 3-bit mantissa is the integer nearest to
    a / 2^(e-3) (8..16, where 16 carries into the next exponent); below
    2^-6 the step is 2^-9 and the code is the nearest multiple of it.
    """
    y = np.asarray(y, dtype=np.float32).astype(np.float64)     # exact
    sign = np.signbit(y).astype(np.int64) << 7
    a = np.abs(y)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, a)
    sat = a >= E4M3_MAX
    a = np.minimum(a, E4M3_MAX)          # saturated entries are replaced below
    # normal range: e = floor(log2 a) from frexp (a = f 2^x with 0.5 <= f < 1)
    _, x = np.frexp(np.where(a > 0, a, 1.0))
    e = x.astype(np.int64) - 1
    q = np.rint(a / np.exp2((e - 3).astype(np.float64))).astype(np.int64)   # 8..16, ties to even
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    normal_code = ((e + 7) << 3) | (q - 8)
    # subnormal range (a < 2^-6): nearest multiple of 2^-9, ties to even (8 is the smallest normal)
    sub_code = np.rint(np.minimum(a, 2.0 ** -6) * 512.0).astype(np.int64)
    code = np.where(a < 2.0 ** -6, sub_code, normal_code)
    code = np.where(sat, 0x7E, code)
    code = np.where(nan, 0x7F, code)
    return (code | sign).astype(np.uint8)
