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
