"""Decoding of OCP e4m3fn codes for the tests (the GPU's FP8 stages are
compared as decoded values). Written from the format's definition: 1 sign
bit, 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
the subnormals m/8 * 2^-6; code 0x7F/0xFF is NaN and there is no infinity."""
import numpy as np


def e4m3_decode(codes: np.ndarray, scale_exp: int = -4) -> np.ndarray:
    """Values of e4m3fn codes stored at scale 2^-scale_exp."""
    c = np.asarray(codes).astype(np.int32)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((e == 0xF) & (m == 7), np.nan, v)
    return s * v * 2.0 ** scale_exp
