"""FP8 E4M3 KV: the exact value of every stored code.

Fitting a Million Tokens, Sec. 02 names FP8 E4M3 as the plain option for
the KV cache: exactly half the bytes of fp16, no calibration, no groups.  The
reading taken here is that codes are stored with no scale (value = code's
E4M3 value).  The format is the OCP 8-bit floating point E4M3 encoding that
the serving stacks that section names use: 1 sign bit, 4 exponent bits with
bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the
all-ones exponent with mantissa 7 is NaN; there is no infinity; the largest
finite value is 448.

Parity pins (tests/test_oracle_fp8.py): hand-derived codes of the format
definition, and torch's float8_e4m3fn decode over all 256 codes.
"""
from __future__ import annotations

import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    """float64 value of each uint8 code."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 8.0, (exp - 7).astype(np.int64))
    subnormal = sign * np.ldexp(man, -9)
    out = np.where(exp == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def decode_pool(pool_codes) -> np.ndarray:
    """float64 array of the same shape as an E4M3 code array (e.g. a pool slice)."""
    table = decode_e4m3(np.arange(256, dtype=np.uint8))
    return table[np.asarray(pool_codes, dtype=np.uint8)]
