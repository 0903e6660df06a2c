"""Exact decoding of the storage formats the SGA inputs arrive in (oracle side).

Test infrastructure only: see the package docstring.

Every decoder maps stored bits to float64 exactly. The tables are written
from the format definitions, not taken from a library, and the tests pin
them against independent implementations (torch's casts) and against code
points the format definitions fix.
"""

from __future__ import annotations

import numpy as np


def _e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN byte.

    Layout s.eeee.mmm with exponent bias 7; exponent field 0 encodes
    subnormals 2^-6 * m/8; there are no infinities and only the two codes
    with every exponent and mantissa bit set (0x7F, 0xFF) are NaN, which
    frees e=15 for the finite values 256..448. This is the element format of
    the MX (microscaling) FP8 blocks the technical report's FP8 section
    trains with (E4M3, one shared scale per 32 consecutive values).
    """
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * (m / 8.0) * 2.0 ** (1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3FN_TABLE = np.array([_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def decode_e4m3fn(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 values (exact)."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_bf16(bits) -> np.ndarray:
    """uint16 bfloat16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e8m0(codes) -> np.ndarray:
    """uint8 E8M0 scale codes -> float64: code e means 2^(e - 127); 0xFF is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def decode_mxfp8(codes, scales, block: int = 32) -> np.ndarray:
    """MXFP8 rows -> float64.

    Element j of a row is its E4M3FN value times the E8M0 scale of block
    j // 32 of the same row (the report's FP8 section: each block of 32
    consecutive values shares one scaling factor).
    """
    v = decode_e4m3fn(codes)
    s = decode_e8m0(scales)
    if v.shape[-1] != s.shape[-1] * block:
        raise ValueError("scale count does not match the row length")
    return v * np.repeat(s, block, axis=-1)


def decode(raw: np.ndarray, dtype: str, scales=None) -> np.ndarray:
    """Decode a raw storage array by its dtype tag ("f32", "bf16", "fp8", "mxfp8")."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "fp8":
        return decode_e4m3fn(raw)
    if dtype == "mxfp8":
        return decode_mxfp8(raw, scales)
    raise ValueError(dtype)
