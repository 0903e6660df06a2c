"""Encoding into the cache storage formats, and the cache append (oracle side).

Test infrastructure only: see the package docstring.

Sources: "A.X K2 Technical Report", FP8 training section (MXFP8: E4M3
elements, one shared scale per block of 32 consecutive values, after the OCP
microscaling formats it cites), and the FP8 KV cache of the serving sweep in
"A.X-K2: a sparse-attention upgrade that costs nothing, trained natively in
FP8", section "Sparse Gated Attention". The pages fix the format, not the
encoder; readings taken from the OCP MX definition the report cites:
  * the shared scale of a block is 2^(floor(log2(max |v|)) - 8), 8 being the
    exponent of E4M3's largest normal value (448 = 1.75 * 2^8), clamped to
    the E8M0 range 2^-127 .. 2^127; an all-zero block takes 2^-127;
  * elements are v / scale rounded to the nearest E4M3FN value, ties to the
    even code, and magnitudes past 448 saturate to 448;
  * a block holding an infinity or a NaN gets the NaN scale code 0xFF and the
    NaN element code 0x7F in every place;
  * index keys (the pages say only that the indexer runs in FP8) are stored as
    plain E4M3FN values with the same rounding, unit scale;
  * a bf16 cache row is the source rounded to bf16, to nearest, ties to even.

Everything here is written from those definitions in float64: the E4M3FN
encoder enumerates every code and picks the nearest value; the bf16 encoder
rounds the significand by plain arithmetic.
"""

from __future__ import annotations

import math

import numpy as np

from .formats import E4M3FN_TABLE

# finite non-negative E4M3FN values and their codes (0x00 .. 0x7E), ascending
_POS_VALUES = E4M3FN_TABLE[:0x7F]
assert np.all(np.diff(_POS_VALUES) > 0)
E4M3_MAX = float(_POS_VALUES[-1])  # 448
E4M3_EMAX = 8                      # 448 = 1.75 * 2^8
MX_BLOCK = 32


def encode_e4m3fn_scalar(x: float) -> int:
    """One value -> its E4M3FN code: nearest value, ties to the even code,
    saturating at 448; NaN -> 0x7F (0xFF when the sign bit is set)."""
    neg = math.copysign(1.0, x) < 0
    if math.isnan(x):
        return 0xFF if neg else 0x7F
    a = abs(x)
    if a >= E4M3_MAX:
        code = 0x7E
    else:
        i = int(np.searchsorted(_POS_VALUES, a))  # _POS_VALUES[i - 1] < a <= _POS_VALUES[i]
        if _POS_VALUES[i] == a:
            code = i
        else:
            lo, hi = i - 1, i
            dlo, dhi = a - _POS_VALUES[lo], _POS_VALUES[hi] - a
            if dlo != dhi:
                code = lo if dlo < dhi else hi
            else:
                code = lo if lo % 2 == 0 else hi
    return code | (0x80 if neg else 0)


def encode_e4m3fn(x) -> np.ndarray:
    """float64 array -> uint8 E4M3FN codes (element by element)."""
    a = np.asarray(x, dtype=np.float64)
    flat = [encode_e4m3fn_scalar(float(v)) for v in a.ravel()]
    return np.array(flat, dtype=np.uint8).reshape(a.shape)


def encode_bf16_scalar(x: float) -> int:
    """One value -> its bfloat16 bit pattern, to nearest, ties to even.

    bf16 keeps 8 significant bits (7 stored) with fp32's exponent range:
    below 2^-126 the quantum stays 2^-133 (subnormals); results of 2^128 and
    above are infinities. NaN -> the quiet NaN of the same sign.
    """
    neg = math.copysign(1.0, x) < 0
    if math.isnan(x):
        return 0xFFC0 if neg else 0x7FC0
    a = abs(x)
    if math.isinf(a):
        r = math.inf
    elif a == 0.0:
        r = 0.0
    else:
        _, e = math.frexp(a)                 # a = m * 2^e, 0.5 <= m < 1
        q = math.ldexp(1.0, max(e, -125) - 8)  # quantum of the bf16 binade holding a
        n = a / q                            # exact: q is a power of two
        f = math.floor(n)
        rem = n - f
        if rem > 0.5 or (rem == 0.5 and f % 2 == 1):
            f += 1
        r = f * q
        if r >= 2.0 ** 128:
            r = math.inf
    bits = int(np.array(r, dtype=np.float32).view(np.uint32)) >> 16
    return bits | (0x8000 if neg else 0)


def encode_bf16(x) -> np.ndarray:
    """float64 array -> uint16 bf16 bit patterns (element by element)."""
    a = np.asarray(x, dtype=np.float64)
    flat = [encode_bf16_scalar(float(v)) for v in a.ravel()]
    return np.array(flat, dtype=np.uint16).reshape(a.shape)


def mx_block_scale_exp(block):
    """Shared exponent of one block; None when the block holds inf or NaN."""
    b = np.asarray(block, dtype=np.float64)
    if not np.all(np.isfinite(b)):
        return None
    amax = float(np.max(np.abs(b))) if b.size else 0.0
    if amax == 0.0:
        return -127
    _, e = math.frexp(amax)  # amax = m * 2^e with 0.5 <= m < 1: floor(log2 amax) = e - 1
    return max(-127, min(127, e - 1 - E4M3_EMAX))


def encode_mxfp8_row(row):
    """One row (length a multiple of 32) -> (E4M3FN codes, E8M0 scale codes)."""
    r = np.asarray(row, dtype=np.float64)
    if r.size % MX_BLOCK:
        raise ValueError("row length is not a multiple of 32")
    nb = r.size // MX_BLOCK
    codes = np.zeros(r.size, dtype=np.uint8)
    scales = np.zeros(nb, dtype=np.uint8)
    for j in range(nb):
        sl = slice(j * MX_BLOCK, (j + 1) * MX_BLOCK)
        se = mx_block_scale_exp(r[sl])
        if se is None:
            scales[j] = 0xFF
            codes[sl] = 0x7F
        else:
            scales[j] = se + 127
            codes[sl] = encode_e4m3fn(np.ldexp(r[sl], -se))
    return codes, scales


def encode_mxfp8(rows):
    """[..., D] float64 -> ([..., D] uint8 codes, [..., D / 32] uint8 scales)."""
    r = np.asarray(rows, dtype=np.float64)
    flat = r.reshape(-1, r.shape[-1])
    codes = np.zeros(flat.shape, dtype=np.uint8)
    scales = np.zeros((flat.shape[0], flat.shape[1] // MX_BLOCK), dtype=np.uint8)
    for i, x in enumerate(flat):
        codes[i], scales[i] = encode_mxfp8_row(x)
    return codes.reshape(r.shape), scales.reshape(r.shape[:-1] + (scales.shape[1],))


def cache_append(kv_new, kidx_new, slots, kv, kv_scale, k_idx, kv_fmt: str, idx_fmt: str):
    """Write N new tokens into the caches, in place (numpy arrays).

    kv_new [N, D] and kidx_new [N, DI] are the new rows as float64 (the
    source values); token i goes to cache row slots[i], and tokens whose slot
    lies outside [0, rows) are dropped. kv_fmt is "f32", "bf16" or "mxfp8"
    (kv then holds fp32 values, uint16 bf16 bits or uint8 codes, with
    kv_scale [rows, D / 32] for "mxfp8"); idx_fmt is "f32" or "fp8".
    """
    rows = kv.shape[0]
    for i, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0 or s >= rows:
            continue
        if kv_fmt == "f32":
            kv[s] = kv_new[i]
        elif kv_fmt == "bf16":
            kv[s] = encode_bf16(kv_new[i])
        else:
            kv[s], kv_scale[s] = encode_mxfp8_row(kv_new[i])
        if idx_fmt == "f32":
            k_idx[s] = kidx_new[i]
        else:
            k_idx[s] = encode_e4m3fn(kidx_new[i])
