"""Pins for the oracle's storage-format decoders (CPU only).

Each decoder is checked against (a) code points fixed by the format
definition, written by hand in tests/golden, and (b) an independent
implementation: torch's own fp8 / bf16 casts.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _code_points():
    out = []
    with open(os.path.join(GOLDEN, "e4m3fn_code_points.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()
            out.append((int(code, 16), float(val)))
    return out


@pytest.mark.parametrize("code,value", _code_points())
def test_e4m3fn_code_points(code, value):
    got = formats.decode_e4m3fn(np.array([code], dtype=np.uint8))[0]
    if math.isnan(value):
        assert math.isnan(got)
    else:
        assert got == value
        assert math.copysign(1.0, got) == math.copysign(1.0, value)


def test_e4m3fn_all_codes_match_torch_cast():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = formats.decode_e4m3fn(codes.numpy())
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))


def test_e4m3fn_integers_used_by_the_indexer_are_exact():
    vals = torch.arange(-8, 9, dtype=torch.float32)
    codes = vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(formats.decode_e4m3fn(codes), vals.numpy().astype(np.float64))


def test_bf16_matches_torch_cast():
    g = torch.Generator().manual_seed(1)
    bits = torch.randint(0, 65536, (20000,), generator=g, dtype=torch.int32)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # drop inf/NaN patterns
    t = bits.to(torch.int16).view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    got = formats.decode_bf16(bits.numpy().astype(np.uint16))
    assert np.array_equal(ref, got)
    assert formats.decode_bf16(np.array([0x3F80], dtype=np.uint16))[0] == 1.0
    assert formats.decode_bf16(np.array([0xC000], dtype=np.uint16))[0] == -2.0


def test_e8m0_code_points():
    got = formats.decode_e8m0(np.array([127, 128, 126, 123, 131, 0, 254, 255], dtype=np.uint8))
    assert list(got[:5]) == [1.0, 2.0, 0.5, 1.0 / 16, 16.0]
    assert got[5] == 2.0 ** -127
    assert got[6] == 2.0 ** 127
    assert math.isnan(got[7])


def test_mxfp8_block_scaling():
    # two blocks of 32: block 0 scaled by 2^-3, block 1 by 2^2
    vals = torch.linspace(-6, 6, 64)
    codes = vals.to(torch.float8_e4m3fn)
    scales = np.array([[127 - 3, 127 + 2]], dtype=np.uint8)
    got = formats.decode_mxfp8(codes.view(torch.uint8).numpy()[None, :], scales)
    e = codes.to(torch.float64).numpy()
    ref = np.concatenate([e[:32] * 0.125, e[32:] * 4.0])
    assert np.array_equal(got[0], ref)
    with pytest.raises(ValueError):
        formats.decode_mxfp8(np.zeros((1, 64), np.uint8), np.zeros((1, 3), np.uint8))
