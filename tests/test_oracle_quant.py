"""Pins for the oracle's encoders and cache append (CPU only).

The encoders are checked against (a) torch's own float32 -> bfloat16 and
float32 -> float8_e4m3fn casts, (b) block encodings worked out by hand from
the OCP microscaling definition (tests/golden/mxfp8_blocks.txt), (c) the
property that fixes an MX scale: it is the power of two that puts the block
maximum in E4M3's top binade [256, 512), and (d) the rounding error bound of
a 3-bit significand.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _wide_f32(n, seed):
    g = np.random.default_rng(seed)
    x = g.standard_normal(n) * np.exp(g.standard_normal(n) * 20)
    with np.errstate(over="ignore"):
        return x.astype(np.float32)


def test_bf16_encoder_matches_torch_cast():
    x = _wide_f32(20000, 0)
    # exact halfway cases: a random bf16 value plus half its last place
    g = np.random.default_rng(1)
    hb = (g.integers(0, 1 << 16, 4000, dtype=np.uint32) << 16) | np.uint32(0x8000)
    half = hb.view(np.float32)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.39e38, 1e-45, -1e-40,
                         1.17549435e-38, np.finfo(np.float32).max], dtype=np.float32)
    x = np.concatenate([x, half[np.isfinite(half)], specials])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = quant.encode_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_encoder_nan_stays_nan():
    got = quant.encode_bf16(np.array([np.nan, -np.nan]))
    assert np.all(np.isnan(formats.decode_bf16(got)))


def test_e4m3fn_encoder_matches_torch_cast_in_range():
    x = _wide_f32(20000, 2) * np.float32(1e-6)
    # midpoints between every pair of adjacent finite codes (ties to even)
    pos = formats.E4M3FN_TABLE[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids, np.float32(pos), np.float32(-pos)])
    x = x[np.abs(x) < 464]  # torch turns larger values into NaN instead of saturating
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(quant.encode_e4m3fn(x.astype(np.float64)), ref)


def test_e4m3fn_encoder_ties_go_to_even_codes():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 halfway
    # between 1.125 (0x39) and 1.25 (0x3A); 2^-10 halfway between 0 and 2^-9
    got = quant.encode_e4m3fn([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -11, -1.0625])
    assert list(got) == [0x38, 0x3A, 0x00, 0x01, 0xB8]


def test_e4m3fn_encoder_saturates_and_keeps_nan():
    got = quant.encode_e4m3fn([448.0, 464.0, 500.0, 1e30, np.inf, -np.inf, -1e9, np.nan])
    assert list(got[:7]) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert math.isnan(formats.decode_e4m3fn(got[7:])[0])


def test_e4m3fn_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(quant.encode_e4m3fn(formats.decode_e4m3fn(codes)), codes)


def _golden_blocks():
    out = []
    with open(os.path.join(GOLDEN, "mxfp8_blocks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                m, s, c = line.split()
                out.append((float(m), int(s, 16), int(c, 16)))
    return out


@pytest.mark.parametrize("vmax,scale_byte,code", _golden_blocks())
def test_mxfp8_hand_worked_blocks(vmax, scale_byte, code):
    blk = np.zeros(32)
    blk[5] = float(np.float32(vmax))
    c, s = quant.encode_mxfp8_row(blk)
    assert s[0] == scale_byte and c[5] == code
    assert np.all(np.delete(c, 5) == 0)


def test_mxfp8_nonfinite_block_is_nan():
    row = np.ones(64)
    row[40] = np.inf
    c, s = quant.encode_mxfp8_row(row)
    assert s[1] == 0xFF and np.all(c[32:] == 0x7F)
    assert s[0] == 0x77 and np.all(c[:32] == 0x78)
    assert np.all(np.isnan(formats.decode_mxfp8(c, s)[32:]))


def test_mxfp8_scale_puts_the_block_max_in_the_top_binade_and_error_is_bounded():
    g = np.random.default_rng(3)
    rows = g.standard_normal((40, 576)) * np.exp(g.standard_normal((40, 18)) * 6).repeat(32, 1)
    rows[0, :32] = 0.0
    rows = rows.astype(np.float32).astype(np.float64)
    c, s = quant.encode_mxfp8(rows)
    scale = formats.decode_e8m0(s).repeat(32, 1)
    blocks = np.abs(rows).reshape(40, 18, 32).max(-1)
    top = blocks / formats.decode_e8m0(s)
    nz = blocks > 0
    assert np.all((top[nz] >= 256) & (top[nz] < 512))
    assert np.all(s[~nz] == 0)
    back = formats.decode_mxfp8(c, s)
    y = np.abs(rows) / scale
    err = np.abs(back - rows)
    normal = (y >= 2.0 ** -6) & (y <= 448)
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(rows[normal]))
    sub = y < 2.0 ** -6
    assert np.all(err[sub] <= 2.0 ** -10 * scale[sub])
    sat = y > 448
    assert np.array_equal(back[sat], np.sign(rows[sat]) * 448 * scale[sat])
    assert np.array_equal(np.signbit(back[rows != 0]), np.signbit(rows[rows != 0]))


def test_cache_append_writes_valid_slots_only():
    g = np.random.default_rng(4)
    rows, D, DI = 10, 64, 32
    kv_new = g.standard_normal((4, D))
    ki_new = np.round(g.standard_normal((4, DI)) * 4)
    slots = np.array([7, -1, 2, 10])
    for fmt in ("f32", "bf16", "mxfp8"):
        dt = {"f32": np.float64, "bf16": np.uint16, "mxfp8": np.uint8}[fmt]
        kv = np.full((rows, D), 3, dtype=dt)
        sc = np.full((rows, D // 32), 9, dtype=np.uint8)
        ki = np.full((rows, DI), 5, dtype=np.uint8)
        quant.cache_append(kv_new, ki_new, slots, kv, sc, ki, fmt, "fp8")
        untouched = [r for r in range(rows) if r not in (7, 2)]
        assert np.all(kv[untouched] == 3) and np.all(ki[untouched] == 5)
        for i, r in ((0, 7), (2, 2)):
            dec = formats.decode(kv[r], fmt, sc[r]) if fmt != "f32" else kv[r]
            assert np.allclose(dec, kv_new[i], rtol=2.0 ** -4, atol=1e-6)
            # small integers are exact in E4M3FN
            assert np.array_equal(formats.decode_e4m3fn(ki[r]), ki_new[i])
        if fmt == "mxfp8":
            assert np.all(sc[untouched] == 9)
