"""GPU parity of the cache append (bit-exact against the oracle's encoders).

Every written byte -- MXFP8 element and scale codes, bf16 and fp32 rows, FP8
and fp32 index keys -- is compared with oracle.quant.cache_append on the same
source values, and every row not named by a valid slot must keep its old
bytes. NaN payloads are not part of the contract: fp32 NaNs are compared as
NaN positions.
"""

import numpy as np
import pytest
import torch

import sparse_top_latent_amd as sga
from gpu_util import say
from oracle import quant
from sga_inputs import block_scaled_rows

pytestmark = pytest.mark.gpu

FMT = {"f32": torch.float32, "bf16": torch.bfloat16, "mxfp8": torch.uint8, "fp8": torch.uint8}


def _raw(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    return t.numpy().copy()


def _src64(t):
    return None if t is None else t.float().cpu().numpy().astype(np.float64)


def _caches(rows, D, DI, kv_fmt, idx_fmt):
    """Caches filled with arbitrary old contents (snapshotted before the call)."""
    dev = "cuda"
    if kv_fmt == "mxfp8":
        kv = torch.randint(0, 256, (rows, D), dtype=torch.uint8, device=dev)
    else:
        kv = torch.randn(rows, D, device=dev).to(FMT[kv_fmt])
    sc = torch.randint(0, 256, (rows, D // 32), dtype=torch.uint8, device=dev)
    ki = (torch.randint(0, 256, (rows, DI), dtype=torch.uint8, device=dev) if idx_fmt == "fp8"
          else torch.randn(rows, DI, device=dev))
    return kv, (sc if kv_fmt == "mxfp8" else None), ki


def _check(label, kv_new, ki_new, slots, rows, D, DI, kv_fmt, idx_fmt, sample=None):
    d_rope = 64 if D == 576 else 16
    prob = sga.Problem.for_cache(num_kv_rows=rows, d_latent=D - d_rope, d_rope=d_rope, idx_dim=DI,
                                 kv_dtype=kv_fmt, idx_dtype=idx_fmt)
    kv, sc, ki = _caches(rows, D, DI, kv_fmt, idx_fmt)
    ref_kv, ref_ki = _raw(kv), _raw(ki)
    ref_sc = _raw(sc) if sc is not None else np.zeros((rows, D // 32), np.uint8)
    say(f"case cache append {label}: N={slots.numel()} rows={rows} D={D} DI={DI} "
        f"{kv_fmt}/{idx_fmt} src={(kv_new if kv_new is not None else ki_new).dtype}")
    sga.sga_cache_append(prob, kv_new, ki_new, slots.cuda(), kv, sc, ki)
    torch.cuda.synchronize()
    got_kv, got_ki = _raw(kv), _raw(ki)
    got_sc = _raw(sc) if sc is not None else ref_sc
    s = slots.numpy()
    n = len(s)
    pick = np.arange(n) if sample is None else np.asarray(sample)
    # the oracle's append on the picked tokens (other valid slots are copied
    # from the GPU result, then checked only for being untouched elsewhere)
    keep = np.full(n, -1, dtype=np.int64)
    keep[pick] = s[pick]
    kvn = _src64(kv_new) if kv_new is not None else None
    kin = _src64(ki_new) if ki_new is not None else None
    kv_ref_full, sc_ref_full, ki_ref_full = ref_kv.copy(), ref_sc.copy(), ref_ki.copy()
    if kvn is not None:
        quant.cache_append(kvn, np.zeros((n, DI)), keep, kv_ref_full, sc_ref_full,
                           np.zeros_like(ki_ref_full), kv_fmt, idx_fmt)
    if kin is not None:
        dummy_kv = np.zeros((rows, D), dtype=np.float64)
        quant.cache_append(np.zeros((n, D)), kin, keep, dummy_kv, np.zeros_like(ref_sc),
                           ki_ref_full, "f32", idx_fmt)
    valid = (s >= 0) & (s < rows)
    written = np.unique(s[valid])
    touched_rows = np.zeros(rows, bool)
    touched_rows[written] = True
    checked = np.zeros(rows, bool)
    checked[keep[(keep >= 0) & (keep < rows)]] = True
    for name, got, ref, part in (("kv", got_kv, kv_ref_full, kvn), ("kv_scale", got_sc, sc_ref_full, kvn),
                                 ("k_idx", got_ki, ki_ref_full, kin)):
        if part is None:
            assert np.array_equal(got, ref, equal_nan=True), f"{label}: {name} changed"
            continue
        rows_chk = checked | ~touched_rows
        a, b = got[rows_chk], ref[rows_chk]
        eq = (a == b) | (np.isnan(a) & np.isnan(b)) if a.dtype == np.float64 else a == b
        if not eq.all():
            bad = np.argwhere(~eq)[:5]
            r = np.flatnonzero(rows_chk)[bad[:, 0]]
            raise AssertionError(f"{label}: {name} differs at rows/cols {list(zip(r, bad[:, 1]))}: "
                                 f"got {a[~eq][:5]} want {b[~eq][:5]}")


def _slots(n, rows, seed, dropped=True):
    g = torch.Generator().manual_seed(seed)
    s = torch.randperm(rows, generator=g)[:n].to(torch.int64)
    if dropped and n >= 8:
        s[1] = -1
        s[3] = rows
        s[5] = 1 << 40
        s[7] = -(1 << 62)
    return s


def _with_specials(x: torch.Tensor) -> torch.Tensor:
    x = x.clone()
    big = torch.finfo(x.dtype).max
    x[0, :32] = 0.0                                    # all-zero block
    x[2, 96:128] = 0.5
    x[2, 100] = float("nan")                           # NaN block
    x[4, 160:192] = -3.0
    x[4, 170] = float("-inf")                          # inf block
    x[6, 32:64] = 2.0 ** -130                          # bf16 / fp32 subnormal block
    x[8, 64:96] = torch.linspace(-448, 448, 32)        # max exactly 448: scale 2^0
    x[9, :32] = big                                    # largest finite: top scale
    x[9, 32:64] = -big / 3
    x[10, :32] = torch.tensor([1.0625, 1.1875] * 16)   # E4M3 ties at scale 2^-8 ... after scaling
    x[10, 0] = 1.0
    return x


def test_append_mxfp8_and_fp8_keys_from_bf16():
    N, rows, D, DI = 300, 1000, 576, 128
    kv_new = _with_specials(block_scaled_rows(N, D, 5, "app.kv", dtype="bf16")).cuda()
    ki = block_scaled_rows(N, DI, 5, "app.ki", dtype="bf16", spread=3)
    ki[1, :8] = torch.tensor([float("nan"), float("-nan"), float("inf"), float("-inf"), 500.0,
                              -1e30, 2.0 ** -130, -(2.0 ** -10)])
    _check("mxfp8+fp8 bf16", kv_new, ki.cuda(), _slots(N, rows, 1), rows, D, DI, "mxfp8", "fp8")


def test_append_every_bf16_pattern():
    # index keys: all 65,536 bf16 bit patterns (NaN, inf, subnormals, values
    # past 448, every tie) cast to E4M3FN at unit scale
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    allv = bits.view(torch.bfloat16)
    N, DI = 512, 128
    _check("every bf16 as an fp8 key", None, allv.view(N, DI).cuda(), _slots(N, 600, 2, False),
           600, 576, DI, "mxfp8", "fp8")
    # latent rows: every finite pattern, shuffled into 32-value MX blocks
    fin = allv[torch.isfinite(allv.float())]
    g = torch.Generator().manual_seed(3)
    fin = fin[torch.randperm(fin.numel(), generator=g)]
    N = fin.numel() // 576
    _check("every finite bf16 in MX blocks", fin[: N * 576].view(N, 576).cuda(), None,
           _slots(N, 200, 4, False), 200, 576, 128, "mxfp8", "fp8")


def test_append_f32_source_to_bf16_and_f32_keys():
    N, rows, D, DI = 200, 400, 576, 128
    x = block_scaled_rows(N, D, 6, "app.f32", dtype="f32", spread=30)
    x = _with_specials(x)
    # exact bf16 ties and round-to-infinity
    x[11, :64] = ((torch.arange(64, dtype=torch.int64) << 16) | 0x3f808000).to(torch.int32) \
        .view(torch.float32)
    x[12, 0] = torch.finfo(torch.float32).max
    x[12, 1] = -torch.finfo(torch.float32).max
    ki = block_scaled_rows(N, DI, 6, "app.f32k", dtype="f32")
    ki[3, 0] = float("nan")
    _check("bf16+f32 from f32", x.cuda(), ki.cuda(), _slots(N, rows, 5), rows, D, DI, "bf16", "f32")


def test_append_f32_source_to_mxfp8_with_fp32_subnormals():
    N, rows, D, DI = 64, 100, 576, 128
    x = block_scaled_rows(N, D, 7, "app.mxf32", dtype="f32", spread=20)
    x = _with_specials(x)
    x[13, :32] = torch.tensor([1e-40, -3e-42, 1e-45, 0.0] * 8)  # fp32 subnormals only
    x[14, :32] = 2.0 ** 127 * 1.5
    ki = block_scaled_rows(N, DI, 7, "app.mxf32k", dtype="f32", spread=4)
    _check("mxfp8+fp8 from f32", x.cuda(), ki.cuda(), _slots(N, rows, 6), rows, D, DI, "mxfp8", "fp8")


@pytest.mark.parametrize("kv_fmt,idx_fmt,src", [("bf16", "f32", "bf16"), ("f32", "fp8", "bf16"),
                                                ("f32", "f32", "f32"), ("bf16", "fp8", "f32")])
def test_append_small_rows(kv_fmt, idx_fmt, src):
    # the fp32 path's geometry: 80-value rows (not a multiple of 32), 32-value keys
    N, rows, D, DI = 70, 90, 80, 32
    x = block_scaled_rows(N, D, 8, "app.small", dtype=src, spread=6)
    ki = block_scaled_rows(N, DI, 8, "app.smallk", dtype=src, spread=2)
    _check(f"small {kv_fmt}/{idx_fmt}", x.cuda(), ki.cuda(), _slots(N, rows, 7), rows, D, DI,
           kv_fmt, idx_fmt)


def test_append_one_part_only_and_empty():
    N, rows, D, DI = 40, 50, 576, 128
    x = block_scaled_rows(N, D, 9, "app.one", dtype="bf16").cuda()
    ki = block_scaled_rows(N, DI, 9, "app.onek", dtype="bf16").cuda()
    _check("latent rows only", x, None, _slots(N, rows, 8), rows, D, DI, "mxfp8", "fp8")
    _check("index keys only", None, ki, _slots(N, rows, 9), rows, D, DI, "mxfp8", "fp8")
    _check("no tokens", x[:0], ki[:0], torch.zeros(0, dtype=torch.int64), rows, D, DI, "mxfp8", "fp8")


def test_append_prefill_chunk_into_full_cache():
    # a 4,096-token prefill chunk appended at positions 126,976 .. 131,071 of a
    # 131,072-row cache, then 16 decode tokens appended to 16 sequences of a
    # 16 x 131,072-row cache; sampled tokens checked against the oracle, every
    # other row checked for being untouched
    rows, D, DI = 131072, 576, 128
    N = 4096
    x = block_scaled_rows(N, D, 10, "app.prefill", dtype="bf16").cuda()
    ki = block_scaled_rows(N, DI, 10, "app.prefillk", dtype="bf16", spread=2).cuda()
    slots = torch.arange(rows - N, rows, dtype=torch.int64)
    _check("prefill chunk", x, ki, slots, rows, D, DI, "mxfp8", "fp8",
           sample=[0, 1, 2, 63, 64, 1000, 2047, 2048, 4000, 4095])
    B = 16
    x = block_scaled_rows(B, D, 11, "app.decode", dtype="bf16").cuda()
    ki = block_scaled_rows(B, DI, 11, "app.decodek", dtype="bf16", spread=2).cuda()
    slots = torch.arange(B, dtype=torch.int64) * rows + rows - 1
    _check("decode step", x, ki, slots, B * rows, D, DI, "mxfp8", "fp8")
