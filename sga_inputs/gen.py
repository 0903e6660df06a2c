"""Counter-based, seeded input generator for the SGA hot path.

Every element is drawn from ``hash32(key(seed, tensor), index)``, where the
hash is two rounds of the 32-bit MurmurHash3 finaliser ("fmix32", A. Appleby,
public domain). Integer arithmetic is carried out in int64 tensors with the
32-bit products split into 16-bit halves, so no intermediate overflows and
the CPU and GPU results are bit-identical. Nothing here knows what the
values are used for.

Distributions (the recipe the design notes restate):

* normal values use a 65,536-level quantile table of N(0, 1): the top 16 bits
  of the hash pick quantile (i + 0.5) / 65536. bf16 and FP8 tensors store
  that quantile rounded to nearest-even in their format;
* integers on {lo..hi} use Lemire's multiply-shift on 24 hash bits;
* the per-(query, head) indexer weight w is dyadic: for the FP8 configs
  ``w = floor(256 u) / 256`` with u ~ U(0, 1); for the fp32 tiny config
  ``w = round(1024 z) / 1024`` with z ~ N(0, 1);
* varlen context lengths are ``floor(exp(U(ln lo, ln hi)))``.
"""

from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import torch

_M32 = 0xFFFFFFFF
_CHUNK = 1 << 24


# --------------------------------------------------------------------------
# counter-based hash
# --------------------------------------------------------------------------
def _mul32(a: torch.Tensor, c: int) -> torch.Tensor:
    """(a * c) mod 2^32 for int64 tensors holding values in [0, 2^32)."""
    lo = c & 0xFFFF
    hi = c >> 16
    return (a * lo + (((a * hi) & 0xFFFF) << 16)) & _M32


def _fmix32(h: torch.Tensor) -> torch.Tensor:
    h = h ^ (h >> 16)
    h = _mul32(h, 0x85EBCA6B)
    h = h ^ (h >> 13)
    h = _mul32(h, 0xC2B2AE35)
    h = h ^ (h >> 16)
    return h


def _keys(seed: int, name: str) -> Tuple[int, int]:
    a = zlib.crc32(f"sga:{seed}:{name}:a".encode()) & _M32
    b = zlib.crc32(f"sga:{seed}:{name}:b".encode()) & _M32
    return a, b


def hash32(seed: int, name: str, idx: torch.Tensor) -> torch.Tensor:
    """32 random bits (as int64 in [0, 2^32)) for each int64 counter in idx."""
    ka, kb = _keys(seed, name)
    lo = idx & _M32
    hi = idx >> 32
    h = _fmix32(lo ^ ka)
    return _fmix32(h ^ ((hi + kb) & _M32))


def _fill(out: torch.Tensor, seed: int, name: str, fn) -> torch.Tensor:
    """out.view(-1)[i] = fn(hash32(seed, name, i)), in bounded chunks."""
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        idx = torch.arange(s, e, dtype=torch.int64, device=out.device)
        flat[s:e] = fn(hash32(seed, name, idx))
    return out


# --------------------------------------------------------------------------
# value tables (built once on the CPU, copied to a device on demand)
# --------------------------------------------------------------------------
_TABLES: Dict[Tuple[str, str], torch.Tensor] = {}


def _quantiles() -> torch.Tensor:
    u = (torch.arange(65536, dtype=torch.float64) + 0.5) / 65536.0
    return torch.special.ndtri(u)


def _table(kind: str, device) -> torch.Tensor:
    key = (kind, str(device))
    t = _TABLES.get(key)
    if t is not None:
        return t
    q = _quantiles()
    if kind == "f32":
        t = q.to(torch.float32)
    elif kind == "bf16_std1":
        t = q.to(torch.float32).to(torch.bfloat16)
    elif kind == "bf16_std_sqrt2":
        t = (q * math.sqrt(2.0)).to(torch.float32).to(torch.bfloat16)
    elif kind == "e4m3":
        t = q.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)
    elif kind == "w1024":
        t = torch.round(q * 1024.0).to(torch.int32)
    elif kind == "int_e4m3":  # code of the integer v at index v + 128 (v in [-8, 8])
        vals = torch.arange(-128, 128, dtype=torch.float32).clamp(-8, 8)
        t = vals.to(torch.float8_e4m3fn).view(torch.uint8)
    else:
        raise KeyError(kind)
    t = t.to(device)
    _TABLES[key] = t
    return t


def normal(shape, seed, name, *, dtype="f32", std=1.0, device="cpu") -> torch.Tensor:
    """Quantised N(0, std^2) values stored as fp32, bf16 or E4M3FN codes (uint8)."""
    if dtype == "f32":
        if std != 1.0:
            raise ValueError("fp32 normals are drawn with std 1")
        tab = _table("f32", device)
        out = torch.empty(shape, dtype=torch.float32, device=device)
    elif dtype == "bf16":
        tab = _table("bf16_std1" if std == 1.0 else "bf16_std_sqrt2", device)
        if std not in (1.0, math.sqrt(2.0)):
            raise ValueError("bf16 normals are drawn with std 1 or sqrt(2)")
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    elif dtype == "e4m3":
        if std != 1.0:
            raise ValueError("E4M3 normals are drawn with std 1")
        tab = _table("e4m3", device)
        out = torch.empty(shape, dtype=torch.uint8, device=device)
    else:
        raise ValueError(dtype)
    return _fill(out, seed, name, lambda h: tab[h >> 16])


def uniform_int(shape, seed, name, lo: int, hi: int, *, device="cpu") -> torch.Tensor:
    """Integers uniform on {lo..hi} (int32)."""
    m = hi - lo + 1
    if not (1 <= m <= 256):
        raise ValueError("range too wide")
    out = torch.empty(shape, dtype=torch.int32, device=device)
    return _fill(out, seed, name, lambda h: (lo + (((h >> 8) * m) >> 24)).to(torch.int32))


def int_values(shape, seed, name, r: int, *, dtype: str, device="cpu") -> torch.Tensor:
    """Integers uniform on {-r..r}, stored as fp32 or as E4M3FN codes."""
    if dtype == "f32":
        out = torch.empty(shape, dtype=torch.float32, device=device)
        m = 2 * r + 1
        return _fill(out, seed, name, lambda h: (-r + (((h >> 8) * m) >> 24)).to(torch.float32))
    if dtype == "fp8":
        if r > 8:
            raise ValueError("E4M3FN holds every integer only up to 16; configs use r <= 8")
        tab = _table("int_e4m3", device)
        out = torch.empty(shape, dtype=torch.uint8, device=device)
        m = 2 * r + 1
        return _fill(out, seed, name, lambda h: tab[128 - r + (((h >> 8) * m) >> 24)])
    raise ValueError(dtype)


def dyadic_weights(shape, seed, name, *, kind: str, device="cpu") -> torch.Tensor:
    """Indexer head weights on a dyadic grid (fp32)."""
    out = torch.empty(shape, dtype=torch.float32, device=device)
    if kind == "u256":  # floor(256 u) / 256, u ~ U(0, 1)
        return _fill(out, seed, name, lambda h: (h >> 24).to(torch.float32) / 256.0)
    if kind == "n1024":  # round(1024 z) / 1024, z ~ N(0, 1)
        tab = _table("w1024", device)
        return _fill(out, seed, name, lambda h: tab[h >> 16].to(torch.float32) / 1024.0)
    raise ValueError(kind)


def block_scaled_rows(n: int, width: int, seed, name, *, dtype="bf16", spread: int = 12,
                      device="cpu") -> torch.Tensor:
    """[n, width] N(0, 1) values (bf16 or fp32) times 2^e, one e per 32 consecutive
    values of a row, e uniform on {-spread..spread}: new cache rows whose blocks
    span a range of magnitudes."""
    x = normal((n, width), seed, name, dtype=dtype, device=device)
    e = uniform_int((n, (width + 31) // 32), seed, name + ".e", -spread, spread, device=device)
    f = torch.exp2(e.to(torch.float32)).repeat_interleave(32, dim=1)[:, :width]
    return (x.float() * f).to(x.dtype)  # exact: scaling by a power of two


def uniform01(n: int, seed: int, name: str) -> List[float]:
    """n floats in [0, 1) (host-side, float64), for metadata such as lengths."""
    h = hash32(seed, name, torch.arange(n, dtype=torch.int64))
    return [(int(v) + 0.5) / 4294967296.0 for v in h.tolist()]


# --------------------------------------------------------------------------
# problem container
# --------------------------------------------------------------------------
@dataclass
class SgaCase:
    """One SGA problem: shapes, dtypes, metadata and input tensors.

    Storage forms: fp32 tensors, torch.bfloat16 tensors, and E4M3FN / E8M0
    bytes as torch.uint8. Sequences are laid out back to back in the caches:
    sequence b owns cache rows kv_start[b] .. kv_start[b] + kv_len[b] - 1, and
    query t attends to positions 0..q_pos[t] of sequence q_seq[t].
    """

    name: str
    heads: int
    d_latent: int
    d_rope: int
    idx_heads: int
    idx_dim: int
    topk: int
    softmax_scale: float
    q_dtype: str
    kv_dtype: str
    idx_dtype: str
    gate_dtype: Optional[str]
    out_dtype: str
    lens: List[int]
    q_seq: torch.Tensor
    q_pos: torch.Tensor
    kv_start: torch.Tensor
    kv_len: torch.Tensor
    q: torch.Tensor
    kv: torch.Tensor
    kv_scale: Optional[torch.Tensor]
    q_idx: torch.Tensor
    k_idx: torch.Tensor
    w: torch.Tensor
    gate: Optional[torch.Tensor]
    seed: int = 0
    extra: Dict = field(default_factory=dict)
    # paged layout: position s of sequence b is cache row
    # block_table[b, s // page_size] * page_size + s % page_size (kv_start unused)
    page_size: int = 0
    block_table: Optional[torch.Tensor] = None

    @property
    def num_seqs(self) -> int:
        return len(self.lens)

    @property
    def num_q(self) -> int:
        return int(self.q_pos.numel())

    @property
    def num_kv_rows(self) -> int:
        return int(self.kv.shape[0]) if self.page_size else int(sum(self.lens))

    @property
    def max_kv_len(self) -> int:
        return int(max(self.lens)) if self.lens else 0

    @property
    def d_qk(self) -> int:
        return self.d_latent + self.d_rope

    @property
    def device(self):
        return self.q.device

    def to(self, device) -> "SgaCase":
        def mv(x):
            return None if x is None else x.to(device)

        c = SgaCase(**{k: getattr(self, k) for k in self.__dataclass_fields__})
        for k in ("q_seq", "q_pos", "kv_start", "kv_len", "q", "kv", "kv_scale",
                  "q_idx", "k_idx", "w", "gate", "block_table"):
            setattr(c, k, mv(getattr(self, k)))
        return c


def paged_copy(case: SgaCase, page_size: int, *, seed: int = 0, spare_pages: int = 3) -> SgaCase:
    """The same logical caches laid out in pages of page_size rows.

    Every sequence takes ceil(len / page_size) pages; the pages of all
    sequences, plus `spare_pages` unused ones, are placed in a seeded random
    order (the order of hash32 values), and block_table[b, j] names the
    physical page of page j of sequence b (-1 past its last page). Rows of a
    page past the sequence's end, and spare pages, hold zeros. Only data moves
    here: the copy holds exactly the rows of `case`.
    """
    P = int(page_size)
    dev = case.kv.device
    lens = [int(n) for n in case.lens]
    npages = [(n + P - 1) // P for n in lens]
    total = sum(npages) + spare_pages
    order = torch.argsort(hash32(seed, "pages", torch.arange(total, dtype=torch.int64)))
    max_pages = max(max(npages), 1)
    table = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    src_of_dst = torch.full((total * P,), -1, dtype=torch.int64)
    starts = case.kv_start.cpu().tolist()
    g = 0
    for b, n in enumerate(lens):
        for j in range(npages[b]):
            phys = int(order[g])
            g += 1
            table[b, j] = phys
            m = min(P, n - j * P)
            src_of_dst[phys * P: phys * P + m] = torch.arange(starts[b] + j * P, starts[b] + j * P + m)
    valid = (src_of_dst >= 0).to(dev)
    src = src_of_dst.clamp(min=0).to(dev)

    def move(x):
        if x is None:
            return None
        y = x.index_select(0, src)
        y[~valid] = 0
        return y

    c = SgaCase(**{k: getattr(case, k) for k in case.__dataclass_fields__})
    c.name = f"{case.name}_paged{P}"
    c.kv, c.kv_scale, c.k_idx = move(case.kv), move(case.kv_scale), move(case.k_idx)
    c.page_size = P
    c.block_table = table.to(dev)
    return c


TINY_DIMS = dict(heads=8, d_latent=64, d_rope=16, idx_heads=2, idx_dim=32, topk=64)
FULL_DIMS = dict(heads=64, d_latent=512, d_rope=64, idx_heads=64, idx_dim=128, topk=2048)


def make_custom(
    lens: Sequence[int],
    queries: Sequence[Tuple[int, int]],
    *,
    dims: Dict[str, int],
    precision: str,
    seed: int = 0,
    device="cpu",
    name: str = "custom",
    gated: bool = True,
    out_dtype: Optional[str] = None,
    softmax_scale: Optional[float] = None,
) -> SgaCase:
    """Build a case from explicit sequence lengths and (sequence, position) queries.

    precision:
      "f32"   - every tensor fp32; indexer q/k integers on {-4..4}; w = round(1024 z)/1024
      "bf16"  - q, kv and gate bf16; indexer q/k E4M3FN integers on {-8..8}; w = floor(256 u)/256
      "mxfp8" - as "bf16" but the latent rows are E4M3FN values with one E8M0 scale per
                32 consecutive elements, the scale exponent uniform on {-4..4}
    """
    lens = [int(x) for x in lens]
    H, Dc, Dr = dims["heads"], dims["d_latent"], dims["d_rope"]
    HI, DI, k = dims["idx_heads"], dims["idx_dim"], dims["topk"]
    D = Dc + Dr
    T = len(queries)
    rows = sum(lens)
    starts = [0]
    for n in lens[:-1]:
        starts.append(starts[-1] + n)
    q_seq = torch.tensor([qs for qs, _ in queries], dtype=torch.int32, device=device)
    q_pos = torch.tensor([qp for _, qp in queries], dtype=torch.int32, device=device)
    kv_start = torch.tensor(starts, dtype=torch.int64, device=device)
    kv_len = torch.tensor(lens, dtype=torch.int32, device=device)
    tau = softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D)

    if precision == "f32":
        q = normal((T, H, D), seed, "q", dtype="f32", device=device)
        kv = normal((rows, D), seed, "kv", dtype="f32", device=device)
        kv_scale = None
        q_idx = int_values((T, HI, DI), seed, "q_idx", 4, dtype="f32", device=device)
        k_idx = int_values((rows, DI), seed, "k_idx", 4, dtype="f32", device=device)
        w = dyadic_weights((T, HI), seed, "w", kind="n1024", device=device)
        gate = normal((T, H, Dc), seed, "gate", dtype="f32", device=device) if gated else None
        q_dt, kv_dt, idx_dt, g_dt = "f32", "f32", "f32", ("f32" if gated else None)
        o_dt = out_dtype or "f32"
    elif precision in ("bf16", "mxfp8"):
        q = normal((T, H, D), seed, "q", dtype="bf16", device=device)
        if precision == "bf16":
            kv = normal((rows, D), seed, "kv", dtype="bf16", device=device)
            kv_scale = None
        else:
            if D % 32:
                raise ValueError("MXFP8 rows need a multiple of 32 elements")
            kv = normal((rows, D), seed, "kv", dtype="e4m3", device=device)
            e = uniform_int((rows, D // 32), seed, "kv_scale", -4, 4, device=device)
            kv_scale = (e + 127).to(torch.uint8)
        q_idx = int_values((T, HI, DI), seed, "q_idx", 8, dtype="fp8", device=device)
        k_idx = int_values((rows, DI), seed, "k_idx", 8, dtype="fp8", device=device)
        w = dyadic_weights((T, HI), seed, "w", kind="u256", device=device)
        gate = (normal((T, H, Dc), seed, "gate", dtype="bf16", std=math.sqrt(2.0), device=device)
                if gated else None)
        q_dt, kv_dt, idx_dt, g_dt = "bf16", precision, "fp8", ("bf16" if gated else None)
        o_dt = out_dtype or "bf16"
    else:
        raise ValueError(precision)

    return SgaCase(
        name=name, heads=H, d_latent=Dc, d_rope=Dr, idx_heads=HI, idx_dim=DI, topk=k,
        softmax_scale=tau, q_dtype=q_dt, kv_dtype=kv_dt, idx_dtype=idx_dt,
        gate_dtype=g_dt, out_dtype=o_dt, lens=lens, q_seq=q_seq, q_pos=q_pos,
        kv_start=kv_start, kv_len=kv_len, q=q, kv=kv, kv_scale=kv_scale,
        q_idx=q_idx, k_idx=k_idx, w=w, gate=gate, seed=seed,
    )


# --------------------------------------------------------------------------
# the five named workloads
# --------------------------------------------------------------------------
CONFIG_NAMES = (
    "tiny_fp32_L512",        # 1 seq x 512 tokens, all 512 as queries, 8 heads, k=64, fp32
    "decode_b32_n32k",       # 32 seqs x 32,768 cached, 1 query each, k=2048
    "decode_b16_n128k",      # 16 seqs x 131,072 cached, 1 query each, k=2048
    "prefill_q4096_n128k",   # 1 seq, 4,096 queries at positions 126,976..131,071
    "varlen_mxfp8_b64",      # 64 seqs, log-uniform lengths in [4,096, 262,144], MXFP8 latent
)
# Further workloads: several queries per sequence in decode (the verification
# step of speculative decoding: the last 4 cached positions of each sequence
# are queries, so the 4 share one scan of the sequence's index keys).
EXTRA_NAMES = (
    "decode_b16_n128k_mq4",  # 16 seqs x 131,072 cached, 4 queries each at n-4 .. n-1, k=2048
)


def varlen_lengths(seed: int, n: int = 64, lo: int = 4096, hi: int = 262144) -> List[int]:
    us = uniform01(n, seed, "varlen_lengths")
    a, b = math.log(lo), math.log(hi)
    return [min(hi, max(lo, int(math.floor(math.exp(a + u * (b - a)))))) for u in us]


def config_dims(name: str) -> Dict[str, int]:
    return dict(TINY_DIMS) if name == "tiny_fp32_L512" else dict(FULL_DIMS)


def make_case(name: str, *, seed: int = 0, device="cpu", out_dtype: Optional[str] = None) -> SgaCase:
    """One of the named workloads (CONFIG_NAMES, EXTRA_NAMES), drawn with `seed`."""
    if name == "tiny_fp32_L512":
        L = 512
        return make_custom([L], [(0, p) for p in range(L)], dims=TINY_DIMS, precision="f32",
                           seed=seed, device=device, name=name, out_dtype=out_dtype)
    if name == "decode_b32_n32k":
        B, n = 32, 32768
        return make_custom([n] * B, [(b, n - 1) for b in range(B)], dims=FULL_DIMS,
                           precision="bf16", seed=seed, device=device, name=name,
                           out_dtype=out_dtype, softmax_scale=1.0 / 24.0)
    if name == "decode_b16_n128k":
        B, n = 16, 131072
        return make_custom([n] * B, [(b, n - 1) for b in range(B)], dims=FULL_DIMS,
                           precision="bf16", seed=seed, device=device, name=name,
                           out_dtype=out_dtype, softmax_scale=1.0 / 24.0)
    if name == "decode_b16_n128k_mq4":
        B, n, Q = 16, 131072, 4
        return make_custom([n] * B, [(b, n - Q + j) for b in range(B) for j in range(Q)], dims=FULL_DIMS,
                           precision="bf16", seed=seed, device=device, name=name,
                           out_dtype=out_dtype, softmax_scale=1.0 / 24.0)
    if name == "prefill_q4096_n128k":
        n, T = 131072, 4096
        return make_custom([n], [(0, n - T + i) for i in range(T)], dims=FULL_DIMS,
                           precision="bf16", seed=seed, device=device, name=name,
                           out_dtype=out_dtype, softmax_scale=1.0 / 24.0)
    if name == "varlen_mxfp8_b64":
        lens = varlen_lengths(seed)
        return make_custom(lens, [(b, n - 1) for b, n in enumerate(lens)], dims=FULL_DIMS,
                           precision="mxfp8", seed=seed, device=device, name=name,
                           out_dtype=out_dtype, softmax_scale=1.0 / 24.0)
    raise KeyError(name)
