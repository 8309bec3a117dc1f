"""Seeded synthetic inputs for exact attention: prefill tensors and a paged KV cache.

This module is shared by the HIP path (tests, bench) and by the fp64 CPU oracle's
tests. It draws random numbers, rounds them to the storage type and lays them out
in memory; it holds none of the attention arithmetic. Everything here is NumPy.

Workloads (shapes follow the problem statement of the page "Donanıma Duyarlı
Algoritma Tasarımı: FlashAttention", section "Transformer Mimarisi ve
Self-Attention Mekanizması": Q, K and V are (sequence length x dimension) per
head; the KV-cache and GQA structure follows the glossary entry "KV Cache
(Anahtar-Değer Önbelleği)" on the yapayzekasozluk.tr "Attention" tag page):

  fp32_single   B=1 H=1  Hkv=1 N=128    d=64  non-causal fp32, N(0,1)
  bf16_causal   B=2 H=8  Hkv=8 N=1024   d=64  causal bf16, N(0,1) x 0.5
  gqa_causal    B=4 H=32 Hkv=8 N=4096   d=128 causal bf16, N(0,1)
  paged_decode  64 sequences x 1 query, H=32 Hkv=8 d=128, KV length ~ U{512..8192},
                pages of 16 tokens, seeded random permutation page table
  long_causal   B=1 H=8  Hkv=8 N=131072 d=128 causal bf16, N(0,1) x 0.5
  window_long   B=1 H=32 Hkv=8 N=32768  d=128 bf16, N(0,1), sliding window (4096, 0)

The backward pass's output gradient dO is drawn from its own generator (make_dout).

Draw order for a prefill workload (one ``numpy.random.default_rng(seed)``):
Q, K, V, each ``standard_normal(dtype=float32)`` in [B, H(kv), N, d] order, then
multiplied by ``value_scale`` (exact: a power of two), then rounded to bf16 with
round-to-nearest-even. Row samples (for the large workloads) are drawn afterwards
from the same generator.

Draw order for the paged decode workload: sequence lengths, then the physical page
permutation, then Q, then K_s and V_s for s = 0..num_seqs-1.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

BF16_NAN_BITS = np.uint16(0x7FC0)


# ----------------------------------------------------------------------------------
# bf16 storage helpers (bit patterns held in uint16 arrays)
# ----------------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest, ties to even.

    Returns the 16-bit patterns as uint16. NaN inputs are not expected (the
    generators draw finite normals); they are mapped to the canonical quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN_BITS
    return out


def bf16_bits_to_f32(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 exactly (bf16 is the top half of fp32)."""
    u = np.ascontiguousarray(u, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(u: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float64 exactly."""
    return bf16_bits_to_f32(u).astype(np.float64)


# ----------------------------------------------------------------------------------
# fp8 storage (OCP e4m3: sign, 4 exponent bits with bias 7, 3 mantissa bits; no
# infinities; 0x7f and 0xff are NaN; largest finite magnitude 448)
# ----------------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_to_f64(u: np.ndarray) -> np.ndarray:
    """Decode e4m3 bytes to float64 exactly, from the format's definition."""
    u = np.asarray(u, dtype=np.uint8).astype(np.int64)
    sign = np.where(u & 0x80, -1.0, 1.0)
    e = (u >> 3) & 0xF
    m = (u & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    val = sign * val
    return np.where((e == 15) & ((u & 7) == 7), np.nan, val)


_E4M3_FINITE = np.array([b for b in range(128) if b != 0x7F], dtype=np.uint8)


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value, ties to the even code, saturating at +-448 (finite
    inputs only). Nearest is found among the 127 non-negative finite codes by search."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3 encoding expects finite values")
    mags = e4m3_to_f64(_E4M3_FINITE)            # increasing with the code
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, len(mags) - 1)
    lo = np.clip(hi - 1, 0, len(mags) - 1)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_E4M3_FINITE[hi] % 2 == 0))
    code = np.where(pick_hi, _E4M3_FINITE[hi], _E4M3_FINITE[lo]).astype(np.uint8)
    return np.where((x < 0) & (code != 0), code | 0x80, code).astype(np.uint8)


# ----------------------------------------------------------------------------------
# Prefill workloads
# ----------------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    dtype: str            # "f32" or "bf16"
    value_scale: float    # N(0,1) draws are multiplied by this before rounding
    scale: float          # softmax scale applied to Q.K^T
    seed: int

    @property
    def flops(self) -> float:
        """Algorithmic flops: 4*d per unmasked (query, key) pair (Q.K^T and P.V)."""
        return 4.0 * self.d * self.B * self.H * unmasked_pairs(self.Nq, self.Nk, self.causal)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    num_seqs: int
    H: int
    Hkv: int
    d: int
    len_lo: int
    len_hi: int           # inclusive
    page_size: int
    max_seq_len: int
    scale: float
    seed: int


def unmasked_pairs(Nq: int, Nk: int, causal: bool) -> int:
    """Number of (query, key) pairs that attend, per (batch, head).

    Causal uses bottom-right alignment: query i sits at absolute position Nk-Nq+i.
    """
    if not causal:
        return Nq * Nk
    off = Nk - Nq
    # sum_{i=0}^{Nq-1} (i + off + 1)
    return Nq * (off + 1) + Nq * (Nq - 1) // 2


def window_pairs(Nq: int, Nk: int, left: int, right: int) -> int:
    """(query, key) pairs inside a sliding window, per (batch, head): query i at
    position p = Nk - Nq + i counts keys max(0, p - left) .. min(Nk - 1, p + right);
    -1 leaves a side unbounded."""
    total = 0
    for i in range(Nq):
        p = Nk - Nq + i
        lo = 0 if left < 0 else max(0, p - left)
        hi = Nk - 1 if right < 0 else min(Nk - 1, p + right)
        total += max(0, hi - lo + 1)
    return total


PREFILL_CONFIGS = {
    "fp32_single": PrefillConfig("fp32_single", 1, 1, 1, 128, 128, 64, False, "f32",
                                 1.0, 1.0 / math.sqrt(64), 1),
    "bf16_causal": PrefillConfig("bf16_causal", 2, 8, 8, 1024, 1024, 64, True, "bf16",
                                 0.5, 1.0 / math.sqrt(64), 2),
    "gqa_causal": PrefillConfig("gqa_causal", 4, 32, 8, 4096, 4096, 128, True, "bf16",
                                1.0, 1.0 / math.sqrt(128), 3),
    "long_causal": PrefillConfig("long_causal", 1, 8, 8, 131072, 131072, 128, True, "bf16",
                                 0.5, 1.0 / math.sqrt(128), 5),
}

# The sliding-window workload: B1 H32 Hkv8 N32768 d128 with a causal window of 4096 keys
# (each query attends its own position and the 4096 before it).
WINDOW_CONFIG = PrefillConfig("window_long", 1, 32, 8, 32768, 32768, 128, False, "bf16",
                              1.0, 1.0 / math.sqrt(128), 6)
WINDOW = (4096, 0)

DECODE_CONFIGS = {
    "paged_decode": DecodeConfig("paged_decode", 64, 32, 8, 128, 512, 8192, 16, 8192,
                                 1.0 / math.sqrt(128), 4),
}


@dataclasses.dataclass
class PrefillInputs:
    cfg: PrefillConfig
    q: np.ndarray   # [B,H,Nq,d]   float32 (f32) or uint16 bf16 bits
    k: np.ndarray   # [B,Hkv,Nk,d]
    v: np.ndarray   # [B,Hkv,Nk,d]
    rng: np.random.Generator  # positioned after V, for row samples

    def as_f64(self):
        """The stored values widened exactly to float64 (what the oracle consumes)."""
        if self.cfg.dtype == "f32":
            return (self.q.astype(np.float64), self.k.astype(np.float64),
                    self.v.astype(np.float64))
        return bf16_bits_to_f64(self.q), bf16_bits_to_f64(self.k), bf16_bits_to_f64(self.v)


def _draw(rng: np.random.Generator, shape, value_scale: float, dtype: str) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if value_scale != 1.0:
        x *= np.float32(value_scale)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_prefill(cfg: PrefillConfig, seed: int | None = None) -> PrefillInputs:
    """Draw Q, K, V for a prefill workload (see the module docstring for the order)."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = _draw(rng, (cfg.B, cfg.H, cfg.Nq, cfg.d), cfg.value_scale, cfg.dtype)
    k = _draw(rng, (cfg.B, cfg.Hkv, cfg.Nk, cfg.d), cfg.value_scale, cfg.dtype)
    v = _draw(rng, (cfg.B, cfg.Hkv, cfg.Nk, cfg.d), cfg.value_scale, cfg.dtype)
    return PrefillInputs(cfg, q, k, v, rng)


def custom_prefill(B, H, Hkv, Nq, Nk, d, causal, dtype="bf16", value_scale=1.0,
                   scale=None, seed=0, name="custom") -> PrefillInputs:
    """Any shape, same recipe (used for ragged tails and edge cases)."""
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cfg = PrefillConfig(name, B, H, Hkv, Nq, Nk, d, causal, dtype, value_scale, scale, seed)
    return make_prefill(cfg)


def make_dout(cfg: PrefillConfig, seed: int) -> np.ndarray:
    """Output gradient dO [B,H,Nq,d] for the backward pass: N(0,1) float32 draws from
    default_rng(seed), rounded to bf16 (bits)."""
    rng = np.random.default_rng(seed)
    return f32_to_bf16_bits(rng.standard_normal((cfg.B, cfg.H, cfg.Nq, cfg.d),
                                                dtype=np.float32))


def sample_rows(inp: PrefillInputs, n_full_pairs: int, n_random_rows: int):
    """Seeded row selection for workloads too large to check in full.

    Returns a dict {(b, h): sorted int64 array of query rows}. ``n_full_pairs``
    (b, h) pairs are checked on every row; ``n_random_rows`` further rows are drawn
    uniformly without replacement from the remaining (b, h, i) triples.
    """
    cfg = inp.cfg
    rng = inp.rng
    BH = cfg.B * cfg.H
    full = rng.choice(BH, size=min(n_full_pairs, BH), replace=False)
    sel: dict[tuple[int, int], np.ndarray] = {}
    for p in sorted(int(x) for x in full):
        sel[(p // cfg.H, p % cfg.H)] = np.arange(cfg.Nq, dtype=np.int64)
    if n_random_rows:
        rest = np.setdiff1d(np.arange(BH), full)
        if rest.size:
            total = rest.size * cfg.Nq
            flat = rng.choice(total, size=min(n_random_rows, total), replace=False)
            pair = rest[flat // cfg.Nq]
            row = flat % cfg.Nq
            for p in np.unique(pair):
                rows = np.sort(row[pair == p]).astype(np.int64)
                sel[(int(p) // cfg.H, int(p) % cfg.H)] = rows
    return sel


def sample_rows_per_head(inp: PrefillInputs, rows_per_head: int):
    """``rows_per_head`` seeded random query rows for every (b, h)."""
    cfg = inp.cfg
    sel = {}
    for b in range(cfg.B):
        for h in range(cfg.H):
            rows = inp.rng.choice(cfg.Nq, size=min(rows_per_head, cfg.Nq), replace=False)
            sel[(b, h)] = np.sort(rows).astype(np.int64)
    return sel


# ----------------------------------------------------------------------------------
# Paged KV-cache decode workload
# ----------------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeInputs:
    cfg: DecodeConfig
    seq_lens: np.ndarray      # [S] int32, each sequence's cached length (current token included)
    q: np.ndarray             # [S,H,d] uint16 bf16 bits
    k_seq: list               # per sequence [L_s,Hkv,d] uint16 (contiguous, before paging)
    v_seq: list
    k_cache: np.ndarray       # [num_pages,page_size,Hkv,d] uint16
    v_cache: np.ndarray
    page_table: np.ndarray    # [S,max_pages_per_seq] int32
    num_pages: int

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    def kv_bytes(self) -> int:
        """K and V bytes the sequences own (the decode step must read all of them)."""
        return int(self.seq_lens.astype(np.int64).sum()) * self.cfg.Hkv * self.cfg.d * 2 * 2


def make_decode(cfg: DecodeConfig, seed: int | None = None, *, seq_lens=None,
                unused_fill: str = "zero", table_pad: int = 0) -> DecodeInputs:
    """Draw a paged KV cache.

    Physical pages are a seeded permutation of 0..P_total-1 (P_total = sum of
    ceil(L_s / page_size)), handed to the sequences in order. Slots of a page past a
    sequence's length hold 0 (``unused_fill="zero"``) or bf16 NaN (``"nan"``); table
    entries past a sequence's last page hold ``table_pad``.
    ``seq_lens`` overrides the length draw (zero-length sequences are allowed).
    """
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    S, P = cfg.num_seqs, cfg.page_size
    if seq_lens is None:
        lens = rng.integers(cfg.len_lo, cfg.len_hi, size=S, endpoint=True).astype(np.int32)
    else:
        lens = np.asarray(seq_lens, dtype=np.int32)
        assert lens.shape == (S,)
    n_pages = (lens.astype(np.int64) + P - 1) // P
    total = int(n_pages.sum())
    perm = rng.permutation(total).astype(np.int32)
    max_pages = max(1, (cfg.max_seq_len + P - 1) // P)
    assert int(lens.max(initial=0)) <= cfg.max_seq_len
    table = np.full((S, max_pages), table_pad, dtype=np.int32)
    off = 0
    for s in range(S):
        table[s, :n_pages[s]] = perm[off:off + n_pages[s]]
        off += int(n_pages[s])

    q = _draw(rng, (S, cfg.H, cfg.d), 1.0, "bf16")
    fill = BF16_NAN_BITS if unused_fill == "nan" else np.uint16(0)
    npool = max(total, 1)
    k_cache = np.full((npool, P, cfg.Hkv, cfg.d), fill, dtype=np.uint16)
    v_cache = np.full((npool, P, cfg.Hkv, cfg.d), fill, dtype=np.uint16)
    k_seq, v_seq = [], []
    for s in range(S):
        L = int(lens[s])
        ks = _draw(rng, (L, cfg.Hkv, cfg.d), 1.0, "bf16")
        vs = _draw(rng, (L, cfg.Hkv, cfg.d), 1.0, "bf16")
        t = np.arange(L)
        pages = table[s, t // P]
        k_cache[pages, t % P] = ks
        v_cache[pages, t % P] = vs
        k_seq.append(ks)
        v_seq.append(vs)
    return DecodeInputs(cfg, lens, q, k_seq, v_seq, k_cache, v_cache, table, npool)


def custom_decode(num_seqs, H, Hkv, d, len_lo, len_hi, page_size=16, max_seq_len=None,
                  scale=None, seed=0, **kw) -> DecodeInputs:
    if max_seq_len is None:
        max_seq_len = max(len_hi, 1)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    cfg = DecodeConfig("custom_decode", num_seqs, H, Hkv, d, len_lo, len_hi, page_size,
                       max_seq_len, scale, seed)
    return make_decode(cfg, **kw)


# ----------------------------------------------------------------------------------
# Chunked prefill through the page table, and KV append
# ----------------------------------------------------------------------------------
@dataclasses.dataclass
class ChunkedPrefillInputs:
    cache: DecodeInputs   # the paged cache; seq_lens include the Nq new tokens
    q: np.ndarray         # [B,H,Nq,d] uint16 bf16 bits: queries of each sequence's last Nq tokens
    Nq: int


def custom_chunked_prefill(B, H, Hkv, d, Nq, len_lo, len_hi, *, seq_lens=None,
                           max_seq_len=None, scale=None, seed=0, **kw) -> ChunkedPrefillInputs:
    """A paged cache of B sequences (lengths U{len_lo..len_hi}, each >= Nq, or
    ``seq_lens``) plus queries for the last Nq tokens of each sequence."""
    assert len_lo >= Nq or seq_lens is not None
    if max_seq_len is None:
        max_seq_len = max(len_hi, int(max(seq_lens)) if seq_lens is not None else 1)
    cache = custom_decode(B, H, Hkv, d, len_lo, len_hi, max_seq_len=max_seq_len, scale=scale,
                          seed=seed, seq_lens=seq_lens, **kw)
    rng = np.random.default_rng(seed + 7919)
    q = _draw(rng, (B, H, Nq, d), 1.0, "bf16")
    return ChunkedPrefillInputs(cache, q, Nq)


@dataclasses.dataclass
class AppendInputs:
    k_cache: np.ndarray    # [num_pages,16,Hkv,d] uint16, random "old" contents
    v_cache: np.ndarray
    page_table: np.ndarray  # [S,max_pages] int32: disjoint pages; unassigned entries -1
    start_pos: np.ndarray   # [S] int32
    k_new: np.ndarray      # [S,n_new,Hkv,d] uint16
    v_new: np.ndarray


def make_append(S, n_new, Hkv, d, max_seq_len, *, page_size=16, seed=0, start_pos=None,
                spare_pages=3) -> AppendInputs:
    """Seeded KV-append workload: sequence s already holds start_pos[s] tokens (drawn
    in [0, max_seq_len - n_new] unless given) and gets n_new more. Its pages up to
    the last new token are assigned (a seeded permutation of the pool, which has
    ``spare_pages`` pages nobody owns); later table entries hold -1."""
    rng = np.random.default_rng(seed)
    P = page_size
    max_pages = (max_seq_len + P - 1) // P
    if start_pos is None:
        start_pos = rng.integers(0, max(max_seq_len - n_new, 0), size=S, endpoint=True)
    start_pos = np.asarray(start_pos, dtype=np.int32)
    need = np.clip((start_pos.astype(np.int64) + n_new + P - 1) // P, 0, max_pages)
    total = int(need.sum()) + spare_pages
    perm = rng.permutation(total).astype(np.int32)
    table = np.full((S, max_pages), -1, dtype=np.int32)
    off = 0
    for s in range(S):
        table[s, :need[s]] = perm[off:off + need[s]]
        off += int(need[s])
    k_cache = rng.integers(0, 1 << 16, size=(total, P, Hkv, d), dtype=np.uint16)
    v_cache = rng.integers(0, 1 << 16, size=(total, P, Hkv, d), dtype=np.uint16)
    k_new = _draw(rng, (S, n_new, Hkv, d), 1.0, "bf16")
    v_new = _draw(rng, (S, n_new, Hkv, d), 1.0, "bf16")
    return AppendInputs(k_cache, v_cache, table, start_pos, k_new, v_new)


@dataclasses.dataclass
class DecodeFp8Inputs:
    base: DecodeInputs       # the bf16 workload the fp8 cache was quantised from
    k_cache: np.ndarray      # [num_pages,16,Hkv,d] uint8 e4m3
    v_cache: np.ndarray
    k_scale: np.ndarray      # [Hkv] float32
    v_scale: np.ndarray
    k_seq: list              # per sequence [L_s,Hkv,d] uint8, quantised before paging
    v_seq: list


def quantize_decode_fp8(base: DecodeInputs, seqs: bool = True) -> DecodeFp8Inputs:
    """Per KV head: scale = max |value| over every cached token / 448, bytes = e4m3(value /
    scale). Slots past a sequence keep their fill (0 stays 0; NaN fill becomes 0x7f).
    seqs=False leaves the per-sequence copies (only a checker needs them) empty."""
    Hkv = base.cfg.Hkv

    def quant(cache, seqs):
        amax = np.zeros(Hkv)
        for x in seqs:
            if x.shape[0]:
                amax = np.maximum(amax, np.abs(bf16_bits_to_f64(x)).max(axis=(0, 2)))
        sc = np.where(amax > 0, amax / E4M3_MAX, 1.0).astype(np.float32)
        div = sc[None, None, :, None].astype(np.float64)
        q = np.empty(cache.shape, dtype=np.uint8)
        for p0 in range(0, cache.shape[0], 2048):  # in pieces: the full cache in f64 is GBs
            vals = bf16_bits_to_f64(cache[p0:p0 + 2048])
            fin = np.isfinite(vals)
            part = f64_to_e4m3(np.where(fin, vals / div, 0.0))
            q[p0:p0 + 2048] = np.where(fin, part, np.uint8(0x7F))
        return q, sc

    kq, ks = quant(base.k_cache, base.k_seq)
    vq, vs = quant(base.v_cache, base.v_seq)

    def quant_seq(x, sc):
        return f64_to_e4m3(bf16_bits_to_f64(x) / sc[None, :, None].astype(np.float64))

    if not seqs:
        return DecodeFp8Inputs(base, kq, vq, ks, vs, [], [])
    return DecodeFp8Inputs(base, kq, vq, ks, vs, [quant_seq(x, ks) for x in base.k_seq],
                           [quant_seq(x, vs) for x in base.v_seq])
