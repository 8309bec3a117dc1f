"""GPU parity of paged-KV decode (fa_decode_paged) against the fp64 oracle.

The oracle reads each sequence's contiguous K/V as drawn before they were scattered
into pages, so the GPU's page-table indexing is checked independently of the
oracle; a peaked-query test makes indexing errors bit-visible.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import inputs
from gpu_helpers import DecodeDev, check_bf16, run_decode

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle(inp):
    c = inp.cfg
    ks = [inputs.bf16_bits_to_f64(x) for x in inp.k_seq]
    vs = [inputs.bf16_bits_to_f64(x) for x in inp.v_seq]
    return oracle.decode(inputs.bf16_bits_to_f64(inp.q), ks, vs, scale=c.scale)


def _check(inp, what):
    c = inp.cfg
    _say(f"[decode] {what}: S{c.num_seqs} H{c.H} Hkv{c.Hkv} d{c.d} lens "
         f"{int(inp.seq_lens.min())}..{int(inp.seq_lens.max())} max_seq_len {c.max_seq_len}")
    o_h, lse_h = run_decode(inp)
    O, L = _oracle(inp)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, what)
    return o_h, lse_h


def test_paged_decode_full():
    """64 sequences, H32/Hkv8, d128, lengths U{512..8192}, 16-token pages, all rows."""
    _check(inputs.make_decode(inputs.DECODE_CONFIGS["paged_decode"]), "paged_decode")


@pytest.mark.parametrize("S,H,Hkv,d,lo,hi", [
    (5, 8, 8, 128, 1, 40),        # g = 1
    (7, 16, 8, 128, 1, 700),      # g = 2
    (3, 32, 4, 128, 100, 3000),   # g = 8
    (4, 16, 1, 128, 2000, 2100),  # g = 16 (MQA)
    (2, 64, 2, 128, 10, 300),     # g = 32: two head groups per KV head
    (6, 12, 4, 128, 1, 100),      # g = 3 (padding columns)
    (9, 32, 8, 64, 1, 1500),      # d = 64
    (3, 8, 2, 64, 16, 16),        # exactly one page
], ids=lambda x: str(x))
def test_decode_shapes(S, H, Hkv, d, lo, hi):
    inp = inputs.custom_decode(S, H, Hkv, d, lo, hi, seed=S * 100 + H + d)
    _check(inp, f"decode S{S} H{H} Hkv{Hkv} d{d}")


def test_decode_long_ranges():
    """max_seq_len 131072 makes every work-group's range 248 pages (62 per wave: a wave's
    page ids fill lanes 0-61 and the two pages it prefetches past its last one lanes
    62-63); the long sequence spans 34 ranges, the others begin and end inside ranges."""
    from kv_cache_fa_amd import _lib
    assert _lib.fa_decode_paged_split_tokens(3, 131072, 16) == 248 * 16
    cfg = inputs.DecodeConfig("long", 3, 4, 1, 64, 0, 0, 16, 131072, 1 / 8, 5)
    inp = inputs.make_decode(cfg, seq_lens=[131072, 4000, 70001])
    _check(inp, "decode long ranges")


def test_decode_edge_lengths():
    """Empty sequence, one token, page boundaries (15, 16, 17), split boundaries."""
    cfg = inputs.DecodeConfig("edges", 10, 8, 2, 128, 0, 0, 16, 1100, 1 / math.sqrt(128), 3)
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 1024, 1100]
    inp = inputs.make_decode(cfg, seq_lens=lens)
    o_h, lse_h = _check(inp, "edge lengths")
    assert np.all(inputs.bf16_bits_to_f32(o_h[0]) == 0.0)
    assert np.all(lse_h[0] == -np.inf)


@pytest.mark.parametrize("S,H,Hkv,d,hi,max_seq_len,seed", [
    (130, 8, 2, 64, 300, 512, 41),        # sequences read in three chunks of 64
    (200, 4, 1, 128, 40, 131072, 42),     # 248-page ranges, each spanning many sequences
    (97, 16, 4, 128, 2000, 4096, 43),     # a chunk boundary inside a range
    (1500, 4, 1, 64, 40, 64, 45),         # the planning kernel's 1024-length passes, twice
    (48, 8, 8, 128, 600, 1024, 46),       # KV head pairs with g = 1 (3 padding columns each)
    (40, 16, 8, 64, 500, 1024, 47),       # pairs, g = 2, d = 64
    (100, 32, 2, 128, 600, 1024, 48),     # g = 16, P.V on the matrix unit, planned ranges
    (70, 16, 2, 64, 900, 1024, 49),       # g = 8, d = 64, matrix-unit P.V
], ids=lambda x: str(x))
def test_decode_many_sequences(S, H, Hkv, d, hi, max_seq_len, seed):
    """More than 64 sequences (the in-kernel page count and prefix sums run over chunks of
    64 lengths), some of them empty, and ranges cut into many sequence pieces."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(0, hi + 1, S)
    lens[rng.integers(0, S, 3)] = 0
    cfg = inputs.DecodeConfig("many", S, H, Hkv, d, 0, 0, 16, max_seq_len, 1 / math.sqrt(d), seed)
    inp = inputs.make_decode(cfg, seq_lens=[int(x) for x in lens])
    o_h, lse_h = _check(inp, f"many sequences S{S}")
    for s in np.nonzero(lens == 0)[0]:
        assert np.all(inputs.bf16_bits_to_f32(o_h[s]) == 0.0) and np.all(lse_h[s] == -np.inf)


@pytest.mark.parametrize("S,H,Hkv", [(12, 16, 4), (40, 16, 4), (40, 32, 2), (50, 12, 3)])
def test_unused_slots_and_table_padding_are_never_read(S, H, Hkv):
    """Slots past a sequence's length hold NaN and unused table entries hold -1: the
    output must be bit-identical to the zero-filled cache's. 12 sequences: one KV head per
    work-group, P.V on the matrix unit (V rows past the sequence must arrive as zeros, since
    0 x NaN is NaN); 40 with H16 Hkv4: KV heads read in pairs (FMA P.V); 40 with H32 Hkv2:
    16 heads per KV head on the matrix unit; 50 with H12 Hkv3: one KV head, FMA P.V."""
    cfg = inputs.DecodeConfig("nan", S, H, Hkv, 128, 1, 900, 16, 1024, 1 / math.sqrt(128), 11)
    a = inputs.make_decode(cfg)
    b = inputs.make_decode(cfg, unused_fill="nan", table_pad=-1)
    assert np.array_equal(a.seq_lens, b.seq_lens)
    oa, la = run_decode(a)
    ob, lb = run_decode(b)
    assert np.all(np.isfinite(inputs.bf16_bits_to_f32(ob)))
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    O, L = _oracle(b)
    check_bf16(inputs.bf16_bits_to_f64(ob), lb, O, L, "nan-filled cache")


@pytest.mark.parametrize("S,H,Hkv", [(16, 32, 8), (40, 32, 8), (40, 32, 4)])
def test_peaked_query_selects_cached_value_bit_exactly(S, H, Hkv):
    """q[s,h] = 64 * K_s[t*] for a seeded target token t* per (sequence, head): every
    other exponential underflows to exactly 0, so O[s,h] must equal the stored
    V_s[t*] bit for bit. A wrong page, slot or head index cannot pass."""
    cfg = inputs.DecodeConfig("peak", S, H, Hkv, 128, 1, 3000, 16, 3000, 1 / math.sqrt(128), 17)
    inp = inputs.make_decode(cfg)
    rng = np.random.default_rng(99)
    g = cfg.H // cfg.Hkv
    tgt = np.zeros((cfg.num_seqs, cfg.H), dtype=np.int64)
    q = np.empty_like(inp.q)
    for s in range(cfg.num_seqs):
        for h in range(cfg.H):
            t = int(rng.integers(0, inp.seq_lens[s]))
            tgt[s, h] = t
            kk = inputs.bf16_bits_to_f32(inp.k_seq[s][t, h // g])
            q[s, h] = inputs.f32_to_bf16_bits(kk * np.float32(64.0))
    inp.q = q
    _say("[decode] peaked query")
    o_h, _ = run_decode(inp)
    n_exact = 0
    for s in range(cfg.num_seqs):
        kf = inputs.bf16_bits_to_f64(inp.k_seq[s])
        for h in range(cfg.H):
            sc = kf[:, h // g] @ inputs.bf16_bits_to_f64(q[s, h]) * cfg.scale * math.log2(math.e)
            t = tgt[s, h]
            others = np.delete(sc, t)
            if others.size and sc[t] - others.max() <= 160.0:
                continue
            assert np.array_equal(o_h[s, h], inp.v_seq[s][t, h // g]), (s, h, t)
            n_exact += 1
    assert n_exact > 0.9 * cfg.num_seqs * cfg.H


def test_decode_is_bitwise_deterministic():
    inp = inputs.custom_decode(8, 32, 8, 128, 100, 5000, seed=4)
    dd = DecodeDev(inp)
    dd.run()
    a = dd.result()
    dd.run()
    b = dd.result()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
