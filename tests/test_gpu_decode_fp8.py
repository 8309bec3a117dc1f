"""GPU parity of paged decode on an fp8 (e4m3) KV cache (fa_decode_paged_fp8).

The oracle attends the dequantised values (byte value x per-head scale) of each
sequence's K/V, quantised from the contiguous sequence before it was paged, so the
kernel's page walk and byte conversion are both checked against an independent path.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import bf16_from_dev, bf16_to_dev, check_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_fp8(f: inputs.DecodeFp8Inputs):
    import torch
    b = f.base
    c = b.cfg
    q = bf16_to_dev(b.q)
    kc = torch.from_numpy(f.k_cache).cuda()
    vc = torch.from_numpy(f.v_cache).cuda()
    ks = torch.from_numpy(f.k_scale).cuda()
    vs = torch.from_numpy(f.v_scale).cuda()
    pt = torch.from_numpy(b.page_table).cuda()
    sl = torch.from_numpy(b.seq_lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((c.num_seqs, c.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(_lib.fa_decode_paged_workspace_size(c.num_seqs, c.H, c.d, c.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    _lib.fa_decode_paged_fp8(q, kc, vc, ks, vs, pt, sl, o, lse, max_seq_len=c.max_seq_len,
                             scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    return bf16_from_dev(o), lse.cpu().numpy()


def oracle_fp8(f: inputs.DecodeFp8Inputs):
    b = f.base
    ks = [inputs.e4m3_to_f64(x) * f.k_scale[None, :, None] for x in f.k_seq]
    vs = [inputs.e4m3_to_f64(x) * f.v_scale[None, :, None] for x in f.v_seq]
    return oracle.decode(inputs.bf16_bits_to_f64(b.q), ks, vs, scale=b.cfg.scale)


def _check(f, what):
    c = f.base.cfg
    _say(f"[decode fp8] {what}: S{c.num_seqs} H{c.H} Hkv{c.Hkv} d{c.d}")
    o_h, lse_h = run_fp8(f)
    O, L = oracle_fp8(f)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, what)
    return o_h, lse_h


def test_fp8_paged_decode_full():
    """64 sequences, H32/Hkv8, d128, lengths U{512..8192}, all rows."""
    base = inputs.make_decode(inputs.DECODE_CONFIGS["paged_decode"])
    _check(inputs.quantize_decode_fp8(base), "fp8 paged_decode")


@pytest.mark.parametrize("S,H,Hkv,d,lo,hi", [
    (5, 8, 8, 128, 1, 40),
    (3, 32, 4, 128, 100, 3000),
    (4, 16, 1, 128, 2000, 2100),
    (2, 64, 2, 128, 10, 300),
    (9, 32, 8, 64, 1, 1500),
], ids=lambda x: str(x))
def test_fp8_decode_shapes(S, H, Hkv, d, lo, hi):
    base = inputs.custom_decode(S, H, Hkv, d, lo, hi, seed=7 * S + H + d)
    _check(inputs.quantize_decode_fp8(base), f"fp8 S{S} H{H} Hkv{Hkv} d{d}")


def test_fp8_decode_wide_groups_full():
    """64 sequences, lengths U{512..8192}, H32 Hkv2 (16 query heads per KV head, the
    one-KV-head matrix-unit kernel on an e4m3 cache), all rows."""
    base = inputs.custom_decode(64, 32, 2, 128, 512, 8192, seed=16)
    _check(inputs.quantize_decode_fp8(base), "fp8 64 seqs H32 Hkv2")


def test_fp8_decode_long_ranges():
    """Work-group ranges of 248 pages (62 per wave) on an e4m3 cache, d = 64 (one 1 KiB
    direct load per page); one sequence spans 34 ranges."""
    cfg = inputs.DecodeConfig("long", 3, 4, 1, 64, 0, 0, 16, 131072, 1 / 8, 6)
    base = inputs.make_decode(cfg, seq_lens=[131072, 4000, 70001])
    _check(inputs.quantize_decode_fp8(base), "fp8 long ranges")


def test_fp8_decode_many_sequences():
    """150 sequences on an e4m3 cache (the planning kernel's path), some empty."""
    rng = np.random.default_rng(44)
    lens = rng.integers(0, 700, 150)
    lens[rng.integers(0, 150, 4)] = 0
    cfg = inputs.DecodeConfig("many", 150, 8, 2, 128, 0, 0, 16, 1024, 1 / math.sqrt(128), 44)
    base = inputs.make_decode(cfg, seq_lens=[int(x) for x in lens])
    o_h, lse_h = _check(inputs.quantize_decode_fp8(base), "fp8 many sequences")
    for s in np.nonzero(lens == 0)[0]:
        assert np.all(inputs.bf16_bits_to_f32(o_h[s]) == 0.0) and np.all(lse_h[s] == -np.inf)


@pytest.mark.parametrize("S,H,Hkv", [(40, 8, 4), (40, 12, 6), (36, 8, 8), (33, 4, 4)])
def test_fp8_decode_grouped_kv_heads_with_padding_columns(S, H, Hkv):
    """KV heads read in pairs with padding columns (32 sequences or more, an even KV head
    count, g <= 4): H8 Hkv4 and H12 Hkv6 (g = 2: two padding columns per head), H8 Hkv8
    and H4 Hkv4 (g = 1: three per head)."""
    base = inputs.custom_decode(S, H, Hkv, 128, 1, 900, seed=48 + Hkv)
    _check(inputs.quantize_decode_fp8(base), f"fp8 S{S} H{H} Hkv{Hkv}")


@pytest.mark.parametrize("S,H,Hkv", [(8, 8, 2), (40, 8, 2), (40, 16, 4), (40, 32, 4),
                                     (40, 32, 2)])
def test_fp8_edge_lengths_and_nan_slots(S, H, Hkv):
    """Empty sequence, page boundaries; unused slots hold e4m3 NaN bytes and the table is
    padded with -1: the output must equal the zero-filled cache's bit for bit. 8 sequences
    take the one-KV-head kernel with P.V on the matrix unit; 40 with H8 Hkv2 and H16 Hkv4
    (g = 4) the kernel that reads two KV heads' rows as one; 40 with H32 Hkv4 and H32 Hkv2
    (g = 8, 16) the one-KV-head matrix-unit kernel, whose V rows past the sequence are
    zeroed when they are written into the bf16 stage."""
    cfg = inputs.DecodeConfig("edges", S, H, Hkv, 128, 0, 0, 16, 600, 1 / math.sqrt(128), 3)
    lens = ([0, 1, 15, 16, 17, 64, 65, 600] * (S // 8))[:S]
    a = inputs.quantize_decode_fp8(inputs.make_decode(cfg, seq_lens=lens))
    b = inputs.quantize_decode_fp8(inputs.make_decode(cfg, seq_lens=lens, unused_fill="nan",
                                                      table_pad=-1))
    assert np.array_equal(a.k_scale, b.k_scale)
    oa, la = _check(a, "fp8 edges")
    ob, lb = run_fp8(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert np.all(inputs.bf16_bits_to_f32(oa[0]) == 0.0) and np.all(la[0] == -np.inf)
