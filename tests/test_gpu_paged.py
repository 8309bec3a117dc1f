"""GPU parity of the KV-cache flow around decode: KV append (fa_kv_append, bit-exact
against the oracle's scatter) and chunked prefill through the page table
(fa_fwd_paged, against the fp64 oracle on the sequences' contiguous K/V, and
bit-identical to the contiguous kernel fa_fwd on the same values).

The oracle reads each sequence's K/V as drawn before it was scattered into pages,
so the kernel's page-table indexing is checked independently of the oracle.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import bf16_from_dev, bf16_to_dev, check_bf16, run_decode

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _torch():
    import torch
    return torch


def _contig(seq_kv):
    """[L, Hkv, d] uint16 -> [1, Hkv, L, d] float64 (the oracle's layout)."""
    return inputs.bf16_bits_to_f64(seq_kv).transpose(1, 0, 2)[None]


def run_paged(ci: inputs.ChunkedPrefillInputs, causal=True, kc=None, vc=None, pt=None):
    torch = _torch()
    c = ci.cache
    q = bf16_to_dev(ci.q)
    kc = bf16_to_dev(c.k_cache) if kc is None else kc
    vc = bf16_to_dev(c.v_cache) if vc is None else vc
    pt = torch.from_numpy(c.page_table).cuda() if pt is None else pt
    sl = torch.from_numpy(c.seq_lens).cuda()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    _lib.fa_fwd_paged(q, kc, vc, pt, sl, o, lse, max_seq_len=c.cfg.max_seq_len, causal=causal,
                      scale=c.cfg.scale)
    torch.cuda.synchronize()
    return bf16_from_dev(o), lse.cpu().numpy()


def oracle_paged(ci: inputs.ChunkedPrefillInputs, causal=True, rows=None):
    """Per sequence: the last Nq positions' queries against all its keys."""
    c = ci.cache
    q = inputs.bf16_bits_to_f64(ci.q)
    O = np.zeros(q.shape)
    L = np.zeros(q.shape[:3])
    for b in range(q.shape[0]):
        k, v = _contig(c.k_seq[b]), _contig(c.v_seq[b])
        Ob, Lb = oracle.attention(q[b:b + 1], k, v, causal=causal, scale=c.cfg.scale)
        O[b], L[b] = Ob[0], Lb[0]
    return O, L


def _describe(ci, what):
    c = ci.cache
    _say(f"[paged prefill] {what}: B{c.cfg.num_seqs} H{c.cfg.H} Hkv{c.cfg.Hkv} d{c.cfg.d} "
         f"Nq{ci.Nq} lens {int(c.seq_lens.min())}..{int(c.seq_lens.max())}")


@pytest.mark.parametrize("B,H,Hkv,d,Nq,lo,hi,causal", [
    (3, 8, 2, 128, 130, 130, 900, True),     # ragged prefix, ragged query tail
    (2, 8, 8, 128, 64, 64, 64, True),        # no cached prefix: plain causal prefill
    (4, 16, 4, 64, 200, 200, 1500, True),    # d = 64
    (3, 8, 1, 128, 77, 77, 700, False),      # non-causal, MQA
    (2, 32, 8, 128, 1, 1, 2000, True),       # one query (decode through the prefill path)
    (5, 4, 2, 128, 17, 17, 33, True),        # lengths around page / tile boundaries
    (70, 4, 2, 64, 16, 16, 200, True),       # more than 64 sequences (kept in order)
], ids=lambda x: str(x))
def test_paged_prefill_vs_oracle(B, H, Hkv, d, Nq, lo, hi, causal):
    ci = inputs.custom_chunked_prefill(B, H, Hkv, d, Nq, lo, hi, seed=B * 31 + Nq + d)
    _describe(ci, "vs oracle")
    o_h, lse_h = run_paged(ci, causal)
    O, L = oracle_paged(ci, causal)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, "paged prefill")


def test_paged_prefill_page_and_tile_boundaries():
    """Sequence lengths on both sides of page (16) and tile (64) boundaries."""
    lens = [40, 47, 48, 49, 63, 64, 65, 127, 128, 129, 1000]
    ci = inputs.custom_chunked_prefill(len(lens), 8, 2, 128, 40, 40, 1000, seq_lens=lens,
                                       seed=5)
    _describe(ci, "boundaries")
    o_h, lse_h = run_paged(ci)
    O, L = oracle_paged(ci)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, "paged prefill boundaries")


def test_paged_prefill_equal_lengths():
    """Sequences are taken longest first; equal lengths must still each be covered once."""
    lens = [300, 100, 300, 50, 100, 300]
    ci = inputs.custom_chunked_prefill(len(lens), 8, 4, 128, 50, 50, 300, seq_lens=lens,
                                       seed=13)
    _describe(ci, "equal lengths")
    o_h, lse_h = run_paged(ci)
    O, L = oracle_paged(ci)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, "paged prefill equal lengths")


@pytest.mark.parametrize("d,causal", [(128, True), (64, True), (128, False)])
def test_paged_prefill_bit_identical_to_contiguous(d, causal):
    """The paged kernel does the contiguous kernel's arithmetic on the same values: per
    sequence, fa_fwd on its contiguous K/V must give the same bits. (256 query heads, so
    that fa_fwd's launch is large enough to run the same ping-pong kernel.)"""
    torch = _torch()
    ci = inputs.custom_chunked_prefill(4, 256, 32, d, 150, 150, 1300, seed=17 + d)
    _describe(ci, f"bit-identity d{d} causal={causal}")
    o_p, lse_p = run_paged(ci, causal)
    c = ci.cache
    for b in range(c.cfg.num_seqs):
        q = bf16_to_dev(ci.q[b:b + 1])
        k = bf16_to_dev(np.ascontiguousarray(c.k_seq[b].transpose(1, 0, 2)[None]))
        v = bf16_to_dev(np.ascontiguousarray(c.v_seq[b].transpose(1, 0, 2)[None]))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        _lib.fa_fwd(q, k, v, o, lse, causal=causal, scale=c.cfg.scale)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_from_dev(o)[0], o_p[b]), f"O differs for sequence {b}"
        assert np.array_equal(lse.cpu().numpy()[0], lse_p[b]), f"LSE differs for sequence {b}"


def test_paged_prefill_never_reads_unused_slots_or_table_padding():
    """Slots past each sequence hold NaN and table entries past its pages hold -1:
    the result must be bit-identical to the zero-filled cache's."""
    a = inputs.custom_chunked_prefill(5, 8, 2, 128, 50, 50, 1000, seed=23)
    b = inputs.custom_chunked_prefill(5, 8, 2, 128, 50, 50, 1000, seed=23, unused_fill="nan",
                                      table_pad=-1)
    assert np.array_equal(a.cache.seq_lens, b.cache.seq_lens)
    _describe(b, "NaN padding")
    oa, la = run_paged(a)
    ob, lb = run_paged(b)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
    assert not np.any(np.isnan(inputs.bf16_bits_to_f32(ob)))


def test_paged_prefill_seq_len_below_nq_is_raised_to_nq():
    """A seq_len below Nq is taken as Nq (the new tokens are always present)."""
    ci = inputs.custom_chunked_prefill(2, 8, 2, 128, 96, 96, 96, seed=29)
    _describe(ci, "short seq_len")
    ref_o, ref_l = run_paged(ci)
    ci.cache.seq_lens[:] = 10
    o, lse = run_paged(ci)
    assert np.array_equal(o, ref_o) and np.array_equal(lse, ref_l)


def test_paged_prefill_long_prefix_sampled():
    """A long-context chunk: 2 sequences with 16K-24K cached tokens, 512 new queries,
    H32/Hkv8 d128; rows sampled for the oracle."""
    ci = inputs.custom_chunked_prefill(2, 32, 8, 128, 512, 16384, 24576, seed=41)
    _describe(ci, "long prefix")
    o_h, lse_h = run_paged(ci)
    c = ci.cache
    q = inputs.bf16_bits_to_f64(ci.q)
    rng = np.random.default_rng(3)
    got, want, gl, wl = [], [], [], []
    for b in range(2):
        k, v = _contig(c.k_seq[b]), _contig(c.v_seq[b])
        rows = {(0, h): np.unique(np.concatenate([[0, 511], rng.integers(0, 512, 6)]))
                for h in rng.choice(32, 6, replace=False)}
        O, L = oracle.attention(q[b:b + 1], k, v, causal=True, scale=c.cfg.scale, rows=rows)
        for (_, h), idx in rows.items():
            got.append(inputs.bf16_bits_to_f64(o_h[b, h, idx]))
            want.append(O[(0, h)])
            gl.append(lse_h[b, h, idx])
            wl.append(L[(0, h)])
    check_bf16(np.concatenate(got), np.concatenate(gl), np.concatenate(want),
               np.concatenate(wl), "paged prefill long prefix (sampled)")


# ---------------------------------------------------------------------------------
# KV append
# ---------------------------------------------------------------------------------
def _run_append(a: inputs.AppendInputs):
    torch = _torch()
    kc, vc = bf16_to_dev(a.k_cache), bf16_to_dev(a.v_cache)
    _lib.fa_kv_append(bf16_to_dev(a.k_new), bf16_to_dev(a.v_new), kc, vc,
                      torch.from_numpy(a.page_table).cuda(),
                      torch.from_numpy(a.start_pos).cuda())
    torch.cuda.synchronize()
    return bf16_from_dev(kc), bf16_from_dev(vc)


@pytest.mark.parametrize("S,n_new,Hkv,d,max_len", [
    (5, 1, 8, 128, 300),       # decode step: one token per sequence
    (3, 37, 2, 64, 500),       # a chunk crossing several pages
    (64, 128, 8, 128, 8192),   # a large prefill chunk for many sequences
], ids=lambda x: str(x))
def test_kv_append_bit_exact(S, n_new, Hkv, d, max_len):
    a = inputs.make_append(S, n_new, Hkv, d, max_len, seed=S + n_new)
    _say(f"[append] S{S} n_new{n_new} Hkv{Hkv} d{d} pool {a.k_cache.shape[0]} pages")
    k_got, v_got = _run_append(a)
    k_want = oracle.scatter_pages(a.k_cache, a.page_table, a.start_pos, a.k_new, 16)
    v_want = oracle.scatter_pages(a.v_cache, a.page_table, a.start_pos, a.v_new, 16)
    assert np.array_equal(k_got, k_want)
    assert np.array_equal(v_got, v_want)


def test_kv_append_drops_tokens_without_a_page():
    """Tokens that land on an unassigned entry (-1), past the table, or at a negative
    position are not written; every other slot keeps its bits."""
    a = inputs.make_append(4, 20, 2, 128, 64, seed=3, start_pos=[0, 40, 60, -5])
    a.page_table[1, 3] = -1          # positions 48..63 of sequence 1
    a.page_table[0, 0] = 10 ** 6     # an id outside the pool
    _say("[append] drops")
    k_got, v_got = _run_append(a)
    k_want = oracle.scatter_pages(a.k_cache, a.page_table, a.start_pos, a.k_new, 16)
    v_want = oracle.scatter_pages(a.v_cache, a.page_table, a.start_pos, a.v_new, 16)
    assert np.array_equal(k_got, k_want) and np.array_equal(v_got, v_want)


# ---------------------------------------------------------------------------------
# The whole flow: chunked prefill of a prompt, then decode steps
# ---------------------------------------------------------------------------------
def test_prefill_append_decode_flow():
    """Prompts of 3 sequences are fed in chunks of 96 tokens (append the chunk's K/V,
    then attend it to everything cached), then 3 decode steps (append one token, then
    decode). Every output is checked against the oracle on the contiguous K/V."""
    torch = _torch()
    S, H, Hkv, d, chunk = 3, 16, 4, 128, 96
    prompt = [250, 96, 400]
    steps = 3
    scale = 1 / math.sqrt(d)
    total = [p + steps for p in prompt]
    max_len = max(total)
    rng = np.random.default_rng(99)
    k_all = [inputs.f32_to_bf16_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32))
             for n in total]
    v_all = [inputs.f32_to_bf16_bits(rng.standard_normal((n, Hkv, d)).astype(np.float32))
             for n in total]
    q_all = [inputs.f32_to_bf16_bits(rng.standard_normal((H, n, d)).astype(np.float32))
             for n in total]
    max_pages = -(-max_len // 16)
    n_pool = S * max_pages + 2
    table = rng.permutation(n_pool)[:S * max_pages].reshape(S, max_pages).astype(np.int32)
    kc = torch.zeros((n_pool, 16, Hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pt = torch.from_numpy(table).cuda()

    def oracle_rows(s, upto, idx):
        q = inputs.bf16_bits_to_f64(q_all[s][:, :upto])[None]
        k, v = _contig(k_all[s][:upto]), _contig(v_all[s][:upto])
        rows = {(0, h): idx for h in range(H)}
        O, L = oracle.attention(q, k, v, causal=True, scale=scale, rows=rows)
        return (np.stack([O[(0, h)] for h in range(H)]), np.stack([L[(0, h)] for h in range(H)]))

    # chunked prefill, one sequence per call (prompt lengths differ)
    for s in range(S):
        pos = 0
        while pos < prompt[s]:
            n = min(chunk, prompt[s] - pos)
            _say(f"[flow] prefill seq {s} chunk {pos}..{pos + n}")
            sp = torch.tensor([pos], dtype=torch.int32, device="cuda")
            kn = bf16_to_dev(np.ascontiguousarray(k_all[s][pos:pos + n][None]))
            vn = bf16_to_dev(np.ascontiguousarray(v_all[s][pos:pos + n][None]))
            _lib.fa_kv_append(kn, vn, kc, vc, pt[s:s + 1].contiguous(), sp)
            q = bf16_to_dev(np.ascontiguousarray(q_all[s][:, pos:pos + n][None]))
            o = torch.empty_like(q)
            lse = torch.empty((1, H, n), dtype=torch.float32, device="cuda")
            sl = torch.tensor([pos + n], dtype=torch.int32, device="cuda")
            _lib.fa_fwd_paged(q, kc, vc, pt[s:s + 1].contiguous(), sl, o, lse,
                              max_seq_len=max_len, causal=True, scale=scale)
            torch.cuda.synchronize()
            O, L = oracle_rows(s, pos + n, np.arange(pos, pos + n))
            check_bf16(inputs.bf16_bits_to_f64(bf16_from_dev(o)[0]), lse.cpu().numpy()[0], O,
                       L, f"flow prefill s{s} @{pos}")
            pos += n

    # decode steps for all sequences at once
    ws = torch.empty(_lib.fa_decode_paged_workspace_size(S, H, d, max_len),
                     dtype=torch.uint8, device="cuda")
    for t in range(steps):
        _say(f"[flow] decode step {t}")
        cur = [p + t for p in prompt]
        kn = bf16_to_dev(np.stack([k_all[s][cur[s]:cur[s] + 1] for s in range(S)]))
        vn = bf16_to_dev(np.stack([v_all[s][cur[s]:cur[s] + 1] for s in range(S)]))
        sp = torch.tensor(cur, dtype=torch.int32, device="cuda")
        _lib.fa_kv_append(kn, vn, kc, vc, pt, sp)
        q = bf16_to_dev(np.stack([q_all[s][:, cur[s]] for s in range(S)]))
        o = torch.empty_like(q)
        lse = torch.empty((S, H), dtype=torch.float32, device="cuda")
        sl = torch.tensor([c + 1 for c in cur], dtype=torch.int32, device="cuda")
        _lib.fa_decode_paged(q, kc, vc, pt, sl, o, lse, max_seq_len=max_len, scale=scale,
                             workspace=ws)
        torch.cuda.synchronize()
        o_h = inputs.bf16_bits_to_f64(bf16_from_dev(o))
        l_h = lse.cpu().numpy()
        for s in range(S):
            O, L = oracle_rows(s, cur[s] + 1, np.array([cur[s]]))
            check_bf16(o_h[s][:, None], l_h[s][:, None], O, L, f"flow decode s{s} t{t}")


def test_one_query_paged_prefill_agrees_with_decode():
    """Nq = 1 through the prefill kernel and the decode kernel: both within the bf16
    bar of the oracle, and within twice that bar of each other."""
    ci = inputs.custom_chunked_prefill(6, 32, 8, 128, 1, 1, 3000, seed=61)
    _describe(ci, "Nq=1 vs decode")
    o_p, l_p = run_paged(ci)
    dec = ci.cache
    dec.q = np.ascontiguousarray(ci.q[:, :, 0, :])
    o_d, l_d = run_decode(dec)
    O, L = oracle_paged(ci)
    check_bf16(inputs.bf16_bits_to_f64(o_p), l_p, O, L, "Nq=1 prefill path")
    check_bf16(inputs.bf16_bits_to_f64(o_d)[:, :, None], l_d[:, :, None], O, L, "decode path")
