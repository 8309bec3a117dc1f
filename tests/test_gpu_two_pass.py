"""GPU parity of the FlashAttention-1 two-pass prefill (fa_fwd_two_pass).

Page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention", section "FlashAttention-1
(İki Geçişli Yaklaşım)": a statistics pass writes each row's (M, L) (here as lse) and an
output pass renormalises recomputed scores with them. Checked against the fp64 oracle,
and against the single-pass kernel: the statistics pass runs the ping-pong kernel's
arithmetic without the P.V products, so where fa_fwd runs that kernel (launches with more
than 128 blocks of 256 rows) its lse must match fa_fwd's bit for bit; where fa_fwd runs
the key-split kernel the two lse agree up to summation order. The two outputs must agree
to the bf16 bar.
"""
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import (BF16_MAX_ABS, bf16_from_dev, bf16_to_dev, check_bf16, errors,
                         shaped_scores)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_both(inp):
    import torch
    c = inp.cfg
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o2, o1 = torch.empty_like(q), torch.empty_like(q)
    l2 = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda")
    l1 = torch.empty_like(l2)
    _lib.fa_fwd_two_pass(q, k, v, o2, l2, causal=c.causal, scale=c.scale)
    _lib.fa_fwd(q, k, v, o1, l1, causal=c.causal, scale=c.scale)
    torch.cuda.synchronize()
    return bf16_from_dev(o2), l2.cpu().numpy(), bf16_from_dev(o1), l1.cpu().numpy()


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", [
    (2, 8, 2, 700, 700, 128, True),
    (2, 8, 8, 513, 1000, 128, True),     # Nq < Nk, ragged
    (1, 4, 1, 300, 450, 128, False),
    (2, 8, 2, 1024, 1024, 64, True),     # d = 64
    (1, 2, 2, 1, 77, 128, True),         # one query
    (1, 256, 32, 300, 450, 128, True),   # fa_fwd on the ping-pong kernel
    (2, 128, 128, 77, 77, 64, False),    # the same, d = 64
], ids=lambda x: str(x))
def test_two_pass_vs_oracle_and_single_pass(B, H, Hkv, Nq, Nk, d, causal):
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, seed=Nq + Nk + d)
    _say(f"[two-pass] B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    o2, l2, o1, l1 = run_both(inp)
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=causal, scale=inp.cfg.scale)
    check_bf16(inputs.bf16_bits_to_f64(o2), l2, O, L, "two-pass vs oracle")
    if -(-Nq // 256) * B * H > 128:
        assert np.array_equal(l2, l1), "statistics pass lse differs from the single pass"
    else:
        assert np.abs(l2 - l1).max() <= 1e-4, "statistics pass lse vs the key-split kernel's"
    mx, _ = errors(inputs.bf16_bits_to_f64(o2), inputs.bf16_bits_to_f64(o1))
    assert mx <= BF16_MAX_ABS, f"two-pass vs single-pass max-abs {mx}"


def test_two_pass_gqa_sampled():
    """B4 H32 Hkv8 N4096 d128 causal; rows sampled for the oracle."""
    cfg = inputs.PREFILL_CONFIGS["gqa_causal"]
    inp = inputs.make_prefill(cfg)
    _say("[two-pass] gqa_causal sampled")
    o2, l2, o1, l1 = run_both(inp)
    assert np.array_equal(l2, l1)
    rows = inputs.sample_rows(inp, 1, 128)
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=True, scale=cfg.scale, rows=rows)
    got = np.concatenate([inputs.bf16_bits_to_f64(o2[b, h, idx]) for (b, h), idx in rows.items()])
    want = np.concatenate([O[key] for key in rows])
    gl = np.concatenate([l2[b, h, idx] for (b, h), idx in rows.items()])
    wl = np.concatenate([L[key] for key in rows])
    check_bf16(got, gl, want, wl, "two-pass gqa sampled")


@pytest.mark.parametrize("pattern", ["rise", "step"])
def test_two_pass_reference_max_agrees_with_single_pass(pattern):
    """Scores that move the reference max on every tile ("rise") or fail the max-free check
    of the statistics pass without moving it ("step"): the statistics pass must still
    reproduce the single pass's lse bit for bit (ping-pong launch), and both outputs
    must meet the oracle."""
    base = inputs.custom_prefill(1, 256, 32, 300, 700, 128, True, seed=63)
    inp = shaped_scores(base, pattern)
    _say(f"[two-pass] reference max, {pattern}")
    o2, l2, o1, l1 = run_both(inp)
    assert np.array_equal(l2, l1), "statistics pass lse differs from the single pass"
    rows = {(0, 0): np.arange(300), (0, 255): np.arange(300)}
    q, k, v = inp.as_f64()
    Or, Lr = oracle.attention(q, k, v, causal=True, scale=inp.cfg.scale, rows=rows)
    for o_h, l_h, what in ((o2, l2, "two-pass"), (o1, l1, "single pass")):
        got = np.concatenate([inputs.bf16_bits_to_f64(o_h[b, h, idx]) for (b, h), idx in rows.items()])
        want = np.concatenate([Or[x] for x in rows])
        lg = np.concatenate([l_h[b, h, idx] for (b, h), idx in rows.items()])
        lw = np.concatenate([Lr[x] for x in rows])
        check_bf16(got, lg, want, lw, f"{what}, reference max {pattern}")
