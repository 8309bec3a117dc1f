"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's analytic gradients.

The oracle (oracle.attention_backward) is pinned by central differences on the CPU. Here
the kernel's dQ, dK, dV (bf16, fp32 accumulation, recomputed probabilities) are compared
element by element; the forward's O and lse come from fa_fwd on the same inputs, as in
training.

Tolerance: every gradient element is a sum of products whose bf16 operands (P and dS
are rounded to bf16 before their MFMAs, the results are rounded to bf16) carry a
relative error of at most 2^-9 each, with independent signs over the summed terms, so
the error is a few 2^-9 of the gradient's magnitude: max-abs error <= 2e-2 x max|ref|
and mean-abs error <= 2e-3 x max|ref| (the forward's 2e-2 / 2e-3 bar, scaled by the
magnitude, since gradients are not bounded by |V| as the forward's output is).
"""
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import bf16_from_dev, bf16_to_dev

pytestmark = pytest.mark.gpu

REL_MAX = 2e-2
REL_MEAN = 2e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_bwd(inp, do_bits):
    import torch
    c = inp.cfg
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda")
    _lib.fa_fwd(q, k, v, o, lse, causal=c.causal, scale=c.scale)
    do = bf16_to_dev(do_bits)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(_lib.fa_bwd_workspace_size(c.B, c.H, c.Nq), dtype=torch.uint8,
                     device="cuda")
    _lib.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, causal=c.causal, scale=c.scale, workspace=ws)
    torch.cuda.synchronize()
    return bf16_from_dev(dq), bf16_from_dev(dk), bf16_from_dev(dv)


def check_grad(got_bits, ref, what):
    got = inputs.bf16_bits_to_f64(got_bits)
    mag = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    mx, mean = float(err.max()) / mag, float(err.mean()) / mag
    msg = f"{what}: max|ref| {mag:.3e} rel max-abs {mx:.2e} rel mean-abs {mean:.2e}"
    _say(msg)
    assert np.all(np.isfinite(got)), msg
    assert mx <= REL_MAX and mean <= REL_MEAN, msg


def _case(B, H, Hkv, Nq, Nk, d, causal, seed):
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, seed=seed)
    rng = np.random.default_rng(seed + 1)
    do = inputs.f32_to_bf16_bits(rng.standard_normal((B, H, Nq, d)).astype(np.float32))
    _say(f"[bwd] B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} causal={causal}")
    dq, dk, dv = run_bwd(inp, do)
    q, k, v = inp.as_f64()
    rq, rk, rv = oracle.attention_backward(q, k, v, inputs.bf16_bits_to_f64(do),
                                           causal=causal, scale=inp.cfg.scale)
    check_grad(dq, rq, "dQ")
    check_grad(dk, rk, "dK")
    check_grad(dv, rv, "dV")


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,causal", [
    (1, 4, 4, 256, 256, 128, True),
    (2, 8, 2, 333, 333, 128, True),      # GQA, ragged tiles
    (1, 4, 1, 200, 517, 128, True),      # Nq < Nk, MQA
    (2, 4, 2, 300, 300, 128, False),
    (1, 8, 2, 640, 640, 64, True),       # d = 64
    (1, 2, 2, 1, 77, 128, False),        # one query
    (1, 4, 4, 1024, 1024, 128, True),
], ids=lambda x: str(x))
def test_backward_vs_oracle(B, H, Hkv, Nq, Nk, d, causal):
    _case(B, H, Hkv, Nq, Nk, d, causal, seed=Nq + 7 * Nk + d + H)


def test_backward_deterministic():
    """Two runs give identical bits (no atomics)."""
    inp = inputs.custom_prefill(1, 8, 2, 500, 500, 128, True, seed=9)
    rng = np.random.default_rng(10)
    do = inputs.f32_to_bf16_bits(rng.standard_normal((1, 8, 500, 128)).astype(np.float32))
    a = run_bwd(inp, do)
    b = run_bwd(inp, do)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_gqa_causal_workload_sampled_groups():
    """The benched backward workload, B4 H32 Hkv8 N4096 d128 causal (the GQA causal
    prefill's inputs, dO from inputs.make_dout): the kernels run on the whole workload and
    two seeded (batch, KV head) groups are compared in full with the oracle: dK and dV of
    the group's KV head and dQ of its g = 4 query heads."""
    import torch
    cfg = inputs.PREFILL_CONFIGS["gqa_causal"]
    inp = inputs.make_prefill(cfg)
    do_bits = inputs.make_dout(cfg, seed=cfg.seed + 100)
    _say(f"[bwd] {cfg.name} full workload")
    dq, dk, dv = run_bwd(inp, do_bits)
    torch.cuda.empty_cache()
    g = cfg.H // cfg.Hkv
    rng = np.random.default_rng(31)
    picks = rng.choice(cfg.B * cfg.Hkv, size=2, replace=False)
    for p in sorted(int(x) for x in picks):
        b, kvh = p // cfg.Hkv, p % cfg.Hkv
        hs = slice(kvh * g, (kvh + 1) * g)
        _say(f"[bwd] oracle group b={b} kv head {kvh}")
        q = inputs.bf16_bits_to_f64(inp.q[b:b + 1, hs])
        k = inputs.bf16_bits_to_f64(inp.k[b:b + 1, kvh:kvh + 1])
        v = inputs.bf16_bits_to_f64(inp.v[b:b + 1, kvh:kvh + 1])
        do = inputs.bf16_bits_to_f64(do_bits[b:b + 1, hs])
        rq, rk, rv = oracle.attention_backward(q, k, v, do, causal=True, scale=cfg.scale)
        check_grad(dq[b:b + 1, hs], rq, f"dQ b{b} heads {hs.start}..{hs.stop - 1}")
        check_grad(dk[b:b + 1, kvh:kvh + 1], rk, f"dK b{b} kv{kvh}")
        check_grad(dv[b:b + 1, kvh:kvh + 1], rv, f"dV b{b} kv{kvh}")
