"""Seeded sweep of random small shapes through every attention entry point, each against
the fp64 oracle.

The hand-picked cases of the other GPU tests cover the edges on purpose; this sweep draws
shapes at random (a fixed seed, so the cases are the same on every run) to reach the
combinations nobody picked: ragged Nq / Nk against the 256-row and 64-key tiles, GQA
group sizes 1-4, d = 64 / 128, causal or not, windows of every kind, cached prefixes of
any length, decode lengths around page and split boundaries.
"""
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import (bf16_from_dev, bf16_to_dev, check_bf16, run_decode, run_prefill,
                         shaped_scores, widen_out)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.integers(1, 5))
        B = int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.integers(0, 2))
        Nq = int(rng.integers(1, 700))
        Nk = Nq + int(rng.integers(0, 500)) if causal else int(rng.integers(1, 900))
        out.append((B, H, Hkv, Nq, Nk, d, causal))
    return out


def _ping_pong_cases(n, seed):
    """Shapes that fa_fwd runs on the ping-pong kernel (more than 128 blocks of 256 rows),
    with a score profile each: plain N(0,1), Q four times larger (peaky rows), scores
    rising along the keys, or stepping up after the first 64 keys."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        d = int(rng.choice([64, 128]))
        Hkv = int(rng.choice([4, 8, 16, 32]))
        H = Hkv * int(rng.choice([1, 2, 4, 8]))
        causal = bool(rng.integers(0, 2))
        Nq = int(rng.integers(129, 1300))
        Nk = Nq + int(rng.integers(0, 700)) if causal else int(rng.integers(1, 1500))
        B = int(rng.integers(1, 3))
        while -(-Nq // 256) * B * H <= 128:
            H *= 2
        out.append((B, H, Hkv, Nq, Nk, d, causal, str(rng.choice(["plain", "x4", "rise", "step"]))))
    return out


def _window_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.integers(1, 4))
        d = int(rng.choice([64, 128]))
        Nq = int(rng.integers(1, 800))
        Nk = Nq + int(rng.integers(0, 400))
        side = lambda: int(rng.choice([-1, 0, int(rng.integers(1, 64)),
                                       int(rng.integers(64, 900))]))
        out.append((int(rng.integers(1, 3)), H, Hkv, Nq, Nk, d, side(), side()))
    return out


def _paged_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4]))
        H = Hkv * int(rng.integers(1, 5))
        d = int(rng.choice([64, 128]))
        Nq = int(rng.integers(1, 300))
        lo = Nq + int(rng.integers(0, 200))
        out.append((int(rng.integers(1, 6)), H, Hkv, d, Nq, lo, lo + int(rng.integers(0, 900)),
                    bool(rng.integers(0, 2))))
    return out


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        H = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
        d = int(rng.choice([64, 128]))
        lo = int(rng.integers(0, 600))
        out.append((int(rng.integers(1, 12)), H, Hkv, d, lo, lo + int(rng.integers(0, 2500))))
    return out


@pytest.mark.parametrize("shape", _prefill_cases(24, 2024), ids=lambda s: str(s))
def test_sweep_prefill(shape):
    B, H, Hkv, Nq, Nk, d, causal = shape
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, "bf16", seed=sum(shape))
    _say(f"[sweep] prefill {shape}")
    o_h, lse_h = run_prefill(inp)
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=causal, scale=inp.cfg.scale)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, f"sweep prefill {shape}")


@pytest.mark.parametrize("shape", _ping_pong_cases(24, 2028), ids=lambda s: str(s))
def test_sweep_prefill_ping_pong(shape):
    """Every row of two seeded (batch, head) pairs against the oracle."""
    B, H, Hkv, Nq, Nk, d, causal, pattern = shape
    base = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, "bf16", seed=Nq + Nk + d + H)
    if pattern in ("rise", "step"):
        inp = shaped_scores(base, pattern)
    elif pattern == "x4":
        q = inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(base.q) * np.float32(4.0))
        inp = inputs.PrefillInputs(base.cfg, q, base.k, base.v, base.rng)
    else:
        inp = base
    _say(f"[sweep] ping-pong prefill {shape}")
    o_h, lse_h = run_prefill(inp)
    rng = np.random.default_rng(Nq * 7 + Nk)
    rows = {(int(rng.integers(0, B)), int(rng.integers(0, H))): np.arange(Nq) for _ in range(2)}
    qf, kf, vf = inp.as_f64()
    O, L = oracle.attention(qf, kf, vf, causal=causal, scale=inp.cfg.scale, rows=rows)
    got = np.concatenate([widen_out(o_h[b, h, idx], "bf16") for (b, h), idx in rows.items()])
    want = np.concatenate([O[x] for x in rows])
    lg = np.concatenate([lse_h[b, h, idx] for (b, h), idx in rows.items()])
    lw = np.concatenate([L[x] for x in rows])
    check_bf16(got, lg, want, lw, f"sweep ping-pong {shape}")


@pytest.mark.parametrize("shape", _window_cases(16, 2025), ids=lambda s: str(s))
def test_sweep_window(shape):
    import torch
    B, H, Hkv, Nq, Nk, d, left, right = shape
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, False, seed=Nq + Nk + 7 * d)
    _say(f"[sweep] window {shape}")
    c = inp.cfg
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda")
    _lib.fa_fwd_window(q, k, v, o, lse, window_left=left, window_right=right, scale=c.scale)
    torch.cuda.synchronize()
    qf, kf, vf = inp.as_f64()
    O, L = oracle.attention(qf, kf, vf, causal=False, scale=c.scale, window=(left, right))
    check_bf16(inputs.bf16_bits_to_f64(bf16_from_dev(o)), lse.cpu().numpy(), O, L,
               f"sweep window {shape}")


@pytest.mark.parametrize("shape", _paged_cases(14, 2026), ids=lambda s: str(s))
def test_sweep_paged_prefill(shape):
    from test_gpu_paged import oracle_paged, run_paged
    B, H, Hkv, d, Nq, lo, hi, causal = shape
    ci = inputs.custom_chunked_prefill(B, H, Hkv, d, Nq, lo, hi, seed=lo + hi + d)
    _say(f"[sweep] paged prefill {shape}")
    o_h, lse_h = run_paged(ci, causal)
    O, L = oracle_paged(ci, causal)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, f"sweep paged {shape}")


@pytest.mark.parametrize("shape", _decode_cases(16, 2027), ids=lambda s: str(s))
def test_sweep_decode(shape):
    S, H, Hkv, d, lo, hi = shape
    inp = inputs.custom_decode(S, H, Hkv, d, lo, hi, seed=S + lo + hi)
    _say(f"[sweep] decode {shape}")
    o_h, lse_h = run_decode(inp)
    ks = [inputs.bf16_bits_to_f64(x) for x in inp.k_seq]
    vs = [inputs.bf16_bits_to_f64(x) for x in inp.v_seq]
    O, L = oracle.decode(inputs.bf16_bits_to_f64(inp.q), ks, vs, scale=inp.cfg.scale)
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, f"sweep decode {shape}")
