"""GPU parity of sliding-window prefill (fa_fwd_window) against the fp64 oracle.

Glossary entry "Kayan Pencere Dikkati (Sliding Window Attention)": each query attends
only the keys within (left, right) of its own position (bottom-right placed, as for
causal). Cases cover symmetric, causal-left and one-sided windows, the degenerate
(0, 0) window (each row selects its own V row), windows wider than the sequence,
Nq < Nk, GQA, d = 64/128 and ragged tails; the (-1, 0) window must reproduce the causal
kernel bit for bit.
"""
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import bf16_from_dev, bf16_to_dev, check_bf16, shaped_scores

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_window(inp, left, right):
    import torch
    c = inp.cfg
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda")
    _lib.fa_fwd_window(q, k, v, o, lse, window_left=left, window_right=right, scale=c.scale)
    torch.cuda.synchronize()
    return bf16_from_dev(o), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk,d,left,right", [
    (2, 8, 2, 1000, 1000, 128, 64, 64),      # symmetric, w = 128
    (2, 8, 2, 1000, 1000, 128, 100, 0),      # causal sliding window
    (1, 4, 4, 777, 777, 128, 300, 17),       # asymmetric, ragged tail
    (2, 8, 8, 500, 500, 128, 0, 0),          # only itself
    (2, 4, 1, 300, 1000, 128, 128, 0),       # Nq < Nk (queries after a prefix), MQA
    (1, 8, 2, 640, 640, 64, 96, 32),         # d = 64
    (1, 4, 2, 200, 200, 128, 5000, 5000),    # wider than the sequence (= no mask)
    (1, 4, 2, 333, 333, 128, 20, -1),        # unbounded right side
    (1, 4, 2, 333, 333, 128, -1, 40),        # unbounded left side
], ids=lambda x: str(x))
def test_window_vs_oracle(B, H, Hkv, Nq, Nk, d, left, right):
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, False, seed=Nq + left + 3 * right)
    _say(f"[window] B{B} H{H} Hkv{Hkv} Nq{Nq} Nk{Nk} d{d} window ({left},{right})")
    o_h, lse_h = run_window(inp, left, right)
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=False, scale=inp.cfg.scale, window=(left, right))
    check_bf16(inputs.bf16_bits_to_f64(o_h), lse_h, O, L, f"window ({left},{right})")


def test_window_zero_selects_own_value_row():
    """Window (0, 0) with peaked data: O must be V[p] exactly (bf16 bits)."""
    inp = inputs.custom_prefill(1, 4, 2, 300, 300, 128, False, seed=77)
    _say("[window] (0,0) bit-exact")
    o_h, _ = run_window(inp, 0, 0)
    g = 2
    for h in range(4):
        assert np.array_equal(o_h[0, h], inp.v[0, h // g]), f"head {h}"


@pytest.mark.parametrize("d", [128, 64])
def test_window_minus_one_zero_is_the_causal_kernel(d):
    """(-1, 0) is plain causal: bit-identical to fa_fwd(causal=True) (256 query heads, so
    that fa_fwd runs the same ping-pong kernel rather than the key-split one)."""
    import torch
    inp = inputs.custom_prefill(2, 128, 16, 700, 900, d, True, seed=5 + d)
    _say(f"[window] (-1,0) vs causal d{d}")
    o_w, l_w = run_window(inp, -1, 0)
    c = inp.cfg
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda")
    _lib.fa_fwd(q, k, v, o, lse, causal=True, scale=c.scale)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_from_dev(o), o_w)
    assert np.array_equal(lse.cpu().numpy(), l_w)


def test_window_long_gqa_sampled():
    """B4 H32 Hkv8 N4096 d128 with a causal window of 1024 keys; rows sampled."""
    inp = inputs.custom_prefill(4, 32, 8, 4096, 4096, 128, False, seed=404)
    _say("[window] long GQA (1024,0) sampled")
    o_h, lse_h = run_window(inp, 1024, 0)
    q, k, v = inp.as_f64()
    rng = np.random.default_rng(8)
    rows = {(int(b), int(h)): np.unique(np.concatenate(
        [[0, 1023, 1024, 4095], rng.integers(0, 4096, 12)]))
        for b, h in zip(rng.integers(0, 4, 10), rng.integers(0, 32, 10))}
    O, L = oracle.attention(q, k, v, causal=False, scale=inp.cfg.scale, rows=rows,
                            window=(1024, 0))
    got = np.concatenate([inputs.bf16_bits_to_f64(o_h[b, h, idx]) for (b, h), idx in rows.items()])
    want = np.concatenate([O[key] for key in rows])
    gl = np.concatenate([lse_h[b, h, idx] for (b, h), idx in rows.items()])
    wl = np.concatenate([L[key] for key in rows])
    check_bf16(got, gl, want, wl, "window long GQA")


def test_window_benched_workload_sampled():
    """The benched sliding-window workload (inputs.WINDOW_CONFIG: B1 H32 Hkv8 N32768 d128,
    window (4096, 0)): 256 seeded rows in each of 4 heads, plus the rows at the window's
    edges (the last row whose window still reaches key 0, the first that does not, their
    neighbours, the first and last rows)."""
    cfg = inputs.WINDOW_CONFIG
    left, right = inputs.WINDOW
    inp = inputs.make_prefill(cfg)
    _say(f"[window] {cfg.name} ({left},{right}) sampled")
    o_h, lse_h = run_window(inp, left, right)
    rng = np.random.default_rng(12)
    edges = np.array([0, 1, left - 1, left, left + 1, 2 * left, cfg.Nq - 2, cfg.Nq - 1])
    heads = rng.choice(cfg.H, size=4, replace=False)
    rows = {(0, int(h)): np.unique(np.concatenate([edges, rng.choice(cfg.Nq, 256, replace=False)]))
            for h in sorted(heads)}
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=False, scale=cfg.scale, rows=rows,
                            window=(left, right))
    got = np.concatenate([inputs.bf16_bits_to_f64(o_h[b, h, idx]) for (b, h), idx in rows.items()])
    want = np.concatenate([O[key] for key in rows])
    gl = np.concatenate([lse_h[b, h, idx] for (b, h), idx in rows.items()])
    wl = np.concatenate([L[key] for key in rows])
    check_bf16(got, gl, want, wl, "window benched workload")


@pytest.mark.parametrize("pattern", ["rise", "step"])
@pytest.mark.parametrize("left,right", [(300, 0), (100, 40), (700, 0)])
def test_window_reference_max(pattern, left, right):
    """Scores rising along the keys, or stepping up after the first 64 keys: rows start
    their windows mid-tile, where any rise moves the reference, and later tiles may take
    the max-free path. Every row of two heads against the oracle."""
    base = inputs.custom_prefill(2, 32, 8, 1024, 1024, 128, False, seed=64 + left + right)
    inp = shaped_scores(base, pattern)
    _say(f"[window] reference max {pattern} ({left},{right})")
    o_h, lse_h = run_window(inp, left, right)
    rows = {(0, 0): np.arange(1024), (1, 31): np.arange(1024)}
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=False, scale=inp.cfg.scale, rows=rows,
                            window=(left, right))
    got = np.concatenate([inputs.bf16_bits_to_f64(o_h[b, h, idx]) for (b, h), idx in rows.items()])
    want = np.concatenate([O[key] for key in rows])
    gl = np.concatenate([lse_h[b, h, idx] for (b, h), idx in rows.items()])
    wl = np.concatenate([L[key] for key in rows])
    check_bf16(got, gl, want, wl, f"window ({left},{right}) reference max {pattern}")


def test_window_launch_matches_launches_of_its_parts():
    """B1 H8 Hkv2 N17000 d128, window (1000, 0): 536 (head, q tile) items in one launch give
    the same bits as each KV head's 4 query heads launched alone (268 items). A few rows per
    head, at the window's edges, are also checked against the oracle."""
    import torch
    inp = inputs.custom_prefill(1, 8, 2, 17000, 17000, 128, False, seed=405)
    _say("[window] one launch vs per-KV-head launches")
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))

    def fwd(qq, kk, vv):
        o = torch.empty_like(qq)
        lse = torch.empty(qq.shape[:3], dtype=torch.float32, device="cuda")
        _lib.fa_fwd_window(qq, kk, vv, o, lse, window_left=1000, window_right=0,
                           scale=inp.cfg.scale)
        torch.cuda.synchronize()
        return bf16_from_dev(o), lse.cpu().numpy()

    o_h, lse_h = fwd(q, k, v)
    for kv in range(2):
        o_p, l_p = fwd(q[:, 4 * kv:4 * kv + 4].contiguous(), k[:, kv:kv + 1].contiguous(),
                       v[:, kv:kv + 1].contiguous())
        assert np.array_equal(o_h[:, 4 * kv:4 * kv + 4], o_p)
        assert np.array_equal(lse_h[:, 4 * kv:4 * kv + 4], l_p)
    rows = {(0, h): np.array([0, 999, 1000, 1001, 8191, 16999]) for h in range(8)}
    O, L = oracle.attention(*inp.as_f64(), causal=False, scale=inp.cfg.scale, rows=rows,
                            window=(1000, 0))
    got = np.concatenate([inputs.bf16_bits_to_f64(o_h[b, h, idx]) for (b, h), idx in rows.items()])
    want = np.concatenate([O[key] for key in rows])
    gl = np.concatenate([lse_h[b, h, idx] for (b, h), idx in rows.items()])
    wl = np.concatenate([L[key] for key in rows])
    check_bf16(got, gl, want, wl, "window launch parts")
