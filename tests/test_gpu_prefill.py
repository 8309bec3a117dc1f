"""GPU parity of the prefill kernels (fa_fwd, fa_fwd_fp32) against the fp64 oracle.

Every case runs the HIP path through the C ABI on seeded inputs and compares element
by element with the oracle on the same stored values. Large workloads are checked
on seeded row samples (every row of some (batch, head) pairs plus random rows).
"""
import math
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import (bf16_from_dev, bf16_to_dev, check_bf16, check_fp32, run_prefill,
                         shaped_scores, widen_out)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _dense_check(inp, what):
    c = inp.cfg
    _say(f"[prefill] {what}: B{c.B} H{c.H} Hkv{c.Hkv} Nq{c.Nq} Nk{c.Nk} d{c.d} "
         f"causal={c.causal} {c.dtype}")
    o_h, lse_h = run_prefill(inp)
    q, k, v = inp.as_f64()
    O, L = oracle.attention(q, k, v, causal=c.causal, scale=c.scale)
    got = widen_out(o_h, c.dtype)
    if c.dtype == "f32":
        return check_fp32(got, lse_h, O, L, what)
    return check_bf16(got, lse_h, O, L, what)


def _sampled_check(inp, rows, what):
    c = inp.cfg
    _say(f"[prefill] {what}: B{c.B} H{c.H} Hkv{c.Hkv} N{c.Nq} d{c.d} causal={c.causal}, "
         f"{sum(len(r) for r in rows.values())} sampled rows")
    o_h, lse_h = run_prefill(inp)
    q, k, v = inp.as_f64()
    Or, Lr = oracle.attention(q, k, v, causal=c.causal, scale=c.scale, rows=rows)
    got = np.concatenate([widen_out(o_h[b, h, idx], c.dtype) for (b, h), idx in sorted(rows.items())])
    want = np.concatenate([Or[x] for x in sorted(rows)])
    lg = np.concatenate([lse_h[b, h, idx] for (b, h), idx in sorted(rows.items())])
    lw = np.concatenate([Lr[x] for x in sorted(rows)])
    return check_bf16(got, lg, want, lw, what)


# ---- the workloads at their full sizes ------------------------------------------
def test_fp32_single_head_full():
    _dense_check(inputs.make_prefill(inputs.PREFILL_CONFIGS["fp32_single"]), "fp32_single")


def test_bf16_causal_full():
    _dense_check(inputs.make_prefill(inputs.PREFILL_CONFIGS["bf16_causal"]), "bf16_causal")


def test_gqa_causal_sampled():
    inp = inputs.make_prefill(inputs.PREFILL_CONFIGS["gqa_causal"])
    rows = inputs.sample_rows(inp, n_full_pairs=2, n_random_rows=512)
    _sampled_check(inp, rows, "gqa_causal")


def test_long_causal_sampled():
    inp = inputs.make_prefill(inputs.PREFILL_CONFIGS["long_causal"])
    rows = inputs.sample_rows_per_head(inp, 256)
    # the last row of every head (longest prefix) and the first one are always checked
    for key in rows:
        rows[key] = np.unique(np.concatenate([rows[key], [0, inp.cfg.Nq - 1]]))
    _sampled_check(inp, rows, "long_causal")


# ---- ragged tails, GQA/MQA, bottom-right causal, tiny and degenerate shapes -------
SHAPES = [
    # B, H, Hkv, Nq, Nk, d, causal
    (1, 2, 1, 1000, 1000, 128, True),
    (1, 4, 2, 1000, 1000, 64, True),
    (2, 4, 4, 77, 300, 128, True),      # Nq < Nk: queries come after 223 cached keys
    (1, 2, 2, 130, 129, 64, False),
    (1, 1, 1, 1, 1, 128, True),
    (1, 1, 1, 1, 5, 64, False),
    (1, 8, 1, 257, 257, 128, True),     # MQA
    (2, 3, 3, 200, 200, 128, False),    # H*B not a multiple of 8
    (1, 16, 2, 64, 4100, 128, True),    # long cache, short query block
    (3, 2, 1, 129, 129, 64, False),
    (1, 2, 2, 4097, 4097, 128, True),
    (2, 4, 2, 1, 777, 64, True),        # one query row over a long cache (key-split kernel)
    (1, 4, 4, 3, 300, 128, False),      # three rows: one 64-row block, mostly empty
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(str(int(x)) for x in s))
def test_bf16_shapes(shape):
    """Launches with at most 128 blocks of 256 rows (half the compute units) and more than
    128 keys run on the key-split kernel (64-row work-groups whose keys run in four parts);
    the ones with at most 128 keys on the ping-pong kernel."""
    B, H, Hkv, Nq, Nk, d, causal = shape
    assert _pp_groups(B, H, Nq) <= 128
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, "bf16", seed=sum(shape))
    _dense_check(inp, f"bf16 {shape}")


def _pp_groups(B, H, Nq):
    return -(-Nq // 256) * B * H


# The same kinds of edge (ragged tails, GQA/MQA, bottom-right causal, one query, one key
# tile) with enough (batch, head) pairs that fa_fwd runs the ping-pong kernel.
SHAPES_PP = [
    (1, 256, 32, 300, 300, 128, True),
    (2, 128, 16, 77, 300, 128, True),
    (1, 256, 256, 130, 129, 64, False),
    (1, 256, 1, 1, 5, 64, False),
    (4, 64, 8, 257, 257, 64, True),
    (2, 128, 128, 1, 1, 128, True),
]


@pytest.mark.parametrize("shape", SHAPES_PP, ids=lambda s: "x".join(str(int(x)) for x in s))
def test_bf16_shapes_ping_pong(shape):
    B, H, Hkv, Nq, Nk, d, causal = shape
    assert _pp_groups(B, H, Nq) > 128
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, "bf16", seed=sum(shape))
    _dense_check(inp, f"bf16 ping-pong {shape}")


@pytest.mark.parametrize("shape", [
    (1, 2, 1, 100, 100, 64, True), (2, 2, 2, 65, 200, 128, False), (1, 4, 2, 33, 70, 64, True),
    (1, 1, 1, 1, 1, 64, False),
], ids=lambda s: "x".join(str(int(x)) for x in s))
def test_fp32_shapes(shape):
    B, H, Hkv, Nq, Nk, d, causal = shape
    inp = inputs.custom_prefill(B, H, Hkv, Nq, Nk, d, causal, "f32", seed=sum(shape))
    _dense_check(inp, f"fp32 {shape}")


def test_bf16_largest_head_slice():
    """The largest K/V slice one head may have (Nk * d * 2 bytes just under 2^31, the
    32-bit buffer-offset limit of the ABI): 8388544 keys, d = 128, 100 ragged query rows,
    non-causal; four rows checked against the oracle over all keys."""
    Nk = (1 << 23) - 64
    assert Nk * 128 * 2 < 1 << 31
    inp = inputs.custom_prefill(1, 1, 1, 100, Nk, 128, False, seed=77)
    _sampled_check(inp, {(0, 0): np.array([0, 37, 63, 99])}, "largest head slice")


def test_bf16_scale_not_default():
    inp = inputs.custom_prefill(1, 2, 2, 300, 300, 128, True, "bf16", scale=0.3, seed=9)
    _dense_check(inp, "bf16 scale=0.3")


def test_bf16_large_scores_stay_finite():
    """Dimension 0 of every q and k is set to 64, adding the same 64*64/8 = 512 to every
    score of a row: the softmax is unchanged, but exp of an unshifted score would
    overflow fp32. The result must match the oracle to the usual tolerance."""
    inp = inputs.custom_prefill(1, 2, 2, 256, 256, 64, True, "bf16", seed=3)
    big = inputs.f32_to_bf16_bits(np.array([64.0], np.float32))[0]
    inp.q[..., 0] = big
    inp.k[..., 0] = big
    _dense_check(inp, "bf16 large scores")


# ---- exactness properties ---------------------------------------------------------
@pytest.mark.parametrize("d,causal", [(128, False), (128, True), (64, True)])
def test_peaked_rows_select_value_row_bit_exactly(d, causal):
    """q_i = 64 k_t(i): the target key wins by a margin that makes every other
    exponential exactly zero in fp32, so O_i must equal the stored V_t(i) bit for bit
    (an indexing error cannot hide inside a tolerance)."""
    rng = np.random.default_rng(d + causal)
    B, H, Hkv, N = 1, 4, 2, 640
    base = inputs.custom_prefill(B, H, Hkv, N, N, d, causal, "bf16", seed=d)
    q = np.empty_like(base.q)
    tgt = np.empty((B, H, N), dtype=np.int64)
    g = H // Hkv
    for h in range(H):
        for i in range(N):
            t = int(rng.integers(0, i + 1)) if causal else int(rng.integers(0, N))
            tgt[0, h, i] = t
        kk = inputs.bf16_bits_to_f32(base.k[0, h // g, tgt[0, h]])
        q[0, h] = inputs.f32_to_bf16_bits(kk * np.float32(64.0))
    inp = inputs.PrefillInputs(base.cfg, q, base.k, base.v, base.rng)
    _say(f"[prefill] peaked d={d} causal={causal}")
    o_h, _ = run_prefill(inp)
    qf, kf, vf = inp.as_f64()
    n_exact = 0
    for h in range(H):
        s = qf[0, h] @ kf[0, h // g].T * base.cfg.scale * math.log2(math.e)
        if causal:
            s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
        top = s[np.arange(N), tgt[0, h]]
        s2 = s.copy()
        s2[np.arange(N), tgt[0, h]] = -np.inf
        margin = top - s2.max(axis=1)
        sure = margin > 160.0      # 2^-160 underflows to exactly 0 in fp32
        want = base.v[0, h // g, tgt[0, h]]
        assert np.array_equal(o_h[0, h][sure], want[sure])
        n_exact += int(sure.sum())
    assert n_exact > 0.9 * H * N


def test_future_keys_do_not_change_causal_rows():
    """Causal rows must be bit-identical when keys/values after them change."""
    inp = inputs.custom_prefill(1, 2, 2, 512, 512, 128, True, "bf16", seed=21)
    o1, l1 = run_prefill(inp)
    k2, v2 = inp.k.copy(), inp.v.copy()
    k2[:, :, 300:] = inputs.f32_to_bf16_bits(np.full(k2[:, :, 300:].shape, 7.0, np.float32))
    v2[:, :, 300:] = inputs.f32_to_bf16_bits(np.full(v2[:, :, 300:].shape, -3.0, np.float32))
    o2, l2 = run_prefill(inputs.PrefillInputs(inp.cfg, inp.q, k2, v2, inp.rng))
    assert np.array_equal(o1[:, :, :300], o2[:, :, :300])
    assert np.array_equal(l1[:, :, :300], l2[:, :, :300])
    assert not np.array_equal(o1[:, :, 300:], o2[:, :, 300:])


def test_runs_are_bitwise_deterministic():
    inp = inputs.custom_prefill(2, 8, 2, 700, 700, 128, True, "bf16", seed=5)
    a, la = run_prefill(inp)
    b, lb = run_prefill(inp)
    assert np.array_equal(a, b) and np.array_equal(la, lb)


def test_lse_optional():
    inp = inputs.custom_prefill(1, 2, 2, 64, 64, 64, True, "bf16", seed=2)
    o1, _ = run_prefill(inp, with_lse=False)
    o2, _ = run_prefill(inp, with_lse=True)
    assert np.array_equal(o1, o2)


# ---- the running reference max: moves, and checks that fail without a move ------------
@pytest.mark.parametrize("pattern", ["rise", "step"])
@pytest.mark.parametrize("B,H,Hkv,N,causal", [
    (2, 32, 8, 1024, True),    # 256 blocks of 256 rows: the ping-pong kernel
    (2, 32, 8, 1024, False),
    (1, 4, 2, 1000, True),     # 16 blocks: the key-split kernel
])
def test_reference_max_moves_and_stays(pattern, B, H, Hkv, N, causal):
    base = inputs.custom_prefill(B, H, Hkv, N, N, 128, causal, "bf16", seed=61)
    inp = shaped_scores(base, pattern)
    rows = {(0, 0): np.arange(N), (B - 1, H - 1): np.arange(N)}
    _sampled_check(inp, rows, f"reference max, {pattern}")


# ---- launch size: an item's result does not depend on what else the launch holds ---------
def _fwd_dev(q, k, v, causal, scale):
    import torch
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    _lib.fa_fwd(q, k, v, o, lse, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return bf16_from_dev(o), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,split", [
    (1, 37, 1, 3600, 64, True, 20),     # 555 items (15 q tiles x 37 heads); parts 300 + 255
    (4, 16, 4, 2100, 128, False, None),  # 576 items, ragged last q tile; per batch 144
    (2, 16, 16, 4096, 128, True, None),  # 512 items; per batch 256
])
def test_large_launch_matches_launches_of_its_parts(B, H, Hkv, N, d, causal, split):
    """A launch of several rounds of work-groups (more (head, q tile) items than compute
    units, ragged tails, counts not a multiple of the XCD count) gives the same bits as
    launches of its parts: each item's arithmetic is independent of the others'."""
    inp = inputs.custom_prefill(B, H, Hkv, N, N, d, causal, "bf16", seed=77)
    _say(f"[prefill] launch parts B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
    o, lse = _fwd_dev(q, k, v, causal, inp.cfg.scale)
    if split is None:  # per batch
        for b in range(B):
            ob, lb = _fwd_dev(q[b:b + 1], k[b:b + 1], v[b:b + 1], causal, inp.cfg.scale)
            assert np.array_equal(o[b:b + 1], ob) and np.array_equal(lse[b:b + 1], lb)
    else:  # by heads (one KV head: both parts read it)
        assert B == 1 and Hkv == 1
        for h0, h1 in ((0, split), (split, H)):
            oh, lh = _fwd_dev(q[:, h0:h1].contiguous(), k, v, causal, inp.cfg.scale)
            assert np.array_equal(o[:, h0:h1], oh) and np.array_equal(lse[:, h0:h1], lh)


def test_many_items_vs_oracle():
    """555 items (not a multiple of 8, ragged last q tile, d = 64) against the oracle in full."""
    _dense_check(inputs.custom_prefill(1, 37, 1, 3600, 3600, 64, True, "bf16", seed=78),
                 "555 items")
