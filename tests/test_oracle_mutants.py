"""Each pin must be able to fail: oracles with one planted mistake (on the CPU).

Every mutant below is the plain attention definition with exactly one plausible
error. The pin suite (tests/pins.py) must reject each of them; a mutant that
passes every pin would mean the pins cannot see that class of mistake.
"""
import numpy as np
import pytest

from pins import ALL_PINS


def _attn(q, k, v, causal, scale, *, scale_fn=None, mask_fn=None, kv_fn=None,
          shift=True, lse_log=np.log, softmax_axis=-1, transpose_k=False):
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    g = H // Hkv
    O = np.zeros((B, H, Nq, d))
    L = np.zeros((B, H, Nq))
    i = np.arange(Nq)[:, None]
    j = np.arange(Nk)[None, :]
    mask = np.ones((Nq, Nk), bool) if not causal else (
        mask_fn(i, j, Nq, Nk) if mask_fn else j <= i + (Nk - Nq))
    for b in range(B):
        for h in range(H):
            kvh = kv_fn(h, H, Hkv) if kv_fn else h // g
            kk = k[b, kvh]
            sc = scale_fn(scale, d) if scale_fn else scale
            if transpose_k and Nk == d:
                S = sc * (q[b, h] @ kk)
            else:
                S = sc * (q[b, h] @ kk.T)
            S = np.where(mask, S, -np.inf)
            m = S.max(axis=softmax_axis, keepdims=True) if shift else np.zeros_like(
                S.max(axis=softmax_axis, keepdims=True))
            with np.errstate(all="ignore"):
                e = np.where(mask, np.exp(S - m), 0.0)
                l = e.sum(axis=softmax_axis, keepdims=True)
                P = e / l
            O[b, h] = P @ v[b, kvh]
            with np.errstate(all="ignore"):
                L[b, h] = (m + lse_log(l)).reshape(-1)[:Nq] if softmax_axis == -1 else \
                    (m + lse_log(l)).reshape(-1)[:Nq]
    return O, L


MUTANTS = {
    "no_scale": dict(scale_fn=lambda s, d: 1.0),
    "sqrt_of_scale": dict(scale_fn=lambda s, d: np.sqrt(s)),
    "scale_squared": dict(scale_fn=lambda s, d: s * s),
    "causal_strict_off_by_one": dict(mask_fn=lambda i, j, Nq, Nk: j < i + (Nk - Nq)),
    "causal_top_left": dict(mask_fn=lambda i, j, Nq, Nk: j <= i),
    "gqa_interleaved_heads": dict(kv_fn=lambda h, H, Hkv: h % Hkv),
    "no_max_shift": dict(shift=False),
    "lse_base2": dict(lse_log=np.log2),
    "softmax_over_queries": dict(softmax_axis=0),
    "k_not_transposed": dict(transpose_k=True),
}


def run_pins(fn):
    failures = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as e:
            failures.append((pin.__name__, type(e).__name__))
    return failures


def test_unmutated_reference_passes_every_pin():
    assert run_pins(lambda q, k, v, causal, scale: _attn(q, k, v, causal, scale)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    kw = MUTANTS[name]
    fails = run_pins(lambda q, k, v, causal, scale: _attn(q, k, v, causal, scale, **kw))
    assert fails, f"mutant {name} passed every pin"
