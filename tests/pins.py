"""Checks that pin an attention implementation to facts fixed outside it.

Each ``pin_*`` function takes ``attn(q, k, v, causal=..., scale=...) -> (O, LSE)``
(dense float64 arrays, q [B,H,Nq,d], k/v [B,Hkv,Nk,d]) and raises AssertionError
when the implementation disagrees with the pages, a closed form, an invariant of
softmax, a library routine or a pure-Python brute force. The oracle must pass all
of them; the mutant oracles in ``test_oracle_mutants.py`` (each with one planted
mistake) must each fail at least one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special

from oracle.brute import attention_brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def parse_num(x):
    """Golden values: numbers, 'lnN' (natural log of N) or 'a/b' fractions."""
    if isinstance(x, (int, float)):
        return float(x)
    if x.startswith("ln"):
        return math.log(float(x[2:]))
    if "/" in x:
        a, b = x.split("/")
        return float(a) / float(b)
    return float(x)


def parse_arr(x):
    if isinstance(x, list):
        return np.array([parse_arr(e) for e in x], dtype=np.float64)
    return parse_num(x)


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand(rng, *shape, scale=1.0):
    return rng.standard_normal(shape) * scale


# --------------------------------------------------------------------------------
def pin_golden_closed_forms(attn):
    """Hand-derived tiny cases (tests/golden/closed_forms.json)."""
    g = load_golden("closed_forms.json")
    for case in g["cases"]:
        q, k, v = parse_arr(case["q"]), parse_arr(case["k"]), parse_arr(case["v"])
        O, LSE = attn(q, k, v, causal=case["causal"], scale=case["scale"])
        np.testing.assert_allclose(O, parse_arr(case["O"]), rtol=0, atol=1e-12,
                                   err_msg=case["name"])
        np.testing.assert_allclose(LSE, parse_arr(case["LSE"]), rtol=0, atol=1e-12,
                                   err_msg=case["name"])


def pin_shift_invariance(attn):
    """Adding u to every key shifts row i's scores by the constant scale*q_i.u.

    softmax(x) = softmax(x - c) (page "Donanıma Duyarlı Algoritma Tasarımı:
    FlashAttention", section "FlashAttention'ın Temelleri"), so O is unchanged and
    LSE moves by exactly that constant. u is dyadic so K + u is exact.
    """
    rng = np.random.default_rng(11)
    B, H, Hkv, N, d = 2, 4, 2, 13, 8
    q = _rand(rng, B, H, N, d)
    k = _rand(rng, B, Hkv, N, d)
    v = _rand(rng, B, Hkv, N, d)
    u = np.array([0.5, -1.25, 2.0, 0.0, -0.75, 1.5, 0.25, -2.5])
    scale = 0.375
    for causal in (False, True):
        O1, L1 = attn(q, k, v, causal=causal, scale=scale)
        O2, L2 = attn(q, k + u, v, causal=causal, scale=scale)
        np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-12)
        shift = scale * (q @ u)
        np.testing.assert_allclose(L2, L1 + shift, rtol=0, atol=1e-11)


def pin_zero_query_means(attn):
    """Q = 0 gives equal weights: O_i = mean of the V rows row i attends; LSE = ln |A_i|."""
    rng = np.random.default_rng(12)
    B, H, Hkv, d = 1, 2, 1, 5
    for (Nq, Nk) in ((9, 9), (4, 11)):
        q = np.zeros((B, H, Nq, d))
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        O, L = attn(q, k, v, causal=False, scale=0.3)
        np.testing.assert_allclose(O[0, 1], np.broadcast_to(v[0, 0].mean(0), (Nq, d)),
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(L, math.log(Nk), rtol=0, atol=1e-13)
        O, L = attn(q, k, v, causal=True, scale=0.3)
        for i in range(Nq):
            n = i + (Nk - Nq) + 1
            np.testing.assert_allclose(O[0, 0, i], v[0, 0, :n].mean(0), rtol=0, atol=1e-13)
            np.testing.assert_allclose(L[0, 0, i], math.log(n), rtol=0, atol=1e-13)


def pin_peaked_selects_one_row(attn):
    """Near one-hot scores: every other exp underflows to 0 so O_i is exactly V_t(i).

    Keys are 900 * basis vectors; q_i = key t(i), scale 1: the chosen score is
    810000 and every other is 0, so exp(0 - 810000) = 0 in float64 and the result
    is the selected value row bit for bit. Also catches a missing max shift (exp
    of 810000 overflows).
    """
    rng = np.random.default_rng(13)
    Nk = d = 8
    k = (900.0 * np.eye(d))[None, None]                 # [1,1,Nk,d]
    v = _rand(rng, 1, 1, Nk, d)
    t = rng.permutation(Nk)
    q = k[0, 0][t][None, None]                           # query i points at key t[i]
    O, L = attn(q, k, v, causal=False, scale=1.0)
    assert np.array_equal(O[0, 0], v[0, 0][t]), "peaked row did not select its V row"
    np.testing.assert_allclose(L[0, 0], 810000.0, rtol=0, atol=1e-9)


def pin_causal_structure(attn):
    """Causal facts: row 0 of a square problem is V_0; future keys do not matter;
    the last row of a square causal problem equals the non-causal one."""
    rng = np.random.default_rng(14)
    B, H, Hkv, N, d = 1, 2, 2, 10, 6
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    O, L = attn(q, k, v, causal=True, scale=0.5)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-13)
    On, Ln = attn(q, k, v, causal=False, scale=0.5)
    np.testing.assert_allclose(O[:, :, -1], On[:, :, -1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[:, :, -1], Ln[:, :, -1], rtol=0, atol=1e-13)
    for i in (0, 3, 7):
        k2, v2 = k.copy(), v.copy()
        k2[:, :, i + 1:] = _rand(rng, B, Hkv, N - i - 1, d) * 5
        v2[:, :, i + 1:] = _rand(rng, B, Hkv, N - i - 1, d) * 5
        O2, L2 = attn(q, k2, v2, causal=True, scale=0.5)
        np.testing.assert_array_equal(O2[:, :, :i + 1], O[:, :, :i + 1])
        np.testing.assert_array_equal(L2[:, :, :i + 1], L[:, :, :i + 1])
        assert not np.allclose(O2[:, :, -1], O[:, :, -1])


def pin_brute_force(attn):
    """Equal (1e-12) to the pure-Python triple loop on tiny shapes."""
    rng = np.random.default_rng(15)
    shapes = [
        # B, H, Hkv, Nq, Nk, d
        (1, 1, 1, 1, 1, 1), (1, 1, 1, 2, 2, 2), (2, 2, 1, 3, 3, 4), (1, 4, 2, 5, 5, 8),
        (2, 4, 4, 3, 8, 2), (1, 2, 1, 1, 5, 4), (1, 4, 1, 8, 8, 1), (2, 2, 2, 2, 3, 8),
    ]
    for (B, H, Hkv, Nq, Nk, d) in shapes:
        q = _rand(rng, B, H, Nq, d)
        k = _rand(rng, B, Hkv, Nk, d)
        v = _rand(rng, B, Hkv, Nk, d)
        scale = float(rng.uniform(0.2, 1.5))
        for causal in (False, True):
            if causal and Nq > Nk:
                continue
            O, L = attn(q, k, v, causal=causal, scale=scale)
            Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), causal, scale)
            np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
            np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)


def pin_small_closed_forms(attn):
    """N = 1: O = V_0, LSE = s_0.  N = 2: O = sigmoid(s0-s1) V0 + sigmoid(s1-s0) V1,
    LSE = logaddexp(s0, s1)."""
    rng = np.random.default_rng(16)
    d = 7
    q, k, v = _rand(rng, 1, 3, 1, d), _rand(rng, 1, 3, 2, d), _rand(rng, 1, 3, 2, d)
    O, L = attn(q, k[:, :, :1], v[:, :, :1], causal=False, scale=0.4)
    np.testing.assert_array_equal(O[0, :, 0], v[0, :, 0])
    np.testing.assert_allclose(L[0, :, 0], 0.4 * np.sum(q[0, :, 0] * k[0, :, 0], -1), atol=1e-14)
    O, L = attn(q, k, v, causal=False, scale=0.4)
    s = 0.4 * np.einsum("hd,hjd->hj", q[0, :, 0], k[0])
    w0 = 1.0 / (1.0 + np.exp(s[:, 1] - s[:, 0]))
    w1 = 1.0 / (1.0 + np.exp(s[:, 0] - s[:, 1]))
    np.testing.assert_allclose(O[0, :, 0], w0[:, None] * v[0, :, 0] + w1[:, None] * v[0, :, 1],
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(L[0, :, 0], np.logaddexp(s[:, 0], s[:, 1]), rtol=0, atol=1e-13)


def pin_gqa_equals_repeated_heads(attn):
    """Grouped heads equal plain multi-head attention on K/V repeated per group."""
    rng = np.random.default_rng(17)
    B, H, Hkv, N, d = 2, 8, 2, 6, 4
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, Hkv, N, d), _rand(rng, B, Hkv, N, d)
    g = H // Hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    for causal in (False, True):
        O1, L1 = attn(q, k, v, causal=causal, scale=0.6)
        O2, L2 = attn(q, kr, vr, causal=causal, scale=0.6)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(L1, L2)


def pin_key_permutation(attn):
    """Non-causal attention does not depend on the order of the (K_j, V_j) pairs."""
    rng = np.random.default_rng(18)
    B, H, N, d = 1, 2, 12, 5
    q, k, v = _rand(rng, B, H, N, d), _rand(rng, B, H, N, d), _rand(rng, B, H, N, d)
    p = rng.permutation(N)
    O1, L1 = attn(q, k, v, causal=False, scale=0.7)
    O2, L2 = attn(q, k[:, :, p], v[:, :, p], causal=False, scale=0.7)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L2, L1, rtol=0, atol=1e-13)


def pin_scipy_rows(attn):
    """Rows agree with scipy.special.softmax / logsumexp applied to the score rows."""
    rng = np.random.default_rng(19)
    B, H, Hkv, Nq, Nk, d = 1, 2, 1, 6, 9, 3
    q, k, v = _rand(rng, B, H, Nq, d), _rand(rng, B, Hkv, Nk, d), _rand(rng, B, Hkv, Nk, d)
    scale = 0.9
    O, L = attn(q, k, v, causal=False, scale=scale)
    for h in range(H):
        s = scale * q[0, h] @ k[0, 0].T
        np.testing.assert_allclose(O[0, h], scipy.special.softmax(s, axis=1) @ v[0, 0],
                                   rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[0, h], scipy.special.logsumexp(s, axis=1), rtol=0,
                                   atol=1e-13)


ALL_PINS = [
    pin_golden_closed_forms,
    pin_shift_invariance,
    pin_zero_query_means,
    pin_peaked_selects_one_row,
    pin_causal_structure,
    pin_brute_force,
    pin_small_closed_forms,
    pin_gqa_equals_repeated_heads,
    pin_key_permutation,
    pin_scipy_rows,
]
