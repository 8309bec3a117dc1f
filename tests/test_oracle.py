"""The fp64 oracle checked against what the pages and the mathematics fix (CPU only)."""
import math

import numpy as np
import pytest

import oracle
from scipy.special import logsumexp as scipy_logsumexp
from scipy.special import softmax as scipy_softmax
from oracle.brute import attention_brute
from kv_cache_fa_amd import inputs
from pins import ALL_PINS, load_golden, parse_arr, parse_num


def dense_attn(q, k, v, causal, scale):
    return oracle.attention(q, k, v, causal=causal, scale=scale)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(dense_attn)


def test_rows_mode_matches_dense():
    rng = np.random.default_rng(1)
    q, k, v = (rng.standard_normal(s) for s in [(2, 4, 9, 8), (2, 2, 9, 8), (2, 2, 9, 8)])
    O, L = oracle.attention(q, k, v, causal=True, scale=0.3)
    rows = {(1, 3): np.array([0, 4, 8]), (0, 0): np.arange(9)}
    Or, Lr = oracle.attention(q, k, v, causal=True, scale=0.3, rows=rows)
    for (b, h), idx in rows.items():
        np.testing.assert_array_equal(Or[(b, h)], O[b, h, idx])
        np.testing.assert_array_equal(Lr[(b, h)], L[b, h, idx])


def test_probability_rows_sum_to_one_and_respect_mask():
    """Each softmax row is a probability distribution over the allowed keys."""
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal(s) * 3 for s in [(1, 2, 7, 4), (1, 1, 11, 4), (1, 1, 11, 4)])
    for causal in (False, True):
        _, _, P = oracle.attention(q, k, v, causal=causal, scale=1.0, return_probs=True)
        mask = oracle.allowed_keys(7, 11, causal)
        for p in P.values():
            np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-13)
            assert np.all(p[~mask] == 0.0)
            assert np.all(p[mask] > 0.0)


def test_softmax_shift_of_score_rows():
    """softmax(x) = softmax(x - c): adding a per-row constant leaves P unchanged."""
    rng = np.random.default_rng(3)
    s = rng.standard_normal((5, 9)) * 4
    c = rng.standard_normal((5, 1)) * 50
    mask = np.ones_like(s, dtype=bool)
    P1, m1, l1 = oracle.softmax_rows(s, mask)
    P2, m2, l2 = oracle.softmax_rows(s + c, mask)
    np.testing.assert_allclose(P2, P1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=1e-13)
    np.testing.assert_allclose(m2, m1 + c[:, 0], rtol=0, atol=1e-12)


# ---- online softmax (the pages' recurrence) and the log-sum-exp merge ------------
def test_online_softmax_golden_steps():
    g = load_golden("online_softmax.json")
    for ex in g["stats"]:
        scores = [parse_num(x) for x in ex["scores"]]
        trace = []
        M, L = oracle.online_softmax_stats(scores, ex["blocks"], trace=trace)
        assert len(trace) == len(ex["steps"])
        for got, want in zip(trace, ex["steps"]):
            for key in ("m_new", "l_block", "M", "L"):
                assert got[key] == pytest.approx(parse_num(want[key]), abs=1e-14), key
            if "L_old_rescaled" in want:
                assert got["L_old_rescaled"] == pytest.approx(want["L_old_rescaled"], abs=1e-14)
        assert M == pytest.approx(parse_num(ex["M"]), abs=1e-14)
        assert L == pytest.approx(ex["L"], abs=1e-14)


def test_merge_golden():
    m = load_golden("online_softmax.json")["merge"]
    O, LSE = oracle.merge_partials(parse_arr(m["o_parts"]), parse_arr(m["lse_parts"]))
    np.testing.assert_allclose(O, parse_arr(m["O"]), rtol=0, atol=1e-13)
    assert LSE == pytest.approx(parse_num(m["LSE"]), abs=1e-14)


@pytest.mark.parametrize("seed", range(5))
def test_online_recurrence_equals_definition(seed):
    """Any blocking of the row gives the whole-row softmax statistics and output."""
    rng = np.random.default_rng(100 + seed)
    N, d = 37, 6
    s = rng.standard_normal(N) * 5
    v = rng.standard_normal((N, d))
    cuts = np.sort(rng.choice(np.arange(1, N), size=rng.integers(1, 8), replace=False))
    blocks = np.diff(np.concatenate([[0], cuts, [N]])).tolist()
    M, L = oracle.online_softmax_stats(s, blocks)
    P, m, l = oracle.softmax_rows(s[None], np.ones((1, N), dtype=bool))
    assert M == m[0]
    assert L == pytest.approx(l[0], rel=1e-13)
    o, lse = oracle.online_attention_row(s, v, blocks)
    np.testing.assert_allclose(o, P[0] @ v, rtol=0, atol=1e-12)
    assert lse == pytest.approx(m[0] + math.log(l[0]), abs=1e-12)


@pytest.mark.parametrize("seed", range(5))
def test_merge_of_splits_equals_whole(seed):
    """Attention over disjoint key sets, merged by log-sum-exp, equals the whole row;
    empty parts (LSE = -inf) weigh nothing."""
    rng = np.random.default_rng(200 + seed)
    Nk, d = 50, 8
    q = rng.standard_normal((1, 1, 1, d)) * 2
    k = rng.standard_normal((1, 1, Nk, d))
    v = rng.standard_normal((1, 1, Nk, d))
    O, L = oracle.attention(q, k, v, causal=False, scale=0.5)
    cuts = np.sort(rng.choice(np.arange(1, Nk), size=4, replace=False))
    parts = np.split(np.arange(Nk), cuts)
    os_, ls_ = [], []
    for idx in parts:
        o, l = oracle.attention(q, k[:, :, idx], v[:, :, idx], causal=False, scale=0.5)
        os_.append(o[0, 0, 0])
        ls_.append(l[0, 0, 0])
    os_.append(np.full(d, 123.0))      # an empty split: its output must not matter
    ls_.append(-np.inf)
    Om, Lm = oracle.merge_partials(os_, ls_)
    np.testing.assert_allclose(Om, O[0, 0, 0], rtol=0, atol=1e-12)
    assert Lm == pytest.approx(L[0, 0, 0], abs=1e-12)


def test_merge_all_empty():
    O, L = oracle.merge_partials(np.zeros((3, 4)), [-np.inf] * 3)
    assert L == -np.inf and np.all(O == 0)


# ---- decode against a paged cache ----------------------------------------------
def test_decode_equals_last_row_of_causal_prefill():
    """The decode query is the newest token: its result is the last row of a causal
    prefill over the same keys (glossary entry 'KV Cache')."""
    rng = np.random.default_rng(4)
    S, H, Hkv, d = 3, 8, 2, 16
    lens = [1, 7, 40]
    ks = [rng.standard_normal((L, Hkv, d)) for L in lens]
    vs = [rng.standard_normal((L, Hkv, d)) for L in lens]
    q = rng.standard_normal((S, H, d))
    O, LSE = oracle.decode(q, ks, vs, scale=0.25)
    for s, L in enumerate(lens):
        qq = np.zeros((1, H, L, d))
        qq[0, :, -1] = q[s]
        kk = ks[s].transpose(1, 0, 2)[None]
        vv = vs[s].transpose(1, 0, 2)[None]
        Op, Lp = oracle.attention(qq, kk, vv, causal=True, scale=0.25)
        np.testing.assert_allclose(O[s], Op[0, :, -1], rtol=0, atol=1e-13)
        np.testing.assert_allclose(LSE[s], Lp[0, :, -1], rtol=0, atol=1e-13)


def test_decode_empty_sequence():
    q = np.ones((2, 4, 8))
    ks = [np.zeros((0, 2, 8)), np.ones((3, 2, 8))]
    O, LSE = oracle.decode(q, ks, ks, scale=1.0)
    assert np.all(O[0] == 0) and np.all(LSE[0] == -np.inf)
    np.testing.assert_allclose(O[1], 1.0)
    np.testing.assert_allclose(LSE[1], 8.0 + math.log(3))


def test_gather_pages_is_bit_exact_and_table_is_a_permutation():
    inp = inputs.custom_decode(5, 8, 2, 16, 1, 100, page_size=16, max_seq_len=100, seed=7)
    n_pages = (inp.seq_lens + 15) // 16
    used = np.concatenate([inp.page_table[s, :n_pages[s]] for s in range(5)])
    assert np.array_equal(np.sort(used), np.arange(int(n_pages.sum())))
    for cache, seqs in ((inp.k_cache, inp.k_seq), (inp.v_cache, inp.v_seq)):
        got = oracle.gather_pages(cache, inp.page_table, inp.seq_lens, 16)
        for a, b in zip(got, seqs):
            assert a.dtype == b.dtype == np.uint16
            assert np.array_equal(a, b)


def test_gather_pages_detects_a_wrong_slot():
    """A one-token shift of the slot index is caught bit-exactly."""
    inp = inputs.custom_decode(2, 4, 1, 8, 20, 40, page_size=16, max_seq_len=40, seed=8)
    s, L = 0, int(inp.seq_lens[0])
    t = np.arange(L)
    wrong = inp.k_cache[inp.page_table[s, t // 16], (t + 1) % 16]
    assert not np.array_equal(wrong, inp.k_seq[s])


# ---- backward pass (analytic gradients, pinned by central differences) ------------
def _loss(q, k, v, w, causal, scale, window=None):
    O, _ = oracle.attention(q, k, v, causal=causal, scale=scale, window=window)
    return float(np.sum(O * w))


@pytest.mark.parametrize("causal,window,Hkv", [(False, None, 2), (True, None, 1),
                                                (False, (1, 2), 2)])
def test_backward_matches_central_differences(causal, window, Hkv):
    """d(sum(O * W))/dX by central differences equals the analytic gradient with dO = W
    (an independent check of every term: a dropped term, a sign or a transpose fails)."""
    rng = np.random.default_rng(3)
    B, H, Nq, Nk, d = 1, 2, 4, 5, 3
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    w = rng.standard_normal((B, H, Nq, d))
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, w, causal=causal, scale=scale, window=window)
    eps = 1e-6
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            f1 = _loss(q, k, v, w, causal, scale, window)
            x[idx] = old - eps
            f0 = _loss(q, k, v, w, causal, scale, window)
            x[idx] = old
            num[idx] = (f1 - f0) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=0, atol=2e-8)


def test_backward_closed_forms():
    """Uniform attention (K = 0) over equal V rows: dV_j = sum_i dO_i / Nk and, since
    every dP row is constant, dS = 0, so dQ = dK = 0."""
    rng = np.random.default_rng(5)
    Nq, Nk, d = 3, 4, 2
    q = rng.standard_normal((1, 1, Nq, d))
    k = np.zeros((1, 1, Nk, d))
    v = np.tile(rng.standard_normal((1, 1, 1, d)), (1, 1, Nk, 1))
    do = rng.standard_normal((1, 1, Nq, d))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal=False, scale=0.5)
    np.testing.assert_allclose(dv[0, 0], np.tile(do[0, 0].sum(0) / Nk, (Nk, 1)), atol=1e-15)
    np.testing.assert_allclose(dq, 0.0, atol=1e-15)
    np.testing.assert_allclose(dk, 0.0, atol=1e-15)


# ---- FlashAttention-1 two passes ---------------------------------------------------
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_two_pass_equals_definition(seed):
    """Statistics pass + normalised output pass = softmax(s) @ v, any blocking."""
    rng = np.random.default_rng(seed)
    n, d = 37, 5
    s = rng.standard_normal(n) * 3
    v = rng.standard_normal((n, d))
    cuts = sorted(rng.choice(np.arange(1, n), size=4, replace=False))
    blocks = np.diff([0, *cuts, n]).tolist()
    o, lse = oracle.two_pass_attention_row(s, v, blocks)
    p = scipy_softmax(s)
    np.testing.assert_allclose(o, p @ v, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, scipy_logsumexp(s), rtol=0, atol=1e-13)


def test_two_pass_statistics_are_the_golden_trace():
    """Pass 1 keeps exactly the page's (M, L) for the hand-worked row."""
    g = load_golden("online_softmax.json")
    for case in g["stats"]:
        s = parse_arr(case["scores"])
        M, L = parse_num(case["M"]), parse_num(case["L"])
        o, lse = oracle.two_pass_attention_row(s, np.eye(len(s)), case["blocks"])
        np.testing.assert_allclose(lse, M + math.log(L), rtol=0, atol=1e-14)
        # V = I, so o is the probability row: [1, 2, 4] / 7
        np.testing.assert_allclose(o, np.array([1, 2, 4]) / 7, rtol=0, atol=1e-14)


# ---- sliding window (glossary entry "Kayan Pencere Dikkati") -----------------------
def _rand_qkv(rng, B, H, Hkv, Nq, Nk, d):
    return (rng.standard_normal((B, H, Nq, d)), rng.standard_normal((B, Hkv, Nk, d)),
            rng.standard_normal((B, Hkv, Nk, d)))


def test_window_zero_attends_only_itself():
    """Window (0, 0): each query sees only its own position p = Nk - Nq + i, so
    O = V[p] exactly and LSE = scale * q . k_p."""
    rng = np.random.default_rng(0)
    q, k, v = _rand_qkv(rng, 2, 4, 2, 5, 9, 8)
    O, L = oracle.attention(q, k, v, causal=False, scale=0.3, window=(0, 0))
    for b in range(2):
        for h in range(4):
            for i in range(5):
                p = 9 - 5 + i
                np.testing.assert_array_equal(O[b, h, i], v[b, h // 2, p])
                np.testing.assert_allclose(L[b, h, i], 0.3 * q[b, h, i] @ k[b, h // 2, p],
                                           rtol=0, atol=1e-13)


@pytest.mark.parametrize("window", [(2, 1), (0, 3), (3, 0), (1, -1), (-1, 2), (4, 4)])
def test_window_brute_force(window):
    rng = np.random.default_rng(sum(window) + 10)
    q, k, v = _rand_qkv(rng, 1, 2, 1, 5, 7, 4)
    O, L = oracle.attention(q, k, v, causal=False, scale=0.5, window=window)
    Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), False, 0.5, window=window)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-13)


def test_window_row_equals_attention_over_its_slice():
    """A windowed row is plain (unmasked) attention over keys p-left .. p+right."""
    rng = np.random.default_rng(4)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 12, 20, 8)
    left, right = 5, 2
    O, L = oracle.attention(q, k, v, causal=False, scale=0.4, window=(left, right))
    for i in range(12):
        p = 20 - 12 + i
        lo, hi = max(0, p - left), min(20, p + right + 1)
        Os, Ls = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi],
                                  causal=False, scale=0.4)
        np.testing.assert_allclose(O[0, 0, i], Os[0, 0, 0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(L[0, 0, i], Ls[0, 0, 0], rtol=0, atol=1e-14)


def test_window_limits_are_causal_and_full():
    """(-1, 0) is bottom-right causal and (-1, -1) is no mask."""
    rng = np.random.default_rng(5)
    q, k, v = _rand_qkv(rng, 1, 2, 2, 6, 10, 4)
    for window, causal in (((-1, 0), True), ((-1, -1), False)):
        Ow, Lw = oracle.attention(q, k, v, causal=False, scale=0.7, window=window)
        Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), causal, 0.7)
        np.testing.assert_allclose(Ow, np.array(Ob), rtol=0, atol=1e-13)
        np.testing.assert_allclose(Lw, np.array(Lb), rtol=0, atol=1e-13)


def test_window_pins_catch_an_off_by_one_edge():
    """A window mask with either edge moved by one key fails the slice pin."""
    rng = np.random.default_rng(6)
    q, k, v = _rand_qkv(rng, 1, 1, 1, 8, 12, 4)
    left, right = 3, 1
    for dl, dr in ((1, 0), (-1, 0), (0, 1), (0, -1)):
        O, _ = oracle.attention(q, k, v, causal=False, scale=0.4, window=(left + dl, right + dr))
        bad = False
        for i in range(8):
            p = 12 - 8 + i
            lo, hi = max(0, p - left), min(12, p + right + 1)
            Os, _ = oracle.attention(q[:, :, i:i + 1], k[:, :, lo:hi], v[:, :, lo:hi],
                                     causal=False, scale=0.4)
            bad |= not np.allclose(O[0, 0, i], Os[0, 0, 0], rtol=0, atol=1e-12)
        assert bad, (dl, dr)


def test_scatter_pages_hand_worked():
    """Hand-placed tokens (page size 4, one head, d = 1): seq 0 starts at position 3,
    so its tokens go to page 2 slot 3 and page 0 slot 0; seq 1 at position 2 fills
    page 1 slots 2-3; a third sequence's tokens hit an unassigned entry (-1) and then
    run past the table, and are dropped."""
    cache = np.zeros((3, 4, 1, 1))
    table = np.array([[2, 0], [1, -1], [0, -1]], dtype=np.int32)
    new = np.array([[10, 11], [20, 21], [30, 31]], dtype=np.float64).reshape(3, 2, 1, 1)
    got = oracle.scatter_pages(cache, table, [3, 2, 7], new, 4)
    want = np.array([[11, 0, 0, 0], [0, 0, 20, 21], [0, 0, 0, 10]], dtype=np.float64)
    assert np.array_equal(got[:, :, 0, 0], want)
    assert np.all(cache == 0)  # the input is not modified


@pytest.mark.parametrize("seed", [0, 1])
def test_scatter_then_gather_round_trip(seed):
    """After appending, reading each sequence back through the table yields its old
    tokens followed by the new ones; pages nobody owns are untouched."""
    a = inputs.make_append(6, 37, 2, 16, 200, seed=seed)
    P = 16
    n_new = a.k_new.shape[1]
    old_lens = a.start_pos
    old = oracle.gather_pages(a.k_cache, a.page_table, old_lens, P)
    got = oracle.scatter_pages(a.k_cache, a.page_table, a.start_pos, a.k_new, P)
    back = oracle.gather_pages(got, a.page_table, old_lens + n_new, P)
    for s in range(6):
        assert np.array_equal(back[s][:old_lens[s]], old[s])
        assert np.array_equal(back[s][old_lens[s]:], a.k_new[s])
    owned = set(int(x) for x in a.page_table.ravel() if x >= 0)
    for pid in range(a.k_cache.shape[0]):
        if pid not in owned:
            assert np.array_equal(got[pid], a.k_cache[pid])
    # exactly n_new token rows changed per sequence (new values differ from old bits)
    changed = np.any(got != a.k_cache, axis=(2, 3)).sum()
    assert changed <= 6 * n_new


def test_size_facts_from_the_pages():
    """The pages' printed sizes agree with the counting used for measurement."""
    facts = load_golden("size_facts.json")["facts"]
    n128k, n8k, kv = facts
    assert n128k["tokens"] ** 2 == n128k["value"]
    assert abs(n128k["value"] - 16.4e9) / 16.4e9 <= n128k["rel_tol"]
    assert n8k["tokens"] ** 2 == n8k["value"]
    assert abs(n8k["value"] - 67e6) / 67e6 <= n8k["rel_tol"]
    b = 2 * kv["layers"] * kv["kv_heads"] * kv["head_dim"] * kv["tokens"] * kv["bytes_per_value"]
    assert b == kv["value"]
    assert abs(b - 500e6) / 500e6 <= kv["rel_tol"]
    # one layer of the decode workload's K+V for a sequence of L tokens, as counted by
    # DecodeInputs.kv_bytes: 2 (K,V) x Hkv x d x L x 2 bytes
    inp = inputs.custom_decode(3, 8, 8, 128, 4096, 4096, max_seq_len=4096, seed=0)
    assert inp.kv_bytes() * kv["layers"] == 3 * kv["value"]
