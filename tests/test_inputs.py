"""Seeded input generation: bf16 rounding, determinism, paging layout (CPU only)."""
import numpy as np
import pytest

from kv_cache_fa_amd import inputs


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("bits,want", [
    (0x3F800000, 0x3F80),   # 1.0 exact
    (0x3F808000, 0x3F80),   # halfway, lower neighbour even -> round down
    (0x3F818000, 0x3F82),   # halfway, lower neighbour odd  -> round up to even
    (0x3F808001, 0x3F81),   # just above halfway -> up
    (0x3F807FFF, 0x3F80),   # just below halfway -> down
    (0xBF818000, 0xBF82),   # negative tie -> even (magnitude rounds up)
    (0x00000000, 0x0000),
    (0x80000000, 0x8000),   # -0 keeps its sign
    (0x7F7FFFFF, 0x7F80),   # largest float rounds to +inf under RNE
    (0x00008000, 0x0000),   # subnormal tie -> even (zero)
])
def test_bf16_round_to_nearest_even(bits, want):
    got = inputs.f32_to_bf16_bits(_f32(bits))[0]
    assert int(got) == want


def test_bf16_widen_is_exact_roundtrip():
    rng = np.random.default_rng(0)
    b = inputs.f32_to_bf16_bits(rng.standard_normal(1000, dtype=np.float32))
    assert np.array_equal(inputs.f32_to_bf16_bits(inputs.bf16_bits_to_f32(b)), b)
    x = inputs.bf16_bits_to_f32(b)
    assert np.all(x.view(np.uint32) & 0xFFFF == 0)


def test_prefill_is_deterministic_and_seeded():
    cfg = inputs.PREFILL_CONFIGS["bf16_causal"]
    small = inputs.PrefillConfig("t", 1, 2, 2, 16, 16, 64, True, "bf16", 0.5, 0.125, 2)
    a, b = inputs.make_prefill(small), inputs.make_prefill(small)
    assert a.q.dtype == np.uint16
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    c = inputs.make_prefill(small, seed=3)
    assert not np.array_equal(a.q, c.q)
    # draw order: Q first, from standard_normal(float32), times 0.5, then RNE
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 16, 64), dtype=np.float32) * np.float32(0.5)
    assert np.array_equal(a.q, inputs.f32_to_bf16_bits(q))
    assert cfg.flops == 4 * 64 * 2 * 8 * (1024 * 1025 // 2)


def test_workload_flop_counts():
    c = inputs.PREFILL_CONFIGS
    assert c["gqa_causal"].flops == pytest.approx(549.9e9, rel=1e-3)
    assert c["long_causal"].flops == pytest.approx(35.18e12, rel=1e-3)
    assert c["fp32_single"].flops == 4 * 64 * 128 * 128
    assert inputs.unmasked_pairs(3, 5, True) == 3 + 4 + 5
    assert inputs.unmasked_pairs(4, 4, True) == 10


def test_row_samples_are_seeded_and_distinct():
    small = inputs.PrefillConfig("t", 2, 4, 2, 64, 64, 64, True, "bf16", 1.0, 0.125, 3)
    a = inputs.sample_rows(inputs.make_prefill(small), 2, 50)
    b = inputs.sample_rows(inputs.make_prefill(small), 2, 50)
    assert a.keys() == b.keys()
    assert all(np.array_equal(a[x], b[x]) for x in a)
    full = [x for x in a if len(a[x]) == 64]
    assert len(full) == 2
    assert sum(len(r) for x, r in a.items() if x not in full) == 50


def test_decode_layout():
    inp = inputs.custom_decode(6, 8, 2, 32, 1, 70, page_size=16, max_seq_len=80, seed=5)
    assert inp.page_table.shape == (6, 5)
    assert inp.page_table.dtype == np.int32 and inp.seq_lens.dtype == np.int32
    assert np.all((inp.seq_lens >= 1) & (inp.seq_lens <= 70))
    n_pages = (inp.seq_lens + 15) // 16
    assert inp.num_pages == int(n_pages.sum())
    for s in range(6):
        L = int(inp.seq_lens[s])
        # unused table entries hold the pad value, unused slots hold the fill value
        assert np.all(inp.page_table[s, n_pages[s]:] == 0)
        last = inp.page_table[s, n_pages[s] - 1]
        tail = L - (n_pages[s] - 1) * 16
        assert np.all(inp.k_cache[last, tail:] == 0)
    nan = inputs.custom_decode(2, 4, 1, 8, 5, 5, max_seq_len=16, seed=1, unused_fill="nan",
                               table_pad=-1)
    assert np.all(nan.k_cache[nan.page_table[0, 0], 5:] == inputs.BF16_NAN_BITS)
    assert np.all(nan.page_table[:, 1:] == -1)


def test_decode_zero_length_sequences():
    cfg = inputs.DecodeConfig("z", 3, 4, 2, 8, 0, 0, 16, 32, 0.35, 0)
    inp = inputs.make_decode(cfg, seq_lens=[0, 17, 0])
    assert inp.num_pages == 2
    assert inp.k_seq[0].shape == (0, 2, 8)


def test_paged_decode_config_lengths():
    cfg = inputs.DECODE_CONFIGS["paged_decode"]
    rng = np.random.default_rng(cfg.seed)
    lens = rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.num_seqs, endpoint=True)
    assert lens.min() >= 512 and lens.max() <= 8192


def test_window_pairs_matches_the_mask():
    for Nq, Nk, left, right in ((7, 7, 2, 1), (5, 9, 0, 0), (6, 6, -1, 0), (4, 10, 3, -1),
                                (8, 8, -1, -1), (3, 3, 100, 100)):
        i = np.arange(Nq)[:, None] + (Nk - Nq)
        j = np.arange(Nk)[None, :]
        m = np.ones((Nq, Nk), bool)
        if left >= 0:
            m &= j >= i - left
        if right >= 0:
            m &= j <= i + right
        assert inputs.window_pairs(Nq, Nk, left, right) == int(m.sum())
    assert inputs.window_pairs(6, 6, -1, 0) == inputs.unmasked_pairs(6, 6, True)


# ---- e4m3 codec (OCP fp8: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits) ----
def test_e4m3_known_codes():
    codes = np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x39, 0x3F, 0x7E, 0xC0, 0xFE, 0x80])
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.125, 1.875, 448.0, -2.0, -448.0,
            -0.0]
    np.testing.assert_array_equal(inputs.e4m3_to_f64(codes), want)
    assert np.isnan(inputs.e4m3_to_f64(np.array([0x7F, 0xFF]))).all()


def test_e4m3_encode_is_nearest_with_ties_to_even_and_saturates():
    finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = inputs.e4m3_to_f64(finite)
    # every finite code round-trips (-0 encodes as +0)
    back = inputs.f64_to_e4m3(vals)
    assert np.array_equal(inputs.e4m3_to_f64(back), vals)
    # brute force: random values map to the nearest code, ties to the even code
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(2000) * 30, rng.standard_normal(500) * 0.01,
                        (vals[:-1] + vals[1:])[::7] / 2])       # some exact midpoints
    enc = inputs.e4m3_to_f64(inputs.f64_to_e4m3(x))
    for xi, ei in zip(x, enc):
        d = np.abs(vals - min(max(xi, -448.0), 448.0))
        best = vals[d == d.min()]
        assert ei in best
        if len(set(best)) > 1:   # a tie: the even code wins
            codes = finite[np.isin(vals, best)]
            assert inputs.f64_to_e4m3(np.array([xi]))[0] % 2 == 0 or ei == 0.0, (xi, codes)
    assert inputs.f64_to_e4m3(np.array([1e6]))[0] == 0x7E
    assert inputs.f64_to_e4m3(np.array([-1e6]))[0] == 0xFE


def test_quantized_decode_cache_dequantises_within_half_a_step():
    base = inputs.custom_decode(5, 8, 2, 128, 1, 200, seed=4)
    f = inputs.quantize_decode_fp8(base)
    for cache, qc, sc in ((base.k_cache, f.k_cache, f.k_scale), (base.v_cache, f.v_cache, f.v_scale)):
        x = inputs.bf16_bits_to_f64(cache)
        deq = inputs.e4m3_to_f64(qc) * sc[None, None, :, None]
        # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normal values, and
        # absolute error <= half the subnormal step 2^-10 * scale below them
        err = np.abs(deq - x)
        bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sc[None, None, :, None])
        assert np.all(err <= bound * (1 + 1e-12))
        assert np.abs(inputs.e4m3_to_f64(qc)).max() <= 448.0
