"""fa_decode_paged_noalloc (the decode workspace in the library's static device array)
against fa_decode_paged (caller's workspace) and the fp64 oracle, through the C ABI.

Two calls in a row on the same device, the second with a smaller workload, so the second
call runs on the array the first one left behind; each result must be bit-identical to
fa_decode_paged's on the same inputs (same kernels) and within the bf16 bar of the
oracle. A request beyond the array's size is refused before anything is enqueued.
"""
import math
import sys

import numpy as np
import pytest

import oracle
from kv_cache_fa_amd import _lib, inputs
from gpu_helpers import DecodeDev, bf16_from_dev, check_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle(inp):
    return oracle.decode(inputs.bf16_bits_to_f64(inp.q),
                         [inputs.bf16_bits_to_f64(x) for x in inp.k_seq],
                         [inputs.bf16_bits_to_f64(x) for x in inp.v_seq], scale=inp.cfg.scale)


def _run_both(inp, what):
    import torch
    c = inp.cfg
    _say(f"[noalloc] {what}: S{c.num_seqs} H{c.H} Hkv{c.Hkv} d{c.d} max_seq_len {c.max_seq_len}")
    dd = DecodeDev(inp)
    dd.run()
    o_ws, lse_ws = dd.result()
    o = torch.full_like(dd.q, float("nan"))
    lse = torch.full_like(dd.lse, float("nan"))
    _lib.fa_decode_paged_noalloc(dd.q, dd.kc, dd.vc, dd.pt, dd.sl, o, lse,
                                 max_seq_len=c.max_seq_len, scale=c.scale)
    torch.cuda.synchronize()
    o_na, lse_na = bf16_from_dev(o), lse.cpu().numpy()
    assert np.array_equal(o_na, o_ws), f"{what}: O differs from fa_decode_paged"
    assert np.array_equal(lse_na, lse_ws), f"{what}: lse differs from fa_decode_paged"
    O, L = _oracle(inp)
    check_bf16(inputs.bf16_bits_to_f64(o_na), lse_na, O, L, what)


def test_noalloc_two_calls_second_smaller():
    # First: 96 sequences (the planning kernel's path), H32 Hkv8 d128, up to 4000 tokens.
    rng = np.random.default_rng(5)
    lens = [int(x) for x in rng.integers(0, 4000, 96)]
    cfg = inputs.DecodeConfig("na1", 96, 32, 8, 128, 0, 0, 16, 4000, 1 / math.sqrt(128), 5)
    _run_both(inputs.make_decode(cfg, seq_lens=lens), "first call")
    # Second, smaller: 6 sequences, H16 Hkv2 d64, up to 700 tokens (one empty).
    cfg = inputs.DecodeConfig("na2", 6, 16, 2, 64, 0, 0, 16, 700, 1 / 8, 6)
    _run_both(inputs.make_decode(cfg, seq_lens=[700, 0, 1, 33, 512, 129]), "second call")


def test_noalloc_full_decode_workload():
    """The 64-sequence decode workload (H32 Hkv8 d128, lengths U{512..8192})."""
    _run_both(inputs.make_decode(inputs.DECODE_CONFIGS["paged_decode"]), "paged_decode")


def test_noalloc_refuses_requests_beyond_its_scratch():
    """A workspace need above FA_NOALLOC_SCRATCH_BYTES gives FA_ERR_SCRATCH, output
    untouched."""
    import torch
    S, H, Hkv, d, L = 256, 32, 8, 128, 8192
    assert _lib.fa_decode_paged_workspace_size(S, H, d, L) > _lib.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((S, H, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 16, Hkv, d), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((S, L // 16), dtype=torch.int32, device="cuda")
    sl = torch.zeros((S,), dtype=torch.int32, device="cuda")
    o = torch.full_like(q, 7.0)
    st = _lib.lib().fa_decode_paged_noalloc(q.data_ptr(), kc.data_ptr(), kc.data_ptr(),
                                            pt.data_ptr(), sl.data_ptr(), 16, o.data_ptr(),
                                            None, S, H, Hkv, d, 4, L // 16, L, 0.088, None)
    torch.cuda.synchronize()
    assert st == _lib.FA_ERR_SCRATCH
    assert torch.all(o == 7.0)
