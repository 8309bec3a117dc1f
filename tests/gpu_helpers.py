"""Helpers for the GPU parity tests: move seeded inputs to the device, run the HIP
path through the C ABI, bring results back, compare with the oracle."""
from __future__ import annotations

import math

import numpy as np

from kv_cache_fa_amd import _lib, inputs

# Tolerances (GPU vs the fp64 oracle on the same stored inputs).
FP32_MAX_ABS = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def torch_dev():
    import torch
    return torch


def bf16_to_dev(bits: np.ndarray):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bf16_from_dev(t) -> np.ndarray:
    torch = torch_dev()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def run_prefill(inp: inputs.PrefillInputs, with_lse=True):
    """Run fa_fwd / fa_fwd_fp32 on the inputs. Returns (O bits/f32, LSE f32) on host."""
    torch = torch_dev()
    c = inp.cfg
    if c.dtype == "f32":
        q, k, v = (torch.from_numpy(x).cuda() for x in (inp.q, inp.k, inp.v))
        o = torch.empty_like(q)
    else:
        q, k, v = (bf16_to_dev(x) for x in (inp.q, inp.k, inp.v))
        o = torch.empty_like(q)
    lse = torch.empty((c.B, c.H, c.Nq), dtype=torch.float32, device="cuda") if with_lse else None
    if c.dtype == "f32":
        _lib.fa_fwd_fp32(q, k, v, o, lse, causal=c.causal, scale=c.scale)
    else:
        _lib.fa_fwd(q, k, v, o, lse, causal=c.causal, scale=c.scale)
    torch.cuda.synchronize()
    o_h = o.cpu().numpy() if c.dtype == "f32" else bf16_from_dev(o)
    return o_h, (lse.cpu().numpy() if with_lse else None)


def widen_out(o_h: np.ndarray, dtype: str) -> np.ndarray:
    return o_h.astype(np.float64) if dtype == "f32" else inputs.bf16_bits_to_f64(o_h)


class DecodeDev:
    """A decode workload resident on the device."""

    def __init__(self, inp: inputs.DecodeInputs):
        torch = torch_dev()
        self.inp = inp
        c = inp.cfg
        self.q = bf16_to_dev(inp.q)
        self.kc = bf16_to_dev(inp.k_cache)
        self.vc = bf16_to_dev(inp.v_cache)
        self.pt = torch.from_numpy(inp.page_table).cuda()
        self.sl = torch.from_numpy(inp.seq_lens).cuda()
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((c.num_seqs, c.H), dtype=torch.float32, device="cuda")
        ws = _lib.fa_decode_paged_workspace_size(c.num_seqs, c.H, c.d, c.max_seq_len,
                                                 c.page_size)
        self.ws = torch.empty(ws, dtype=torch.uint8, device="cuda")

    def run(self, stream=None):
        c = self.inp.cfg
        _lib.fa_decode_paged(self.q, self.kc, self.vc, self.pt, self.sl, self.o, self.lse,
                             max_seq_len=c.max_seq_len, scale=c.scale, workspace=self.ws,
                             stream=stream)

    def result(self):
        torch = torch_dev()
        torch.cuda.synchronize()
        return bf16_from_dev(self.o), self.lse.cpu().numpy()


def run_decode(inp: inputs.DecodeInputs):
    dd = DecodeDev(inp)
    dd.run()
    return dd.result()


def errors(got: np.ndarray, want: np.ndarray):
    d = np.abs(got.astype(np.float64) - want)
    return float(d.max(initial=0.0)), float(d.mean()) if d.size else 0.0


def check_bf16(o_got, lse_got, o_ref, lse_ref, what=""):
    """bf16-in / fp32-accumulate tolerances; LSE -inf must match exactly."""
    mx, mean = errors(o_got, o_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_got), fin), f"{what}: LSE finiteness differs"
    lmx = float(np.max(np.abs(lse_got[fin] - lse_ref[fin]), initial=0.0))
    msg = f"{what}: O max-abs {mx:.3e} mean-abs {mean:.3e} LSE max-abs {lmx:.3e}"
    print(msg)
    assert mx <= BF16_MAX_ABS, msg
    assert mean <= BF16_MEAN_ABS, msg
    assert lmx <= LSE_ABS, msg
    return mx, mean, lmx


def check_fp32(o_got, lse_got, o_ref, lse_ref, what=""):
    mx, mean = errors(o_got, o_ref)
    lmx = float(np.max(np.abs(lse_got - lse_ref)))
    msg = f"{what}: O max-abs {mx:.3e} mean-abs {mean:.3e} LSE max-abs {lmx:.3e}"
    print(msg)
    assert mx <= FP32_MAX_ABS, msg
    assert lmx <= LSE_ABS, msg
    return mx, mean, lmx


def shaped_scores(inp, pattern):
    """Put a score profile along the keys into dimension 0 (q0 = 8 for every query): with
    "rise" the score grows by ~0.4 (log2 units) per key, ~26 per 64-key tile, so the
    reference max moves on every tile; with "step" every key from 64 on scores ~6 (log2
    units) above keys 0..63, so against a reference taken in the first tile the
    exponentials of a later tile sum far above 128 per lane while the max never rises by
    8 (the reference stays). Other dimensions keep their N(0,1) draws."""
    c = inp.cfg
    q, k = inp.q.copy(), inp.k.copy()
    unit = c.scale * math.log2(math.e) * 8.0          # log2 units per unit of k0
    t = np.arange(c.Nk, dtype=np.float64)
    if pattern == "rise":
        k0 = np.minimum(t * 0.4 / unit, 120.0 / unit)  # scores stay below ~120 (log2 units)
    else:
        k0 = np.where(t >= 64, 6.0 / unit, 0.0)
    q[..., 0] = inputs.f32_to_bf16_bits(np.full(q.shape[:-1], 8.0, np.float32))
    k[..., 0] = inputs.f32_to_bf16_bits(np.broadcast_to(k0.astype(np.float32), k.shape[:-1]))
    return inputs.PrefillInputs(c, q, k, inp.v, inp.rng)
