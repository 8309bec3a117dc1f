"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--prefill long_causal|gqa_causal]
                    [--no-cpu-baseline] [--no-extra] [--calibrate-copy]

One step = one pass over every stage of the path on one batch of synthetic,
seeded input already resident in HBM:
  * causal bf16 prefill, fa_fwd (default: B1 H8 N131072 d128, the long-context
    workload), and
  * paged-KV decode, fa_decode_paged (64 sequences x 1 query, H32 Hkv8 d128,
    lengths U{512..8192}, 16-token pages; split-K kernel + log-sum-exp combine).
W untimed steps, then K timed steps bracketed by device synchronisation. Prints one
JSON line. Every launch goes through the C ABI of libkvfa.so on torch's current
stream; HIP events on that stream time each call.

Only the cpu_baseline leg touches the fp64 oracle (timed on a bounded sample).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kv_cache_fa_amd import _lib, inputs  # noqa: E402

METRIC = "prefill attn TFLOP/s (bf16 causal) + decode KV GB/s, % of MI355X peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CSRC = os.path.join(ROOT, "kv_cache_fa_amd", "csrc")
# The sources each leg's kernels are built from (their hash dates the counter runs).
_COMMON = ["common.h", "launch.h"]
LEG_SOURCES = {
    "prefill": ["prefill_pp.hip", "prefill_ks.hip", "prefill_common.h"] + _COMMON,
    "prefill_gqa_causal": ["prefill_pp.hip", "prefill_ks.hip", "prefill_common.h"] + _COMMON,
    "prefill_small_causal": ["prefill_pp.hip", "prefill_ks.hip", "prefill_common.h"] + _COMMON,
    "chunked_prefill_paged": ["prefill_pp.hip", "prefill_common.h"] + _COMMON,
    "prefill_sliding_window": ["prefill_pp.hip", "prefill_common.h"] + _COMMON,
    "prefill_gqa_causal_two_pass": ["prefill_bf16.hip", "prefill_common.h"] + _COMMON,
    "backward_gqa_causal": ["backward.hip", "prefill_common.h"] + _COMMON,
    "decode": ["decode.hip", "prefill_common.h"] + _COMMON,
    "decode_fp8": ["decode.hip", "prefill_common.h"] + _COMMON,
    "decode_g16": ["decode.hip", "prefill_common.h"] + _COMMON,
    "kv_append": ["kv_append.hip"] + _COMMON,
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(files) -> str:
    h = hashlib.sha256()
    for name in files:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(leg: str, workload: str):
    """HBM bytes per call of a leg from the committed counter runs (FETCH_SIZE +
    WRITE_SIZE, each scaled by its reading for a device copy of known size), if they
    still describe the current kernel sources (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(leg)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("workload") != workload:
        return None
    if rec.get("source_sha") != source_sha(LEG_SOURCES[leg]):
        return None
    return rec.get("bytes_per_call")


def decode_bytes(inp: inputs.DecodeInputs) -> int:
    """Algorithmic bytes of one decode call: the K/V the sequences own, Q, O, lse,
    the page-table entries read and seq_lens (the split-K workspace is not counted)."""
    c = inp.cfg
    n_pages = int(((inp.seq_lens.astype(np.int64) + c.page_size - 1) // c.page_size).sum())
    return (inp.kv_bytes() + 2 * c.num_seqs * c.H * c.d * 2 + c.num_seqs * c.H * 4
            + n_pages * 4 + c.num_seqs * 4)


def decode_flops(inp: inputs.DecodeInputs) -> float:
    return 4.0 * inp.cfg.d * inp.cfg.H * float(inp.seq_lens.astype(np.int64).sum())


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()
                    if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def cpu_baseline_small(name: str):
    """The fp64 oracle on a whole small prefill workload (every row), timed."""
    import oracle  # test infrastructure, used only for the baseline legs
    c = inputs.PREFILL_CONFIGS[name]
    q, k, v = inputs.make_prefill(c).as_f64()
    t0 = time.perf_counter()
    oracle.attention(q, k, v, causal=c.causal, scale=c.scale)
    t = time.perf_counter() - t0
    return {"s": round(t, 4), "GFLOP/s": round(c.flops / t / 1e9, 3), "cores": blas_threads(),
            "sample": f"the whole {name} workload (all {c.B * c.H * c.Nq} rows), fp64 NumPy"}


def cpu_baseline_decode(dinp: inputs.DecodeInputs, d_bytes: int):
    """The fp64 oracle on the whole paged-decode workload (all sequences and heads, from
    each sequence's contiguous K/V), timed; rate in the decode metric's unit."""
    import oracle  # test infrastructure, used only for the baseline legs
    q = inputs.bf16_bits_to_f64(dinp.q)
    ks = [inputs.bf16_bits_to_f64(x) for x in dinp.k_seq]
    vs = [inputs.bf16_bits_to_f64(x) for x in dinp.v_seq]
    t0 = time.perf_counter()
    oracle.decode(q, ks, vs, scale=dinp.cfg.scale)
    t = time.perf_counter() - t0
    return {"value": round(d_bytes / t / 1e9, 3), "unit": "GB/s", "cores": blas_threads(),
            "kind": "oracle", "s": round(t, 3),
            "sample": f"the whole paged_decode workload ({dinp.cfg.num_seqs} sequences x "
                      f"{dinp.cfg.H} heads, {int(dinp.seq_lens.sum())} cached tokens), fp64 "
                      "NumPy; rate = the call's algorithmic bytes / oracle time"}


def cpu_baseline(pinp: inputs.PrefillInputs, budget_s: float = 12.0):
    """The fp64 oracle (as it stands) on a bounded sample of the prefill workload:
    random query rows of head 0, each against its full causal prefix."""
    import oracle  # test infrastructure, used only for this baseline leg
    cores = blas_threads()
    c = pinp.cfg
    q = inputs.bf16_bits_to_f64(pinp.q[:1, :1])
    k = inputs.bf16_bits_to_f64(pinp.k[:1, :1])
    v = inputs.bf16_bits_to_f64(pinp.v[:1, :1])
    rng = np.random.default_rng(1234)
    done_rows, flops, t_used = 0, 0.0, 0.0
    batch = 32
    while t_used < budget_s:
        rows = np.sort(rng.choice(c.Nq, size=batch, replace=False))
        t0 = time.perf_counter()
        oracle.attention(q, k, v, causal=c.causal, scale=c.scale, rows={(0, 0): rows})
        t_used += time.perf_counter() - t0
        n_keys = (rows + (c.Nk - c.Nq) + 1) if c.causal else np.full(batch, c.Nk)
        flops += 4.0 * c.d * float(n_keys.sum())
        done_rows += batch
    rate = flops / t_used
    return {"value": rate / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"{done_rows} random query rows of head 0 of {c.name} (each over its "
                      f"full causal prefix), fp64 NumPy, {t_used:.1f} s",
            "extrapolated_full_config_s": round(c.flops / rate, 1)}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--prefill", default="long_causal", choices=["long_causal", "gqa_causal"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the separately timed GQA prefill measurement")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--reps", type=int, default=20,
                    help="timed calls per extra leg (the small prefill leg takes 5x)")
    ap.add_argument("--warm-s", type=float, default=0.2,
                    help="warm-up seconds before each extra leg (0: none; for profiling)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    _lib.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs (seeded, synthetic), resident in HBM before timing ----
    pcfg = inputs.PREFILL_CONFIGS[args.prefill]
    log(f"[bench] generating {pcfg.name} inputs")
    pinp = inputs.make_prefill(pcfg)
    pq, pk, pv = to_dev(pinp.q), to_dev(pinp.k), to_dev(pinp.v)
    po = torch.empty_like(pq)
    plse = torch.empty((pcfg.B, pcfg.H, pcfg.Nq), dtype=torch.float32, device=dev)

    dcfg = inputs.DECODE_CONFIGS["paged_decode"]
    log("[bench] generating paged_decode inputs")
    dinp = inputs.make_decode(dcfg)
    dq, dkc, dvc = to_dev(dinp.q), to_dev(dinp.k_cache), to_dev(dinp.v_cache)
    dpt = torch.from_numpy(dinp.page_table).to(dev)
    dsl = torch.from_numpy(dinp.seq_lens).to(dev)
    do = torch.empty_like(dq)
    dlse = torch.empty((dcfg.num_seqs, dcfg.H), dtype=torch.float32, device=dev)
    ws = torch.empty(_lib.fa_decode_paged_workspace_size(dcfg.num_seqs, dcfg.H, dcfg.d,
                                                         dcfg.max_seq_len), dtype=torch.uint8,
                     device=dev)
    torch.cuda.synchronize()

    def prefill():
        _lib.fa_fwd(pq, pk, pv, po, plse, causal=pcfg.causal, scale=pcfg.scale, stream=stream)

    def decode():
        _lib.fa_decode_paged(dq, dkc, dvc, dpt, dsl, do, dlse, max_seq_len=dcfg.max_seq_len,
                             scale=dcfg.scale, workspace=ws, stream=stream)

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {K} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for i in range(K):
        ev[i][0].record(stream)
        prefill()
        ev[i][1].record(stream)
        ev[i][2].record(stream)
        decode()
        ev[i][3].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    step_ms = start.elapsed_time(end) / K
    p_ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    d_ms = np.array([e[2].elapsed_time(e[3]) for e in ev])

    p_flops = pcfg.flops
    d_bytes = decode_bytes(dinp)
    d_flops = decode_flops(dinp)
    value = (p_flops + d_flops) / (step_ms * 1e-3) / 1e12
    p_tflops = p_flops / (p_ms.mean() * 1e-3) / 1e12
    d_gbs = d_bytes / (d_ms.mean() * 1e-3) / 1e9

    p_traffic = measured_traffic("prefill", pcfg.name)
    d_traffic = measured_traffic("decode", dcfg.name)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16; paged cache with seeded page permutation)",
        "config": {
            "workload": f"{pcfg.name} prefill + paged_decode",
            "prefill": {"B": pcfg.B, "H": pcfg.H, "Hkv": pcfg.Hkv, "N": pcfg.Nq, "d": pcfg.d,
                        "causal": pcfg.causal, "flops": p_flops},
            "decode": {"num_seqs": dcfg.num_seqs, "H": dcfg.H, "Hkv": dcfg.Hkv, "d": dcfg.d,
                       "seq_len": f"U{{{dcfg.len_lo}..{dcfg.len_hi}}}",
                       "total_kv_tokens": int(dinp.seq_lens.sum()), "page_size": dcfg.page_size,
                       "bytes": d_bytes},
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "fwd_pp_kernel",
            "bound": "mfma",
            "achieved": round(p_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(p_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": p_traffic,
        },
        "legs": {
            "prefill": {"ms_mean": round(float(p_ms.mean()), 4),
                        "ms_median": round(float(np.median(p_ms)), 4),
                        "ms_p10": round(float(np.percentile(p_ms, 10)), 4),
                        "ms_p90": round(float(np.percentile(p_ms, 90)), 4),
                        "TFLOP/s": round(p_tflops, 2),
                        "frac_of_bf16_peak": round(p_tflops / PEAK_BF16_TFLOPS, 4)},
            "decode": {"ms_mean": round(float(d_ms.mean()), 4),
                       "ms_median": round(float(np.median(d_ms)), 4),
                       "ms_p10": round(float(np.percentile(d_ms, 10)), 4),
                       "ms_p90": round(float(np.percentile(d_ms, 90)), 4),
                       "GB/s": round(d_gbs, 1),
                       "frac_of_hbm_peak": round(d_gbs / PEAK_HBM_GBS, 4),
                       "roofline": {"kernel": "decode_split_kernel + decode_combine_kernel",
                                    "bound": "hbm", "achieved": round(d_gbs, 1),
                                    "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": round(d_gbs / PEAK_HBM_GBS, 4),
                                    "traffic": d_traffic}},
        },
        "wall_s_timed": round(t_wall, 3),
    }

    def timed(fn, n=None):
        """Mean ms of fn over n back-to-back launches, after ~--warm-s of warm-up (the
        clock ramps up under sustained load)."""
        n = args.reps if n is None else n
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < args.warm_s:
            for _ in range(n):
                fn()
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    if not args.no_extra and args.prefill != "gqa_causal":
        gcfg = inputs.PREFILL_CONFIGS["gqa_causal"]
        log("[bench] extra: gqa_causal prefill")
        ginp = inputs.make_prefill(gcfg)
        gq, gk, gv = to_dev(ginp.q), to_dev(ginp.k), to_dev(ginp.v)
        go = torch.empty_like(gq)
        glse = torch.empty((gcfg.B, gcfg.H, gcfg.Nq), dtype=torch.float32, device=dev)
        g_ms = timed(lambda: _lib.fa_fwd(gq, gk, gv, go, glse, causal=True, scale=gcfg.scale,
                                         stream=stream))
        g_tf = gcfg.flops / (g_ms * 1e-3) / 1e12
        out["legs"]["prefill_gqa_causal"] = {
            "B": gcfg.B, "H": gcfg.H, "Hkv": gcfg.Hkv, "N": gcfg.Nq, "d": gcfg.d,
            "ms_mean": round(g_ms, 4), "TFLOP/s": round(g_tf, 2),
            "frac_of_bf16_peak": round(g_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_gqa_causal", gcfg.name)}
        # The small causal case (B2 H8 N1024 d64): a few microseconds, so launch-bound;
        # reported, not a target.
        scfg = inputs.PREFILL_CONFIGS["bf16_causal"]
        log("[bench] extra: bf16_causal prefill")
        sinp = inputs.make_prefill(scfg)
        sq, sk, sv = to_dev(sinp.q), to_dev(sinp.k), to_dev(sinp.v)
        so = torch.empty_like(sq)
        slse = torch.empty((scfg.B, scfg.H, scfg.Nq), dtype=torch.float32, device=dev)
        s_ms = timed(lambda: _lib.fa_fwd(sq, sk, sv, so, slse, causal=True, scale=scfg.scale,
                                         stream=stream), n=5 * args.reps)
        s_tf = scfg.flops / (s_ms * 1e-3) / 1e12
        out["legs"]["prefill_small_causal"] = {
            "B": scfg.B, "H": scfg.H, "Hkv": scfg.Hkv, "N": scfg.Nq, "d": scfg.d,
            "ms_mean": round(s_ms, 4), "TFLOP/s": round(s_tf, 2),
            "frac_of_bf16_peak": round(s_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_small_causal", scfg.name)}
        del sq, sk, sv, so, slse
        # The same workload through the FlashAttention-1 two-pass path (statistics pass +
        # output pass); TFLOP/s counts the algorithmic flops, not the recomputed Q.K^T.
        log("[bench] extra: gqa_causal two-pass")
        t_ms = timed(lambda: _lib.fa_fwd_two_pass(gq, gk, gv, go, glse, causal=True,
                                                  scale=gcfg.scale, stream=stream))
        t_tf = gcfg.flops / (t_ms * 1e-3) / 1e12
        out["legs"]["prefill_gqa_causal_two_pass"] = {
            "ms_mean": round(t_ms, 4), "TFLOP/s": round(t_tf, 2),
            "frac_of_bf16_peak": round(t_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_gqa_causal_two_pass", gcfg.name),
            "mfma_flops_executed_per_algorithmic": 1.5}
        # Backward pass on the same workload: algorithmic flops 2.5x the forward's (dV,
        # dP, dQ, dK and the recomputed S: 5 products of 2d flops per attending pair); the
        # kernels execute 7 (S and dP are computed again for dQ).
        log("[bench] extra: gqa_causal backward")
        gdo = to_dev(inputs.make_dout(gcfg, seed=gcfg.seed + 100))
        gdq, gdk, gdv = torch.empty_like(gq), torch.empty_like(gk), torch.empty_like(gv)
        gws = torch.empty(_lib.fa_bwd_workspace_size(gcfg.B, gcfg.H, gcfg.Nq), dtype=torch.uint8,
                          device=dev)
        _lib.fa_fwd(gq, gk, gv, go, glse, causal=True, scale=gcfg.scale, stream=stream)
        b_ms = timed(lambda: _lib.fa_bwd(gq, gk, gv, go, glse, gdo, gdq, gdk, gdv, causal=True,
                                         scale=gcfg.scale, workspace=gws, stream=stream))
        b_tf = 2.5 * gcfg.flops / (b_ms * 1e-3) / 1e12
        out["legs"]["backward_gqa_causal"] = {
            "ms_mean": round(b_ms, 4), "TFLOP/s": round(b_tf, 2),
            "frac_of_bf16_peak": round(b_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("backward_gqa_causal", gcfg.name),
            "flops": 2.5 * gcfg.flops, "mfma_flops_executed_per_algorithmic": 1.4}
        del gdo, gdq, gdk, gdv, gws
        del gq, gk, gv, go, glse

    if not args.no_extra:
        # Chunked prefill through the page table: a 1024-token chunk for each of 8
        # sequences whose caches (chunk included) hold U{4096..16384} tokens.
        B, H, Hkv, d, Nq = 8, 32, 8, 128, 1024
        log("[bench] extra: chunked prefill through the page table")
        ci = inputs.custom_chunked_prefill(B, H, Hkv, d, Nq, 4096, 16384, seed=1234)
        c = ci.cache
        cq, ckc, cvc = to_dev(ci.q), to_dev(c.k_cache), to_dev(c.v_cache)
        cpt = torch.from_numpy(c.page_table).to(dev)
        csl = torch.from_numpy(c.seq_lens).to(dev)
        co = torch.empty_like(cq)
        clse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
        c_ms = timed(lambda: _lib.fa_fwd_paged(cq, ckc, cvc, cpt, csl, co, clse,
                                               max_seq_len=c.cfg.max_seq_len, causal=True,
                                               scale=c.cfg.scale, stream=stream))
        c_flops = sum(4.0 * d * H * inputs.unmasked_pairs(Nq, int(L), True)
                      for L in c.seq_lens)
        c_tf = c_flops / (c_ms * 1e-3) / 1e12
        out["legs"]["chunked_prefill_paged"] = {
            "B": B, "H": H, "Hkv": Hkv, "Nq": Nq, "d": d,
            "seq_lens": [int(x) for x in c.seq_lens], "flops": c_flops,
            "ms_mean": round(c_ms, 4), "TFLOP/s": round(c_tf, 2),
            "frac_of_bf16_peak": round(c_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("chunked_prefill_paged", "chunked_prefill_paged")}
        del cq, ckc, cvc, co, clse

        # Sliding-window prefill: B1 H32 Hkv8 N32768 d128, causal window of 4096 keys.
        log("[bench] extra: sliding-window prefill")
        wcfg = inputs.WINDOW_CONFIG
        wB, wH, wHkv, wN, wd = wcfg.B, wcfg.H, wcfg.Hkv, wcfg.Nq, wcfg.d
        wl, wr = inputs.WINDOW
        winp = inputs.make_prefill(wcfg)
        wq, wk, wv = to_dev(winp.q), to_dev(winp.k), to_dev(winp.v)
        del winp
        wo = torch.empty_like(wq)
        wlse = torch.empty((wB, wH, wN), dtype=torch.float32, device=dev)
        w_ms = timed(lambda: _lib.fa_fwd_window(wq, wk, wv, wo, wlse, window_left=wl,
                                                window_right=wr, scale=wcfg.scale, stream=stream))
        w_flops = 4.0 * wd * wB * wH * inputs.window_pairs(wN, wN, wl, wr)
        w_tf = w_flops / (w_ms * 1e-3) / 1e12
        out["legs"]["prefill_sliding_window"] = {
            "B": wB, "H": wH, "Hkv": wHkv, "N": wN, "d": wd, "window": [wl, wr],
            "flops": w_flops, "ms_mean": round(w_ms, 4), "TFLOP/s": round(w_tf, 2),
            "frac_of_bf16_peak": round(w_tf / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic("prefill_sliding_window", wcfg.name)}
        del wq, wk, wv, wo, wlse

        # Paged decode on an fp8 (e4m3) copy of the decode workload's cache.
        log("[bench] extra: fp8 paged decode")
        f8 = inputs.quantize_decode_fp8(dinp, seqs=False)
        fkc = torch.from_numpy(f8.k_cache).to(dev)
        fvc = torch.from_numpy(f8.v_cache).to(dev)
        fks = torch.from_numpy(f8.k_scale).to(dev)
        fvs = torch.from_numpy(f8.v_scale).to(dev)
        f_ms = timed(lambda: _lib.fa_decode_paged_fp8(dq, fkc, fvc, fks, fvs, dpt, dsl, do, dlse,
                                                      max_seq_len=dcfg.max_seq_len,
                                                      scale=dcfg.scale, workspace=ws,
                                                      stream=stream))
        f_bytes = decode_bytes(dinp) - dinp.kv_bytes() // 2  # K/V bytes halve, the rest stays
        f_gbs = f_bytes / (f_ms * 1e-3) / 1e9
        out["legs"]["decode_fp8"] = {
            "bytes": f_bytes, "ms_mean": round(f_ms, 4), "GB/s": round(f_gbs, 1),
            "frac_of_hbm_peak": round(f_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("decode_fp8", "paged_decode"),
            "tokens_per_s": round(float(dinp.seq_lens.sum()) / (f_ms * 1e-3), 1)}
        del fkc, fvc, fks, fvs

        # Paged decode with a wide GQA group: the decode workload's shape with two KV
        # heads (H32 Hkv2, 16 query heads per KV head), lengths U{512..8192}.
        log("[bench] extra: paged decode, 16 query heads per KV head")
        ginp16 = inputs.custom_decode(dcfg.num_seqs, 32, 2, dcfg.d, dcfg.len_lo, dcfg.len_hi,
                                      seed=dcfg.seed)
        gq16 = to_dev(ginp16.q)
        gkc16, gvc16 = to_dev(ginp16.k_cache), to_dev(ginp16.v_cache)
        gpt16 = torch.from_numpy(ginp16.page_table).to(dev)
        gsl16 = torch.from_numpy(ginp16.seq_lens).to(dev)
        go16 = torch.empty_like(gq16)
        glse16 = torch.empty((dcfg.num_seqs, 32), dtype=torch.float32, device=dev)
        gws16 = torch.empty(_lib.fa_decode_paged_workspace_size(dcfg.num_seqs, 32, dcfg.d,
                                                                 ginp16.cfg.max_seq_len),
                            dtype=torch.uint8, device=dev)
        g16_ms = timed(lambda: _lib.fa_decode_paged(gq16, gkc16, gvc16, gpt16, gsl16, go16,
                                                     glse16, max_seq_len=ginp16.cfg.max_seq_len,
                                                     scale=dcfg.scale, workspace=gws16,
                                                     stream=stream))
        g16_bytes = decode_bytes(ginp16)
        g16_gbs = g16_bytes / (g16_ms * 1e-3) / 1e9
        out["legs"]["decode_g16"] = {
            "num_seqs": dcfg.num_seqs, "H": 32, "Hkv": 2, "d": dcfg.d,
            "total_kv_tokens": int(ginp16.seq_lens.sum()), "bytes": g16_bytes,
            "ms_mean": round(g16_ms, 4), "GB/s": round(g16_gbs, 1),
            "frac_of_hbm_peak": round(g16_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("decode_g16", "decode_g16")}
        del gq16, gkc16, gvc16, go16, gws16

        # KV append of that chunk size: 8 sequences x 1024 new tokens into a cache
        # with room for 16384 tokens each.
        log("[bench] extra: kv append")
        a = inputs.make_append(B, Nq, Hkv, d, 16384, seed=4321)
        akn, avn = to_dev(a.k_new), to_dev(a.v_new)
        akc, avc = to_dev(a.k_cache), to_dev(a.v_cache)
        apt = torch.from_numpy(a.page_table).to(dev)
        asp = torch.from_numpy(a.start_pos).to(dev)
        a_ms = timed(lambda: _lib.fa_kv_append(akn, avn, akc, avc, apt, asp, stream=stream))
        a_bytes = 2 * 2 * a.k_new.nbytes  # K and V, each read once and written once
        a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
        out["legs"]["kv_append"] = {
            "num_seqs": B, "n_new": Nq, "Hkv": Hkv, "d": d, "bytes": a_bytes,
            "ms_mean": round(a_ms, 4), "GB/s": round(a_gbs, 1),
            "frac_of_hbm_peak": round(a_gbs / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("kv_append", "kv_append")}
        del akn, avn, akc, avc

        # Context, not part of the path: the rate the vendor's GEMM (torch.mm, hipBLASLt)
        # reaches on a large square bf16 product on the same chip, in the same run. The
        # chip lowers its clock under sustained matrix load, so this is the practical
        # ceiling against which the attention kernels' fraction of the nominal peak reads.
        log("[bench] context: bf16 GEMM rate (torch.mm)")
        gemm = {}
        for n in (8192, 16384):
            ga = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
            gb = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
            gc = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
            m_ms = timed(lambda: torch.mm(ga, gb, out=gc), n=max(4, args.reps // 4))
            m_tf = 2.0 * n ** 3 / (m_ms * 1e-3) / 1e12
            gemm[f"{n}^3"] = {"ms_mean": round(m_ms, 4), "TFLOP/s": round(m_tf, 1),
                              "frac_of_bf16_peak": round(m_tf / PEAK_BF16_TFLOPS, 4)}
            del ga, gb, gc
        # The attention rates over the 16384^3 GEMM rate of the same run: a figure that
        # does not move with the clock a given chip sustains.
        ref = gemm["16384^3"]["TFLOP/s"]
        gemm["attention_rate_over_gemm_16384"] = {
            k: round(out["legs"][k]["TFLOP/s"] / ref, 4)
            for k in ("prefill", "prefill_gqa_causal", "prefill_sliding_window",
                      "chunked_prefill_paged") if k in out["legs"]}
        out["context_gemm_bf16"] = gemm

    if args.calibrate_copy:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        out["calibration_copy_bytes"] = n

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle sample)")
        out["cpu_baseline"] = cpu_baseline(pinp)
        log("[bench] cpu baseline (oracle, whole decode workload)")
        dec = cpu_baseline_decode(dinp, d_bytes)
        out["cpu_baseline"]["decode"] = dec
        out["legs"]["decode"]["cpu_baseline"] = dec
        log("[bench] cpu baseline (oracle, whole small prefill workloads)")
        for name in ("fp32_single", "bf16_causal"):
            out["cpu_baseline"][name] = cpu_baseline_small(name)

    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
