"""Exact attention for AMD MI355X (gfx950): bf16/fp32 prefill, paged-KV decode,
chunked prefill through the page table and the KV append that fills it.

The kernels are hand-written HIP in ``csrc/`` behind the C ABI of
``include/kvfa.h`` (``libkvfa.so``); ``kv_cache_fa_amd._lib`` is the ctypes binding
with the same function names. ``kv_cache_fa_amd.inputs`` generates the seeded
synthetic workloads. Importing the package does not load the library; the first
call does, and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    KvfaError,
    fa_bwd,
    fa_bwd_workspace_size,
    fa_decode_paged,
    fa_decode_paged_fp8,
    fa_decode_paged_noalloc,
    fa_decode_paged_split_tokens,
    fa_decode_paged_workspace_size,
    fa_fwd,
    fa_fwd_fp32,
    fa_fwd_paged,
    fa_fwd_two_pass,
    fa_fwd_window,
    fa_kv_append,
    fa_status_string,
    lib,
)
