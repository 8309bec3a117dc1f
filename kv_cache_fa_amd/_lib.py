"""ctypes binding of libkvfa.so (C ABI in include/kvfa.h).

Argument marshalling only: every step of the attention computation runs in the HIP
kernels behind the C ABI. PyTorch tensors are accepted as containers of device
memory; their data pointers, the sizes read from their shapes and torch's current
HIP stream are passed through unchanged. There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvfa.so")

FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_SCRATCH = 0, -1, -2, -3, -4
# Size of the static device array behind fa_decode_paged_noalloc (kvfa.h)
FA_NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None

_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_fwd_fp32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_decode_paged_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "fa_decode_paged_split_tokens": (_i, [_i, _i, _i]),
    "fa_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i,
                             _f, _vp, _sz, _vp]),
    "fa_decode_paged_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i,
                                     _i, _i, _f, _vp]),
    "fa_fwd_two_pass": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_fwd_window": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_fwd_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                          _i, _f, _vp]),
    "fa_kv_append": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "fa_decode_paged_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _vp, _vp, _i, _i, _i, _i,
                                 _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_bwd_workspace_size": (_sz, [_i, _i, _i]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                    _vp, _sz, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
}


class KvfaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status}: {fa_status_string(status)}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded library (loads it on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m kv_cache_fa_amd.build` (hipcc, gfx950)")
        # torch's HIP and HSA runtimes load first: the library's own HIP runtime then runs
        # on the HSA runtime torch already loaded. Loaded the other way round (the library
        # before torch), the library's runtime found no device once torch had initialised
        # the GPU.
        import torch  # noqa: F401
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def fa_status_string(status: int) -> str:
    return lib().fa_status_string(status).decode()


def _check(fn: str, status: int):
    if status != FA_OK:
        raise KvfaError(fn, status)


def _ptr(t):
    """Device pointer of a tensor (or an int / None passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_tensor(t, dtype, name):
    import torch  # noqa: F401
    _require(t.is_cuda, f"{name} must be a device tensor")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(t.is_contiguous(), f"{name} must be contiguous")


def fa_fwd(q, k, v, o, lse=None, *, causal: bool, scale: float, stream=None):
    """bf16 prefill: q,o [B,H,Nq,d]; k,v [B,Hkv,Nk,d]; lse [B,H,Nq] fp32 or None."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _require(tuple(k.shape) == tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _check("fa_fwd", lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq,
                                  Nk, d, int(bool(causal)), float(scale), _stream(stream)))


def fa_fwd_two_pass(q, k, v, o, lse, *, causal: bool, scale: float, stream=None):
    """bf16 prefill in two passes (statistics, then output); lse [B,H,Nq] fp32 required."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _require(tuple(k.shape) == tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    _require(lse is not None, "lse is required: it carries the statistics between the passes")
    _check_tensor(lse, torch.float32, "lse")
    _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _check("fa_fwd_two_pass", lib().fa_fwd_two_pass(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, int(bool(causal)),
        float(scale), _stream(stream)))


def fa_fwd_window(q, k, v, o, lse=None, *, window_left: int, window_right: int, scale: float,
                  stream=None):
    """bf16 prefill with a sliding window (-1 = unbounded side); layouts as fa_fwd."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _require(tuple(k.shape) == tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _check("fa_fwd_window", lib().fa_fwd_window(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, Hkv, Nq, Nk, d, int(window_left),
        int(window_right), float(scale), _stream(stream)))


def fa_fwd_fp32(q, k, v, o, lse=None, *, causal: bool, scale: float, stream=None):
    """fp32 prefill, same layouts as fa_fwd."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o")):
        _check_tensor(t, torch.float32, n)
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _require(tuple(k.shape) == tuple(v.shape) == (B, Hkv, Nk, d), "k/v shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _check("fa_fwd_fp32", lib().fa_fwd_fp32(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H,
                                            Hkv, Nq, Nk, d, int(bool(causal)), float(scale),
                                            _stream(stream)))


def fa_decode_paged_workspace_size(num_seqs, H, d, max_seq_len, page_size=16) -> int:
    return int(lib().fa_decode_paged_workspace_size(num_seqs, H, d, max_seq_len, page_size))


def fa_decode_paged_split_tokens(num_seqs, max_seq_len, page_size=16) -> int:
    return int(lib().fa_decode_paged_split_tokens(num_seqs, max_seq_len, page_size))


def fa_decode_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse=None, *, max_seq_len: int,
                    scale: float, workspace, stream=None):
    """Paged decode. q,o [S,H,d] bf16; caches [P,16,Hkv,d] bf16; page_table [S,M] int32;
    seq_lens [S] int32 (device); workspace: uint8 device tensor."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    _check_tensor(page_table, torch.int32, "page_table")
    _check_tensor(seq_lens, torch.int32, "seq_lens")
    S, H, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    _require(dk == d and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    _require(page_table.dim() == 2 and page_table.shape[0] == S, "page_table must be [S, M]")
    _require(tuple(seq_lens.shape) == (S,), "seq_lens must be [S]")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (S, H), "lse must be [S,H]")
    _require(workspace.is_cuda and workspace.is_contiguous(), "workspace must be device memory")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fa_decode_paged", lib().fa_decode_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), page_size,
        _ptr(o), _ptr(lse), S, H, Hkv, d, num_pages, int(page_table.shape[1]), int(max_seq_len),
        float(scale), _ptr(workspace), ws_bytes, _stream(stream)))


def fa_decode_paged_noalloc(q, k_cache, v_cache, page_table, seq_lens, o, lse=None, *,
                            max_seq_len: int, scale: float, stream=None):
    """Paged decode with the workspace in the library's static device array (no
    allocation anywhere in the call). Same tensors as fa_decode_paged, no workspace."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    _check_tensor(page_table, torch.int32, "page_table")
    _check_tensor(seq_lens, torch.int32, "seq_lens")
    S, H, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    _require(dk == d and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    _require(page_table.dim() == 2 and page_table.shape[0] == S, "page_table must be [S, M]")
    _require(tuple(seq_lens.shape) == (S,), "seq_lens must be [S]")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (S, H), "lse must be [S,H]")
    _check("fa_decode_paged_noalloc", lib().fa_decode_paged_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), page_size,
        _ptr(o), _ptr(lse), S, H, Hkv, d, num_pages, int(page_table.shape[1]), int(max_seq_len),
        float(scale), _stream(stream)))


def fa_fwd_paged(q, k_cache, v_cache, page_table, seq_lens, o, lse=None, *, max_seq_len: int,
                 causal: bool, scale: float, stream=None):
    """Chunked prefill through the page table. q,o [B,H,Nq,d] bf16; caches [P,16,Hkv,d]
    bf16; page_table [B,M] int32; seq_lens [B] int32 (device, new tokens included)."""
    import torch
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    _check_tensor(page_table, torch.int32, "page_table")
    _check_tensor(seq_lens, torch.int32, "seq_lens")
    B, H, Nq, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    _require(dk == d and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    _require(page_table.dim() == 2 and page_table.shape[0] == B, "page_table must be [B, M]")
    _require(tuple(seq_lens.shape) == (B,), "seq_lens must be [B]")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _check("fa_fwd_paged", lib().fa_fwd_paged(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table), _ptr(seq_lens), page_size,
        _ptr(o), _ptr(lse), B, H, Hkv, Nq, d, num_pages, int(page_table.shape[1]),
        int(max_seq_len), int(bool(causal)), float(scale), _stream(stream)))


def fa_kv_append(k_new, v_new, k_cache, v_cache, page_table, start_pos, *, stream=None):
    """Scatter new tokens' K/V into the paged cache. k_new,v_new [S,n_new,Hkv,d] bf16;
    caches [P,16,Hkv,d] bf16; page_table [S,M] int32; start_pos [S] int32 (device)."""
    import torch
    for t, n in ((k_new, "k_new"), (v_new, "v_new"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_tensor(t, torch.bfloat16, n)
    _check_tensor(page_table, torch.int32, "page_table")
    _check_tensor(start_pos, torch.int32, "start_pos")
    S, n_new, Hkv, d = k_new.shape
    num_pages, page_size, Hkv_c, dk = k_cache.shape
    _require(tuple(v_new.shape) == tuple(k_new.shape), "k_new/v_new shape mismatch")
    _require(Hkv_c == Hkv and dk == d and tuple(v_cache.shape) == tuple(k_cache.shape),
             "cache shape mismatch")
    _require(page_table.dim() == 2 and page_table.shape[0] == S, "page_table must be [S, M]")
    _require(tuple(start_pos.shape) == (S,), "start_pos must be [S]")
    _check("fa_kv_append", lib().fa_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        _ptr(start_pos), page_size, S, n_new, Hkv, d, num_pages, int(page_table.shape[1]),
        _stream(stream)))


def fa_decode_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, page_table, seq_lens, o,
                        lse=None, *, max_seq_len: int, scale: float, workspace, stream=None):
    """Paged decode on an e4m3 cache. q,o [S,H,d] bf16; caches [P,16,Hkv,d] uint8 (e4m3
    bytes); k_scale, v_scale [Hkv] fp32 (device); page_table [S,M] int32; seq_lens [S]."""
    import torch
    for t, n in ((q, "q"), (o, "o")):
        _check_tensor(t, torch.bfloat16, n)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_tensor(t, torch.uint8, n)
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _check_tensor(t, torch.float32, n)
    _check_tensor(page_table, torch.int32, "page_table")
    _check_tensor(seq_lens, torch.int32, "seq_lens")
    S, H, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    _require(dk == d and tuple(v_cache.shape) == tuple(k_cache.shape), "cache shape mismatch")
    _require(tuple(k_scale.shape) == tuple(v_scale.shape) == (Hkv,), "scales must be [Hkv]")
    _require(tuple(o.shape) == tuple(q.shape), "o must have q's shape")
    _require(page_table.dim() == 2 and page_table.shape[0] == S, "page_table must be [S, M]")
    _require(tuple(seq_lens.shape) == (S,), "seq_lens must be [S]")
    if lse is not None:
        _check_tensor(lse, torch.float32, "lse")
        _require(tuple(lse.shape) == (S, H), "lse must be [S,H]")
    _require(workspace.is_cuda and workspace.is_contiguous(), "workspace must be device memory")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fa_decode_paged_fp8", lib().fa_decode_paged_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(page_table),
        _ptr(seq_lens), page_size, _ptr(o), _ptr(lse), S, H, Hkv, d, num_pages,
        int(page_table.shape[1]), int(max_seq_len), float(scale), _ptr(workspace), ws_bytes,
        _stream(stream)))


def fa_bwd_workspace_size(B, H, Nq) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, Nq))


def fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, *, causal: bool, scale: float, workspace,
           stream=None):
    """Backward pass. q,o,dout,dq [B,H,Nq,d] bf16; k,v,dk,dv [B,Hkv,Nk,d] bf16; lse
    [B,H,Nq] fp32 from the forward; workspace: uint8 device tensor."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout"), (dq, "dq"),
                 (dk, "dk"), (dv, "dv")):
        _check_tensor(t, torch.bfloat16, n)
    _check_tensor(lse, torch.float32, "lse")
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    _require(tuple(k.shape) == tuple(v.shape) == tuple(dk.shape) == tuple(dv.shape)
             == (B, Hkv, Nk, d), "k/v/dk/dv shape mismatch")
    _require(tuple(o.shape) == tuple(dout.shape) == tuple(dq.shape) == tuple(q.shape),
             "o/dout/dq must have q's shape")
    _require(tuple(lse.shape) == (B, H, Nq), "lse must be [B,H,Nq]")
    _require(workspace.is_cuda and workspace.is_contiguous(), "workspace must be device memory")
    ws_bytes = workspace.numel() * workspace.element_size()
    _check("fa_bwd", lib().fa_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, H, Hkv, Nq, Nk, d, int(bool(causal)), float(scale), _ptr(workspace), ws_bytes,
        _stream(stream)))
