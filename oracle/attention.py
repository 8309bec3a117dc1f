"""fp64 CPU oracle for exact attention (prefill and paged-KV decode).

TEST INFRASTRUCTURE ONLY. Only the test-suite, the smoke check and the bench's CPU
baseline leg may import this module. The product path (the HIP library and its
Python binding) never imports, calls or links anything here, and this module
imports nothing from the product path.

Every function is the plain definition written out in float64, materialising the
full score matrix (or full score rows) and the probability matrix. Nothing is
tiled, fused or reordered.

Sources (the pages; translations are mine):
* Page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention" (fatihsoysal.com),
  section "Transformer Mimarisi ve Self-Attention Mekanizması": attention is
  softmax(Q K^T / sqrt(d_k)) V; Q, K, V are (sequence length x dim); Q K^T is the
  (seq x seq) compatibility matrix; softmax turns each row into a probability
  distribution; the result weights the rows of V.
* Same page, section "FlashAttention'ın Temelleri": softmax(x) = softmax(x - c)
  for any constant c, usually c = max(x) (shift-stable softmax).
* Same page, "Online Softmax Prensibi", steps 1-5: the blockwise merge of a
  running max M and running sum L (``online_softmax_stats``).
* Same page, "FlashAttention-1 (İki Geçişli Yaklaşım)": only the per-row M and L
  (O(N) numbers) are kept between passes; here they are exported as one
  log-sum-exp per row, LSE = M + ln L.
* Glossary page yapayzekasozluk.tr/etiket/attention, entry "Flash Attention": the
  result equals standard attention exactly (FAQ "does it change the output").
* Same glossary page, entry "KV Cache (Anahtar-Değer Önbelleği)": token n+1 reads
  the cached K/V of the earlier tokens and its own K/V is appended; GQA/MQA give
  one K-V head to several query heads; paged caches keep K/V in fixed-size pages
  (``gather_pages`` reads them back, ``scatter_pages`` appends new tokens).

Readings where the pages are silent (each also listed in the design notes):
* causal alignment is bottom-right: query i sits at absolute position Nk-Nq+i and
  attends keys j <= i + (Nk - Nq);
* GQA head mapping is contiguous: kv head = h // (H // Hkv);
* LSE is in natural-log units;
* a decode query attends all L_s cached keys (its own K/V already appended);
* an empty row (L_s = 0) gives O = 0 and LSE = -inf.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        raise TypeError("oracle inputs must already be float64 (widen stored values first)")
    return a


def window_mask(idx, Nq: int, Nk: int, causal: bool, window=None) -> np.ndarray:
    """Boolean [len(idx), Nk] mask of the keys that query rows ``idx`` attend.

    Query i sits at position p = i + (Nk - Nq) (bottom-right). Causal: keys j <= p.
    Sliding window (glossary entry "Kayan Pencere Dikkati (Sliding Window
    Attention)": a token attends only the tokens within a fixed distance of its own
    position): ``window = (left, right)`` keeps keys p - left <= j <= p + right, where
    -1 leaves that side unbounded; the symmetric window of width w is (w/2, w/2).
    """
    p = np.asarray(idx, dtype=np.int64)[:, None] + (Nk - Nq)
    j = np.arange(Nk)[None, :]
    mask = np.ones((p.shape[0], Nk), dtype=bool)
    if causal:
        mask &= j <= p
    if window is not None:
        left, right = window
        if left >= 0:
            mask &= j >= p - left
        if right >= 0:
            mask &= j <= p + right
    return mask


def allowed_keys(Nq: int, Nk: int, causal: bool, window=None) -> np.ndarray:
    """Boolean [Nq, Nk] mask of the keys each query attends (see ``window_mask``)."""
    return window_mask(np.arange(Nq), Nq, Nk, causal, window)


def softmax_rows(scores: np.ndarray, mask: np.ndarray):
    """Row softmax over the allowed entries, shifted by the row max.

    Returns (P, m, l): probabilities (0 where masked), the row max m over allowed
    entries, and the row sum l = sum_j exp(s_j - m). Rows with no allowed entry get
    P = 0, m = -inf, l = 0.
    """
    s = np.where(mask, scores, NEG_INF)
    m = np.max(s, axis=-1, initial=NEG_INF)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(mask, np.exp(s - safe_m[..., None]), 0.0)
    l = np.sum(e, axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        P = np.where(l[..., None] > 0, e / np.where(l > 0, l, 1.0)[..., None], 0.0)
    return P, m, l


def attention(q, k, v, *, causal: bool, scale: float, rows=None, return_probs=False,
              window=None):
    """Exact attention in float64.

    q: [B, H, Nq, d]; k, v: [B, Hkv, Nk, d] (float64, the stored values widened).
    window: None, or (left, right) for a sliding window (``window_mask``).
    rows: None for every row, else a dict {(b, h): int array of query rows}.
    Returns (O, LSE) as dicts keyed by (b, h) when ``rows`` is given, else dense
    arrays O [B, H, Nq, d] and LSE [B, H, Nq]. With ``return_probs`` the probability
    matrix of each computed (b, h) is returned as a third item (dict).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("shape mismatch")
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    g = H // Hkv

    pairs = [(b, h) for b in range(B) for h in range(H)] if rows is None else sorted(rows)
    outs, lses, probs = {}, {}, {}
    for (b, h) in pairs:
        idx = np.arange(Nq) if rows is None else np.asarray(rows[(b, h)], dtype=np.int64)
        kvh = h // g
        # full score rows: (len(idx) x Nk), the "compatibility matrix" restricted to idx
        S = scale * (q[b, h, idx, :] @ k[b, kvh].T)
        mask = window_mask(idx, Nq, Nk, causal, window)
        P, m, l = softmax_rows(S, mask)
        O = P @ v[b, kvh]
        with np.errstate(divide="ignore"):
            lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
        outs[(b, h)], lses[(b, h)] = O, lse
        if return_probs:
            probs[(b, h)] = P
    if rows is not None:
        return (outs, lses, probs) if return_probs else (outs, lses)
    O = np.zeros((B, H, Nq, d))
    LSE = np.zeros((B, H, Nq))
    for (b, h) in pairs:
        O[b, h], LSE[b, h] = outs[(b, h)], lses[(b, h)]
    return (O, LSE, probs) if return_probs else (O, LSE)


def attention_backward(q, k, v, do, *, causal: bool, scale: float, window=None):
    """Gradients of O = softmax(scale Q K^T + mask) V, in float64 (dense).

    The forward's definition (page "Donanıma Duyarlı Algoritma Tasarımı:
    FlashAttention", section "Transformer Mimarisi ve Self-Attention Mekanizması")
    differentiated by the chain rule, per (b, h), with P the probability matrix:
    dV = P^T dO; dP = dO V^T; dS = P * (dP - rowsum(dP * P)) (softmax's Jacobian
    applied row by row); dQ = scale dS K; dK = scale dS^T Q. Under GQA, dK and dV of a
    K/V head sum over the query heads that read it. The forward keeps no P for this:
    the backward recomputes it from Q, K and the rows' statistics (section
    "FlashAttention'ın Temelleri", recomputation instead of storing intermediates).
    Returns (dq [B,H,Nq,d], dk, dv [B,Hkv,Nk,d]).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    g = H // Hkv
    mask = window_mask(np.arange(Nq), Nq, Nk, causal, window)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            kvh = h // g
            S = scale * (q[b, h] @ k[b, kvh].T)
            P, _, _ = softmax_rows(S, mask)
            dO = do[b, h]
            dv[b, kvh] += P.T @ dO
            dP = dO @ v[b, kvh].T
            dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dq[b, h] = scale * (dS @ k[b, kvh])
            dk[b, kvh] += scale * (dS.T @ q[b, h])
    return dq, dk, dv


def decode(q, k_seq, v_seq, *, scale: float):
    """Single-token decode against per-sequence cached K/V, in float64.

    q: [S, H, d]; k_seq[s], v_seq[s]: [L_s, Hkv, d] (the contiguous cache of sequence
    s, current token included). Every query attends all L_s keys (no mask).
    Returns O [S, H, d] and LSE [S, H].
    """
    q = _as_f64(q)
    S, H, d = q.shape
    O = np.zeros((S, H, d))
    LSE = np.full((S, H), NEG_INF)
    for s in range(S):
        ks, vs = _as_f64(k_seq[s]), _as_f64(v_seq[s])
        L, Hkv, _ = ks.shape
        if L == 0:
            continue
        g = H // Hkv
        for h in range(H):
            kvh = h // g
            sc = scale * (ks[:, kvh, :] @ q[s, h])          # [L]
            P, m, l = softmax_rows(sc[None, :], np.ones((1, L), dtype=bool))
            O[s, h] = P[0] @ vs[:, kvh, :]
            LSE[s, h] = m[0] + math.log(l[0])
    return O, LSE


def gather_pages(cache: np.ndarray, page_table: np.ndarray, seq_lens, page_size: int):
    """Read each sequence's tokens back out of a paged cache, in token order.

    cache: [num_pages, page_size, Hkv, d]; token t of sequence s lives in physical
    page page_table[s, t // page_size], slot t % page_size. Pure indexing (exact).
    """
    out = []
    for s, L in enumerate(np.asarray(seq_lens)):
        t = np.arange(int(L))
        out.append(cache[page_table[s, t // page_size], t % page_size])
    return out


def scatter_pages(cache: np.ndarray, page_table: np.ndarray, start_pos, new: np.ndarray,
                  page_size: int) -> np.ndarray:
    """Append new tokens to a paged cache; returns the updated copy (pure indexing).

    Glossary entry "KV Cache (Anahtar-Değer Önbelleği)": each token's K (or V) is
    stored once in the cache, after the tokens already there. new: [S, n_new, Hkv, d];
    token t of sequence s is position p = start_pos[s] + t, which lives in slot
    p % page_size of physical page page_table[s, p // page_size]. A token whose
    position is negative or past the table, or whose page id is outside
    [0, num_pages), is not stored. One token at a time, in order.
    """
    out = cache.copy()
    num_pages = cache.shape[0]
    S, n_new = new.shape[0], new.shape[1]
    max_pages = page_table.shape[1]
    for s in range(S):
        for t in range(n_new):
            p = int(start_pos[s]) + t
            if p < 0 or p >= max_pages * page_size:
                continue
            pid = int(page_table[s, p // page_size])
            if not 0 <= pid < num_pages:
                continue
            out[pid, p % page_size] = new[s, t]
    return out


def online_softmax_stats(scores_row, block_sizes, trace=None):
    """The page's blockwise softmax statistics, steps 1-5, in float64.

    Page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention", "Online Softmax
    Prensibi": per block, take its max m_new and its own sum l_new (relative to
    m_new); M_new = max(M_old, m_new); rescale L_old by exp(M_old - M_new) and
    l_new by exp(m_new - M_new); L_new is their sum. Returns (M, L) for the row.
    If ``trace`` is a list, one dict per block is appended with the step values.
    """
    s = np.asarray(scores_row, dtype=np.float64)
    M, L = NEG_INF, 0.0
    pos = 0
    for bs in block_sizes:
        blk = s[pos:pos + bs]
        pos += bs
        m_blk = np.max(blk)                       # step 1
        l_blk = np.sum(np.exp(blk - m_blk))
        M_new = max(M, m_blk)                     # step 2
        L_old = L * math.exp(M - M_new) if L else 0.0   # step 3
        l_blk = l_blk * math.exp(m_blk - M_new)   # step 4
        L = L_old + l_blk                         # step 5
        if trace is not None:
            trace.append({"m_new": float(m_blk), "l_block": float(np.sum(np.exp(blk - m_blk))),
                          "M": float(M_new), "L_old_rescaled": float(L_old), "L": float(L)})
        M = M_new
    assert pos == s.size, "block sizes must cover the row"
    return M, L


def online_attention_row(scores_row, v, block_sizes):
    """Single pass over key blocks with an output accumulator rescaled like L.

    The page keeps O for a second pass once M and L are known; the single-pass form
    multiplies the unnormalised accumulator by the same exp(M_old - M_new) factor
    as L and divides by L at the end. Both equal softmax(s) @ v in exact
    arithmetic. Returns (o, lse).
    """
    s = np.asarray(scores_row, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, L = NEG_INF, 0.0
    acc = np.zeros(v.shape[1])
    pos = 0
    for bs in block_sizes:
        blk, vb = s[pos:pos + bs], v[pos:pos + bs]
        pos += bs
        M_new = max(M, np.max(blk))
        alpha = math.exp(M - M_new) if np.isfinite(M) else 0.0
        p = np.exp(blk - M_new)
        L = L * alpha + np.sum(p)
        acc = acc * alpha + p @ vb
        M = M_new
    return acc / L, M + math.log(L)


def two_pass_attention_row(scores_row, v, block_sizes):
    """FlashAttention-1's two passes over one row's key blocks, in float64.

    Page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention", section
    "FlashAttention-1 (İki Geçişli Yaklaşım)": the first pass runs the online softmax
    over the blocks and keeps only the row's global max M and sum L
    (``online_softmax_stats``); the second pass recomputes each block's scores,
    normalises them with M and L (exp(s - M) / L) and accumulates them times the
    block's V rows. ``scores_row`` holds only the row's attended keys (masked keys
    dropped) and v their value rows. Returns (o, lse = M + ln L).
    """
    s = np.asarray(scores_row, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    M, L = online_softmax_stats(s, block_sizes)       # pass 1: statistics only
    acc = np.zeros(v.shape[1])
    pos = 0
    for bs in block_sizes:                            # pass 2: normalised blocks
        p = np.exp(s[pos:pos + bs] - M) / L
        acc = acc + p @ v[pos:pos + bs]
        pos += bs
    return acc, M + math.log(L)


def merge_partials(o_parts, lse_parts):
    """Combine attention results over disjoint key sets by their log-sum-exps.

    Each part k holds the normalised output o_k over its keys and lse_k = m_k +
    ln l_k. The whole row's LSE = ln sum_k exp(lse_k) (taken relative to the
    largest lse_k) and O = sum_k exp(lse_k - LSE) o_k; parts with lse_k = -inf
    (no keys) weigh 0. This is the same merge as steps 2-5 of the page's online
    softmax, applied to (max, sum) pairs expressed as one log-sum-exp each.
    """
    lse = np.asarray(lse_parts, dtype=np.float64)
    o = np.asarray(o_parts, dtype=np.float64)
    if lse.size == 0 or not np.isfinite(lse).any():
        return np.zeros(o.shape[1:] if o.ndim > 1 else ()), NEG_INF
    mx = np.max(lse)
    w = np.exp(lse - mx)
    tot = np.sum(w)
    LSE = mx + math.log(tot)
    return np.tensordot(w / tot, o, axes=(0, 0)), LSE
