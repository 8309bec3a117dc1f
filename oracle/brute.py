"""Pure-Python scalar attention for tiny shapes (an independent second code path).

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): used to pin the
NumPy oracle by brute force. Triple loops over Python floats, ``math.exp`` and
``math.fsum``; no NumPy arithmetic at all.

Definition followed: page "Donanıma Duyarlı Algoritma Tasarımı: FlashAttention",
section "Transformer Mimarisi ve Self-Attention Mekanizması" (softmax of the scaled
Q K^T rows, then the weighted sum of V rows). Causal rows attend keys j <= i +
(Nk - Nq); a sliding window (glossary entry "Kayan Pencere Dikkati") keeps the keys
within (left, right) of the query's position; query head h uses key/value head
h // (H // Hkv).
"""
from __future__ import annotations

import math


def attention_brute(q, k, v, causal, scale, window=None):
    """q: nested lists [B][H][Nq][d]; k, v: [B][Hkv][Nk][d]. Returns (O, LSE) lists.
    window: None or (left, right); query i at position p = i + Nk - Nq sees keys
    p - left .. p + right (-1: that side unbounded)."""
    B, H = len(q), len(q[0])
    Nq, d = len(q[0][0]), len(q[0][0][0])
    Hkv, Nk = len(k[0]), len(k[0][0])
    g = H // Hkv
    O = [[[[0.0] * d for _ in range(Nq)] for _ in range(H)] for _ in range(B)]
    LSE = [[[0.0] * Nq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            kh = h // g
            for i in range(Nq):
                p = i + (Nk - Nq)
                keys = [j for j in range(Nk) if (not causal) or j <= p]
                if window is not None:
                    lo = p - window[0] if window[0] >= 0 else -math.inf
                    hi = p + window[1] if window[1] >= 0 else math.inf
                    keys = [j for j in keys if lo <= j <= hi]
                if not keys:
                    LSE[b][h][i] = -math.inf
                    continue
                s = {j: scale * math.fsum(q[b][h][i][c] * k[b][kh][j][c] for c in range(d))
                     for j in keys}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in keys}
                tot = math.fsum(e.values())
                for c in range(d):
                    O[b][h][i][c] = math.fsum(e[j] * v[b][kh][j][c] for j in keys) / tot
                LSE[b][h][i] = m + math.log(tot)
    return O, LSE
