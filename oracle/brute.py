"""Pure-Python brute-force attention for tiny inputs (n <= 16, d <= 8).

Test infrastructure only (see the package docstring).

This is a second, independent statement of the definition used to pin the
NumPy oracle: nested Python loops, ``math.fsum`` for every sum, and the
textbook softmax exp(s_j) / sum_k exp(s_k) *without* subtracting the row
maximum (safe at these sizes), so that it shares neither code nor evaluation
order with ``oracle.attention``.

Definition: "Attention Is O(n^2): FlashAttention vs Linear Attention",
section "Why Attention Is O(n^2)" (A = softmax(Q K^T / sqrt(d_k)) V);
"Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", section 3.3 (query
head i reads K/V group i // (H // G)); "Modern Attention", section 4 (a token
sees the last W tokens, itself included).  Causal alignment is bottom-right
(query row i at position i + Nk - Nq).
"""
from __future__ import annotations

import math


def attention_brute(q, k, v, scale: float, causal: bool = False, window: int = 0):
    """q [B][Nq][Hq][d], k and v [B][Nk][Hkv][d] as nested lists of floats.

    Returns (O [B][Nq][Hq][d], LSE [B][Hq][Nq]) as nested lists.
    """
    B, Nq, Hq, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Nk, Hkv = len(k[0]), len(k[0][0])
    dv = len(v[0][0][0])
    group = Hq // Hkv
    O = [[[[0.0] * dv for _ in range(Hq)] for _ in range(Nq)] for _ in range(B)]
    LSE = [[[-math.inf] * Nq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for i in range(Nq):
                pos = i + (Nk - Nq)
                keys = []
                for j in range(Nk):
                    if causal and j > pos:
                        continue
                    if window > 0 and pos - j >= window:
                        continue
                    keys.append(j)
                if not keys:
                    continue
                w = {}
                for j in keys:
                    s = scale * math.fsum(q[b][i][h][c] * k[b][j][g][c] for c in range(d))
                    w[j] = math.exp(s)
                total = math.fsum(w.values())
                for c in range(dv):
                    O[b][i][h][c] = math.fsum(w[j] * v[b][j][g][c] for j in keys) / total
                LSE[b][h][i] = math.log(total)
    return O, LSE
