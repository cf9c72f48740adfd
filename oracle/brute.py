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


def attention_brute_packed(q, k, v, cu_q, cu_k, scale: float, causal: bool = False,
                           window: int = 0):
    """Packed sequences over one token axis, by brute force (tiny inputs).

    q [total_q][Hq][d], k and v [total_k][Hkv][d] as nested lists; cu_q, cu_k
    the boundary offsets (sequence s owns rows cu[s] .. cu[s+1]-1).  Every
    packed query row is tested against every packed key row: the key is seen
    when both belong to the same sequence and the key's index within it passes
    the causal and window tests at the row's position within it (bottom-right:
    row i of a sequence with nq queries and nk keys sits at i + nk - nq).

    Returns (O [total_q][Hq][d], LSE [Hq][total_q]); a row outside every
    sequence, or seeing no key, gives O = 0 and LSE = -inf.
    """
    total_q, Hq, d = len(q), len(q[0]) if q else 0, len(q[0][0]) if q else 0
    total_k = len(k)
    Hkv = len(k[0]) if k else 1
    dv = len(v[0][0]) if v else d
    group = Hq // Hkv if Hq else 1
    S = len(cu_q) - 1

    def owner(cu, t):
        for s in range(S):
            if cu[s] <= t < cu[s + 1]:
                return s
        return -1

    O = [[[0.0] * dv for _ in range(Hq)] for _ in range(total_q)]
    LSE = [[-math.inf] * total_q for _ in range(Hq)]
    for i in range(total_q):
        s = owner(cu_q, i)
        if s < 0:
            continue
        nq, nk = cu_q[s + 1] - cu_q[s], cu_k[s + 1] - cu_k[s]
        pos = (i - cu_q[s]) + (nk - nq)
        keys = []
        for j in range(total_k):
            if owner(cu_k, j) != s:
                continue
            jj = j - cu_k[s]
            if causal and jj > pos:
                continue
            if window > 0 and pos - jj >= window:
                continue
            keys.append(j)
        if not keys:
            continue
        for h in range(Hq):
            g = h // group
            w = {j: math.exp(scale * math.fsum(q[i][h][c] * k[j][g][c] for c in range(d)))
                 for j in keys}
            total = math.fsum(w.values())
            for c in range(dv):
                O[i][h][c] = math.fsum(w[j] * v[j][g][c] for j in keys) / total
            LSE[h][i] = math.log(total)
    return O, LSE


def prefill_paged_brute(q, kcache, vcache, block_table, seq_lens, cu_q, scale: float,
                        window: int = 0):
    """Chunked prefill over a paged cache by brute force (tiny inputs).

    q [total_q][Hq][d]; kcache, vcache [num_blocks][block_size][Hkv][d];
    block_table [S][max_blocks]; seq_lens [S]; cu_q [S + 1], all nested lists.
    Each sequence's cached tokens are copied out one by one through the table
    (token t: block table[s][t // block_size], slot t % block_size), then the
    dense brute force runs on that sequence with the chunk's queries as the
    last rows (bottom-right causal).  Returns (O [total_q][Hq][d],
    LSE [Hq][total_q]); every block id must be valid.
    """
    total_q = len(q)
    Hq, d = len(q[0]), len(q[0][0])
    bs = len(kcache[0])
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(total_q)]
    LSE = [[-math.inf] * total_q for _ in range(Hq)]
    for s in range(len(seq_lens)):
        n = seq_lens[s]
        kk = [kcache[block_table[s][t // bs]][t % bs] for t in range(n)]
        vv = [vcache[block_table[s][t // bs]][t % bs] for t in range(n)]
        rows = q[cu_q[s]:cu_q[s + 1]]
        if not rows:
            continue
        if n == 0:
            continue
        o, l = attention_brute([rows], [kk], [vv], scale, causal=True, window=window)
        for i in range(len(rows)):
            for h in range(Hq):
                O[cu_q[s] + i][h] = o[0][i][h]
                LSE[h][cu_q[s] + i] = l[0][h][i]
    return O, LSE
