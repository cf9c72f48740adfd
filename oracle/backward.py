"""fp64 gradients of exact softmax attention — test infrastructure only.

What it computes: the gradients dQ, dK, dV of the loss L = sum(dO * O),
where O is the plain attention of ``oracle.attention`` (same masks, same
query-head to KV-head map) and dO is given.

The pages fix the method in words only: the backward pass recomputes the
local probabilities from the statistics saved by the forward pass instead of
storing the attention matrix ("Ch. 3: MHA Limitations, MQA, GQA, and
FlashAttention", section 3.5), and the forward keeps a float32 log-sum-exp
for it ("Attention Is O(n^2): FlashAttention vs Linear Attention", section
"FlashAttention - Same FLOPs, Linear Memory", its memory estimate).  They
print no gradient formula, so the oracle is the derivative of the
definition, written out with every matrix materialised:

    S = scale * Q K^T (masked keys -inf),  P = row softmax of S,  O = P V
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij               (equal to sum_c dO_ic O_ic)
    dS = P * (dP - D)                    (elementwise; D broadcast over keys)
    dQ = scale * dS K,   dK = scale * dS^T Q

A key that a row cannot see has P = 0 there and gets no gradient from that
row; a row that sees no key contributes nothing.  A KV head shared by G query
heads receives the sum of the G heads' dK and dV.

Pinned by central finite differences of the forward oracle and by closed
forms (``tests/test_oracle_backward.py``).  Everything is float64.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, visible_mask


def attention_backward_head(q, k, v, do, scale: float, causal: bool = False, window: int = 0,
                            row_chunk: int = 1024):
    """One (batch, query-head) pair: q [Nq, d], k [Nk, d], v [Nk, dv], do [Nq, dv].

    Returns (dQ [Nq, d], dK [Nk, d], dV [Nk, dv], D [Nq]) in float64.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    do = _f64(do)
    Nq, Nk = q.shape[0], k.shape[0]
    scale = float(scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsum = np.zeros(Nq)
    if Nk == 0 or Nq == 0:
        return dq, dk, dv, dsum
    for c0 in range(0, Nq, row_chunk):
        r = np.arange(c0, min(Nq, c0 + row_chunk))
        s = (q[r] @ k.T) * scale
        vis = visible_mask(Nq, Nk, causal, window, rows=r)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1)
        live = np.isfinite(m)
        p = np.zeros_like(s)
        p[live] = np.exp(s[live] - m[live, None])
        P = np.zeros_like(p)
        P[live] = p[live] / p[live].sum(axis=1)[:, None]    # softmax rows
        dv += P.T @ do[r]                                    # dV = P^T dO
        dp = do[r] @ v.T                                     # dP = dO V^T
        D = (P * dp).sum(axis=1)                             # D_i = sum_j P_ij dP_ij
        ds = P * (dp - D[:, None])                           # dS = P (dP - D)
        dq[r] = scale * (ds @ k)                             # dQ = scale dS K
        dk += scale * (ds.T @ q[r])                          # dK = scale dS^T Q
        dsum[r] = D
    return dq, dk, dv, dsum


def attention_backward(q, k, v, do, scale=None, causal: bool = False, window: int = 0,
                       heads=None, row_chunk: int = 1024):
    """Batched gradients in the [B, N, H, d] layout.

    q, do [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d]; query head h reads KV head
    h // (Hq // Hkv).  Returns (dQ [B, Nq, Hq, d], dK [B, Nk, Hkv, d],
    dV [B, Nk, Hkv, d], D [B, Hq, Nq]).  With ``heads`` (a list of (b, h)
    pairs) only those query heads are computed and only their contributions
    are added into dK and dV (the other entries stay zero).
    """
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dQ = np.zeros((B, Nq, Hq, d))
    dK = np.zeros((B, Nk, Hkv, d))
    dV = np.zeros((B, Nk, Hkv, v.shape[3]))
    Dsum = np.zeros((B, Hq, Nq))
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in pairs:
        hk = h // G
        dq, dk, dv, D = attention_backward_head(q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :],
                                                do[b, :, h, :], scale, causal, window, row_chunk)
        dQ[b, :, h, :] = dq
        dK[b, :, hk, :] += dk
        dV[b, :, hk, :] += dv
        Dsum[b, h, :] = D
    return dQ, dK, dV, Dsum
