"""The online softmax and the tiled recurrence, as the pages describe them.

Test infrastructure only (see the package docstring).

* ``online_softmax`` follows "Modern Attention: MQA, GQA, FlashAttention,
  Sliding Window and RoPE", section 3: one pass keeps a running maximum m and
  a running denominator; when a new value raises the maximum the old
  denominator is multiplied by exp(old m - new m).
* ``tiled_attention_head`` follows "Attention Is O(n^2): FlashAttention vs
  Linear Attention", section "FlashAttention - Same FLOPs, Linear Memory": an
  outer loop over query blocks, an inner loop over K/V blocks, a running row
  maximum and row sum, the accumulator rescaled by exp(old max - new max),
  and one division by the running sum at the end.  Masked logits are -inf;
  key blocks holding no visible key are skipped (they add nothing).
* ``merge_states`` combines two partial softmax states (m, l, acc).  The
  formula is missing from the extracted text of "Ch. 3", section 3.5 (only its
  lead-in survives); it is reconstructed from the rescale step above:
  M = max(m_a, m_b), l = l_a e^(m_a-M) + l_b e^(m_b-M), and the accumulator
  scaled the same way.  It is exact algebra, since l e^m is invariant.

All arithmetic is float64.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _f64


def online_softmax(xs):
    """Softmax of a list by the one-pass recurrence.

    Returns (probabilities, final running max, final running denominator).
    """
    m, den = -math.inf, 0.0
    for x in xs:
        new_m = max(m, x)
        den = den * math.exp(m - new_m) + math.exp(x - new_m)
        m = new_m
    return [math.exp(x - m) / den for x in xs], m, den


def _rescale(old_m, new_m):
    """exp(old - new), taken as 0 where both are -inf (nothing seen yet)."""
    out = np.zeros_like(old_m)
    ok = np.isfinite(new_m)
    out[ok] = np.exp(old_m[ok] - new_m[ok])
    return out


def merge_states(a, b):
    """Combine two partial states (m [R], l [R], acc [R, dv]) of one row set."""
    m_a, l_a, acc_a = (np.asarray(x, dtype=np.float64) for x in a)
    m_b, l_b, acc_b = (np.asarray(x, dtype=np.float64) for x in b)
    M = np.maximum(m_a, m_b)
    fa = _rescale(m_a, M)
    fb = _rescale(m_b, M)
    return M, l_a * fa + l_b * fb, acc_a * fa[:, None] + acc_b * fb[:, None]


def tiled_attention_head(q, k, v, scale: float, causal: bool = False, window: int = 0,
                         block_q: int = 32, block_k: int = 32, return_stats: bool = False):
    """Online-softmax attention for one head; q [Nq, d], k [Nk, d], v [Nk, dv].

    Returns (O [Nq, dv], LSE [Nq]), plus the number of (query block, key
    block) pairs visited when ``return_stats``.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    Nq, Nk, dv = q.shape[0], k.shape[0], v.shape[1]
    delta = Nk - Nq
    out = np.zeros((Nq, dv))
    lse = np.full(Nq, -np.inf)
    visited = 0
    for i0 in range(0, Nq, block_q):
        i1 = min(i0 + block_q, Nq)
        pos = np.arange(i0, i1)[:, None] + delta
        acc = np.zeros((i1 - i0, dv))
        run_max = np.full(i1 - i0, -np.inf)
        run_sum = np.zeros(i1 - i0)
        for j0 in range(0, Nk, block_k):
            j1 = min(j0 + block_k, Nk)
            j = np.arange(j0, j1)[None, :]
            vis = np.ones((i1 - i0, j1 - j0), dtype=bool)
            if causal:
                vis &= j <= pos
            if window > 0:
                vis &= (pos - j) < window
            if not vis.any():
                continue  # a block with no visible key changes nothing
            visited += 1
            s = np.where(vis, (q[i0:i1] @ k[j0:j1].T) * scale, -np.inf)
            new_max = np.maximum(run_max, s.max(axis=1))
            p = np.zeros_like(s)
            live = np.isfinite(new_max)
            p[live] = np.exp(s[live] - new_max[live, None])
            corr = _rescale(run_max, new_max)
            run_sum = run_sum * corr + p.sum(axis=1)
            acc = acc * corr[:, None] + p @ v[j0:j1]
            run_max = new_max
        live = run_sum > 0
        out[i0:i1][live] = acc[live] / run_sum[live, None]
        l_blk = np.full(i1 - i0, -np.inf)
        l_blk[live] = run_max[live] + np.log(run_sum[live])
        lse[i0:i1] = l_blk
    if return_stats:
        return out, lse, visited
    return out, lse
