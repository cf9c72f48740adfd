"""Partial softmax states and their exact merge; a key-blocked CPU model.

Test infrastructure only (see the package docstring).

The online softmax of "Modern Attention: MQA, GQA, FlashAttention, Sliding
Window and RoPE", section 3, and the key-block loop of "Attention Is O(n^2):
FlashAttention vs Linear Attention", section "FlashAttention - Same FLOPs,
Linear Memory", rest on one fact: the softmax state of a set of logits,

    m = max of the logits,   l = sum of exp(logit - m),
    acc = sum of exp(logit - m) * value,

can be formed for disjoint pieces separately and combined exactly, because
l * e^m (and acc * e^m) is the same whatever reference maximum is used.  This
module is written in those terms: a state per piece, an associative combine,
and a fold.

* ``merge_states`` is the combine: M = max(m_a, m_b), and l and acc are each
  side rescaled by exp(m - M) and added.  The formula itself is missing from
  the extracted text of "Ch. 3", section 3.5 (only its lead-in survives); this
  is the rescale those pages describe, applied to two states.
* ``online_softmax`` folds single-logit states (m = x, l = 1) with the
  combine, which gives the page's running maximum and denominator after each
  prefix; the probabilities are exp(x - m) / l.
* ``tiled_attention_head`` forms one state per (query block, key block) from
  that block's masked logits, skips key blocks with no visible key, and folds
  each query block's states in key order.  It is a model of the GPU kernel's
  tiling (which blocks are visited), checked against the plain definition.

All arithmetic is float64.
"""
from __future__ import annotations

import functools
import math

import numpy as np

from .attention import _f64


def _rescale(old_m, new_m):
    """exp(old - new), taken as 0 where the new maximum is -inf (nothing seen)."""
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


def _logit_state(x: float):
    """The state of a single logit: its own maximum, weight exp(0) = 1."""
    return np.array([float(x)]), np.array([1.0]), np.zeros((1, 0))


def online_softmax(xs):
    """Softmax of a list as a fold of single-logit states.

    Returns (probabilities, final maximum, final denominator).
    """
    empty = (np.array([-math.inf]), np.array([0.0]), np.zeros((1, 0)))
    m, l, _ = functools.reduce(merge_states, map(_logit_state, xs), empty)
    m, l = float(m[0]), float(l[0])
    return [math.exp(x - m) / l for x in xs], m, l


def _block_state(s, v):
    """State of one block of masked logits s [R, C] (-inf = hidden) with its
    values v [C, dv]: per row the block maximum, the sum of exp(s - max) and
    the exp-weighted sum of the values."""
    m = s.max(axis=1)
    w = np.zeros_like(s)
    live = np.isfinite(m)
    w[live] = np.exp(s[live] - m[live, None])
    return m, w.sum(axis=1), w @ v


def tiled_attention_head(q, k, v, scale: float, causal: bool = False, window: int = 0,
                         block_q: int = 32, block_k: int = 32, return_stats: bool = False):
    """Key-blocked attention for one head; q [Nq, d], k [Nk, d], v [Nk, dv].

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
        rows = np.arange(i0, min(i0 + block_q, Nq))
        pos = rows[:, None] + delta  # absolute positions (bottom-right causal)
        states = []
        for j0 in range(0, Nk, block_k):
            keys = np.arange(j0, min(j0 + block_k, Nk))[None, :]
            vis = np.ones((rows.size, keys.size), dtype=bool)
            if causal:
                vis &= keys <= pos
            if window > 0:
                vis &= (pos - keys) < window
            if not vis.any():
                continue  # a block with no visible key contributes nothing
            visited += 1
            s = np.where(vis, (q[rows] @ k[keys[0]].T) * scale, -np.inf)
            states.append(_block_state(s, v[keys[0]]))
        if not states:
            continue  # rows that see no key: O = 0, LSE = -inf
        m, l, acc = functools.reduce(merge_states, states)
        live = l > 0
        out[rows[live]] = acc[live] / l[live, None]
        lse[rows[live]] = m[live] + np.log(l[live])
    if return_stats:
        return out, lse, visited
    return out, lse
