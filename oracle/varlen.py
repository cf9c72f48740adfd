"""fp64 attention over packed sequences — test infrastructure only.

Several sequences of different lengths are stored back to back along one
token axis with no padding, and the offsets of their boundaries
(``cu_seqlens``: sequence s owns rows cu[s] .. cu[s+1]-1) say where each one
starts.  Each sequence attends only to itself: the masks (causal, sliding
window) and the bottom-right causal alignment apply within the sequence, and
no token sees a token of another sequence.

The pages motivate this, not define it: "How to Reduce Attention Computation
Cost in LLM Training" names packed sequence boundaries as the case that needs
variable-length ("varlen") kernels (section "FlashAttention Is Table Stakes
Now"), and counts sequence packing among the largest savings (its comparison
table, section "What Most Teams Get Wrong", and the FAQ on how much packing
helps).  So the oracle is the plain definition of ``oracle.attention``
applied to each sequence's slice.  Readings (also in the design notes):
  * a sequence with more queries than keys under a causal mask is allowed;
    its first rows see no key and give O = 0, LSE = -inf;
  * LSE is laid out [Hq, total_q] (each head's rows in token order).

Pinned by a pure-Python brute force over the whole packed axis with a
segment mask (``oracle.brute.attention_brute_packed``), and by reductions to
the dense oracle (``tests/test_oracle_varlen.py``).  The gradients are those
of ``oracle.backward`` per sequence, pinned by finite differences of
``attention_varlen`` itself.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_head
from .backward import attention_backward_head


def attention_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, scale=None, causal: bool = False,
                     window: int = 0, seqs=None, heads=None):
    """q [total_q, Hq, d]; k, v [total_k, Hkv, d]; cu_seqlens_* of length S+1.

    Returns (O [total_q, Hq, dv], LSE [Hq, total_q]) in float64.  Rows of
    sequences not computed (outside ``seqs``, or heads outside ``heads``) and
    rows outside every sequence are NaN.
    """
    total_q, Hq, d = q.shape
    Hkv = k.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    if len(cq) != len(ck):
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    S = len(cq) - 1
    O = np.full((total_q, Hq, v.shape[2]), np.nan)
    L = np.full((Hq, total_q), np.nan)
    for s in (range(S) if seqs is None else seqs):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        for h in (range(Hq) if heads is None else heads):
            hk = h // G
            o, l = attention_head(q[q0:q1, h, :], k[k0:k1, hk, :], v[k0:k1, hk, :], scale,
                                  causal, window)
            O[q0:q1, h, :] = o
            L[h, q0:q1] = l
    return O, L


def attention_varlen_backward(q, k, v, do, cu_seqlens_q, cu_seqlens_k, scale=None,
                              causal: bool = False, window: int = 0, heads=None):
    """Gradients of sum(dO * O) for ``attention_varlen``.

    Returns (dQ [total_q, Hq, d], dK [total_k, Hkv, d], dV [total_k, Hkv, dv],
    D [Hq, total_q]) in float64; a KV head's gradients sum over the query
    heads of its group.  Rows outside every sequence stay zero.  With
    ``heads`` only those query heads are computed and added in.
    """
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    cq = [int(x) for x in np.asarray(cu_seqlens_q).reshape(-1)]
    ck = [int(x) for x in np.asarray(cu_seqlens_k).reshape(-1)]
    dQ = np.zeros((total_q, Hq, d))
    dK = np.zeros((total_k, Hkv, d))
    dV = np.zeros((total_k, Hkv, v.shape[2]))
    Ds = np.zeros((Hq, total_q))
    for s in range(len(cq) - 1):
        q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]
        for h in (range(Hq) if heads is None else heads):
            hk = h // G
            dq, dk, dv, D = attention_backward_head(q[q0:q1, h, :], k[k0:k1, hk, :],
                                                    v[k0:k1, hk, :], do[q0:q1, h, :], scale,
                                                    causal, window)
            dQ[q0:q1, h] = dq
            dK[k0:k1, hk] += dk
            dV[k0:k1, hk] += dv
            Ds[h, q0:q1] = D
    return dQ, dK, dV, Ds

