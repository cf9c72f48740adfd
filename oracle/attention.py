"""Naive fp64 attention — the plain definition, materialising S and P.

Test infrastructure only (see the package docstring).

Definition followed:
  * "Attention Is O(n^2): FlashAttention vs Linear Attention", section "Why
    Attention Is O(n^2)": A = softmax(Q K^T / sqrt(d_k)) V for one layer and
    head; section "Wall-Clock Impact of Tiling", the naive NumPy version, which
    subtracts the row maximum before exponentiating.
  * "Ch. 3: MHA Limitations, MQA, GQA, and FlashAttention", section 3.5:
    naive attention forms S = Q K^T, then P = softmax(S), then P V; section 3.3:
    query head i reads K/V group i // (H // G) (contiguous groups, the
    repeat-interleave construction).
  * "Modern Attention: MQA, GQA, FlashAttention, Sliding Window and RoPE",
    section 4: token i may look at the last W tokens, itself included (the
    n = 8, W = 3 picture has three allowed keys per full row, 21 in all).
  * "Inference Engineering", section 2.5 "Optimizing Attention": a paged KV
    cache is split into fixed-size blocks reached through a lookup table.

Readings where the pages are silent (each also listed in the design notes):
  * causal alignment when Nq != Nk is bottom-right: query row i sits at
    absolute position i + (Nk - Nq), so a single decode query sees the whole
    cache;
  * a row with no visible key gives O = 0 and LSE = -inf;
  * LSE is the natural log of the sum of exp over the scaled, masked logits,
    laid out [B, Hq, Nq];
  * a paged sequence whose table names a block outside the pool gives NaN.

Everything here is float64.  Inputs may be numpy arrays or CPU torch tensors
of any float dtype; they are widened exactly to float64.
"""
from __future__ import annotations

import numpy as np

try:  # torch is only used to widen bf16 tensors; numpy does all arithmetic
    import torch
except ImportError:  # pragma: no cover
    torch = None


def _f64(x) -> np.ndarray:
    if torch is not None and isinstance(x, torch.Tensor):
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def visible_mask(Nq: int, Nk: int, causal: bool, window: int, rows=None) -> np.ndarray:
    """Boolean [len(rows), Nk]: may query row i attend to key j?

    Row i sits at absolute position i + (Nk - Nq).  Causal: j <= position.
    Window W > 0: position - j < W (the last W keys, the query's own included).
    """
    if rows is None:
        rows = np.arange(Nq)
    pos = np.asarray(rows, dtype=np.int64)[:, None] + (Nk - Nq)
    j = np.arange(Nk, dtype=np.int64)[None, :]
    vis = np.ones((pos.shape[0], Nk), dtype=bool)
    if causal:
        vis &= j <= pos
    if window > 0:
        vis &= (pos - j) < window
    return vis


def attention_head(q, k, v, scale: float, causal: bool = False, window: int = 0,
                   rows=None, row_chunk: int = 1024, return_p: bool = False):
    """One (batch, query-head) pair.

    q [Nq, d], k [Nk, d], v [Nk, dv].  Returns (O [R, dv], LSE [R]) for the
    requested rows R (all rows by default), and P [R, Nk] when ``return_p``.
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    Nq, Nk = q.shape[0], k.shape[0]
    scale = float(scale)
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((R, v.shape[1]), dtype=np.float64)
    lse = np.full((R,), -np.inf, dtype=np.float64)
    p_all = np.zeros((R, Nk), dtype=np.float64) if return_p else None
    if Nk == 0:
        return (out, lse, p_all) if return_p else (out, lse)
    for c0 in range(0, R, row_chunk):
        r = rows[c0: c0 + row_chunk]
        s = (q[r] @ k.T) * scale                      # S = scale * Q K^T
        vis = visible_mask(Nq, Nk, causal, window, rows=r)
        s = np.where(vis, s, -np.inf)                 # additive -inf mask
        m = s.max(axis=1)                             # row maximum
        live = np.isfinite(m)
        p = np.zeros_like(s)
        p[live] = np.exp(s[live] - m[live, None])     # unnormalised weights
        l = p.sum(axis=1)                             # row sum
        P = np.zeros_like(p)
        P[live] = p[live] / l[live, None]             # softmax rows
        out[c0: c0 + r.shape[0]] = P @ v              # O = P V
        lse_c = np.full(r.shape[0], -np.inf)
        lse_c[live] = m[live] + np.log(l[live])
        lse[c0: c0 + r.shape[0]] = lse_c
        if return_p:
            p_all[c0: c0 + r.shape[0]] = P
    return (out, lse, p_all) if return_p else (out, lse)


def attention(q, k, v, scale=None, causal: bool = False, window: int = 0, heads=None,
              rows=None, row_chunk: int = 1024):
    """Batched, multi-head attention in the [B, N, H, d] layout.

    q [B, Nq, Hq, d]; k, v [B, Nk, Hkv, d] with Hq divisible by Hkv.  Query
    head h reads KV head h // (Hq // Hkv).

    With ``heads=None`` returns (O [B, Nq, Hq, dv], LSE [B, Hq, Nq]) for every
    head.  With a list of (b, h) pairs returns {(b, h): (O [R, dv], LSE [R])},
    computing only those heads (and only ``rows`` when given).
    """
    B, Nq, Hq, d = q.shape
    Bk, Nk, Hkv, dk = k.shape
    if Bk != B or dk != d or v.shape[:3] != k.shape[:3]:
        raise ValueError("q, k, v shapes disagree")
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    res = {}
    for b, h in pairs:
        hk = h // G
        res[(b, h)] = attention_head(q[b, :, h, :], k[b, :, hk, :], v[b, :, hk, :], scale,
                                     causal, window, rows=rows, row_chunk=row_chunk)
    if heads is not None:
        return res
    dv = v.shape[3]
    O = np.zeros((B, Nq, Hq, dv), dtype=np.float64)
    L = np.zeros((B, Hq, Nq), dtype=np.float64)
    for (b, h), (o, l) in res.items():
        O[b, :, h, :] = o
        L[b, h, :] = l
    return O, L


def gather_paged(cache, table_row, seq_len: int):
    """Contiguous [seq_len, Hkv, d] float64 from a paged cache.

    Logical token t lives in block table_row[t // block_size], slot
    t % block_size.  Returns None when a needed block id is outside the pool.
    """
    nb, bs = cache.shape[0], cache.shape[1]
    ids = np.asarray(table_row, dtype=np.int64)[: (seq_len + bs - 1) // bs]
    if seq_len > 0 and (ids.min() < 0 or ids.max() >= nb):
        return None
    t = np.arange(seq_len)
    blk = ids[t // bs]
    slot = t % bs
    if torch is not None and isinstance(cache, torch.Tensor):
        g = cache[torch.from_numpy(blk), torch.from_numpy(slot)]
        return _f64(g)
    return _f64(np.asarray(cache)[blk, slot])


def decode_paged(q, kcache, vcache, block_table, seq_lens, scale, window: int = 0,
                 seqs=None):
    """Single-query decode over a paged cache.

    q [B, Hq, d] holds the query of the token at position seq_len - 1, whose
    own K/V are already in the cache ("Ch. 3", section 3.1: the new token's
    K/V are appended before it attends).  kcache, vcache
    [num_blocks, block_size, Hkv, d]; block_table [B, max_blocks]; seq_lens [B].
    The query attends every cached token (or the last ``window`` of them).

    Returns (O [B, Hq, d], LSE [B, Hq]) in float64; sequences not in ``seqs``
    are left NaN.
    """
    B, Hq, d = q.shape
    Hkv = kcache.shape[2]
    G = Hq // Hkv
    table = np.asarray(block_table.numpy() if hasattr(block_table, "numpy") else block_table)
    lens = np.asarray(seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens)
    O = np.full((B, Hq, d), np.nan)
    L = np.full((B, Hq), np.nan)
    for b in (range(B) if seqs is None else seqs):
        n = int(lens[b])
        kc = gather_paged(kcache, table[b], n)
        vc = gather_paged(vcache, table[b], n)
        if kc is None or vc is None:
            continue  # bad block id: NaN
        qb = _f64(q[b])
        for h in range(Hq):
            o, l = attention_head(qb[h][None, :], kc[:, h // G, :], vc[:, h // G, :], scale,
                                  causal=True, window=window)
            O[b, h] = o[0]
            L[b, h] = l[0]
    return O, L


def prefill_paged(q, kcache, vcache, block_table, seq_lens, cu_seqlens_q, scale,
                  window: int = 0, seqs=None):
    """Chunked prefill over a paged cache: several new tokens per sequence.

    Sequence s has seq_lens[s] cached tokens, the last Nq_s of which are its
    new tokens, whose queries are rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1
    of q [total_q, Hq, d]; their K/V are already in the cache ("Ch. 3",
    section 3.1: a new token's K/V are appended before it attends; the GQA
    code of its section 3.3 notes that attention over a cache needs its own
    causal handling, the plain causal flag covering only equal lengths).  Query row i of the chunk sits at position seq_len - Nq_s + i
    and sees the cached tokens up to that position (the last ``window`` of
    them when window > 0): bottom-right causal, as in ``attention_head``.

    Returns (O [total_q, Hq, d], LSE [Hq, total_q]) in float64.  A sequence
    whose table names a block outside the pool, or whose length is negative,
    gets NaN; rows of sequences not in ``seqs`` stay NaN.
    """
    total_q, Hq, d = q.shape
    Hkv = kcache.shape[2]
    G = Hq // Hkv
    table = np.asarray(block_table.numpy() if hasattr(block_table, "numpy") else block_table)
    lens = np.asarray(seq_lens.numpy() if hasattr(seq_lens, "numpy") else seq_lens)
    cu = np.asarray(cu_seqlens_q.numpy() if hasattr(cu_seqlens_q, "numpy") else cu_seqlens_q)
    O = np.full((total_q, Hq, d), np.nan)
    L = np.full((Hq, total_q), np.nan)
    for s in (range(len(lens)) if seqs is None else seqs):
        n = int(lens[s])
        q0, q1 = int(cu[s]), int(cu[s + 1])
        if n < 0 or n > table.shape[1] * kcache.shape[1]:
            continue
        kc = gather_paged(kcache, table[s], n)
        vc = gather_paged(vcache, table[s], n)
        if kc is None or vc is None:
            continue  # bad block id: NaN
        qs = _f64(q[q0:q1])
        for h in range(Hq):
            o, l = attention_head(qs[:, h, :], kc[:, h // G, :], vc[:, h // G, :], scale,
                                  causal=True, window=window)
            O[q0:q1, h] = o
            L[h, q0:q1] = l
    return O, L

