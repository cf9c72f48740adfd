"""Algorithmic work counts used to report throughput and roofline fractions.

FLOPs: 4 * d per visible (query, key) pair — 2 flops per multiply-add in each
of the two products Q K^T and P V; exp, max and sums are not counted.  For a
square, unmasked score matrix this is twice the per-head figure of "Attention
Is O(n^2): FlashAttention vs Linear Attention" (section "Why Attention Is
O(n^2)"), which counts only Q K^T.  Causal and windowed runs count only the
visible pairs.

Bytes: every input read once and every output written once — Q, K, V, O and
LSE for the forward pass ("Attention Is O(n^2)", section "What FLOPs Can't Be
Avoided": the tiled method's traffic is Q, K, V in and O out), and for paged
decode the used K/V slots of each sequence (once per KV head, however many
query heads share it), the queries, outputs, LSE, the used block-table
entries and the lengths.  Split-K partials are an implementation artefact
and are not counted.
"""
from __future__ import annotations

import numpy as np

# MI355X published peaks
PEAK_BF16_TFLOPS = 2516.6    # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_F32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def visible_pairs(Nq: int, Nk: int, causal: bool, window: int) -> int:
    """Number of (query, key) pairs a mask leaves visible, for one head.

    Query row i sits at position i + Nk - Nq; causal keeps keys j <= position,
    a window W > 0 keeps keys with position - j < W.
    """
    pos = np.arange(Nq, dtype=np.int64) + (Nk - Nq)
    hi = np.minimum(pos, Nk - 1) if causal else np.full(Nq, Nk - 1, dtype=np.int64)
    lo = np.maximum(pos - window + 1, 0) if window > 0 else np.zeros(Nq, dtype=np.int64)
    return int(np.clip(hi - lo + 1, 0, None).sum())


def fwd_flops(B: int, Hq: int, Nq: int, Nk: int, d: int, causal: bool, window: int) -> float:
    return 4.0 * d * visible_pairs(Nq, Nk, causal, window) * B * Hq


def varlen_fwd_flops(lens_q, lens_k, Hq: int, d: int, causal: bool, window: int) -> float:
    """Forward flops of packed sequences: each sequence's own visible pairs."""
    pairs = sum(visible_pairs(int(a), int(b), causal, window) for a, b in zip(lens_q, lens_k))
    return 4.0 * d * pairs * Hq


def prefill_paged_flops(seq_lens, chunks, Hq: int, d: int, window: int) -> float:
    """Chunked prefill: each chunk's visible pairs against its sequence's cache."""
    pairs = sum(visible_pairs(int(c), int(n), True, window) for n, c in zip(seq_lens, chunks))
    return 4.0 * d * pairs * Hq


def bwd_flops(B: int, Hq: int, Nq: int, Nk: int, d: int, causal: bool, window: int) -> float:
    """Algorithmic flops of the backward pass: five products the size of the
    forward's two (S recomputed, dP = dO V^T, dV, dK, dQ), i.e. 2.5x forward."""
    return 2.5 * fwd_flops(B, Hq, Nq, Nk, d, causal, window)


def bwd_executed_flops(B: int, Hq: int, Nq: int, Nk: int, d: int, causal: bool,
                       window: int) -> float:
    """Flops the backward kernels execute on the visible pairs: the dK/dV pass
    forms S, dP, dV and dK, the dQ pass S, dP and dQ again: seven products the
    size of the forward's two, 3.5x forward."""
    return 3.5 * fwd_flops(B, Hq, Nq, Nk, d, causal, window)


def fwd_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, elt: int = 2,
              with_lse: bool = True) -> int:
    qo = 2 * B * Nq * Hq * d * elt
    kv = 2 * B * Nk * Hkv * d * elt
    lse = B * Hq * Nq * 4 if with_lse else 0
    return qo + kv + lse


def decode_bytes(seq_lens, Hq: int, Hkv: int, d: int, block_size: int, elt: int = 2,
                 with_lse: bool = True) -> int:
    lens = np.asarray(seq_lens, dtype=np.int64)
    B = lens.shape[0]
    kv = int(lens.sum()) * Hkv * d * elt * 2
    qo = 2 * B * Hq * d * elt
    lse = B * Hq * 4 if with_lse else 0
    table = int(((lens + block_size - 1) // block_size).sum()) * 4
    return kv + qo + lse + table + B * 4


def kv_cache_bytes(B: int, layers: int, kv_heads: int, head_dim: int, tokens: int,
                   elt: int) -> int:
    """Dense KV cache size: K and V for every layer, KV head, position and element."""
    return 2 * B * layers * kv_heads * head_dim * tokens * elt
