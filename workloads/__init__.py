"""Seeded synthetic inputs for exact softmax attention.

This module only draws random numbers and lays them out.  It holds none of
the attention arithmetic, so both the fp64 oracle (under ``oracle/``) and the
HIP path can be fed from it without sharing any of the method.

Inputs follow the workloads the pages describe: random Q/K/V in the
``(B, N, H, d)`` layout of the fused-kernel example in "How to Reduce
Attention Computation Cost in LLM Training" (section "FlashAttention Is Table
Stakes"), head counts 32 query / 8 KV heads (same page, GQA/MQA section), a
4096-token window (same page, sliding-window section), head size 64 with
sequences up to 1024 ("Attention Is O(n^2)", section "Wall-Clock Impact of
Tiling"), and caches of up to 32000 tokens ("Ch. 3: MHA Limitations, MQA, GQA,
and FlashAttention", section 3.2).

Recipe: every tensor is viewed as rows of its last two dimensions' product
(e.g. [B*N, H*d]) and cut into fixed chunks of ``CHUNK_ROWS`` rows; chunk c of
tensor number t (Q = 0, K = 1, V = 2; for the paged cache K = 1, V = 2 per
sequence) is drawn with ``numpy.random.default_rng`` seeded by child c of
``SeedSequence([seed, t])``, ``standard_normal`` in float32.  The chunks are
independent, so they are drawn on several threads and the values do not
depend on the thread count.  bf16 tensors are rounded from those float32
values with round-to-nearest-even (torch's CPU cast).
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os

import numpy as np
import torch

__all__ = [
    "DenseConfig",
    "PagedConfig",
    "DENSE_CONFIGS",
    "PAGED_CONFIGS",
    "make_dense",
    "make_dout",
    "make_paged",
    "draw_normal",
    "PackedConfig",
    "PACKED_CONFIGS",
    "draw_lengths",
    "make_packed",
    "make_packed_config",
    "PrefillPagedConfig",
    "PREFILL_PAGED_CONFIGS",
    "make_prefill_paged",
    "make_prefill_paged_config",
]


@dataclasses.dataclass(frozen=True)
class DenseConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    window: int
    dtype: str  # "bf16" or "f32"
    seed: int

    @property
    def scale(self) -> float:
        # the fp32 value both sides use: 1/sqrt(d) rounded once to float32
        return float(np.float32(1.0 / math.sqrt(self.d)))


@dataclasses.dataclass(frozen=True)
class PagedConfig:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    len_lo: int
    len_hi: int
    window: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The five workloads: one fp32 single head, then the bf16 prefill shapes and
# the paged decode shape.
DENSE_CONFIGS = {
    "f32_single_head_256": DenseConfig("f32_single_head_256", 1, 1, 1, 256, 256, 64,
                                       False, 0, "f32", 0),
    "mha_causal_8k": DenseConfig("mha_causal_8k", 4, 32, 32, 8192, 8192, 128,
                                 True, 0, "bf16", 2),
    "gqa_causal_16k": DenseConfig("gqa_causal_16k", 2, 32, 8, 16384, 16384, 128,
                                  True, 0, "bf16", 3),
    "mqa_causal_16k": DenseConfig("mqa_causal_16k", 2, 32, 1, 16384, 16384, 128,
                                  True, 0, "bf16", 3),
    "swa_causal_32k_w4096": DenseConfig("swa_causal_32k_w4096", 1, 32, 8, 32768, 32768,
                                        128, True, 4096, "bf16", 4),
}

PAGED_CONFIGS = {
    "paged_decode_16x32k": PagedConfig("paged_decode_16x32k", 16, 32, 8, 128, 16, 40000,
                                       2000, 8000, 32000, 0, 5),
}


@dataclasses.dataclass(frozen=True)
class PackedConfig:
    """Packed sequences: lengths drawn by ``draw_lengths`` until ``total``
    tokens, each sequence's queries and keys of the same length."""
    name: str
    total: int
    mean_len: int
    max_len: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    window: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# Packed training batch: sequences averaging about 600 tokens, none longer
# than 2048 ("How to Reduce Attention Computation Cost in LLM Training",
# section "What Most Teams Get Wrong": such sequences padded to 2048), with
# the 32 heads of 128 of that page's fused-kernel example.
PACKED_CONFIGS = {
    "packed_causal_64k_mean600": PackedConfig("packed_causal_64k_mean600", 65536, 600, 2048,
                                              32, 32, 128, True, 0, 6),
}


@dataclasses.dataclass(frozen=True)
class PrefillPagedConfig:
    """Chunked prefill: B sequences with cached contexts of len_lo..len_hi
    tokens (the last ``chunk`` of them new) in a paged cache."""
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    len_lo: int
    len_hi: int
    chunk: int
    window: int
    seed: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d)))


# The paged decode batch (16 sequences of 8000..32000 cached tokens, 32 query
# and 8 KV heads of 128, 16-token blocks) taking a 512-token prefill chunk
# each instead of one token.
PREFILL_PAGED_CONFIGS = {
    "paged_prefill_16x32k_chunk512": PrefillPagedConfig("paged_prefill_16x32k_chunk512", 16,
                                                        32, 8, 128, 16, 40000, 2000, 8000,
                                                        32000, 512, 0, 7),
}


CHUNK_ROWS = 4096
_THREADS = min(16, os.cpu_count() or 1)


def _child_rngs(key, n: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(list(key)).spawn(n)]


def draw_normal(seed: int, tag: int, shape, sub=None) -> np.ndarray:
    """float32 N(0,1) of ``shape``; chunk c of CHUNK_ROWS rows uses child c of
    SeedSequence([seed, tag]) (or [seed, tag, sub])."""
    shape = tuple(int(x) for x in shape)
    cols = int(np.prod(shape[-2:])) if len(shape) >= 2 else 1
    rows = int(np.prod(shape)) // cols if cols else 0
    out = np.empty((rows, cols), dtype=np.float32)
    nchunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS
    rngs = _child_rngs([seed, tag] + ([] if sub is None else [sub]), nchunks)

    def fill(c):
        r0 = c * CHUNK_ROWS
        r1 = min(rows, r0 + CHUNK_ROWS)
        out[r0:r1] = rngs[c].standard_normal((r1 - r0, cols), dtype=np.float32)

    if nchunks > 1:
        with cf.ThreadPoolExecutor(max_workers=_THREADS) as ex:
            list(ex.map(fill, range(nchunks)))
    elif nchunks == 1:
        fill(0)
    return out.reshape(shape)


def draw_normal_device(seed: int, tag: int, shape, dtype=torch.bfloat16, device="cuda"):
    """N(0,1) of ``shape`` drawn on the device by torch's generator seeded from
    (seed, tag): for inputs too large to draw on the host (tens of GB).  The
    values differ from ``draw_normal``'s; only their seeding matches."""
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence([seed, tag]).generate_state(1, np.uint64)[0] >> 1))
    return torch.randn(tuple(int(x) for x in shape), generator=g, device=device, dtype=dtype)


def _to(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(x)
    if dtype == "bf16":
        return t.to(torch.bfloat16)
    if dtype == "f32":
        return t
    raise ValueError(f"unknown dtype {dtype!r}")


def make_dense(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, d: int, seed: int,
               dtype: str = "bf16"):
    """Q [B,Nq,Hq,d], K and V [B,Nk,Hkv,d] as CPU torch tensors (bf16 or fp32)."""
    q = _to(draw_normal(seed, 0, (B, Nq, Hq, d)), dtype)
    k = _to(draw_normal(seed, 1, (B, Nk, Hkv, d)), dtype)
    v = _to(draw_normal(seed, 2, (B, Nk, Hkv, d)), dtype)
    return q, k, v


def make_dout(B: int, Nq: int, Hq: int, d: int, seed: int, dtype: str = "bf16"):
    """The upstream gradient dO [B, Nq, Hq, d] of a backward pass (tag 3 of ``seed``)."""
    return _to(draw_normal(seed, 3, (B, Nq, Hq, d)), dtype)


def make_dense_config(cfg: DenseConfig):
    return make_dense(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, cfg.seed, cfg.dtype)


def draw_lengths(total: int, mean_len: int, max_len: int, seed: int) -> np.ndarray:
    """Sequence lengths summing to ``total``: from ``default_rng(seed)``, each
    length is 1 + floor(exponential(mean_len - 1)) clipped to ``max_len``,
    drawn until the sum reaches ``total``; the last one is cut to fit."""
    rng = np.random.default_rng(seed)
    lens = []
    left = int(total)
    while left > 0:
        n = min(int(max_len), 1 + int(rng.exponential(mean_len - 1)), left)
        lens.append(n)
        left -= n
    return np.asarray(lens, dtype=np.int64)


def make_packed(lens_q, lens_k, Hq: int, Hkv: int, d: int, seed: int, dtype: str = "bf16"):
    """Packed Q [sum(lens_q), Hq, d], K and V [sum(lens_k), Hkv, d] (tags 0, 1, 2
    of ``seed``, drawn as one tensor each) and the int32 boundaries
    cu_seqlens_q, cu_seqlens_k ([num_seqs + 1], starting at 0), as CPU tensors."""
    lq = np.asarray(lens_q, dtype=np.int64)
    lk = np.asarray(lens_k, dtype=np.int64)
    if lq.shape != lk.shape:
        raise ValueError("lens_q and lens_k differ in count")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = _to(draw_normal(seed, 0, (int(cu_q[-1]), Hq, d)), dtype)
    k = _to(draw_normal(seed, 1, (int(cu_k[-1]), Hkv, d)), dtype)
    v = _to(draw_normal(seed, 2, (int(cu_k[-1]), Hkv, d)), dtype)
    return q, k, v, torch.from_numpy(cu_q), torch.from_numpy(cu_k)


def make_packed_config(cfg: PackedConfig):
    lens = draw_lengths(cfg.total, cfg.mean_len, cfg.max_len, cfg.seed)
    return make_packed(lens, lens, cfg.Hq, cfg.Hkv, cfg.d, cfg.seed, "bf16")


def make_prefill_paged(seq_lens, chunks, Hq: int, Hkv: int, d: int, block_size: int,
                       num_blocks: int, max_blocks_per_seq: int, seed: int, poison: bool = True):
    """A paged cache as ``make_paged`` (with the given lengths) plus the new
    tokens' queries: q [sum(chunks), Hq, d] bf16 from tag 5 of ``seed`` and
    cu_seqlens_q [B + 1] int32.  Returns a dict of CPU tensors."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    inp = make_paged(len(lens), Hq, Hkv, d, block_size, num_blocks, max_blocks_per_seq, seed,
                     seq_lens=lens, poison=poison)
    ch = np.asarray(chunks, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(ch)]).astype(np.int32)
    inp["q"] = _to(draw_normal(seed, 5, (int(cu[-1]), Hq, d)), "bf16")
    inp["cu_seqlens_q"] = torch.from_numpy(cu)
    return inp


def make_prefill_paged_config(cfg: PrefillPagedConfig, poison: bool = True):
    rng = np.random.default_rng([cfg.seed, 6])
    lens = rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.B, endpoint=True)
    chunks = np.minimum(lens, cfg.chunk)
    return make_prefill_paged(lens, chunks, cfg.Hq, cfg.Hkv, cfg.d, cfg.block_size,
                              cfg.num_blocks, cfg.max_blocks_per_seq, cfg.seed, poison)


def make_paged(B: int, Hq: int, Hkv: int, d: int, block_size: int, num_blocks: int,
               max_blocks_per_seq: int, seed: int, len_lo: int = 1, len_hi: int = 1,
               seq_lens=None, poison: bool = True):
    """A block-paged KV cache with seeded contents.

    From ``default_rng(seed)``, in order: ``seq_lens`` (uniform integers in
    [len_lo, len_hi], unless given), a permutation of the physical block ids,
    then q [B,Hq,d].  The K values of sequence b's used slots, in logical order
    (t, h, c), come from ``draw_normal(seed, 1, (len_b, Hkv, d), sub=b)`` and
    the V values from tag 2 likewise.
    Sequence b takes the next ceil(len_b / block_size) ids of the permutation.
    Unused blocks and the unused tail slots of a sequence's last block hold NaN
    when ``poison`` is set, so that reading one shows up in the result.

    Returns a dict of CPU tensors: q (bf16), kcache, vcache (bf16,
    [num_blocks, block_size, Hkv, d]), block_table (int32 [B, max_blocks_per_seq],
    -1 past each sequence's end) and seq_lens (int32 [B]).
    """
    rng = np.random.default_rng(seed)
    if seq_lens is None:
        lens = rng.integers(len_lo, len_hi, size=B, endpoint=True).astype(np.int64)
    else:
        lens = np.asarray(seq_lens, dtype=np.int64)
        if lens.shape != (B,):
            raise ValueError("seq_lens must have B entries")
    nblk = [(int(n) + block_size - 1) // block_size for n in lens]
    if max(nblk, default=0) > max_blocks_per_seq:
        raise ValueError("a sequence needs more blocks than max_blocks_per_seq")
    if sum(nblk) > num_blocks:
        raise ValueError("pool too small for the drawn lengths")
    perm = rng.permutation(num_blocks)
    table = np.full((B, max_blocks_per_seq), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        table[b, : nblk[b]] = perm[pos: pos + nblk[b]]
        pos += nblk[b]
    q = torch.from_numpy(rng.standard_normal((B, Hq, d), dtype=np.float32)).to(torch.bfloat16)

    fill = float("nan") if poison else 0.0
    caches = []
    for tag in (1, 2):  # K then V
        pool = torch.full((num_blocks, block_size, Hkv, d), fill, dtype=torch.bfloat16)
        for b in range(B):
            n = int(lens[b])
            if n == 0:
                continue
            vals = torch.from_numpy(draw_normal(seed, tag, (n, Hkv, d), sub=b))
            vals = vals.to(torch.bfloat16)
            full, tail = divmod(n, block_size)
            ids = torch.from_numpy(table[b, :full].astype(np.int64))
            if full:
                pool[ids] = vals[: full * block_size].reshape(full, block_size, Hkv, d)
            if tail:
                pool[int(table[b, full]), :tail] = vals[full * block_size:]
        caches.append(pool)
    return {
        "q": q,
        "kcache": caches[0],
        "vcache": caches[1],
        "block_table": torch.from_numpy(table),
        "seq_lens": torch.from_numpy(lens.astype(np.int32)),
    }


def paged_seq_lens(cfg: PagedConfig):
    """The sequence lengths make_paged_config draws (its generator's first draw)."""
    rng = np.random.default_rng(cfg.seed)
    return rng.integers(cfg.len_lo, cfg.len_hi, size=cfg.B, endpoint=True).astype(np.int64)


def make_paged_config(cfg: PagedConfig, poison: bool = True):
    return make_paged(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.block_size, cfg.num_blocks,
                      cfg.max_blocks_per_seq, cfg.seed, cfg.len_lo, cfg.len_hi,
                      poison=poison)
