"""GPU parity of chunked prefill over a paged cache (attn_prefill_paged) and of
sliding-window decode at full size, against the fp64 oracle.

All calls go through the C ABI of libattn.so via the Python binding.  The
caches are poisoned (unused blocks and tail slots hold NaN), so reading a
slot that is not the sequence's shows up as a non-finite output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import (attn_decode_paged, attn_fwd_varlen, attn_prefill_paged,
                                         metrics)
from tests.parity import check

pytestmark = pytest.mark.gpu

# (seq_lens, chunks, Hq, Hkv, d, window): contexts off the 16-token block and
# 64-key tile grid, chunks of 1, of a whole context, over 256 rows, empty
# chunks and an empty context, GQA / MQA, windows.
SMALL = [
    ([100, 37, 300], [20, 37, 1], 4, 2, 128, 0),
    ([64, 65, 1000], [64, 1, 300], 8, 2, 128, 0),
    ([513, 16, 0, 250], [257, 0, 0, 250], 2, 1, 64, 0),
    ([700, 701], [100, 600], 4, 4, 128, 77),
    ([2000], [511], 8, 1, 128, 1000),
    ([33, 1], [33, 1], 2, 2, 64, 1),
]


def _ids(c):
    lens, ch, Hq, Hkv, d, w = c
    return f"n{len(lens)}_k{sum(lens)}_q{sum(ch)}_h{Hq}x{Hkv}_d{d}_w{w}"


def _make(lens, chunks, Hq, Hkv, d, seed, poison=True):
    bs = 16
    need = sum((n + bs - 1) // bs for n in lens)
    max_blocks = max(1, max((n + bs - 1) // bs for n in lens))
    return workloads.make_prefill_paged(lens, chunks, Hq, Hkv, d, bs, need + 7, max_blocks,
                                        seed, poison=poison)


def _run(inp, scale, window):
    d = {k: t.cuda() for k, t in inp.items()}
    out, lse = attn_prefill_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                  d["seq_lens"], d["cu_seqlens_q"], scale=scale, window=window)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _oracle(inp, scale, window, seqs=None):
    return oracle.prefill_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                                inp["seq_lens"], inp["cu_seqlens_q"], scale, window, seqs)


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_small_chunks(case):
    lens, chunks, Hq, Hkv, d, window = case
    seed = 3000 + SMALL.index(case)
    print(f"case {_ids(case)} seed {seed}", flush=True)
    inp = _make(lens, chunks, Hq, Hkv, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _run(inp, scale, window)
    O, L = _oracle(inp, scale, window)
    check(out, O, lse, L, "bf16", _ids(case))


SPLIT = [
    # contexts past one 8192-key chunk: query tiles whose keys span 2..3 chunks
    ([9000, 300, 20000], [100, 300, 257], 4, 2, 128, 0),
    ([16385, 8193], [600, 1], 2, 1, 64, 0),
    ([20000, 12000], [300, 260], 4, 4, 128, 9000),  # windows across a chunk boundary
    # window starts 8101..8356 straddle the 8192-key chunk boundary inside one
    # query tile: part of its rows see nothing of chunk 0 (partial LSE = -inf)
    ([9356, 600], [256, 100], 4, 2, 128, 1000),
]


@pytest.mark.parametrize("case", SPLIT, ids=_ids)
def test_key_chunk_split(case):
    lens, chunks, Hq, Hkv, d, window = case
    seed = 3050 + SPLIT.index(case)
    print(f"case {_ids(case)} seed {seed}", flush=True)
    inp = _make(lens, chunks, Hq, Hkv, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _run(inp, scale, window)
    O, L = _oracle(inp, scale, window)
    check(out, O, lse, L, "bf16", _ids(case))


def test_negative_scale_chunked_prefill():
    lens, chunks = [700, 9000], [300, 257]   # the second spans two key chunks
    inp = _make(lens, chunks, 4, 2, 128, 3090)
    out, lse = _run(inp, -0.09, 0)
    O, L = _oracle(inp, -0.09, 0)
    check(out, O, lse, L, "bf16", "chunked prefill, scale -0.09")


def test_more_sequences_than_the_lds_table():
    # past 2047 sequences the kernel reads cu_seqlens_q and the lengths from
    # global memory rather than from its LDS copy
    rng = np.random.default_rng(3095)
    lens = [int(x) for x in rng.integers(1, 60, size=2100)]
    chunks = [int(rng.integers(0, n + 1)) for n in lens]
    inp = _make(lens, chunks, 2, 1, 64, 3095)
    out, lse = _run(inp, 0.125, 0)
    O, L = _oracle(inp, 0.125, 0)
    check(out, O, lse, L, "bf16", "2100 sequences")


def test_one_new_token_matches_decode():
    lens = [40, 700, 1234, 16]
    inp = _make(lens, [1] * 4, 8, 2, 128, 3100)
    out, lse = _run(inp, 0.088, 0)
    d = {k: t.cuda() for k, t in inp.items()}
    od, ld = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"], d["seq_lens"],
                               scale=0.088)
    O, L = _oracle(inp, 0.088, 0)
    check(out, O, lse, L, "bf16", "prefill with one token")
    check(od.cpu(), O, ld.cpu().T, L, "bf16", "decode")


def test_block_aligned_contiguous_cache_equals_packed_kernel_bitwise():
    # contexts of whole blocks laid out in block order are the packed-sequence
    # layout: the two entry points must load the same keys into the same tiles
    lens = [64, 320, 1024, 16]
    chunks = [64, 100, 300, 16]
    Hq, Hkv, d = 4, 2, 128
    inp = _make(lens, chunks, Hq, Hkv, d, 3200)
    nb = sum(n // 16 for n in lens)
    ids = torch.arange(nb, dtype=torch.int32)
    table = torch.full(inp["block_table"].shape, -1, dtype=torch.int32)
    pos = 0
    for s, n in enumerate(lens):
        table[s, : n // 16] = ids[pos: pos + n // 16]
        pos += n // 16
    kc = inp["kcache"].clone()
    vc = inp["vcache"].clone()
    kflat = kc[:nb].reshape(-1, Hkv, d)
    vflat = vc[:nb].reshape(-1, Hkv, d)
    # fill the contiguous blocks with finite values
    g = torch.Generator().manual_seed(5)
    kflat.copy_(torch.randn(kflat.shape, generator=g).to(torch.bfloat16))
    vflat.copy_(torch.randn(vflat.shape, generator=g).to(torch.bfloat16))
    kc[:nb] = kflat.reshape(nb, 16, Hkv, d)
    vc[:nb] = vflat.reshape(nb, 16, Hkv, d)
    inp.update(kcache=kc, vcache=vc, block_table=table)
    out, lse = _run(inp, 0.1, 0)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    ov, lv = attn_fwd_varlen(inp["q"].cuda(), kflat.cuda(), vflat.cuda(), inp["cu_seqlens_q"].cuda(),
                             cu_k.cuda(), causal=True, scale=0.1)
    assert torch.equal(out, ov.cpu()) and torch.equal(lse, lv.cpu())


def test_bad_block_id_and_bad_length_give_nan():
    lens, chunks = [200, 300, 150], [100, 200, 50]
    inp = _make(lens, chunks, 2, 1, 128, 3300)
    nbk = inp["kcache"].shape[0]
    inp["block_table"][1, 3] = nbk + 100   # sequence 1 (one 256-row tile, no window)
    inp["seq_lens"][2] = inp["block_table"].shape[1] * 16 + 1  # longer than its table
    out, lse = _run(inp, 0.1, 0)
    cu = inp["cu_seqlens_q"].tolist()
    assert torch.isfinite(out[cu[0]:cu[1]].float()).all()
    assert torch.isnan(out[cu[1]:cu[3]].float()).all()
    assert torch.isnan(lse[:, cu[1]:cu[3]]).all()
    O, L = _oracle(inp, 0.1, 0, seqs=[0])
    check(out[cu[0]:cu[1]], O[cu[0]:cu[1]], lse[:, cu[0]:cu[1]], L[:, cu[0]:cu[1]], "bf16", "seq 0")


def test_bad_block_id_makes_the_whole_sequence_nan():
    """A block id outside the pool gives NaN in every row of its sequence, as in
    the oracle, also where the bad block is read by only one of several query
    tiles, by only one of two key chunks, or by none (before the window)."""
    # sequence 0: 600 new tokens (3 query tiles), block 55 (keys 880..895) is
    # not seen by the rows at positions 400..655; sequence 1: 9000 keys (two
    # chunks of 8192), block 10 lies in the first chunk only; sequence 2 clean
    lens, chunks = [1000, 9000, 300], [600, 300, 100]
    inp = _make(lens, chunks, 2, 1, 128, 3350)
    nbk = inp["kcache"].shape[0]
    inp["block_table"][0, 55] = nbk
    inp["block_table"][1, 10] = -3
    out, lse = _run(inp, 0.1, 0)
    O, L = _oracle(inp, 0.1, 0)
    cu = inp["cu_seqlens_q"].tolist()
    assert np.isnan(O[cu[0]:cu[2]]).all() and np.isnan(L[:, cu[0]:cu[2]]).all()
    assert torch.isnan(out[cu[0]:cu[2]].float()).all()
    assert torch.isnan(lse[:, cu[0]:cu[2]]).all()
    check(out[cu[2]:cu[3]], O[cu[2]:cu[3]], lse[:, cu[2]:cu[3]], L[:, cu[2]:cu[3]], "bf16", "seq 2")
    # window 256 over 3000 keys: block 5 (keys 80..95) is before every row's window
    inp = _make([3000], [50], 2, 2, 64, 3351)
    inp["block_table"][0, 5] = inp["kcache"].shape[0] + 1
    out, lse = _run(inp, 0.1, 256)
    O, L = _oracle(inp, 0.1, 256)
    assert np.isnan(O).all() and np.isnan(L).all()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


def test_deterministic():
    inp = _make([900, 1500], [300, 700], 8, 2, 128, 3400)
    a = _run(inp, 0.088, 0)
    b = _run(inp, 0.088, 0)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_chunked_prefill_workload_full_size():
    """16 sequences of 8000..32000 cached tokens taking 512 new tokens each
    (32 query / 8 KV heads of 128, 16-token blocks), in the launch the
    benchmark times; sampled sequences and heads against the oracle."""
    cfg = workloads.PREFILL_PAGED_CONFIGS["paged_prefill_16x32k_chunk512"]
    inp = workloads.make_prefill_paged_config(cfg)
    out, lse = _run(inp, cfg.scale, cfg.window)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    lens = inp["seq_lens"].numpy()
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 5})
    heads = [0, 3, 4, 31]  # both sides of a GQA group boundary
    O, L = oracle.prefill_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                                inp["seq_lens"], inp["cu_seqlens_q"], cfg.scale, cfg.window,
                                seqs=seqs)
    cu = inp["cu_seqlens_q"].numpy()
    for s in seqs:
        r = slice(int(cu[s]), int(cu[s + 1]))
        check(out[r][:, heads], O[r][:, heads], lse[heads][:, r], L[heads][:, r], "bf16",
              f"sequence {s} (context {lens[s]})")
    chunks = np.diff(cu)
    f = metrics.prefill_paged_flops(lens, chunks, cfg.Hq, cfg.d, cfg.window)
    assert f == 4.0 * cfg.d * cfg.Hq * float(sum(c * (n - c) + c * (c + 1) // 2
                                                 for n, c in zip(lens, chunks)))


def test_sliding_window_decode_full_size():
    """Decode over the 16 x 8000..32000-token paged batch with a 4096-token
    window: sampled sequences against the oracle, every output finite."""
    pc = workloads.PAGED_CONFIGS["paged_decode_16x32k"]
    inp = workloads.make_paged_config(pc)
    d = {k: t.cuda() for k, t in inp.items()}
    out, lse = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                 d["seq_lens"], scale=pc.scale, window=4096)
    torch.cuda.synchronize()
    out, lse = out.cpu(), lse.cpu()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    lens = inp["seq_lens"].numpy()
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 3, 11})
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], pc.scale, window=4096, seqs=seqs)
    for s in seqs:
        check(out[s], O[s], lse[s], L[s], "bf16", f"sequence {s} (context {lens[s]})")
