"""GPU parity of the packed-sequence forward (attn_fwd_varlen) against the fp64 oracle.

All calls go through the C ABI of libattn.so via the Python binding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_fwd, attn_fwd_varlen, metrics
from tests.parity import check, to_f64

pytestmark = pytest.mark.gpu

# (lens_q, lens_k, Hq, Hkv, d, causal, window): sequences shorter than, equal
# to and longer than a 256-row query tile and a 64-key tile, empty sequences
# (no queries, no keys, neither), length 1, more queries than keys under
# causal (the first rows see nothing), GQA / MQA, windows.
SMALL = [
    ([5, 300, 1, 64], [5, 300, 1, 64], 2, 1, 128, True, 0),
    ([256, 257, 255], [256, 257, 255], 4, 2, 64, True, 0),
    ([0, 17, 0, 600], [0, 17, 3, 600], 2, 2, 128, True, 0),
    ([40, 513], [700, 600], 4, 1, 128, True, 0),            # Nq < Nk: bottom-right
    ([90, 300], [30, 64], 2, 1, 64, True, 0),                # Nq > Nk under causal
    ([100, 1000, 7], [100, 1000, 7], 4, 2, 128, True, 33),   # windows
    ([333, 1], [333, 1], 2, 2, 64, True, 333),
    ([123, 456], [77, 0], 2, 1, 128, False, 0),              # no keys: O = 0, LSE = -inf
    ([1] * 40, list(range(1, 41)), 8, 2, 128, True, 0),     # many one-query sequences
    ([700, 5, 1024], [700, 5, 1024], 4, 4, 64, False, 0),
]


def _ids(c):
    lq, lk, Hq, Hkv, d, causal, w = c
    return f"n{len(lq)}_q{sum(lq)}_k{sum(lk)}_h{Hq}x{Hkv}_d{d}_{'c' if causal else 'n'}{w}"


def _run(q, k, v, cu_q, cu_k, causal, window, scale, out=None):
    o, l = attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(),
                           causal=causal, window=window, scale=scale,
                           out=None if out is None else out.cuda())
    torch.cuda.synchronize()
    return o.cpu(), l.cpu()


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_small_packed(case):
    lens_q, lens_k, Hq, Hkv, d, causal, window = case
    seed = 2000 + SMALL.index(case)
    print(f"case {_ids(case)} seed {seed}", flush=True)
    q, k, v, cu_q, cu_k = workloads.make_packed(lens_q, lens_k, Hq, Hkv, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _run(q, k, v, cu_q, cu_k, causal, window, scale)
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), scale, causal, window)
    check(out, O, lse, L, "bf16", _ids(case))


@pytest.mark.parametrize("scale", [-0.09, 0.0])
def test_non_positive_scale_packed(scale):
    lens = [5, 300, 513]
    q, k, v, cu_q, cu_k = workloads.make_packed(lens, lens, 4, 2, 128, 2050)
    out, lse = _run(q, k, v, cu_q, cu_k, True, 90, scale)
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), scale, True, 90)
    check(out, O, lse, L, "bf16", f"packed scale {scale}")


def test_more_sequences_than_the_lds_table():
    # past 2047 sequences the kernel searches cu_seqlens in global memory
    # rather than in its LDS copy
    rng = np.random.default_rng(2060)
    lens = [int(x) for x in rng.integers(0, 40, size=2100)]
    q, k, v, cu_q, cu_k = workloads.make_packed(lens, lens, 2, 1, 64, 2060)
    out, lse = _run(q, k, v, cu_q, cu_k, True, 0, 0.125)
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), 0.125, True, 0)
    check(out, O, lse, L, "bf16", "2100 packed sequences")


def test_rows_outside_every_sequence_are_not_written():
    # the sequences cover rows 3 .. 3+sum-1 of a longer q; the rest keep a sentinel
    lens = [70, 300]
    q, k, v, cu_q, cu_k = workloads.make_packed(lens, lens, 2, 1, 128, 2100)
    pad = 3
    cu_q2 = cu_q + pad
    q2 = torch.cat([torch.zeros(pad, 2, 128, dtype=q.dtype), q, torch.zeros(5, 2, 128, dtype=q.dtype)])
    sentinel = torch.full_like(q2, 7.0)
    out, lse = _run(q2, k, v, cu_q2, cu_k, True, 0, 0.125, out=sentinel)
    assert torch.all(out[:pad] == 7.0) and torch.all(out[pad + sum(lens):] == 7.0)
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), 0.125, True, 0)
    check(out[pad:pad + sum(lens)], O, lse[:, pad:pad + sum(lens)], L, "bf16", "offset rows")


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 100)])
def test_equal_lengths_match_the_dense_kernel_bitwise(causal, window):
    # the same tiles in the same order: packing changes only addressing and schedule
    B, N, Hq, Hkv, d = 3, 700, 8, 2, 128
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, 2200)
    od, ld = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, window=window, scale=0.09)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32)
    ov, lv = _run(q.reshape(B * N, Hq, d), k.reshape(B * N, Hkv, d), v.reshape(B * N, Hkv, d),
                  cu, cu, causal, window, 0.09)
    assert torch.equal(ov, od.cpu().reshape(B * N, Hq, d))
    assert torch.equal(lv, ld.cpu().permute(1, 0, 2).reshape(Hq, B * N))


@pytest.mark.parametrize("window", [0, 150])
def test_ragged_lengths_match_per_sequence_dense_calls_bitwise(window):
    # A row's keys are visited in the same 64-key tiles, in the same order,
    # whichever 256-row query tile holds it: the packed kernel's tiles end at
    # each sequence's last row (the partial tile holds its first rows), the
    # dense kernel's start at row 0, and the results agree bit for bit.
    lens_q, lens_k = [5, 300, 513, 1000, 257], [5, 300, 700, 1000, 257]
    Hq, Hkv, d, scale = 4, 2, 128, 0.09
    q, k, v, cu_q, cu_k = workloads.make_packed(lens_q, lens_k, Hq, Hkv, d, 2250)
    ov, lv = _run(q, k, v, cu_q, cu_k, True, window, scale)
    for s_, (nq, nk) in enumerate(zip(lens_q, lens_k)):
        q0, k0 = int(cu_q[s_]), int(cu_k[s_])
        od, ld = attn_fwd(q[q0:q0 + nq][None].cuda(), k[k0:k0 + nk][None].cuda(),
                          v[k0:k0 + nk][None].cuda(), causal=True, window=window, scale=scale)
        assert torch.equal(ov[q0:q0 + nq], od.cpu()[0]), (s_, nq, nk)
        assert torch.equal(lv[:, q0:q0 + nq], ld.cpu()[0]), (s_, nq, nk)


def test_deterministic():
    lens = workloads.draw_lengths(5000, 600, 2048, 2300)
    q, k, v, cu_q, cu_k = workloads.make_packed(lens, lens, 8, 2, 128, 2300)
    a = _run(q, k, v, cu_q, cu_k, True, 0, 0.088)
    b = _run(q, k, v, cu_q, cu_k, True, 0, 0.088)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_packed_workload_full_size():
    """The packed training batch (65536 tokens, lengths averaging ~600, at most
    2048, 32 heads of 128, causal), in the launch the benchmark times; the
    longest, the shortest, the first and the last sequences are checked on
    sampled heads against the oracle, and every output is finite."""
    cfg = workloads.PACKED_CONFIGS["packed_causal_64k_mean600"]
    q, k, v, cu_q, cu_k = workloads.make_packed_config(cfg)
    out, lse = _run(q, k, v, cu_q, cu_k, cfg.causal, cfg.window, cfg.scale)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    lens = np.diff(cu_q.numpy())
    seqs = sorted({int(np.argmax(lens)), int(np.argmin(lens)), 0, len(lens) - 1})
    heads = [0, 13, 31]
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), cfg.scale, cfg.causal,
                                   cfg.window, seqs=seqs, heads=heads)
    cq = cu_q.numpy()
    for s in seqs:
        r = slice(int(cq[s]), int(cq[s + 1]))
        check(out[r][:, heads], O[r][:, heads], lse[heads][:, r], L[heads][:, r], "bf16",
              f"sequence {s} (length {lens[s]})")
    # work count sanity: the benchmark's flop figure is each sequence's own triangle
    f = metrics.varlen_fwd_flops(lens, lens, cfg.Hq, cfg.d, True, 0)
    assert f == 4.0 * cfg.d * cfg.Hq * float((lens * (lens + 1) // 2).sum())
