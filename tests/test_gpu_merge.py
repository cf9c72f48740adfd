"""GPU parity of the partial-result merge (attn_merge): attention split along the
keys into shards, each shard done by attn_fwd, merged with attn_merge, equals
the fp64 oracle's attention over all keys.  This is one device's step of ring
attention (its queries against one K/V shard at a time), shown on one GPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_fwd, attn_merge
from tests.parity import check

pytestmark = pytest.mark.gpu


def _shard_attention(q, k, v, bounds, causal, scale):
    """The last shard's query rows against key shards [bounds[s], bounds[s+1]),
    merged in place shard by shard; under causal the last shard is the
    diagonal block and the earlier ones are fully visible."""
    q0 = bounds[-2]
    qs = q[:, q0:].cuda()
    out = lse = None
    for s in range(len(bounds) - 1):
        ks = k[:, bounds[s]:bounds[s + 1]].cuda()
        vs = v[:, bounds[s]:bounds[s + 1]].cuda()
        diag = s == len(bounds) - 2
        o, l = attn_fwd(qs, ks, vs, causal=causal and diag, scale=scale)
        if out is None:
            out, lse = o, l
        else:
            attn_merge(out, lse, o, l, out=out, lse=lse)  # in place
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


CASES = [
    # B, N, Hq, Hkv, d, shard bounds (the last shard holds the queries), causal
    (2, 700, 4, 2, 128, [0, 350, 700], True),
    (1, 900, 2, 1, 64, [0, 300, 600, 900], True),
    (1, 513, 4, 4, 128, [0, 13, 300, 513], False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}_N{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_s{len(c[5]) - 1}_{'c' if c[6] else 'n'}")
def test_shards_merged_equal_full_attention(case):
    B, N, Hq, Hkv, d, bounds, causal = case
    seed = 5000 + CASES.index(case)
    print(f"case {case} seed {seed}", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _shard_attention(q, k, v, bounds, causal, scale)
    q0 = bounds[-2]
    O, L = oracle.attention(q, k, v, scale, causal, 0, rows=None)
    check(out, O[:, q0:], lse, L[:, :, q0:], "bf16", str(case))


# Ring attention over 8 or 16 devices: the running result is kept in bf16 and
# merged in place once per shard, so each merge adds one bf16 rounding of O.
MANY = [
    # B, N, Hq, Hkv, d, shards (equal; the last holds the queries), causal
    (1, 4096, 4, 2, 128, 8, True),
    (1, 2048, 2, 1, 64, 16, False),
]


@pytest.mark.parametrize("case", MANY, ids=lambda c: f"N{c[1]}_h{c[2]}x{c[3]}_d{c[4]}_s{c[5]}_{'c' if c[6] else 'n'}")
def test_many_shards_merged_in_place(case):
    """8 and 16 shards merged into one running bf16 result stay within the
    fp64 oracle's tolerance, and the rounding added by the merges stays within
    a few times that of one launch over all keys."""
    B, N, Hq, Hkv, d, S, causal = case
    seed = 5300 + MANY.index(case)
    print(f"case {case} seed {seed}", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    bounds = [N * i // S for i in range(S + 1)]
    out, lse = _shard_attention(q, k, v, bounds, causal, scale)
    q0 = bounds[-2]
    res = oracle.attention(q, k, v, scale, causal, 0,
                           heads=[(b, h) for b in range(B) for h in range(Hq)],
                           rows=np.arange(q0, N))
    O = np.zeros((B, N - q0, Hq, d))
    L = np.zeros((B, Hq, N - q0))
    for (b, h), (o, l) in res.items():
        O[b, :, h] = o
        L[b, h] = l
    _, merged_mean, _ = check(out, O, lse, L, "bf16", f"{S} shards")
    # one launch over all keys, for the same rows
    o1, l1 = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    _, one_mean, _ = check(o1.cpu()[:, q0:], O, l1.cpu()[:, :, q0:], L, "bf16", "one launch")
    print(f"mean-abs error: {S} shards merged {merged_mean:.3e}, one launch {one_mean:.3e}")
    assert merged_mean <= 4 * one_mean + 1e-6


def test_merge_with_an_empty_side_is_exact():
    # a partial over no keys (O = 0, LSE = -inf) leaves the other side unchanged
    B, N, H, d = 2, 100, 4, 128
    q, k, v = workloads.make_dense(B, H, H, N, 300, d, 5100)
    o, l = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=0.09)
    z = torch.zeros_like(o)
    zl = torch.full_like(l, float("-inf"))
    m1, ml1 = attn_merge(o, l, z, zl)
    m2, ml2 = attn_merge(z, zl, o, l)
    e, el = attn_merge(z, zl, z, zl)
    torch.cuda.synchronize()
    assert torch.equal(m1, o) and torch.equal(ml1, l)
    assert torch.equal(m2, o) and torch.equal(ml2, l)
    assert torch.all(e == 0) and torch.all(el == float("-inf"))


def test_merge_is_symmetric_and_propagates_nan():
    B, N, H, d = 1, 64, 2, 64
    g = torch.Generator().manual_seed(5200)
    a = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).cuda()
    b = torch.randn(B, N, H, d, generator=g).to(torch.bfloat16).cuda()
    la = torch.randn(B, H, N, generator=g).cuda()
    lb = torch.randn(B, H, N, generator=g).cuda()
    x, lx = attn_merge(a, la, b, lb)
    y, ly = attn_merge(b, lb, a, la)
    lb2 = lb.clone()
    lb2[0, 1, 5] = float("nan")
    z, lz = attn_merge(a, la, b, lb2)
    torch.cuda.synchronize()
    # every step is symmetric in the two sides (the weighted sum rounds each
    # product before the add), so swapping them changes no bit
    assert torch.equal(lx, ly)
    assert torch.equal(x, y)
    assert torch.isnan(z[0, 5, 1].float()).all() and torch.isnan(lz[0, 1, 5])
    assert torch.isfinite(z[0, 5, 0].float()).all() and torch.isfinite(z[0, 4, 1].float()).all()
    # the merge formula itself, against the oracle's merge of (m, l, acc) states
    M, Ls, acc = oracle.merge_states((la.cpu().numpy().reshape(-1), np.ones(B * H * N),
                                      a.cpu().double().numpy().transpose(0, 2, 1, 3).reshape(-1, d)),
                                     (lb.cpu().numpy().reshape(-1), np.ones(B * H * N),
                                      b.cpu().double().numpy().transpose(0, 2, 1, 3).reshape(-1, d)))
    want_o = (acc / Ls[:, None]).reshape(B, H, N, d).transpose(0, 2, 1, 3)
    want_l = (M + np.log(Ls)).reshape(B, H, N)
    check(x.cpu(), want_o, lx.cpu(), want_l, "bf16", "merge formula")


def test_ring_step_at_the_prefill_shape():
    """The MHA causal 8K shape (B=4, 32 heads of 128) split into two 4096-key
    shards: the second half's queries against the first shard (all visible)
    and the diagonal shard, merged; sampled heads against the oracle."""
    cfg = workloads.DENSE_CONFIGS["mha_causal_8k"]
    q, k, v = workloads.make_dense_config(cfg)
    half = cfg.Nq // 2
    out, lse = _shard_attention(q, k, v, [0, half, cfg.Nq], True, cfg.scale)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    heads = [(0, 0), (3, 31)]
    rows = np.arange(half, cfg.Nq, 7)
    res = oracle.attention(q, k, v, cfg.scale, True, 0, heads=heads, rows=rows)
    for (b, h), (o, l) in res.items():
        check(out[b, rows - half, h], o, lse[b, h, rows - half], l, "bf16", f"head {(b, h)}")
