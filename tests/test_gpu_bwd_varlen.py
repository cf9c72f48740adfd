"""GPU parity of the packed-sequence backward (attn_bwd_varlen) against the fp64
gradient oracle, with the tolerance of the dense backward (each gradient's
error against its own scale: max-abs <= 2e-2 * max|ref|, mean-abs <= 5e-3 *
mean|ref|).  The GPU packed forward supplies out and lse.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_bwd, attn_bwd_varlen, attn_fwd, attn_fwd_varlen
from tests.test_gpu_bwd import check_grad

pytestmark = pytest.mark.gpu

# (lens_q, lens_k, Hq, Hkv, d, causal, window): sequences shorter and longer
# than a 128-row tile, empty query or key sets, Nq != Nk, GQA, windows.
SMALL = [
    ([5, 300, 1, 64], [5, 300, 1, 64], 2, 1, 128, True, 0),
    ([129, 0, 200], [129, 40, 260], 4, 2, 64, True, 0),
    ([90, 130], [0, 130], 2, 2, 128, False, 0),
    ([257, 100], [257, 100], 4, 1, 128, True, 33),
    ([40, 513], [700, 600], 4, 2, 128, True, 0),
]


def _ids(c):
    lq, lk, Hq, Hkv, d, causal, w = c
    return f"n{len(lq)}_q{sum(lq)}_k{sum(lk)}_h{Hq}x{Hkv}_d{d}_{'c' if causal else 'n'}{w}"


def _run(q, k, v, do, cu_q, cu_k, causal, window, scale):
    qg, kg, vg, dg, cq, ck = q.cuda(), k.cuda(), v.cuda(), do.cuda(), cu_q.cuda(), cu_k.cuda()
    out, lse = attn_fwd_varlen(qg, kg, vg, cq, ck, causal=causal, window=window, scale=scale)
    dq, dk, dv = attn_bwd_varlen(qg, kg, vg, out, dg, lse, cq, ck, causal=causal, window=window,
                                 scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_small_packed(case):
    lens_q, lens_k, Hq, Hkv, d, causal, window = case
    seed = 4000 + SMALL.index(case)
    print(f"case {_ids(case)} seed {seed}", flush=True)
    q, k, v, cu_q, cu_k = workloads.make_packed(lens_q, lens_k, Hq, Hkv, d, seed)
    do = workloads.make_dout(1, q.shape[0], Hq, d, seed)[0]
    scale = float(np.float32(1.0 / math.sqrt(d)))
    dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, causal, window, scale)
    rq, rk, rv, _ = oracle.attention_varlen_backward(q, k, v, do, cu_q.numpy(), cu_k.numpy(),
                                                     scale, causal, window)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_equal_lengths_match_the_dense_backward_bitwise():
    B, N, Hq, Hkv, d = 3, 300, 4, 2, 128
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, 4100)
    do = workloads.make_dout(B, N, Hq, d, 4100)
    qg, kg, vg, dg = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = attn_fwd(qg, kg, vg, causal=True, scale=0.09)
    rq, rk, rv = attn_bwd(qg, kg, vg, out, dg, lse, causal=True, scale=0.09)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    lse_p = lse.permute(1, 0, 2).reshape(Hq, B * N).contiguous()
    dq, dk, dv = attn_bwd_varlen(qg.reshape(B * N, Hq, d), kg.reshape(B * N, Hkv, d),
                                 vg.reshape(B * N, Hkv, d), out.reshape(B * N, Hq, d),
                                 dg.reshape(B * N, Hq, d), lse_p, cu, cu, causal=True, scale=0.09)
    torch.cuda.synchronize()
    assert torch.equal(dq.cpu(), rq.cpu().reshape(B * N, Hq, d))
    assert torch.equal(dk.cpu(), rk.cpu().reshape(B * N, Hkv, d))
    assert torch.equal(dv.cpu(), rv.cpu().reshape(B * N, Hkv, d))


def test_packed_workload_full_size():
    """The packed training batch (65536 tokens, ~600-token sequences, at most
    2048, 32 heads of 128, causal): gradients of the longest and the shortest
    sequence on two heads against the oracle; every gradient finite."""
    cfg = workloads.PACKED_CONFIGS["packed_causal_64k_mean600"]
    q, k, v, cu_q, cu_k = workloads.make_packed_config(cfg)
    do = workloads.make_dout(1, q.shape[0], cfg.Hq, cfg.d, cfg.seed)[0]
    dq, dk, dv = _run(q, k, v, do, cu_q, cu_k, cfg.causal, cfg.window, cfg.scale)
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    lens = np.diff(cu_q.numpy())
    cq = cu_q.numpy()
    heads = [0, 31]
    for s in sorted({int(np.argmax(lens)), int(np.argmin(lens))}):
        r = slice(int(cq[s]), int(cq[s + 1]))
        sub_cu = np.array([0, lens[s]])
        rq, rk, rv, _ = oracle.attention_varlen_backward(q[r], k[r], v[r], do[r], sub_cu, sub_cu,
                                                         cfg.scale, cfg.causal, cfg.window,
                                                         heads=heads)
        # MHA: a KV head is its query head, so the selected heads' dK, dV are complete
        check_grad(dq[r][:, heads], rq[:, heads], f"dq sequence {s}")
        check_grad(dk[r][:, heads], rk[:, heads], f"dk sequence {s}")
        check_grad(dv[r][:, heads], rv[:, heads], f"dv sequence {s}")
