"""GPU parity of the backward pass (attn_bwd) against the fp64 gradient oracle.

The GPU forward supplies out and lse (as a training step would); the oracle
computes the exact gradients of the plain definition from the same bf16
inputs.  Tolerance (the pages give none for gradients): the error of each
gradient is measured against its own scale, max-abs <= 2e-2 * max|ref| and
mean-abs <= 5e-3 * mean|ref|.  The GPU path rounds P and dS to bf16 for the
matrix products (relative 2^-9 each), reads O as bf16 for D, and rounds the
results to bf16 (2^-9), so errors of a few 1e-3 of the scale are expected.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_bwd, attn_fwd
from tests.parity import to_f64

pytestmark = pytest.mark.gpu

# (B, Nq, Nk, Hq, Hkv, d, causal, window): 32-row blocks, 64-key steps and
# 128-key tiles cut at ragged places; GQA / MQA; windows; Nq != Nk; empty sides.
SMALL = [
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 33, 33, 2, 1, 128, True, 0),
    (2, 100, 100, 4, 2, 64, True, 0),
    (1, 130, 130, 2, 2, 128, False, 0),
    (1, 200, 260, 4, 1, 128, True, 0),
    (1, 257, 257, 2, 1, 64, True, 40),
    (1, 300, 90, 2, 2, 128, False, 0),
    (2, 129, 129, 6, 3, 128, True, 17),
    (1, 512, 512, 2, 1, 128, True, 0),
    (1, 5, 0, 2, 1, 64, False, 0),
    (1, 0, 7, 2, 1, 64, False, 0),
    # d = 64 through many steps of the staging ring (MQA: 4 heads per key tile)
    (1, 700, 700, 4, 1, 64, True, 0),
    (1, 150, 333, 2, 2, 64, False, 0),
]


def _ids(c):
    B, Nq, Nk, Hq, Hkv, d, causal, w = c
    return f"B{B}_q{Nq}_k{Nk}_h{Hq}x{Hkv}_d{d}_{'c' if causal else 'n'}{w}"


def check_grad(got, want, what):
    g, w = to_f64(got), to_f64(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite gradient"
    if w.size == 0:
        return 0.0, 0.0
    err = np.abs(g - w)
    ref_max, ref_mean = float(np.abs(w).max()), float(np.abs(w).mean())
    mx, mn = float(err.max()), float(err.mean())
    print(f"  {what}: max-abs {mx:.3e} (ref max {ref_max:.3e})  mean-abs {mn:.3e} (ref mean {ref_mean:.3e})")
    assert mx <= 2e-2 * ref_max + 1e-6, f"{what}: max-abs {mx:.3e} > 2e-2 * {ref_max:.3e}"
    assert mn <= 5e-3 * ref_mean + 1e-7, f"{what}: mean-abs {mn:.3e} > 5e-3 * {ref_mean:.3e}"
    return mx, mn


def _run(q, k, v, do, causal, window, scale):
    qg, kg, vg, dg = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = attn_fwd(qg, kg, vg, causal=causal, window=window, scale=scale)
    dq, dk, dv = attn_bwd(qg, kg, vg, out, dg, lse, causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return dq.cpu(), dk.cpu(), dv.cpu()


@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_small_shapes(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    seed = 3000 + SMALL.index(case)
    print(f"case {_ids(case)} seed {seed}", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, Nq, Nk, d, seed)
    do = workloads.make_dout(B, Nq, Hq, d, seed)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    dq, dk, dv = _run(q, k, v, do, causal, window, scale)
    rq, rk, rv, _ = oracle.attention_backward(q, k, v, do, scale, causal, window)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


@pytest.mark.parametrize("causal,window", [(True, 0), (True, 50)])
def test_negative_scale(causal, window):
    # the forward's variant for scale <= 0 and the gradients' sign of scale
    B, N, Hq, Hkv, d, scale = 1, 200, 4, 2, 128, -0.09
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, 3900)
    do = workloads.make_dout(B, N, Hq, d, 3900)
    dq, dk, dv = _run(q, k, v, do, causal, window, scale)
    rq, rk, rv, _ = oracle.attention_backward(q, k, v, do, scale, causal, window)
    check_grad(dq, rq, "dq")
    check_grad(dk, rk, "dk")
    check_grad(dv, rv, "dv")


def test_deterministic():
    """Two calls give the same bits (no atomics)."""
    q, k, v = workloads.make_dense(1, 4, 2, 300, 300, 128, 3100)
    do = workloads.make_dout(1, 300, 4, 128, 3100)
    a = _run(q, k, v, do, True, 0, 0.0883883)
    b = _run(q, k, v, do, True, 0, 0.0883883)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ---------------------------------------------------------------- full-size workloads

def _full(name, kv_heads):
    """The bench's backward call on a full workload; every gradient of the
    listed (batch, KV head) groups is checked: dQ of their query heads, dK and
    dV summed over those heads."""
    cfg = workloads.DENSE_CONFIGS[name]
    print(f"config {name}: generating inputs", flush=True)
    q, k, v = workloads.make_dense_config(cfg)
    do = workloads.make_dout(cfg.B, cfg.Nq, cfg.Hq, cfg.d, cfg.seed)
    dq, dk, dv = _run(q, k, v, do, cfg.causal, cfg.window, cfg.scale)
    print(f"config {name}: kernels done", flush=True)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item()
    G = cfg.Hq // cfg.Hkv
    for b, hk in kv_heads:
        rk_sum = rv_sum = 0.0
        for h in range(hk * G, hk * G + G):
            rq, rk, rv, _ = oracle.attention_backward_head(
                q[b, :, h], k[b, :, hk], v[b, :, hk], do[b, :, h], cfg.scale, cfg.causal,
                cfg.window)
            check_grad(dq[b, :, h], rq, f"{name} b{b} h{h} dq")
            rk_sum = rk_sum + rk
            rv_sum = rv_sum + rv
        check_grad(dk[b, :, hk], rk_sum, f"{name} b{b} hk{hk} dk")
        check_grad(dv[b, :, hk], rv_sum, f"{name} b{b} hk{hk} dv")


def test_mha_causal_8k_full_size():
    _full("mha_causal_8k", [(0, 0), (3, 31)])


def test_gqa_causal_16k_full_size():
    _full("gqa_causal_16k", [(1, 7)])
