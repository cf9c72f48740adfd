"""GPU parity of the prefill forward (attn_fwd, attn_fwd_f32) against the fp64 oracle.

All calls go through the C ABI of libattn.so via the Python binding.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_fwd, attn_fwd_f32
from tests.parity import check, to_f64

pytestmark = pytest.mark.gpu

# (B, Nq, Nk, Hq, Hkv, d, causal, window): tile edges (64 / 128 rows and
# 32 / 64 / 128 keys), ragged tails, GQA / MQA, windows, Nq != Nk, empty keys.
SMALL = [
    (1, 1, 1, 1, 1, 64, False, 0),
    (1, 2, 2, 2, 1, 128, True, 0),
    (2, 17, 17, 4, 2, 64, True, 0),
    (1, 63, 63, 2, 2, 128, False, 0),
    (1, 64, 64, 4, 1, 128, True, 0),
    (1, 65, 65, 2, 2, 64, True, 5),
    (1, 127, 127, 2, 1, 128, True, 1),
    (1, 128, 128, 8, 2, 128, True, 0),
    (1, 129, 129, 4, 4, 64, True, 17),
    (2, 255, 255, 4, 2, 128, True, 64),
    (1, 256, 256, 2, 1, 64, False, 0),
    (1, 1000, 1000, 4, 2, 128, True, 0),
    (1, 1000, 1000, 4, 1, 64, True, 100),
    (1, 100, 700, 4, 2, 128, True, 0),
    (1, 300, 90, 2, 2, 64, False, 0),
    (1, 37, 1000, 2, 1, 128, True, 128),
    (1, 1, 1000, 4, 4, 128, True, 0),
    (1, 5, 0, 2, 1, 64, False, 0),
    (1, 333, 333, 2, 2, 128, True, 333),
    (3, 200, 200, 6, 3, 64, True, 0),
    # groups wider than a work item's head count (8, 4 or 2 of the group's
    # heads per item, 256 / that many positions each): MQA 32 and 16 query
    # heads, a group of 12 and of 6, with windows, ragged lengths, Nq < Nk
    (1, 300, 300, 32, 1, 128, True, 0),
    (2, 257, 400, 16, 1, 64, True, 50),
    (1, 333, 333, 12, 1, 128, True, 77),
    (1, 100, 130, 12, 2, 128, False, 0),
]


def _ids(c):
    B, Nq, Nk, Hq, Hkv, d, causal, w = c
    return f"B{B}_q{Nq}_k{Nk}_h{Hq}x{Hkv}_d{d}_{'c' if causal else 'n'}{w}"


def _run(dtype, q, k, v, causal, window, scale):
    fn = attn_fwd if dtype == "bf16" else attn_fwd_f32
    out, lse = fn(q.cuda(), k.cuda(), v.cuda(), causal=causal, window=window, scale=scale)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SMALL, ids=_ids)
def test_small_shapes(case, dtype):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    seed = 1000 + SMALL.index(case)
    print(f"case {_ids(case)} {dtype} seed {seed}", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, Nq, Nk, d, seed, dtype)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _run(dtype, q, k, v, causal, window, scale)
    O, L = oracle.attention(q, k, v, scale, causal, window)
    check(out, O, lse, L, dtype, _ids(case))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [-0.09, 0.0])
@pytest.mark.parametrize("causal,window", [(True, 0), (True, 70), (False, 0)])
def test_non_positive_scale(scale, causal, window, dtype):
    # scale <= 0 takes the bf16 kernel's variant that scales every score before
    # its row maximum; scale = 0 weights every visible key equally
    B, Nq, Nk, Hq, Hkv, d = 2, 300, 333, 4, 2, 128
    seed = 1900
    print(f"scale {scale} causal {causal} window {window} {dtype} seed {seed}", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, Nq, Nk, d, seed, dtype)
    out, lse = _run(dtype, q, k, v, causal, window, scale)
    O, L = oracle.attention(q, k, v, scale, causal, window)
    check(out, O, lse, L, dtype, f"scale {scale} causal {causal} window {window} {dtype}")


def test_f32_single_head_config():
    """The fp32 single-head workload: B=1, H=1, N=256, d=64, non-causal."""
    cfg = workloads.DENSE_CONFIGS["f32_single_head_256"]
    q, k, v = workloads.make_dense_config(cfg)
    out, lse = _run("f32", q, k, v, cfg.causal, cfg.window, cfg.scale)
    O, L = oracle.attention(q, k, v, cfg.scale, cfg.causal, cfg.window)
    check(out, O, lse, L, "f32", cfg.name)


def test_worked_example_on_gpu():
    """Scores [1, 3] (one query, two keys, V = I) give p = 0.1192..., 0.8807..."""
    q = torch.zeros(1, 1, 1, 64)
    k = torch.zeros(1, 2, 1, 64)
    v = torch.zeros(1, 2, 1, 64)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, 0, 0] = 1.0
    k[0, 1, 0, 0] = 3.0
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    out, lse = _run("f32", q, k, v, False, 0, 1.0)
    assert abs(out[0, 0, 0, 0].item() - 1 / (1 + math.e ** 2)) < 1e-6
    assert abs(out[0, 0, 0, 1].item() - 1 / (1 + math.e ** -2)) < 1e-6
    assert abs(lse[0, 0, 0].item() - (3 + math.log(1 + math.e ** -2))) < 1e-6


def test_causal_first_row_exact_bf16():
    q, k, v = workloads.make_dense(1, 4, 2, 300, 300, 128, 77)
    out, lse = _run("bf16", q, k, v, True, 0, 0.0883883)
    # row 0 sees only key 0: p = 1 exactly, so O is v0 bit for bit
    for h in range(4):
        assert torch.equal(out[0, 0, h], v[0, 0, h // 2])


def test_constant_values_bf16():
    q, k, _ = workloads.make_dense(1, 4, 1, 500, 500, 64, 78)
    c = torch.randn(64).to(torch.bfloat16)
    v = c.expand(1, 500, 1, 64).contiguous()
    out, _ = _run("bf16", q, k, v, True, 37, 0.125)
    assert torch.equal(out, c.expand(1, 500, 4, 64))


def test_gqa_equals_repeated_mha():
    q, k, v = workloads.make_dense(2, 8, 2, 200, 200, 128, 79)
    out_g, lse_g = _run("bf16", q, k, v, True, 0, 0.0883883)
    kr = k.repeat_interleave(4, dim=2).contiguous()
    vr = v.repeat_interleave(4, dim=2).contiguous()
    out_m, lse_m = _run("bf16", q, kr, vr, True, 0, 0.0883883)
    assert torch.equal(out_g, out_m) and torch.equal(lse_g, lse_m)


def test_deterministic():
    q, k, v = workloads.make_dense(2, 4, 2, 700, 700, 128, 80)
    a = _run("bf16", q, k, v, True, 0, 0.0883883)
    b = _run("bf16", q, k, v, True, 0, 0.0883883)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_input_validation_errors():
    q = torch.zeros(1, 8, 3, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        attn_fwd(q, k, k)  # 3 query heads over 2 KV heads
    with pytest.raises(ValueError):
        attn_fwd(q[:, :, :2], k, k, window=3)  # window without causal


# ---------------------------------------------------------------- full-size workloads

def _sample_rows(N, seed, extra=()):
    rng = np.random.default_rng(seed)
    rows = set(range(0, 48)) | set(range(N - 16, N)) | set(extra)
    for t in (64, 128, 4096, N // 2):
        rows |= {t - 1, t, t + 1}
    rows |= set(int(x) for x in rng.integers(0, N, 96))
    return np.array(sorted(r for r in rows if 0 <= r < N))


def _full_config(name, heads, window_override=None):
    cfg = workloads.DENSE_CONFIGS[name]
    print(f"config {name}: generating inputs", flush=True)
    q, k, v = workloads.make_dense_config(cfg)
    window = cfg.window if window_override is None else window_override
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    out, lse = attn_fwd(qd, kd, vd, causal=cfg.causal, window=window, scale=cfg.scale)
    torch.cuda.synchronize()
    print(f"config {name}: kernel done", flush=True)
    assert torch.isfinite(out).all().item() and torch.isfinite(lse).all().item()
    rows = _sample_rows(cfg.Nq, cfg.seed)
    ref = oracle.attention(q, k, v, cfg.scale, cfg.causal, window, heads=heads, rows=rows)
    out_c, lse_c = out.cpu(), lse.cpu()
    worst = (0.0, 0.0, 0.0)
    for (b, h), (O, L) in ref.items():
        r = check(out_c[b, rows, h], O, lse_c[b, h, rows], L, "bf16", f"{name} b{b} h{h}")
        worst = tuple(max(x, y) for x, y in zip(worst, r))
    print(f"config {name}: worst max-abs {worst[0]:.3e} mean-abs {worst[1]:.3e} "
          f"lse {worst[2]:.3e}", flush=True)
    return out, lse, (qd, kd, vd)


def test_mha_causal_8k():
    cfg = workloads.DENSE_CONFIGS["mha_causal_8k"]
    heads = [(0, 0), (0, 31), (1, 7), (2, 16), (3, 31), (3, 0), (1, 30), (2, 1)]
    out, lse, (qd, kd, vd) = _full_config(cfg.name, heads)
    out2, lse2 = attn_fwd(qd, kd, vd, causal=True, scale=cfg.scale)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)   # deterministic


@pytest.mark.parametrize("name", ["gqa_causal_16k", "mqa_causal_16k"])
def test_gqa_mqa_causal_16k(name):
    cfg = workloads.DENSE_CONFIGS[name]
    G = cfg.Hq // cfg.Hkv
    heads = sorted({(0, 0), (0, G - 1), (0, min(G, cfg.Hq - 1)), (1, cfg.Hq - 1),
                    (1, cfg.Hq - G), (1, 13), (0, 22), (1, 5)})
    _full_config(name, heads)


def test_swa_causal_32k():
    cfg = workloads.DENSE_CONFIGS["swa_causal_32k_w4096"]
    out, lse, (qd, kd, vd) = _full_config(cfg.name, [(0, 0), (0, 31)])
    # a window at least as long as the sequence is plain causal attention
    oc, lc = attn_fwd(qd, kd, vd, causal=True, window=0, scale=cfg.scale)
    ow, lw = attn_fwd(qd, kd, vd, causal=True, window=cfg.Nk, scale=cfg.scale)
    assert torch.equal(oc, ow) and torch.equal(lc, lw)
    assert not torch.equal(out, oc)


def test_paired_schedule_odd_query_tiles():
    """33 query tiles per head (an odd count) and enough heads that the
    persistent schedule pairs heavy and light query tiles of a head; the
    middle tile runs alone.  Rows of the first, middle, last and a ragged
    tile are checked against the oracle on heads across the KV groups."""
    B, Hq, Hkv, N, d = 1, 16, 4, 33 * 256 - 100, 64
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, 81)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    out, lse = _run("bf16", q, k, v, True, 0, scale)
    assert torch.isfinite(out).all().item()
    rows = np.array(sorted({0, 1, 255, 256, 16 * 256 - 1, 16 * 256, 16 * 256 + 17, 17 * 256 - 1,
                            17 * 256, 31 * 256 + 5, N - 1, N - 2} | set(range(N - 40, N, 7))))
    heads = [(0, 0), (0, 3), (0, 4), (0, 9), (0, 15)]
    ref = oracle.attention(q, k, v, scale, True, 0, heads=heads, rows=rows)
    for (b, h), (O, L) in ref.items():
        check(out[b, rows, h], O, lse[b, h, rows], L, "bf16", f"paired b{b} h{h}")


def _sched_inputs():
    shapes = [
        (4, 32, 8, 8192, 8192, 128, True, 0),   # paired query tiles, a long launch
        (1, 4, 2, 700, 700, 64, True, 0),       # single tiles
        (2, 8, 8, 1500, 1500, 128, False, 0),
        (1, 8, 2, 3000, 3000, 128, True, 1000),
    ]
    inputs, refs = [], []
    for i, (B, Hq, Hkv, Nq, Nk, d, causal, w) in enumerate(shapes):
        q, k, v = workloads.make_dense(B, Hq, Hkv, Nq, Nk, d, 90 + i)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        inputs.append((qd, kd, vd, causal, w))
        refs.append(attn_fwd(qd, kd, vd, causal=causal, window=w))
        torch.cuda.synchronize()
    return inputs, refs


def test_persistent_queue_reuse_and_streams():
    """The persistent kernel takes its work from counters in device memory that
    launches reuse: each launch takes a fresh tag and a slot, set up by a
    one-wave kernel before it.  Many launches in a row, of shapes that
    alternate between the paired and the single-tile schedules, and 4 streams
    with 20 launches each in flight at once must all reproduce the result of
    a lone launch bit for bit."""
    inputs, refs = _sched_inputs()
    for it in range(70):
        s = it % len(inputs)
        qd, kd, vd, causal, w = inputs[s]
        out, lse = attn_fwd(qd, kd, vd, causal=causal, window=w)
        torch.cuda.synchronize()
        assert torch.equal(out, refs[s][0]) and torch.equal(lse, refs[s][1]), f"launch {it}"
    streams = [torch.cuda.Stream() for _ in range(4)]
    results = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for it in range(20):
        for j, st in enumerate(streams):
            s = (it + j) % len(inputs)
            qd, kd, vd, causal, w = inputs[s]
            with torch.cuda.stream(st):
                results.append((s, attn_fwd(qd, kd, vd, causal=causal, window=w)))
    torch.cuda.synchronize()
    for n, (s, (out, lse)) in enumerate(results):
        assert torch.equal(out, refs[s][0]) and torch.equal(lse, refs[s][1]), f"launch {n} shape {s}"


def test_single_counter_slot_still_exact():
    """With a single counter slot every launch reuses the slot of the launch
    before it: one long launch on one stream and 70 short launches of three
    shapes on another, enqueued together, must each wait for the slot's
    previous user and reproduce a lone launch bit for bit."""
    from exact_softmax_attention_amd import _lib
    inputs, refs = _sched_inputs()
    prev = _lib.lib().attn_set_fwd_sched_slots(1)
    try:
        a, b = torch.cuda.Stream(), torch.cuda.Stream()
        a.wait_stream(torch.cuda.current_stream())
        b.wait_stream(torch.cuda.current_stream())
        qd, kd, vd, causal, w = inputs[0]
        with torch.cuda.stream(a):
            long_res = attn_fwd(qd, kd, vd, causal=causal, window=w)
        short = []
        for it in range(70):
            s = 1 + it % 3
            qd, kd, vd, causal, w = inputs[s]
            with torch.cuda.stream(b):
                short.append((s, attn_fwd(qd, kd, vd, causal=causal, window=w)))
        torch.cuda.synchronize()
    finally:
        _lib.lib().attn_set_fwd_sched_slots(prev)
    assert torch.equal(long_res[0], refs[0][0]) and torch.equal(long_res[1], refs[0][1])
    for n, (s, (out, lse)) in enumerate(short):
        assert torch.equal(out, refs[s][0]) and torch.equal(lse, refs[s][1]), f"short {n} shape {s}"


def test_captured_graph_replays_match_eager():
    """A forward call captured into a graph (its counter set-up kernel and the
    kernel, on a slot of its own) replayed several times, with eager launches
    and synchronisations between the replays, reproduces the eager result bit
    for bit on every replay."""
    inputs, refs = _sched_inputs()
    qd, kd, vd, causal, w = inputs[3]
    out = torch.empty_like(qd)
    lse = torch.empty((qd.shape[0], qd.shape[2], qd.shape[1]), dtype=torch.float32,
                      device=qd.device)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        attn_fwd(qd, kd, vd, causal=causal, window=w, out=out, lse=lse)  # warm-up
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn_fwd(qd, kd, vd, causal=causal, window=w, out=out, lse=lse)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        # eager work on other shapes between the replays
        o1, l1 = attn_fwd(*inputs[1][:3], causal=inputs[1][3], window=inputs[1][4])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, refs[3][0]) and torch.equal(lse, refs[3][1]), f"replay {rep}"
        assert torch.equal(o1, refs[1][0]) and torch.equal(l1, refs[1][1])
