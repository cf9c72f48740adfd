"""GPU parity of the paged decode (attn_decode_paged) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import attn_decode_paged, attn_fwd
from tests.parity import check

pytestmark = pytest.mark.gpu


def _to_dev(inp):
    return {k: v.cuda() for k, v in inp.items()}


def _decode(inp, scale, window=0):
    d = _to_dev(inp)
    out, lse = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                 d["seq_lens"], scale=scale, window=window)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


# (B, Hq, Hkv, d, lens, window): group sizes 1..32, both head dims, lengths
# around block (16) and split (256) edges, empty and single-token sequences.
SMALL = [
    (4, 8, 2, 128, [1, 16, 17, 300], 0),
    (3, 32, 8, 128, [255, 256, 257], 0),
    (2, 4, 4, 64, [0, 33], 0),
    (3, 32, 1, 128, [600, 1, 1000], 0),
    (2, 16, 2, 64, [513, 40], 0),
    (3, 8, 8, 128, [1000, 999, 5], 100),
    (2, 12, 4, 64, [770, 300], 256),
    (2, 6, 3, 128, [31, 1100], 1),
    # a query-head group wider than 16 (two waves per KV head: 16 + 8 heads)
    (2, 24, 1, 128, [700, 65], 0),
    # more than 64 sequences (several rounds of the on-device prefix sum), with
    # empty sequences between non-empty ones
    (70, 4, 2, 64, [0 if i % 7 == 0 else (37 * i) % 300 + 1 for i in range(70)], 0),
]


def _sid(c):
    B, Hq, Hkv, d, lens, w = c
    ls = "-".join(map(str, lens)) if len(lens) <= 4 else f"{len(lens)}seqs"
    return f"B{B}_h{Hq}x{Hkv}_d{d}_L{ls}_w{w}"


@pytest.mark.parametrize("case", SMALL, ids=_sid)
def test_small_decode(case):
    B, Hq, Hkv, d, lens, window = case
    seed = 2000 + SMALL.index(case)
    print(f"case {_sid(case)} seed {seed}", flush=True)
    maxb = max(1, max((n + 15) // 16 for n in lens)) + 3
    inp = workloads.make_paged(B, Hq, Hkv, d, 16, sum(maxb for _ in lens) + 7, maxb, seed,
                               seq_lens=lens)
    scale = float(np.float32(1 / math.sqrt(d)))
    out, lse = _decode(inp, scale, window)
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], scale, window)
    check(out, O, lse, L, "bf16", _sid(case))


def test_decode_equals_prefill_single_query():
    """Paged decode == the forward kernel with Nq = 1 on the gathered cache."""
    inp = workloads.make_paged(3, 16, 4, 128, 16, 300, 80, seed=2100, seq_lens=[1200, 77, 513])
    out, lse = _decode(inp, 0.0883883)
    for b, n in enumerate([1200, 77, 513]):
        kc = torch.from_numpy(oracle.gather_paged(inp["kcache"], inp["block_table"][b].numpy(), n))
        vc = torch.from_numpy(oracle.gather_paged(inp["vcache"], inp["block_table"][b].numpy(), n))
        q = inp["q"][b][None, None].cuda()
        o2, l2 = attn_fwd(q, kc[None].to(torch.bfloat16).cuda(), vc[None].to(torch.bfloat16).cuda(),
                          causal=True, scale=0.0883883)
        torch.cuda.synchronize()
        assert (out[b].float() - o2[0, 0].cpu().float()).abs().max().item() <= 2e-2
        assert (lse[b] - l2[0, :, 0].cpu()).abs().max().item() <= 1e-3


def test_gather_selects_the_matching_token_exactly():
    """q equal to one cached key (scale 1) puts all weight on that token: O must
    be that token's V bit for bit, for tokens spread over blocks and slots."""
    B, Hq, Hkv, d = 4, 8, 2, 128
    lens = [2000, 517, 16, 1000]
    inp = workloads.make_paged(B, Hq, Hkv, d, 16, 300, 130, seed=2200, seq_lens=lens)
    rng = np.random.default_rng(0)
    targets = {}
    for b in range(B):
        kc = oracle.gather_paged(inp["kcache"], inp["block_table"][b].numpy(), lens[b])
        for h in range(Hq):
            t = int(rng.integers(0, lens[b]))
            targets[(b, h)] = t
            inp["q"][b, h] = torch.from_numpy(kc[t, h // (Hq // Hkv)]).to(torch.bfloat16) * 2
    out, _ = _decode(inp, 1.0)
    O, _ = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], 1.0)
    for (b, h), t in targets.items():
        vc = oracle.gather_paged(inp["vcache"], inp["block_table"][b].numpy(), lens[b])
        want = torch.from_numpy(vc[t, h // (Hq // Hkv)]).to(torch.bfloat16)
        assert torch.equal(torch.from_numpy(O[b, h]).to(torch.bfloat16), want)  # oracle agrees
        assert torch.equal(out[b, h], want), (b, h, t)


def test_negative_scale_decode():
    inp = workloads.make_paged(3, 8, 2, 128, 16, 120, 40, seed=1990, seq_lens=[300, 17, 600])
    out, lse = _decode(inp, -0.09, 0)
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], -0.09, 0)
    check(out, O, lse, L, "bf16", "decode, scale -0.09")


def test_zero_scale_gives_exact_mean_of_small_integers():
    lens = [1, 7, 16, 17, 48]
    inp = workloads.make_paged(5, 4, 2, 64, 16, 40, 4, seed=2300, seq_lens=lens)
    c = inp["vcache"]
    fin = torch.isfinite(c)
    ints = torch.randint(-1, 2, c.shape, generator=torch.Generator().manual_seed(1))
    c[fin] = ints[fin].to(torch.bfloat16)
    out, lse = _decode(inp, 0.0)
    for b, n in enumerate(lens):
        vc = oracle.gather_paged(c, inp["block_table"][b].numpy(), n)
        for h in range(4):
            mean = vc[:, h // 2].sum(axis=0) / n
            # within half a bf16 ulp of the exact mean: a dropped, doubled or
            # wrong token moves the mean by at least 1/48, far more than that
            _, e = np.frexp(mean)
            half_ulp = np.where(mean == 0, 0.0, np.ldexp(1.0, e - 9))
            got = out[b, h].double().numpy()
            assert np.all(np.abs(got - mean) <= half_ulp * (1 + 1e-6) + 1e-12), (b, h)
        assert torch.allclose(lse[b], torch.full((4,), math.log(n)), atol=1e-5)


def test_bad_lengths_and_block_ids_give_nan_only_there():
    lens = [40, 20, 33, 50]
    inp = workloads.make_paged(4, 4, 1, 128, 16, 30, 4, seed=2400, seq_lens=lens)
    inp["block_table"][1, 1] = 30          # outside the pool
    inp["block_table"][2, 0] = -5          # negative id
    inp["seq_lens"][3] = 4 * 16 + 1        # longer than the table allows
    out, lse = _decode(inp, 0.0883883)
    for b in (1, 2, 3):
        assert torch.isnan(out[b].float()).all() and torch.isnan(lse[b]).all()
    assert torch.isfinite(out[0].float()).all()
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], 0.0883883, seqs=[0])
    check(out[0], O[0], lse[0], L[0], "bf16", "good sequence")


def test_paged_decode_config():
    cfg = workloads.PAGED_CONFIGS["paged_decode_16x32k"]
    print("paged config: generating inputs", flush=True)
    inp = workloads.make_paged_config(cfg)
    d = _to_dev(inp)
    out, lse = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                 d["seq_lens"], scale=cfg.scale)
    out2, lse2 = attn_decode_paged(d["q"], d["kcache"], d["vcache"], d["block_table"],
                                   d["seq_lens"], scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)  # deterministic
    print("paged config: oracle", flush=True)
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], cfg.scale)
    r = check(out.cpu(), O, lse.cpu(), L, "bf16", cfg.name)
    print(f"paged config: max-abs {r[0]:.3e} mean-abs {r[1]:.3e} lse {r[2]:.3e}", flush=True)
