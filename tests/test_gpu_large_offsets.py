"""GPU parity where element offsets pass 2**31: the kernels' address arithmetic.

A prefill (dense and packed) and a backward pass whose Q, O, dO and dQ hold
more than 2**31 elements (rows past 524288 of 32 heads of 128 sit beyond it),
and a paged decode and chunked prefill whose cache blocks sit past element
2**31 of the pool, each checked
against the fp64 oracle on the rows, keys and sequences that straddle the
boundary.  A 32-bit product anywhere in the addressing would read or write the
wrong rows (and, for the decode, NaN blocks).  The merge of two partial
results is checked where its 16-byte piece indices pass 2**31, which its
64-bit variant serves.

The sliding window keeps the GPU work small and every result local: a query
row sees only the W keys ending at its own position, so the oracle runs on a
slice of the sequence (rows [a, b) against keys [a - W + 1, b), whose
bottom-right alignment puts row a + i at key position a + i) and gives the
same exact values as on the whole sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from exact_softmax_attention_amd import (attn_bwd, attn_decode_paged, attn_fwd, attn_fwd_varlen,
                                         attn_merge, attn_prefill_paged)
from tests.parity import check, to_f64

pytestmark = pytest.mark.gpu

_E31 = 2 ** 31


def test_prefill_past_2_31_elements():
    # GQA 32 x 8 heads of 128, causal with a 4096-key window (so the kernel's
    # work stays small), 557056 tokens: Q and O hold 2.28e9 elements
    B, N, Hq, Hkv, d, W, seed = 1, 557056, 32, 8, 128, 4096, 7301
    assert B * N * Hq * d > _E31
    print("large prefill: generating inputs", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, seed)
    scale = 1.0 / np.sqrt(d)
    out, lse = attn_fwd(q.cuda(), k.cuda(), v.cuda(), causal=True, window=W, scale=scale)
    torch.cuda.synchronize()
    print("large prefill: kernel done", flush=True)
    # row r of head h starts at element (r * Hq + h) * d: row 524288 is the
    # first whose every head lies past 2**31
    first = _E31 // (Hq * d)
    rng = np.random.default_rng(seed)
    rows = {0, 1, 4095, 4096, first // 2, first - 2, first - 1, first, first + 1, first + 255,
            first + 256, N - 257, N - 256, N - 2, N - 1}
    rows |= set(int(x) for x in rng.integers(first - 4096, N, 24))
    rows = np.array(sorted(rows))
    heads = [(0, 0), (0, 9), (0, 22), (0, 31)]
    ref = oracle.attention(q, k, v, scale, True, W, heads=heads, rows=rows, row_chunk=64)
    out_c, lse_c = out[0, rows].cpu(), lse[0, :, rows].cpu()
    for (b, h), (O, L) in ref.items():
        check(out_c[:, h], O, lse_c[h], L, "bf16", f"large prefill head {h}")


def test_decode_blocks_past_2_31_elements():
    # a 135000-block pool of 16 x 8 heads x 128 (2.21e9 elements per cache);
    # the sequences' blocks are numbered around block 131072, the first that
    # starts past element 2**31, and every other block holds NaN
    B, Hq, Hkv, d, seed = 4, 32, 8, 128, 7302
    lens = [3001, 1, 4096, 2500]
    nblk = sum((n + 15) // 16 for n in lens)
    maxb = max((n + 15) // 16 for n in lens)
    print("large decode: generating inputs", flush=True)
    inp = workloads.make_paged(B, Hq, Hkv, d, 16, nblk, maxb, seed, seq_lens=lens)
    num_blocks = 135000
    blk_elems = 16 * Hkv * d
    shift = _E31 // blk_elems - nblk // 2
    assert (shift + nblk) * blk_elems > _E31 and shift + nblk <= num_blocks
    table = inp["block_table"].clone()
    table[table >= 0] += shift
    kc = torch.full((num_blocks, 16, Hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[shift: shift + nblk] = inp["kcache"].cuda()
    vc[shift: shift + nblk] = inp["vcache"].cuda()
    scale = 1.0 / np.sqrt(d)
    out, lse = attn_decode_paged(inp["q"].cuda(), kc, vc, table.cuda(), inp["seq_lens"].cuda(),
                                 scale=scale)
    torch.cuda.synchronize()
    print("large decode: kernel done", flush=True)
    # the oracle reads the same blocks from the compact pool (ids before the shift)
    O, L = oracle.decode_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                               inp["seq_lens"], scale)
    check(out.cpu(), O, lse.cpu(), L, "bf16", "large decode")


def _check_grad(got, want, what):
    # the backward tests' tolerance: each gradient against its own scale
    g, w = to_f64(got), to_f64(want)
    assert g.shape == w.shape and np.all(np.isfinite(g)), what
    err = np.abs(g - w)
    assert err.max() <= 2e-2 * np.abs(w).max() + 1e-6, f"{what}: max-abs {err.max():.3e}"
    assert err.mean() <= 5e-3 * np.abs(w).mean() + 1e-7, f"{what}: mean-abs {err.mean():.3e}"


def test_backward_past_2_31_elements():
    B, N, Hq, Hkv, d, W, seed = 1, 557056, 32, 8, 128, 4096, 7303
    G = Hq // Hkv
    print("large backward: generating inputs", flush=True)
    q, k, v = workloads.make_dense(B, Hq, Hkv, N, N, d, seed)
    do = workloads.make_dout(B, N, Hq, d, seed)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    qg, kg, vg, dg = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = attn_fwd(qg, kg, vg, causal=True, window=W, scale=scale)
    dq, dk, dv = attn_bwd(qg, kg, vg, out, dg, lse, causal=True, window=W, scale=scale)
    torch.cuda.synchronize()
    print("large backward: kernels done", flush=True)
    first = _E31 // (Hq * d)
    r0, r1 = first - 128, first + 128          # dQ rows around the boundary
    k0, k1 = first - 2048, first - 1920        # keys whose rows cross it
    a, b = k0, k1 + W - 1                      # the rows those keys see
    dq_c, dk_c, dv_c = dq[0, r0:r1].cpu(), dk[0, k0:k1].cpu(), dv[0, k0:k1].cpu()
    for hk in (0, Hkv - 1):
        rk_sum = rv_sum = 0.0
        for h in range(hk * G, hk * G + G):
            rq, _, _, _ = oracle.attention_backward_head(
                q[0, r0:r1, h], k[0, r0 - W + 1:r1, hk], v[0, r0 - W + 1:r1, hk],
                do[0, r0:r1, h], scale, True, W)
            _check_grad(dq_c[:, h], rq, f"large backward dq h{h}")
            _, rk, rv, _ = oracle.attention_backward_head(
                q[0, a:b, h], k[0, a - W + 1:b, hk], v[0, a - W + 1:b, hk], do[0, a:b, h],
                scale, True, W)
            # keys k0 .. k1 - 1 are entries W - 1 .. W + 126 of the key slice
            rk_sum = rk_sum + rk[W - 1: W - 1 + (k1 - k0)]
            rv_sum = rv_sum + rv[W - 1: W - 1 + (k1 - k0)]
        _check_grad(dk_c[:, hk], rk_sum, f"large backward dk hk{hk}")
        _check_grad(dv_c[:, hk], rv_sum, f"large backward dv hk{hk}")


def test_packed_prefill_past_2_31_elements():
    # three packed sequences of 557056 tokens in all; the third starts at row
    # 500000, so its rows from 24288 on lie past element 2**31
    lens = [300000, 200000, 57056]
    Hq, Hkv, d, W, seed = 32, 8, 128, 4096, 7304
    print("large packed prefill: generating inputs", flush=True)
    q, k, v, cu_q, cu_k = workloads.make_packed(lens, lens, Hq, Hkv, d, seed)
    scale = 1.0 / np.sqrt(d)
    out, lse = attn_fwd_varlen(q.cuda(), k.cuda(), v.cuda(), cu_q.cuda(), cu_k.cuda(), causal=True,
                               window=W, scale=scale)
    torch.cuda.synchronize()
    print("large packed prefill: kernel done", flush=True)
    first = _E31 // (Hq * d)
    # (sequence, local rows [a, b)): each sequence's first and last rows, and
    # the third's rows around the boundary
    spans = [(0, 0, 40), (0, lens[0] - 40, lens[0]), (1, 0, 40), (1, lens[1] - 40, lens[1]),
             (2, 0, 40), (2, first - 500000 - 64, first - 500000 + 64), (2, lens[2] - 40, lens[2])]
    for s, a, b in spans:
        t0 = int(cu_q[s])
        c = max(0, a - W + 1)
        for h in (0, 9, 31):
            O, L = oracle.attention_head(q[t0 + a: t0 + b, h], k[t0 + c: t0 + b, h // 4],
                                         v[t0 + c: t0 + b, h // 4], scale, True, W)
            check(out[t0 + a: t0 + b, h].cpu(), O, lse[h, t0 + a: t0 + b].cpu(), L, "bf16",
                  f"large packed prefill seq {s} rows {a}..{b} head {h}")


def test_chunked_prefill_blocks_past_2_31_elements():
    # the chunked prefill over a pool laid out as in the decode case
    lens, chunks = [3001, 700, 4096, 2500], [512, 700, 1, 1000]
    Hq, Hkv, d, seed = 32, 8, 128, 7305
    nblk = sum((n + 15) // 16 for n in lens)
    maxb = max((n + 15) // 16 for n in lens)
    print("large chunked prefill: generating inputs", flush=True)
    inp = workloads.make_prefill_paged(lens, chunks, Hq, Hkv, d, 16, nblk, maxb, seed)
    num_blocks = 135000
    shift = _E31 // (16 * Hkv * d) - nblk // 2
    table = inp["block_table"].clone()
    table[table >= 0] += shift
    kc = torch.full((num_blocks, 16, Hkv, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[shift: shift + nblk] = inp["kcache"].cuda()
    vc[shift: shift + nblk] = inp["vcache"].cuda()
    scale = 1.0 / np.sqrt(d)
    out, lse = attn_prefill_paged(inp["q"].cuda(), kc, vc, table.cuda(), inp["seq_lens"].cuda(),
                                  inp["cu_seqlens_q"].cuda(), scale=scale)
    torch.cuda.synchronize()
    print("large chunked prefill: kernel done", flush=True)
    O, L = oracle.prefill_paged(inp["q"], inp["kcache"], inp["vcache"], inp["block_table"],
                                inp["seq_lens"], inp["cu_seqlens_q"], scale)
    check(out.cpu(), O, lse.cpu(), L, "bf16", "large chunked prefill")


def test_merge_past_2_31_pieces():
    # 4718592 rows x 32 heads x 128: 2.42e9 16-byte pieces per tensor (38.7 GB
    # of O each), so the pieces of rows from 4194304 on have indices past 2**31
    B, N, H, d, seed = 1, 4718592, 32, 128, 7306
    first = _E31 // (H * (d // 8))
    assert B * N * H * (d // 8) > _E31 and first < N
    print("large merge: generating inputs on the device", flush=True)
    oa = workloads.draw_normal_device(seed, 0, (B, N, H, d))
    ob = workloads.draw_normal_device(seed, 1, (B, N, H, d))
    la = workloads.draw_normal_device(seed, 2, (B, H, N), torch.float32)
    lb = workloads.draw_normal_device(seed, 3, (B, H, N), torch.float32)
    out, lse = attn_merge(oa, la, ob, lb)
    torch.cuda.synchronize()
    print("large merge: kernel done", flush=True)
    rng = np.random.default_rng(seed)
    rows = {0, 1, N // 2, first - 2, first - 1, first, first + 1, N - 2, N - 1}
    rows |= set(int(x) for x in rng.integers(first - 1000, N, 24))
    rows = torch.tensor(sorted(rows), device="cuda")
    R = rows.numel()
    pick = lambda o: o[0].index_select(0, rows).cpu().double().numpy()       # [R, H, d]
    pickl = lambda l: l[0].index_select(1, rows).cpu().double().numpy()      # [H, R]
    xa, xb, xl_a, xl_b = pick(oa), pick(ob), pickl(la), pickl(lb)
    # the oracle's merge of (m, l, acc) states with m = LSE, l = 1, acc = O
    M, Ls, acc = oracle.merge_states(
        (xl_a.T.reshape(-1), np.ones(R * H), xa.reshape(-1, d)),
        (xl_b.T.reshape(-1), np.ones(R * H), xb.reshape(-1, d)))
    want_o = (acc / Ls[:, None]).reshape(R, H, d)
    want_l = (M + np.log(Ls)).reshape(R, H).T
    check(pick(out), want_o, pickl(lse), want_l, "bf16", "large merge")
