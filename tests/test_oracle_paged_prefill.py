"""Pins of the chunked-prefill-over-a-paged-cache oracle, CPU only.

The oracle gathers each sequence's cache with numpy fancy indexing and runs
the dense definition with the chunk's queries as the last rows.  It is pinned
to a brute force that copies tokens one at a time through the table and
runs the pure-Python definition, to the decode oracle (one new token per
sequence) and to the packed-sequence oracle (a table that lays the cache
out contiguously).  Planted mistakes must each fail one of these pins.
"""
import importlib
import inspect
import math
import types

import numpy as np
import pytest

import oracle
from oracle.brute import prefill_paged_brute


def _case(lens, chunks, Hq, Hkv, d, bs, seed, contiguous=False):
    rng = np.random.default_rng(seed)
    S = len(lens)
    max_blocks = max(1, max((n + bs - 1) // bs for n in lens))
    need = sum((n + bs - 1) // bs for n in lens)
    num_blocks = need + 3
    ids = np.arange(num_blocks) if contiguous else rng.permutation(num_blocks)
    table = np.full((S, max_blocks), -1, dtype=np.int64)
    pos = 0
    for s, n in enumerate(lens):
        nb = (n + bs - 1) // bs
        table[s, :nb] = ids[pos:pos + nb]
        pos += nb
    kc = rng.standard_normal((num_blocks, bs, Hkv, d))
    vc = rng.standard_normal((num_blocks, bs, Hkv, d))
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int64)
    q = rng.standard_normal((int(cu[-1]), Hq, d))
    return q, kc, vc, table, np.asarray(lens), cu


CASES = [
    # lens, chunks, Hq, Hkv, d, bs, window
    ([7, 5, 9], [3, 5, 1], 2, 1, 3, 4, 0),
    ([12, 0, 6], [4, 0, 6], 2, 2, 2, 4, 0),     # an empty sequence, a chunk = whole context
    ([10, 11], [6, 2], 4, 2, 3, 4, 3),          # window
    ([13], [13], 1, 1, 4, 5, 0),               # one sequence, block size 5
]


@pytest.mark.parametrize("case", CASES)
def test_brute_force_matches_oracle(case):
    lens, chunks, Hq, Hkv, d, bs, window = case
    q, kc, vc, table, sl, cu = _case(lens, chunks, Hq, Hkv, d, bs, 71)
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.prefill_paged(q, kc, vc, table, sl, cu, scale, window)
    Ob, Lb = prefill_paged_brute(q.tolist(), kc.tolist(), vc.tolist(), table.tolist(),
                                 sl.tolist(), cu.tolist(), scale, window)
    np.testing.assert_allclose(O, np.array(Ob).reshape(O.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb).reshape(L.shape), rtol=0, atol=1e-12)


def test_one_new_token_is_decode():
    lens = [9, 16, 3]
    q, kc, vc, table, sl, cu = _case(lens, [1, 1, 1], 4, 2, 3, 4, 72)
    O, L = oracle.prefill_paged(q, kc, vc, table, sl, cu, 0.5, 5)
    Od, Ld = oracle.decode_paged(q, kc, vc, table, sl, 0.5, window=5)
    np.testing.assert_allclose(O, Od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Ld.T, rtol=0, atol=1e-12)


def test_contiguous_table_is_packed_attention():
    lens, chunks = [8, 12, 5], [8, 4, 2]
    bs = 4
    q, kc, vc, table, sl, cu = _case(lens, chunks, 2, 1, 3, bs, 73, contiguous=True)
    # blocks of sequence s are consecutive: the cache read in block order is
    # the sequences' tokens back to back once each sequence's tail slots are cut
    flat_k = kc.reshape(-1, 1, 3)
    flat_v = vc.reshape(-1, 1, 3)
    starts = np.concatenate([[0], np.cumsum([(n + bs - 1) // bs * bs for n in lens])])
    keep = np.concatenate([np.arange(starts[s], starts[s] + n) for s, n in enumerate(lens)])
    cu_k = np.concatenate([[0], np.cumsum(lens)])
    O, L = oracle.prefill_paged(q, kc, vc, table, sl, cu, 0.7)
    Ov, Lv = oracle.attention_varlen(q, flat_k[keep], flat_v[keep], cu, cu_k, 0.7, causal=True)
    np.testing.assert_allclose(O, Ov, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lv, rtol=0, atol=1e-12)


def test_bad_block_gives_nan_for_that_sequence_only():
    q, kc, vc, table, sl, cu = _case([6, 6], [2, 2], 1, 1, 2, 4, 74)
    table[1, 1] = kc.shape[0] + 5
    O, L = oracle.prefill_paged(q, kc, vc, table, sl, cu, 1.0)
    assert np.isfinite(O[:2]).all() and np.isnan(O[2:]).all() and np.isnan(L[:, 2:]).all()


MUTATIONS = {
    "none": None,
    "values from the key cache": ("vc = gather_paged(vcache, table[s], n)",
                                  "vc = gather_paged(kcache, table[s], n)"),
    "interleaved heads": ("o, l = attention_head(qs[:, h, :], kc[:, h // G, :]",
                          "o, l = attention_head(qs[:, h, :], kc[:, h % Hkv, :]"),
    "window ignored": ("causal=True, window=window)\n            O[q0:q1, h] = o",
                       "causal=True, window=0)\n            O[q0:q1, h] = o"),
    "cache cut to the chunk": ("kc = gather_paged(kcache, table[s], n)",
                               "kc = gather_paged(kcache, table[s], n)[: max(q1 - q0, 1)]"),
    "not causal": ("causal=True, window=window)\n            O[q0:q1, h] = o",
                   "causal=False, window=window)\n            O[q0:q1, h] = o"),
}


def _mutant(name):
    real = importlib.import_module("oracle.attention")
    src = inspect.getsource(real)
    m = MUTATIONS[name]
    if m is not None:
        old, new = m
        assert src.count(old) == 1, f"mutation site for {name!r} not unique"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_paged_prefill_mutant_{name.replace(' ', '_')}")
    exec(compile(src, mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_reject_planted_mistakes(name):
    mod = _mutant(name)
    ok = True
    for case in CASES:
        lens, chunks, Hq, Hkv, d, bs, window = case
        q, kc, vc, table, sl, cu = _case(lens, chunks, Hq, Hkv, d, bs, 75)
        Ob, Lb = prefill_paged_brute(q.tolist(), kc.tolist(), vc.tolist(), table.tolist(),
                                     sl.tolist(), cu.tolist(), 0.6, window)
        try:
            O, L = mod.prefill_paged(q, kc, vc, table, sl, cu, 0.6, window)
            ok &= np.allclose(O, np.array(Ob).reshape(O.shape), rtol=0, atol=1e-12)
            ok &= np.allclose(L, np.array(Lb).reshape(L.shape), rtol=0, atol=1e-12)
        except Exception:
            ok = False
    if name == "none":
        assert ok, "the unmutated oracle must pass the brute-force pin"
    else:
        assert not ok, f"planted mistake {name!r} was not caught"
