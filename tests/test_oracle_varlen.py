"""Pins of the packed-sequence (varlen) oracle, CPU only.

The oracle slices each sequence and applies the dense definition.  It is
pinned to a pure-Python brute force that never slices: it tests every packed
query row against every packed key row through the segment each belongs to.
Reductions: one sequence is the dense oracle on that sequence; sequences of
equal lengths are the dense batched oracle.  Planted mistakes in a copy of
the oracle's source must each fail one of these pins.
"""
import importlib
import inspect
import math
import types

import numpy as np
import pytest

import oracle
from oracle.brute import attention_brute_packed


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _packed(lens_q, lens_k, Hq, Hkv, d, seed):
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    q = _rand((int(cu_q[-1]), Hq, d), seed)
    k = _rand((int(cu_k[-1]), Hkv, d), seed + 1)
    v = _rand((int(cu_k[-1]), Hkv, d), seed + 2)
    return q, k, v, cu_q, cu_k


BRUTE_CASES = [
    # lens_q, lens_k, Hq, Hkv, d, causal, window
    ([3, 5, 2], [3, 5, 2], 2, 1, 3, True, 0),
    ([4, 0, 3], [6, 2, 3], 2, 2, 4, True, 0),        # an empty query set, Nq < Nk
    ([2, 4], [5, 4], 4, 2, 2, True, 2),             # windows
    ([3, 2, 4], [1, 6, 0], 1, 1, 3, False, 0),       # a sequence with no keys
    ([4, 3], [2, 3], 2, 1, 3, True, 0),              # more queries than keys, causal
    ([1, 1, 1, 1], [1, 2, 3, 4], 3, 1, 2, True, 0),  # one query each (decode-like)
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force_matches_varlen_oracle(case):
    lens_q, lens_k, Hq, Hkv, d, causal, window = case
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, Hq, Hkv, d, sum(lens_q) * 7 + Hq)
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal, window)
    Ob, Lb = attention_brute_packed(q.tolist(), k.tolist(), v.tolist(), cu_q.tolist(),
                                    cu_k.tolist(), scale, causal, window)
    np.testing.assert_allclose(O, np.array(Ob).reshape(O.shape), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb).reshape(L.shape), rtol=0, atol=1e-12)


def test_one_sequence_is_the_dense_oracle():
    q, k, v, cu_q, cu_k = _packed([9], [12], 4, 2, 5, 31)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.4, True, 5)
    Od, Ld = oracle.attention(q[None], k[None], v[None], 0.4, True, 5)
    np.testing.assert_array_equal(O, Od[0])
    np.testing.assert_array_equal(L, Ld[0])


def test_equal_lengths_are_the_dense_batch():
    B, Nq, Nk, Hq, Hkv, d = 3, 5, 7, 2, 1, 4
    q, k, v, cu_q, cu_k = _packed([Nq] * B, [Nk] * B, Hq, Hkv, d, 41)
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.6, True, 0)
    Od, Ld = oracle.attention(q.reshape(B, Nq, Hq, d), k.reshape(B, Nk, Hkv, d),
                              v.reshape(B, Nk, Hkv, d), 0.6, True, 0)
    np.testing.assert_array_equal(O, Od.reshape(B * Nq, Hq, d))
    np.testing.assert_array_equal(L, Ld.transpose(1, 0, 2).reshape(Hq, B * Nq))


def test_uncovered_rows_and_unselected_sequences_stay_nan():
    q, k, v, cu_q, cu_k = _packed([2, 3], [2, 3], 1, 1, 2, 51)
    q = np.concatenate([q, _rand((2, 1, 2), 52)])  # two rows after the last sequence
    O, L = oracle.attention_varlen(q, k, v, cu_q, cu_k, 1.0, True, 0, seqs=[1])
    assert np.isnan(O[:2]).all() and np.isnan(O[5:]).all() and np.isfinite(O[2:5]).all()
    assert np.isnan(L[:, :2]).all() and np.isfinite(L[:, 2:5]).all()


MUTATIONS = {
    "none": None,
    "keys sliced at the query offsets": ("k[k0:k1, hk, :], v[k0:k1, hk, :]",
                                         "k[q0:q0 + k1 - k0, hk, :], v[q0:q0 + k1 - k0, hk, :]"),
    "keys of earlier sequences leak in": ("k[k0:k1, hk, :], v[k0:k1, hk, :]",
                                          "k[:k1, hk, :], v[:k1, hk, :]"),
    "interleaved heads": ("hk = h // G", "hk = h % Hkv"),
    "next sequence's end": ("q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[s + 1]",
                            "q0, q1, k0, k1 = cq[s], cq[s + 1], ck[s], ck[min(s + 2, S)]"),
    "LSE of the wrong head": ("L[h, q0:q1] = l", "L[Hq - 1 - h, q0:q1] = l"),
}


def _mutant(name):
    real = importlib.import_module("oracle.varlen")
    src = inspect.getsource(real)
    m = MUTATIONS[name]
    if m is not None:
        old, new = m
        # the forward comes first in the module: its site is the first occurrence
        assert src.count(old) >= 1, f"mutation site for {name!r} not found"
        src = src.replace(old, new, 1)
    src = src.replace("from .attention import", "from oracle.attention import")
    src = src.replace("from .backward import", "from oracle.backward import")
    mod = types.ModuleType(f"oracle_varlen_mutant_{name.replace(' ', '_')}")
    exec(compile(src, mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_reject_planted_mistakes(name):
    mod = _mutant(name)
    ok = True
    for case in BRUTE_CASES:
        lens_q, lens_k, Hq, Hkv, d, causal, window = case
        q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, Hq, Hkv, d, 61)
        Ob, Lb = attention_brute_packed(q.tolist(), k.tolist(), v.tolist(), cu_q.tolist(),
                                        cu_k.tolist(), 0.7, causal, window)
        try:
            O, L = mod.attention_varlen(q, k, v, cu_q, cu_k, 0.7, causal, window)
            ok &= np.allclose(O, np.array(Ob).reshape(O.shape), rtol=0, atol=1e-12)
            ok &= np.allclose(L, np.array(Lb).reshape(L.shape), rtol=0, atol=1e-12)
        except Exception:
            ok = False
    if name == "none":
        assert ok, "the unmutated oracle must pass the brute-force pin"
    else:
        assert not ok, f"planted mistake {name!r} was not caught"


# ------------------------------------------------------------- gradients

def _numeric(fwd, xs, do, eps=1e-6):
    """Central differences of L = sum(dO * O) for every entry of each x."""
    grads = []
    for x in xs:
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = float(np.nansum(do * fwd()[0]))
            x[i] = old - eps
            lm = float(np.nansum(do * fwd()[0]))
            x[i] = old
            g[i] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


GRAD_CASES = [
    ([3, 4], [3, 4], 2, 1, 3, True, 0),
    ([2, 0, 3], [5, 2, 3], 2, 2, 2, True, 2),   # no queries in one sequence: its dK = dV = 0
    ([3, 2], [2, 0], 1, 1, 3, False, 0),         # no keys: dQ = 0
]


@pytest.mark.parametrize("case", GRAD_CASES)
def test_varlen_gradients_match_finite_differences(case):
    lens_q, lens_k, Hq, Hkv, d, causal, window = case
    q, k, v, cu_q, cu_k = _packed(lens_q, lens_k, Hq, Hkv, d, 81)
    do = _rand(q.shape, 82)

    def fwd():
        return oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.8, causal, window)

    nq, nk, nv = _numeric(fwd, (q, k, v), do)
    dq, dk, dv, _ = oracle.attention_varlen_backward(q, k, v, do, cu_q, cu_k, 0.8, causal, window)
    for name, a, n in (("dQ", dq, nq), ("dK", dk, nk), ("dV", dv, nv)):
        err = np.abs(a - n).max() / max(1.0, np.abs(n).max())
        assert err < 1e-7, f"{name} differs from finite differences by {err:.2e}"


def test_varlen_gradients_of_equal_lengths_are_the_dense_batch():
    B, N, Hq, Hkv, d = 2, 5, 2, 1, 3
    q, k, v, cu_q, cu_k = _packed([N] * B, [N] * B, Hq, Hkv, d, 83)
    do = _rand(q.shape, 84)
    dq, dk, dv, D = oracle.attention_varlen_backward(q, k, v, do, cu_q, cu_k, 0.5, True)
    rq, rk, rv, rD = oracle.attention_backward(q.reshape(B, N, Hq, d), k.reshape(B, N, Hkv, d),
                                               v.reshape(B, N, Hkv, d), do.reshape(B, N, Hq, d),
                                               0.5, True)
    np.testing.assert_array_equal(dq, rq.reshape(dq.shape))
    np.testing.assert_array_equal(dk, rk.reshape(dk.shape))
    np.testing.assert_array_equal(dv, rv.reshape(dv.shape))
    np.testing.assert_array_equal(D, rD.transpose(1, 0, 2).reshape(Hq, B * N))
