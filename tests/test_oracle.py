"""Pins of the fp64 oracle against the pages, closed forms and invariants.

None of these compares the oracle with itself: each expected value comes from
a page (the fixtures under tests/golden/, each naming its source), from a
closed form that holds for the definition, from a pure-Python brute force
written independently, or from an invariant of the mathematics.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.brute import attention_brute
from tests.conftest import load_golden


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


# ---------------------------------------------------------------- pages' values

def test_online_softmax_worked_example():
    g = load_golden("online_softmax_worked_example.json")
    probs, m, den = oracle.online_softmax(g["scores"])
    assert round(den, g["denominator_decimals"]) == g["denominator_after"][-1]
    assert m == g["running_max_after"][-1]
    for p, want in zip(probs, g["probabilities"]):
        assert round(p, g["probability_decimals"]) == want
    # after the first score alone the state is (m=1, d=1)
    _, m1, d1 = oracle.online_softmax(g["scores"][:1])
    assert (m1, d1) == (g["running_max_after"][0], g["denominator_after"][0])


def test_worked_example_as_attention():
    """Scores [1, 3] as one query over two keys: q=[1,0], k=[[1,0],[3,0]], V=I."""
    g = load_golden("online_softmax_worked_example.json")
    q = np.array([[1.0, 0.0]])
    k = np.array([[1.0, 0.0], [3.0, 0.0]])
    v = np.eye(2)
    d_print = g["denominator_decimals"]
    p_print = g["probability_decimals"]
    for o, lse in [oracle.attention_head(q, k, v, scale=1.0),
                   oracle.tiled_attention_head(q, k, v, scale=1.0, block_q=1, block_k=1)]:
        assert [round(x, p_print) for x in o[0]] == g["probabilities"]
        # LSE = running max + ln(running denominator)
        den = math.exp(lse[0] - g["running_max_after"][-1])
        assert round(den, d_print) == g["denominator_after"][-1]
    O, L = attention_brute([[[[1.0, 0.0]]]], [[[[1.0, 0.0]], [[3.0, 0.0]]]],
                           [[[[1.0, 0.0]], [[0.0, 1.0]]]], 1.0)
    assert [round(x, p_print) for x in O[0][0][0]] == g["probabilities"]
    assert round(math.exp(L[0][0][0] - 3.0), d_print) == g["denominator_after"][-1]


def test_sliding_window_picture():
    g = load_golden("sliding_window_mask_n8_w3.json")
    n, w = g["n"], g["window"]
    vis = oracle.visible_mask(n, n, causal=True, window=w)
    drawn = ["".join("X" if x else "." for x in row) for row in vis]
    assert drawn == g["pattern"]
    assert int(vis.sum()) == g["allowed_pairs_window"]
    assert int(oracle.visible_mask(n, n, True, 0).sum()) == g["allowed_pairs_causal"]
    # the tiled recurrence with 1x1 blocks visits exactly the allowed pairs
    q = k = v = _rand((n, 2), 0)
    *_, visited = oracle.tiled_attention_head(q, k, v, 1.0, True, w, 1, 1, return_stats=True)
    assert visited == g["allowed_pairs_window"]


# ---------------------------------------------------------------- brute force

BRUTE_CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, window
    (1, 5, 5, 1, 1, 3, False, 0),
    (2, 6, 6, 4, 2, 4, True, 0),
    (1, 7, 7, 4, 1, 8, True, 3),
    (2, 3, 9, 2, 2, 5, True, 0),     # Nq < Nk: bottom-right causal
    (1, 4, 11, 4, 4, 3, True, 5),    # Nq < Nk with a window
    (1, 8, 8, 2, 1, 6, False, 0),
    (1, 1, 13, 4, 2, 8, True, 0),    # single decode-like query
    (1, 16, 16, 2, 2, 2, True, 16),  # window equal to n
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_brute_force_matches_oracle(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    seed = hash(case) % 1000
    q = _rand((B, Nq, Hq, d), seed)
    k = _rand((B, Nk, Hkv, d), seed + 1)
    v = _rand((B, Nk, Hkv, d), seed + 2)
    scale = 1.0 / math.sqrt(d)
    O, L = oracle.attention(q, k, v, scale, causal, window)
    Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, window)
    np.testing.assert_allclose(O, np.array(Ob), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, np.array(Lb), rtol=0, atol=1e-12)
    To = np.stack([np.stack([oracle.tiled_attention_head(
        q[b, :, h], k[b, :, h // (Hq // Hkv)], v[b, :, h // (Hq // Hkv)], scale, causal, window,
        block_q=3, block_k=4)[0] for h in range(Hq)], axis=1) for b in range(B)])
    np.testing.assert_allclose(To, np.array(Ob), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_constant_values_give_constant_output():
    q = _rand((2, 40, 4, 16), 1)
    k = _rand((2, 40, 2, 16), 2)
    c = _rand((16,), 3)
    v = np.broadcast_to(c, (2, 40, 2, 16)).copy()
    for causal, window in [(False, 0), (True, 0), (True, 7)]:
        O, _ = oracle.attention(q, k, v, 0.25, causal, window)
        np.testing.assert_allclose(O, np.broadcast_to(c, O.shape), rtol=0, atol=1e-13)


def test_causal_first_row_is_first_value():
    q = _rand((1, 33, 2, 8), 4)
    k = _rand((1, 33, 2, 8), 5)
    v = _rand((1, 33, 2, 8), 6)
    O, L = oracle.attention(q, k, v, 0.3, causal=True)
    for h in range(2):
        np.testing.assert_array_equal(O[0, 0, h], v[0, 0, h])
        assert L[0, h, 0] == pytest.approx(0.3 * float(q[0, 0, h] @ k[0, 0, h]), abs=1e-14)


def test_zero_scale_gives_mean_of_visible_values():
    n, W = 30, 4
    q = _rand((1, n, 1, 8), 7)
    k = _rand((1, n, 1, 8), 8)
    v = _rand((1, n, 1, 8), 9)
    O, L = oracle.attention(q, k, v, 0.0, causal=True, window=W)
    for i in range(n):
        lo = max(0, i - W + 1)
        np.testing.assert_allclose(O[0, i, 0], v[0, lo:i + 1, 0].mean(axis=0), atol=1e-14)
        assert L[0, 0, i] == pytest.approx(math.log(i + 1 - lo), abs=1e-14)


def test_single_key():
    q = _rand((1, 5, 3, 4), 10)
    k = _rand((1, 1, 3, 4), 11)
    v = _rand((1, 1, 3, 4), 12)
    O, L = oracle.attention(q, k, v, 0.5)
    for h in range(3):
        np.testing.assert_array_equal(O[0, :, h], np.broadcast_to(v[0, 0, h], (5, 4)))
        np.testing.assert_allclose(L[0, h], 0.5 * (q[0, :, h] @ k[0, 0, h]), atol=1e-14)


def test_no_visible_key_gives_zero_and_minus_inf():
    # window without causal restriction from above, but a query can still
    # have nothing visible only when Nk == 0; use the head function directly
    o, l = oracle.attention_head(np.ones((2, 4)), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(l == -np.inf)


# ---------------------------------------------------------------- invariants

def test_softmax_rows_sum_to_one():
    q = _rand((50, 16), 13, 3.0)
    k = _rand((70, 16), 14, 3.0)
    v = _rand((70, 16), 15)
    for causal, window in [(False, 0), (True, 0), (True, 9)]:
        _, _, P = oracle.attention_head(q, k, v, 0.25, causal, window, return_p=True)
        np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
        assert np.all(P >= 0)
        vis = oracle.visible_mask(50, 70, causal, window)
        assert np.all(P[~vis] == 0)


def test_window_at_least_n_equals_causal():
    q = _rand((1, 64, 2, 8), 16)
    k = _rand((1, 64, 2, 8), 17)
    v = _rand((1, 64, 2, 8), 18)
    Oc, Lc = oracle.attention(q, k, v, 0.35, causal=True)
    for W in (64, 65, 1000):
        Ow, Lw = oracle.attention(q, k, v, 0.35, causal=True, window=W)
        np.testing.assert_array_equal(Ow, Oc)
        np.testing.assert_array_equal(Lw, Lc)
    Ow, _ = oracle.attention(q, k, v, 0.35, causal=True, window=63)
    assert not np.array_equal(Ow, Oc)


@pytest.mark.parametrize("Hkv", [1, 2, 4])
def test_gqa_equals_mha_on_repeated_kv(Hkv):
    Hq = 8
    q = _rand((2, 20, Hq, 8), 19)
    k = _rand((2, 20, Hkv, 8), 20)
    v = _rand((2, 20, Hkv, 8), 21)
    O, L = oracle.attention(q, k, v, 0.3, causal=True)
    # repeat each KV head Hq/Hkv times, in place (head 0 0 0 .. 1 1 1 ..)
    kr = np.repeat(k, Hq // Hkv, axis=2)
    vr = np.repeat(v, Hq // Hkv, axis=2)
    Om, Lm = oracle.attention(q, kr, vr, 0.3, causal=True)
    np.testing.assert_array_equal(O, Om)
    np.testing.assert_array_equal(L, Lm)
    if Hkv > 1:  # an interleaved (h % Hkv) mapping would differ
        ki = np.tile(k, (1, 1, Hq // Hkv, 1))
        vi = np.tile(v, (1, 1, Hq // Hkv, 1))
        Oi, _ = oracle.attention(q, ki, vi, 0.3, causal=True)
        assert not np.allclose(O, Oi)


def test_non_causal_key_permutation_invariance():
    q = _rand((1, 12, 2, 8), 22)
    k = _rand((1, 30, 2, 8), 23)
    v = _rand((1, 30, 2, 8), 24)
    perm = np.random.default_rng(0).permutation(30)
    O, L = oracle.attention(q, k, v, 0.4)
    Op, Lp = oracle.attention(q, k[:, perm], v[:, perm], 0.4)
    np.testing.assert_allclose(Op, O, atol=1e-14)
    np.testing.assert_allclose(Lp, L, atol=1e-14)


def test_lse_reproduces_the_output():
    q = _rand((25, 8), 25, 2.0)
    k = _rand((40, 8), 26, 2.0)
    v = _rand((40, 8), 27)
    for causal, window in [(False, 0), (True, 0), (True, 6)]:
        O, L = oracle.attention_head(q, k, v, 0.5, causal, window)
        vis = oracle.visible_mask(25, 40, causal, window)
        S = (q @ k.T) * 0.5
        W = np.where(vis, np.exp(S - L[:, None]), 0.0)
        np.testing.assert_allclose(W.sum(axis=1), 1.0, atol=1e-12)
        np.testing.assert_allclose(W @ v, O, atol=1e-12)


@pytest.mark.parametrize("bq,bk", [(32, 32), (16, 48), (7, 5), (64, 128)])
@pytest.mark.parametrize("causal,window", [(False, 0), (True, 0), (True, 40)])
def test_tiled_recurrence_equals_naive(bq, bk, causal, window):
    q = _rand((150, 16), 28, 2.0)
    k = _rand((170, 16), 29, 2.0)
    v = _rand((170, 16), 30)
    O, L = oracle.attention_head(q, k, v, 0.25, causal, window)
    To, TL = oracle.tiled_attention_head(q, k, v, 0.25, causal, window, bq, bk)
    np.testing.assert_allclose(To, O, atol=1e-12)
    np.testing.assert_allclose(TL, L, atol=1e-12)


def test_tiled_causal_visits_half_the_blocks():
    n, b = 256, 32
    q = k = v = _rand((n, 4), 31)
    *_, visited = oracle.tiled_attention_head(q, k, v, 1.0, True, 0, b, b, return_stats=True)
    t = n // b
    assert visited == t * (t + 1) // 2


def test_merge_of_two_halves_equals_whole():
    q = _rand((20, 8), 32)
    k = _rand((64, 8), 33)
    v = _rand((64, 8), 34)
    O, L = oracle.attention_head(q, k, v, 0.4)
    Oa, La = oracle.attention_head(q, k[:23], v[:23], 0.4)
    Ob, Lb = oracle.attention_head(q, k[23:], v[23:], 0.4)
    # (LSE, 1, O) is a valid partial state: l * e^m equals the sum of exp
    M, Lsum, acc = oracle.merge_states((La, np.ones(20), Oa), (Lb, np.ones(20), Ob))
    np.testing.assert_allclose(acc / Lsum[:, None], O, atol=1e-13)
    np.testing.assert_allclose(M + np.log(Lsum), L, atol=1e-13)
    # merging with an empty state changes nothing
    M2, L2, A2 = oracle.merge_states((La, np.ones(20), Oa),
                                     (np.full(20, -np.inf), np.zeros(20), np.zeros((20, 8))))
    np.testing.assert_array_equal(A2, Oa)
    np.testing.assert_array_equal(M2, La)


def test_bf16_inputs_are_widened_exactly():
    t = torch.randn(3, 5, 2, 8).to(torch.bfloat16)
    o1, l1 = oracle.attention(t, t[:, :, :1], t[:, :, :1], 0.5)
    a = t.to(torch.float64).numpy()
    o2, l2 = oracle.attention(a, a[:, :, :1], a[:, :, :1], 0.5)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
