"""Pins of the backward oracle (fp64 gradients), CPU only.

The gradients are pinned to the forward oracle by central finite differences
of L = sum(dO * O) (an independent route: only the forward definition is
evaluated), to closed forms (keys or values that are all equal), and to the
identity D_i = sum_c dO_ic O_ic.  Planted mistakes in a copy of the backward
source must each fail one of these pins.
"""
import importlib
import inspect
import types

import numpy as np
import pytest

from oracle import attention, attention_backward


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _numeric_grads(fwd, q, k, v, do, eps=1e-6):
    """Central differences of L = sum(dO * O(q, k, v)) for every entry."""
    def loss(q_, k_, v_):
        O, _ = fwd(q_, k_, v_)
        return float((do * O).sum())
    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = loss(q, k, v)
            x[i] = old - eps
            lm = loss(q, k, v)
            x[i] = old
            g[i] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


CASES = [
    # B, Nq, Nk, Hq, Hkv, d, causal, window
    (1, 5, 5, 1, 1, 3, False, 0),
    (1, 6, 6, 2, 1, 4, True, 0),      # GQA: two query heads share one KV head
    (2, 4, 7, 2, 2, 3, True, 0),      # Nq < Nk: bottom-right causal
    (1, 7, 7, 3, 1, 2, True, 3),      # sliding window of 3 keys
    (1, 3, 6, 1, 1, 4, True, 2),      # window with Nq < Nk
]


@pytest.mark.parametrize("case", CASES)
def test_backward_matches_finite_differences(case):
    B, Nq, Nk, Hq, Hkv, d, causal, window = case
    q = _rand((B, Nq, Hq, d), 1)
    k = _rand((B, Nk, Hkv, d), 2)
    v = _rand((B, Nk, Hkv, d), 3)
    do = _rand((B, Nq, Hq, d), 4)
    scale = 0.7

    def fwd(q_, k_, v_):
        return attention(q_, k_, v_, scale=scale, causal=causal, window=window)

    nq, nk, nv = _numeric_grads(fwd, q, k, v, do)
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale=scale, causal=causal, window=window)
    for name, a, n in (("dQ", dq, nq), ("dK", dk, nk), ("dV", dv, nv)):
        err = np.abs(a - n).max() / max(1.0, np.abs(n).max())
        assert err < 1e-7, f"{name} differs from finite differences by {err:.2e}"


def test_equal_keys_give_no_query_gradient():
    # every score of a row is the same: the softmax is flat whatever q is
    q = _rand((1, 4, 1, 3), 5)
    row = _rand((3,), 6)
    k = np.tile(row, (1, 6, 1, 1))
    v = _rand((1, 6, 1, 3), 7)
    do = _rand((1, 4, 1, 3), 8)
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale=0.5)
    assert np.abs(dq).max() < 1e-12
    # dK sums to zero over the keys (softmax rows sum to one)
    assert np.abs(dk.sum(axis=1)).max() < 1e-12


def test_equal_values_give_no_score_gradient():
    # O = v for every row whatever P is, so only dV is nonzero: dV_j = sum_i P_ij dO_i
    q = _rand((1, 5, 1, 3), 9)
    k = _rand((1, 5, 1, 3), 10)
    row = _rand((3,), 11)
    v = np.tile(row, (1, 5, 1, 1))
    do = _rand((1, 5, 1, 3), 12)
    dq, dk, dv, _ = attention_backward(q, k, v, do, scale=0.9, causal=True)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # causal rows: P is a softmax over keys 0..i; column sums of dV give sum_i dO_i
    assert np.allclose(dv.sum(axis=1), do.sum(axis=1), atol=1e-12)


def test_row_dot_identity():
    q = _rand((1, 6, 2, 4), 13)
    k = _rand((1, 6, 1, 4), 14)
    v = _rand((1, 6, 1, 4), 15)
    do = _rand((1, 6, 2, 4), 16)
    O, _ = attention(q, k, v, scale=0.5, causal=True)
    _, _, _, D = attention_backward(q, k, v, do, scale=0.5, causal=True)
    want = (do * O).sum(axis=3).transpose(0, 2, 1)  # [B, Hq, Nq]
    assert np.abs(D - want).max() < 1e-12


def test_row_without_visible_key_contributes_nothing():
    # an empty key set: no row sees a key
    q = _rand((1, 2, 1, 3), 17)
    k = np.zeros((1, 0, 1, 3))
    v = np.zeros((1, 0, 1, 3))
    do = _rand((1, 2, 1, 3), 18)
    dq, dk, dv, D = attention_backward(q, k, v, do, scale=1.0)
    assert np.all(dq == 0) and dk.size == 0 and dv.size == 0 and np.all(D == 0)


MUTATIONS = {
    "none": None,
    "D sign": ("ds = P * (dp - D[:, None])", "ds = P * (dp + D[:, None])"),
    "D dropped": ("ds = P * (dp - D[:, None])", "ds = P * dp"),
    "dQ scale dropped": ("dq[r] = scale * (ds @ k)", "dq[r] = (ds @ k)"),
    "dK from P instead of dS": ("dk += scale * (ds.T @ q[r])", "dk += scale * (P.T @ q[r])"),
    "dK with the queries reversed": ("dk += scale * (ds.T @ q[r])", "dk += scale * (ds.T @ q[r][::-1])"),
    "dV from unnormalised weights": ("dv += P.T @ do[r]", "dv += p.T @ do[r]"),
    "dP with V not V^T": ("dp = do[r] @ v.T", "dp = do[r] @ v[::-1].T"),
    "GQA overwrite": ("dK[b, :, hk, :] += dk", "dK[b, :, hk, :] = dk"),
    "mask ignored": ("s = np.where(vis, s, -np.inf)", "s = s"),
}


def _mutant(name):
    real = importlib.import_module("oracle.backward")
    src = inspect.getsource(real)
    m = MUTATIONS[name]
    if m is not None:
        old, new = m
        assert src.count(old) == 1, f"mutation site for {name!r} not unique"
        src = src.replace(old, new)
    src = src.replace("from .attention import", "from oracle.attention import")
    mod = types.ModuleType(f"oracle_backward_mutant_{name.replace(' ', '_')}")
    exec(compile(src, mod.__name__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_reject_planted_mistakes(name):
    mod = _mutant(name)
    B, Nq, Nk, Hq, Hkv, d, causal, window = (1, 5, 6, 2, 1, 3, True, 0)
    q = _rand((B, Nq, Hq, d), 21)
    k = _rand((B, Nk, Hkv, d), 22)
    v = _rand((B, Nk, Hkv, d), 23)
    do = _rand((B, Nq, Hq, d), 24)

    def fwd(q_, k_, v_):
        return attention(q_, k_, v_, scale=0.8, causal=causal, window=window)

    nq, nk, nv = _numeric_grads(fwd, q, k, v, do)
    try:
        dq, dk, dv, _ = mod.attention_backward(q, k, v, do, scale=0.8, causal=causal, window=window)
        err = max(np.abs(a - n).max() for a, n in ((dq, nq), (dk, nk), (dv, nv)))
        ok = err < 1e-7
    except Exception:
        ok = False
    if name == "none":
        assert ok, "the unmutated oracle must pass its finite-difference pin"
    else:
        assert not ok, f"planted mistake {name!r} was not caught"
