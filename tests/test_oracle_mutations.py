"""The oracle's pins catch plausible mistakes.

Each case plants one mistake into a copy of the oracle's source (on the CPU,
never touching the real module) and checks that at least one pin — the
pages' worked example and window picture, the brute force, or a closed form
or invariant — rejects the mutant.  The unmutated copy must pass them all.
"""
import importlib
import inspect
import math
import types

import numpy as np
import pytest

from oracle.brute import attention_brute
from tests.conftest import load_golden

MUTATIONS = {
    "none": None,
    "dropped scale": ("s = (q[r] @ k.T) * scale", "s = (q[r] @ k.T)"),
    "causal off by one": ("vis &= j <= pos", "vis &= j < pos"),
    "window off by one": ("vis &= (pos - j) < window", "vis &= (pos - j) <= window"),
    "top-left causal": ("[:, None] + (Nk - Nq)", "[:, None]"),
    "interleaved heads": ("hk = h // G", "hk = h % Hkv"),
    "lse sign": ("m[live] + np.log(l[live])", "m[live] - np.log(l[live])"),
    "no normalisation": ("p[live] / l[live, None]", "p[live]"),
    "values of wrong key": ("out[c0: c0 + r.shape[0]] = P @ v",
                            "out[c0: c0 + r.shape[0]] = P @ v[::-1]"),
    "transposed product": ("s = (q[r] @ k.T) * scale", "s = (k[:r.shape[0]] @ q.T) * scale"),
}


def _mutant(name):
    # the submodule itself (the package re-exports a function of the same name)
    real = importlib.import_module("oracle.attention")
    src = inspect.getsource(real)
    m = MUTATIONS[name]
    if m is not None:
        old, new = m
        assert src.count(old) == 1, f"mutation site for {name!r} not unique"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle_mutant_{name.replace(' ', '_')}")
    exec(compile(src, mod.__name__, "exec"), mod.__dict__)
    return mod


def _pins(mod):
    """Return the names of the pins the module fails."""
    failed = []
    # worked example (scores [1, 3])
    g = load_golden("online_softmax_worked_example.json")
    try:
        o, l = mod.attention_head(np.array([[1.0, 0.0]]), np.array([[1.0, 0.0], [3.0, 0.0]]),
                                  np.eye(2), scale=1.0)
        ok = [round(x, 3) for x in o[0]] == g["probabilities"] and \
            round(math.exp(l[0] - 3.0), 4) == g["denominator_after"][-1]
    except Exception:
        ok = False
    if not ok:
        failed.append("worked example")
    # window picture
    gw = load_golden("sliding_window_mask_n8_w3.json")
    vis = mod.visible_mask(8, 8, True, 3)
    if ["".join("X" if x else "." for x in row) for row in vis] != gw["pattern"]:
        failed.append("window picture")
    # brute force on square and bottom-right shapes with GQA
    rng = np.random.default_rng(0)
    for (Nq, Nk, Hq, Hkv, causal, W) in [(6, 6, 4, 2, True, 0), (3, 8, 4, 2, True, 3),
                                         (5, 5, 2, 1, False, 0)]:
        q = rng.standard_normal((1, Nq, Hq, 4))
        k = rng.standard_normal((1, Nk, Hkv, 4))
        v = rng.standard_normal((1, Nk, Hkv, 4))
        try:
            O, L = mod.attention(q, k, v, 0.5, causal, W)
            Ob, Lb = attention_brute(q.tolist(), k.tolist(), v.tolist(), 0.5, causal, W)
            ok = np.allclose(O, Ob, atol=1e-12) and np.allclose(L, Lb, atol=1e-12)
        except Exception:
            ok = False
        if not ok:
            failed.append(f"brute {Nq}x{Nk}")
    # closed form: causal row 0 is v0
    q = rng.standard_normal((1, 5, 1, 4))
    k = rng.standard_normal((1, 5, 1, 4))
    v = rng.standard_normal((1, 5, 1, 4))
    try:
        O, _ = mod.attention(q, k, v, 0.5, True)
        ok = np.array_equal(O[0, 0, 0], v[0, 0, 0])
    except Exception:
        ok = False
    if not ok:
        failed.append("causal row 0")
    return failed


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_reject_mutant(name):
    failed = _pins(_mutant(name))
    if name == "none":
        assert failed == []
    else:
        assert failed, f"no pin caught the mutation {name!r}"
