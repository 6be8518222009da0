"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutant is the oracle's own source with one textual change (a dropped
term, a wrong sign, index or axis, a transposed operand), executed as a
throw-away module on the CPU.  The real oracle is never modified.
"""

import importlib.util
import os
import types

import pytest

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "scale dropped from scores": ("return float(scale) * (q @ k.T)", "return (q @ k.T)"),
    "causal mask off by one": ("vis &= j <= pos", "vis &= j < pos"),
    "causal mask transposed": ("vis &= j <= pos", "vis &= j >= pos"),
    "causal keys aligned to the start": ("pos = rows[:, None] + (n_k - n_q)", "pos = rows[:, None] + 0"),
    "causal offset sign reversed": ("pos = rows[:, None] + (n_k - n_q)", "pos = rows[:, None] + (n_q - n_k)"),
    "window one key too wide": ("vis &= np.abs(pos - j) < window", "vis &= np.abs(pos - j) <= window"),
    "window one-sided": ("vis &= np.abs(pos - j) < window", "vis &= (pos - j) < window"),
    "window ignored by the backward": ("visible_mask(q.shape[0], k.shape[0], causal, None, window)",
                                       "visible_mask(q.shape[0], k.shape[0], causal, None, 0)"),
    "query heads spread round-robin over K/V heads": ("return h // (n_heads // n_kv_heads)",
                                                      "return h % n_kv_heads"),
    "shared K/V gradient overwritten, not summed": ("dk[b, :, hk, :] += gk", "dk[b, :, hk, :] = gk"),
    "softmax summed over the wrong axis": ("l = e.sum(axis=1)", "l = e.sum(axis=0)"),
    "max shift not undone in LSE": ("m + np.log(np.where(l > 0, l, 1.0))",
                                    "np.log(np.where(l > 0, l, 1.0))"),
    "probabilities transposed in PV": ("o = p @ v", "o = p.T @ v"),
    "dV without transpose": ("dv = p.T @ do", "dv = p @ do"),
    "dP with V untransposed rows": ("dp = do @ v.T", "dp = do @ v.T[:, ::-1]"),
    "Jacobian sign flipped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                              "ds = p * (dp + (p * dp).sum(axis=1, keepdims=True))"),
    "Jacobian term dropped": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                              "ds = p * dp"),
    "dQ missing scale": ("dq = float(scale) * (ds @ k)", "dq = (ds @ k)"),
    "dK without transpose": ("dk = float(scale) * (ds.T @ q)", "dk = float(scale) * (ds @ q)"),
    "dK from K instead of Q": ("dk = float(scale) * (ds.T @ q)", "dk = float(scale) * (ds.T @ k)"),
}


def _load_mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _load_mutant(*MUTANTS[name])
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except Exception as exc:  # AssertionError, or a shape error from the mutant
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutant: {name}"
