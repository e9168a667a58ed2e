"""Each plausible mistake planted in the oracle (on the CPU, via monkeypatch)
makes at least one pin fail: the pins are not blind to it."""
import numpy as np
import pytest

import tests.test_oracle_pins as pins
from oracle import aoh, fasa

PINS = [getattr(pins, n) for n in dir(pins) if n.startswith("test_") and
        not hasattr(getattr(pins, n), "pytestmark")]


def _any_pin_fails():
    for fn in PINS:
        try:
            fn()
        except AssertionError:
            return True
    return False


def _er_sigma_squared(eigenvalues):
    lam = np.clip(np.asarray(eigenvalues, dtype=np.float64), 0.0, None)
    return aoh.effective_rank_from_singular(lam)


def _proxy_without_congruence(wq_h, wk_g):
    gq, gk = aoh.gram(wq_h), aoh.gram(wk_g)
    return np.linalg.eigvalsh(0.5 * (gq + gq.T)) * np.trace(gk) / gk.shape[0]


def _interleaved_pairing(i_dom, d_head, pairing="rotate_half"):
    f = np.asarray(i_dom, dtype=np.int64)
    return np.concatenate([2 * f, 2 * f + 1])


def _attend_unscaled(q, keys, values):
    z = np.asarray(keys) @ np.asarray(q)
    p = np.exp(z - z.max())
    return (p / p.sum()) @ np.asarray(values)


def _top_n_unstable(scores, n):
    return np.sort(np.argsort(-np.asarray(scores), kind="quicksort")[:n])


def _top_n_lowest(scores, n):
    return np.sort(np.lexsort((np.arange(len(scores)), np.asarray(scores)))[:n])


def _group_query_first_head(q_group):
    return np.asarray(q_group, dtype=np.float64)[0]


def _window_off_by_one(T, n_sink, window):
    s_end = min(n_sink, T)
    w_start = max(T - window + 1, s_end)
    return np.concatenate([np.arange(0, s_end), np.arange(w_start, T)]).astype(np.int64)


def _group_max(er_head, n_kv_heads):
    L, Hq = er_head.shape
    return er_head.reshape(L, n_kv_heads, Hq // n_kv_heads).max(axis=2)


MUTANTS = [
    (aoh, "effective_rank", _er_sigma_squared),
    (aoh, "proxy_eigenvalues", _proxy_without_congruence),
    (aoh, "group_scores", _group_max),
    (fasa, "fc_channels", _interleaved_pairing),
    (fasa, "attend", _attend_unscaled),
    (fasa, "top_n", _top_n_unstable),
    (fasa, "top_n", _top_n_lowest),
    (fasa, "group_query", _group_query_first_head),
    (fasa, "stream_rows", _window_off_by_one),
]


@pytest.mark.parametrize("mod,name,mutant", MUTANTS, ids=[f"{m.__name__}.{n}:{f.__name__}" for m, n, f in MUTANTS])
def test_pins_catch_mutant(monkeypatch, mod, name, mutant):
    assert not _any_pin_fails()  # the unmutated oracle passes every pin
    monkeypatch.setattr(mod, name, mutant)
    assert _any_pin_fails()
