"""Plant plausible mistakes in the DSA oracle (CPU only) and check that its
pins catch every one of them."""
import numpy as np
import pytest

import oracle.dsa as dsa
import tests.test_oracle_dsa_pins as pins
from tests.conftest import load_golden

_orig = {n: getattr(dsa, n) for n in ("indexer_scores", "topk_select", "sparse_decode",
                                       "gather_positions", "gather_index_keys", "pair_count")}


def _no_relu(q, w, K):
    return (np.asarray(K, float) @ np.asarray(q, float).T) @ np.asarray(w, float)


def _relu_after_sum(q, w, K):
    return np.maximum(_no_relu(q, w, K), 0.0)


def _no_weights(q, w, K):
    return _orig["indexer_scores"](q, np.ones_like(np.asarray(w, float)), K)


def _softmax_over_candidates(q, w, K):
    s = np.asarray(K, float) @ np.asarray(q, float).T
    if s.shape[0] == 0:
        return np.zeros(0)
    e = np.exp(s - s.max(axis=0, keepdims=True))
    return (e / e.sum(axis=0, keepdims=True)) @ np.asarray(w, float)


def _topk_lowest(scores, k):
    return _orig["topk_select"](-np.asarray(scores, float), k)


def _topk_ties_late(scores, k):
    s = np.asarray(scores, float)
    T = s.shape[0]
    if T <= k:
        return np.arange(T)
    order = np.lexsort((-np.arange(T), -s))
    return np.sort(order[:k])


def _topk_one_short(scores, k):
    return _orig["topk_select"](scores, max(k - 1, 0))


def _topk_recent_window(scores, k):
    T = np.asarray(scores).shape[0]
    return np.arange(max(0, T - k), T)


def _sparse_ignores_selection(q, c_kv, c_kv_scale, k_rope, block_table, selections, *a, **kw):
    full = [np.arange(int(np.max(s)) + 1) if len(s) else np.arange(0) for s in selections]
    return _orig["sparse_decode"](q, c_kv, c_kv_scale, k_rope, block_table, full, *a, **kw)


def _gather_slot_shift(c_kv, k_rope, c_kv_scale, block_table, positions, b, page_size, *a):
    pos = np.asarray(positions)
    shifted = np.where(pos % page_size == page_size - 1, pos, pos + 1)
    return _orig["gather_positions"](c_kv, k_rope, c_kv_scale, block_table, shifted, b,
                                     page_size, *a)


def _index_keys_no_scale(k_I_pool, k_I_scale, block_table, seq_len, b, page_size):
    return _orig["gather_index_keys"](k_I_pool, np.ones_like(k_I_scale), block_table, seq_len,
                                      b, page_size)


def _pairs_dense_off_by_one(L, k, sparse):
    return _orig["pair_count"](L, k, sparse) if sparse else L * (L - 1) // 2


MUTANTS = {
    "indexer without ReLU": ("indexer_scores", _no_relu),
    "ReLU after the head sum": ("indexer_scores", _relu_after_sum),
    "head weights ignored": ("indexer_scores", _no_weights),
    "softmax over candidates": ("indexer_scores", _softmax_over_candidates),
    "top-k keeps the lowest": ("topk_select", _topk_lowest),
    "ties to the later position": ("topk_select", _topk_ties_late),
    "one position short": ("topk_select", _topk_one_short),
    "recency window instead of scores": ("topk_select", _topk_recent_window),
    "sparse decode ignores the selection": ("sparse_decode", _sparse_ignores_selection),
    "selected slot off by one": ("gather_positions", _gather_slot_shift),
    "index keys without their scale": ("gather_index_keys", _index_keys_no_scale),
    "dense pair count off by one": ("pair_count", _pairs_dense_off_by_one),
}


def _run_pins():
    failed = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        argnames, cases = [], [()]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            cases = [c if isinstance(c, tuple) else (c,) for c in params[0].args[1]]
        for case in cases:
            kw = dict(zip(argnames, case))
            if "golden" in fn.__code__.co_varnames[: fn.__code__.co_argcount]:
                kw["golden"] = load_golden
            try:
                with np.errstate(all="ignore"):
                    fn(**kw)
            except Exception:
                failed.append(name)
                break
    return failed


def test_dsa_pins_pass_unmutated():
    assert _run_pins() == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_dsa_pins_catch(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(dsa, attr, fn)
    if hasattr(pins, attr):
        monkeypatch.setattr(pins, attr, fn)
    assert _run_pins(), f"no pin caught: {mutant}"
