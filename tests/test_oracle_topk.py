"""Pins the oracle's per-query top-k (step 2).

Definition followed: CLSA article, "Comment CLSA fonctionne" (keep the top-k
tokens of the indexer's scores); IndexCache summary, "1. Problématique" (the
k most relevant tokens per query). Readings: ties go to the lower position,
-0 equals +0, output ascending, -1 padding past the visible count.

Pins: hand-worked cases; brute force with numpy's lexsort on small rows
(Gaussian, heavy ties, signed zeros); k = 1 against numpy's argmax (first
occurrence); the order invariants of a correct selection; causal rows.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_cases():
    g = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    for case in g["cases"]:
        s = np.array(case["scores"], np.float64)[None, None]
        got = oracle.topk(s, case["k"])[0, 0].tolist()
        assert got == case["idx"], case["why"]


def _brute(row, k):
    # lexsort: last key is primary -> (-score) primary, position secondary
    pos = np.arange(len(row))
    order = np.lexsort((pos, -row))
    chosen = np.sort(order[:k])
    return np.concatenate([chosen, -np.ones(max(0, k - len(row)), np.int64)])


def _rows(kind, rng, n, L):
    if kind == "gauss":
        return rng.standard_normal((n, L))
    if kind == "ties":
        return rng.integers(0, 5, (n, L)).astype(np.float64)
    if kind == "zeros":
        return np.where(rng.random((n, L)) < 0.5, -0.0, 0.0)
    if kind == "relu":
        x = rng.standard_normal((n, L))
        return np.where(x > 0, x, np.where(rng.random((n, L)) < 0.5, -0.0, 0.0))
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["gauss", "ties", "zeros", "relu"])
@pytest.mark.parametrize("k", [1, 7, 64, 300])
def test_brute_force(kind, k):
    rng = np.random.default_rng(["gauss", "ties", "zeros", "relu"].index(kind) * 1000 + k)
    L = 257
    rows = _rows(kind, rng, 12, L)
    got = oracle.topk(rows.reshape(12, 1, L), k).reshape(12, k)   # T = 1: every position visible
    for r in range(12):
        assert np.array_equal(got[r], _brute(rows[r], k)[:k])


@pytest.mark.parametrize("kind", ["gauss", "ties", "relu"])
def test_k1_is_first_argmax(kind):
    rng = np.random.default_rng(11)
    rows = _rows(kind, rng, 20, 1000)
    got = oracle.topk(rows[:, None], 1)[:, 0, 0]
    assert np.array_equal(got, np.argmax(rows, axis=1))


def test_invariants_on_ties():
    rng = np.random.default_rng(12)
    L, k = 2000, 333
    rows = rng.integers(0, 6, (8, L)).astype(np.float64)
    got = oracle.topk(rows[:, None], k)[:, 0]
    for r in range(8):
        sel = got[r]
        assert np.all(np.diff(sel) > 0)                       # ascending, distinct
        mask = np.zeros(L, bool)
        mask[sel] = True
        assert rows[r][mask].min() >= rows[r][~mask].max()    # nothing better left out
        theta = rows[r][mask].min()
        eq = np.flatnonzero(rows[r] == theta)
        taken = np.flatnonzero(mask & (rows[r] == theta))
        assert np.array_equal(taken, eq[: len(taken)])        # lowest positions among ties


def test_k_at_least_visible_returns_all():
    rng = np.random.default_rng(13)
    rows = rng.standard_normal((1, 1, 50))
    got = oracle.topk(rows, 64)[0, 0]
    assert np.array_equal(got[:50], np.arange(50)) and np.all(got[50:] == -1)


def test_causal_rows_only_pick_visible_positions():
    rng = np.random.default_rng(14)
    T, L, k = 6, 40, 38
    rows = rng.standard_normal((1, T, L))
    rows[0, :, :] += np.arange(L)[None, :] * 10.0     # late positions score highest
    got = oracle.topk(rows, k)[0]
    for t in range(T):
        vis = L - T + t + 1
        valid = got[t][got[t] >= 0]
        assert valid.max() < vis
        assert len(valid) == min(k, vis)
        assert np.array_equal(valid, _brute(rows[0, t, :vis], k)[: len(valid)])
