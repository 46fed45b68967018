"""Pins the oracle's ordered skipping (orc_topk_margin).

CoSA summary (gist.science), the paragraphs on the Kernel-Aware Proxy and the
Ordered-Skipping Kernel: the proxy hands the kernel a priority list, and the
kernel reads the most important entries first and then skips the rest. The
page gives no stopping rule. Reading: the priority list is the top-k in
(score descending, position ascending) order, and reading stops at the first
entry whose score is below thr = (first score) - margin, with thr formed in
float32 because the scores are float32 values.

Pins: hand-worked cases (tests/golden/ordered_skip_hand.json, including one
where the float32 threshold and exact arithmetic disagree); an infinite or
huge margin reproduces the plain top-k; margin 0 keeps exactly the entries
tied with the row maximum (up to k, lowest positions first); on random rows
the kept set satisfies its defining conditions (inside the top-k, every kept
score at or above thr, every dropped top-k score below it); kept sets grow
with the margin; per-query counts compose with the margin; a decode step with
a margin attends over the margin index.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_cases():
    g = json.load(open(os.path.join(GOLD, "ordered_skip_hand.json")))
    for case in g["cases"]:
        s = np.array(case["scores"], np.float64)[None, None]
        idx, kept = oracle.topk_margin(s, case["k"], case["margin"])
        assert idx[0, 0].tolist() == case["idx"], case["why"]
        assert int(kept[0, 0]) == case["kept"], case["why"]


@pytest.mark.parametrize("margin", [float("inf"), 1e30])
def test_unbounded_margin_is_the_plain_top_k(margin):
    rng = np.random.default_rng(1)
    s = rng.standard_normal((2, 4, 300)).astype(np.float32).astype(np.float64)
    idx, kept = oracle.topk_margin(s, 40, margin)
    assert np.array_equal(idx, oracle.topk(s, 40))
    vis = 300 - 4 + np.arange(4) + 1
    assert np.array_equal(kept, np.broadcast_to(np.minimum(40, vis), (2, 4)))


def test_zero_margin_keeps_the_ties_of_the_maximum():
    rng = np.random.default_rng(2)
    s = rng.integers(0, 6, (3, 1, 200)).astype(np.float64)  # several entries equal the max
    for k in (1, 3, 50):
        idx, kept = oracle.topk_margin(s, k, 0.0)
        for b in range(3):
            ties = np.flatnonzero(s[b, 0] == s[b, 0].max())[:k]
            assert kept[b, 0] == ties.size
            assert idx[b, 0, :ties.size].tolist() == ties.tolist()
            assert np.all(idx[b, 0, ties.size:] == -1)


@pytest.mark.parametrize("seed,T,L,k", [(3, 1, 500, 64), (4, 6, 120, 40), (5, 3, 30, 64)])
def test_kept_set_meets_its_defining_conditions(seed, T, L, k):
    rng = np.random.default_rng(seed)
    B = 2
    s = (rng.standard_normal((B, T, L)) * 3).astype(np.float32).astype(np.float64)
    top = oracle.topk(s, k)
    for margin in (0.0, 0.25, 1.0, 4.0):
        idx, kept = oracle.topk_margin(s, k, margin)
        for b in range(B):
            for t in range(T):
                vis = L - T + t + 1
                topset = set(top[b, t][top[b, t] >= 0].tolist())
                keep = idx[b, t][idx[b, t] >= 0]
                assert keep.size == kept[b, t]
                assert np.all(idx[b, t][keep.size:] == -1) and np.all(np.diff(keep) > 0)
                thr = np.float32(np.float32(s[b, t, :vis].max()) - np.float32(margin))
                assert set(keep.tolist()) <= topset
                assert all(s[b, t, p] >= thr for p in keep)
                assert all(s[b, t, p] < thr for p in topset - set(keep.tolist()))


def test_kept_sets_grow_with_the_margin():
    rng = np.random.default_rng(6)
    s = rng.standard_normal((1, 1, 400)).astype(np.float32).astype(np.float64)
    prev, prev_n = set(), 0
    for margin in (0.0, 0.1, 0.3, 0.7, 1.5, 3.0, 10.0):
        idx, kept = oracle.topk_margin(s, 80, margin)
        cur = set(idx[0, 0][idx[0, 0] >= 0].tolist())
        assert prev <= cur and kept[0, 0] >= prev_n
        prev, prev_n = cur, kept[0, 0]
    assert prev_n == 80


def test_per_query_counts_compose_with_the_margin():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((2, 3, 150)).astype(np.float32).astype(np.float64)
    kr = np.array([[0, 5, 60], [1, 30, 12]], np.int32)
    idx, kept = oracle.topk_margin(s, 40, 1.0, k_rows=kr)
    base = oracle.topk(s, 40, k_rows=kr)
    for b in range(2):
        for t in range(3):
            n = kept[b, t]
            assert n <= min(max(kr[b, t], 0), 40)
            assert set(idx[b, t, :n].tolist()) <= set(base[b, t][base[b, t] >= 0].tolist())
    assert kept[0, 0] == 0 and np.all(idx[0, 0] == -1)


def test_negative_margin_is_rejected():
    with pytest.raises(ValueError):
        oracle.topk_margin(np.zeros((1, 1, 8)), 2, -1.0)


def test_decode_step_with_a_margin_attends_over_the_margin_index():
    rng = np.random.default_rng(9)
    B, T, L, Hq, Hkv, D, H, DI, k, n = 2, 3, 80, 4, 2, 16, 3, 8, 24, 2
    f32 = lambda a: np.ascontiguousarray(np.asarray(a, np.float32))
    K, V = f32(rng.standard_normal((B, L, Hkv, D))), f32(rng.standard_normal((B, L, Hkv, D)))
    q = [f32(rng.standard_normal((B, T, Hq, D))) for _ in range(n)]
    qi = [f32(rng.integers(-8, 9, (B, T, H, DI))), None]
    ki = [f32(rng.integers(-8, 9, (B, L, DI))), None]
    w = [f32(rng.integers(0, 17, (B, T, H)) / 16), None]
    outs, lses, idx, _ = oracle.decode_step([0, 0], q, [K, K], [V, V], oracle.F32, qi, ki, w, oracle.F32,
                                            kv_len=L, k=k, skip_margin=20.0)
    scores = oracle.index_score(qi[0], ki[0], oracle.F32, w[0], L)
    ref_idx, kept = oracle.topk_margin(scores, k, 20.0)
    assert np.array_equal(idx, ref_idx) and kept.min() < k  # the margin cuts some rows
    for l in range(n):
        ref_o, ref_l = oracle.sparse_attn(q[l], K, V, oracle.F32, idx, L)
        assert np.array_equal(outs[l], ref_o) and np.array_equal(lses[l], ref_l)
