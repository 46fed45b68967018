"""Pins the oracle's per-query k (the query-dependent k reading).

CLSA article, "Le coût : limites de compatibilité": k is fixed in the paper,
and letting the indexer layer adjust k is left as future work; "Ce que cela
signifie pour l'inférence sur longs contextes" names dynamic k as an open
question. Reading: each query (b, t) keeps its own count k_bt <= k of best
positions (the rule that picks k_bt is the caller's); the remaining slots of
its k-wide index row hold -1, and attention runs over the kept entries.

Pins: brute force per row (numpy lexsort on (score desc, position asc)) with
each row's own count; equal counts reproduce the fixed-k top-k; the kept set
for a smaller count is contained in the one for a larger count; counts are
clamped to [0, k]; a decode step with per-query counts equals attention over
each query's truncated index.
"""

import numpy as np
import pytest

import oracle


def _brute(row, vis, kk, k):
    order = np.lexsort((np.arange(vis), -row[:vis]))
    keep = np.sort(order[:min(kk, vis)])
    out = np.full(k, -1, np.int32)
    out[:keep.size] = keep
    return out


@pytest.mark.parametrize("seed,B,T,L,k", [(1, 3, 1, 200, 40), (2, 2, 5, 90, 30), (3, 1, 1, 64, 64)])
def test_per_row_counts_match_brute_force(seed, B, T, L, k):
    rng = np.random.default_rng(seed)
    s = rng.integers(-20, 21, (B, T, L)).astype(np.float64)  # many ties
    kr = rng.integers(-3, k + 5, (B, T)).astype(np.int32)    # includes <= 0 and > k
    got = oracle.topk(s, k, k_rows=kr)
    for b in range(B):
        for t in range(T):
            vis = L - T + t + 1
            kk = int(np.clip(kr[b, t], 0, k))
            assert np.array_equal(got[b, t], _brute(s[b, t], vis, kk, k))


def test_equal_counts_reproduce_fixed_k():
    rng = np.random.default_rng(4)
    s = rng.standard_normal((2, 3, 150))
    assert np.array_equal(oracle.topk(s, 25, k_rows=np.full((2, 3), 25, np.int32)), oracle.topk(s, 25))
    assert np.array_equal(oracle.topk(s, 25, k_rows=np.full((2, 3), 99, np.int32)), oracle.topk(s, 25))


def test_smaller_count_keeps_a_subset():
    rng = np.random.default_rng(5)
    s = rng.standard_normal((1, 1, 500))
    prev = set()
    for kk in range(0, 60, 7):
        cur = oracle.topk(s, 60, k_rows=np.array([[kk]], np.int32))[0, 0]
        kept = set(cur[cur >= 0].tolist())
        assert len(kept) == kk and prev <= kept and np.all(cur[kk:] == -1)
        prev = kept


def test_decode_step_attends_over_each_querys_kept_entries():
    rng = np.random.default_rng(9)
    B, T, L, Hq, Hkv, D, H, DI, k, n = 2, 3, 80, 4, 2, 16, 3, 8, 24, 2
    f32 = lambda a: np.ascontiguousarray(np.asarray(a, np.float32))
    K, V = f32(rng.standard_normal((B, L, Hkv, D))), f32(rng.standard_normal((B, L, Hkv, D)))
    q = [f32(rng.standard_normal((B, T, Hq, D))) for _ in range(n)]
    qi = [f32(rng.integers(-8, 9, (B, T, H, DI))), None]
    ki = [f32(rng.integers(-8, 9, (B, L, DI))), None]
    w = [f32(rng.integers(0, 17, (B, T, H)) / 16), None]
    kr = np.array([[0, 5, 24], [1, 30, 12]], np.int32)
    outs, lses, idx, _ = oracle.decode_step([0, 0], q, [K, K], [V, V], oracle.F32, qi, ki, w, oracle.F32,
                                            kv_len=L, k=k, k_rows=kr)
    scores = oracle.index_score(qi[0], ki[0], oracle.F32, w[0], L)
    assert np.array_equal(idx, oracle.topk(scores, k, k_rows=kr))
    for l in range(n):
        ref_o, ref_l = oracle.sparse_attn(q[l], K, V, oracle.F32, idx, L)
        assert np.array_equal(outs[l], ref_o) and np.array_equal(lses[l], ref_l)
    # Query (0, 0) keeps nothing: zero output, -inf lse.
    assert np.all(outs[0][0, 0] == 0) and np.all(np.isneginf(lses[0][0, 0]))
