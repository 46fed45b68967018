"""Pins the oracle's indexer score (step 1).

Definition followed: IndexCache summary, "1. Problématique" (the lightning
indexer scores every previous token of the cache); CLSA article, "Comment CLSA
fonctionne" (the shared indexer layer computes those scores once). Score
reading: sum over heads of w_h * ReLU(q_h . k_s); -inf where the query does
not see the position.

Pins: a hand-worked example; the one-head, unit-weight case against numpy's
dot product; linearity in w plus one-hot weights (which together fix the
whole formula); positive homogeneity in the keys; causal masking against a
truncated cache; exactness of the integer recipe.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def test_hand_example():
    g = json.load(open(os.path.join(GOLD, "index_score_hand.json")))
    q = _f32(g["q"])[None, None]            # [1,1,H=2,D=3]
    k = _f32(g["k"])[None]                  # [1,L=4,D=3]
    w = _f32(g["w"])[None, None]            # [1,1,2]
    s = oracle.index_score(q, k, oracle.F32, w, kv_len=4)
    assert np.array_equal(s[0, 0], np.array(g["scores"]))


def test_hand_example_causal_two_queries():
    g = json.load(open(os.path.join(GOLD, "index_score_hand.json")))
    q = np.ascontiguousarray(np.repeat(_f32(g["q"])[None, None], 2, axis=1))   # [1,2,2,3]
    w = np.ascontiguousarray(np.repeat(_f32(g["w"])[None, None], 2, axis=1))
    k = _f32(g["k"])[None]
    s = oracle.index_score(q, k, oracle.F32, w, kv_len=4)
    exp0 = [float(x) for x in g["causal_T2"]["scores_t0"]]
    assert np.array_equal(s[0, 0], np.array(exp0))
    assert np.array_equal(s[0, 1], np.array(g["causal_T2"]["scores_t1"], dtype=np.float64))


def test_one_head_unit_weight_is_relu_dot():
    rng = np.random.default_rng(1)
    q = _f32(rng.standard_normal((2, 1, 1, 16)))
    k = _f32(rng.standard_normal((2, 50, 16)))
    w = np.ones((2, 1, 1), np.float32)
    s = oracle.index_score(q, k, oracle.F32, w, kv_len=50)
    for b in range(2):
        ref = np.maximum(0.0, k[b].astype(np.float64) @ q[b, 0, 0].astype(np.float64))
        np.testing.assert_allclose(s[b, 0], ref, rtol=1e-13, atol=1e-13)


def test_linear_in_weights_and_onehot_heads():
    rng = np.random.default_rng(2)
    H, D, L = 5, 12, 40
    q = _f32(rng.integers(-8, 9, (1, 1, H, D)))
    k = _f32(rng.integers(-8, 9, (1, L, D)))
    per_head = []
    for h in range(H):
        w = np.zeros((1, 1, H), np.float32)
        w[0, 0, h] = 1.0
        sh = oracle.index_score(q, k, oracle.F32, w, kv_len=L)[0, 0]
        ref = np.maximum(0.0, k[0].astype(np.float64) @ q[0, 0, h].astype(np.float64))
        assert np.array_equal(sh, ref)
        per_head.append(sh)
    w = _f32(rng.integers(0, 17, (1, 1, H)) / 16.0)
    s = oracle.index_score(q, k, oracle.F32, w, kv_len=L)[0, 0]
    assert np.array_equal(s, sum(float(w[0, 0, h]) * per_head[h] for h in range(H)))


def test_positive_homogeneity_keeps_topk():
    rng = np.random.default_rng(3)
    q = _f32(rng.integers(-8, 9, (1, 1, 4, 16)))
    k = _f32(rng.integers(-8, 9, (1, 300, 16)))
    w = _f32(rng.integers(0, 257, (1, 1, 4)) / 256.0)
    s1 = oracle.index_score(q, k, oracle.F32, w, kv_len=300)
    s2 = oracle.index_score(q, _f32(4 * k), oracle.F32, w, kv_len=300)
    assert np.array_equal(s2, 4 * s1)
    assert np.array_equal(oracle.topk(s1, 20), oracle.topk(s2, 20))


def test_causal_rows_match_truncated_cache():
    rng = np.random.default_rng(4)
    B, T, H, D, L = 2, 5, 3, 8, 30
    q = _f32(rng.standard_normal((B, T, H, D)))
    k = _f32(rng.standard_normal((B, L + 7, D)))  # L_cap > kv_len
    w = _f32(rng.random((B, T, H)))
    s = oracle.index_score(q, k, oracle.F32, w, kv_len=L)
    for t in range(T):
        vis = L - T + t + 1
        assert np.all(np.isneginf(s[:, t, vis:]))
        one = oracle.index_score(np.ascontiguousarray(q[:, t:t + 1]), k, oracle.F32,
                                 np.ascontiguousarray(w[:, t:t + 1]), kv_len=vis)
        assert np.array_equal(s[:, t, :vis], one[:, 0])


@pytest.mark.parametrize("dt", [oracle.BF16, oracle.FP8_E4M3FN])
def test_low_precision_storage_decodes_to_the_same_integers(dt):
    import torch
    rng = np.random.default_rng(5)
    qi = rng.integers(-8, 9, (1, 2, 4, 32)).astype(np.float32)
    ki = rng.integers(-8, 9, (1, 64, 32)).astype(np.float32)
    w = _f32(rng.integers(0, 17, (1, 2, 4)) / 16.0)
    tdt = torch.bfloat16 if dt == oracle.BF16 else torch.float8_e4m3fn

    def raw(a):
        t = torch.from_numpy(a).to(tdt)
        return t.view(torch.int16).numpy().view(np.uint16) if dt == oracle.BF16 else t.view(torch.uint8).numpy()

    s_lo = oracle.index_score(raw(qi), raw(ki), dt, w, kv_len=64)
    s_32 = oracle.index_score(qi, ki, oracle.F32, w, kv_len=64)
    assert np.array_equal(s_lo, s_32)


def test_integer_recipe_is_exact_in_float32():
    # 64 heads x 128 dims, integers in [-8, 8], weights j/16: every score and
    # every partial sum fits 24 bits, so float32 evaluation in any order is exact.
    rng = np.random.default_rng(6)
    q = _f32(rng.integers(-8, 9, (1, 1, 64, 128)))
    k = _f32(rng.integers(-8, 9, (1, 256, 128)))
    w = _f32(rng.integers(0, 17, (1, 1, 64)) / 16.0)
    s, bound = oracle.index_score(q, k, oracle.F32, w, kv_len=256, with_bound=True)
    assert np.all(s * 16 == np.round(s * 16))
    assert bound.max() * 16 < 2 ** 24
