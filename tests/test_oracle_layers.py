"""Pins the oracle's layer map (step 3) and block-union comparator (step 5).

Layer map: CLSA article, "Comment CLSA fonctionne" (one indexer pass serves
every following cross-decoder layer); IndexCache summary, "2. Méthodologie :
IndexCache" (F layers index and overwrite the cached indices, S layers reuse
the nearest F above them; a 1-in-4 pattern removes 75% of indexer work).

Block union: CompactAttention summary, "Méthodologie", selection step (union
over the chunk's queries and the group's heads; minimal and coverage
preserving) and execution step (dense attention over the listed blocks).

Pins: the page's 75% figure; all-F equals independent per-layer pipelines;
S layers equal attention with their F layer's index; invalid maps rejected;
a hand-worked union; coverage and minimality; block size 1 reduces to token
attention; the full union equals dense causal attention (torch, float64).
"""

import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def _layers(rng, n, layer_src, B=2, T=1, L=64, Hq=4, Hkv=2, D=16, H=3, DI=8, shared=True):
    K = [_f32(rng.standard_normal((B, L, Hkv, D)))]
    V = [_f32(rng.standard_normal((B, L, Hkv, D)))]
    if not shared:
        K += [_f32(rng.standard_normal((B, L, Hkv, D))) for _ in range(n - 1)]
        V += [_f32(rng.standard_normal((B, L, Hkv, D))) for _ in range(n - 1)]
    kc = [K[0 if shared else l] for l in range(n)]
    vc = [V[0 if shared else l] for l in range(n)]
    q = [_f32(rng.standard_normal((B, T, Hq, D))) for _ in range(n)]
    qi = [(_f32(rng.integers(-8, 9, (B, T, H, DI))) if layer_src[l] == l else None) for l in range(n)]
    ki = [(_f32(rng.integers(-8, 9, (B, L, DI))) if layer_src[l] == l else None) for l in range(n)]
    w = [(_f32(rng.integers(0, 17, (B, T, H)) / 16) if layer_src[l] == l else None) for l in range(n)]
    return q, kc, vc, qi, ki, w


def test_indexcache_pattern_removes_three_quarters_of_indexer_calls():
    g = json.load(open(os.path.join(GOLD, "indexcache_pattern.json")))
    n, every = g["n_layers"], g["every"]
    src = [every * (l // every) for l in range(n)]
    rng = np.random.default_rng(31)
    q, kc, vc, qi, ki, w = _layers(rng, n, src, B=1, L=16, Hq=2, Hkv=1, D=4, H=2, DI=4)
    _, _, _, calls = oracle.decode_step(src, q, kc, vc, oracle.F32, qi, ki, w, oracle.F32, kv_len=16, k=4)
    assert 1 - calls / n == g["indexer_fraction_removed"]


def test_all_full_layers_equal_independent_pipelines():
    rng = np.random.default_rng(32)
    n, L, k = 3, 64, 10
    src = list(range(n))
    q, kc, vc, qi, ki, w = _layers(rng, n, src, L=L, shared=False)
    outs, lses, _, calls = oracle.decode_step(src, q, kc, vc, oracle.F32, qi, ki, w, oracle.F32, L, k)
    assert calls == n
    for l in range(n):
        idx = oracle.topk(oracle.index_score(qi[l], ki[l], oracle.F32, w[l], L), k)
        o, s = oracle.sparse_attn(q[l], kc[l], vc[l], oracle.F32, idx, L)
        assert np.array_equal(o, outs[l]) and np.array_equal(s, lses[l])


def test_shared_layers_use_nearest_full_layer_index():
    rng = np.random.default_rng(33)
    src = [0, 0, 2, 2, 2, 5]
    n, L, k, T = len(src), 64, 12, 2
    q, kc, vc, qi, ki, w = _layers(rng, n, src, T=T, L=L, shared=False)
    outs, lses, idx_final, calls = oracle.decode_step(src, q, kc, vc, oracle.F32, qi, ki, w, oracle.F32,
                                                      L, k)
    assert calls == 3
    for l in range(n):
        f = src[l]
        idx = oracle.topk(oracle.index_score(qi[f], ki[f], oracle.F32, w[f], L), k)
        o, s = oracle.sparse_attn(q[l], kc[l], vc[l], oracle.F32, idx, L)
        assert np.array_equal(o, outs[l]) and np.array_equal(s, lses[l])
    assert np.array_equal(idx_final, oracle.topk(oracle.index_score(qi[5], ki[5], oracle.F32, w[5], L), k))


def test_identical_queries_in_sharing_layers_give_identical_outputs():
    rng = np.random.default_rng(34)
    src = [0, 0, 0, 0]
    q, kc, vc, qi, ki, w = _layers(rng, 4, src, L=48)
    q = [q[0]] * 4
    outs, lses, _, calls = oracle.decode_step(src, q, kc, vc, oracle.F32, qi, ki, w, oracle.F32, 48, 9)
    assert calls == 1
    for l in range(1, 4):
        assert np.array_equal(outs[l], outs[0]) and np.array_equal(lses[l], lses[0])


@pytest.mark.parametrize("src", [[1, 1], [0, 2, 2], [0, 0, 1], [0, 1, 0]])
def test_invalid_layer_maps_rejected(src):
    rng = np.random.default_rng(35)
    n = len(src)
    full = [l for l in range(n)]
    q, kc, vc, qi, ki, w = _layers(rng, n, full, L=16, H=2, DI=4)
    with pytest.raises(ValueError):
        oracle.decode_step(src, q, kc, vc, oracle.F32, qi, ki, w, oracle.F32, 16, 4)


def test_block_union_hand_example():
    g = json.load(open(os.path.join(GOLD, "block_union_hand.json")))
    idx = np.array(g["idx"], np.int32)
    indptr, indices = oracle.block_union(idx, g["kv_len"], g["block"], g["Hkv"])
    assert indptr.tolist() == g["kv_indptr"] and indices.tolist() == g["kv_indices"]


def test_block_union_coverage_and_minimality():
    rng = np.random.default_rng(36)
    B, T, k, L, blk, Hkv = 3, 16, 20, 500, 16, 2
    idx = rng.integers(-1, L, (B, T, k)).astype(np.int32)
    indptr, indices = oracle.block_union(idx, L, blk, Hkv)
    for b in range(B):
        hits = set()
        for t in range(T):
            vis = L - T + t + 1
            hits |= {int(s) // blk for s in idx[b, t] if 0 <= s < vis}
        for g_ in range(Hkv):
            tab = indices[indptr[b * Hkv + g_]:indptr[b * Hkv + g_ + 1]].tolist()
            assert tab == sorted(hits)          # covers every hit block, nothing else, ascending


def test_block_size_one_reduces_to_token_attention():
    rng = np.random.default_rng(37)
    B, Hq, Hkv, D, L, k = 2, 4, 2, 16, 80, 25
    q = _f32(rng.standard_normal((B, 1, Hq, D)))
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    idx = np.stack([np.sort(rng.choice(L, k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    indptr, indices = oracle.block_union(idx, L, 1, Hkv)
    a, la = oracle.block_attn(q, K, V, oracle.F32, indptr, indices, 1, L)
    b, lb = oracle.sparse_attn(q, K, V, oracle.F32, idx, L)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13, atol=1e-13)


def test_full_union_equals_dense_causal_attention():
    rng = np.random.default_rng(38)
    B, T, Hq, Hkv, D, L, blk = 1, 5, 4, 2, 16, 70, 8
    q = _f32(rng.standard_normal((B, T, Hq, D)))
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    idx = np.ascontiguousarray(np.broadcast_to(np.arange(L, dtype=np.int32), (B, T, L)))
    indptr, indices = oracle.block_union(idx, L, blk, Hkv)
    assert len(indices) == Hkv * math.ceil(L / blk)
    out, lse = oracle.block_attn(q, K, V, oracle.F32, indptr, indices, blk, L)
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(K.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, 1).contiguous()
    vt = torch.from_numpy(V.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, 1).contiguous()
    mask = torch.arange(L)[None, :] < (L - T + torch.arange(T) + 1)[:, None]
    ref = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_block_attention_head_major_layout_gives_the_same_result():
    """CompactAttention summary, "Méthodologie": the execution step reads the
    blocks in place from a head-major cache. The layout changes addresses
    only, so the oracle's result is bit-identical on the permuted cache."""
    rng = np.random.default_rng(77)
    B, T, L, Hq, Hkv, D, k, block = 2, 6, 90, 4, 2, 8, 10, 16
    q = _f32(rng.standard_normal((B, T, Hq, D)))
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    idx = oracle.topk(rng.standard_normal((B, T, L)), k)
    ptr, ind = oracle.block_union(idx, L, block, Hkv)
    o1, l1 = oracle.block_attn(q, K, V, oracle.F32, ptr, ind, block, L)
    Kh, Vh = (np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in (K, V))
    o2, l2 = oracle.block_attn(q, Kh, Vh, oracle.F32, ptr, ind, block, L, head_major=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # And a head-major cache read as if token-major gives a different answer.
    o3, _ = oracle.block_attn(q, np.ascontiguousarray(Kh.reshape(K.shape)),
                              np.ascontiguousarray(Vh.reshape(V.shape)), oracle.F32, ptr, ind, block, L)
    assert not np.allclose(o1, o3)
