"""Pins the oracle's gathered sparse attention (step 4).

Definition followed: IndexCache summary, "1. Problématique" (main attention
over the k selected tokens); CompactAttention summary, "Méthodologie" (query
heads grouped onto shared KV heads). Readings: softmax scale 1/sqrt(D) by
default, contiguous GQA groups, entries outside the visible range skipped.

Pins: a hand-worked example; k = L (every position selected) against torch's
scaled_dot_product_attention in float64 on CPU, with GQA and causal rows;
lse against torch.logsumexp; k = 1 returns the V row exactly; equal K rows
give the mean of the selected V rows (repeats counted); permuting the index
changes nothing; no valid entry gives zeros and -inf.
"""

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


def test_hand_example():
    g = json.load(open(os.path.join(GOLD, "attention_hand.json")))
    L, D = 6, 2
    K = np.zeros((1, L, 1, D), np.float32)
    V = np.zeros((1, L, 1, D), np.float32)
    for s, row in g["k_rows"].items():
        K[0, int(s), 0] = row
    for s, row in g["v_rows"].items():
        V[0, int(s), 0] = row
    q = _f32(g["q"]).reshape(1, 1, 1, D)
    idx = np.array(g["idx"], np.int32).reshape(1, 1, -1)
    out, lse = oracle.sparse_attn(q, K, V, oracle.F32, idx, kv_len=L, scale=1.0)
    np.testing.assert_allclose(out[0, 0, 0], g["out"], rtol=1e-6, atol=1e-6)
    assert abs(lse[0, 0, 0] - g["lse"]) < 1e-6


def _dense_reference(q, K, V, T, kv_len, scale):
    """torch SDPA in float64 with GQA expansion and bottom-right causal rows."""
    B, _, Hq, D = q.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)                 # [B,Hq,T,D]
    kt = torch.from_numpy(K[:, :kv_len].astype(np.float64)).permute(0, 2, 1, 3)     # [B,Hkv,L,D]
    vt = torch.from_numpy(V[:, :kv_len].astype(np.float64)).permute(0, 2, 1, 3)
    kt = kt.repeat_interleave(G, dim=1).contiguous()
    vt = vt.repeat_interleave(G, dim=1).contiguous()
    pos = torch.arange(kv_len)
    vis = kv_len - T + torch.arange(T) + 1
    mask = pos[None, :] < vis[:, None]                                               # [T,L]
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = (qt @ kt.transpose(-1, -2)) * scale
    logits = logits.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return out.permute(0, 2, 1, 3).numpy(), lse.permute(0, 2, 1).numpy()


def test_all_positions_selected_equals_dense_attention():
    rng = np.random.default_rng(21)
    B, T, Hq, Hkv, D, L = 2, 3, 8, 2, 16, 37
    q = _f32(rng.standard_normal((B, T, Hq, D)))
    K = _f32(rng.standard_normal((B, L + 3, Hkv, D)))
    V = _f32(rng.standard_normal((B, L + 3, Hkv, D)))
    idx = np.ascontiguousarray(np.broadcast_to(np.arange(L, dtype=np.int32), (B, T, L)))
    out, lse = oracle.sparse_attn(q, K, V, oracle.F32, idx, kv_len=L)
    ref_out, ref_lse = _dense_reference(q, K, V, T, L, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_bf16_storage_matches_dense_on_decoded_values():
    rng = np.random.default_rng(22)
    B, T, Hq, Hkv, D, L = 1, 1, 4, 1, 128, 50
    qt = torch.from_numpy(rng.standard_normal((B, T, Hq, D)).astype(np.float32)).bfloat16()
    Kt = torch.from_numpy(rng.standard_normal((B, L, Hkv, D)).astype(np.float32)).bfloat16()
    Vt = torch.from_numpy(rng.standard_normal((B, L, Hkv, D)).astype(np.float32)).bfloat16()
    raw = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    idx = np.arange(L, dtype=np.int32).reshape(1, 1, L)
    out, lse = oracle.sparse_attn(raw(qt), raw(Kt), raw(Vt), oracle.BF16, idx, kv_len=L)
    ref_out, ref_lse = _dense_reference(qt.float().numpy(), Kt.float().numpy(), Vt.float().numpy(),
                                        T, L, 1.0 / math.sqrt(D))
    np.testing.assert_allclose(out, ref_out, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_single_entry_returns_that_value_row():
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D, L = 2, 4, 2, 8, 20
    q = _f32(rng.standard_normal((B, 1, Hq, D)))
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    idx = np.array([[[7]], [[13]]], np.int32)
    out, _ = oracle.sparse_attn(q, K, V, oracle.F32, idx, kv_len=L)
    for b, s in ((0, 7), (1, 13)):
        for h in range(Hq):
            assert np.array_equal(out[b, 0, h], V[b, s, h // 2].astype(np.float64))


def test_equal_keys_give_mean_of_values_with_repeats():
    rng = np.random.default_rng(24)
    D, L = 8, 30
    q = _f32(rng.standard_normal((1, 1, 1, D)))
    K = np.ascontiguousarray(np.broadcast_to(_f32(rng.standard_normal(D)), (1, L, 1, D)))
    V = _f32(rng.standard_normal((1, L, 1, D)))
    sel = [3, 3, 10, 29, -1, 5]
    idx = np.array(sel, np.int32).reshape(1, 1, -1)
    out, _ = oracle.sparse_attn(q, K, V, oracle.F32, idx, kv_len=L)
    valid = [s for s in sel if s >= 0]
    ref = V[0, valid, 0].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0, 0, 0], ref, rtol=1e-13, atol=1e-13)


def test_index_order_does_not_matter():
    rng = np.random.default_rng(25)
    B, Hq, Hkv, D, L, k = 1, 8, 2, 32, 100, 40
    q = _f32(rng.standard_normal((B, 1, Hq, D)))
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    idx = rng.choice(L, k, replace=False).astype(np.int32).reshape(1, 1, k)
    perm = np.ascontiguousarray(idx[:, :, rng.permutation(k)])
    a, la = oracle.sparse_attn(q, K, V, oracle.F32, np.sort(idx, axis=-1), kv_len=L)
    b, lb = oracle.sparse_attn(q, K, V, oracle.F32, perm, kv_len=L)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-13, atol=1e-13)


def test_no_valid_entry_gives_zero_and_neg_inf():
    q = np.ones((1, 2, 2, 4), np.float32)
    K = np.ones((1, 10, 1, 4), np.float32)
    V = np.ones((1, 10, 1, 4), np.float32)
    # T=2, kv_len=10: query 0 sees 0..8, so position 9 is invalid for it only.
    idx = np.array([[[-1, 9, 11], [9, -1, -5]]], np.int32)
    out, lse = oracle.sparse_attn(q, K, V, oracle.F32, idx, kv_len=10)
    assert np.all(out[0, 0] == 0) and np.all(np.isneginf(lse[0, 0]))
    assert np.all(out[0, 1] == 1) and np.all(lse[0, 1] == 0.5 * 4)  # one entry: lse = z = 4/sqrt(4)
