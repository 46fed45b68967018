"""GPU parity of the per-query k (clsa_topk_vark and the decode step's
k_per_query; CLSA article, "Le coût : limites de compatibilité": the
indexer layer adjusting k is the paper's open extension). Each query keeps
its own count of best positions; the rest of its row holds -1, and attention
runs over the kept entries."""

import numpy as np
import pytest
import torch

import oracle
import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import inputs as inp

from gpu_util import DEV, TOL_LSE, TOL_OUT, announce, check_out, lse_close, max_abs, out_f64, raw, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _counts(B, T, k, seed):
    g = np.random.default_rng(seed)
    c = g.integers(-2, k + 3, (B, T)).astype(np.int32)   # includes <= 0 and > k (clamped)
    c.flat[0] = k
    if c.size > 1:
        c.flat[1] = 1
    return c


@pytest.mark.parametrize("kind,B,T,L,k", [
    ("gauss", 4, 1, 131072, 2048),
    ("ties", 3, 1, 50000, 2048),
    ("gauss", 1, 16, 6000, 1000),      # causal rows
    ("strided", 2, 1, 131072, 3000),   # full-row redo path
    ("desc", 2, 1, 40000, 2048),       # overflowing chunk path
    ("gauss", 2, 1, 700, 2048),        # k above the visible count
])
def test_topk_per_query_counts_match_oracle(kind, B, T, L, k):
    announce("topk_vark", kind, B, T, L, k)
    s = inp.score_rows(kind, B, T, L, 61, DEV)
    kr = _counts(B, T, k, 62)
    got = clsa.topk(s, k, k_per_query=torch.from_numpy(kr).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.topk(s.double().cpu().numpy(), k, k_rows=kr)
    assert np.array_equal(got.cpu().numpy(), ref)


def test_decode_step_with_per_query_counts_matches_oracle():
    announce("decode step with k_per_query")
    wl = inp.config("decode128k", B=3, kv_len=12000, layer_src=[0, 0, 0])
    X = inp.make(wl, "int", seed=5, device=DEV)
    kr = np.array([[2048], [300], [1]], np.int32)
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len, k_per_query=torch.from_numpy(kr).to(DEV))
    st.run()
    torch.cuda.synchronize()
    outs, lses, idx, _ = oracle.decode_step(
        wl.layer_src, [raw(t) for t in X.q], [raw(t) for t in X.k_cache], [raw(t) for t in X.v_cache],
        wl.dtype, [None if t is None else raw(t) for t in X.q_idx],
        [None if t is None else raw(t) for t in X.k_idx], [None if t is None else raw(t) for t in X.w],
        wl.idx_dtype, wl.kv_len, wl.k, k_rows=kr)
    assert np.array_equal(st.idx.cpu().numpy(), idx)
    assert np.all(idx[1, 0, 300:] == -1) and np.all(idx[2, 0, 1:] == -1)
    for l in range(wl.n_layers):
        check_out(out_f64(st.out[l]), outs[l], TOL_OUT[wl.dtype], f"layer {l}")
        lse_close(st.lse[l].cpu().numpy(), lses[l], TOL_LSE[wl.dtype])
