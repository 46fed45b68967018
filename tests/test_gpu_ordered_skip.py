"""GPU parity of ordered skipping (clsa_topk_margin and the decode step's
skip_margin; CoSA summary, the paragraphs on the Kernel-Aware Proxy and the
Ordered-Skipping Kernel). Each query's selection, read in priority order,
stops at the first entry more than the margin below its best score (the
threshold formed in float32 on both sides); the kept positions are written
ascending and the rest of the row is -1. Index rows and kept counts must
match the oracle exactly; attention outputs within the usual tolerances."""

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


def _margins(s, k):
    """Margins that cut row 0's selection at several depths: fractions of the
    gap between its best and its k-th best visible score, plus 0 and +inf."""
    row = np.sort(s[0, -1])[::-1]
    gap = float(row[0] - row[min(k, row.size) - 1])
    return [0.0, float(np.float32(0.3 * gap)), float(np.float32(0.8 * gap)), float(np.float32(1.5 * gap)),
            float("inf")]


@pytest.mark.parametrize("kind,B,T,L,k", [
    ("gauss", 4, 1, 131072, 2048),     # the 128K decode shape
    ("ties", 3, 1, 50000, 2048),       # huge tie classes; margin 0 keeps the max ties
    ("relu", 2, 1, 30000, 1000),       # exact zeros of both signs
    ("gauss", 1, 16, 6000, 1000),      # causal rows
    ("strided", 2, 1, 131072, 3000),   # full-row redo path
    ("desc", 2, 1, 40000, 2048),       # overflowing chunk path
    ("gauss", 2, 3, 700, 2048),        # k above the visible count
    ("ties", 2, 1, 8000, 1000),        # short rows: one launch, row in LDS
    ("gauss", 3, 2, 12000, 2048),
])
def test_topk_margin_matches_oracle(kind, B, T, L, k):
    s = inp.score_rows(kind, B, T, L, 71, DEV)
    s64 = s.double().cpu().numpy()
    for margin in _margins(s64, k):
        announce("topk_margin", kind, B, T, L, k, margin)
        idx, kept = clsa.topk_margin(s, k, margin)
        torch.cuda.synchronize()
        ref_idx, ref_kept = oracle.topk_margin(s64, k, margin)
        assert np.array_equal(kept.cpu().numpy(), ref_kept), margin
        assert np.array_equal(idx.cpu().numpy(), ref_idx), margin


def test_topk_margin_cuts_and_keeps():
    # The margins above do cut the 128K decode rows at several depths, and an
    # infinite margin is the plain top-k.
    s = inp.score_rows("gauss", 4, 1, 131072, 72, DEV)
    k = 2048
    ms = _margins(s.double().cpu().numpy(), k)
    counts = []
    for m in ms:
        announce("topk_margin depth", m)
        idx, kept = clsa.topk_margin(s, k, m)
        counts.append(int(kept[0, 0]))
    assert counts[0] == 1 and counts[1] < counts[2] < counts[3] == k == counts[4]
    plain = clsa.topk(s, k)
    idx, _ = clsa.topk_margin(s, k, float("inf"), want_kept=False)
    torch.cuda.synchronize()
    assert torch.equal(idx, plain)


def test_topk_margin_with_per_query_counts_matches_oracle():
    announce("topk_margin with k_per_query")
    B, T, L, k = 3, 4, 20000, 1500
    s = inp.score_rows("gauss", B, T, L, 73, DEV)
    s64 = s.double().cpu().numpy()
    kr = np.random.default_rng(74).integers(-2, k + 3, (B, T)).astype(np.int32)
    kr.flat[0] = 0
    for margin in (0.5, 1.5):
        idx, kept = clsa.topk_margin(s, k, margin, k_per_query=torch.from_numpy(kr).to(DEV))
        torch.cuda.synchronize()
        ref_idx, ref_kept = oracle.topk_margin(s64, k, margin, k_rows=kr)
        assert np.array_equal(idx.cpu().numpy(), ref_idx)
        assert np.array_equal(kept.cpu().numpy(), ref_kept)


def test_topk_margin_threshold_on_a_score_is_inclusive():
    # Integer scores with integer margins: thr = max - margin is itself a
    # score of the row, and entries equal to it are kept on both sides.
    s = inp.score_rows("ties", 3, 2, 30000, 75, DEV)  # integers 0..7
    s64 = s.double().cpu().numpy()
    for margin in (1.0, 2.0, 3.0):
        announce("topk_margin exact threshold", margin)
        idx, kept = clsa.topk_margin(s, 2048, margin)
        torch.cuda.synchronize()
        ref_idx, ref_kept = oracle.topk_margin(s64, 2048, margin)
        assert np.array_equal(idx.cpu().numpy(), ref_idx) and np.array_equal(kept.cpu().numpy(), ref_kept)


def test_decode_step_fp32_with_skip_margin_matches_oracle():
    # The fp32 attention kernel's per-row entry counts (tiny fp32 workload).
    announce("decode step fp32 with skip_margin")
    wl = inp.config("tiny")
    X = inp.make(wl, "int", seed=8, device=DEV)
    sc = oracle.index_score(raw(X.q_idx[0]), raw(X.k_idx[0]), wl.idx_dtype, raw(X.w[0]), wl.kv_len)
    margin = _margins(sc, wl.k)[2]
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len, skip_margin=margin)
    st.run()
    torch.cuda.synchronize()
    outs, lses, idx, _ = oracle.decode_step(
        wl.layer_src, [raw(t) for t in X.q], [raw(t) for t in X.k_cache], [raw(t) for t in X.v_cache],
        wl.dtype, [None if t is None else raw(t) for t in X.q_idx],
        [None if t is None else raw(t) for t in X.k_idx], [None if t is None else raw(t) for t in X.w],
        wl.idx_dtype, wl.kv_len, wl.k, skip_margin=margin)
    assert (idx >= 0).sum(-1).min() < wl.k
    assert np.array_equal(st.idx.cpu().numpy(), idx)
    for l in range(wl.n_layers):
        check_out(out_f64(st.out[l]), outs[l], TOL_OUT[wl.dtype], f"layer {l}")
        lse_close(st.lse[l].cpu().numpy(), lses[l], TOL_LSE[wl.dtype])


def test_topk_margin_rejects_negative_or_nan():
    s = torch.zeros((1, 1, 64), device=DEV)
    for bad in (-1.0, float("nan")):
        with pytest.raises(clsa.ClsaError):
            clsa.topk_margin(s, 8, bad)


def test_decode_step_with_skip_margin_matches_oracle():
    announce("decode step with skip_margin")
    wl = inp.config("decode128k", B=3, kv_len=12000, layer_src=[0, 0, 0])
    X = inp.make(wl, "int", seed=6, device=DEV)  # integer indexer inputs: exact scores
    # A margin that cuts: a fraction of batch element 0's gap between its
    # best and its k-th best score, taken from the oracle's scores.
    sc = oracle.index_score(raw(X.q_idx[0]), raw(X.k_idx[0]), wl.idx_dtype, raw(X.w[0]), wl.kv_len)
    margin = _margins(sc, wl.k)[2]
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len, skip_margin=margin)
    st.run()
    torch.cuda.synchronize()
    outs, lses, idx, _ = oracle.decode_step(
        wl.layer_src, [raw(t) for t in X.q], [raw(t) for t in X.k_cache], [raw(t) for t in X.v_cache],
        wl.dtype, [None if t is None else raw(t) for t in X.q_idx],
        [None if t is None else raw(t) for t in X.k_idx], [None if t is None else raw(t) for t in X.w],
        wl.idx_dtype, wl.kv_len, wl.k, skip_margin=margin)
    assert (idx >= 0).sum(-1).min() < wl.k  # the margin cuts at least one query
    assert np.array_equal(st.idx.cpu().numpy(), idx)
    for l in range(wl.n_layers):
        check_out(out_f64(st.out[l]), outs[l], TOL_OUT[wl.dtype], f"layer {l}")
        lse_close(st.lse[l].cpu().numpy(), lses[l], TOL_LSE[wl.dtype])
