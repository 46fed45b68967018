"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

import os
import sys

import numpy as np
import pytest
import torch

import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import inputs as inp

DEV = "cuda"

# Tolerances of the attention outputs against the float64 oracle (max-abs),
# and of lse (float32 accumulation, |lse| of order 10).
TOL_OUT = {inp.F32: 1e-4, inp.BF16: 2e-2}
TOL_LSE = {inp.F32: 1e-4, inp.BF16: 1e-3}


def announce(*what):
    """Name the case on stderr before its GPU work starts."""
    print("[gpu-case]", *what, file=sys.stderr, flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test selected but no HIP device is visible")
    clsa.load()


def raw(t):
    return inp.raw(t)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0


# Largest observed max-abs output error per test (and its tolerance); the
# session summary in conftest.py prints them, so the margins are visible.
OBSERVED = {}


def check_out(got, ref, tol, what=""):
    """Asserts max|got - ref| <= tol and records the observed error."""
    err = max_abs(got, ref)
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    if test not in OBSERVED or err > OBSERVED[test][0]:
        OBSERVED[test] = (err, tol)
    assert err <= tol, f"{what}: max-abs error {err:.4g} above {tol}"


def lse_close(gpu, ref, tol):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    inf_g, inf_r = np.isneginf(gpu), np.isneginf(ref)
    assert np.array_equal(inf_g, inf_r), "lse -inf pattern differs"
    if (~inf_r).any():
        assert max_abs(gpu[~inf_r], ref[~inf_r]) <= tol


def out_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def idx_from_scores(scores, k):
    """A valid index (ascending distinct positions, -1 padding) drawn from seeded scores."""
    import oracle
    return torch.from_numpy(oracle.topk(scores.double().cpu().numpy(), k))


# ---------------------------------------------------------------------------
# The oracle over many queries: independent (batch element, query range)
# pieces on several host threads (the ctypes calls release the GIL). A piece
# of queries [t0, t1) of a T-query call is a call with T' = t1 - t0 queries
# over the first kv_len - T + t1 positions, which keeps every query's own
# visible range [0, kv_len - T + t].
# ---------------------------------------------------------------------------

N_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _pieces(B, T, n):
    step = max(1, -(-T // max(1, n // B)))
    return [(b, t0, min(T, t0 + step)) for b in range(B) for t0 in range(0, T, step)]


def _parallel(fn, pieces):
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    oracle.decode(np.zeros(1, np.uint16), 1)  # fills the oracle's decode tables once, here
    with ThreadPoolExecutor(N_THREADS) as ex:
        for _ in ex.map(fn, pieces):
            pass


def oracle_topk_rows(scores, k):
    """oracle.topk of float scores [B, T, kv_len] (causal rows), piecewise."""
    import oracle
    s = np.asarray(scores)
    B, T, L = s.shape
    out = np.empty((B, T, k), np.int32)

    def one(p):
        b, t0, t1 = p
        out[b:b + 1, t0:t1] = oracle.topk(np.ascontiguousarray(s[b:b + 1, t0:t1, :L - T + t1], np.float64), k)

    _parallel(one, _pieces(B, T, 8 * N_THREADS))
    return out


def oracle_attn_rows(q, kc, vc, dt, idx, kv_len):
    """oracle.sparse_attn on host copies (raw bits), piecewise over queries."""
    import oracle
    B, T, Hq, D = q.shape
    out = np.empty((B, T, Hq, D), np.float64)
    lse = np.empty((B, T, Hq), np.float64)

    def one(p):
        b, t0, t1 = p
        o, l = oracle.sparse_attn(q[b:b + 1, t0:t1], kc[b:b + 1], vc[b:b + 1], dt, idx[b:b + 1, t0:t1],
                                  kv_len - T + t1)
        out[b:b + 1, t0:t1], lse[b:b + 1, t0:t1] = o, l

    _parallel(one, _pieces(B, T, 4 * N_THREADS))
    return out, lse


def oracle_index_rows(q, k, dt, w, kv_len, with_bound=False):
    """oracle.index_score on host copies (raw bits), piecewise over queries."""
    import oracle
    B, T = q.shape[:2]
    s = np.empty((B, T, kv_len), np.float64)
    bnd = np.empty((B, T, kv_len), np.float64) if with_bound else None

    def one(p):
        b, t0, t1 = p
        L1 = kv_len - T + t1
        r = oracle.index_score(q[b:b + 1, t0:t1], k[b:b + 1], dt, w[b:b + 1, t0:t1], L1, with_bound=with_bound)
        sc, bd = r if with_bound else (r, None)
        s[b:b + 1, t0:t1, :L1] = sc
        s[b:b + 1, t0:t1, L1:] = -np.inf
        if with_bound:
            bnd[b:b + 1, t0:t1, :L1] = bd
            bnd[b:b + 1, t0:t1, L1:] = 0.0

    _parallel(one, _pieces(B, T, 4 * N_THREADS))
    return (s, bnd) if with_bound else s
