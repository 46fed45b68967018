"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

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
