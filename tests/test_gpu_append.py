"""GPU parity of clsa_cache_append (a new token's K, V and indexer-key rows
written into the shared caches; CLSA article, opening section and "Comment
CLSA fonctionne") against the oracle's byte copy, and of a decode step over
a cache whose newest rows were written by the append."""

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


@pytest.mark.parametrize("dt,idt,B,T,Hkv,D,DI,pos,cap", [
    (inp.BF16, inp.BF16, 4, 1, 8, 128, 128, 4095, 4096),   # decode: last row of the cache
    (inp.BF16, inp.FP8_E4M3FN, 3, 5, 8, 128, 128, 0, 300), # first rows, fp8 indexer keys (128-byte rows)
    (inp.F32, inp.F32, 2, 2, 1, 128, 3, 17, 64),           # 12-byte indexer rows: byte-copy path
    (inp.BF16, None, 2, 7, 2, 64, 0, 100, 200),            # no indexer keys
    (inp.F32, inp.BF16, 1, 33, 4, 5, 64, 31, 64),          # 20-element K/V rows (80 bytes)
])
def test_cache_append_matches_oracle(dt, idt, B, T, Hkv, D, DI, pos, cap):
    announce("cache_append", dt, idt, B, T, Hkv, D, DI, pos, cap)
    kc = inp.randn((B, cap, Hkv, D), dt, 11, DEV)
    vc = inp.randn((B, cap, Hkv, D), dt, 12, DEV)
    kn = inp.randn((B, T, Hkv, D), dt, 13, DEV)
    vn = inp.randn((B, T, Hkv, D), dt, 14, DEV)
    ki = kin = None
    if idt is not None:
        ki = inp.randint((B, cap, DI), -8, 8, idt, 15, DEV)
        kin = inp.randint((B, T, DI), -8, 8, idt, 16, DEV)
    ref = [oracle.cache_append(raw(kn), raw(kc), pos), oracle.cache_append(raw(vn), raw(vc), pos)]
    if idt is not None:
        ref.append(oracle.cache_append(raw(kin), raw(ki), pos))
    clsa.cache_append(kn, vn, kc, vc, pos, kin, ki)
    torch.cuda.synchronize()
    got = [raw(kc), raw(vc)] + ([raw(ki)] if idt is not None else [])
    for r, g in zip(ref, got):
        assert r.tobytes() == g.tobytes()


def test_decode_step_over_appended_token_matches_oracle():
    """Clear the newest row of a decode workload's caches, append it back as
    the new token, then run the step: index bit-exact (integer recipe) and
    attention within tolerance against the oracle on the original inputs."""
    announce("decode step after cache_append")
    wl = inp.config("decode128k", B=2, kv_len=8192, layer_src=[0] * 3)
    X = inp.make(wl, "int", seed=3, device=DEV)
    pos = wl.kv_len - 1
    kc, vc, ki = X.k_cache[0], X.v_cache[0], X.k_idx[0]
    kn, vn, kin = (t[:, pos:].clone() for t in (kc, vc, ki))
    ref = oracle.decode_step(wl.layer_src, [raw(t) for t in X.q], [raw(t) for t in X.k_cache],
                             [raw(t) for t in X.v_cache], wl.dtype,
                             [None if t is None else raw(t) for t in X.q_idx],
                             [None if t is None else raw(t) for t in X.k_idx],
                             [None if t is None else raw(t) for t in X.w], wl.idx_dtype, wl.kv_len, wl.k)
    for t in (kc, vc, ki):
        t[:, pos:] = 0
    clsa.cache_append(kn, vn, kc, vc, pos, kin, ki)
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len)
    st.run()
    torch.cuda.synchronize()
    outs, lses, idx, _ = ref
    assert np.array_equal(st.idx.cpu().numpy(), idx)
    for l in range(wl.n_layers):
        check_out(out_f64(st.out[l]), outs[l], TOL_OUT[wl.dtype], f"layer {l}")
        lse_close(st.lse[l].cpu().numpy(), lses[l], TOL_LSE[wl.dtype])
