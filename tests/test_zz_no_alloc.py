"""clsa_decode_step_static, the decode step on the library's own device
scratch (it allocates nothing), against clsa_decode_step with a caller
workspace. Both run the same kernels, so the index cache, every layer's
output and lse must agree bit for bit. Two calls in a row, the second with a
smaller step (and per-query counts, so the kept-count region of the scratch
is used too): the second call finds the first call's contents in the scratch
and must not depend on them."""

import pytest
import torch

import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import inputs as inp

from gpu_util import DEV, announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _agree(st):
    st.run_static()
    torch.cuda.synchronize()
    idx = st.idx.clone()
    outs = [o.clone() for o in st.out]
    lses = [l.clone() for l in st.lse]
    st.idx.fill_(-7)
    for o, l in zip(st.out, st.lse):
        o.fill_(0.5)
        l.fill_(0.5)
    st.run()  # the caller-workspace entry point
    torch.cuda.synchronize()
    assert torch.equal(idx, st.idx)
    for l in range(st.n):
        assert torch.equal(outs[l], st.out[l]), l
        assert torch.equal(lses[l], st.lse[l]), l


def test_static_step_matches_workspace_step_on_two_calls():
    # first call: the 128K-context decode's per-batch scratch at half the context
    wl = inp.config("decode128k", kv_len=65536, layer_src=[0] * 4)
    announce("decode_step_static 1", wl.name, wl.B, wl.kv_len, wl.n_layers)
    X = inp.make(wl, "gauss", seed=21, device=DEV)
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len)
    _agree(st)
    del st, X
    # second call, smaller: two F layers, per-query counts
    wl = inp.config("indexcache48", B=2, kv_len=9000, layer_src=[0, 0, 2, 2])
    announce("decode_step_static 2", wl.name, wl.B, wl.kv_len, wl.n_layers)
    X = inp.make(wl, "gauss", seed=22, device=DEV)
    kr = torch.tensor([[700], [2048]], dtype=torch.int32, device=DEV)
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len, k_per_query=kr)
    _agree(st)
    assert int((st.idx[0] >= 0).sum()) == 700


def test_static_step_rejects_a_step_above_its_scratch():
    # a 2048-query chunk needs about 1 GiB of scores: rejected before any launch
    wl = inp.config("prefill2k", T=2048, kv_len=131072 + 2048)
    announce("decode_step_static reject", wl.T, wl.kv_len)
    q = torch.zeros((1, wl.T, wl.Hq, wl.D), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((1, wl.kv_len, wl.Hkv, wl.D), dtype=torch.bfloat16, device=DEV)
    qi = torch.zeros((1, wl.T, wl.H_I, wl.D_I), dtype=torch.bfloat16, device=DEV)
    ki = torch.zeros((1, wl.kv_len, wl.D_I), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((1, wl.T, wl.H_I), dtype=torch.float32, device=DEV)
    st = clsa.DecodeStep([0], [q], [kc], [kc], [qi], [ki], [w], wl.k, kv_len=wl.kv_len)
    with pytest.raises(clsa.ClsaError) as e:
        st.run_static()
    assert e.value.status == -3 and "scratch" in str(e.value)
