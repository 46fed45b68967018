"""Decode steps recorded in a HIP graph and replayed.

The step is deterministic, so every replay must reproduce the eager step
bit for bit. Between replays the test does eager work of its own and
synchronises: it overwrites the step's outputs and index buffer, and runs
an unrelated step through the allocation-free entry point, which rewrites
the library's per-GPU scratch. Both the workspace entry point and the
allocation-free one are recorded (the latter's callers include work recorded
under graph capture); neither records a memset node, since the step's
buffers are cleared by its own kernels.
"""

import pytest
import torch

import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import inputs as inp

from gpu_util import DEV, announce, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _state(st):
    return [t.clone() for t in st.out] + [t.clone() for t in (st.lse or [])] + [st.idx.clone()]


@pytest.mark.parametrize("static", [False, True])
def test_decode_step_graph_replays_match_eager(static):
    wl = inp.config("decode128k", B=2, kv_len=8192, layer_src=[0, 0, 0, 0])
    announce("decode step graph replay", "static scratch" if static else "workspace", wl.B, wl.kv_len)
    X = inp.make(wl, "int", seed=5, device=DEV)
    st = clsa.DecodeStep(wl.layer_src, X.q, X.k_cache, X.v_cache, X.q_idx, X.k_idx, X.w, wl.k,
                         kv_len=wl.kv_len)
    run = st.run_static if static else st.run
    run()
    torch.cuda.synchronize()
    ref = _state(st)

    # another step (other inputs and sizes) run eagerly between the replays
    wl2 = inp.config("decode128k", B=1, kv_len=5000, layer_src=[0, 0])
    X2 = inp.make(wl2, "int", seed=6, device=DEV)
    other = clsa.DecodeStep(wl2.layer_src, X2.q, X2.k_cache, X2.v_cache, X2.q_idx, X2.k_idx, X2.w, wl2.k,
                            kv_len=wl2.kv_len)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        run()

    for rep in range(4):
        for t in st.out:
            t.fill_(float("nan"))
        for t in st.lse or []:
            t.fill_(float("nan"))
        st.idx.fill_(-7)
        other.run_static()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(_state(st), ref):
            assert torch.equal(got, want), f"replay {rep}"
