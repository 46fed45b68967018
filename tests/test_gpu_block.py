"""GPU parity of the block-union comparator (CompactAttention summary,
"Méthodologie"): the union table must equal the oracle's bit for bit, and
dense attention over the table's blocks must match the float64 oracle."""

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


def _index(B, T, L, k, seed):
    s = inp.score_rows("gauss", B, T, L, seed, "cpu")
    return torch.from_numpy(oracle.topk(s.double().numpy(), k))


@pytest.mark.parametrize("B,T,L,k,block,Hkv", [
    (1, 16, 2000, 64, 64, 8),
    (2, 5, 777, 100, 16, 2),
    (1, 64, 4096, 256, 64, 8),
    (3, 1, 1000, 1000, 7, 1),      # every visible position selected
    (1, 32, 300, 500, 64, 4),      # k above the visible count: -1 padding
])
def test_block_union_table_matches_oracle(B, T, L, k, block, Hkv):
    announce("block_union", B, T, L, k, block, Hkv)
    idx = _index(B, T, L, k, 71)
    indptr, indices = clsa.block_union_build(idx.to(DEV), L, block, Hkv)
    torch.cuda.synchronize()
    r_ptr, r_ind = oracle.block_union(idx.numpy(), L, block, Hkv)
    assert np.array_equal(indptr.cpu().numpy(), r_ptr)
    assert np.array_equal(indices[: r_ptr[-1]].cpu().numpy(), r_ind)


@pytest.mark.parametrize("B,T,L,k,block,Hq,Hkv", [
    (1, 8, 1500, 64, 64, 32, 8),
    (2, 3, 700, 50, 16, 8, 2),
    (1, 4, 500, 500, 64, 8, 8),    # full union: dense causal attention
    (1, 40, 3000, 64, 64, 32, 8),  # two query tiles, ~45 KV tiles, a partial last block
    (2, 70, 1000, 20, 16, 16, 16), # G = 1, block 16, tiles spanning 4 blocks
    (1, 9, 2000, 30, 48, 64, 8),   # G = 8, block size not dividing the 64-position tile
])
def test_block_paged_attention_matches_oracle(B, T, L, k, block, Hq, Hkv):
    announce("block_paged_attn", B, T, L, k, block, Hq, Hkv)
    D = 128
    q = inp.randn((B, T, Hq, D), inp.BF16, 81, DEV)
    kc = inp.randn((B, L, Hkv, D), inp.BF16, 82, DEV)
    vc = inp.randn((B, L, Hkv, D), inp.BF16, 83, DEV)
    idx = _index(B, T, L, k, 84)
    indptr, indices = clsa.block_union_build(idx.to(DEV), L, block, Hkv)
    out, lse = clsa.block_paged_attn(q, kc, vc, indptr, indices, block, kv_len=L)
    torch.cuda.synchronize()
    r_ptr, r_ind = oracle.block_union(idx.numpy(), L, block, Hkv)
    ref_o, ref_l = oracle.block_attn(raw(q), raw(kc), raw(vc), inp.BF16, r_ptr, r_ind, block, L)
    check_out(out_f64(out), ref_o, TOL_OUT[inp.BF16])
    lse_close(lse.cpu().numpy(), ref_l, TOL_LSE[inp.BF16])


@pytest.mark.parametrize("B,T,L,k,block,Hq,Hkv", [
    (1, 8, 1500, 64, 64, 32, 8),
    (2, 70, 1000, 20, 16, 16, 16),
    (1, 9, 2000, 30, 48, 64, 8),
])
def test_block_paged_attention_head_major_matches_oracle(B, T, L, k, block, Hq, Hkv):
    """Head-major caches [B, Hkv, L, D] (CompactAttention summary,
    "Méthodologie": blocks read in place from the head-major layout)."""
    announce("block_paged_attn_hm", B, T, L, k, block, Hq, Hkv)
    D = 128
    q = inp.randn((B, T, Hq, D), inp.BF16, 91, DEV)
    kh = inp.randn((B, Hkv, L, D), inp.BF16, 92, DEV)
    vh = inp.randn((B, Hkv, L, D), inp.BF16, 93, DEV)
    idx = _index(B, T, L, k, 94)
    indptr, indices = clsa.block_union_build(idx.to(DEV), L, block, Hkv)
    out, lse = clsa.block_paged_attn(q, kh, vh, indptr, indices, block, kv_len=L, head_major=True)
    torch.cuda.synchronize()
    r_ptr, r_ind = oracle.block_union(idx.numpy(), L, block, Hkv)
    ref_o, ref_l = oracle.block_attn(raw(q), raw(kh), raw(vh), inp.BF16, r_ptr, r_ind, block, L, head_major=True)
    check_out(out_f64(out), ref_o, TOL_OUT[inp.BF16])
    lse_close(lse.cpu().numpy(), ref_l, TOL_LSE[inp.BF16])
