"""GPU parity of each kernel on its own, through the C ABI, against the oracle.

Inputs are seeded and synthetic (token_sparse_attention_clsa_amd.inputs); the
oracle receives the exact bits the device saw. Sizes span several tiles and
ragged tails while the oracle still finishes in seconds.
Bars: indexer scores bit-exact on the integer recipe (float32 sums of
integers below 2**24 are exact in any order) and within the float32 rounding
bound on Gaussian inputs; top-k index sets bit-exact; attention within
1e-4 (fp32) / 2e-2 (bf16) max-abs of the float64 oracle fed the same index.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import token_sparse_attention_clsa_amd as clsa
from token_sparse_attention_clsa_amd import inputs as inp

from gpu_util import (DEV, TOL_LSE, TOL_OUT, announce, check_out, lse_close, oracle_attn_rows, oracle_topk_rows,
                      out_f64, raw, require_gpu)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---------------------------------------------------------------------------
# indexer score
# ---------------------------------------------------------------------------

IDX_CASES = [
    # dtype, B, T, H_I, D_I, kv_len, L_cap, weight bits
    (inp.F32, 1, 1, 4, 64, 4096, 4096, 8),
    (inp.F32, 2, 3, 3, 40, 517, 530, 8),
    (inp.BF16, 2, 1, 64, 128, 4097, 4100, 4),
    (inp.BF16, 1, 3, 16, 64, 1000, 1000, 4),
    (inp.BF16, 3, 2, 48, 128, 3001, 3001, 4),
    (inp.BF16, 1, 5, 32, 128, 70, 80, 4),
    (inp.FP8_E4M3FN, 2, 1, 64, 128, 5000, 5000, 4),
    (inp.FP8_E4M3FN, 1, 2, 32, 64, 777, 800, 4),
    # T >= 8: the multi-query (LDS-tiled) form
    (inp.BF16, 1, 8, 64, 128, 3000, 3000, 4),
    (inp.BF16, 2, 19, 32, 64, 1000, 1100, 4),    # a partial group of queries
    (inp.FP8_E4M3FN, 1, 16, 64, 128, 2049, 2049, 4),
    (inp.FP8_E4M3FN, 2, 9, 48, 64, 600, 640, 4),
    (inp.BF16, 1, 64, 16, 128, 700, 700, 4),     # kv_len close to T: short visible rows
    (inp.BF16, 1, 40, 64, 128, 40, 40, 4),       # T == kv_len: query 0 sees one key
    (inp.BF16, 2, 12, 32, 128, 1500, 1600, 4),   # multi-query form, 32 heads, L_cap > kv_len
    (inp.BF16, 1, 9, 64, 128, 1100, 1100, 4),    # multi-query form, 64 heads, a partial group of queries
]


@pytest.mark.parametrize("dt,B,T,H,DI,L,cap,m", IDX_CASES)
def test_index_score_integer_inputs_bit_exact(dt, B, T, H, DI, L, cap, m):
    announce("index_score int", inp.DTYPE_NAME[dt], B, T, H, DI, L, cap)
    q = inp.randint((B, T, H, DI), -8, 8, dt, 11, DEV)
    k = inp.randint((B, cap, DI), -8, 8, dt, 12, DEV)
    w = inp.weights((B, T, H), "int", 13, DEV, bits=m)
    s = clsa.index_score(q, k, w, kv_len=L)
    torch.cuda.synchronize()
    ref = oracle.index_score(raw(q), raw(k), dt, raw(w), L)
    assert np.array_equal(s.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("dt,T", [(inp.BF16, 2), (inp.FP8_E4M3FN, 2), (inp.BF16, 16), (inp.FP8_E4M3FN, 16)])
def test_index_score_gaussian_within_float32_bound(dt, T):
    # T = 2: the decode form; T = 16: the multi-query (LDS-tiled) form
    B, H, DI, L = 2, 64, 128, 3000
    announce("index_score gauss", inp.DTYPE_NAME[dt], B, T, H, DI, L)
    q = inp.randn((B, T, H, DI), dt, 21, DEV)
    k = inp.randn((B, L, DI), dt, 22, DEV)
    w = inp.weights((B, T, H), "gauss", 23, DEV)
    s = clsa.index_score(q, k, w, kv_len=L)
    torch.cuda.synchronize()
    ref, bound = oracle.index_score(raw(q), raw(k), dt, raw(w), L, with_bound=True)
    got = s.cpu().numpy().astype(np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(got), ~fin)
    # float32 dot of <= 128 exact products plus a 64-term head sum: |err| <= 2^-16 * bound
    assert np.all(np.abs(got[fin] - ref[fin]) <= 2.0 ** -16 * bound[fin] + 1e-30)


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------

TOPK_CASES = [
    # kind, B, T, kv_len, k
    ("gauss", 2, 1, 4096, 256),
    ("gauss", 1, 1, 131072, 2048),
    ("gauss", 3, 1, 40000, 2048),
    ("needle", 4, 1, 65536, 2048),
    ("ties", 2, 1, 50000, 2048),       # 8 distinct values: giant tie classes
    ("relu", 2, 1, 30000, 1000),       # half exact zeros with mixed signs
    ("zeros", 1, 1, 20000, 777),       # all zeros (+0/-0 mixed): lowest positions
    ("const", 1, 1, 40000, 2048),      # every candidate tied: global fallback path
    ("desc", 1, 1, 9000, 100),
    ("wide", 2, 1, 12345, 333),
    ("gauss", 1, 1, 1000, 1),
    ("gauss", 1, 1, 1000, 1000),       # k == visible
    ("gauss", 2, 1, 700, 2048),        # k > visible: -1 padding
    ("gauss", 1, 6, 5000, 4997),       # causal rows: 2 with fewer than k visible, 1 with exactly k
    ("ties", 1, 64, 8192, 512),        # many causal rows
    ("gauss", 1, 1, 4097, 4096),
    ("strided", 1, 1, 131072, 3000),   # 2048 tied high positions, then Gaussian ones
    ("strided", 2, 1, 131072, 1000),
    ("sampled", 1, 1, 131072, 3000),   # the filter's sample sees only the high positions: full-row redo
    ("sampled", 1, 1, 50001, 1000),
    ("needle", 2, 1, 131073, 2048),    # misaligned second row
    ("desc", 1, 1, 40000, 2048),       # the top k fill one 4096-chunk: its candidate segment overflows
    # Short rows: one launch with the row in LDS (kv_len <= 8192, or <= 16384 with 8k >= kv_len).
    ("ties", 3, 1, 8192, 700),         # giant tie classes
    ("zeros", 2, 1, 8000, 300),        # all zeros, mixed signs
    ("const", 1, 1, 6000, 2000),       # every key tied
    ("relu", 2, 2, 7000, 999),         # causal rows, half exact zeros
    ("needle", 4, 1, 8191, 64),        # odd length: rows after the first are misaligned
    ("wide", 2, 1, 5000, 17),
    ("desc", 1, 1, 8192, 2048),
    ("sampled", 1, 1, 8192, 1000),
    ("gauss", 2, 1, 12000, 2048),      # k >= kv_len / 8 up to 16384
    ("ties", 1, 3, 16384, 2048),
    # Many long causal rows (a chunk's queries): the filter takes several
    # chunks per workgroup under one threshold (rows x chunks >= 16384).
    ("gauss", 1, 1024, 65536, 2048),   # 2 chunks per filter workgroup
    ("ties", 1, 512, 131072, 2048),    # 2 chunks per workgroup, giant tie classes
    ("needle", 2, 600, 66000, 1000),   # 2 chunks per workgroup, a ragged last chunk
    # Large k: at twice the k-th rank a 4096-chunk holds about 1024 candidates,
    # the size of its segment, so rows overflow it and are redone from their
    # scores, with more candidates than the selection keeps in LDS.
    ("gauss", 1, 1, 131072, 16384),
    ("needle", 2, 1, 65536, 8192),
    # Small tie classes at the k-th key (a few tens of equal keys): the
    # selection takes the first of them in position order.
    ("grid", 4, 1, 131072, 2048),
    ("grid", 2, 1, 65536, 1000),
    ("grid", 1, 3, 50000, 2048),
    # The one-launch top-k's row histogram: a k-th key in a bin of a few
    # hundred equal keys (radix passes inside that bin, part of the ties
    # taken), and a small k whose k-th key lies above the sample's largest
    # (the open last bin: the general path) or inside the sampled range.
    ("coarse", 4, 1, 131072, 2048),
    ("coarse", 2, 1, 65536, 1000),
    ("gauss", 2, 1, 131072, 16),
    ("needle", 3, 1, 100000, 64),
    # Many rows through the one-launch form (up to its 64 rows): 16 rows of
    # 16 chunks, and 48 causal rows of a 40000-position cache.
    ("gauss", 16, 1, 65536, 2048),
    ("grid", 1, 48, 40000, 1000),
]


@pytest.mark.parametrize("kind,B,T,L,k", TOPK_CASES)
def test_topk_bit_exact(kind, B, T, L, k):
    announce("topk", kind, B, T, L, k)
    s = inp.score_rows(kind, B, T, L, 31, DEV)
    idx = clsa.topk(s, k)
    torch.cuda.synchronize()
    ref = oracle_topk_rows(s.cpu().numpy(), k)
    assert np.array_equal(idx.cpu().numpy(), ref)


def test_topk_repeat_is_deterministic_and_workspace_reusable():
    B, T, L, k = 2, 1, 70000, 2048
    announce("topk repeat", B, T, L, k)
    s = inp.score_rows("ties", B, T, L, 32, DEV)
    ws = torch.empty(clsa.workspace_bytes(0, B=B, T=T, kv_len=L, k=k), dtype=torch.uint8, device=DEV)
    a = clsa.topk(s, k, ws=ws).clone()
    b = clsa.topk(s, k, ws=ws).clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# sparse attention
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # dtype, B, T, Hq, Hkv, kv_len, L_cap, k
    (inp.F32, 1, 1, 4, 1, 4096, 4096, 256),
    (inp.BF16, 2, 1, 32, 8, 5000, 5000, 2048),
    (inp.BF16, 1, 3, 8, 1, 3000, 3100, 700),
    (inp.BF16, 2, 1, 16, 8, 2000, 2000, 64),
    (inp.BF16, 1, 1, 8, 8, 1500, 1500, 1500),
    (inp.BF16, 1, 2, 32, 4, 4096, 4096, 4096),
    (inp.BF16, 1, 4, 16, 2, 900, 900, 33),
    (inp.F32, 2, 2, 8, 4, 1000, 1024, 100),
    # B*T*Hkv >= 2048: one wave per (query, KV head) walks the whole row, no
    # split states (the chunked-prefill plan): 64 and 128 steps of 32 entries
    (inp.BF16, 1, 256, 32, 8, 8192, 8192, 2048),
    (inp.BF16, 1, 300, 32, 8, 9000, 9100, 4096),
    # large k: the plan's maximum of 256 splits, the combine's largest merge
    (inp.BF16, 1, 1, 32, 8, 20000, 20000, 16384),
    (inp.F32, 1, 1, 8, 2, 12000, 12000, 9000),
    # the decode plans of the benchmark's larger batches (the plan depends on
    # B, T, Hkv and k only): 8 splits of 8 steps per wave (B = 32) and 4
    # splits of 16 steps per wave (B = 64), k = 2048
    (inp.BF16, 32, 1, 32, 8, 3000, 3000, 2048),
    (inp.BF16, 64, 1, 32, 8, 2500, 2600, 2048),
]


def _index(B, T, L, k, seed, holes=True):
    s = inp.score_rows("gauss", B, T, L, seed, "cpu")
    idx = torch.from_numpy(oracle.topk(s.double().numpy(), k))
    if holes:
        g = torch.Generator().manual_seed(seed)
        bad = torch.rand(idx.shape, generator=g) < 0.03
        idx = torch.where(bad, torch.full_like(idx, -1), idx)
        if k > 4:  # out-of-range entries and a repeated position
            idx[..., 1] = L + 5
            idx[..., 2] = idx[..., 3]
    return idx


@pytest.mark.parametrize("dt,B,T,Hq,Hkv,L,cap,k", ATTN_CASES)
def test_sparse_attn_matches_oracle(dt, B, T, Hq, Hkv, L, cap, k):
    announce("sparse_attn", inp.DTYPE_NAME[dt], B, T, Hq, Hkv, L, cap, k)
    D = 128
    q = inp.randn((B, T, Hq, D), dt, 41, DEV)
    kc = inp.randn((B, cap, Hkv, D), dt, 42, DEV)
    vc = inp.randn((B, cap, Hkv, D), dt, 43, DEV)
    idx = _index(B, T, L, k, 44).to(DEV)
    out, lse = clsa.sparse_attn(q, kc, vc, idx, kv_len=L)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_attn_rows(raw(q), raw(kc), raw(vc), dt, raw(idx), L)
    check_out(out_f64(out), ref_o, TOL_OUT[dt])
    lse_close(lse.cpu().numpy(), ref_l, TOL_LSE[dt])


def test_sparse_attn_no_valid_entries():
    announce("sparse_attn empty rows")
    B, T, Hq, Hkv, D, L, k = 1, 2, 8, 2, 128, 300, 128
    q = inp.randn((B, T, Hq, D), inp.BF16, 51, DEV)
    kc = inp.randn((B, L, Hkv, D), inp.BF16, 52, DEV)
    vc = inp.randn((B, L, Hkv, D), inp.BF16, 53, DEV)
    idx = torch.full((B, T, k), -1, dtype=torch.int32)
    idx[0, 0, :] = L - 1          # query 0 sees 0..L-2: all invalid for it
    idx[0, 1, 5] = 7              # query 1: a single valid entry
    out, lse = clsa.sparse_attn(q, kc, vc, idx.to(DEV), kv_len=L)
    torch.cuda.synchronize()
    assert torch.all(out[0, 0] == 0) and torch.all(torch.isneginf(lse[0, 0]))
    # one valid entry: output is that V row (bf16 round trip is exact)
    for h in range(Hq):
        assert torch.equal(out[0, 1, h].float(), vc[0, 7, h // 4].float())


def test_sparse_attn_repeat_is_bitwise_deterministic():
    announce("sparse_attn repeat")
    B, T, Hq, Hkv, D, L, k = 4, 1, 32, 8, 128, 8192, 2048
    q = inp.randn((B, T, Hq, D), inp.BF16, 61, DEV)
    kc = inp.randn((B, L, Hkv, D), inp.BF16, 62, DEV)
    vc = inp.randn((B, L, Hkv, D), inp.BF16, 63, DEV)
    idx = _index(B, T, L, k, 64, holes=False).to(DEV)
    a, la = clsa.sparse_attn(q, kc, vc, idx)
    a, la = a.clone(), la.clone()
    b, lb = clsa.sparse_attn(q, kc, vc, idx)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
