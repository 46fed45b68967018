"""Arithmetic consistency of the ratios the pages print (CPU only).

The pages give no worked example of the method itself, but several of their
headline figures are ratios of two printed numbers; these tests check that the
figures used to size the benchmark workloads agree with each other. They test
the pages' arithmetic, not the library.
"""

import pytest

from token_sparse_attention_clsa_amd import inputs as inp


def test_indexcache_prefill_speedup_matches_its_latencies():
    # IndexCache summary, "3. Résultats Clés": prefill latency at 200k tokens
    # falls from 19.5 s to 10.7 s, reported as a 1.82x speedup.
    assert round(19.5 / 10.7, 2) == 1.82


def test_indexcache_decode_speedup_matches_its_throughputs():
    # IndexCache summary, "3. Résultats Clés": decode throughput at 200k tokens
    # rises from 58 to 86 tokens/s, reported as 1.48x.
    assert round(86 / 58, 2) == 1.48


def test_indexcache_removed_fraction_matches_the_workload_layer_map():
    # IndexCache summary, "3. Résultats Clés" and "2. Méthodologie : IndexCache":
    # keeping one full layer in four removes 75% of indexer computation.
    wl = inp.config("indexcache48")
    removed = 1 - len(wl.f_layers) / wl.n_layers
    assert removed == pytest.approx(0.75)
    assert len(wl.f_layers) == 12 and wl.n_layers == 48


def test_clsa_decode_speedup_matches_its_example_time():
    # CLSA article, "D'où vient l'accélération": a 7.6x decode speedup turns an
    # 8 s full-attention generation into a little over one second.
    t = 8 / 7.6
    assert 1.0 < t < 1.1


def test_clsa_topk_density_matches_its_cache_size():
    # CLSA article, "Le coût : limites de compatibilité": k = 512 over a 128K
    # cache is about 0.4% density.
    assert round(100 * 512 / 131072, 1) == 0.4
    # The 128K decode workload keeps k = 2048 of 131072 positions (1.56%).
    wl = inp.config("decode128k")
    assert wl.k / wl.kv_len == pytest.approx(2048 / 131072)
