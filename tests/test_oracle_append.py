"""Pins the oracle's cache append (the path's input side).

CLSA article, opening section: each new token of context adds keys and
values to the stored cache; "Comment CLSA fonctionne": that cache is shared
by the cross-decoder layers, so a token's rows are written once. The token's
indexer key goes with them.

Pins: appending T rows at once equals T single-row appends; rows outside
[pos, pos + T) keep their bytes; invalid ranges are rejected; a decode step
over a cache whose last rows were cleared and appended back equals the step
over the original cache, and stepping at kv_len = pos ignores every row from
pos on (so the step sees exactly the rows the append wrote).
"""

import numpy as np
import pytest

import oracle


def _f32(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float32))


@pytest.mark.parametrize("dt,shape", [(np.uint16, (3, 20, 2, 8)), (np.uint8, (2, 17, 5)),
                                      (np.float32, (1, 10, 3))])
def test_block_append_equals_row_by_row(dt, shape):
    rng = np.random.default_rng(5)
    cache = rng.integers(0, 200, shape).astype(dt)
    T, pos = 4, 6
    new = rng.integers(0, 200, (shape[0], T) + shape[2:]).astype(dt)
    whole = oracle.cache_append(new, cache, pos)
    step = cache
    for t in range(T):
        step = oracle.cache_append(new[:, t:t + 1], step, pos + t)
    assert whole.tobytes() == step.tobytes()


def test_other_rows_keep_their_bytes():
    rng = np.random.default_rng(6)
    cache = rng.integers(0, 65535, (2, 30, 4, 8)).astype(np.uint16)
    new = rng.integers(0, 65535, (2, 3, 4, 8)).astype(np.uint16)
    out = oracle.cache_append(new, cache, 27)  # the last rows of the cache
    keep = np.ones(30, bool)
    keep[27:30] = False
    assert out[:, keep].tobytes() == cache[:, keep].tobytes()
    assert not np.array_equal(out, cache)


@pytest.mark.parametrize("pos,T,cap", [(-1, 1, 8), (8, 1, 8), (6, 3, 8)])
def test_out_of_range_rows_rejected(pos, T, cap):
    with pytest.raises(ValueError):
        oracle.cache_append(np.zeros((1, T, 4), np.uint16), np.zeros((1, cap, 4), np.uint16), pos)


@pytest.mark.parametrize("T_new", [1, 3])
def test_step_over_appended_cache_equals_original(T_new):
    rng = np.random.default_rng(40 + T_new)
    B, L, Hq, Hkv, D, H, DI, k, n = 2, 48, 4, 2, 16, 3, 8, 12, 3
    src = [0] * n
    K = _f32(rng.standard_normal((B, L, Hkv, D)))
    V = _f32(rng.standard_normal((B, L, Hkv, D)))
    KI = _f32(rng.integers(-8, 9, (B, L, DI)))
    q = [_f32(rng.standard_normal((B, 1, Hq, D))) for _ in range(n)]
    qi = [_f32(rng.integers(-8, 9, (B, 1, H, DI)))] + [None] * (n - 1)
    w = [_f32(rng.integers(0, 17, (B, 1, H)) / 16)] + [None] * (n - 1)
    pos = L - T_new
    # Clear the last rows, then append them back as the new tokens.
    Kc, Vc, KIc = K.copy(), V.copy(), KI.copy()
    Kc[:, pos:] = 0
    Vc[:, pos:] = 0
    KIc[:, pos:] = 0
    Ka = oracle.cache_append(K[:, pos:], Kc, pos)
    Va = oracle.cache_append(V[:, pos:], Vc, pos)
    KIa = oracle.cache_append(KI[:, pos:], KIc, pos)

    def run(Kx, Vx, KIx, kv_len):
        return oracle.decode_step(src, q, [Kx] * n, [Vx] * n, oracle.F32, qi, [KIx] + [None] * (n - 1), w,
                                  oracle.F32, kv_len=kv_len, k=k)

    ref, got = run(K, V, KI, L), run(Ka, Va, KIa, L)
    for a, b in zip(ref[:3], got[:3]):
        for x, y in zip(a if isinstance(a, list) else [a], b if isinstance(b, list) else [b]):
            assert np.array_equal(np.asarray(x), np.asarray(y))
    # At kv_len = pos the cleared rows and the original rows give the same step.
    before_a, before_b = run(Kc, Vc, KIc, pos), run(K, V, KI, pos)
    for a, b in zip(before_a[:3], before_b[:3]):
        for x, y in zip(a if isinstance(a, list) else [a], b if isinstance(b, list) else [b]):
            assert np.array_equal(np.asarray(x), np.asarray(y))
