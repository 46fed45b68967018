"""Pins the oracle's element decoders against torch's own conversions.

Every bfloat16 bit pattern and every fp8 E4M3FN bit pattern is decoded by the
oracle and by torch (an independent implementation of the same formats).
"""

import numpy as np
import torch

import oracle


def _same(a, b):
    nan = np.isnan(a)
    assert np.array_equal(nan, np.isnan(b))
    assert np.array_equal(a[~nan], b[~nan])
    # signed zeros keep their sign
    assert np.array_equal(np.signbit(a[~nan]), np.signbit(b[~nan]))


def test_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits, oracle.BF16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    _same(ours, ref)


def test_fp8_e4m3fn_all_patterns():
    bits = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(bits, oracle.FP8_E4M3FN)
    ref = torch.from_numpy(bits).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    _same(ours, ref)
    assert np.nanmax(ours) == 448.0 and np.nanmin(ours) == -448.0
    assert np.isnan(ours).sum() == 2  # 0x7f and 0xff only: no infinities


def test_f32_patterns_sample():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    special = np.array([0, 0x80000000, 1, 0x7f800000, 0xff800000, 0x7fc00000, 0x00800000, 0x7f7fffff],
                       dtype=np.uint32)
    bits = np.concatenate([bits, special])
    ours = oracle.decode(bits.view(np.float32), oracle.F32)
    with np.errstate(invalid="ignore"):
        ref = bits.view(np.float32).astype(np.float64)
    _same(ours, ref)


def test_integer_grid_exact_in_every_storage_type():
    # The "int" input recipe relies on integers in [-8, 8] being exact in all three types.
    ints = np.arange(-8, 9, dtype=np.float32)
    for dt, tdt in ((oracle.BF16, torch.bfloat16), (oracle.FP8_E4M3FN, torch.float8_e4m3fn)):
        t = torch.from_numpy(ints).to(tdt)
        raw = t.view(torch.int16 if dt == oracle.BF16 else torch.uint8).numpy()
        raw = raw.view(np.uint16) if dt == oracle.BF16 else raw
        assert np.array_equal(oracle.decode(raw, dt), ints.astype(np.float64))
    assert np.array_equal((ints * 4).astype(np.float64),
                          oracle.decode(torch.from_numpy(ints * 4).to(torch.bfloat16).view(torch.int16)
                                        .numpy().view(np.uint16), oracle.BF16))
