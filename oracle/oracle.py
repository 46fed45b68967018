"""ctypes front end of the C oracle (``clsa_oracle.c``).

TEST INFRASTRUCTURE ONLY (see the package docstring). Arrays go in as numpy
arrays holding the raw element bits (``float32`` for F32, ``uint16`` for
bfloat16, ``uint8`` for fp8 E4M3FN) and results come back as float64 /
int32 numpy arrays. The C side is single-threaded scalar code accumulating in
double; this module only marshals arguments.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

F32, BF16, FP8_E4M3FN = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "clsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_DT = {F32: np.float32, BF16: np.uint16, FP8_E4M3FN: np.uint8}


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
            lib.orc_decode.argtypes = [P, I, ctypes.c_long, P]
            lib.orc_index_score.argtypes = [P, P, I, P, P, P] + [I] * 6
            lib.orc_topk.argtypes = [P, I, I, I, I, P, P]
            lib.orc_topk_margin.argtypes = [P, I, I, I, I, P, P, P, P]
            lib.orc_sparse_attn.argtypes = [P, P, P, I, P, I, P, P] + [I] * 7 + [D]
            lib.orc_decode_step.argtypes = (
                [I, P, P, P, P, I, P, P, P, I, P, P, P] + [I] * 10 + [P, P, D, P]
            )
            lib.orc_block_union.argtypes = [P, I, I, I, I, I, I, P, P]
            lib.orc_block_attn.argtypes = [P, P, P, I, P, P, I, P, P] + [I] * 7 + [D, I]
            lib.orc_cache_append.argtypes = [P, P, I, I, ctypes.c_long, I, I]
            for f in (
                lib.orc_decode,
                lib.orc_index_score,
                lib.orc_topk,
                lib.orc_topk_margin,
                lib.orc_sparse_attn,
                lib.orc_decode_step,
                lib.orc_block_union,
                lib.orc_block_attn,
                lib.orc_cache_append,
            ):
                f.restype = ctypes.c_int
            lib.orc_decode.restype = None
            _lib = lib
    return _lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)} raw elements, got {a.dtype}")
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def decode(raw: np.ndarray, dtype: int) -> np.ndarray:
    """Decode raw element bits to float64 (used to pin the decoders)."""
    raw = _c(raw, _DT[dtype])
    out = np.empty(raw.shape, np.float64)
    _load().orc_decode(_p(raw), dtype, raw.size, _p(out))
    return out


def index_score(q_idx, k_idx, dtype, w, kv_len, with_bound=False):
    """Indexer scores. q_idx [B,T,H,D], k_idx [B,L_cap,D] raw, w [B,T,H] float32.

    Returns scores [B,T,kv_len] float64 (and the rounding-scale magnitude
    sum_h |w| sum_d |q k| when ``with_bound``).
    """
    q_idx, k_idx = _c(q_idx, _DT[dtype]), _c(k_idx, _DT[dtype])
    w = _c(w, np.float32)
    B, T, H, D = q_idx.shape
    L_cap = k_idx.shape[1]
    if k_idx.shape != (B, L_cap, D) or w.shape != (B, T, H):
        raise ValueError("index_score: inconsistent shapes")
    scores = np.empty((B, T, kv_len), np.float64)
    bound = np.empty((B, T, kv_len), np.float64) if with_bound else None
    rc = _load().orc_index_score(_p(q_idx), _p(k_idx), dtype, _p(w), _p(scores), _p(bound),
                                 B, T, H, D, kv_len, L_cap)
    _check(rc, "index_score")
    return (scores, bound) if with_bound else scores


def topk(scores, k, kv_len=None, k_rows=None):
    """Top-k positions per (b,t). scores [B,T,kv_len] (any float dtype, taken exactly).
    k_rows (optional int32 [B,T]): per-query count of kept positions, clamped to [0, k]."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    B, T, L = scores.shape
    kv_len = L if kv_len is None else kv_len
    if kv_len != L:
        raise ValueError("topk: scores last dim must equal kv_len")
    kr = None if k_rows is None else _c(np.asarray(k_rows).reshape(B, T), np.int32)
    idx = np.empty((B, T, k), np.int32)
    _check(_load().orc_topk(_p(scores), B, T, kv_len, k, _p(kr), _p(idx)), "topk")
    return idx


def topk_margin(scores, k, margin, kv_len=None, k_rows=None):
    """Top-k with ordered skipping (orc_topk_margin). margin: float >= 0, taken
    as float32. Returns (idx [B,T,k] int32, kept [B,T] int32)."""
    scores = np.ascontiguousarray(scores, dtype=np.float64)
    B, T, L = scores.shape
    kv_len = L if kv_len is None else kv_len
    if kv_len != L:
        raise ValueError("topk_margin: scores last dim must equal kv_len")
    kr = None if k_rows is None else _c(np.asarray(k_rows).reshape(B, T), np.int32)
    m = np.array([margin], np.float32)
    idx = np.empty((B, T, k), np.int32)
    kept = np.empty((B, T), np.int32)
    _check(_load().orc_topk_margin(_p(scores), B, T, kv_len, k, _p(kr), _p(m), _p(idx), _p(kept)),
           "topk_margin")
    return idx, kept


def sparse_attn(q, k_cache, v_cache, dtype, idx, kv_len, scale=0.0):
    """Gathered attention. q [B,T,Hq,D], caches [B,L_cap,Hkv,D] raw, idx [B,T,k] int32.

    Returns (out [B,T,Hq,D] float64, lse [B,T,Hq] float64).
    """
    q, k_cache, v_cache = (_c(x, _DT[dtype]) for x in (q, k_cache, v_cache))
    idx = _c(idx, np.int32)
    B, T, Hq, D = q.shape
    L_cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    k = idx.shape[2]
    if k_cache.shape != (B, L_cap, Hkv, D) or v_cache.shape != k_cache.shape or idx.shape[:2] != (B, T):
        raise ValueError("sparse_attn: inconsistent shapes")
    out = np.empty((B, T, Hq, D), np.float64)
    lse = np.empty((B, T, Hq), np.float64)
    rc = _load().orc_sparse_attn(_p(q), _p(k_cache), _p(v_cache), dtype, _p(idx), k, _p(out), _p(lse),
                                 B, T, Hq, Hkv, D, kv_len, L_cap, float(scale))
    _check(rc, "sparse_attn")
    return out, lse


def decode_step(layer_src, q, k_cache, v_cache, dtype, q_idx, k_idx, w, idx_dtype, kv_len, k,
                scale=0.0, k_rows=None, skip_margin=None):
    """One step over len(layer_src) layers sharing routing.

    Per-layer lists of numpy arrays (indexer inputs may be None on S layers).
    Returns (outs, lses, idx_final, n_indexer_calls).
    """
    n = len(layer_src)
    src = np.ascontiguousarray(layer_src, dtype=np.int32)
    qs = [_c(x, _DT[dtype]) for x in q]
    ks = [_c(x, _DT[dtype]) for x in k_cache]
    vs = [_c(x, _DT[dtype]) for x in v_cache]
    qi = [None if x is None else _c(x, _DT[idx_dtype]) for x in q_idx]
    ki = [None if x is None else _c(x, _DT[idx_dtype]) for x in k_idx]
    ws = [None if x is None else _c(x, np.float32) for x in w]
    B, T, Hq, D = qs[0].shape
    L_cap, Hkv = ks[0].shape[1], ks[0].shape[2]
    f0 = next(i for i in range(n) if qi[i] is not None)
    H_I, D_I = qi[f0].shape[2], qi[f0].shape[3]
    outs = [np.empty((B, T, Hq, D), np.float64) for _ in range(n)]
    lses = [np.empty((B, T, Hq), np.float64) for _ in range(n)]
    idx = np.empty((B, T, k), np.int32)
    kr = None if k_rows is None else _c(np.asarray(k_rows).reshape(B, T), np.int32)
    sm = None if skip_margin is None else np.array([skip_margin], np.float32)
    calls = ctypes.c_int(0)
    VP = ctypes.c_void_p * n

    def arr(xs):
        return VP(*[None if x is None else x.ctypes.data for x in xs])

    rc = _load().orc_decode_step(
        n, _p(src), arr(qs), arr(ks), arr(vs), dtype, arr(qi), arr(ki), arr(ws), idx_dtype, _p(idx),
        arr(outs), arr(lses), B, T, Hq, Hkv, D, H_I, D_I, kv_len, L_cap, k, _p(kr), _p(sm), float(scale),
        ctypes.byref(calls),
    )
    _check(rc, "decode_step")
    return outs, lses, idx, calls.value


def block_union(idx, kv_len, block, Hkv):
    """Block-union table per (b, g). Returns (kv_indptr [B*Hkv+1], kv_indices [nnz])."""
    idx = _c(idx, np.int32)
    B, T, k = idx.shape
    nblk = (kv_len + block - 1) // block
    indptr = np.zeros(B * Hkv + 1, np.int32)
    indices = np.empty(B * Hkv * nblk, np.int32)
    rc = _load().orc_block_union(_p(idx), B, T, k, kv_len, block, Hkv, _p(indptr), _p(indices))
    _check(rc, "block_union")
    return indptr, indices[: indptr[-1]].copy()


def block_attn(q, k_cache, v_cache, dtype, kv_indptr, kv_indices, block, kv_len, scale=0.0,
               head_major=False):
    """Dense causal attention over a block table. Returns (out, lse) float64.
    Caches [B,L_cap,Hkv,D], or [B,Hkv,L_cap,D] with head_major."""
    q, k_cache, v_cache = (_c(x, _DT[dtype]) for x in (q, k_cache, v_cache))
    kv_indptr, kv_indices = _c(kv_indptr, np.int32), _c(kv_indices, np.int32)
    B, T, Hq, D = q.shape
    if head_major:
        Hkv, L_cap = k_cache.shape[1], k_cache.shape[2]
    else:
        L_cap, Hkv = k_cache.shape[1], k_cache.shape[2]
    out = np.empty((B, T, Hq, D), np.float64)
    lse = np.empty((B, T, Hq), np.float64)
    rc = _load().orc_block_attn(_p(q), _p(k_cache), _p(v_cache), dtype, _p(kv_indptr), _p(kv_indices),
                                block, _p(out), _p(lse), B, T, Hq, Hkv, D, kv_len, L_cap, float(scale),
                                1 if head_major else 0)
    _check(rc, "block_attn")
    return out, lse


def cache_append(new, cache, pos):
    """Cache with the T rows of new [B, T, ...] written at rows pos .. pos+T-1
    of cache [B, L_cap, ...] (same trailing shape and element type). Returns a
    new array; the input cache is not modified."""
    new = np.ascontiguousarray(new)
    out = np.array(cache, copy=True, order="C")
    if new.dtype != out.dtype or new.shape[0] != out.shape[0] or new.shape[2:] != out.shape[2:]:
        raise TypeError(f"cache_append: new {new.shape} {new.dtype} vs cache {out.shape} {out.dtype}")
    B, T = new.shape[:2]
    row_bytes = int(np.prod(new.shape[2:], dtype=np.int64)) * new.dtype.itemsize
    rc = _load().orc_cache_append(_p(new), _p(out), B, T, row_bytes, int(pos), out.shape[1])
    _check(rc, "cache_append")
    return out
