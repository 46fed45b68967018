"""Seeded synthetic inputs for the CLSA hot path.

This module only draws random tensors and moves raw bits around; it holds
none of the method's arithmetic. Both the HIP library's callers and the
oracle's callers take their inputs from here, so both sides see the same
bits: tensors are drawn once (on the device that will run the kernels) and
copied to host as raw element bits for the oracle.

Workload shapes follow the decode and chunked-prefill settings the pages
describe (CLSA article: 128K-token context; IndexCache summary: 1-in-4
F-layer pattern; CompactAttention summary: chunked prefill against a long
cached prefix, 64-token blocks, GQA). Value recipes:
  * "gauss": indexer q/k, attention q/K/V ~ N(0,1) rounded once to the
    storage type; head weights ~ U[0,1).
  * "int":   indexer q/k integers uniform in [-8, 8] (exact in f32, bf16 and
    fp8 E4M3FN); head weights j / 2**m, j uniform in [0, 2**m]; with these
    the float32 indexer score is exact in any summation order, so the top-k
    set is unique and bit-exact.
  * needles: a seeded 1% of positions per batch element get their indexer
    key row and attention K rows multiplied by 4 (V untouched).
"""

from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

F32, BF16, FP8_E4M3FN = 0, 1, 2
TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, FP8_E4M3FN: torch.float8_e4m3fn}
DTYPE_NAME = {F32: "f32", BF16: "bf16", FP8_E4M3FN: "fp8_e4m3fn"}


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    T: int
    kv_len: int
    H_I: int
    D_I: int
    k: int
    Hq: int
    Hkv: int
    D: int
    layer_src: List[int]
    dtype: int = BF16
    idx_dtype: int = BF16
    shared_kv: bool = True        # one YOCO cache for every layer
    needle_frac: float = 0.0
    weight_bits: int = 4          # m for the "int" weights j / 2**m
    L_cap: Optional[int] = None   # allocated cache rows (default kv_len)

    @property
    def n_layers(self) -> int:
        return len(self.layer_src)

    @property
    def cap(self) -> int:
        return self.kv_len if self.L_cap is None else self.L_cap

    @property
    def f_layers(self) -> List[int]:
        return [l for l, s in enumerate(self.layer_src) if s == l]


def _cfgs():
    return {
        # Tiny decode, fp32: 4 layers share one index over one cache.
        "tiny": Workload("tiny", B=1, T=1, kv_len=4096, H_I=4, D_I=64, k=256, Hq=4, Hkv=1, D=128,
                         layer_src=[0] * 4, dtype=F32, idx_dtype=F32, weight_bits=8),
        # Decode, bf16, 8 cross-decoder layers over one shared cache.
        "decode32k": Workload("decode32k", B=8, T=1, kv_len=32768, H_I=64, D_I=128, k=2048, Hq=32,
                              Hkv=8, D=128, layer_src=[0] * 8),
        # Long-context decode, bf16, 16 YOCO layers reuse one index; 1% needles.
        "decode128k": Workload("decode128k", B=4, T=1, kv_len=131072, H_I=64, D_I=128, k=2048,
                               Hq=32, Hkv=8, D=128, layer_src=[0] * 16, needle_frac=0.01,
                               weight_bits=3),
        # IndexCache pattern: 48 layers, F every 4th, per-layer caches.
        "indexcache48": Workload("indexcache48", B=16, T=1, kv_len=65536, H_I=64, D_I=128, k=2048,
                                 Hq=32, Hkv=8, D=128, layer_src=[4 * (l // 4) for l in range(48)],
                                 shared_kv=False),
        # Chunked prefill: 2048-query chunk after 131072 cached tokens.
        "prefill2k": Workload("prefill2k", B=1, T=2048, kv_len=131072 + 2048, H_I=64, D_I=128,
                              k=4096, Hq=32, Hkv=8, D=128, layer_src=[0]),
    }


CONFIGS = _cfgs()


def config(name: str, **overrides) -> Workload:
    return dataclasses.replace(CONFIGS[name], **overrides)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def randn(shape, dtype: int, seed: int, device="cpu") -> torch.Tensor:
    """N(0,1) drawn in float32, rounded once to the storage type."""
    x = torch.randn(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)
    return x.to(TORCH_DTYPE[dtype])


def randint(shape, lo: int, hi: int, dtype: int, seed: int, device="cpu") -> torch.Tensor:
    """Integers uniform in [lo, hi], stored exactly in the given type."""
    x = torch.randint(lo, hi + 1, shape, generator=_gen(seed, device), device=device,
                      dtype=torch.int32)
    return x.to(torch.float32).to(TORCH_DTYPE[dtype])


def weights(shape, variant: str, seed: int, device="cpu", bits: int = 4) -> torch.Tensor:
    if variant == "int":
        j = torch.randint(0, 2 ** bits + 1, shape, generator=_gen(seed, device), device=device,
                          dtype=torch.int32)
        return j.to(torch.float32) / float(2 ** bits)
    return torch.rand(shape, generator=_gen(seed, device), device=device, dtype=torch.float32)


def needle_positions(B: int, kv_len: int, frac: float, seed: int, device="cpu") -> torch.Tensor:
    """[B, n] int64: a seeded random frac of positions per batch element."""
    n = int(round(frac * kv_len))
    g = _gen(seed, device)
    rows = [torch.randperm(kv_len, generator=g, device=device)[:n] for _ in range(B)]
    return torch.stack(rows) if rows else torch.zeros((B, 0), dtype=torch.int64, device=device)


def scale_rows_(x: torch.Tensor, pos: torch.Tensor, factor: float) -> None:
    """x[b, pos[b], ...] *= factor for a [B, L, ...] tensor (exact for factor 4)."""
    for b in range(x.shape[0]):
        sel = x[b].index_select(0, pos[b])
        x[b].index_copy_(0, pos[b], (sel.float() * factor).to(x.dtype))


@dataclasses.dataclass
class Tensors:
    """Device tensors of one workload. Indexer lists hold None on S layers."""
    wl: Workload
    q: List[torch.Tensor]
    k_cache: List[torch.Tensor]
    v_cache: List[torch.Tensor]
    q_idx: List[Optional[torch.Tensor]]
    k_idx: List[Optional[torch.Tensor]]
    w: List[Optional[torch.Tensor]]
    needles: Optional[torch.Tensor] = None


def make(wl: Workload, variant: str = "gauss", seed: int = 0, device="cpu") -> Tensors:
    """Draw every input of a workload. variant in {"gauss", "int"}.

    In "int" the indexer q/k are integers in [-8, 8]; attention q/K/V stay
    Gaussian (attention parity is a tolerance check either way).
    """
    B, T, L, cap = wl.B, wl.T, wl.kv_len, wl.cap
    s = 1000 * int(seed)
    needles = None
    if wl.needle_frac > 0:
        needles = needle_positions(B, L, wl.needle_frac, s + 1, device)
    n_kv = 1 if wl.shared_kv else wl.n_layers
    ks, vs = [], []
    for c in range(n_kv):
        kc = randn((B, cap, wl.Hkv, wl.D), wl.dtype, s + 10 + 2 * c, device)
        if needles is not None:
            scale_rows_(kc, needles, 4.0)
        ks.append(kc)
        vs.append(randn((B, cap, wl.Hkv, wl.D), wl.dtype, s + 11 + 2 * c, device))
    k_cache = [ks[0 if wl.shared_kv else l] for l in range(wl.n_layers)]
    v_cache = [vs[0 if wl.shared_kv else l] for l in range(wl.n_layers)]
    q = [randn((B, T, wl.Hq, wl.D), wl.dtype, s + 200 + l, device) for l in range(wl.n_layers)]
    q_idx, k_idx, w = [], [], []
    for l in range(wl.n_layers):
        if wl.layer_src[l] != l:
            q_idx.append(None)
            k_idx.append(None)
            w.append(None)
            continue
        base = s + 400 + 4 * l
        if variant == "int":
            qi = randint((B, T, wl.H_I, wl.D_I), -8, 8, wl.idx_dtype, base, device)
            ki = randint((B, cap, wl.D_I), -8, 8, wl.idx_dtype, base + 1, device)
        else:
            qi = randn((B, T, wl.H_I, wl.D_I), wl.idx_dtype, base, device)
            ki = randn((B, cap, wl.D_I), wl.idx_dtype, base + 1, device)
        if needles is not None:
            scale_rows_(ki, needles, 4.0)
        q_idx.append(qi)
        k_idx.append(ki)
        w.append(weights((B, T, wl.H_I), variant, base + 2, device, bits=wl.weight_bits))
    return Tensors(wl, q, k_cache, v_cache, q_idx, k_idx, w, needles)


def score_rows(kind: str, B: int, T: int, L: int, seed: int, device="cpu") -> torch.Tensor:
    """float32 [B, T, L] score rows for exercising top-k on its own.

    kinds: "gauss" (N(0,1)), "ties" (integers in [0, 7]: huge tie classes),
    "zeros" (all +0/-0, mixed), "relu" (half exact zeros, signed zeros mixed,
    rest Gaussian), "needle" (N(0,1) with 1% of entries +8), "const" (all 3.5),
    "desc" (strictly decreasing with position), "wide" (spans many octaves),
    "strided" (every 64th position far above the rest), "sampled" (far
    above the rest exactly at the positions the top-k filter samples for its
    threshold: 128 evenly spaced runs of 16, run j starting at
    j * (L - 16) // 127; single-query rows, L > 2048), "grid" (N(0,1)
    rounded to multiples of 1/256: near the k-th largest of a long row each
    value is shared by a few tens of positions, small tie classes), "coarse"
    (N(0,1) rounded to multiples of 1/16: a few hundred positions share the
    k-th largest value of a long row).
    """
    g = _gen(seed, device)
    shape = (B, T, L)
    if kind == "gauss":
        return torch.randn(shape, generator=g, device=device)
    if kind == "ties":
        return torch.randint(0, 8, shape, generator=g, device=device).float()
    if kind == "zeros":
        sign = torch.randint(0, 2, shape, generator=g, device=device).bool()
        return torch.where(sign, torch.tensor(-0.0, device=device), torch.tensor(0.0, device=device))
    if kind == "relu":
        x = torch.randn(shape, generator=g, device=device)
        sign = torch.randint(0, 2, shape, generator=g, device=device).bool()
        z = torch.where(sign, torch.tensor(-0.0, device=device), torch.tensor(0.0, device=device))
        return torch.where(x > 0, x, z)
    if kind == "needle":
        x = torch.randn(shape, generator=g, device=device)
        m = torch.rand(shape, generator=g, device=device) < 0.01
        return torch.where(m, x + 8.0, x)
    if kind == "const":
        return torch.full(shape, 3.5, device=device)
    if kind == "grid":
        return torch.round(torch.randn(shape, generator=g, device=device) * 256.0) / 256.0
    if kind == "coarse":
        return torch.round(torch.randn(shape, generator=g, device=device) * 16.0) / 16.0
    if kind == "desc":
        return (-torch.arange(L, device=device, dtype=torch.float32)).expand(shape).contiguous()
    if kind == "strided":  # every 64th position far above the rest
        x = torch.randn(shape, generator=g, device=device)
        pos = torch.arange(L, device=device)
        return torch.where((pos % 64 == 0).expand(shape), torch.full_like(x, 100.0), x)
    if kind == "sampled":
        x = torch.randn(shape, generator=g, device=device)
        hit = torch.zeros(L, dtype=torch.bool, device=device)
        for j in range(128):
            st = j * (L - 16) // 127
            hit[st:st + 16] = True
        return torch.where(hit.expand(shape), torch.full_like(x, 100.0), x)
    if kind == "wide":
        e = torch.randint(-60, 60, shape, generator=g, device=device).float()
        x = torch.randn(shape, generator=g, device=device)
        return x * torch.exp2(e)
    raise ValueError(kind)


def raw(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy of a tensor's raw element bits (float32 / uint16 / uint8)."""
    t = t.detach().contiguous()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    if t.dtype == torch.int32:
        return t.cpu().numpy()
    raise TypeError(t.dtype)
