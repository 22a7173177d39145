"""Seeded synthetic inputs for exact scaled-dot-product attention.

Every tensor is drawn as float32 standard normals from numpy's PCG64
``default_rng`` with a tuple seed, multiplied by a power-of-two standard
deviation (exact in float32), and then rounded to its 16-bit storage format
with round-to-nearest-even.  Both the GPU path and the CPU oracle consume the
same 16-bit bit patterns, so they see bit-identical inputs; the oracle widens
them exactly to float64.

Layout is ``[B, H, N, d]`` with ``d`` innermost (page 1, example 2: query,
key and value are ``(batch, heads, len, head_dim)``).

Seed convention: ``default_rng([workload_id, (extra,) tensor_id])`` with tensor
ids q=0, k=1, v=2, dO=3, after page 1 example 2, which draws q, k and v from
PRNG keys 0, 1 and 2.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

FMT_F16 = "f16"
FMT_BF16 = "bf16"

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "do": 3}


# ----------------------------------------------------------------------------
# 16-bit storage formats (formats only: no attention arithmetic here)
# ----------------------------------------------------------------------------
def f32_to_bits(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float32 values to fp16 or bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if fmt == FMT_F16:
        return x.astype(np.float16).view(np.uint16)
    if fmt == FMT_BF16:
        u = x.view(np.uint32).astype(np.uint64)
        if np.any(((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)):
            raise ValueError("NaN in bf16 input generation")  # +-inf round to themselves
        rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return rounded.astype(np.uint16)
    raise ValueError(f"unknown format {fmt!r}")


def bits_to_f32(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Exact widening of fp16/bf16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if fmt == FMT_F16:
        return bits.view(np.float16).astype(np.float32)
    if fmt == FMT_BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown format {fmt!r}")


def bits_to_f64(bits: np.ndarray, fmt: str) -> np.ndarray:
    """Exact widening of fp16/bf16 bit patterns to float64."""
    return bits_to_f32(bits, fmt).astype(np.float64)


def normal_bits(seed, shape, std: float, fmt: str) -> np.ndarray:
    """i.i.d. N(0, std^2) draws rounded to ``fmt``; ``std`` must be a power of two."""
    m, e = math.frexp(std)
    if m != 0.5:
        raise ValueError("std must be a power of two so that scaling is exact")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return f32_to_bits(x, fmt)


def default_scale(d: int) -> float:
    """1/sqrt(d) rounded to float32 (the value handed to the kernel), as a Python float."""
    return float(np.float32(1.0 / math.sqrt(d)))


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    fmt: str
    causal: bool
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    do: Optional[np.ndarray] = None
    notes: dict = field(default_factory=dict)

    @property
    def shape(self):
        return (self.B, self.H, self.N, self.d)

    def f64(self, name: str) -> np.ndarray:
        return bits_to_f64(getattr(self, name), self.fmt)


def _draw(seed_prefix, shape, std, fmt, with_do):
    out = {}
    names = ["q", "k", "v"] + (["do"] if with_do else [])
    for n in names:
        out[n] = normal_bits(list(seed_prefix) + [TENSOR_IDS[n]], shape, std, fmt)
    return out


def random_case(B, H, N, d, fmt=FMT_F16, causal=False, seed=0, std=1.0,
                with_do=False, scale=None, name=None) -> Workload:
    """Generic seeded case used by the small parity and edge-case tests."""
    shape = (B, H, N, d)
    t = _draw([1000, seed, B, H, N, d], shape, std, fmt, with_do)
    return Workload(name or f"random_B{B}H{H}N{N}d{d}_{fmt}_{'c' if causal else 'nc'}_s{seed}",
                    B, H, N, d, fmt, causal,
                    default_scale(d) if scale is None else float(np.float32(scale)),
                    t["q"], t["k"], t["v"], t.get("do"))


def tiny_fwd() -> Workload:
    """Non-causal fwd, B=1 H=4 N=128 d=64, fp16 N(0,1), scale 1/sqrt(64)."""
    shape = (1, 4, 128, 64)
    t = _draw([1], shape, 1.0, FMT_F16, False)
    return Workload("tiny_fwd_B1H4N128d64_f16", *shape, FMT_F16, False, default_scale(64),
                    t["q"], t["k"], t["v"])


def a100_sweep(N: int, with_do: bool = False) -> Workload:
    """Non-causal fwd at the A100 table's shape, B=2 H=12 d=64, fp16 N(0,1)."""
    shape = (2, 12, N, 64)
    t = _draw([2, N], shape, 1.0, FMT_F16, with_do)
    return Workload(f"a100_shape_B2H12N{N}d64_f16", *shape, FMT_F16, False, default_scale(64),
                    t["q"], t["k"], t["v"], t.get("do"))


def spiked_causal(N: int = 4096, H: int = 16) -> Workload:
    """Causal fwd, B=2 H=16 N=4096 d=128, bf16 N(0,1); key rows j = 0 mod 64 scaled by 8.

    The x8 is applied to the bf16 values (exact: it only moves the exponent).
    """
    shape = (2, H, N, 128)
    t = _draw([3], shape, 1.0, FMT_BF16, False)
    k32 = bits_to_f32(t["k"], FMT_BF16)
    k32[:, :, ::64, :] *= np.float32(8.0)
    t["k"] = f32_to_bits(k32, FMT_BF16)
    return Workload(f"spiked_causal_B2H{H}N{N}d128_bf16", *shape, FMT_BF16, True,
                    default_scale(128), t["q"], t["k"], t["v"],
                    notes={"spike": "K rows j%64==0 scaled x8"})


def long_causal(N: int = 32768, with_do: bool = False) -> Workload:
    """Long-sequence causal attention, B=1 H=8 d=64, bf16 N(0, 0.5^2) (dO too,
    for the backward at the same shape)."""
    shape = (1, 8, N, 64)
    t = _draw([4, N], shape, 0.5, FMT_BF16, with_do)
    return Workload(f"long_causal_B1H8N{N}d64_bf16", *shape, FMT_BF16, True, default_scale(64),
                    t["q"], t["k"], t["v"], t.get("do"))


def attn_bias(shape, fmt: str, seed, kind: str = "random", **kw) -> np.ndarray:
    """Seeded additive attention bias bits of ``shape`` (..., N, N), 16-bit.

    kinds:
      "random": N(0, std^2) (std = kw "std", default 2) with a fraction
                kw "hole" (default 0.2) of entries set to -inf, and row
                kw "dead_row" (default 3, if < N) entirely -inf.
      "window": 0 where |i - j| <= kw "width", -inf elsewhere (a band).
      "keypad": 0 for keys j < L_b, -inf beyond, with L_b from kw "lengths"
                (one per leading index of ``shape``).
    """
    shape = tuple(shape)
    n_q, n_k = shape[-2], shape[-1]
    if kind == "random":
        rng = np.random.default_rng(list(seed) + [7])
        x = (rng.standard_normal(shape, dtype=np.float32) * np.float32(kw.get("std", 2.0)))
        x[rng.random(shape) < kw.get("hole", 0.2)] = -np.inf
        r = kw.get("dead_row", 3)
        if r is not None and r < n_q:
            x[..., r, :] = -np.inf
    elif kind == "window":
        i = np.arange(n_q)[:, None]
        j = np.arange(n_k)[None, :]
        band = np.where(np.abs(i - j) <= kw["width"], 0.0, -np.inf).astype(np.float32)
        x = np.broadcast_to(band, shape).copy()
    elif kind == "keypad":
        lengths = list(kw["lengths"])
        x = np.zeros(shape, dtype=np.float32)
        for b, L in enumerate(lengths):
            x[b, ..., L:] = -np.inf
    else:
        raise ValueError(kind)
    return f32_to_bits(x, fmt)


def long_causal_sample_rows(H: int, N: int, count: int = 256):
    """(h, i) rows checked for the long causal workload: ``count`` distinct random
    pairs from ``default_rng([4, 99])`` plus fixed boundary rows on the first and
    last head. Returned sorted, unique, as an int64 array of shape [R, 2]."""
    rng = np.random.default_rng([4, 99])
    flat = rng.choice(H * N, size=count, replace=False)
    pairs = {(int(f // N), int(f % N)) for f in flat}
    for h in (0, H - 1):
        for i in (0, 1, 63, 64, 127, 128, N - 1):
            if i < N:
                pairs.add((h, i))
    return np.array(sorted(pairs), dtype=np.int64)


def fwd_bwd(causal: bool, N: int = 4096) -> Workload:
    """Fwd+bwd, B=2 H=12 N=4096 d=64, fp16 Q/K/V/dO N(0,1)."""
    shape = (2, 12, N, 64)
    t = _draw([5, N], shape, 1.0, FMT_F16, True)
    return Workload(f"fwd_bwd_B2H12N{N}d64_f16_{'causal' if causal else 'noncausal'}",
                    *shape, FMT_F16, causal, default_scale(64),
                    t["q"], t["k"], t["v"], t["do"])
