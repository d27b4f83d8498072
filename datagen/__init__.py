"""Seeded synthetic Q/K/V inputs for the attention forward.

This module draws and rounds random numbers and nothing else: it holds none of
the attention arithmetic, so both the fp64 oracle (tests only) and the HIP path
can consume its output without sharing any of the method's code.

Recipe (identical for every workload):

1. ``numpy.random.Generator(PCG64(seed))``.
2. ``standard_normal`` in float64, drawn in the order Q, K, V, each of shape
   ``[B, H, N, d]`` in C order.
3. The workload's multiplier is applied to all three tensors (x0.5 for the
   fp16 long-sequence workload; a power of two, so exact).
4. Hot keys (the 64K-length workload only): per (b, h), ``floor(frac * N)``
   distinct key indices are drawn uniformly without replacement from the same
   generator, after V, in (b, h) C order; those K rows are multiplied by
   ``hot_mult`` (8, a power of two).
5. Cast to the workload dtype on the CPU: numpy's round-to-nearest-even
   float64->fp32 for fp32; for bf16/fp16, torch's conversion, which rounds
   float64->fp32->dtype, each step to nearest even.

Both the GPU path and the oracle read these rounded values, so input rounding
is never counted as kernel error.

The five workloads stand in for the pages' examples: page 1 section 4 runs a
single head with N=512, d=64 in fp16; page 3 section 1.1 discusses seq_len 4096
(a 4096x4096 score matrix) and sequences of 64K or longer.  No public dataset
or benchmark suite is involved.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_qkv_kv", "make_grad", "workload_inputs",
           "TORCH_DTYPE", "DECODE"]

TORCH_DTYPE = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic attention-forward workload: shape, dtype and value recipe."""

    key: int
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str  # "f32" | "f16" | "bf16"
    mult: float = 1.0
    hot_frac: float = 0.0
    hot_mult: float = 1.0

    @property
    def scale(self) -> float:
        # 1/sqrt(d), rounded to fp32 once: the value the kernel receives, and
        # the value the oracle is given, so scale rounding is shared.
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Algorithmic flops of the two contractions: 4*B*H*N^2*d."""
        return 4.0 * self.B * self.H * self.N * self.N * self.d

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def hot_keys(self) -> int:
        return int(math.floor(self.hot_frac * self.N))

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "B": self.B,
            "H": self.H,
            "N": self.N,
            "d": self.d,
            "dtype": self.dtype,
            "scale": self.scale,
            "causal": False,
            "values": self.values_recipe(),
        }

    def values_recipe(self) -> str:
        s = "N(0,1)"
        if self.mult != 1.0:
            s += f"*{self.mult:g}"
        if self.hot_keys:
            s += f"; {self.hot_keys} keys/head x{self.hot_mult:g}"
        return s


WORKLOADS = {
    1: Workload(1, "single-head N=128 d=64 fp32", 1, 1, 128, 64, "f32"),
    2: Workload(2, "B4 H8 N1024 d64 bf16", 4, 8, 1024, 64, "bf16"),
    3: Workload(3, "B2 H16 N4096 d128 bf16", 2, 16, 4096, 128, "bf16"),
    4: Workload(4, "B1 H32 N16384 d128 fp16 x0.5", 1, 32, 16384, 128, "f16", mult=0.5),
    5: Workload(5, "B1 H8 N65536 d64 bf16 hot-keys", 1, 8, 65536, 64, "bf16",
                hot_frac=0.01, hot_mult=8.0),
}


def _round_to(x64: np.ndarray, dtype: str) -> torch.Tensor:
    """RNE cast of a float64 array to the workload dtype, as a CPU tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    # torch rounds float64 -> fp32 -> bf16/fp16 (RNE at each step).  Whatever
    # the rounding, both sides of a comparison read the same rounded values.
    return torch.from_numpy(np.ascontiguousarray(x64)).to(TORCH_DTYPE[dtype])


def make_qkv(B: int, H: int, N: int, d: int, dtype: str, seed: int,
             mult: float = 1.0, hot_frac: float = 0.0, hot_mult: float = 1.0):
    """Return (q, k, v) as contiguous CPU tensors of ``dtype``, shape [B,H,N,d]."""
    if dtype not in TORCH_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (B, H, N, d)
    q = rng.standard_normal(shape)
    k = rng.standard_normal(shape)
    v = rng.standard_normal(shape)
    if mult != 1.0:
        q *= mult
        k *= mult
        v *= mult
    n_hot = int(math.floor(hot_frac * N))
    if n_hot:
        for b in range(B):
            for h in range(H):
                idx = rng.choice(N, size=n_hot, replace=False)
                k[b, h, idx, :] *= hot_mult
    return _round_to(q, dtype), _round_to(k, dtype), _round_to(v, dtype)


def make_qkv_kv(B: int, H: int, N: int, Nk: int, d: int, dtype: str, seed: int,
                mult: float = 1.0, hot_frac: float = 0.0, hot_mult: float = 1.0):
    """``make_qkv`` with a key length of its own: q of shape [B, H, N, d], k and
    v of shape [B, H, Nk, d], drawn in that order from one generator, hot keys
    (``floor(hot_frac * Nk)`` per head) drawn after v.  With Nk = N the values
    are those of ``make_qkv``."""
    if dtype not in TORCH_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, Nk, d))
    v = rng.standard_normal((B, H, Nk, d))
    if mult != 1.0:
        q *= mult
        k *= mult
        v *= mult
    n_hot = int(math.floor(hot_frac * Nk))
    if n_hot:
        for b in range(B):
            for h in range(H):
                idx = rng.choice(Nk, size=n_hot, replace=False)
                k[b, h, idx, :] *= hot_mult
    return _round_to(q, dtype), _round_to(k, dtype), _round_to(v, dtype)


# Decode-shaped inputs: one new query per head scored against a long cache of
# keys and values (page 3 section 4: in generation each step computes a
# 1 x seq_len row of scores against the growing K/V cache, which makes memory
# bandwidth the bottleneck).  The heads and head dimension of the N=16384
# workload, the 64K length page 3 section 1.1 mentions, bf16, N(0,1) values.
DECODE = dict(name="decode B1 H32 N1 Nk65536 d128 bf16", B=1, H=32, N=1, Nk=65536, d=128,
              dtype="bf16", seed=6)


def hot_key_indices(B: int, H: int, N: int, d: int, seed: int, hot_frac: float):
    """The hot-key indices ``make_qkv`` draws for the same arguments, per (b, h)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    for _ in range(3):
        rng.standard_normal((B, H, N, d))
    n_hot = int(math.floor(hot_frac * N))
    out = {}
    for b in range(B):
        for h in range(H):
            out[(b, h)] = np.sort(rng.choice(N, size=n_hot, replace=False))
    return out


def workload_inputs(key: int, seed: int | None = None):
    """(q, k, v) for one of the five workloads; ``seed`` defaults to its number."""
    w = WORKLOADS[key]
    return make_qkv(w.B, w.H, w.N, w.d, w.dtype, w.key if seed is None else seed,
                    w.mult, w.hot_frac, w.hot_mult)


def make_grad(B: int, H: int, N: int, d: int, dtype: str, seed: int):
    """A seeded upstream gradient dO of shape [B, H, N, d]: standard normal
    from its own generator (seed offset so it never repeats Q/K/V's stream),
    rounded to ``dtype`` as in ``make_qkv``."""
    if dtype not in TORCH_DTYPE:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.Generator(np.random.PCG64(seed + 0x5EED_0000))
    g = rng.standard_normal((B, H, N, d))
    return torch.from_numpy(g.astype(np.float32)).to(TORCH_DTYPE[dtype]).contiguous()
