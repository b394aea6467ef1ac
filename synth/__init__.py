"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and lays them out; it holds none of the
LoRA arithmetic.  Floating-point tensors are drawn in float64 with numpy's PCG64
generator and converted to bfloat16 with torch's own CPU dtype conversion, so the
bf16 bytes a test hands to the GPU path and to the CPU reference are the same
bytes.  bf16 tensors are returned as numpy ``uint16`` bit patterns.

Shapes follow the LoRA notation of "Reproducible LoRA Inference Through
Deterministic Split-K Reduction" (Balusamy & Mohan), Eq. 1:

* ``x``  [M x K]  tokens x hidden (the paper's X in R^{M x H});
* ``A``  [r x K]  the down projection, stored as the paper stores it
  (A in R^{r x H}, the shrink is X A^T);
* ``B``  [N x r]  the up projection (B in R^{H_out x r}, the expand is (.) B^T);
* ``y``  [M x N]  the bf16 layer output the expand adds into.

``N(0, s)`` in a workload description is read as a normal with standard
deviation ``s``.  Every tensor gets its own child stream of one seed, keyed by a
name, so adding a tensor never shifts the values of another.
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "rng_for", "normal_bf16", "integer_bf16", "segments_to_ids", "random_segments",
    "single_adapter_case", "sgmv_case", "bf16_bits_to_f32", "SgmvCase", "SingleCase",
]


def rng_for(seed: int, name: str) -> np.random.Generator:
    """An independent PCG64 stream for tensor ``name`` under ``seed``."""
    key = zlib.crc32(name.encode("utf-8"))
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(key)]))


def _to_bf16_bits(a64: np.ndarray) -> np.ndarray:
    import torch  # CPU dtype conversion only
    t = torch.from_numpy(np.ascontiguousarray(a64, dtype=np.float64)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, std: float, seed: int, name: str) -> np.ndarray:
    """N(0, std) drawn in float64, stored as bf16 bit patterns."""
    g = rng_for(seed, name)
    return _to_bf16_bits(g.standard_normal(size=shape) * float(std))


def integer_bf16(shape, lo: int, hi: int, seed: int, name: str) -> np.ndarray:
    """Uniform integers in [lo, hi] stored as bf16 (exact for |v| <= 256)."""
    g = rng_for(seed, name)
    return _to_bf16_bits(g.integers(lo, hi + 1, size=shape).astype(np.float64))


def random_segments(M: int, lo: int, hi: int, n_adapters: int, seed: int, name: str):
    """Contiguous runs of tokens with uniform lengths in [lo, hi] (inclusive).

    Each run gets an adapter id uniform in {0..n_adapters-1}; the last run is
    cut to fit M.  Returns a list of (start, length, adapter)."""
    g = rng_for(seed, name)
    segs = []
    start = 0
    while start < M:
        ln = int(g.integers(lo, hi + 1))
        ln = min(ln, M - start)
        segs.append((start, ln, int(g.integers(0, n_adapters))))
        start += ln
    return segs


def segments_to_ids(M: int, segs) -> np.ndarray:
    ids = np.full((M,), -1, dtype=np.int32)
    for (s, ln, a) in segs:
        ids[s:s + ln] = a
    return ids


@dataclass
class SingleCase:
    x: np.ndarray          # bf16 bits [M, K]
    A: np.ndarray          # bf16 bits [r, K]
    B: np.ndarray | None   # bf16 bits [N, r]
    y: np.ndarray | None   # bf16 bits [M, N]
    M: int
    K: int
    r: int
    N: int
    split_k: int
    scale: float


def single_adapter_case(M: int, K: int, r: int, N: int = 0, split_k: int = 8,
                        scale: float = 2.0, seed: int = 0, x_std: float = 1.0,
                        w_std: float = 0.02, y_std: float = 1.0, tag: str = "") -> SingleCase:
    """One adapter: x ~ N(0, x_std), A, B ~ N(0, w_std), y ~ N(0, y_std)."""
    x = normal_bf16((M, K), x_std, seed, f"x{tag}")
    A = normal_bf16((r, K), w_std, seed, f"A{tag}")
    B = normal_bf16((N, r), w_std, seed, f"B{tag}") if N else None
    y = normal_bf16((M, N), y_std, seed, f"y{tag}") if N else None
    return SingleCase(x, A, B, y, M, K, r, N, split_k, scale)


@dataclass
class SgmvCase:
    x: np.ndarray
    As: list               # bf16 bits [r_i, K]
    Bs: list               # bf16 bits [N, r_i]
    ranks: np.ndarray      # int32 [n]
    scales: np.ndarray     # float32 [n]
    ids: np.ndarray        # int32 [M]
    y: np.ndarray
    M: int
    K: int
    N: int
    r_max: int
    split_k: int
    segs: list = field(default_factory=list)


def sgmv_case(M: int, K: int, N: int, ranks, seg_lo: int, seg_hi: int, split_k: int,
              scale: float = 2.0, seed: int = 0, tag: str = "", ids=None) -> SgmvCase:
    """Several adapters with per-token ids in contiguous runs of random length."""
    ranks = np.asarray(ranks, dtype=np.int32)
    n = len(ranks)
    x = normal_bf16((M, K), 1.0, seed, f"sx{tag}")
    As = [normal_bf16((int(ranks[a]), K), 0.02, seed, f"sA{tag}{a}") for a in range(n)]
    Bs = [normal_bf16((N, int(ranks[a])), 0.02, seed, f"sB{tag}{a}") for a in range(n)]
    y = normal_bf16((M, N), 1.0, seed, f"sy{tag}")
    segs = []
    if ids is None:
        segs = random_segments(M, seg_lo, seg_hi, n, seed, f"seg{tag}")
        ids = segments_to_ids(M, segs)
    ids = np.asarray(ids, dtype=np.int32)
    scales = np.full((n,), scale, dtype=np.float32)
    return SgmvCase(x, As, Bs, ranks, scales, ids, y, M, K, N, int(ranks.max()), split_k, segs)
