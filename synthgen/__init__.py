"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds only random-number generation and workload shapes; none of
the tile-movement arithmetic (addressing, swizzle, fill, reduction) lives
here.  Every stream is NumPy's PCG64 seeded with an integer, so the CPU oracle
and the GPU path see identical bits.
"""
from __future__ import annotations

import numpy as np

from .workloads import WORKLOADS  # noqa: F401


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def u16_bits(seed: int, shape) -> np.ndarray:
    """Uniform 16-bit patterns (covers NaN, Inf and subnormal encodings)."""
    return rng(seed).integers(0, 1 << 16, size=shape, dtype=np.uint16)


def random_bytes(seed: int, nbytes: int) -> np.ndarray:
    return rng(seed).integers(0, 256, size=nbytes, dtype=np.uint8)


def normal_bf16_bits(seed: int, shape) -> np.ndarray:
    """N(0,1) float32 draws rounded to bfloat16 (nearest-even) as uint16 bits."""
    f = rng(seed).standard_normal(size=shape, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def uniform_f32(seed: int, shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return rng(seed).uniform(lo, hi, size=shape).astype(np.float32)


def normal_f32(seed: int, shape) -> np.ndarray:
    return rng(seed).standard_normal(size=shape, dtype=np.float32)


def int32_range(seed: int, shape, lo: int, hi: int) -> np.ndarray:
    """Uniform integers in the closed range [lo, hi]."""
    return rng(seed).integers(lo, hi, size=shape, dtype=np.int32, endpoint=True)


def edge_mix_coords(seed: int, dims, extents, estrides, nbox: int, edge_every: int = 4,
                    align0: int = 1) -> np.ndarray:
    """Box origins (nbox x rank, innermost first).

    A box reads coordinates c_i + k_i * es_i for k_i < extent_i.  Box b with
    b % edge_every == edge_every - 1 straddles a tensor edge (some loaded
    coordinates in range, some out) in at least one seeded dimension; every
    other box lies fully inside.  ``align0`` rounds dimension-0 origins down to
    a multiple of itself (interior boxes stay inside).
    """
    g = rng(seed)
    rank = len(dims)
    span = [(int(extents[i]) - 1) * int(estrides[i]) + 1 for i in range(rank)]
    out = np.zeros((nbox, rank), dtype=np.int32)
    can_straddle = [i for i in range(rank) if span[i] > 1]
    for b in range(nbox):
        for i in range(rank):
            hi = int(dims[i]) - span[i]
            out[b, i] = g.integers(0, hi + 1) if hi > 0 else 0
        if b % edge_every == edge_every - 1:
            nd = int(g.integers(1, len(can_straddle) + 1))
            chosen = g.choice(can_straddle, size=nd, replace=False)
            for i in chosen:
                if g.integers(0, 2) == 0:      # low edge: origin in [-span+1, -1]
                    out[b, i] = -int(g.integers(1, span[i]))
                else:                          # high edge: origin in [dim-span+1, dim-1]
                    out[b, i] = int(dims[i]) - span[i] + int(g.integers(1, span[i]))
        if align0 > 1:
            out[b, 0] = (int(out[b, 0]) // align0) * align0
    return out


def uniform_coords(seed: int, nbox: int, lo, hi) -> np.ndarray:
    """nbox origins, dimension i uniform in the closed range [lo[i], hi[i]]."""
    g = rng(seed)
    cols = [g.integers(int(lo[i]), int(hi[i]), size=nbox, endpoint=True) for i in range(len(lo))]
    return np.stack(cols, axis=1).astype(np.int32)


def sample_pairs(seed: int, n: int, M: int, N: int):
    g = rng(seed)
    return (g.integers(0, M, size=n).astype(np.uint32),
            g.integers(0, N, size=n).astype(np.uint32))
