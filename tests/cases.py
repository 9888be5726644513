"""Random small tensor-map cases shared by the oracle pins and GPU parity
tests (shapes and seeds only; no tile-movement arithmetic)."""
import math

import numpy as np

import synthgen

ESIZE = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8,
         "f16": 2, "bf16": 2, "f32": 4, "f64": 8}
FLOATS = ("f16", "bf16", "f32", "f64")


class Case:
    pass


def random_case(g: np.random.Generator, swizzle=None, dtype=None, rank=None):
    """A small random legal map: dims, byte strides (padded), box, element
    strides, swizzle, fill and a buffer covering the footprint."""
    c = Case()
    c.dtype = dtype or str(g.choice(list(ESIZE)))
    es = ESIZE[c.dtype]
    c.rank = rank or int(g.integers(1, 6))
    c.swizzle = swizzle or str(g.choice(["none", "32b", "64b", "128b", "32b_k256", "64b_k256", "128b_k256"]))
    c.estride = [int(g.integers(1, 4)) for _ in range(c.rank)]
    if c.swizzle == "none":
        L0 = (16 // es) * int(g.integers(1, 4))
    else:
        L0 = (16 << {"32b": 1, "64b": 2, "128b": 3}[c.swizzle.split("_")[0]]) // es
    box0 = (L0 - 1) * c.estride[0] + int(g.integers(1, c.estride[0] + 1))
    if box0 * es % 16 != 0 or box0 > 256:
        c.estride[0] = 1
        box0 = L0
    c.box = [box0] + [int(g.integers(1, 7)) for _ in range(c.rank - 1)]
    c.dims = [int(g.integers(1, 3 * max(box0, 4)))] + [int(g.integers(1, 12)) for _ in range(c.rank - 1)]
    c.strides, s = [], c.dims[0] * es
    for i in range(1, c.rank):
        s = (s + 15) // 16 * 16 + 16 * int(g.integers(0, 2))
        c.strides.append(s)
        s = s * c.dims[i]
    c.footprint = (c.dims[0] * es if c.rank == 1 else c.strides[-1] * c.dims[-1])
    c.buf = synthgen.random_bytes(int(g.integers(0, 1 << 30)), c.footprint + 64)
    c.fill = "nan" if c.dtype in FLOATS and g.integers(0, 2) else "zero"
    c.extent = [math.ceil(c.box[i] / c.estride[i]) for i in range(c.rank)]
    c.span = [(c.extent[i] - 1) * c.estride[i] + 1 for i in range(c.rank)]
    return c


def sweep_coords(g: np.random.Generator, c, nbox: int) -> np.ndarray:
    """Origins from fully below to fully above each dimension."""
    out = np.zeros((nbox, c.rank), dtype=np.int32)
    for i in range(c.rank):
        out[:, i] = g.integers(-c.span[i] - 1, c.dims[i] + 2, size=nbox)
    return out
