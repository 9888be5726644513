"""CPU oracle for descriptor-driven tile movement -- TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product library
(``async_tensor_tile_amd``) never imports it, and this package imports
nothing from the product.

The arithmetic lives in ``oracle.c`` (plain C, scalar loops written from the
reference pages); this module only compiles it with gcc and marshals NumPy
arrays through ctypes.

Parity status (see the comments in ``oracle.c`` for the passages followed;
the pins are in ``tests/test_oracle_pins.py``): the 128-byte swizzle, the
worked examples and the byte-counted barrier trace are pinned by the pages'
printed tables; the 32-byte and 64-byte swizzles, for which the pages print
no pattern, by the grouping section's bank-sector criterion and its
128-byte-unit key (the rejected row-index reading fails both); the _K256
modes, this library's addition for a 64-bank LDS, by their definition from
the base modes (the key of row r is the base key of row r // 2) and the
sixteen-sector criterion; loads, stores and reductions by NumPy slicing,
torch ``unfold`` and library adds on tiny cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"u8": 0, "u16": 1, "u32": 2, "i32": 3, "u64": 4, "i64": 5,
          "f16": 6, "bf16": 7, "f32": 8, "f64": 9}
ESIZE = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8,
         "f16": 2, "bf16": 2, "f32": 4, "f64": 8}
SWIZZLES = {"none": 0, "32b": 1, "64b": 2, "128b": 3, "32b_k256": 5, "64b_k256": 6, "128b_k256": 7}
FILLS = {"zero": 0, "nan": 1}
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_RANK", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
          5: "ERR_DIM", 6: "ERR_STRIDE", 7: "ERR_BOX", 8: "ERR_ESTRIDE",
          9: "ERR_SWIZZLE_WIDTH", 10: "ERR_OOB_FILL_DTYPE",
          11: "ERR_LDS_CAPACITY", 12: "ERR_UNSUPPORTED"}


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O2, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                               "-fno-fast-math", "-ffp-contract=off",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OrcMap(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("base_addr", ctypes.c_uint64),
                ("dim", ctypes.c_uint64 * 5), ("stride", ctypes.c_uint64 * 5),
                ("box", ctypes.c_uint32 * 5), ("estride", ctypes.c_uint32 * 5),
                ("swizzle", ctypes.c_int32), ("fill", ctypes.c_int32)]


class OrcTxbar(ctypes.Structure):
    _fields_ = [("expected_arrivals", ctypes.c_int32), ("arrivals_left", ctypes.c_int32),
                ("pending_bytes", ctypes.c_int64), ("phase", ctypes.c_int32)]


REDUCE_OPS = {"add": 0, "min": 1, "max": 2}

class OrcIm2col(ctypes.Structure):
    _fields_ = [("t", OrcMap), ("lower", ctypes.c_int32 * 3), ("upper", ctypes.c_int32 * 3),
                ("channels", ctypes.c_uint32), ("pixels", ctypes.c_uint32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        u8p = P(ctypes.c_uint8)
        i32p = P(ctypes.c_int32)
        mp = P(OrcMap)
        L.orc_esize.argtypes = [ctypes.c_int]
        L.orc_validate.argtypes = [mp]
        L.orc_lds_extent.argtypes = [mp, ctypes.c_int]
        L.orc_lds_extent.restype = ctypes.c_uint32
        L.orc_box_bytes.argtypes = [mp]
        L.orc_box_bytes.restype = ctypes.c_uint32
        L.orc_swizzle.argtypes = [ctypes.c_uint32, ctypes.c_int]
        L.orc_swizzle.restype = ctypes.c_uint32
        for name in ("orc_load", "orc_store", "orc_reduce_add"):
            getattr(L, name).argtypes = [mp, u8p, i32p, u8p]
        for name in ("orc_load_batch", "orc_store_batch", "orc_reduce_add_batch"):
            getattr(L, name).argtypes = [mp, u8p, i32p, ctypes.c_uint32, u8p]
        ip = P(OrcIm2col)
        L.orc_im2col_validate.argtypes = [ip]
        L.orc_im2col_box_bytes.argtypes = [ip]
        L.orc_im2col_box_bytes.restype = ctypes.c_uint32
        L.orc_im2col_load_batch.argtypes = [ip, u8p, i32p, i32p, ctypes.c_uint32, u8p]
        L.orc_reduce_minmax_batch.argtypes = [mp, ctypes.c_int, u8p, i32p, ctypes.c_uint32, u8p]
        L.orc_reduce_add_f64_accumulate.argtypes = [mp, P(ctypes.c_double), P(ctypes.c_double),
                                                    i32p, ctypes.c_uint32, u8p]
        tp = P(OrcTxbar)
        L.orc_txbar_init.argtypes = [tp, ctypes.c_int32]
        L.orc_txbar_expect_tx.argtypes = [tp, ctypes.c_int64]
        L.orc_txbar_arrive.argtypes = [tp, ctypes.c_int32]
        L.orc_txbar_arrive_expect_tx.argtypes = [tp, ctypes.c_int64]
        L.orc_txbar_complete_tx.argtypes = [tp, ctypes.c_int64]
        L.orc_txbar_try_wait.argtypes = [tp, ctypes.c_int32]
        L.orc_bank_sector_hist.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p]
        L.orc_gemm_bf16_sample.argtypes = [P(ctypes.c_uint16), P(ctypes.c_uint16), ctypes.c_uint32,
                                           P(ctypes.c_uint32), P(ctypes.c_uint32), ctypes.c_uint32,
                                           P(ctypes.c_double)]
        L.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f64.restype = ctypes.c_double
        L.orc_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.orc_f16_to_f64.restype = ctypes.c_double
        L.orc_f64_to_bf16.argtypes = [ctypes.c_double]
        L.orc_f64_to_bf16.restype = ctypes.c_uint16
        L.orc_f64_to_f16.argtypes = [ctypes.c_double]
        L.orc_f64_to_f16.restype = ctypes.c_uint16
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class Map:
    """A tensor map for the oracle.  dims / strides / box / estride innermost
    first; ``strides`` has rank-1 entries (bytes, dims 1..rank-1)."""

    def __init__(self, dtype, dims, strides, box, estride=None, swizzle="none",
                 fill="zero", base_addr=0x1000):
        rank = len(dims)
        m = OrcMap()
        m.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        m.rank = rank
        m.base_addr = base_addr
        # a rank above 5 is kept in m.rank (and rejected by orc_validate);
        # only the first five entries fit the fixed arrays
        for i, d in enumerate(list(dims)[:5]):
            m.dim[i] = int(d)
        for i, s in enumerate(list(strides)[:4]):
            m.stride[i + 1] = int(s)
        for i, b in enumerate(list(box)[:5]):
            m.box[i] = int(b)
        es = estride if estride is not None else [1] * rank
        for i, e in enumerate(list(es)[:5]):
            m.estride[i] = int(e)
        m.swizzle = SWIZZLES[swizzle] if isinstance(swizzle, str) else int(swizzle)
        m.fill = FILLS[fill] if isinstance(fill, str) else int(fill)
        self.m = m
        self.dtype = dtype
        self.rank = rank

    @property
    def esize(self) -> int:
        return lib().orc_esize(self.m.dtype)

    def validate(self) -> str:
        return STATUS[lib().orc_validate(ctypes.byref(self.m))]

    def box_bytes(self) -> int:
        return lib().orc_box_bytes(ctypes.byref(self.m))

    def lds_extent(self, d: int) -> int:
        return lib().orc_lds_extent(ctypes.byref(self.m), d)

    def _coords(self, coords) -> np.ndarray:
        c = np.ascontiguousarray(np.asarray(coords, dtype=np.int32).reshape(-1, self.rank))
        return c

    def load(self, gmem: np.ndarray, coords) -> np.ndarray:
        """LDS images (uint8, nbox x box_bytes) for each box origin."""
        c = self._coords(coords)
        g = np.ascontiguousarray(gmem).view(np.uint8)
        out = np.zeros((c.shape[0], self.box_bytes()), dtype=np.uint8)
        lib().orc_load_batch(ctypes.byref(self.m), _ptr(g.reshape(-1), ctypes.c_uint8),
                             _ptr(c, ctypes.c_int32), c.shape[0], _ptr(out, ctypes.c_uint8))
        return out

    def store(self, gmem: np.ndarray, coords, images: np.ndarray) -> None:
        """Writes in place into ``gmem`` (must be C-contiguous)."""
        assert gmem.flags.c_contiguous
        c = self._coords(coords)
        g = gmem.view(np.uint8).reshape(-1)
        img = np.ascontiguousarray(images).view(np.uint8).reshape(-1)
        assert img.size == c.shape[0] * self.box_bytes()
        lib().orc_store_batch(ctypes.byref(self.m), _ptr(g, ctypes.c_uint8),
                              _ptr(c, ctypes.c_int32), c.shape[0], _ptr(img, ctypes.c_uint8))

    def reduce_add(self, gmem: np.ndarray, coords, images: np.ndarray) -> None:
        assert gmem.flags.c_contiguous
        c = self._coords(coords)
        g = gmem.view(np.uint8).reshape(-1)
        img = np.ascontiguousarray(images).view(np.uint8).reshape(-1)
        assert img.size == c.shape[0] * self.box_bytes()
        lib().orc_reduce_add_batch(ctypes.byref(self.m), _ptr(g, ctypes.c_uint8),
                                   _ptr(c, ctypes.c_int32), c.shape[0], _ptr(img, ctypes.c_uint8))

    def reduce(self, gmem: np.ndarray, coords, images: np.ndarray, op: str = "add") -> None:
        """Reduce store with op "add", "min" or "max" (boxes in index order)."""
        if op == "add":
            self.reduce_add(gmem, coords, images)
            return
        assert gmem.flags.c_contiguous
        c = self._coords(coords)
        g = gmem.view(np.uint8).reshape(-1)
        img = np.ascontiguousarray(images).view(np.uint8).reshape(-1)
        assert img.size == c.shape[0] * self.box_bytes()
        lib().orc_reduce_minmax_batch(ctypes.byref(self.m), REDUCE_OPS[op], _ptr(g, ctypes.c_uint8),
                                      _ptr(c, ctypes.c_int32), c.shape[0], _ptr(img, ctypes.c_uint8))

    def reduce_add_f64(self, acc: np.ndarray, mag: np.ndarray, coords, images: np.ndarray) -> None:
        """Order-free float64 accumulation of every contribution (in place)."""
        assert acc.dtype == np.float64 and mag.dtype == np.float64
        assert acc.flags.c_contiguous and mag.flags.c_contiguous
        c = self._coords(coords)
        img = np.ascontiguousarray(images).view(np.uint8).reshape(-1)
        lib().orc_reduce_add_f64_accumulate(ctypes.byref(self.m), _ptr(acc, ctypes.c_double),
                                            _ptr(mag, ctypes.c_double), _ptr(c, ctypes.c_int32),
                                            c.shape[0], _ptr(img, ctypes.c_uint8))


class Im2colMap:
    """An im2col-mode map: dims (C, W[, H[, D]], N) innermost first, rank 3..5;
    ``strides`` has rank-1 byte entries; ``lower`` / ``upper`` one entry per
    spatial dimension; ``estride`` full rank (spatial entries are the
    convolution strides)."""

    def __init__(self, dtype, dims, strides, lower, upper, channels, pixels, estride=None,
                 swizzle="none", fill="zero", base_addr=0x1000):
        rank = len(dims)
        m = OrcIm2col()
        t = m.t
        t.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        t.rank = rank
        t.base_addr = base_addr
        for i, d in enumerate(list(dims)[:5]):
            t.dim[i] = int(d)
        for i, st in enumerate(list(strides)[:4]):
            t.stride[i + 1] = int(st)
        es = estride if estride is not None else [1] * rank
        for i, e in enumerate(list(es)[:5]):
            t.estride[i] = int(e)
        t.swizzle = SWIZZLES[swizzle] if isinstance(swizzle, str) else int(swizzle)
        t.fill = FILLS[fill] if isinstance(fill, str) else int(fill)
        for i, v in enumerate(list(lower)[:3]):
            m.lower[i] = int(v)
        for i, v in enumerate(list(upper)[:3]):
            m.upper[i] = int(v)
        m.channels = int(channels)
        m.pixels = int(pixels)
        self.m = m
        self.rank = rank

    def validate(self) -> str:
        return STATUS[lib().orc_im2col_validate(ctypes.byref(self.m))]

    def box_bytes(self) -> int:
        return lib().orc_im2col_box_bytes(ctypes.byref(self.m))

    def load(self, gmem: np.ndarray, coords, offsets) -> np.ndarray:
        """LDS images (uint8, nbox x box_bytes); coords nbox x rank, offsets
        nbox x (rank - 2)."""
        c = np.ascontiguousarray(np.asarray(coords, dtype=np.int32).reshape(-1, self.rank))
        o = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32).reshape(-1, self.rank - 2))
        assert c.shape[0] == o.shape[0]
        g = np.ascontiguousarray(gmem).view(np.uint8)
        out = np.zeros((c.shape[0], self.box_bytes()), dtype=np.uint8)
        lib().orc_im2col_load_batch(ctypes.byref(self.m), _ptr(g.reshape(-1), ctypes.c_uint8),
                                    _ptr(c, ctypes.c_int32), _ptr(o, ctypes.c_int32), c.shape[0],
                                    _ptr(out, ctypes.c_uint8))
        return out


def swizzle(offset: int, mode: str) -> int:
    return lib().orc_swizzle(offset, SWIZZLES[mode])


class Txbar:
    """Transaction-count barrier model; ``state()`` = (arrivals_left, pending, phase)."""

    def __init__(self, count: int):
        self.b = OrcTxbar()
        lib().orc_txbar_init(ctypes.byref(self.b), count)

    def expect_tx(self, n):
        lib().orc_txbar_expect_tx(ctypes.byref(self.b), n)

    def arrive(self, c=1):
        lib().orc_txbar_arrive(ctypes.byref(self.b), c)

    def arrive_expect_tx(self, n):
        lib().orc_txbar_arrive_expect_tx(ctypes.byref(self.b), n)

    def complete_tx(self, n):
        lib().orc_txbar_complete_tx(ctypes.byref(self.b), n)

    def try_wait(self, parity) -> bool:
        return bool(lib().orc_txbar_try_wait(ctypes.byref(self.b), parity))

    def state(self):
        return (self.b.arrivals_left, self.b.pending_bytes, self.b.phase)


def bank_sector_hist(grouped: bool, row0: int, col: int) -> list:
    h = np.zeros(8, dtype=np.int32)
    lib().orc_bank_sector_hist(1 if grouped else 0, row0, col, _ptr(h, ctypes.c_int32))
    return h.tolist()


def gemm_bf16_sample(A_bits: np.ndarray, B_colmajor_bits: np.ndarray, K: int,
                     rows, cols) -> np.ndarray:
    """fp64 C[i,j] for sampled (i, j); A row-major (M,K) bits, B stored (N,K)."""
    A = np.ascontiguousarray(A_bits, dtype=np.uint16).reshape(-1)
    B = np.ascontiguousarray(B_colmajor_bits, dtype=np.uint16).reshape(-1)
    r = np.ascontiguousarray(rows, dtype=np.uint32)
    c = np.ascontiguousarray(cols, dtype=np.uint32)
    out = np.zeros(r.size, dtype=np.float64)
    lib().orc_gemm_bf16_sample(_ptr(A, ctypes.c_uint16), _ptr(B, ctypes.c_uint16), K,
                               _ptr(r, ctypes.c_uint32), _ptr(c, ctypes.c_uint32), r.size,
                               _ptr(out, ctypes.c_double))
    return out


def bf16_to_f64(bits: int) -> float:
    return lib().orc_bf16_to_f64(bits)


def f16_to_f64(bits: int) -> float:
    return lib().orc_f16_to_f64(bits)


def f64_to_bf16(x: float) -> int:
    return lib().orc_f64_to_bf16(x)


def f64_to_f16(x: float) -> int:
    return lib().orc_f64_to_f16(x)
