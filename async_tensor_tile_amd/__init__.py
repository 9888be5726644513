"""Python binding of the MI355X descriptor-driven tile mover.

Argument marshalling only: every function here forwards to the C ABI declared
in ``include/tmap.h`` (same names), implemented by hand-written gfx950 HIP
kernels in ``libatt_amd.so``.  There is no fallback: if the library has not
been built, every call raises ``NativeLibraryMissing``.

Device pointers are plain integers (``tensor.data_ptr()`` of a torch CUDA
tensor, or any object with ``data_ptr()``); streams are ``hipStream_t`` handles
as integers (``torch.cuda.current_stream().cuda_stream``), 0 = null stream.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ATT_DEBUG=1 in the environment selects the debug build (LDS poisoning and
# device-side checks, reported by tile_device_status).
DEBUG = os.environ.get("ATT_DEBUG", "") not in ("", "0")
LIB_PATH = os.path.join(HERE, "libatt_amd_debug.so" if DEBUG else "libatt_amd.so")

DTYPE = {"u8": 0, "u16": 1, "u32": 2, "i32": 3, "u64": 4, "i64": 5,
         "f16": 6, "bf16": 7, "f32": 8, "f64": 9}
ESIZE = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8,
         "f16": 2, "bf16": 2, "f32": 4, "f64": 8}
SWIZZLE = {"none": 0, "32b": 1, "64b": 2, "128b": 3, "32b_k256": 5, "64b_k256": 6, "128b_k256": 7}
OOB = {"zero": 0, "nan": 1}
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_RANK", 3: "ERR_DTYPE", 4: "ERR_ALIGN",
          5: "ERR_DIM", 6: "ERR_STRIDE", 7: "ERR_BOX", 8: "ERR_ESTRIDE",
          9: "ERR_SWIZZLE_WIDTH", 10: "ERR_OOB_FILL_DTYPE", 11: "ERR_LDS_CAPACITY",
          12: "ERR_UNSUPPORTED", 13: "ERR_HIP", 14: "ERR_TIMEOUT", 15: "ERR_DEVICE_CHECK"}


class NativeLibraryMissing(RuntimeError):
    pass


class TmapError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = f"{where}: {self.name} ({tmap_strerror(status)})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


class tmap_t(ctypes.Structure):
    """Opaque 128-byte descriptor (copied bytewise by the library)."""
    _fields_ = [("opaque", ctypes.c_uint8 * 128)]


class tmap_info_t(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("rank", ctypes.c_int32), ("esize", ctypes.c_int32),
                ("swizzle", ctypes.c_int32), ("oob", ctypes.c_int32),
                ("lds_extent", ctypes.c_uint32 * 5), ("box_bytes", ctypes.c_uint32),
                ("row_bytes", ctypes.c_uint32), ("atom_bytes", ctypes.c_uint32),
                ("base", ctypes.c_uint64)]


_lib = None
_P = ctypes.POINTER
_V = ctypes.c_void_p
_U32 = ctypes.c_uint32
_I32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise NativeLibraryMissing(
                f"{LIB_PATH} is not built; run __graft_entry__.build() "
                "(hipcc --offload-arch=gfx950; the debug build with "
                "async_tensor_tile_amd/_build.py --debug) first")
        L = ctypes.CDLL(LIB_PATH)
        tp = _P(tmap_t)
        L.tmap_encode.argtypes = [tp, _I32, _U32, _V, _P(ctypes.c_uint64), _P(ctypes.c_uint64),
                                  _P(_U32), _P(_U32), _I32, _I32]
        L.tmap_replace_address.argtypes = [tp, _V]
        L.tmap_box_bytes.argtypes = [tp]
        L.tmap_box_bytes.restype = _U32
        L.tmap_query.argtypes = [tp, _P(tmap_info_t)]
        L.tmap_strerror.argtypes = [_I32]
        L.tmap_strerror.restype = ctypes.c_char_p
        L.tmap_last_error.argtypes = []
        L.tmap_last_error.restype = ctypes.c_char_p
        L.tmap_selftest_divide.argtypes = []
        L.tmap_selftest_divide.restype = ctypes.c_uint64
        for name in ("tile_load", "tile_store", "tile_reduce_add"):
            getattr(L, name).argtypes = [tp, _V, _U32, _V, _V]
        L.tile_reduce.argtypes = [tp, _I32, _V, _U32, _V, _V]
        L.tmap_encode_im2col.argtypes = [tp, _I32, _U32, _V, _P(ctypes.c_uint64), _P(ctypes.c_uint64),
                                         _P(_I32), _P(_I32), _U32, _U32, _P(_U32), _I32, _I32]
        L.tile_load_im2col.argtypes = [tp, _V, _V, _U32, _V, _V]
        L.tile_copy.argtypes = [tp, tp, _U32, _V]
        L.tile_copy_ex.argtypes = [tp, tp, _U32, _U32, _U32, _V]
        L.txbar_selftest.argtypes = [tp, _V, _U32, _V, _V, _V]
        L.txbar_selftest_ex.argtypes = [tp, _V, _U32, _U32, _U32, _V, _V, _V]
        L.tile_device_status.argtypes = [_V]
        L.lds_bank_probe.argtypes = [_I32, _U32, _V, _V]
        L.hbm_probe.argtypes = [_I32, _V, _V, ctypes.c_uint64, _V]
        L.hbm_probe_copy_ex.argtypes = [_V, _V, ctypes.c_uint64, _U32, _U32, _V]
        L.hbm_probe_box_copy.argtypes = [_V, _V, _U32, _U32, _U32, _U32, _V]
        L.gemm_bf16.argtypes = [tp, tp, _V, _U32, _U32, _U32, _U32, _U32, _V]
        L.gemm_bf16_ex.argtypes = [tp, tp, _V, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _V]
        L.gemm_bf16_f32.argtypes = [tp, tp, _V, _U32, _U32, _U32, _U32, _U32, _V]
        for name in ("tmap_encode", "tmap_replace_address", "tmap_query", "tile_load", "tile_store",
                     "tile_reduce_add", "tile_reduce", "tmap_encode_im2col", "tile_load_im2col", "tile_copy", "tile_copy_ex",
                     "txbar_selftest", "txbar_selftest_ex", "tile_device_status",
                     "lds_bank_probe", "hbm_probe", "hbm_probe_copy_ex", "hbm_probe_box_copy", "gemm_bf16", "gemm_bf16_ex", "gemm_bf16_f32"):
            getattr(L, name).restype = _I32
        _lib = L
    return _lib


def _addr(x) -> int:
    if x is None:
        return 0
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _check(status: int, where: str):
    if status != 0:
        detail = lib().tmap_last_error().decode() if status == 13 else ""
        raise TmapError(status, where, detail)


def _arr(ctype, vals):
    if vals is None:
        return None
    vals = [int(v) for v in vals]
    return (ctype * max(1, len(vals)))(*vals)


def tmap_strerror(status: int) -> str:
    return lib().tmap_strerror(int(status)).decode()


def tmap_encode(dtype, rank, gaddr, gdim, gstride, box, estride=None, swizzle="none",
                oob="zero") -> tmap_t:
    """Encode a tensor map; dims / strides / box innermost first.  Raises
    TmapError with the library's status on a violated constraint."""
    m = tmap_t()
    dt = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    sw = SWIZZLE[swizzle] if isinstance(swizzle, str) else int(swizzle)
    ob = OOB[oob] if isinstance(oob, str) else int(oob)
    st = lib().tmap_encode(ctypes.byref(m), dt, int(rank), _addr(gaddr),
                           _arr(ctypes.c_uint64, gdim), _arr(ctypes.c_uint64, gstride),
                           _arr(_U32, box), _arr(_U32, estride), sw, ob)
    _check(st, "tmap_encode")
    return m


def tmap_encode_im2col(dtype, rank, gaddr, gdim, gstride, lower, upper, channels_per_pixel,
                       pixels_per_column, estride=None, swizzle="none", oob="zero") -> tmap_t:
    """Encode an im2col-mode map: gdim (C, W[, H[, D]], N) innermost first,
    lower / upper one corner per spatial dimension.  Raises TmapError."""
    m = tmap_t()
    dt = DTYPE[dtype] if isinstance(dtype, str) else int(dtype)
    sw = SWIZZLE[swizzle] if isinstance(swizzle, str) else int(swizzle)
    ob = OOB[oob] if isinstance(oob, str) else int(oob)
    st = lib().tmap_encode_im2col(ctypes.byref(m), dt, int(rank), _addr(gaddr),
                                  _arr(ctypes.c_uint64, gdim), _arr(ctypes.c_uint64, gstride),
                                  _arr(_I32, lower), _arr(_I32, upper), int(channels_per_pixel),
                                  int(pixels_per_column), _arr(_U32, estride), sw, ob)
    _check(st, "tmap_encode_im2col")
    return m


def tmap_replace_address(m: tmap_t, gaddr) -> None:
    _check(lib().tmap_replace_address(ctypes.byref(m), _addr(gaddr)), "tmap_replace_address")


def tmap_box_bytes(m: tmap_t) -> int:
    return int(lib().tmap_box_bytes(ctypes.byref(m)))


def tmap_query(m: tmap_t) -> dict:
    info = tmap_info_t()
    _check(lib().tmap_query(ctypes.byref(m), ctypes.byref(info)), "tmap_query")
    return {"dtype": info.dtype, "rank": info.rank, "esize": info.esize, "swizzle": info.swizzle,
            "oob": info.oob, "lds_extent": list(info.lds_extent), "box_bytes": info.box_bytes,
            "row_bytes": info.row_bytes, "atom_bytes": info.atom_bytes, "base": info.base}


def tile_load(m: tmap_t, d_coords, nbox: int, d_lds_image_out, stream=0) -> None:
    _check(lib().tile_load(ctypes.byref(m), _addr(d_coords), int(nbox), _addr(d_lds_image_out),
                           _addr(stream)), "tile_load")


def tile_load_im2col(m: tmap_t, d_coords, d_offsets, nbox: int, d_lds_image_out, stream=0) -> None:
    _check(lib().tile_load_im2col(ctypes.byref(m), _addr(d_coords), _addr(d_offsets), int(nbox),
                                  _addr(d_lds_image_out), _addr(stream)), "tile_load_im2col")


def tile_store(m: tmap_t, d_coords, nbox: int, d_lds_image_in, stream=0) -> None:
    _check(lib().tile_store(ctypes.byref(m), _addr(d_coords), int(nbox), _addr(d_lds_image_in),
                            _addr(stream)), "tile_store")


def tile_reduce_add(m: tmap_t, d_coords, nbox: int, d_lds_image_in, stream=0) -> None:
    _check(lib().tile_reduce_add(ctypes.byref(m), _addr(d_coords), int(nbox),
                                 _addr(d_lds_image_in), _addr(stream)), "tile_reduce_add")


REDUCE_OPS = {"add": 0, "min": 1, "max": 2}


def tile_reduce(m: tmap_t, op, d_coords, nbox: int, d_lds_image_in, stream=0) -> None:
    """Reduce store with op "add", "min" or "max" (or the TMAP_REDUCE_* value)."""
    code = REDUCE_OPS.get(op, op) if isinstance(op, str) else int(op)
    if isinstance(code, str):
        raise ValueError(f"unknown reduce op {op!r}")
    _check(lib().tile_reduce(ctypes.byref(m), int(code), _addr(d_coords), int(nbox),
                             _addr(d_lds_image_in), _addr(stream)), "tile_reduce")


def tile_copy(src: tmap_t, dst: tmap_t, stages: int = 2, stream=0) -> None:
    _check(lib().tile_copy(ctypes.byref(src), ctypes.byref(dst), int(stages), _addr(stream)),
           "tile_copy")


def tile_copy_ex(src: tmap_t, dst: tmap_t, stages: int = 2, grid: int = 0, variant: int = 0,
                 stream=0) -> None:
    _check(lib().tile_copy_ex(ctypes.byref(src), ctypes.byref(dst), int(stages), int(grid),
                              int(variant), _addr(stream)), "tile_copy_ex")


def txbar_selftest(m: tmap_t, d_coords, ntile: int, d_trace, d_lds_image_out, stream=0) -> None:
    _check(lib().txbar_selftest(ctypes.byref(m), _addr(d_coords), int(ntile), _addr(d_trace),
                                _addr(d_lds_image_out), _addr(stream)), "txbar_selftest")


def txbar_selftest_ex(m: tmap_t, d_coords, ntile: int, extra_bytes: int, max_polls: int, d_trace,
                      d_lds_image_out, stream=0) -> None:
    _check(lib().txbar_selftest_ex(ctypes.byref(m), _addr(d_coords), int(ntile), int(extra_bytes), int(max_polls),
                                   _addr(d_trace), _addr(d_lds_image_out), _addr(stream)), "txbar_selftest_ex")


def tile_device_status(stream=0) -> None:
    """Synchronise `stream` and raise TmapError (ERR_TIMEOUT,
    ERR_DEVICE_CHECK) if a batch kernel recorded a device-side failure since
    the last call; the record is cleared."""
    _check(lib().tile_device_status(_addr(stream)), "tile_device_status")


def hbm_probe(kind, d_src, d_dst, nbytes: int, stream=0) -> None:
    """Streaming HBM probe: kind "read" (0), "write" (1) or "copy" (2)."""
    k = {"read": 0, "write": 1, "copy": 2}.get(kind, kind)
    _check(lib().hbm_probe(int(k), _addr(d_src), _addr(d_dst), int(nbytes), _addr(stream)), "hbm_probe")


def hbm_probe_copy_ex(d_src, d_dst, nbytes: int, variant: int, wg_per_cu: int, stream=0) -> None:
    """The probe's copy in another launch shape (see tmap.h)."""
    _check(lib().hbm_probe_copy_ex(_addr(d_src), _addr(d_dst), int(nbytes), int(variant), int(wg_per_cu),
                                   _addr(stream)), "hbm_probe_copy_ex")


def hbm_probe_box_copy(d_src, d_dst, width: int, height: int, boxes_per_wg: int, variant: int, stream=0) -> None:
    """Box-shaped register copy with the tile copy's access shape (see tmap.h)."""
    _check(lib().hbm_probe_box_copy(_addr(d_src), _addr(d_dst), int(width), int(height), int(boxes_per_wg),
                                    int(variant), _addr(stream)), "hbm_probe_box_copy")


def lds_bank_probe(layout: int, iters: int, d_hist, stream=0) -> None:
    _check(lib().lds_bank_probe(int(layout), int(iters), _addr(d_hist), _addr(stream)),
           "lds_bank_probe")


def gemm_bf16(A: tmap_t, B: tmap_t, d_C, M: int, N: int, K: int, ldc: int, stages: int = 2,
              stream=0) -> None:
    _check(lib().gemm_bf16(ctypes.byref(A), ctypes.byref(B), _addr(d_C), int(M), int(N), int(K),
                           int(ldc), int(stages), _addr(stream)), "gemm_bf16")


def gemm_bf16_f32(A: tmap_t, B: tmap_t, d_C, M: int, N: int, K: int, ldc: int, stages: int = 2,
                  stream=0) -> None:
    """gemm_bf16 with an fp32 C: the unrounded accumulators."""
    _check(lib().gemm_bf16_f32(ctypes.byref(A), ctypes.byref(B), _addr(d_C), int(M), int(N), int(K),
                               int(ldc), int(stages), _addr(stream)), "gemm_bf16_f32")


def gemm_bf16_ex(A: tmap_t, B: tmap_t, d_C, M: int, N: int, K: int, ldc: int, stages: int = 2,
                 group_m: int = 0, xcd: int = 1, stream=0, mfma: int = 0) -> None:
    """mfma: 0 default, 16 (16x16x32 tiles) or 32 (32x32x16 tiles)."""
    _check(lib().gemm_bf16_ex(ctypes.byref(A), ctypes.byref(B), _addr(d_C), int(M), int(N), int(K),
                              int(ldc), int(stages), int(group_m), int(xcd), int(mfma), _addr(stream)),
           "gemm_bf16_ex")
