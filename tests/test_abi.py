"""Host-side checks of the C-ABI library (no GPU needed): it loads, exports
every symbol that include/*.h declares, and its descriptor validator agrees
with the oracle's on the constraint table of the reference pages."""
import ctypes
import glob
import os
import re

import pytest

import async_tensor_tile_amd as att
import oracle
import synthgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(([^;{]*?)\)\s*;", text, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert "tmap_encode" in names and "tile_load" in names and "gemm_bf16" in names
    L = ctypes.CDLL(att.LIB_PATH)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_invariant_division_exact():
    assert att.lib().tmap_selftest_divide() == 0


BASE = 0x7F0000000000   # a 16-byte aligned stand-in address; encode never dereferences it

CASES = [
    dict(),
    dict(dims=(16,) * 6, strides=(32,) * 5, box=(16,) * 6, swizzle="none"),
    dict(box=(64, 257)), dict(box=(64, 0)), dict(box=(4, 8), swizzle="none"),
    dict(strides=(264,)), dict(strides=(1 << 40,)), dict(strides=((1 << 40) - 16,)), dict(strides=(0,)),
    dict(base=BASE + 8), dict(box=(128, 8)), dict(box=(32, 8)), dict(box=(32, 8), swizzle="64b"),
    dict(box=(16, 8), swizzle="32b"), dict(box=(256, 8), swizzle="none"),
    dict(dtype="i32", box=(32, 8), fill="nan"), dict(dtype="f32", box=(32, 8), fill="nan"),
    dict(estride=(1, 9)), dict(estride=(2, 1), box=(128, 8)), dict(estride=(3, 1), box=(128, 8), swizzle="none"),
    dict(dims=(0, 64)), dict(dims=((1 << 32) + 1, 64)), dict(dims=((1 << 32), 64)),
    dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 8)),
    dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 5)),
    dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 4)),
    dict(dtype="f32", dims=(32, 159, 8), strides=(128, 20352), box=(32, 159, 8)),
    dict(dtype="f32", dims=(32, 160, 8), strides=(128, 20480), box=(32, 160, 8)),
    dict(dtype="u8", box=(128, 8)), dict(dtype="f64", box=(16, 8), fill="nan"),
    dict(swizzle="128b_k256"), dict(swizzle="64b_k256", box=(32, 8)), dict(swizzle="32b_k256", box=(16, 8)),
    dict(swizzle="64b_k256"), dict(swizzle=4), dict(swizzle=8),
]


def _both(dtype="bf16", dims=(128, 64), strides=(256,), box=(64, 32), estride=None, swizzle="128b",
          fill="zero", base=BASE):
    om = oracle.Map(dtype, dims, strides, box, estride, swizzle, fill, base_addr=base)
    want = om.validate()
    try:
        att.tmap_encode(dtype, len(dims), base, dims, strides, box, estride, swizzle, fill)
        got = "OK"
    except att.TmapError as e:
        got = e.name
    return got, want


@pytest.mark.parametrize("case", range(len(CASES)))
def test_encode_agrees_with_oracle_validator(case):
    got, want = _both(**CASES[case])
    assert got == want


def test_encode_random_agreement():
    g = synthgen.rng(99)
    dts = list(att.DTYPE)
    for _ in range(3000):
        rank = int(g.integers(1, 6))
        dtype = dts[int(g.integers(0, len(dts)))]
        dims = [int(g.choice([0, 1, 7, 300, 1 << 32, (1 << 32) + 1])) if g.random() < 0.1
                else int(g.integers(1, 5000)) for _ in range(rank)]
        strides = [int(g.choice([0, 8, 16, 48, 1 << 40, (1 << 40) - 16, 4096])) for _ in range(rank - 1)]
        box = [int(g.choice([0, 1, 2, 4, 8, 16, 32, 64, 128, 256, 257])) for _ in range(rank)]
        es = [int(g.integers(0, 10)) for _ in range(rank)] if g.random() < 0.5 else None
        sw = int(g.integers(0, 9))
        fill = ["zero", "nan"][int(g.integers(0, 2))]
        base = BASE + int(g.choice([0, 0, 0, 8]))
        got, want = _both(dtype, dims, strides, box, es, sw, fill, base)
        assert got == want, (dtype, dims, strides, box, es, sw, fill, base)


def test_encode_query_and_replace():
    m = att.tmap_encode("f32", 5, BASE, (260, 129, 33, 7, 3), (1040, 134160, 4427280, 30990960),
                        (32, 32, 8, 2, 1), (1, 2, 1, 1, 1), "128b", "nan")
    q = att.tmap_query(m)
    assert att.tmap_query(att.tmap_encode("bf16", 2, BASE, (64, 64), (128,), (64, 16), None,
                                          "128b_k256"))["atom_bytes"] == 2048
    assert q["lds_extent"] == [32, 16, 8, 2, 1]
    assert q["box_bytes"] == 32768 == att.tmap_box_bytes(m)
    assert q["row_bytes"] == 128 and q["atom_bytes"] == 1024 and q["esize"] == 4
    assert q["base"] == BASE
    att.tmap_replace_address(m, BASE + 4096)
    assert att.tmap_query(m)["base"] == BASE + 4096
    with pytest.raises(att.TmapError) as ei:
        att.tmap_replace_address(m, BASE + 4)
    assert ei.value.name == "ERR_ALIGN"
    # the 4096-byte expectation of two 2048-byte operand tiles ([MLC] load wait)
    a = att.tmap_encode("bf16", 2, BASE, (64, 64), (128,), (64, 16), None, "128b")
    assert 2 * att.tmap_box_bytes(a) == 4096


def test_launch_argument_errors_without_gpu():
    m = att.tmap_encode("bf16", 2, BASE, (64, 64), (128,), (64, 16), None, "128b")
    # nbox == 0 is a no-op and NULL pointers are rejected before any HIP call
    att.tile_load(m, 0, 0, 0)
    with pytest.raises(att.TmapError) as ei:
        att.tile_load(m, 0, 3, 0)
    assert ei.value.name == "ERR_NULL"
    with pytest.raises(att.TmapError) as ei:
        att.lds_bank_probe(0, 1, 0)
    assert ei.value.name == "ERR_NULL"
    # tile_reduce: unknown op, and NULL pointers, rejected without a HIP call
    att.tile_reduce(m, "max", 0, 0, 0)
    with pytest.raises(att.TmapError) as ei:
        att.tile_reduce(m, 7, BASE, 1, BASE)
    assert ei.value.name == "ERR_UNSUPPORTED"
    with pytest.raises(att.TmapError) as ei:
        att.tile_reduce(m, "min", 0, 2, BASE)
    assert ei.value.name == "ERR_NULL"
    # hbm_probe: argument checks come before any HIP call
    att.hbm_probe("copy", BASE, BASE, 0)
    att.hbm_probe_copy_ex(BASE, BASE, 0, 15, 1)
    for args, name in (((BASE, BASE, 16, 16, 1), "ERR_UNSUPPORTED"), ((BASE, BASE, 16, 0, 0), "ERR_UNSUPPORTED"),
                       ((BASE, BASE, 16, 0, 33), "ERR_UNSUPPORTED"), ((BASE, BASE, 24, 0, 1), "ERR_UNSUPPORTED"),
                       ((0, BASE, 16, 0, 1), "ERR_NULL"), ((BASE, BASE + 8, 16, 0, 1), "ERR_ALIGN")):
        with pytest.raises(att.TmapError) as ei:
            att.hbm_probe_copy_ex(*args)
        assert ei.value.name == name, args
    # gemm: empty outputs are no-ops, the rest is checked before any HIP call
    mA = att.tmap_encode("bf16", 2, BASE, (96, 256), (192,), (64, 256), None, "128b")
    mB = att.tmap_encode("bf16", 2, BASE, (96, 512), (192,), (64, 256), None, "128b")
    mB128 = att.tmap_encode("bf16", 2, BASE, (96, 512), (192,), (64, 128), None, "128b")
    att.gemm_bf16(mA, mB, BASE, 0, 512, 96, 512, 2)
    att.gemm_bf16(mA, mB, BASE, 256, 0, 96, 512, 2)
    for call, name in ((lambda: att.gemm_bf16(mA, mB, BASE, 256, 512, 0, 512, 2), "ERR_UNSUPPORTED"),   # K == 0
                       (lambda: att.gemm_bf16(mA, mB, BASE, 256, 512, 64, 512, 2), "ERR_UNSUPPORTED"),  # dims != K
                       (lambda: att.gemm_bf16(mA, mB, BASE, 256, 512, 96, 500, 2), "ERR_UNSUPPORTED"),  # ldc < N
                       (lambda: att.gemm_bf16(mA, mB, 0, 256, 512, 96, 512, 2), "ERR_NULL"),
                       (lambda: att.gemm_bf16(mA, mB, BASE, 256, 512, 96, 512, 3), "ERR_UNSUPPORTED"),  # K % 64
                       (lambda: att.gemm_bf16(mA, mB, BASE, 256, 512, 96, 512, 4), "ERR_UNSUPPORTED"),  # stages
                       (lambda: att.gemm_bf16_ex(mA, mB, BASE, 256, 512, 96, 512, 2, 0, 1, 0, 7), "ERR_UNSUPPORTED"),
                       (lambda: att.gemm_bf16(mA, mB128, BASE, 256, 512, 96, 512, 2), "ERR_UNSUPPORTED")):  # box
        with pytest.raises(att.TmapError) as ei:
            call()
        assert ei.value.name == name
    # txbar_selftest_ex: poll bound and extra bytes are checked on the host
    m = att.tmap_encode("bf16", 2, BASE, (64, 64), (128,), (64, 16), None, "128b")
    with pytest.raises(att.TmapError) as ei:
        att.txbar_selftest_ex(m, 0, 1, 0, 1, BASE, BASE)
    assert ei.value.name == "ERR_NULL"
    for args, name in ((("copy", BASE, BASE, 17), "ERR_UNSUPPORTED"), ((3, BASE, BASE, 16), "ERR_UNSUPPORTED"),
                       (("copy", 0, BASE, 16), "ERR_NULL"), (("write", 0, 0, 16), "ERR_NULL"),
                       (("read", BASE, BASE + 8, 16), "ERR_ALIGN")):
        with pytest.raises(att.TmapError) as ei:
            att.hbm_probe(*args)
        assert ei.value.name == name, args


# ------------------------------- im2col maps ---------------------------------

IM2COL_CASES = [
    dict(), dict(channels=6), dict(channels=0), dict(channels=260), dict(pixels=0), dict(pixels=1025),
    dict(estride=(2, 2, 2, 1)), dict(estride=(1, 9, 2, 1)), dict(estride=(1, 2, 2, 2)),
    dict(upper=(-12, -1)), dict(lower=(40000, 0)), dict(swizzle="128b"), dict(channels=32, swizzle="128b"),
    dict(channels=16, swizzle="64b_k256"), dict(dtype="i32", fill="nan"), dict(dtype="bf16", channels=64, fill="nan"),
    dict(channels=256, pixels=1024), dict(strides=(24, 352, 3168)), dict(strides=(32, 0, 3168)),
    dict(dims=(8, 11), strides=(32,), lower=(), upper=(), estride=(1, 1)),
    dict(dims=(8, 11, 2), strides=(32, 352), lower=(-2,), upper=(1,), estride=(1, 3, 1)),
    dict(dims=(8, 5, 5, 5, 2), strides=(32, 160, 800, 4000), lower=(0, -1, 0), upper=(0, 0, -4),
         estride=(1, 1, 2, 1, 1)),
    dict(dims=(0, 11, 9, 2)), dict(base=BASE + 8),
]

# More windows than a signed 64-bit index counts: accepted by the oracle (the
# pages set no bound), rejected by the library, whose kernels decode a
# window's position from a 64-bit linear index.
HUGE_WINDOWS = dict(dims=(8, 1 << 32, 1 << 32, 1 << 32, 4), strides=(32, 1 << 35, 1 << 36, 1 << 37),
                    lower=(0, 0, 0), upper=(0, 0, 0), estride=(1, 1, 1, 1, 1))


def _im2col_args(**kw):
    a = dict(dtype="f32", dims=(8, 11, 9, 2), strides=(32, 352, 3168), lower=(-1, -1), upper=(-1, -1),
             channels=8, pixels=16, estride=(1, 2, 2, 1), swizzle="none", fill="zero", base=BASE)
    a.update(kw)
    return a


@pytest.mark.parametrize("case", range(len(IM2COL_CASES)))
def test_im2col_encode_agrees_with_oracle(case):
    """The library's im2col encoder accepts and rejects exactly what the
    oracle's validator does, with the same status."""
    a = _im2col_args(**IM2COL_CASES[case])
    om = oracle.Im2colMap(a["dtype"], a["dims"], a["strides"], a["lower"], a["upper"], a["channels"],
                          a["pixels"], a["estride"], a["swizzle"], a["fill"], base_addr=a["base"])
    want = om.validate()
    try:
        m = att.tmap_encode_im2col(a["dtype"], len(a["dims"]), a["base"], a["dims"], a["strides"], a["lower"],
                                   a["upper"], a["channels"], a["pixels"], a["estride"], a["swizzle"], a["fill"])
        got = "OK"
    except att.TmapError as e:
        got = e.name
    assert got == want
    if got == "OK":
        q = att.tmap_query(m)
        assert q["box_bytes"] == om.box_bytes()
        assert q["lds_extent"] == [a["channels"], a["pixels"], 1, 1, 1]


def test_im2col_window_count_limit_of_the_library():
    """The library's own limit (at most 2^62 windows, one 64-bit linear
    index each); the oracle validates the same map."""
    a = _im2col_args(**HUGE_WINDOWS)
    om = oracle.Im2colMap(a["dtype"], a["dims"], a["strides"], a["lower"], a["upper"], a["channels"],
                          a["pixels"], a["estride"], a["swizzle"], a["fill"], base_addr=a["base"])
    assert om.validate() == "OK"
    with pytest.raises(att.TmapError) as ei:
        att.tmap_encode_im2col(a["dtype"], len(a["dims"]), a["base"], a["dims"], a["strides"], a["lower"],
                               a["upper"], a["channels"], a["pixels"], a["estride"], a["swizzle"], a["fill"])
    assert ei.value.name == "ERR_DIM"
    # 2^62 windows exactly are accepted: 2^20 x 2^20 x 2^20 positions x 4 images
    ok = dict(HUGE_WINDOWS, dims=(8, 1 << 20, 1 << 20, 1 << 20, 4), strides=(32, 1 << 25, 1 << 30, 1 << 35))
    b = _im2col_args(**ok)
    att.tmap_encode_im2col(b["dtype"], len(b["dims"]), b["base"], b["dims"], b["strides"], b["lower"], b["upper"],
                           b["channels"], b["pixels"], b["estride"], b["swizzle"], b["fill"])


def test_im2col_map_rejected_by_tiled_entry_points():
    m = att.tmap_encode_im2col("bf16", 4, BASE, (64, 8, 8, 2), (128, 1024, 8192), (-1, -1), (-1, -1), 64, 32,
                               None, "128b")
    t = att.tmap_encode("bf16", 2, BASE, (64, 64), (128,), (64, 16), None, "128b")
    for call in (lambda: att.tile_load(m, BASE, 1, BASE), lambda: att.tile_store(m, BASE, 1, BASE),
                 lambda: att.tile_reduce(m, "add", BASE, 1, BASE), lambda: att.tile_copy(m, m, 2),
                 lambda: att.gemm_bf16(m, m, BASE, 256, 256, 64, 256, 2)):
        with pytest.raises(att.TmapError) as ei:
            call()
        assert ei.value.name == "ERR_UNSUPPORTED"
    # and a tiled map is not an im2col map
    with pytest.raises(att.TmapError) as ei:
        att.tile_load_im2col(t, BASE, BASE, 1, BASE)
    assert ei.value.name == "ERR_UNSUPPORTED"
    att.tile_load_im2col(m, 0, 0, 0, 0)          # nbox == 0: no-op
    with pytest.raises(att.TmapError) as ei:
        att.tile_load_im2col(m, BASE, 0, 1, BASE)
    assert ei.value.name == "ERR_NULL"
