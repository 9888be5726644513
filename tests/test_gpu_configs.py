"""GPU parity at the full workload sizes: the 8192^2 bf16 round trip, the
rank-5 fp32 edge-crossing load with zero / NaN fill, and the 4096^2 reduce-add
store, each against the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
from synthgen import workloads as W  # noqa: E402

from gpu_util import empty_dev, encode, require_native, stream, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


# ------------------------- bf16 8192^2 round trip ---------------------------

def _copy_case(dims, box, swizzle, stages, variant=0, grid=0, seed=2):
    H, Wd = dims[1], dims[0]
    src = synthgen.u16_bits(seed, (H, Wd))
    sd = to_dev(src)
    dd = empty_dev(src.nbytes, 0x33)
    ms = encode(sd, "bf16", dims, (Wd * 2,), box, swizzle=swizzle)
    md = encode(dd, "bf16", dims, (Wd * 2,), box, swizzle=swizzle)
    att.tile_copy_ex(ms, md, stages, grid, variant, stream())
    torch.cuda.synchronize()
    same = torch.equal(sd, dd)
    return src, sd, dd, ms, same


@pytest.mark.parametrize("stages,variant", [(2, 0), (1, 0), (3, 0), (4, 0), (2, 1), (2, 2), (2, 65), (3, 65), (4, 73),
                                            (2, 64), (4, 201), (2, 193), (3, 193), (2, 321), (4, 457),
                                            (1, 513), (2, 513), (4, 512)])
def test_copy_8192_round_trip(stages, variant):
    ex = W.COPY_8192
    say("copy 8192^2 stages", stages, "variant", variant)
    src, sd, dd, ms, same = _copy_case(ex["dims"], ex["box"], ex["swizzle"], stages, variant)
    assert same, "destination differs from source"
    if stages == 2 and variant == 0:
        # sampled tiles: the LDS image the loader builds matches the oracle
        g = synthgen.rng(202)
        coords = np.stack([g.integers(0, 128, 64) * 64, g.integers(0, 64, 64) * 128], axis=1).astype(np.int32)
        out = empty_dev(64 * 16384, 0)
        att.tile_load(ms, to_dev(coords), 64, out, stream())
        om = oracle.Map("bf16", ex["dims"], ex["strides"], ex["box"], swizzle="128b")
        np.testing.assert_array_equal(to_host(out).reshape(64, 16384), om.load(src, coords))


@pytest.mark.parametrize("dims,box,swizzle", [
    ((1000, 777), (64, 128), "128b"),     # ragged in both dims: generic path with edge tiles
    ((8192, 640), (64, 128), "128b"),     # ring path, 5 row tiles
    ((2048, 512), (32, 64), "64b"),       # 4 KiB boxes (GPW = 1)
    ((4096, 256), (128, 128), "none"),    # 32 KiB boxes (GPW = 8)
])
def test_copy_other_shapes(dims, box, swizzle):
    say("copy", dims, box, swizzle)
    src, sd, dd, ms, same = _copy_case(dims, box, swizzle, 2, seed=12)
    assert same
    # the producer / consumer form (two boxes per workgroup where the box
    # size allows it, else the ring)
    src, sd, dd, ms, same = _copy_case(dims, box, swizzle, 2, 513, seed=13)
    assert same


def _tensor_byte_mask(c):
    """Bytes of the buffer that hold tensor elements (the rest is stride
    padding, which a round trip must leave alone)."""
    es = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8,
          "f16": 2, "bf16": 2, "f32": 4, "f64": 8}[c.dtype]
    mask = np.zeros(c.buf.size, dtype=bool)
    row = np.arange(c.dims[0] * es)
    idx = [np.arange(n) for n in c.dims[1:]]
    grids = np.meshgrid(*idx, indexing="ij") if idx else []
    offs = np.zeros(grids[0].shape if grids else (), dtype=np.int64)
    for d, gr in enumerate(grids):
        offs = offs + gr.astype(np.int64) * c.strides[d]
    for o in np.ravel(offs):
        mask[o + row] = True
    return mask


@pytest.mark.parametrize("seed", range(30))
def test_copy_random_maps(seed):
    """tile_copy_ex over random legal maps (ranks 1-5, every element type and
    swizzle, element strides 1) with random ring depth, grid and variant
    flags (stores, tile order, XCD renumbering, boxes per stage): every
    tensor byte arrives, stride padding in the destination is untouched."""
    from cases import random_case
    g = synthgen.rng(95000 + seed)
    c = random_case(g)
    c.estride = [1] * c.rank
    if c.swizzle == "none":
        c.box[0] = (16 // {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8, "f16": 2, "bf16": 2,
                           "f32": 4, "f64": 8}[c.dtype]) * int(g.integers(1, 4))
    else:
        es = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8, "f16": 2, "bf16": 2, "f32": 4, "f64": 8}
        c.box[0] = (16 << {"32b": 1, "64b": 2, "128b": 3}[c.swizzle.split("_")[0]]) // es[c.dtype]
    stages = int(g.choice([1, 2, 3, 4, 5, 6, 8]))
    variant = int(g.integers(0, 64))
    grid = int(g.choice([0, 0, 1, 3, 64, 1000]))
    if g.integers(0, 2):
        variant |= 64                      # batch mode (where the box count and depth allow it)
    if g.integers(0, 2):
        variant |= 128                     # row-group-major issue in batch mode
    if g.integers(0, 2):
        variant |= 256                     # batch mode through registers instead of the LDS-DMA
    if g.integers(0, 3) == 0:
        variant |= 512                     # producer / consumer form (where the box size allows it)
    say("copy random", seed, c.dtype, c.dims, c.box, c.swizzle, stages, variant, grid)
    sd = to_dev(c.buf)
    dd = empty_dev(c.buf.size, 0x5A)
    ms = encode(sd, c.dtype, c.dims, c.strides, c.box, None, c.swizzle)
    md = encode(dd, c.dtype, c.dims, c.strides, c.box, None, c.swizzle)
    att.tile_copy_ex(ms, md, stages, grid, variant, stream())
    torch.cuda.synchronize()
    got = to_host(dd)
    mask = _tensor_byte_mask(c)
    want = np.where(mask, c.buf, np.uint8(0x5A))
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("dims", [(8192, 8192), (8192, 640), (1984, 1408)])
def test_copy_default_entry(dims):
    """tile_copy, the launch the benchmark times (non-temporal stores, two
    boxes per workgroup, each box row walked from a rotated start), on the
    full workload and on shapes whose box-row count is below, or not a
    multiple of, the boxes per row."""
    ex = W.COPY_8192
    say("copy default entry", dims)
    H, Wd = dims[1], dims[0]
    src = synthgen.u16_bits(7, (H, Wd))
    sd = to_dev(src)
    dd = empty_dev(src.nbytes, 0x33)
    ms = encode(sd, "bf16", dims, (Wd * 2,), ex["box"], swizzle=ex["swizzle"])
    md = encode(dd, "bf16", dims, (Wd * 2,), ex["box"], swizzle=ex["swizzle"])
    att.tile_copy(ms, md, 2, stream())
    torch.cuda.synchronize()
    assert torch.equal(sd, dd)


def test_copy_grid_sweep_small():
    ex = W.COPY_8192
    for grid in (1, 255, 256, 1024, 4096):
        say("copy grid", grid)
        _, _, _, _, same = _copy_case((2048, 2048), ex["box"], ex["swizzle"], 2, 0, grid)
        assert same, grid


# ------------------------ rank-5 fp32 with edge boxes -----------------------

def _rank5(fill, pad, align0, seed_off=0):
    ex = W.RANK5
    dims = ex["dims"]
    strides, s = [], dims[0] * 4
    for i in range(1, 5):
        s = (s + 15) // 16 * 16 + pad
        strides.append(s)
        s *= dims[i]
    foot = strides[-1] * dims[-1]
    vals = synthgen.uniform_f32(ex["seed"] + seed_off, foot // 4)
    L = [32, 16, 8, 2, 1]
    coords = synthgen.edge_mix_coords(ex["seed"] * 1000 + seed_off, dims, L, ex["estride"], ex["nbox"],
                                      align0=align0)
    return dims, strides, vals, coords


@pytest.mark.parametrize("fill,pad,align0", [("zero", 0, 1), ("nan", 0, 1), ("zero", 16, 1), ("nan", 0, 4)])
def test_rank5_edge_boxes(fill, pad, align0):
    ex = W.RANK5
    dims, strides, vals, coords = _rank5(fill, pad, align0)
    say("rank5", fill, pad, align0, strides)
    assert strides[:1] == [1040 + pad]
    om = oracle.Map("f32", dims, strides, ex["box"], ex["estride"], ex["swizzle"], fill)
    assert om.validate() == "OK" and om.box_bytes() == 32768
    sd = to_dev(vals)
    m = encode(sd, "f32", dims, strides, ex["box"], ex["estride"], ex["swizzle"], fill)
    out = empty_dev(len(coords) * 32768, 0)
    att.tile_load(m, to_dev(coords), len(coords), out, stream())
    got = to_host(out).reshape(len(coords), 32768)
    want = om.load(vals, coords)
    np.testing.assert_array_equal(got, want)
    # a quarter of the boxes straddle an edge and hold fill bits
    fb = np.uint32(0x7FC00000 if fill == "nan" else 0)
    edge = got[3::4].view(np.uint32)
    assert (edge == fb).any(axis=1).all()
    # round trip through the store into a sentinel buffer
    dst = to_dev(np.full(vals.size, 0xDEADBEEF, dtype=np.uint32))
    md = encode(dst, "f32", dims, strides, ex["box"], ex["estride"], ex["swizzle"], fill)
    att.tile_store(md, to_dev(coords), len(coords), out, stream())
    hw = np.full(vals.size, 0xDEADBEEF, dtype=np.uint32)
    om.store(hw, coords, want)
    np.testing.assert_array_equal(to_host(dst).view(np.uint32), hw)


def test_rank5_fully_outside_boxes():
    ex = W.RANK5
    dims, strides, vals, _ = _rank5("nan", 0, 1)
    coords = np.array([[-40, 0, 0, 0, 0], [300, 0, 0, 0, 0], [0, -40, 0, 0, 0], [0, 0, 0, 0, 3],
                       [0, 0, 0, -2, 0]], dtype=np.int32)
    sd = to_dev(vals)
    m = encode(sd, "f32", dims, strides, ex["box"], ex["estride"], ex["swizzle"], "nan")
    out = empty_dev(len(coords) * 32768, 0)
    att.tile_load(m, to_dev(coords), len(coords), out, stream())
    assert (to_host(out).view(np.uint32) == 0x7FC00000).all()


# ------------------------------ reduce-add ----------------------------------

def test_reduce_int32_four_passes():
    ex = W.REDUCE_4096
    dst0 = synthgen.int32_range(ex["seed"], (4096, 4096), -(1 << 20), 1 << 20)
    dd = to_dev(dst0)
    m = encode(dd, "i32", ex["dims"], ex["strides"], ex["box"])
    om = oracle.Map("i32", ex["dims"], ex["strides"], ex["box"])
    hw = dst0.copy()
    for p in range(ex["passes"]):
        say("reduce int32 pass", p)
        coords = synthgen.uniform_coords(ex["seed"] * 1000 + 10 + p, ex["nbox"], (0, 0), (4032, 4032))
        srcs = synthgen.int32_range(ex["seed"] * 1000 + 20 + p, (ex["nbox"], 64, 64), -(1 << 20), 1 << 20)
        att.tile_reduce_add(m, to_dev(coords), ex["nbox"], to_dev(srcs), stream())
        om.reduce_add(hw, coords, srcs.view(np.uint8))
    got = to_host(dd).view(np.int32).reshape(4096, 4096)
    np.testing.assert_array_equal(got, hw)
    # checksum invariant: total added equals the sum of all sources (mod 2^32)
    assert int(got.astype(np.int64).sum() - dst0.astype(np.int64).sum()) == int(
        hw.astype(np.int64).sum() - dst0.astype(np.int64).sum())


def test_reduce_f32_four_passes_within_tolerance():
    """fp32 with N(0,1) values: |gpu - exact| <= 1e-6 * (sum of |contributions|)
    per element (order of concurrent additions is unspecified)."""
    ex = W.REDUCE_4096
    dst0 = synthgen.normal_f32(ex["seed"] + 100, (4096, 4096))
    dd = to_dev(dst0)
    m = encode(dd, "f32", ex["dims"], ex["strides"], ex["box"])
    om = oracle.Map("f32", ex["dims"], ex["strides"], ex["box"])
    acc = dst0.astype(np.float64).reshape(-1).copy()
    mag = np.abs(acc)
    for p in range(ex["passes"]):
        say("reduce f32 pass", p)
        coords = synthgen.uniform_coords(ex["seed"] * 1000 + 30 + p, ex["nbox"], (0, 0), (4032, 4032))
        srcs = synthgen.normal_f32(ex["seed"] * 1000 + 40 + p, (ex["nbox"], 64, 64))
        att.tile_reduce_add(m, to_dev(coords), ex["nbox"], to_dev(srcs), stream())
        om.reduce_add_f64(acc, mag, coords, srcs.view(np.uint8))
    got = to_host(dd).view(np.float32).astype(np.float64)
    err = np.abs(got - acc)
    assert np.isfinite(got).all()
    assert (err <= 1e-6 * mag).all(), float((err / np.maximum(mag, 1e-300)).max())


# ------------------------------ reduce min / max ----------------------------

@pytest.mark.parametrize("op", ["min", "max"])
@pytest.mark.parametrize("dtype", ["i32", "f32", "bf16", "u16"])
def test_reduce_minmax_four_passes(dtype, op):
    """The 4096^2 reduce workload with min / max instead of add: four passes of
    1024 overlapping 64x64 boxes; integers from the workload's range, floats as
    random bit patterns (NaNs, infinities, both zeros).  Bit-exact."""
    ex = W.REDUCE_4096
    es = {"i32": 4, "f32": 4, "bf16": 2, "u16": 2}[dtype]
    dims = (4096, 4096)
    strides = (4096 * es,)
    box = (64, 64)
    if dtype == "i32":
        dst0 = synthgen.int32_range(ex["seed"], (4096, 4096), -(1 << 20), 1 << 20).view(np.uint8).reshape(-1)
    else:
        dst0 = synthgen.random_bytes(ex["seed"] * 7 + es, 4096 * 4096 * es)
    acc = to_dev(dst0)
    m = att.tmap_encode(dtype, 2, acc.data_ptr(), dims, strides, box, None, "none")
    om = oracle.Map(dtype, dims, strides, box, swizzle="none")
    hw = dst0.copy()
    for p in range(4):
        say("reduce", op, dtype, "pass", p)
        coords = synthgen.uniform_coords(ex["seed"] * 1000 + 10 + p, ex["nbox"], (0, 0), (4032, 4032))
        if dtype == "i32":
            srcs = synthgen.int32_range(ex["seed"] * 1000 + 20 + p, (ex["nbox"], 64, 64), -(1 << 20), 1 << 20)
            srcs = srcs.view(np.uint8).reshape(-1)
        else:
            srcs = synthgen.random_bytes(ex["seed"] * 1000 + 30 + p, ex["nbox"] * 64 * 64 * es)
        att.tile_reduce(m, op, to_dev(coords), ex["nbox"], to_dev(srcs), stream())
        om.reduce(hw, coords, srcs, op)
    np.testing.assert_array_equal(to_host(acc), hw)
