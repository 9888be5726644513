"""GPU parity: the HIP tile loader / storer / reducer against the CPU oracle,
element by element on the same seeded inputs (bit-exact for all moves and
integer reductions).  Every call goes through the C ABI."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
from synthgen import workloads as W  # noqa: E402

from cases import ESIZE, random_case, sweep_coords  # noqa: E402
from gpu_util import empty_dev, encode, require_native, stream, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_load(c, buf_dev, coords):
    m = encode(buf_dev, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    bb = att.tmap_box_bytes(m)
    cd = to_dev(np.ascontiguousarray(coords, dtype=np.int32))
    out = empty_dev(bb * len(coords), 0x5A)
    att.tile_load(m, cd, len(coords), out, stream())
    return to_host(out).reshape(len(coords), bb), m


# ----------------------------- worked examples ------------------------------

@pytest.mark.parametrize("mode", ["none", "128b"])
def test_example_2d(mode, table):
    """[MLC] 16x128 fp16 tensor, 8x64 box at (row 0, col 0) and (row 8, col 64)."""
    ex = W.EXAMPLE_2D
    src = synthgen.u16_bits(ex["seed"], (16, 128))
    sd = to_dev(src)
    m = encode(sd, "f16", ex["dims"], ex["strides"], ex["box"], swizzle=mode)
    coords = np.array(ex["coords"], dtype=np.int32)
    out = empty_dev(2 * 1024, 0)
    att.tile_load(m, to_dev(coords), 2, out, stream())
    got = to_host(out).reshape(2, 1024)
    om = oracle.Map("f16", ex["dims"], ex["strides"], ex["box"], swizzle=mode)
    np.testing.assert_array_equal(got, om.load(src, coords))
    # the page's own table, independently of the oracle
    for b, (c0, c1) in enumerate(coords):
        img = got[b].view(np.uint16).reshape(8, 8, 8)
        for rec in table("mlc_example_2d_sectors.txt"):
            if rec[0] != mode:
                continue
            r = int(rec[1])
            for p in range(8):
                lg = int(rec[2 + p])
                np.testing.assert_array_equal(img[r, p], src[c1 + r, c0 + 8 * lg: c0 + 8 * lg + 8])
    # round trip LDS -> global into a sentinel buffer
    dst = to_dev(np.full((16, 128), 0xDEAD, dtype=np.uint16))
    md = encode(dst, "f16", ex["dims"], ex["strides"], ex["box"], swizzle=mode)
    att.tile_store(md, to_dev(coords), 2, out, stream())
    want = np.full((16, 128), 0xDEAD, dtype=np.uint16)
    om.store(want, coords, got)
    np.testing.assert_array_equal(to_host(dst).view(np.uint16).reshape(16, 128), want)


def test_example_3d_four_atoms(table):
    """[MLC] (group=2, row=16, col=64) view of a 16x256 fp16 matrix."""
    ex = W.EXAMPLE_3D
    src = synthgen.u16_bits(ex["seed"], (16, 256))
    sd = to_dev(src)
    m = encode(sd, "f16", ex["dims"], ex["strides"], ex["box"], swizzle="128b")
    coords = np.array(ex["coords"], dtype=np.int32)
    out = empty_dev(2 * 4096, 0)
    att.tile_load(m, to_dev(coords), 2, out, stream())
    got = to_host(out).reshape(2, 4096)
    om = oracle.Map("f16", ex["dims"], ex["strides"], ex["box"], swizzle="128b")
    np.testing.assert_array_equal(got, om.load(src, coords))
    for rec in table("mlc_example_3d_atoms.txt"):
        off, grp, row, p, grow, gcol = map(int, rec)
        img = got[off // 128]
        lds = grp * 2048 + row * 128 + p * 16
        np.testing.assert_array_equal(img[lds:lds + 16].view(np.uint16), src[grow, gcol:gcol + 8])


def test_bank_sector_probe(table):
    """[MLC] grouping requirement: sector histograms of the device's
    swizzled addresses, grouped and 256-byte-stride layouts."""
    for layout in (0, 1):
        h = empty_dev(9 * 16 * 8 * 4, 0)
        att.lds_bank_probe(layout, 4, h, stream())
        got = to_host(h).view(np.int32).reshape(9, 16, 8)
        for row0 in range(9):
            for col in range(16):
                want = oracle.bank_sector_hist(layout == 1, row0, col)
                assert got[row0, col].tolist() == want, (layout, row0, col)


@pytest.mark.parametrize("layout,mode", [(2, "128b"), (3, "128b_k256")])
def test_bank_probe_mfma_fragment_addresses(layout, mode):
    """The fragment read addresses the device generates equal the oracle's
    swizzle of (row l % 32, chunk l / 32) in a 128-byte-row box."""
    h = empty_dev(65 * 4, 0)
    att.lds_bank_probe(layout, 4, h, stream())
    got = to_host(h).view(np.int32)[:64]
    want = [oracle.swizzle((l % 32) * 128 + (l // 32) * 16, mode) for l in range(64)]
    assert got.tolist() == want


@pytest.mark.parametrize("layout,mode", [(4, "128b_k256"), (5, "128b_k256"), (6, "128b")])
def test_bank_probe_c_staging_addresses(layout, mode):
    """The GEMM epilogue's C staging addresses replayed by the probe equal the
    oracle's swizzle: 8-byte writes at (row l % 16, column 4 (l / 16)) and
    16-byte reads at (row l / 8, chunk l % 8) of a 128-byte-row image."""
    h = empty_dev(65 * 4, 0)
    att.lds_bank_probe(layout, 4, h, stream())
    got = to_host(h).view(np.int32)[:64]
    if layout == 5:
        want = [oracle.swizzle((l // 8) * 128 + (l % 8) * 16, mode) for l in range(64)]
    else:
        want = [oracle.swizzle((l % 16) * 128 + (l // 16) * 8, mode) for l in range(64)]
    assert got.tolist() == want


def test_txbar_4096_bytes(table):
    """[MLC] waiting for a TMA load: two 2048-byte tiles complete one phase
    with expect_tx(4096); states replayed on the oracle barrier model."""
    src = synthgen.u16_bits(7, (64, 64))
    sd = to_dev(src)
    m = encode(sd, "bf16", (64, 64), (128,), (64, 16), swizzle="128b")
    assert att.tmap_box_bytes(m) == 2048
    coords = np.array([[0, 0], [0, 16]], dtype=np.int32)
    trace = empty_dev(4 * 4 * 4, 0xFF)
    out = empty_dev(2 * 2048, 0)
    att.txbar_selftest(m, to_dev(coords), 2, trace, out, stream())
    tr = to_host(trace).view(np.int32).reshape(4, 4)
    ob = oracle.Txbar(1)
    assert tuple(tr[0]) == (-1,) + ob.state()
    ob.arrive_expect_tx(4096)
    assert tuple(tr[1]) == (-2,) + ob.state() == (-2, 0, 4096, 0)
    seen = set()
    for rec in tr[2:]:
        t = int(rec[0])
        assert t in (0, 1) and t not in seen
        seen.add(t)
        ob.complete_tx(2048)
        assert tuple(int(x) for x in rec[1:]) == ob.state()
    assert ob.try_wait(0) and tuple(tr[3, 1:]) == (1, 0, 1)
    om = oracle.Map("bf16", (64, 64), (128,), (64, 16), swizzle="128b")
    np.testing.assert_array_equal(to_host(out).reshape(2, 2048), om.load(src, coords))


@pytest.mark.parametrize("ntile", [1, 3, 8])
def test_txbar_several_tiles(ntile):
    src = synthgen.u16_bits(8, (128, 64))
    sd = to_dev(src)
    m = encode(sd, "bf16", (64, 128), (128,), (64, 16), swizzle="128b")
    coords = np.array([[0, 16 * t] for t in range(ntile)], dtype=np.int32)
    trace = empty_dev(4 * 4 * (2 + ntile), 0xFF)
    out = empty_dev(ntile * 2048, 0)
    att.txbar_selftest(m, to_dev(coords), ntile, trace, out, stream())
    tr = to_host(trace).view(np.int32).reshape(2 + ntile, 4)
    ob = oracle.Txbar(1)
    ob.arrive_expect_tx(2048 * ntile)
    # Copies complete concurrently and take their trace slot after their
    # barrier operation, so slots need not follow operation order; each
    # operation's own state is exact, and the pending count orders them.
    recs = sorted((tuple(int(x) for x in r[1:]) for r in tr[2:]),
                  key=lambda s: (s[2], -s[1]))
    want = []
    for _ in range(ntile):
        ob.complete_tx(2048)
        want.append(ob.state())
    assert recs == sorted(want, key=lambda s: (s[2], -s[1]))
    assert sorted(tr[2:, 0].tolist()) == list(range(ntile))
    om = oracle.Map("bf16", (64, 128), (128,), (64, 16), swizzle="128b")
    np.testing.assert_array_equal(to_host(out).reshape(ntile, 2048), om.load(src, coords))


def test_txbar_timeout_is_reported():
    """A barrier expecting 16 bytes more than its copies deliver never
    completes; its bounded wait gives up after a host-chosen 64 polls, the
    kernel exits normally, and tile_device_status reports ERR_TIMEOUT once
    (the record is cleared by reading it).  The copies themselves land."""
    att.tile_device_status(stream())                    # nothing recorded yet
    src = synthgen.u16_bits(9, (64, 64))
    sd = to_dev(src)
    m = encode(sd, "bf16", (64, 64), (128,), (64, 16), swizzle="128b")
    coords = np.array([[0, 0], [0, 16]], dtype=np.int32)
    trace = empty_dev(4 * 4 * 4, 0xFF)
    out = empty_dev(2 * 2048, 0)
    att.txbar_selftest_ex(m, to_dev(coords), 2, 16, 64, trace, out, stream())
    with pytest.raises(att.TmapError) as ei:
        att.tile_device_status(stream())
    assert ei.value.name == "ERR_TIMEOUT"
    att.tile_device_status(stream())                    # cleared
    tr = to_host(trace).view(np.int32).reshape(4, 4)
    assert tuple(tr[1]) == (-2, 0, 4096 + 16, 0)
    assert sorted(int(r[2]) for r in tr[2:]) == [16, 2064] and (tr[2:, 3] == 0).all()
    om = oracle.Map("bf16", (64, 64), (128,), (64, 16), swizzle="128b")
    np.testing.assert_array_equal(to_host(out).reshape(2, 2048), om.load(src, coords))
    # a good run afterwards records nothing
    att.txbar_selftest(m, to_dev(coords), 2, trace, out, stream())
    att.tile_device_status(stream())
    with pytest.raises(att.TmapError) as ei:
        att.txbar_selftest_ex(m, to_dev(coords), 2, 0, 0, trace, out, stream())
    assert ei.value.name == "ERR_UNSUPPORTED"


# --------------------------- brute force, tiny ------------------------------

@pytest.mark.parametrize("seed", range(40))
def test_random_maps_load_store_reduce(seed):
    """Ranks 1-5, all element types, all swizzles, element strides 1-3,
    origins sweeping from below to above every dimension."""
    g = synthgen.rng(20000 + seed)
    c = random_case(g)
    coords = sweep_coords(g, c, 24)
    say("case", seed, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    om = oracle.Map(c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    assert om.validate() == "OK"
    sd = to_dev(c.buf)
    got, m = gpu_load(c, sd, coords)
    want = om.load(c.buf, coords)
    np.testing.assert_array_equal(got, want)
    # store the loaded images into a sentinel buffer: overlapping boxes write
    # identical values, so the result is unique
    dst = to_dev(np.full(c.buf.size, 0xA5, dtype=np.uint8))
    md = encode(dst, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    att.tile_store(md, to_dev(coords), len(coords), to_dev(got), stream())
    hw = np.full(c.buf.size, 0xA5, dtype=np.uint8)
    om.store(hw, coords, want)
    np.testing.assert_array_equal(to_host(dst), hw)
    # reduce-add of random images (integer types: order-free, bit-exact)
    if c.dtype not in ("f16", "bf16", "f32", "f64"):
        imgs = synthgen.random_bytes(seed + 7, got.size).reshape(got.shape)
        acc = to_dev(c.buf)
        ma = encode(acc, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, "zero")
        att.tile_reduce_add(ma, to_dev(coords), len(coords), to_dev(imgs), stream())
        hw = c.buf.copy()
        oracle.Map(c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle).reduce_add(hw, coords, imgs)
        np.testing.assert_array_equal(to_host(acc)[: c.buf.size], hw)
    # reduce min / max of random bit patterns (NaNs and signed zeros in the
    # float types): order-free, bit-exact for every type
    imgs = synthgen.random_bytes(seed + 11, got.size).reshape(got.shape)
    for op in ("min", "max"):
        acc = to_dev(c.buf)
        ma = encode(acc, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, "zero")
        att.tile_reduce(ma, op, to_dev(coords), len(coords), to_dev(imgs), stream())
        hw = c.buf.copy()
        oracle.Map(c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle).reduce(hw, coords, imgs, op)
        np.testing.assert_array_equal(to_host(acc)[: c.buf.size], hw, err_msg=op)


@pytest.mark.parametrize("dtype", ["u8", "u16", "f16", "bf16", "u32", "i32", "f32", "u64", "i64", "f64"])
@pytest.mark.parametrize("rank", [1, 2])
@pytest.mark.parametrize("seed", range(6))
def test_reduce_rank12_edges(dtype, rank, seed):
    """Reductions on rank-1 and rank-2 maps with element stride 1 in dim 0,
    the paths that locate a box's rows with one multiply-high (8- and 16-bit
    elements also work out the elements inside the tensor once per box):
    origins from fully below to fully above both dimensions, element strides
    1-3 in dim 1, odd and even dim-0 origins (for 8- and 16-bit elements,
    words cut by the box row's ends).  Integer add, and min / max of every
    type (NaNs and signed zeros among the random bit patterns), bit-exact
    against the oracle."""
    types = ["u8", "u16", "f16", "bf16", "u32", "i32", "f32", "u64", "i64", "f64"]
    g = synthgen.rng(30000 + 1000 * types.index(dtype) + 100 * rank + seed)
    while True:
        c = random_case(g, dtype=dtype, rank=rank)
        if c.estride[0] == 1:
            break
    coords = sweep_coords(g, c, 32)
    say("case", dtype, rank, seed, c.dims, c.strides, c.box, c.estride, c.swizzle)
    om = oracle.Map(c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle)
    assert om.validate() == "OK"
    probe = encode(to_dev(c.buf), c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, "zero")
    bb = att.tmap_box_bytes(probe)
    imgs = synthgen.random_bytes(seed + 40 * rank + 3, len(coords) * bb).reshape(len(coords), bb)
    ops = (["add"] if dtype not in ("f16", "bf16", "f32", "f64") else []) + ["min", "max"]
    for op in ops:
        acc = to_dev(c.buf)
        ma = encode(acc, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, "zero")
        att.tile_reduce(ma, op, to_dev(coords), len(coords), to_dev(imgs), stream())
        hw = c.buf.copy()
        if op == "add":
            om.reduce_add(hw, coords, imgs)
        else:
            om.reduce(hw, coords, imgs, op)
        np.testing.assert_array_equal(to_host(acc)[: c.buf.size], hw, err_msg=op)


@pytest.mark.parametrize("dtype", ["u8", "u16", "f16", "bf16", "u32", "i32", "f32", "u64", "i64", "f64"])
@pytest.mark.parametrize("rank", [1, 2, 3])
@pytest.mark.parametrize("seed", range(3))
def test_store_rows_at_any_alignment(dtype, rank, seed):
    """Plain stores on maps with element stride 1 in dim 0, whose boxes
    start anywhere in a row (rows not on a 16-byte boundary take one element
    per lane): random images, one box per call so that overlapping boxes
    end with the later one, against the oracle's stores in the same order
    on a sentinel buffer (bytes outside every box untouched)."""
    types = ["u8", "u16", "f16", "bf16", "u32", "i32", "f32", "u64", "i64", "f64"]
    g = synthgen.rng(40000 + 1000 * types.index(dtype) + 100 * rank + seed)
    while True:
        c = random_case(g, dtype=dtype, rank=rank)
        if c.estride[0] == 1:
            break
    coords = sweep_coords(g, c, 24)
    say("case", dtype, rank, seed, c.dims, c.strides, c.box, c.estride, c.swizzle)
    om = oracle.Map(c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    assert om.validate() == "OK"
    dst = to_dev(np.full(c.buf.size, 0xA5, dtype=np.uint8))
    md = encode(dst, c.dtype, c.dims, c.strides, c.box, c.estride, c.swizzle, c.fill)
    bb = att.tmap_box_bytes(md)
    imgs = synthgen.random_bytes(seed + 50 * rank + 5, len(coords) * bb).reshape(len(coords), bb)
    cd, di = to_dev(coords), to_dev(imgs)
    for i in range(len(coords)):
        att.tile_store(md, cd[i * rank * 4:], 1, di[i * bb:], stream())
    hw = np.full(c.buf.size, 0xA5, dtype=np.uint8)
    om.store(hw, coords, imgs)
    np.testing.assert_array_equal(to_host(dst), hw)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32", "f64"])
def test_float_reduce_single_contribution_exact(dtype):
    """Non-overlapping boxes: one IEEE addition per element, rounded once;
    bit-exact against the oracle."""
    es = ESIZE[dtype]
    L0 = 64 // es
    dims, strides, box = (4 * L0, 24), (4 * L0 * es + 32,), (L0, 8)
    foot = strides[0] * dims[1]
    g = synthgen.rng(31)
    if dtype == "bf16":
        dst0 = synthgen.normal_bf16_bits(32, foot // 2).view(np.uint8)
        imgs = synthgen.normal_bf16_bits(33, (12, L0 * 8)).view(np.uint8)
    else:
        npt = {"f16": np.float16, "f32": np.float32, "f64": np.float64}[dtype]
        dst0 = g.standard_normal(foot // es).astype(npt).view(np.uint8)
        imgs = (g.standard_normal((12, L0 * 8)) * 4).astype(npt).view(np.uint8)
    coords = np.array([[L0 * (i % 4), 8 * (i // 4)] for i in range(12)], dtype=np.int32)
    acc = to_dev(dst0)
    m = encode(acc, dtype, dims, strides, box)
    att.tile_reduce_add(m, to_dev(coords), 12, to_dev(imgs), stream())
    hw = dst0.copy()
    oracle.Map(dtype, dims, strides, box).reduce_add(hw, coords, imgs)
    np.testing.assert_array_equal(to_host(acc), hw)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("layout", ["aligned", "even_origin_edge", "odd_origin_edges"])
def test_half_reduce_special_values_exact(dtype, layout):
    """16-bit float reduce-add with random bit patterns on both sides (NaNs
    with payloads, infinities of both signs, subnormals, signed zeros): one
    contribution per element, bit-exact against the oracle, canonical NaN
    results included.  Word-aligned boxes take the packed hardware add for
    whole words; odd origins and boxes cut by the dim-0 edge also take the
    per-word compare-and-swap."""
    L0 = 32
    dims, strides, box = (133, 24), (288,), (L0, 8)     # odd width: a word cut by the edge
    foot = strides[0] * dims[1]
    dst0 = synthgen.random_bytes(41, foot)
    imgs = synthgen.random_bytes(42, 12 * L0 * 8 * 2)
    # disjoint boxes in every layout
    xs = {"aligned": [0, 32, 64, 96],                   # whole words only
          "even_origin_edge": [-6, 34, 70, 104],        # crossing x = 0 and x = 133
          "odd_origin_edges": [-7, 27, 59, 117]}[layout]
    coords = np.array([[xs[i % 4], 8 * (i // 4)] for i in range(12)], dtype=np.int32)
    acc = to_dev(dst0)
    m = encode(acc, dtype, dims, strides, box)
    att.tile_reduce_add(m, to_dev(coords), 12, to_dev(imgs), stream())
    hw = dst0.copy()
    oracle.Map(dtype, dims, strides, box).reduce_add(hw, coords, imgs)
    np.testing.assert_array_equal(to_host(acc), hw)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_half_reduce_odd_origins_keep_neighbours(dtype):
    """16-bit reduce-add at odd origins: the words at each box row's ends
    take the packed add with -0 in the half outside the box.  Every element
    outside the boxes holds a signalling NaN, a quiet non-canonical NaN, -0
    or a subnormal, and must keep its bits; inside, bit-exact against the
    oracle."""
    dims, strides, box = (133, 16), (288,), (32, 8)
    g = synthgen.rng(43)
    snan, qnan = (0x7F81, 0xFFC3) if dtype == "bf16" else (0x7C01, 0xFE03)
    pats = np.array([snan, qnan, 0x8000, 0x0001], dtype=np.uint16)
    dst0 = pats[g.integers(0, 4, strides[0] * dims[1] // 2)]
    imgs = synthgen.normal_bf16_bits(44, (8, 32 * 8)) if dtype == "bf16" else \
        g.standard_normal((8, 32 * 8)).astype(np.float16).view(np.uint16)
    coords = np.array([[1, 0], [35, 0], [69, 0], [101, 0], [-3, 8], [33, 8], [67, 8], [103, 8]], dtype=np.int32)
    acc = to_dev(dst0)
    m = encode(acc, dtype, dims, strides, box)
    att.tile_reduce_add(m, to_dev(coords), 8, to_dev(imgs), stream())
    hw = dst0.view(np.uint8).copy()
    oracle.Map(dtype, dims, strides, box).reduce_add(hw, coords, imgs.view(np.uint8))
    np.testing.assert_array_equal(to_host(acc).view(np.uint16), hw.view(np.uint16))


def _float_class_mix(dtype, n, seed):
    """n f32 / f64 bit patterns, each drawn from one of thirteen classes
    picked uniformly: random bits, +0, -0, subnormals, the smallest normal,
    values around the size below which the library's add leaves the
    hardware atomic (exponent field p .. p + 4), small and ordinary normals,
    +inf, -inf, the canonical quiet NaN, NaNs with random payloads (quiet and
    signalling, either sign), the largest finite value."""
    ut, ft, mb, ew = {"f32": (np.uint32, np.float32, 23, 8), "f64": (np.uint64, np.float64, 52, 11)}[dtype]
    emax = (1 << ew) - 1
    U = np.uint64
    g = synthgen.rng(seed)
    cls = g.integers(0, 13, n)
    sign = g.integers(0, 2, n, dtype=np.uint64) << U(mb + ew)
    man = g.integers(0, 1 << mb, n, dtype=np.uint64)
    exp_near = g.integers(mb + 1, mb + 6, n, dtype=np.uint64)
    exp_small = g.integers(1, 40, n, dtype=np.uint64)
    raw = g.integers(0, 1 << (mb + ew + 1), n, dtype=np.uint64) if dtype == "f32" else \
        g.integers(0, np.iinfo(np.uint64).max, n, dtype=np.uint64, endpoint=True)
    ordinary = g.standard_normal(n).astype(ft).view(ut).astype(np.uint64)
    one = np.ones(n, dtype=np.uint64)
    top = U(emax) << U(mb)
    choices = [raw, np.zeros(n, np.uint64), U(1) << U(mb + ew) | np.zeros(n, np.uint64),
               sign | np.maximum(man, one), sign | (U(1) << U(mb)), sign | (exp_near << U(mb)) | man,
               sign | (exp_small << U(mb)) | man, ordinary, top | np.zeros(n, np.uint64),
               (U(1) << U(mb + ew)) | top, top | (U(1) << U(mb - 1)), sign | top | np.maximum(man, one),
               sign | (U(emax - 1) << U(mb)) | U((1 << mb) - 1)]
    out = np.choose(cls, choices)
    return out.astype(ut)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("layout", ["aligned", "edges"])
def test_float_reduce_special_values_exact(dtype, layout):
    """f32 / f64 reduce-add with operands of every class on both sides
    (subnormals, signed zeros, infinities, NaN payloads, values at the size
    where the add leaves the hardware atomic), one contribution per element:
    IEEE addition rounded to nearest even, bit-exact against the oracle; a
    NaN result must be a NaN (IEEE 754 leaves its payload open)."""
    es = ESIZE[dtype]
    L0 = 128 // es
    dims = (4 * L0 + 5, 24)
    strides = ((dims[0] * es + 15) // 16 * 16,)
    box = (L0, 8)
    ut = np.uint32 if dtype == "f32" else np.uint64
    foot = strides[0] * dims[1]
    dst0 = _float_class_mix(dtype, foot // es, 71).view(np.uint8)
    imgs = _float_class_mix(dtype, 12 * L0 * 8, 72).view(np.uint8)
    xs = {"aligned": [0, L0, 2 * L0, 3 * L0], "edges": [-3, L0 - 3, 2 * L0 + 1, 3 * L0 + 9]}[layout]
    coords = np.array([[xs[i % 4], 8 * (i // 4)] for i in range(12)], dtype=np.int32)
    acc = to_dev(dst0)
    m = encode(acc, dtype, dims, strides, box)
    att.tile_reduce_add(m, to_dev(coords), 12, to_dev(imgs), stream())
    hw = dst0.copy()
    oracle.Map(dtype, dims, strides, box).reduce_add(hw, coords, imgs)
    got = to_host(acc).view(ut)
    want = hw.view(ut)
    ft = np.float32 if dtype == "f32" else np.float64
    want_nan = np.isnan(want.view(ft))
    assert (np.isnan(got.view(ft)) == want_nan).all()
    np.testing.assert_array_equal(got[~want_nan], want[~want_nan])
    # the mix really reaches the cases the CAS path serves
    assert (want.view(ft)[~want_nan] != 0).any() and want_nan.any()


# ------------------------------- edge cases ---------------------------------

def test_empty_and_fully_outside():
    src = synthgen.u16_bits(3, (32, 64))
    sd = to_dev(src)
    m = encode(sd, "bf16", (64, 32), (128,), (64, 8), swizzle="128b", fill="nan")
    att.tile_load(m, 0, 0, 0, stream())        # nbox == 0: no launch
    coords = np.array([[-64, 0], [64, 0], [0, -8], [0, 32], [-1000, -1000]], dtype=np.int32)
    out = empty_dev(5 * 1024, 0)
    att.tile_load(m, to_dev(coords), 5, out, stream())
    got = to_host(out).view(np.uint16)
    assert (got == 0x7FC0).all()
    dst = to_dev(src)
    att.tile_store(encode(dst, "bf16", (64, 32), (128,), (64, 8), swizzle="128b"), to_dev(coords), 5,
                   to_dev(np.zeros(5 * 1024, np.uint8)), stream())
    np.testing.assert_array_equal(to_host(dst).view(np.uint16).reshape(32, 64), src)


def test_maximum_box():
    """Largest box a map may describe (162816 bytes: 32 x 159 x 8 fp32)."""
    dims, strides, box = (32, 159, 9), (128, 128 * 159), (32, 159, 8)
    src = synthgen.uniform_f32(5, (9, 159, 32))
    om = oracle.Map("f32", dims, strides, box, swizzle="128b")
    assert om.validate() == "OK" and om.box_bytes() == 162816
    sd = to_dev(src)
    m = encode(sd, "f32", dims, strides, box, swizzle="128b")
    coords = np.array([[0, 0, 0], [0, 0, 1], [3, -5, 2]], dtype=np.int32)
    out = empty_dev(3 * 162816, 0)
    att.tile_load(m, to_dev(coords), 3, out, stream())
    np.testing.assert_array_equal(to_host(out).reshape(3, -1), om.load(src, coords))


def test_rank1_and_u8_extremes():
    buf = synthgen.random_bytes(9, 1000 + 16)
    for box in (16, 256):
        c = np.array([[-300], [-17], [0], [1], [15], [500], [999], [1000]], dtype=np.int32)
        om = oracle.Map("u8", (1000,), (), (box,))
        sd = to_dev(buf)
        m = encode(sd, "u8", (1000,), (), (box,))
        out = empty_dev(len(c) * box, 0)
        att.tile_load(m, to_dev(c), len(c), out, stream())
        np.testing.assert_array_equal(to_host(out).reshape(len(c), box), om.load(buf, c))
