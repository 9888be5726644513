"""Pins for the CPU oracle: each test ties an oracle routine to something other
than itself -- a worked example printed on the reference pages, an independent
NumPy formulation, a library routine, a closed form or an invariant -- so that
a dropped term, a wrong sign or index, or a transposed operand fails here.

Page keys: [MLC] Modern GPU Programming for MLSys (zh), chapter "TMA";
[H200] blog.coolgpu.cn "H200 // TMA" feature card; [HPC] gpu-hpc-book ch. 08.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synthgen
from synthgen import workloads as W

NP_BITS = {1: np.uint8, 2: np.uint16, 4: np.uint32, 8: np.uint64}
NAN_BITS = {"f32": 0x7FC00000, "f16": 0x7E00, "bf16": 0x7FC0, "f64": 0x7FF8000000000000}


# ---------------------------------------------------------------------------
# An independent formulation of the NONE-swizzle load: view the tensor through
# NumPy strides, pad with the fill pattern, take a strided slice per
# dimension and flatten innermost-fastest.  Shares nothing with oracle.c.
# ---------------------------------------------------------------------------

def np_tensor_view(buf: np.ndarray, dtype: str, dims, strides):
    es = oracle.ESIZE[dtype]
    shape = tuple(int(d) for d in reversed(dims))
    st = tuple(reversed((es,) + tuple(int(s) for s in strides)))
    return np.lib.stride_tricks.as_strided(buf.view(NP_BITS[es]), shape=shape, strides=st)


def np_load_none(buf, dtype, dims, strides, box, estride, coords, fill):
    es = oracle.ESIZE[dtype]
    rank = len(dims)
    view = np.array(np_tensor_view(buf, dtype, dims, strides))
    L = [math.ceil(box[i] / estride[i]) for i in range(rank)]
    fb = NAN_BITS[dtype] if fill == "nan" else 0
    pads, sls = [], []
    for i in reversed(range(rank)):
        first = int(coords[i])
        last = first + (L[i] - 1) * estride[i]
        lo = max(0, -first)
        hi = max(0, last + 1 - int(dims[i]))
        pads.append((lo, hi))
        sls.append(slice(first + lo, last + lo + 1, estride[i]))
    padded = np.pad(view, pads, mode="constant", constant_values=NP_BITS[es](fb))
    return np.ascontiguousarray(padded[tuple(sls)]).reshape(-1).view(np.uint8)


def page_swizzle_128b(image: np.ndarray) -> np.ndarray:
    """[MLC] swizzled layout: in each 128-byte row r, logical sector c goes to
    physical sector c XOR (r % 8)."""
    rows = image.reshape(-1, 8, 16)
    out = np.empty_like(rows)
    for r in range(rows.shape[0]):
        for c in range(8):
            out[r, c ^ (r % 8)] = rows[r, c]
    return out.reshape(-1)


def random_case(g: np.random.Generator, swizzle_choice=None):
    """A small random legal map plus a buffer that covers its footprint."""
    dtype = g.choice(list(oracle.ESIZE))
    es = oracle.ESIZE[dtype]
    rank = int(g.integers(1, 6))
    sw = swizzle_choice if swizzle_choice is not None else g.choice(["none", "32b", "64b", "128b", "32b_k256",
                                                                     "64b_k256", "128b_k256"])
    estride = [int(g.integers(1, 4)) for _ in range(rank)]
    if sw == "none":
        L0 = (16 // es) * int(g.integers(1, 4))
    else:
        L0 = (16 << {"32b": 1, "64b": 2, "128b": 3}[str(sw).split("_")[0]]) // es
    # choose box0 with ceil(box0 / estride0) == L0
    box0 = (L0 - 1) * estride[0] + int(g.integers(1, estride[0] + 1))
    if box0 * es % 16 != 0 or box0 > 256:
        estride[0] = 1
        box0 = L0
    box = [box0] + [int(g.integers(1, 7)) for _ in range(rank - 1)]
    dims = [int(g.integers(1, 3 * max(box0, 4)))] + [int(g.integers(1, 12)) for _ in range(rank - 1)]
    strides, s = [], dims[0] * es
    for i in range(1, rank):
        s = (s + 15) // 16 * 16 + 16 * int(g.integers(0, 2))
        strides.append(s)
        s = s * dims[i]
    foot = (dims[0] * es if rank == 1 else strides[-1] * dims[-1]) + 64
    buf = synthgen.random_bytes(int(g.integers(0, 1 << 30)), foot)
    fill = "nan" if dtype in NAN_BITS and g.integers(0, 2) else "zero"
    coords = []
    for i in range(rank):
        span = (math.ceil(box[i] / estride[i]) - 1) * estride[i] + 1
        coords.append(int(g.integers(-span - 1, dims[i] + 2)))
    m = oracle.Map(dtype, dims, strides, box, estride, sw, fill)
    return m, buf, dtype, dims, strides, box, estride, coords, fill, sw


# ------------------------------- load / store ------------------------------

@pytest.mark.parametrize("seed", range(300))
def test_load_matches_numpy_pad_slice(seed):
    g = np.random.Generator(np.random.PCG64(1000 + seed))
    sw = ["none", "128b"][seed % 2]
    m, buf, dtype, dims, strides, box, estride, coords, fill, sw = random_case(g, sw)
    assert m.validate() == "OK", (dims, strides, box, estride, sw)
    got = m.load(buf, [coords])[0]
    want = np_load_none(buf, dtype, dims, strides, box, estride, coords, fill)
    if sw == "128b":
        want = page_swizzle_128b(want)
    assert got.size == m.box_bytes()
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("seed", range(120))
def test_store_roundtrip_covers_exactly_inbounds(seed):
    g = np.random.Generator(np.random.PCG64(5000 + seed))
    m, buf, dtype, dims, strides, box, estride, coords, fill, sw = random_case(g)
    assert m.validate() == "OK"
    es = oracle.ESIZE[dtype]
    img = m.load(buf, [coords])
    dst = np.full(buf.size, 0xA5, dtype=np.uint8)
    m.store(dst, [coords], img)
    # Expected: covered in-bounds elements copied, every other byte untouched.
    want = np.full(buf.size, 0xA5, dtype=np.uint8)
    src_v = np_tensor_view(buf, dtype, dims, strides)
    dst_v = np_tensor_view(want, dtype, dims, strides)
    sl = []
    for i in reversed(range(len(dims))):
        L = math.ceil(box[i] / estride[i])
        idx = [coords[i] + k * estride[i] for k in range(L)]
        sl.append([x for x in idx if 0 <= x < dims[i]])
    if all(len(s) for s in sl):
        ix = np.ix_(*sl)
        dst_v[ix] = src_v[ix]
    np.testing.assert_array_equal(dst, want)


def test_swizzle_k256_invariants():
    """The 256-byte-key modes (this library's addition, not on the pages): a XOR
    permutation of the 16-byte sectors of each row whose key is constant per
    row, 16 B granularity kept, involution, keys repeating with twice the
    period of the pages' modes; the key of row r is the pages' key of row
    r // 2 (for 128-byte rows: (r // 2) % 8)."""
    for mode, base, span in (("32b_k256", "32b", 32), ("64b_k256", "64b", 64), ("128b_k256", "128b", 128)):
        nsec = span // 16
        keys = []
        for r in range(64):
            row_keys = set()
            for c in range(nsec):
                off = r * span + c * 16
                phys = oracle.swizzle(off, mode)
                assert phys // span == r and oracle.swizzle(phys, mode) == off
                for b in range(16):
                    assert oracle.swizzle(off + b, mode) == phys + b
                row_keys.add((phys // 16 % nsec) ^ c)
            assert len(row_keys) == 1
            keys.append(row_keys.pop())
        period = 16                                    # nsec * 256 / span rows
        base_keys = []
        for r in range(64):
            base_keys.append((oracle.swizzle(r * span, base) // 16) % nsec)
        assert keys == [base_keys[r // 2] for r in range(64)]
        assert keys[:period] == keys[period:2 * period]
    assert [(oracle.swizzle(r * 128, "128b_k256") // 16) % 8 for r in range(16)] == [r // 2 for r in range(16)]


def test_swizzle_invariants_all_modes():
    """32B/64B carry no printed example (pinned by the bank criterion below); invariants:
    XOR permutation of 16-byte sectors inside each N-byte row, key constant
    along a row, 8-row period, row 0 identity, involution, every key value of
    the span used equally often within one atom; 128B equals the page rule."""
    for mode, span in (("32b", 32), ("64b", 64), ("128b", 128)):
        nsec = span // 16
        keys = []
        for r in range(32):
            row_keys = set()
            for c in range(nsec):
                off = r * span + c * 16
                phys = oracle.swizzle(off, mode)
                assert phys // span == r                      # stays in its row
                assert oracle.swizzle(phys, mode) == off      # involution
                for b in range(16):
                    assert oracle.swizzle(off + b, mode) == phys + b
                row_keys.add((phys // 16 % nsec) ^ c)
            assert len(row_keys) == 1                         # one XOR key per row
            keys.append(row_keys.pop())
        assert keys[0] == 0
        assert keys[:8] == keys[8:16] == keys[16:24]          # 8-row atom
        counts = np.bincount(keys[:8], minlength=nsec)
        assert (counts == 8 // nsec).all()
        if mode == "128b":
            assert keys[:8] == list(range(8))                 # col XOR row


def _row_index_key_swizzle(off, mode):
    """The rejected reading of the narrower modes: XOR key = row % (N/16) on
    N-byte rows.  Kept here only to show that the pins below reject it."""
    span = {"32b": 32, "64b": 64, "128b": 128}[mode]
    nsec = span // 16
    row, c = off // span, (off % span) // 16
    return row * span + ((c ^ (row % nsec)) * 16) + off % 16


def _narrow_mode_violations(swz, mode):
    """Ways a swizzle of N-byte rows breaks what [MLC] 'grouping requirement'
    fixes for the 128-byte mode, carried over to the narrower spans:
    (a) bank sectors -- eight consecutive rows of one atom reading the same
        16-byte column must hit eight distinct bank sectors of the pages'
        model (32 banks x 4 bytes, sector = (address >> 4) % 8), the
        section's stated purpose of the swizzle;
    (b) the XOR key is the 128-byte unit index of the address -- the
        section's 256-byte-row formula, local_col XOR ((2*row + col//8) % 8),
        keys the two 128-byte halves of one row 2*row and 2*row + 1 -- so the
        rows that share a 128-byte unit share a key."""
    span = {"32b": 32, "64b": 64, "128b": 128}[mode]
    nsec = span // 16
    bad = []
    for atom in range(4):
        for c in range(nsec):
            sectors = {(swz((8 * atom + r) * span + 16 * c, mode) >> 4) % 8 for r in range(8)}
            if len(sectors) != 8:
                bad.append(("sectors", atom, c, len(sectors)))
    keys = [((swz(r * span, mode) // 16) % nsec) for r in range(32)]
    for r in range(32):
        if keys[r] != keys[(r * span // 128) * 128 // span]:
            bad.append(("unit key", r))
    return bad


def test_swizzle_narrow_modes_pinned_by_bank_criterion():
    """32B / 64B: the pages print no pattern; the reading (XOR key = 128-byte
    unit index mod N/16) is pinned by the bank-sector criterion and the
    address-unit key of [MLC] 'grouping requirement'.  The row-index key
    (row % (N/16)) fails both, so a planted row-index key fails here."""
    for mode in ("32b", "64b", "128b"):
        assert _narrow_mode_violations(oracle.swizzle, mode) == [], mode
    for mode in ("32b", "64b"):
        bad = _narrow_mode_violations(_row_index_key_swizzle, mode)
        assert any(b[0] == "sectors" for b in bad) and any(b[0] == "unit key" for b in bad), mode
    # the 128-byte mode is the same under both readings (128-byte rows)
    assert _narrow_mode_violations(_row_index_key_swizzle, "128b") == []


def test_swizzle_key_sequences():
    """The key of each row of an N-byte-row box (the physical sector that
    logical sector 0 lands in), rows 0..15: the reading written out."""
    def keys(mode, span, n=16):
        return [(oracle.swizzle(r * span, mode) // 16) % (span // 16) for r in range(n)]
    assert keys("128b", 128) == [r % 8 for r in range(16)]            # [MLC]: col XOR (row % 8)
    assert keys("64b", 64)[:8] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert keys("64b", 64)[8:] == [0, 0, 1, 1, 2, 2, 3, 3]
    assert keys("32b", 32)[:8] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert keys("128b_k256", 128) == [r // 2 for r in range(16)]
    assert keys("64b_k256", 64) == [0, 0, 0, 0, 1, 1, 1, 1, 2, 2, 2, 2, 3, 3, 3, 3]
    assert keys("32b_k256", 32) == [0] * 8 + [1] * 8
    # every sector of a row moves by the row's key
    for mode, span in (("32b", 32), ("64b", 64), ("128b", 128), ("64b_k256", 64)):
        k = keys(mode, span, 32)
        for r in range(32):
            for c in range(span // 16):
                assert oracle.swizzle(r * span + 16 * c, mode) == r * span + 16 * (c ^ k[r])


def test_swizzle_k256_sixteen_sectors():
    """The _K256 modes exist for a 64-bank LDS (gfx950: one ds_read_b128 wave
    instruction reads 256 bytes per clock).  Sixteen consecutive rows of one
    16-byte column must then hit sixteen distinct 16-byte sectors of a
    256-byte bank line, sector = (address >> 4) % 16; the pages' 8-row modes
    hit eight sectors twice each on 128-byte rows."""
    for mode, span in (("128b_k256", 128), ("64b_k256", 64), ("32b_k256", 32)):
        for atom in range(2):
            for c in range(span // 16):
                sectors = {(oracle.swizzle((16 * atom + r) * span + 16 * c, mode) >> 4) % 16 for r in range(16)}
                assert len(sectors) == 16, (mode, atom, c)
    sectors = {(oracle.swizzle(r * 128, "128b") >> 4) % 16 for r in range(16)}
    assert len(sectors) == 8


# ------------------------- the pages' worked examples -----------------------

def test_example_2d_sector_table(table):
    """[MLC] swizzled-layout example: 16x128 fp16 tensor, 8x64 box at
    (row 0, col 0) and (row 8, col 64), NONE and 128B."""
    ex = W.EXAMPLE_2D
    src = synthgen.u16_bits(ex["seed"], (16, 128))
    rows = table("mlc_example_2d_sectors.txt")
    for mode in ("none", "128b"):
        m = oracle.Map("f16", ex["dims"], ex["strides"], ex["box"], swizzle=mode)
        assert m.validate() == "OK" and m.box_bytes() == 1024
        for c0, c1 in ex["coords"]:
            img = m.load(src, [(c0, c1)])[0].view(np.uint16).reshape(8, 8, 8)
            for rec in rows:
                if rec[0] != mode:
                    continue
                r = int(rec[1])
                for p in range(8):
                    logical = int(rec[2 + p])
                    want = src[c1 + r, c0 + 8 * logical: c0 + 8 * logical + 8]
                    np.testing.assert_array_equal(img[r, p], want)
            # round trip into a sentinel buffer
            dst = np.full((16, 128), 0xDEAD, dtype=np.uint16)
            m.store(dst, [(c0, c1)], m.load(src, [(c0, c1)]))
            want = np.full((16, 128), 0xDEAD, dtype=np.uint16)
            want[c1:c1 + 8, c0:c0 + 64] = src[c1:c1 + 8, c0:c0 + 64]
            np.testing.assert_array_equal(dst, want)


def test_example_3d_four_atoms(table):
    """[MLC] 3D TMA example: 16x256 fp16 viewed as (group, row, col), one
    2x16x64 box per 128-column slice, four atoms keyed by row % 8."""
    ex = W.EXAMPLE_3D
    src = synthgen.u16_bits(ex["seed"], (16, 256))
    m = oracle.Map("f16", ex["dims"], ex["strides"], ex["box"], swizzle="128b")
    assert m.validate() == "OK" and m.box_bytes() == 4096
    imgs = {c[2] * 64: m.load(src, [c])[0] for c in ex["coords"]}
    for rec in table("mlc_example_3d_atoms.txt"):
        off, grp, row, p, grow, gcol = map(int, rec)
        img = imgs[off]
        lds = grp * 2048 + row * 128 + p * 16
        np.testing.assert_array_equal(img[lds:lds + 16].view(np.uint16), src[grow, gcol:gcol + 8])
    # The regroup only reinterprets coordinates: a 2D descriptor over the same
    # slice (NONE) holds global[row, j] at row*256 + 2*j, and the 3D NONE image
    # holds global3[group, row, col] = global[row, 64*group + col].
    m3n = oracle.Map("f16", ex["dims"], ex["strides"], ex["box"], swizzle="none")
    for off in (0, 128):
        img3 = m3n.load(src, [(0, 0, off // 64)])[0].view(np.uint16).reshape(2, 16, 64)
        for grp in range(2):
            np.testing.assert_array_equal(img3[grp], src[:, off + 64 * grp: off + 64 * grp + 64])


def test_bank_sector_counts(table):
    """[MLC] grouping requirement: 8 distinct sectors when grouped, 4 sectors
    hit twice with a 256-byte stride, for every start row and column."""
    for rec in table("mlc_bank_sectors.txt"):
        layout, row0, col = rec[0], int(rec[1]), int(rec[2])
        want = [int(x) for x in rec[3:]]
        got = oracle.bank_sector_hist(layout == "grouped", row0, col)
        assert got == want, (layout, row0, col)
        if layout == "grouped":
            assert sorted(got) == [1] * 8
        else:
            assert sorted(got) == [0, 0, 0, 0, 2, 2, 2, 2]


# ---------------------------------- txbar ----------------------------------

def test_txbar_4096_trace(table):
    """[MLC] waiting for a TMA load: 2048 + 2048 = 4096 expected bytes."""
    b = None
    for rec in table("mlc_txbar_4096.txt"):
        op, arg = rec[0], int(rec[1])
        want = tuple(int(x) for x in rec[2:5])
        want_wait = bool(int(rec[5]))
        if op == "init":
            b = oracle.Txbar(arg)
        else:
            getattr(b, op)(arg)
        assert b.state() == want, (op, b.state())
        assert b.try_wait(0) == want_wait


def test_txbar_orderings():
    """[H200] pitfalls: expect the bytes before the copy is issued; arriving
    first releases the phase before any byte lands.  [HPC] single-load
    example order: expect bytes, issue, arrive, wait."""
    b = oracle.Txbar(1)
    b.arrive(1)                       # arrival without expect_tx: early release
    assert b.try_wait(0) and b.state() == (1, 0, 1)
    b = oracle.Txbar(1)
    b.expect_tx(4096)
    b.complete_tx(4096)               # copy lands before the arrive
    assert not b.try_wait(0)
    b.arrive(1)
    assert b.try_wait(0)
    # several arrivals and several expect_tx in one phase, then a second phase
    b = oracle.Txbar(3)
    b.arrive_expect_tx(100)
    b.expect_tx(50)
    b.arrive(1)
    b.complete_tx(150)
    assert not b.try_wait(0)
    b.arrive(1)
    assert b.try_wait(0) and not b.try_wait(1)
    b.arrive_expect_tx(10)
    b.arrive(2)
    assert not b.try_wait(1)
    b.complete_tx(10)
    assert b.try_wait(1) and b.state() == (3, 0, 0)


# ------------------------------- validation --------------------------------

def _map(**kw):
    base = dict(dtype="bf16", dims=(128, 64), strides=(256,), box=(64, 32), estride=None,
                swizzle="128b", fill="zero", base_addr=0x10000)
    base.update(kw)
    return oracle.Map(base["dtype"], base["dims"], base["strides"], base["box"], base["estride"],
                      base["swizzle"], base["fill"], base["base_addr"])


@pytest.mark.parametrize("kw,want", [
    (dict(), "OK"),
    # [H200] section 03: rank <= 5
    (dict(dims=(16,) * 6, strides=(32,) * 5, box=(16,) * 6, swizzle="none"), "ERR_RANK"),
    # boxDim <= 256 per dimension
    (dict(box=(64, 257)), "ERR_BOX"),
    (dict(box=(64, 0)), "ERR_BOX"),
    # boxDim[0] * esize a multiple of 16 bytes
    (dict(box=(4, 8), swizzle="none"), "ERR_BOX"),
    # globalStrides multiples of 16 and below 2^40
    (dict(strides=(264,)), "ERR_STRIDE"),
    (dict(strides=(1 << 40,)), "ERR_STRIDE"),
    (dict(strides=((1 << 40) - 16,)), "OK"),
    # base address 16-byte aligned
    (dict(base_addr=0x10008), "ERR_ALIGN"),
    (dict(base_addr=0), "ERR_NULL"),
    # [MLC] 3D example: a 128B box's contiguous extent must be 128 bytes
    (dict(box=(128, 8)), "ERR_SWIZZLE_WIDTH"),
    (dict(box=(32, 8)), "ERR_SWIZZLE_WIDTH"),
    (dict(box=(32, 8), swizzle="64b"), "OK"),
    (dict(box=(16, 8), swizzle="32b"), "OK"),
    (dict(box=(256, 8), swizzle="none"), "OK"),
    # NaN fill only for float element types
    (dict(dtype="i32", box=(32, 8), fill="nan"), "ERR_OOB_FILL_DTYPE"),
    (dict(dtype="f32", box=(32, 8), fill="nan"), "OK"),
    # element strides
    (dict(estride=(1, 9)), "ERR_ESTRIDE"),
    (dict(estride=(2, 1), box=(128, 8)), "OK"),
    (dict(estride=(3, 1), box=(128, 8), swizzle="none"), "ERR_ESTRIDE"),
    # dims
    (dict(dims=(0, 64)), "ERR_DIM"),
    (dict(dims=((1 << 32) + 1, 64)), "ERR_DIM"),
    # LDS capacity
    (dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 8)), "ERR_LDS_CAPACITY"),
    (dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 5)), "ERR_LDS_CAPACITY"),
    (dict(dims=(256, 256, 8), strides=(512, 131072), box=(64, 256, 4)), "OK"),
    (dict(dtype="f32", dims=(32, 159, 8), strides=(128, 20352), box=(32, 159, 8)), "OK"),
    (dict(dtype="f32", dims=(32, 160, 8), strides=(128, 20480), box=(32, 160, 8)), "ERR_LDS_CAPACITY"),
    (dict(dtype="u8", box=(128, 8)), "OK"),
])
def test_validate_constraint_table(kw, want):
    assert _map(**kw).validate() == want


def test_box_bytes_and_extents():
    # elementStrides read as a traversal stride: ceil(box / estride) on chip
    m = oracle.Map("f32", W.RANK5["dims"], (1040, 134160, 4427280, 30990960),
                   W.RANK5["box"], W.RANK5["estride"], "128b")
    assert m.validate() == "OK"
    assert [m.lds_extent(d) for d in range(5)] == [32, 16, 8, 2, 1]
    assert m.box_bytes() == 32768
    m = oracle.Map("bf16", (8192, 8192), (16384,), (64, 128), swizzle="128b")
    assert m.box_bytes() == 16384


# --------------------------------- reduce ----------------------------------

def _place(dtype, dims, strides, box, coords, buf):
    v = np_tensor_view(buf, dtype, dims, strides)
    sl = tuple(slice(coords[i], coords[i] + box[i]) for i in reversed(range(len(dims))))
    return v, sl


@pytest.mark.parametrize("dtype", ["u8", "u16", "u32", "i32", "u64", "i64", "f32", "f64", "f16", "bf16"])
def test_reduce_add_single_box_matches_library(dtype):
    """One in-bounds box: each element is dst + src rounded once, compared
    with NumPy / torch element-wise addition of the same type."""
    es = oracle.ESIZE[dtype]
    dims, strides, box = (64, 12), (64 * es + 16,), (32, 8)
    if box[0] * es % 16:
        box = (16, 8)
    foot = strides[0] * dims[1]
    g = np.random.Generator(np.random.PCG64(77))
    if dtype in ("f32", "f64", "f16"):
        npt = {"f32": np.float32, "f64": np.float64, "f16": np.float16}[dtype]
        dst = g.standard_normal(foot // es).astype(npt).view(np.uint8).copy()
        src = (g.standard_normal(box[0] * box[1]) * 3).astype(npt)
    elif dtype == "bf16":
        dst = synthgen.normal_bf16_bits(5, foot // 2).view(np.uint8).copy()
        src = synthgen.normal_bf16_bits(6, box[0] * box[1])
    else:
        dst = synthgen.random_bytes(8, foot)
        src = synthgen.random_bytes(9, box[0] * box[1] * es).view(NP_BITS[es])
    m = oracle.Map(dtype, dims, strides, box, swizzle="none")
    assert m.validate() == "OK"
    coords = (8, 3)
    before = dst.copy()
    m.reduce_add(dst, [coords], src.view(np.uint8))
    v_before, sl = _place(dtype, dims, strides, box, coords, before)
    v_after, _ = _place(dtype, dims, strides, box, coords, dst)
    a = np.array(v_before[sl])
    s = src.view(NP_BITS[es]).reshape(box[1], box[0])
    if dtype in ("f32", "f64", "f16"):
        npt = {"f32": np.float32, "f64": np.float64, "f16": np.float16}[dtype]
        want = (a.view(npt) + s.view(npt)).view(NP_BITS[es])
    elif dtype == "bf16":
        ta = torch.from_numpy(a.astype(np.int32) << 16).view(torch.float32).to(torch.bfloat16)
        ts = torch.from_numpy(s.astype(np.int32) << 16).view(torch.float32).to(torch.bfloat16)
        want = (ta + ts).view(torch.int16).numpy().view(np.uint16)
    else:
        want = a + s      # NumPy unsigned arithmetic wraps modulo 2^w
    np.testing.assert_array_equal(np.array(v_after[sl]), want)
    # everything outside the box is untouched
    mask = np.ones(foot, dtype=bool)
    mask_v = np_tensor_view(mask.view(np.uint8), "u8", (dims[0] * es, dims[1]), strides)
    mask_v[sl[0], coords[0] * es:(coords[0] + box[0]) * es] = False
    np.testing.assert_array_equal(dst[mask], before[mask])


def test_reduce_add_int32_overlapping_closed_form():
    """Overlapping int32 boxes: dst_after = dst_before + sum of sources
    modulo 2^32, independent of order; global checksum invariant."""
    dims, strides, box = (96, 80), (384,), (16, 16)
    dst0 = synthgen.int32_range(11, (80, 96), -(1 << 20), 1 << 20)
    coords = synthgen.uniform_coords(12, 40, (0, 0), (80, 64))
    srcs = synthgen.int32_range(13, (40, 16, 16), -(1 << 20), 1 << 20)
    m = oracle.Map("i32", dims, strides, box, swizzle="none")
    dst = dst0.copy()
    m.reduce_add(dst, coords, srcs.view(np.uint8))
    want = dst0.astype(np.int64)
    for b in range(40):
        c0, c1 = coords[b]
        want[c1:c1 + 16, c0:c0 + 16] += srcs[b]
    want = ((want + (1 << 31)) % (1 << 32) - (1 << 31)).astype(np.int32)
    np.testing.assert_array_equal(dst, want)
    # reversing box order gives the same bits
    dst_r = dst0.copy()
    m.reduce_add(dst_r, coords[::-1].copy(), srcs[::-1].copy().view(np.uint8))
    np.testing.assert_array_equal(dst_r, dst)


def test_reduce_f64_accumulate_exact_sum():
    dims, strides, box = (64, 40), (256,), (16, 8)
    dst0 = synthgen.normal_f32(21, (40, 64))
    coords = synthgen.uniform_coords(22, 30, (0, 0), (48, 32))
    srcs = synthgen.normal_f32(23, (30, 8, 16))
    m = oracle.Map("f32", dims, strides, box, swizzle="none")
    acc = dst0.astype(np.float64).reshape(-1).copy()
    mag = np.abs(acc)
    m.reduce_add_f64(acc, mag, coords, srcs.view(np.uint8))
    want = dst0.astype(np.float64)
    wmag = np.abs(want)
    for b in range(30):
        c0, c1 = coords[b]
        want[c1:c1 + 8, c0:c0 + 16] += srcs[b].astype(np.float64)
        wmag[c1:c1 + 8, c0:c0 + 16] += np.abs(srcs[b].astype(np.float64))
    np.testing.assert_allclose(acc.reshape(40, 64), want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(mag.reshape(40, 64), wmag, rtol=0, atol=1e-12)


# ------------------------------ conversions --------------------------------

def test_half_conversions_against_libraries():
    allbits = np.arange(1 << 16, dtype=np.uint32)
    f16 = allbits.astype(np.uint16).view(np.float16).astype(np.float64)
    bf = torch.from_numpy((allbits << 16).astype(np.uint32).view(np.int32)).view(torch.float32).double().numpy()
    for b in range(0, 1 << 16, 7):
        o = oracle.f16_to_f64(b)
        assert (math.isnan(o) and math.isnan(f16[b])) or o == f16[b]
        o = oracle.bf16_to_f64(b)
        assert (math.isnan(o) and math.isnan(bf[b])) or o == bf[b]
    g = np.random.Generator(np.random.PCG64(3))
    xs = np.concatenate([g.standard_normal(3000) * 10.0 ** g.integers(-8, 6, 3000),
                         [0.0, -0.0, 65504.0, 65520.0, 65519.99, 6e-8, 2.0 ** -25, 2.0 ** -24 * 1.5,
                          1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, np.inf, -np.inf, 3e38, 3.4e38]])
    for x in xs:
        with np.errstate(over="ignore"):   # values past the f16 range round to infinity on purpose
            want = np.array([x]).astype(np.float16).view(np.uint16)[0]
        assert oracle.f64_to_f16(float(x)) == want, x
    # bf16: values that are sums of two bf16 (how the reduce uses it); torch
    # rounds float32 -> bf16 to nearest-even and float32 holds these sums
    # closely enough that the two roundings agree.
    a = synthgen.normal_bf16_bits(31, 4000)
    b = synthgen.normal_bf16_bits(32, 4000)
    ta = torch.from_numpy(a.astype(np.int32) << 16).view(torch.float32)
    tb = torch.from_numpy(b.astype(np.int32) << 16).view(torch.float32)
    s64 = ta.double() + tb.double()
    want = (ta.to(torch.bfloat16) + tb.to(torch.bfloat16)).view(torch.int16).numpy().view(np.uint16)
    for i in range(4000):
        assert oracle.f64_to_bf16(float(s64[i])) == want[i]
    # explicit ties to even
    assert oracle.f64_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f64_to_bf16(3.5e38) == 0x7F80
    assert oracle.f64_to_bf16(-2.0 ** -133) == 0x8001


# ---------------------------------- GEMM -----------------------------------

def _bf16_to_np64(bits):
    return torch.from_numpy(bits.astype(np.int32) << 16).view(torch.float32).double().numpy()


def test_gemm_sample_matches_numpy_matmul():
    M, N, K = 48, 40, 96
    A = synthgen.normal_bf16_bits(41, (M, K))
    Bt = synthgen.normal_bf16_bits(42, (N, K))       # column-major B stored as (N, K)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    got = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    want = _bf16_to_np64(A) @ _bf16_to_np64(Bt).T
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_gemm_sample_identity_and_permutation_exact():
    K = 64
    Bt = synthgen.normal_bf16_bits(43, (32, K))
    eye = np.zeros((K, K), dtype=np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80            # bf16 1.0
    rows, cols = np.meshgrid(np.arange(K), np.arange(32), indexing="ij")
    got = oracle.gemm_bf16_sample(eye, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(K, 32)
    np.testing.assert_array_equal(got, _bf16_to_np64(Bt).T)
    perm = synthgen.rng(44).permutation(K)
    P = np.zeros((K, K), dtype=np.uint16)
    P[np.arange(K), perm] = 0x3F80
    got = oracle.gemm_bf16_sample(P, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(K, 32)
    np.testing.assert_array_equal(got, _bf16_to_np64(Bt).T[perm])


# ------------------------------ min / max reduce -----------------------------

_FLOAT_NP = {"f32": np.float32, "f64": np.float64, "f16": np.float16}


def _as_f64_values(dtype, bits):
    """Element values of raw bits as float64 (bf16 through float32); the
    random bit patterns include NaNs on purpose."""
    with np.errstate(invalid="ignore"):
        if dtype == "bf16":
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return bits.view(_FLOAT_NP[dtype]).astype(np.float64)


@pytest.mark.parametrize("op", ["min", "max"])
@pytest.mark.parametrize("dtype", ["u8", "u16", "u32", "i32", "u64", "i64", "f32", "f64", "f16", "bf16"])
def test_reduce_minmax_single_box_matches_numpy(dtype, op):
    """One in-bounds box of random bit patterns (floats include NaN, infinities,
    subnormals and both zeros): integers against NumPy minimum / maximum of the
    signed or unsigned type, floats against NumPy fmin / fmax (IEEE minNum /
    maxNum: a NaN operand yields the other one) as values, with two NaNs giving
    the canonical NaN and -0 ordered below +0."""
    es = oracle.ESIZE[dtype]
    dims, strides, box = (64, 12), (64 * es + 16,), (32, 8)
    if box[0] * es % 16:
        box = (16, 8)
    foot = strides[0] * dims[1]
    dst = synthgen.random_bytes(31 + es, foot)
    src = synthgen.random_bytes(41 + es, box[0] * box[1] * es)
    m = oracle.Map(dtype, dims, strides, box, swizzle="none")
    coords = (8, 3)
    before = dst.copy()
    m.reduce(dst, [coords], src, op)
    v_before, sl = _place(dtype, dims, strides, box, coords, before)
    v_after, _ = _place(dtype, dims, strides, box, coords, dst)
    a = np.array(v_before[sl])
    s = src.view(NP_BITS[es]).reshape(box[1], box[0])
    got = np.array(v_after[sl])
    if dtype in ("i32", "i64"):
        sig = {4: np.int32, 8: np.int64}[es]
        f = np.minimum if op == "min" else np.maximum
        np.testing.assert_array_equal(got.view(sig), f(a.view(sig), s.view(sig)))
    elif dtype in ("u8", "u16", "u32", "u64"):
        f = np.minimum if op == "min" else np.maximum
        np.testing.assert_array_equal(got, f(a, s))
    else:
        av, sv, gv = _as_f64_values(dtype, a), _as_f64_values(dtype, s), _as_f64_values(dtype, got)
        f = np.fmin if op == "min" else np.fmax
        want = f(av, sv)
        np.testing.assert_array_equal(gv, want)          # NaN == NaN here
        both_nan = np.isnan(av) & np.isnan(sv)
        assert (got[both_nan] == NAN_BITS[dtype]).all()
        assert not np.isnan(gv[~both_nan]).any()
        # the bits are those of one operand (no canonicalisation of values)
        assert ((got == a) | (got == s) | both_nan).all()
    mask = np.ones(foot, dtype=bool)
    mask_v = np_tensor_view(mask.view(np.uint8), "u8", (dims[0] * es, dims[1]), strides)
    mask_v[sl[0], coords[0] * es:(coords[0] + box[0]) * es] = False
    np.testing.assert_array_equal(dst[mask], before[mask])


SPECIAL = {
    # dtype: [(dst bits, src bits, min bits, max bits), ...]
    "f32": [(0x80000000, 0x00000000, 0x80000000, 0x00000000),      # -0 vs +0
            (0x00000000, 0x80000000, 0x80000000, 0x00000000),
            (0x7FC00001, 0x3F800000, 0x3F800000, 0x3F800000),      # NaN vs 1
            (0x3F800000, 0xFFC00000, 0x3F800000, 0x3F800000),      # 1 vs NaN
            (0x7FC00001, 0xFFFFFFFF, 0x7FC00000, 0x7FC00000),      # NaN vs NaN
            (0xFF800000, 0x40400000, 0xFF800000, 0x40400000),      # -inf vs 3
            (0x00000001, 0x00000000, 0x00000000, 0x00000001),      # smallest subnormal vs +0
            (0x80000001, 0x00000000, 0x80000001, 0x00000000)],
    "bf16": [(0x8000, 0x0000, 0x8000, 0x0000), (0x7FC1, 0xBF80, 0xBF80, 0xBF80),
             (0xFFC0, 0x7F81, 0x7FC0, 0x7FC0), (0x0001, 0x8001, 0x8001, 0x0001)],
    "f16": [(0x8000, 0x0000, 0x8000, 0x0000), (0x7E01, 0x3C00, 0x3C00, 0x3C00),
            (0xFE00, 0x7C01, 0x7E00, 0x7E00), (0xFC00, 0x7C00, 0xFC00, 0x7C00)],
    "f64": [(0x8000000000000000, 0x0, 0x8000000000000000, 0x0),
            (0x7FF8000000000001, 0x3FF0000000000000, 0x3FF0000000000000, 0x3FF0000000000000),
            (0x7FF0000000000001, 0xFFF8000000000000, 0x7FF8000000000000, 0x7FF8000000000000)],
    "i32": [(0xFFFFFFFB, 0x00000003, 0xFFFFFFFB, 0x00000003),      # -5 vs 3 (signed)
            (0x80000000, 0x7FFFFFFF, 0x80000000, 0x7FFFFFFF)],
    "u32": [(0xFFFFFFFF, 0x00000001, 0x00000001, 0xFFFFFFFF)],
    "u8": [(200, 100, 100, 200)],
    "u16": [(0x8000, 0x7FFF, 0x7FFF, 0x8000)],
    "i64": [(0xFFFFFFFFFFFFFFFF, 0x1, 0xFFFFFFFFFFFFFFFF, 0x1)],
    "u64": [(0x8000000000000000, 0x1, 0x1, 0x8000000000000000)],
}


@pytest.mark.parametrize("dtype", sorted(SPECIAL))
def test_reduce_minmax_special_cases(dtype):
    """Hand-listed cases of the readings: signed / unsigned compares, -0 < +0,
    minNum / maxNum NaN handling, canonical NaN from two NaNs, subnormals and
    infinities kept bit for bit."""
    es = oracle.ESIZE[dtype]
    cases = SPECIAL[dtype]
    n = 16 // es * ((len(cases) * es + 15) // 16)      # whole 16-byte rows
    nt = NP_BITS[es]
    for col, op in ((2, "min"), (3, "max")):
        dst = np.zeros(n, dtype=nt)
        src = np.zeros(n, dtype=nt)
        for i, c in enumerate(cases):
            dst[i], src[i] = c[0], c[1]
        m = oracle.Map(dtype, (n, 1), (n * es,), (n, 1), swizzle="none")
        m.reduce(dst, [(0, 0)], src.view(np.uint8), op)
        for i, c in enumerate(cases):
            assert int(dst[i]) == c[col], (dtype, op, i, hex(int(dst[i])), hex(c[col]))


@pytest.mark.parametrize("op", ["min", "max"])
@pytest.mark.parametrize("dtype", ["i32", "f32", "bf16"])
def test_reduce_minmax_overlapping_order_free(dtype, op):
    """Overlapping boxes: the result is the element-wise min / max over the
    initial value and every contribution, whatever the box order."""
    es = oracle.ESIZE[dtype]
    W_, H_ = 96, 80
    box = (16, 16)
    dst0 = synthgen.random_bytes(61, W_ * H_ * es)
    coords = synthgen.uniform_coords(62, 40, (0, 0), (W_ - 16, H_ - 16))
    srcs = synthgen.random_bytes(63, 40 * 16 * 16 * es)
    m = oracle.Map(dtype, (W_, H_), (W_ * es,), box, swizzle="none")
    d1 = dst0.copy()
    m.reduce(d1, coords, srcs, op)
    d2 = dst0.copy()
    rev = srcs.reshape(40, -1)[::-1].copy().reshape(-1)
    m.reduce(d2, coords[::-1].copy(), rev, op)
    np.testing.assert_array_equal(d1, d2)
    # element-wise over all contributions, computed per element with NumPy
    nt = NP_BITS[es]
    grid = dst0.view(nt).reshape(H_, W_)
    contrib = [[[grid[r, c]] for c in range(W_)] for r in range(H_)]
    sb = srcs.view(nt).reshape(40, 16, 16)
    for b in range(40):
        c0, c1 = coords[b]
        for r in range(16):
            for c in range(16):
                contrib[c1 + r][c0 + c].append(sb[b, r, c])
    got = d1.view(nt).reshape(H_, W_)
    for r in range(H_):
        for c in range(W_):
            vals = np.array(contrib[r][c], dtype=nt)
            if len(vals) == 1:                       # no box covers it: untouched
                assert got[r, c] == vals[0]
                continue
            if dtype == "i32":
                v = vals.view(np.int32)
                want = (v.min() if op == "min" else v.max())
                assert got[r, c].view(np.int32) == want
            else:
                fv = _as_f64_values(dtype, vals)
                if np.isnan(fv).all():
                    assert got[r, c] == NAN_BITS[dtype]
                    continue
                f = np.nanmin if op == "min" else np.nanmax
                w = f(fv)
                gv = _as_f64_values(dtype, np.array([got[r, c]], dtype=nt))[0]
                assert gv == w
                if w == 0.0:
                    zeros = vals[(fv == 0.0)]
                    neg = any(int(z) >> (8 * es - 1) for z in zeros)
                    pos = any(not (int(z) >> (8 * es - 1)) for z in zeros)
                    want_neg = neg if op == "min" else not pos
                    assert (int(got[r, c]) >> (8 * es - 1)) == int(want_neg)
