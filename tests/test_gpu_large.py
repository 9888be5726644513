"""GPU parity where byte offsets inside one tensor pass 4 GiB (so that any
32-bit offset arithmetic would wrap): box loads, stores and reductions in the
last rows of a 4.3 GB pitched tensor, checked against the oracle on a window
that holds those rows; the tile copy of a 4.4 GB bf16 tensor (a copy is the
identity on the tensor's bytes); the GEMM with a 4.9 GB operand, and a 4.9 GB
output, whose last rows are sampled against the oracle."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402

from gpu_util import empty_dev, encode, require_native, stream, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

GiB4 = 1 << 32


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def release():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# One 128-byte row segment per row, rows 128 KiB apart: 33000 rows span
# 4.33 GB, and the last 64 rows (the window) start past 4 GiB.
PITCH = 1 << 17
ROWS = 33000
WIN = 64
ESIZE = {"u8": 1, "bf16": 2, "i32": 4, "f64": 8}


@pytest.mark.parametrize("dtype", ["u8", "bf16", "i32", "f64"])
def test_box_ops_past_4gib(dtype):
    """Loads, stores and reductions of 16-row boxes whose origins sweep the
    window (dim-0 origins from half a row below to half a row above, rows up
    to past the tensor's end) in a tensor whose window starts at byte
    4,316,987,392: each against the oracle on the window alone, and no byte
    before the window written."""
    es = ESIZE[dtype]
    L0 = 128 // es
    dims, box = (L0, ROWS), (L0, 16)
    w0 = (ROWS - WIN) * PITCH
    assert w0 > GiB4
    fill = "nan" if dtype in ("bf16", "f64") else "zero"
    g = synthgen.rng(61000 + es)
    n = 24
    coords = np.stack([g.integers(-(L0 // 2), L0 // 2 + 1, n), g.integers(ROWS - WIN, ROWS + 2, n)],
                      axis=1).astype(np.int32)
    wcoords = coords.copy()
    wcoords[:, 1] -= ROWS - WIN
    say("past 4 GiB", dtype, "coords", coords[:4].tolist(), "...")
    win = synthgen.random_bytes(61100 + es, WIN * PITCH)
    om = oracle.Map(dtype, (L0, WIN), (PITCH,), box, None, "128b", fill)
    assert om.validate() == "OK"

    big = torch.empty(ROWS * PITCH, dtype=torch.uint8, device="cuda")
    big.fill_(0xA5)
    wdev = big[w0:]
    wdev.copy_(torch.from_numpy(win).cuda())
    m = encode(big, dtype, dims, (PITCH,), box, None, "128b", fill)
    bb = att.tmap_box_bytes(m)
    cd = to_dev(coords)

    # load
    out = empty_dev(n * bb, 0x5A)
    att.tile_load(m, cd, n, out, stream())
    np.testing.assert_array_equal(to_host(out).reshape(n, bb), om.load(win, wcoords))

    # reductions: integer add and every type's min / max over overlapping
    # boxes (order-free); bf16 add (its own word loop) over boxes that do not
    # overlap (one contribution per element, exact, NaN results canonical),
    # the last one past the tensor's end.  f64 add walks the elements as the
    # int32 add and the f64 min / max do; its NaN results have no fixed
    # payload, so it is left to the special-value tests.
    imgs = synthgen.random_bytes(61200 + es, n * bb).reshape(n, bb)
    ops = (["add"] if dtype in ("u8", "i32") else []) + ["min", "max"]
    for op in ops:
        wdev.copy_(torch.from_numpy(win).cuda())
        att.tile_reduce(m, op, cd, n, to_dev(imgs), stream())
        want = win.copy()
        om.reduce(want, wcoords, imgs, op)
        np.testing.assert_array_equal(to_host(wdev), want, err_msg=op)
    if dtype == "bf16":
        sc = np.stack([g.integers(-(L0 // 2), L0 // 2 + 1, 4), ROWS - np.array([60, 44, 28, 12])],
                      axis=1).astype(np.int32)
        swc = sc.copy()
        swc[:, 1] -= ROWS - WIN
        wdev.copy_(torch.from_numpy(win).cuda())
        att.tile_reduce(m, "add", to_dev(sc), 4, to_dev(imgs[:4]), stream())
        want = win.copy()
        om.reduce_add(want, swc, imgs[:4])
        np.testing.assert_array_equal(to_host(wdev), want, err_msg="add")

    # store, one box per call so that overlapping boxes end with the later one
    wdev.fill_(0xA5)
    di = to_dev(imgs)
    for i in range(n):
        att.tile_store(m, cd[i * 8:], 1, di[i * bb:], stream())
    want = np.full(WIN * PITCH, 0xA5, dtype=np.uint8)
    om.store(want, wcoords, imgs)
    np.testing.assert_array_equal(to_host(wdev), want)

    torch.cuda.synchronize()
    assert not bool((big[:w0] != 0xA5).any()), "a byte before the window was written"
    del big, wdev, out
    release()


def test_copy_past_4gib():
    """The default tile copy (producer / consumer) and the ring of a bf16
    8192 x 266112 tensor (4.36 GB, 128 x 64 boxes, 128B swizzle): the
    destination equals the source byte for byte.  The source is a seeded
    random block repeated with a period that does not divide 2^32, so bytes
    fetched 4 GiB away from where they belong would differ."""
    W_, H_ = 8192, 266112
    nbytes = W_ * 2 * H_
    assert nbytes > GiB4
    period = (1 << 26) + 16
    assert GiB4 % period != 0
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    pat = to_dev(synthgen.random_bytes(62000, period))
    for off in range(0, nbytes, period):
        k = min(period, nbytes - off)
        src[off:off + k].copy_(pat[:k])
    ms = encode(src, "bf16", (W_, H_), (W_ * 2,), (64, 128), swizzle="128b")
    for variant in (None, 0):
        say("copy past 4 GiB, variant", variant)
        dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        dst.fill_(0x33)
        md = encode(dst, "bf16", (W_, H_), (W_ * 2,), (64, 128), swizzle="128b")
        if variant is None:
            att.tile_copy(ms, md, 2, stream())
        else:
            att.tile_copy_ex(ms, md, 2, 0, variant, stream())
        torch.cuda.synchronize()
        assert torch.equal(src, dst), f"variant {variant}"
        del dst
        release()
    del src, pat
    release()


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("big_operand", ["A", "B"])
def test_gemm_past_4gib(big_operand):
    """bf16 GEMM, K = 8192, with one operand of 300000 rows (4.9 GB; zero
    but for its last 512 rows, which start past 4 GiB) and the other of 256
    rows; with the big A, C has a leading dimension of 8192 and also spans
    4.9 GB.  4096 sampled outputs of the last 512 rows (or columns) against
    the oracle within |C - ref| <= 2e-2 + 2^-8 |ref|; every other output
    exactly +0 and C's padding columns untouched."""
    K, BIG, SMALL, WR = 8192, 300000, 256, 512
    assert (BIG - WR) * K * 2 > GiB4
    say("gemm past 4 GiB, big", big_operand)
    win = synthgen.normal_bf16_bits(63000, (WR, K))
    small = synthgen.normal_bf16_bits(63001, (SMALL, K))
    bigt = torch.zeros((BIG, K), dtype=torch.int16, device="cuda")
    bigt[BIG - WR:].copy_(torch.from_numpy(win.view(np.int16)).cuda())
    smallt = torch.from_numpy(small.view(np.int16)).cuda()
    if big_operand == "A":
        M, N, ldc = BIG, SMALL, 8192
        Ad, Bd = bigt, smallt
    else:
        M, N, ldc = SMALL, BIG, BIG
        Ad, Bd = smallt, bigt
    Cd = torch.full((M, ldc), 0x7FFF, dtype=torch.int16, device="cuda")
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (K * 2,), (64, 256), None, "128b_k256")
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (K * 2,), (64, 256), None, "128b_k256")
    att.gemm_bf16_ex(mA, mB, Cd.data_ptr(), M, N, K, ldc, 3, 0, 1, stream(), 16)
    torch.cuda.synchronize()
    g = synthgen.rng(63002)
    wi = g.integers(0, WR, 4096)
    oi = g.integers(0, SMALL, 4096)
    if big_operand == "A":
        rows, cols = BIG - WR + wi, oi
        ref = oracle.gemm_bf16_sample(win, small, K, wi, oi)
        zero = Cd[: BIG - WR, :N]
    else:
        rows, cols = oi, BIG - WR + wi
        ref = oracle.gemm_bf16_sample(small, win, K, oi, wi)
        zero = Cd[:, : BIG - WR]
    got = bf16_to_f64(Cd[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()].cpu().numpy().view(np.uint16))
    err = np.abs(got - ref)
    bad = err > 2e-2 + 2.0 ** -8 * np.abs(ref)
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance, worst {err.max()}"
    assert bool((zero == 0).all()), "outputs outside the window are not +0"
    if ldc > N:
        assert bool((Cd[:, N:] == 0x7FFF).all()), "padding columns written"
    del bigt, smallt, Cd, zero, Ad, Bd
    release()
