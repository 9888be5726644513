"""GPU parity of the device API (include/tile.hpp) in a kernel of its own:
tests/device_api/user_tiles.hip is compiled as a user would compile it (its
own shared library, include/ as the only include path) and loads a box with
byte-counted completion, stores it through a second map and adds it into a
third.  Every result is compared with the oracle: int32 bit-exact with
overlapping boxes (integer adds commute), bf16 bit-exact with disjoint boxes
(one add per element, rounded once)."""
import ctypes
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402

from gpu_util import encode, require_native, stream, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
USER_LIB = os.path.join(ROOT, "tests", "device_api", "libuser_tiles.so")


def setup_module(module):
    require_native()


def user_lib():
    if not os.path.exists(USER_LIB):
        pytest.fail(f"{USER_LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(USER_LIB)
    tp = ctypes.POINTER(att.tmap_t)
    L.user_load_store_reduce_launch.argtypes = [tp, tp, tp, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32,
                                                ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    L.user_load_store_reduce_launch.restype = ctypes.c_int
    return L


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(dtype, host_src, host_acc, dims, strides, box, swizzle, coords):
    """Runs the user kernel; returns (dst, acc, landed) on the host."""
    L = user_lib()
    sentinel = np.empty_like(host_src)
    sentinel.view(np.uint8)[...] = 0xAD
    sd, dd, ad = to_dev(host_src), to_dev(sentinel), to_dev(host_acc)
    ms = encode(sd, dtype, dims, strides, box, None, swizzle)
    md = encode(dd, dtype, dims, strides, box, None, swizzle)
    ma = encode(ad, dtype, dims, strides, box, None, swizzle)
    c = np.ascontiguousarray(np.asarray(coords, dtype=np.int32))
    cd = to_dev(c)
    landed = torch.zeros(len(c), dtype=torch.int32, device="cuda")
    rc = L.user_load_store_reduce_launch(ctypes.byref(ms), ctypes.byref(md), ctypes.byref(ma), cd.data_ptr(),
                                         len(dims), len(c), att.tmap_box_bytes(ms), landed.data_ptr(), stream())
    assert rc == 0, rc
    dst = to_host(dd).view(host_src.dtype).reshape(host_src.shape)
    acc = to_host(ad).view(host_acc.dtype).reshape(host_acc.shape)
    return dst, acc, to_host(landed), sentinel


def oracle_case(dtype, host_src, host_acc, sentinel, dims, strides, box, swizzle, coords):
    om = oracle.Map(dtype, dims, strides, box, swizzle=swizzle)
    imgs = om.load(host_src, coords)
    dst = sentinel.copy()
    om.store(dst, coords, imgs)
    acc = host_acc.copy()
    om.reduce_add(acc, coords, imgs)
    return dst, acc


def test_int32_overlapping_boxes_with_edges():
    """300 x 200 int32, 32 x 32 boxes (128-byte rows, 128B swizzle) inside,
    across every edge, at negative and unaligned origins and wholly outside,
    many of them overlapping."""
    H, W = 300, 200
    dims, strides, box = (W, H), (W * 4,), (32, 32)
    src = synthgen.int32_range(71, (H, W), -(1 << 20), 1 << 20)
    acc = synthgen.int32_range(72, (H, W), -(1 << 20), 1 << 20)
    g = synthgen.rng(73)
    coords = [[int(g.integers(-40, 220)), int(g.integers(-40, 320))] for _ in range(120)]
    coords += [[0, 0], [168, 268], [-32, -32], [200, 300], [-5, 7], [171, 3], [1000, 0], [0, -1000]]
    say("device api int32", len(coords), "boxes")
    dst, accg, landed, sentinel = run_case("i32", src, acc, dims, strides, box, "128b", coords)
    want_dst, want_acc = oracle_case("i32", src, acc, sentinel, dims, strides, box, "128b", coords)
    assert landed.all()
    np.testing.assert_array_equal(dst, want_dst)
    np.testing.assert_array_equal(accg, want_acc)


@pytest.mark.parametrize("swizzle", ["none", "128b", "128b_k256"])
def test_bf16_disjoint_boxes(swizzle):
    """256 x 320 bf16, 64 x 48 boxes on a grid offset by (-16, -8), so edge
    boxes are cut on every side; each element gets one add."""
    H, W = 256, 320
    dims, strides, box = (W, H), (W * 2,), (64, 48)
    src = synthgen.normal_bf16_bits(74, (H, W))
    acc = synthgen.normal_bf16_bits(75, (H, W))
    coords = [[x, y] for y in range(-8, H, 48) for x in range(-16, W, 64)]
    say("device api bf16", swizzle, len(coords), "boxes")
    dst, accg, landed, sentinel = run_case("bf16", src, acc, dims, strides, box, swizzle, coords)
    want_dst, want_acc = oracle_case("bf16", src, acc, sentinel, dims, strides, box, swizzle, coords)
    assert landed.all()
    np.testing.assert_array_equal(dst, want_dst)
    np.testing.assert_array_equal(accg, want_acc)


def staged_lib():
    L = ctypes.CDLL(USER_LIB)
    tp = ctypes.POINTER(att.tmap_t)
    L.user_staged_copy_launch.argtypes = [tp, tp, ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.user_staged_copy_launch.restype = ctypes.c_int
    return L


def whole_chunk_groups(dims, box, c, wave=0, nwaves=4):
    """Lower bound a wave's store of box c reports for its group: its 64-chunk
    groups (bf16, 128-byte rows: 8 rows each) holding at least one 16-byte
    chunk wholly inside the tensor."""
    rows, cols = box[1], box[0]
    n = 0
    for g in range(wave, rows * cols * 2 // 16 // 64, nwaves):
        whole = False
        for r in range(8 * g, 8 * g + 8):
            for j in range(8):
                x0, y = c[0] + 8 * j, c[1] + r
                whole |= 0 <= y < dims[1] and x0 >= 0 and x0 + 8 <= dims[0]
        n += whole
    return n


@pytest.mark.parametrize("stages,wait_n", [(1, 0), (2, 1)])
def test_store_groups_reuse_stages(stages, wait_n):
    """[HPC] "TMA store" commit / wait groups, [MLC] "waiting for a TMA
    store": boxes copied through one LDS stage reused after store_wait<0>,
    or two stages each reused after store_wait<1>, every load in the
    barrier form; the destination bit-exact against the oracle (sentinel
    outside the boxes), the group sizes equal to the whole-chunk groups of
    each box, every wave's barrier waits completed."""
    L = staged_lib()
    dims, strides, box = (512, 256), (1024,), (64, 128)
    src = synthgen.u16_bits(81, (256, 512))
    sentinel = np.full((256, 512), 0xBEEF, dtype=np.uint16)
    coords = np.array([[0, 0], [64, 0], [128, 128], [320, 0], [192, 128], [384, 128], [-100, -300],
                       [480, 200], [256, 64 - 128], [0, 128]], dtype=np.int32)
    sd, dd = to_dev(src), to_dev(sentinel)
    ms = encode(sd, "bf16", dims, strides, box, None, "128b")
    md = encode(dd, "bf16", dims, strides, box, None, "128b")
    cd = to_dev(coords)
    sizes = torch.full((len(coords),), -1, dtype=torch.int32, device="cuda")
    landed = torch.zeros(4, dtype=torch.int32, device="cuda")
    say("store groups", stages, wait_n)
    rc = L.user_staged_copy_launch(ctypes.byref(ms), ctypes.byref(md), cd.data_ptr(), 2, len(coords), stages,
                                   att.tmap_box_bytes(ms), sizes.data_ptr(), landed.data_ptr(), stream())
    assert rc == 0, rc
    got = to_host(dd).view(np.uint16).reshape(256, 512)
    om = oracle.Map("bf16", dims, strides, box, swizzle="128b")
    want = sentinel.copy()
    om.store(want, coords, om.load(src, coords))
    np.testing.assert_array_equal(got, want)
    assert (to_host(landed) == 1).all()
    assert to_host(sizes).tolist() == [whole_chunk_groups(dims, box, c) for c in coords.tolist()]
