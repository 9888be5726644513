"""GPU checks of the HBM streaming probe used for the bandwidth ceiling the
benchmark reports beside the tile copy: the copy is bit-exact (ragged sizes
included), the write covers exactly the requested bytes, the read leaves
its sink alone for ordinary data."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402

from gpu_util import require_native, stream  # noqa: E402

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_native()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 20, (1 << 24) + 16 * 777])
def test_probe_copy_write_read(nbytes):
    print("hbm_probe", nbytes, flush=True)
    rng = np.random.default_rng(nbytes)
    src = torch.from_numpy(rng.integers(0, 256, nbytes + 64, dtype=np.uint8)).cuda()
    dst = torch.full((nbytes + 64,), 0xEE, dtype=torch.uint8, device="cuda")
    att.hbm_probe("copy", src, dst, nbytes, stream())
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert (dst[nbytes:] == 0xEE).all()
    att.hbm_probe("write", None, dst, nbytes, stream())
    torch.cuda.synchronize()
    assert not torch.equal(dst[:nbytes], src[:nbytes]) or nbytes == 0
    assert (dst[nbytes:] == 0xEE).all()
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    att.hbm_probe("read", src, sink, nbytes, stream())
    torch.cuda.synchronize()


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (1 << 22) + 16 * 333])
def test_probe_copy_variants(nbytes):
    """Every launch shape of the ceiling sweep copies exactly the requested
    bytes (ragged sizes, every vector count, store kind and order, 1 to 16
    workgroups per CU)."""
    print("hbm_probe_copy_ex", nbytes, flush=True)
    rng = np.random.default_rng(nbytes + 1)
    src = torch.from_numpy(rng.integers(0, 256, nbytes + 64, dtype=np.uint8)).cuda()
    for variant in range(16):
        for wpc in (1, 2, 16):
            dst = torch.full((nbytes + 64,), 0xEE, dtype=torch.uint8, device="cuda")
            att.hbm_probe_copy_ex(src, dst, nbytes, variant, wpc, stream())
            torch.cuda.synchronize()
            assert torch.equal(dst[:nbytes], src[:nbytes]), (variant, wpc)
            assert (dst[nbytes:] == 0xEE).all(), (variant, wpc)


def test_probe_box_copy_variants():
    """The box-shaped register copy moves every byte of the matrix for every
    boxes-per-workgroup count and variant (the rotated row walk on a matrix
    with more box rows than boxes per row, so the rotation wraps)."""
    W_, H_ = 4096, 5120
    rng = np.random.default_rng(7)
    src = torch.from_numpy(rng.integers(0, 256, W_ * H_, dtype=np.uint8)).cuda()
    for nbx in (1, 2, 4, 8):
        for variant in list(range(8)) + [32, 33, 35, 39]:
            dst = torch.zeros_like(src)
            att.hbm_probe_box_copy(src, dst, W_, H_, nbx, variant, stream())
            torch.cuda.synchronize()
            assert torch.equal(dst, src), (nbx, variant)
