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
