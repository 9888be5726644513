"""The device API header (include/tile.hpp) is self-contained: a user kernel
that includes only it, with only include/ on the path, compiles for gfx950
and uses every documented call.  The library's own batch kernels are written
against the same calls, so the GPU parity tests of tile_load, tile_store,
tile_reduce, tile_load_im2col and txbar_selftest run through them."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

USER_KERNEL = r"""
#include "tile.hpp"

// Load one box, reduce it into a second tensor and store it into a third;
// then an im2col load of the same workgroup's LDS.
__global__ __launch_bounds__(256) void user_tiles(tmap_t src, tmap_t acc, tmap_t dst, tmap_t win,
                                                  const int32_t* coords, int32_t* ok) {
    __shared__ att::TxBar bar;
    extern __shared__ __attribute__((aligned(1024))) uint8_t img[];
    const uint32_t w = threadIdx.x / 64, nw = blockDim.x / 64;
    int32_t c[5];
    for (int d = 0; d < 5; ++d) c[d] = coords[blockIdx.x * 5 + d];
    if (threadIdx.x == 0) {
        att::txbar_init(&bar, 1);
        att::txbar_arrive_expect_tx(&bar, (int32_t)att::tile_box_bytes(src));
    }
    __syncthreads();
    const uint32_t bytes = att::tile_load_async(src, c, img, w, nw);
    att::tile_load_arrive(&bar, bytes);
    const bool landed = att::txbar_wait(&bar, 0);
    __syncthreads();
    att::tile_reduce_async<TMAP_REDUCE_ADD>(acc, c, img, w, nw);
    att::tile_reduce_async<TMAP_REDUCE_MIN>(acc, c, img, w, nw);
    att::tile_reduce_async<TMAP_REDUCE_MAX>(acc, c, img, w, nw);
    att::tile_store_async(dst, c, img, w, nw);
    att::tile_store_wait();
    __syncthreads();
    if (threadIdx.x == 0) {
        att::txbar_init(&bar, (int32_t)nw);
    }
    __syncthreads();
    const int32_t off[3] = {1, 1, 0};
    // every wave announces, reports and arrives for its own share
    const uint32_t b2 = att::tile_load_im2col_async(win, c, off, img, w, nw);
    if (att::lane_id() == 0) att::txbar_expect_tx(&bar, (int32_t)b2);
    att::tile_load_arrive(&bar, b2);
    if (att::lane_id() == 0) att::txbar_arrive(&bar, 1);
    const bool again = att::txbar_try_wait(&bar, 0) || att::txbar_wait(&bar, 0);
    if (threadIdx.x == 0) ok[blockIdx.x] = (int32_t)(landed && again) + (int32_t)att::tmap_tiled(src).rank;
}
"""


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_user_kernel_compiles_against_public_header_only(tmp_path):
    src = tmp_path / "user_tiles.hip"
    src.write_text(USER_KERNEL)
    asm = tmp_path / "user_tiles.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument",
           "--cuda-device-only", "-S", str(src), "-o", str(asm)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    text = asm.read_text()
    assert "user_tiles" in text
    # the load goes through the LDS DMA, the reductions through atomics
    assert "global_load_lds_dwordx4" in text
    assert re.search(r"global_atomic_\w+", text)
    # nothing private: the map is read from the kernel arguments
    m = re.search(r"\.private_segment_fixed_size:\s+(\d+)", text)
    assert m and int(m.group(1)) == 0


def test_public_headers_do_not_reach_into_the_package():
    inc = os.path.join(ROOT, "include")
    for dirpath, _, files in os.walk(inc):
        for f in files:
            text = open(os.path.join(dirpath, f)).read()
            for m in re.finditer(r'#include\s+"([^"]+)"', text):
                target = m.group(1)
                here = os.path.join(dirpath, target)
                top = os.path.join(inc, target)
                assert os.path.exists(here) or os.path.exists(top), (f, target)


def test_batch_kernels_use_the_device_api():
    text = open(os.path.join(ROOT, "async_tensor_tile_amd", "csrc", "kernels_tile.hip")).read()
    assert '#include "tile.hpp"' in text
    for call in ("tile_load_async(", "tile_load_arrive(", "tile_store_async(", "tile_reduce_async<",
                 "tile_load_im2col_async(", "tile_box_bytes("):
        assert call in text, call
