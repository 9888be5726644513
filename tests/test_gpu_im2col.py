"""GPU parity for the im2col-mode load: the LDS images written by
tile_load_im2col equal the oracle's bit for bit -- random channel-innermost
tensors of rank 3..5 and every element type, corners, convolution strides,
filter-tap offsets, swizzles and fills, starts inside and outside the window
grid, channel coordinates negative, unaligned or past the end -- and a
convolution-shaped workload (bf16 NHWC 8 x 56 x 56 x 64, 3 x 3 window,
padding 1, every tap over every window)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402

from gpu_util import empty_dev, require_native, stream, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu

ESIZE = {"u8": 1, "u16": 2, "u32": 4, "i32": 4, "u64": 8, "i64": 8, "f16": 2, "bf16": 2, "f32": 4, "f64": 8}
SPAN = {32: "32b", 64: "64b", 128: "128b"}


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_case(dtype, dims, strides, lower, upper, channels, pixels, estride, swizzle, fill, buf, coords, offsets):
    rank = len(dims)
    om = oracle.Im2colMap(dtype, dims, strides, lower, upper, channels, pixels, estride, swizzle, fill)
    assert om.validate() == "OK"
    want = om.load(buf, coords, offsets)
    sd = to_dev(buf)
    m = att.tmap_encode_im2col(dtype, rank, sd.data_ptr(), dims, strides, lower, upper, channels, pixels,
                               estride, swizzle, fill)
    nb = len(coords)
    out = empty_dev(nb * om.box_bytes(), 0xCD)
    c = to_dev(np.asarray(coords, dtype=np.int32).reshape(nb, rank))
    o = to_dev(np.asarray(offsets, dtype=np.int32).reshape(nb, rank - 2))
    att.tile_load_im2col(m, c, o, nb, out, stream())
    got = to_host(out).reshape(nb, -1)
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("seed", range(24))
def test_im2col_random_configs(seed):
    g = synthgen.rng(70000 + seed)
    dtype = ["u8", "u16", "u32", "i32", "u64", "i64", "f16", "bf16", "f32", "f64"][seed % 10]
    es = ESIZE[dtype]
    rank = 3 + seed % 3
    S = rank - 2
    step = 16 // es
    channels = step * int(g.integers(1, 5))
    C = int(g.integers(1, 3 * channels + 2))
    spatial = [int(g.integers(1, 9)) for _ in range(S)]
    N = int(g.integers(1, 4))
    dims = [C] + spatial + [N]
    strides, acc = [], C * es
    for d in range(1, rank):
        acc = (acc + 15) // 16 * 16 + 16 * int(g.integers(0, 2))     # padded strides
        strides.append(acc)
        acc *= dims[d]
    estride = [1] + [int(g.integers(1, 4)) for _ in range(S)] + [1]
    lower, upper = [], []
    for s in range(S):
        lo = int(g.integers(-3, 2))
        hi_min = lo - (spatial[s] - 1)            # keep the grid non-empty: dim - 1 + upper >= lower
        up = int(g.integers(max(-3, hi_min), 2))
        lower.append(lo)
        upper.append(up)
    row_bytes = channels * es
    swizzle = "none"
    if row_bytes in SPAN and g.integers(0, 3):
        swizzle = SPAN[row_bytes] + ("_k256" if g.integers(0, 2) else "")
    fill = "nan" if dtype in ("f16", "bf16", "f32", "f64") and g.integers(0, 2) else "zero"
    pixels = int(g.integers(1, 80))
    say("im2col", seed, dtype, dims, strides, lower, upper, channels, pixels, estride, swizzle, fill)
    buf = synthgen.random_bytes(seed + 500, strides[-1] * dims[-1])
    coords, offsets = [], []
    for b in range(20):
        ch = int(g.integers(-step, C + step)) if b % 5 else 0
        if b % 7 == 3:
            ch += 1                              # channel coordinate off the 16-byte grid
        sp = [int(g.integers(lower[s] - 2 * estride[s + 1], spatial[s] + 3)) for s in range(S)]
        img = int(g.integers(-1, N + 1))
        coords.append([ch] + sp + [img])
        offsets.append([int(g.integers(0, 4)) for _ in range(S)])
    run_case(dtype, dims, strides, lower, upper, channels, pixels, estride, swizzle, fill, buf, coords, offsets)


def test_im2col_conv_workload():
    """bf16 NHWC 8 x 56 x 56 x 64, 3 x 3 window, padding 1, stride 1: 128-pixel
    boxes of all 64 channels (128-byte rows, 128-byte swizzle) for every tap
    over every window -- the loads an implicit-GEMM convolution issues."""
    N, H, W, C = 8, 56, 56, 64
    k, pad, P = 3, 1, 128
    x = synthgen.normal_bf16_bits(77, (N, H, W, C))
    dims = (C, W, H, N)
    strides = (C * 2, W * C * 2, H * W * C * 2)
    lower, upper = (-pad, -pad), (pad - k + 1, pad - k + 1)
    total = N * H * W
    coords, offsets = [], []
    for L0 in range(0, total, P):
        t_w, t_h, n = L0 % W, (L0 // W) % H, L0 // (W * H)
        for i in range(k):
            for j in range(k):
                coords.append((0, -pad + t_w, -pad + t_h, n))
                offsets.append((j, i))
    say("conv workload boxes", len(coords))
    run_case("bf16", dims, strides, lower, upper, C, P, (1, 1, 1, 1), "128b", "zero", x.view(np.uint8),
             coords, offsets)


def test_im2col_degenerate():
    """One pixel of one 16-byte chunk; starts wholly outside (every element is
    fill); a single-position grid."""
    x = synthgen.random_bytes(88, 4 * 3 * 16)
    dims, strides = (4, 3, 4), (16, 48)
    run_case("f32", dims, strides, (0,), (0,), 4, 1, (1, 1, 1), "none", "nan", x,
             [(0, 0, 0), (0, 2, 3), (-4, 0, 0), (4, 0, 0), (0, 0, 9), (0, -5, -1)], [(0,), (0,), (0,), (0,), (0,), (7,)])
    run_case("u8", (16, 5, 2), (16, 80), (2,), (-2,), 16, 7, (1, 1, 1), "none", "zero",
             synthgen.random_bytes(89, 160), [(0, 2, 0), (0, 3, 1)], [(0,), (1,)])
