"""Pins for the oracle's im2col-mode load.  The pages name im2col tensor-map
encoding (with its own swizzle parameter) and define nothing further, so the
definition is a reading (channel-innermost tensor, window origins on a
per-dimension grid between a lower and an upper corner, consecutive origins
W-fastest then H, D and image, channels from the load's channel coordinate,
filter-tap offsets added to the origin, outside elements filled).  It is
pinned here against torch's unfold -- the library routine that lays out
exactly these patches for 1-D and 2-D convolutions -- and against a NumPy
pad-and-index formulation for 3-D."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synthgen

from test_oracle_pins import page_swizzle_128b


def nhwc_map(x, k, pad, stride, cp, pixels, swizzle="none", fill="zero", dtype="f32"):
    """Im2col map over an (N, H, W, C) array for a k x k window."""
    N, H, W, C = x.shape
    es = x.itemsize
    dims = (C, W, H, N)
    strides = (C * es, W * C * es, H * W * C * es)
    lo = (-pad, -pad)
    up = (pad - k + 1, pad - k + 1)
    return oracle.Im2colMap(dtype, dims, strides, lo, up, cp, pixels, (1, stride, stride, 1), swizzle, fill)


def unfold_expect(x, k, pad, stride, c0, tap, L0, cp, pixels):
    """Image rows from torch's unfold: unfold[n, c*k*k + i*k + j, l] is input
    channel c at window l shifted by tap (i, j); windows continue into the next
    image, and anything past the last image or channel is fill (zero)."""
    N, H, W, C = x.shape
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 3, 1, 2)))
    unf = F.unfold(xt, (k, k), padding=pad, stride=stride).numpy()
    L = unf.shape[2]
    i, j = tap
    out = np.zeros((pixels, cp), dtype=x.dtype)
    for p in range(pixels):
        n, l = divmod(L0 + p, L)
        if n >= N:
            continue
        for kk in range(cp):
            c = c0 + kk
            if c < C:
                out[p, kk] = unf[n, c * k * k + i * k + j, l]
    return out


def start_coords(L0, pad, stride, ow, oh, c0):
    t_w = L0 % ow
    t_h = (L0 // ow) % oh
    n0 = L0 // (ow * oh)
    return (c0, -pad + t_w * stride, -pad + t_h * stride, n0)


@pytest.mark.parametrize("N,H,W,C,k,pad,stride,cp,pixels", [
    (2, 9, 11, 8, 3, 1, 2, 8, 16),
    (1, 7, 7, 16, 3, 0, 1, 8, 32),
    (3, 5, 6, 4, 2, 1, 1, 4, 40),
    (2, 8, 8, 12, 5, 2, 3, 4, 9),
])
def test_im2col_2d_matches_unfold(N, H, W, C, k, pad, stride, cp, pixels):
    x = synthgen.normal_f32(900 + C, (N, H, W, C))
    m = nhwc_map(x, k, pad, stride, cp, pixels)
    assert m.validate() == "OK"
    oh = (H + 2 * pad - k) // stride + 1
    ow = (W + 2 * pad - k) // stride + 1
    total = N * oh * ow
    g = synthgen.rng(901)
    cases = [(c0, (i, j), int(L0)) for c0 in range(0, C, cp) for i in range(k) for j in range(k)
             for L0 in (0, total - 1, int(g.integers(0, total)))]
    coords = [start_coords(L0, pad, stride, ow, oh, c0) for c0, _, L0 in cases]
    offsets = [(j, i) for _, (i, j), _ in cases]          # offsets listed W first
    got = m.load(x, coords, offsets).view(np.float32).reshape(len(cases), pixels, cp)
    for b, (c0, tap, L0) in enumerate(cases):
        want = unfold_expect(x, k, pad, stride, c0, tap, L0, cp, pixels)
        np.testing.assert_array_equal(got[b], want, err_msg=str((c0, tap, L0)))


def test_im2col_1d_matches_unfold():
    """Rank 3 (C, W, N): a 1-D convolution, unfold over a height-1 image."""
    N, W, C, k, pad, stride, cp, pixels = 3, 17, 8, 3, 1, 2, 8, 20
    x = synthgen.normal_f32(910, (N, W, C))
    m = oracle.Im2colMap("f32", (C, W, N), (C * 4, W * C * 4), (-pad,), (pad - k + 1,), cp, pixels,
                         (1, stride, 1))
    assert m.validate() == "OK"
    ow = (W + 2 * pad - k) // stride + 1
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1)))[:, :, None, :]
    unf = F.unfold(xt, (1, k), padding=(0, pad), stride=(1, stride)).numpy()
    for j in range(k):
        for L0 in (0, 5, N * ow - 3):
            got = m.load(x, [(0, -pad + (L0 % ow) * stride, L0 // ow)], [(j,)]).view(np.float32).reshape(pixels, cp)
            want = np.zeros((pixels, cp), np.float32)
            for p in range(pixels):
                n, l = divmod(L0 + p, ow)
                if n < N:
                    want[p] = unf[n, np.arange(cp) * k + j, l]
            np.testing.assert_array_equal(got, want)


def test_im2col_3d_pad_and_index():
    """Rank 5 (C, W, H, D, N): a 3-D window, checked against a zero-padded
    NumPy array indexed at origin * stride + tap."""
    N, D, H, W, C = 2, 4, 5, 6, 4
    k, pad, stride, cp, pixels = 3, 1, 2, 4, 30
    x = synthgen.normal_f32(920, (N, D, H, W, C))
    es = 4
    m = oracle.Im2colMap("f32", (C, W, H, D, N), (C * es, W * C * es, H * W * C * es, D * H * W * C * es),
                         (-pad,) * 3, (pad - k + 1,) * 3, cp, pixels, (1, stride, stride, stride, 1))
    assert m.validate() == "OK"
    od, oh, ow = [(n + 2 * pad - k) // stride + 1 for n in (D, H, W)]
    xp = np.pad(x, ((0, 0), (pad, pad), (pad, pad), (pad, pad), (0, 0)))
    for tap in ((0, 0, 0), (2, 1, 0), (1, 2, 2)):
        for L0 in (0, 7, N * od * oh * ow - 5):
            t_w, r = L0 % ow, L0 // ow
            t_h, r = r % oh, r // oh
            t_d, n0 = r % od, r // od
            coords = (0, -pad + t_w * stride, -pad + t_h * stride, -pad + t_d * stride, n0)
            got = m.load(x, [coords], [tap]).view(np.float32).reshape(pixels, cp)
            want = np.zeros((pixels, cp), np.float32)
            for p in range(pixels):
                L = L0 + p
                w_, L = L % ow, L // ow
                h_, L = L % oh, L // oh
                d_, n = L % od, L // od
                if n < N:
                    want[p] = xp[n, d_ * stride + tap[2], h_ * stride + tap[1], w_ * stride + tap[0], :cp]
            np.testing.assert_array_equal(got, want, err_msg=str((tap, L0)))


def test_im2col_swizzle_and_nan_fill():
    """128-byte rows (32 f32 channels) under the 128-byte swizzle give the
    pages' per-row sector permutation of the unswizzled image; padding
    positions carry the canonical NaN with NaN fill."""
    x = synthgen.normal_f32(930, (1, 6, 6, 32))
    plain = nhwc_map(x, 3, 1, 1, 32, 16)
    sw = nhwc_map(x, 3, 1, 1, 32, 16, swizzle="128b")
    nanm = nhwc_map(x, 3, 1, 1, 32, 16, fill="nan")
    coords, offs = [(0, -1, -1, 0)], [(0, 0)]
    a = plain.load(x, coords, offs)[0]
    np.testing.assert_array_equal(sw.load(x, coords, offs)[0], page_swizzle_128b(a))
    b = nanm.load(x, coords, offs)[0].view(np.uint32).reshape(16, 32)
    # pixels 0..5 sit at origin row -1 (all taps (0,0) read row -1: padding)
    assert (b[:6] == 0x7FC00000).all()
    # pixel 6: origin (-1, 0): column -1 is padding
    assert (b[6] == 0x7FC00000).all()
    # pixel 7: origin (0, 0): inside
    np.testing.assert_array_equal(b[7].view(np.float32), x[0, 0, 0])


def test_im2col_start_snaps_to_grid():
    """A start between grid positions behaves as the grid position below it;
    a start one past the last W position is the first of the next row."""
    x = synthgen.normal_f32(940, (2, 9, 9, 8))
    m = nhwc_map(x, 3, 1, 2, 8, 12)
    ow = (9 + 2 - 3) // 2 + 1
    a = m.load(x, [(0, -1 + 2 * 2, -1 + 2 * 1, 0)], [(1, 1)])
    b = m.load(x, [(0, -1 + 2 * 2 + 1, -1 + 2 * 1, 0)], [(1, 1)])
    np.testing.assert_array_equal(a, b)
    c = m.load(x, [(0, -1 + 2 * ow, -1 + 2 * 1, 0)], [(1, 1)])
    d = m.load(x, [(0, -1, -1 + 2 * 2, 0)], [(1, 1)])
    np.testing.assert_array_equal(c, d)


def _im(**kw):
    base = dict(dtype="f32", dims=(8, 11, 9, 2), strides=(32, 352, 3168), lower=(-1, -1), upper=(-1, -1),
                channels=8, pixels=16, estride=(1, 2, 2, 1), swizzle="none", fill="zero")
    base.update(kw)
    return oracle.Im2colMap(base["dtype"], base["dims"], base["strides"], base["lower"], base["upper"],
                            base["channels"], base["pixels"], base["estride"], base["swizzle"], base["fill"])


@pytest.mark.parametrize("kw,status", [
    (dict(), "OK"),
    (dict(dims=(8, 11), strides=(32,), lower=(), upper=(), estride=(1, 1)), "ERR_RANK"),
    (dict(channels=6), "ERR_BOX"), (dict(channels=0), "ERR_BOX"), (dict(channels=260), "ERR_BOX"),
    (dict(pixels=0), "ERR_BOX"), (dict(pixels=1025), "ERR_BOX"),
    (dict(estride=(2, 2, 2, 1)), "ERR_ESTRIDE"), (dict(estride=(1, 9, 2, 1)), "ERR_ESTRIDE"),
    (dict(estride=(1, 2, 2, 2)), "ERR_ESTRIDE"),
    (dict(upper=(-12, -1)), "ERR_BOX"), (dict(lower=(40000, 0)), "ERR_BOX"),
    (dict(swizzle="128b"), "ERR_SWIZZLE_WIDTH"), (dict(channels=32, swizzle="128b"), "OK"),
    (dict(dtype="i32", fill="nan"), "ERR_OOB_FILL_DTYPE"),
    (dict(channels=256, pixels=1024), "ERR_LDS_CAPACITY"),
    (dict(strides=(24, 352, 3168)), "ERR_STRIDE"),
    # the pages set no bound on the number of windows: 2^98 windows validate
    (dict(dims=(8, 1 << 32, 1 << 32, 1 << 32, 4), strides=(32, 1 << 35, 1 << 36, 1 << 37), lower=(0, 0, 0),
          upper=(0, 0, 0), estride=(1, 1, 1, 1, 1)), "OK"),
])
def test_im2col_validate(kw, status):
    assert _im(**kw).validate() == status
