"""GPU parity for the bf16 GEMM mainloop fed by the tile loader: exact special
cases (identity, permutation), full comparison against the fp64 oracle on
sizes spanning several tiles and ragged edges, and 4096 sampled outputs at
M = N = K = 8192.  Tolerance: |C - ref| <= 2e-2 + 2^-8 |ref| (fp32
accumulation plus one bf16 rounding of the output)."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402
from synthgen import workloads as W  # noqa: E402

from gpu_util import require_native, stream  # noqa: E402

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def run_gemm(A_bits, Bt_bits, M, N, K, bk=64, stages=2, group_m=0, xcd=1, k256=False, mfma=0):
    """A_bits (M, K) row-major; Bt_bits (N, K) = column-major B.  Rows are
    stored with a leading dimension padded to a multiple of 8 elements (the
    maps need 16-byte strides).  Returns the bf16 bits of C (M, N)."""
    ld = (K + 7) // 8 * 8
    Ap = np.zeros((M, ld), dtype=np.uint16)
    Ap[:, :K] = A_bits
    Bp = np.zeros((N, ld), dtype=np.uint16)
    Bp[:, :K] = Bt_bits
    Ad = torch.from_numpy(Ap.view(np.int16)).cuda()
    Bd = torch.from_numpy(Bp.view(np.int16)).cuda()
    Cd = torch.full((M, N), 0x7FFF, dtype=torch.int16, device="cuda")
    sw = ("128b" if bk == 64 else "64b") + ("_k256" if k256 else "")
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (ld * 2,), (bk, 256), None, sw)
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (ld * 2,), (bk, 256), None, sw)
    att.gemm_bf16_ex(mA, mB, Cd.data_ptr(), M, N, K, N, stages, group_m, xcd, stream(), mfma)
    torch.cuda.synchronize()
    return Cd.cpu().numpy().view(np.uint16)


def check_close(got_bits, ref):
    got = bf16_to_f64(got_bits)
    tol = 2e-2 + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} outputs out of tolerance, worst {err.max()}"


@pytest.mark.parametrize("k256", [False, True])
@pytest.mark.parametrize("bk,stages,mfma", [(64, 2, 16), (64, 2, 32), (64, 3, 16), (32, 2, 32), (32, 3, 32),
                                           (32, 4, 32), (32, 5, 32)])
def test_identity_exact(bk, stages, mfma, k256):
    """A = I: C equals B exactly (one product per output, exact in fp32)."""
    K = N = 512
    M = K
    eye = np.zeros((M, K), dtype=np.uint16)
    eye[np.arange(M), np.arange(K)] = 0x3F80
    Bt = synthgen.normal_bf16_bits(51, (N, K))
    C = run_gemm(eye, Bt, M, N, K, bk, stages, k256=k256, mfma=mfma)
    np.testing.assert_array_equal(C, Bt.T)


def test_mfma_shape_argument():
    """mfma 16 needs the 64-deep K step; unknown shapes are rejected."""
    A = np.zeros((256, 64), dtype=np.uint16)
    with pytest.raises(att.TmapError) as ei:
        run_gemm(A, A, 256, 256, 64, 32, 2, mfma=16)
    assert ei.value.name == "ERR_UNSUPPORTED"
    with pytest.raises(att.TmapError) as ei:
        run_gemm(A, A, 256, 256, 64, 64, 2, mfma=8)
    assert ei.value.name == "ERR_UNSUPPORTED"


@pytest.mark.parametrize("K", [64, 128, 192, 320, 384, 704])
@pytest.mark.parametrize("k256", [False, True])
def test_operand_ring(K, k256):
    """64-deep boxes, three stages: the five-slot operand ring
    (A three deep, B two deep, loop unrolled by five).  K from one K-step up
    to two unrolled groups plus one, so every slot pattern and the clamped
    copies past the last K-step run."""
    M, N = 512, 256
    say("gemm ring5", K, k256)
    A = synthgen.normal_bf16_bits(58, (M, K))
    Bt = synthgen.normal_bf16_bits(59, (N, K))
    C = run_gemm(A, Bt, M, N, K, 64, 3, k256=k256, mfma=16)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_close(C, ref)


@pytest.mark.parametrize("K,M,N", [(64, 4352, 4352), (128, 4352, 4352), (192, 4352, 4352), (576, 4352, 4352),
                                   (192, 4252, 4315), (128, 4097, 33)])
def test_operand_ring_many_tiles_exact(K, M, N):
    """More 256 x 256 tiles (17 x 17) than the GPU has CUs, so workgroups of
    the operand ring run in several rounds, whole or with partial tiles in M
    and N.  A selects one K index per row (A[m, sel[m]] = 1), so C[m, :] =
    B[sel[m], :] exactly: every output of every tile checked."""
    say("gemm ring5 many tiles", K, M, N)
    sel = synthgen.rng(62).integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), sel] = 0x3F80
    Bt = synthgen.normal_bf16_bits(63, (N, K))
    C = run_gemm(A, Bt, M, N, K, 64, 3, k256=True, mfma=16)
    np.testing.assert_array_equal(C, Bt[:, sel].T)


@pytest.mark.parametrize("offset,ldc", [(0, 264), (1, 264), (0, 258)])
def test_operand_ring_c_leading_dimension(offset, ldc):
    """The operand ring's C epilogue with leading dimension ldc >= N: the
    LDS-staged tile store (16-byte aligned C, ldc a multiple of 8) and the
    element stores otherwise; padding columns and the bytes around C stay
    untouched."""
    M, N, K = 512, 256, 192
    say("gemm ring5 ldc", offset, ldc)
    A = synthgen.normal_bf16_bits(64, (M, K))
    Bt = synthgen.normal_bf16_bits(65, (N, K))
    Ad = torch.from_numpy(A.view(np.int16)).cuda()
    Bd = torch.from_numpy(Bt.view(np.int16)).cuda()
    buf = torch.full((M * ldc + 16,), 0x7FFF, dtype=torch.int16, device="cuda")
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (K * 2,), (64, 256), None, "128b_k256")
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (K * 2,), (64, 256), None, "128b_k256")
    att.gemm_bf16(mA, mB, buf.data_ptr() + 2 * offset, M, N, K, ldc, 3, stream())
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint16)
    C = out[offset:offset + M * ldc].reshape(M, ldc)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_close(C[:, :N], ref)
    assert (C[:, N:] == 0x7FFF).all()
    assert (out[:offset] == 0x7FFF).all() and (out[offset + M * ldc:] == 0x7FFF).all()


def test_operand_ring_shape_limits():
    """The operand ring takes K a multiple of 64 and 16 x 16 x 32 MFMAs;
    other requests for three 64-deep stages are rejected, as are 16 x 16
    MFMAs with 32-deep boxes."""
    A = np.zeros((300, 128), dtype=np.uint16)
    for args in [(256, 256, 96, 64, 3, 16), (256, 256, 128, 64, 3, 32), (256, 256, 128, 32, 5, 16)]:
        M, N, K, bk, st, mf = args
        with pytest.raises(att.TmapError) as ei:
            run_gemm(A[:M, :K], A[:N, :K], M, N, K, bk, st, mfma=mf)
        assert ei.value.name == "ERR_UNSUPPORTED", args


def test_permutation_exact():
    K = N = M = 768
    perm = synthgen.rng(52).permutation(K)
    P = np.zeros((M, K), dtype=np.uint16)
    P[np.arange(M), perm] = 0x3F80
    Bt = synthgen.normal_bf16_bits(53, (N, K))
    C = run_gemm(P, Bt, M, N, K)
    np.testing.assert_array_equal(C, Bt.T[perm])


@pytest.mark.parametrize("M,N,K,bk,stages,k256,mfma", [
    (512, 768, 1024, 64, 2, False, 0), (768, 512, 1024, 32, 3, False, 0), (512, 512, 2048, 32, 4, False, 0),
    (512, 768, 1024, 64, 2, True, 0), (768, 512, 1024, 32, 4, True, 0), (300, 200, 100, 32, 3, True, 0),
    (300, 200, 100, 64, 2, False, 0), (257, 513, 96, 32, 2, False, 0), (1, 1, 64, 64, 2, False, 0),
    (256, 256, 8, 64, 2, False, 0), (512, 768, 1024, 64, 2, True, 32), (300, 200, 100, 64, 2, True, 32),
    (257, 513, 96, 64, 2, True, 16), (1, 1, 64, 64, 2, True, 16),
    # partial M / N tiles with K a multiple of the box depth: the fast loader
    # with clamped rows (double buffer, operand ring, 32-deep ring)
    (300, 200, 192, 64, 2, True, 16), (257, 513, 128, 64, 3, True, 16), (1, 1, 64, 64, 3, False, 16),
    (300, 520, 320, 64, 3, False, 0), (511, 257, 128, 32, 4, True, 0), (300, 200, 192, 64, 2, False, 32),
    # K not a multiple of the box depth with two slots: the fast loader, and
    # the general loader for the partial last K tile only
    (512, 256, 4000, 64, 2, True, 16), (300, 520, 136, 64, 2, False, 32), (256, 256, 40, 64, 2, True, 0),
    (257, 300, 1000, 32, 2, True, 0)])
def test_against_oracle_full(M, N, K, bk, stages, k256, mfma):
    say("gemm", M, N, K, bk, stages, k256, mfma)
    A = synthgen.normal_bf16_bits(54, (M, K))
    Bt = synthgen.normal_bf16_bits(55, (N, K))
    C = run_gemm(A, Bt, M, N, K, bk, stages, k256=k256, mfma=mfma)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_close(C, ref)


@pytest.mark.parametrize("bk,stages,k256,mfma", [(64, 2, False, 0), (32, 4, True, 0), (64, 2, True, 16),
                                                 (64, 2, True, 32), (64, 3, True, 16)])
def test_8192_sampled(bk, stages, k256, mfma):
    ex = W.GEMM_8192
    M, N, K = ex["M"], ex["N"], ex["K"]
    say("gemm 8192^3", bk, stages, k256, mfma)
    A = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 1, (M, K))
    Bt = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 2, (N, K))
    C = run_gemm(A, Bt, M, N, K, bk, stages, k256=k256, mfma=mfma)
    rows, cols = synthgen.sample_pairs(ex["seed"] * 1000 + 3, ex["nsample"], M, N)
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows, cols)
    check_close(C[rows, cols], ref)
    # the unsampled output is finite and was written everywhere
    assert not (C == 0x7FFF).any()


# Tile grids (256 x 256 C tiles) for the rasterisation orders: 8 x 4 and
# 12 x 2 let xcd = 2 give each XCD a 2-D block, 4 x 6 gives 1 x 3 blocks;
# 2000 x 1000 has partial last tiles on the same 8 x 4 grid; 5 x 3 tiles
# (15 workgroups) make both XCD-aware orders fall back to plain order.
RASTER_GRIDS = [(2048, 1024), (3072, 512), (1024, 1536), (2000, 1000), (1280, 768)]


@pytest.mark.parametrize("stages", [2, 3])
@pytest.mark.parametrize("MN", RASTER_GRIDS)
@pytest.mark.parametrize("group_m", [1, 3, 4, 8])
@pytest.mark.parametrize("xcd", [0, 1, 2])
def test_raster_orders_exact(xcd, group_m, MN, stages):
    """Every rasterisation order writes every C tile, with the right data:
    A selects one K index per row, so C[m, :] = B[sel[m], :] exactly and a
    tile that is skipped (left at the sentinel) or taken from the wrong A /
    B panel fails."""
    M, N = MN
    K = 128
    say("gemm raster", xcd, group_m, M, N, stages)
    sel = synthgen.rng(66).integers(0, K, M)
    A = np.zeros((M, K), dtype=np.uint16)
    A[np.arange(M), sel] = 0x3F80
    Bt = synthgen.normal_bf16_bits(67, (N, K))
    C = run_gemm(A, Bt, M, N, K, 64, stages, group_m=group_m, xcd=xcd, k256=True, mfma=16)
    np.testing.assert_array_equal(C, Bt[:, sel].T)


_OPERANDS_8192 = {}


def _operands_8192():
    if not _OPERANDS_8192:
        ex = W.GEMM_8192
        M, N, K = ex["M"], ex["N"], ex["K"]
        _OPERANDS_8192["A"] = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 1, (M, K))
        _OPERANDS_8192["Bt"] = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 2, (N, K))
    return _OPERANDS_8192["A"], _OPERANDS_8192["Bt"]


@pytest.mark.parametrize("xcd,group_m", [(0, 1), (0, 8), (2, 4), (2, 8)])
def test_8192_sampled_rasters(xcd, group_m):
    """The full-size product under the rasterisation orders the benchmark
    times beside the default: 4096 sampled outputs against the oracle, and
    every output written."""
    ex = W.GEMM_8192
    M, N, K = ex["M"], ex["N"], ex["K"]
    say("gemm 8192^3 raster", xcd, group_m)
    A, Bt = _operands_8192()
    C = run_gemm(A, Bt, M, N, K, 64, 3, group_m=group_m, xcd=xcd, k256=True, mfma=16)
    rows, cols = synthgen.sample_pairs(ex["seed"] * 1000 + 3, ex["nsample"], M, N)
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows, cols)
    check_close(C[rows, cols], ref)
    assert not (C == 0x7FFF).any()


def _random_gemm_case(seed):
    g = synthgen.rng(90000 + seed)
    bk, stages, mfma = [(64, 2, 16), (64, 2, 32), (64, 3, 16), (64, 2, 0), (32, 2, 32), (32, 3, 32),
                        (32, 4, 32), (32, 5, 32)][int(g.integers(0, 8))]
    M, N = (int(x) for x in g.integers(1, 1100, 2))
    K = int(g.integers(1, 900))
    if stages == 3 and bk == 64:
        K = max(64, K // 64 * 64)          # the operand ring takes K a multiple of 64
    return M, N, K, bk, stages, mfma, bool(g.integers(0, 2))


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes_sampled(seed):
    """Random M, N, K (partial tiles in every direction, K below one box
    up to many), every ring depth and MFMA form: 2048 sampled outputs
    against the oracle, plus the four corners."""
    M, N, K, bk, stages, mfma, k256 = _random_gemm_case(seed)
    say("gemm random", seed, M, N, K, bk, stages, mfma, k256)
    A = synthgen.normal_bf16_bits(91000 + seed, (M, K))
    Bt = synthgen.normal_bf16_bits(92000 + seed, (N, K))
    C = run_gemm(A, Bt, M, N, K, bk, stages, k256=k256, mfma=mfma)
    rows, cols = synthgen.sample_pairs(93000 + seed, 2048, M, N)
    rows = np.concatenate([rows, [0, 0, M - 1, M - 1]])
    cols = np.concatenate([cols, [0, N - 1, 0, N - 1]])
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows, cols)
    check_close(C[rows, cols], ref)
    assert not (C == 0x7FFF).any()


@pytest.mark.parametrize("offset,ldc", [(0, 264), (1, 264), (0, 203)])
def test_c_leading_dimension(offset, ldc):
    """C written with leading dimension ldc >= N: the LDS-staged tile store
    (16-byte aligned C, ldc a multiple of 8) and the element-store fallback
    (offset by one element, or odd ldc) both clip at the M / N edges and leave
    the padding columns and the bytes around C untouched."""
    M, N, K = 300, 200, 192
    say("gemm ldc", offset, ldc)
    A = synthgen.normal_bf16_bits(56, (M, K))
    Bt = synthgen.normal_bf16_bits(57, (N, K))
    Ad = torch.from_numpy(A.view(np.int16)).cuda()
    Bd = torch.from_numpy(Bt.view(np.int16)).cuda()
    buf = torch.full((M * ldc + 16,), 0x7FFF, dtype=torch.int16, device="cuda")
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (K * 2,), (64, 256), None, "128b_k256")
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (K * 2,), (64, 256), None, "128b_k256")
    att.gemm_bf16(mA, mB, buf.data_ptr() + 2 * offset, M, N, K, ldc, 2, stream())
    torch.cuda.synchronize()
    out = buf.cpu().numpy().view(np.uint16)
    C = out[offset:offset + M * ldc].reshape(M, ldc)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_close(C[:, :N], ref)
    assert (C[:, N:] == 0x7FFF).all()
    assert (out[:offset] == 0x7FFF).all() and (out[offset + M * ldc:] == 0x7FFF).all()


# ---- fp32 C: the accumulators before the bf16 rounding ----------------------

def run_gemm_f32(A_bits, Bt_bits, M, N, K, stages, k256=True, ldc=None, offset=0):
    """gemm_bf16_f32 on the 64-deep K step; returns C (M, N) as float32 and
    the whole output buffer (for the untouched-padding check)."""
    ld = (K + 7) // 8 * 8
    ldc = ldc or N
    Ap = np.zeros((M, ld), dtype=np.uint16)
    Ap[:, :K] = A_bits
    Bp = np.zeros((N, ld), dtype=np.uint16)
    Bp[:, :K] = Bt_bits
    Ad = torch.from_numpy(Ap.view(np.int16)).cuda()
    Bd = torch.from_numpy(Bp.view(np.int16)).cuda()
    buf = torch.full((offset + M * ldc,), float("nan"), dtype=torch.float32, device="cuda")
    sw = "128b_k256" if k256 else "128b"
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (ld * 2,), (64, 256), None, sw)
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (ld * 2,), (64, 256), None, sw)
    att.gemm_bf16_f32(mA, mB, buf.data_ptr() + 4 * offset, M, N, K, ldc, stages, stream())
    torch.cuda.synchronize()
    full = buf.cpu().numpy()
    C = full[offset:].reshape(M, ldc)[:, :N]
    return C, full


def check_f32(got, ref):
    """The accumulator itself: 2e-2 absolute, as stated for the GEMM."""
    err = np.abs(got.astype(np.float64) - ref)
    assert np.isfinite(got).all()
    assert err.max() <= 2e-2, f"worst {err.max()}"


@pytest.mark.parametrize("stages", [2, 3])
def test_f32_identity_exact(stages):
    """A = I: the fp32 C equals B exactly."""
    K = N = M = 512
    eye = np.zeros((M, K), dtype=np.uint16)
    eye[np.arange(M), np.arange(K)] = 0x3F80
    Bt = synthgen.normal_bf16_bits(61, (N, K))
    C, _ = run_gemm_f32(eye, Bt, M, N, K, stages)
    np.testing.assert_array_equal(C, bf16_to_f64(Bt.T).astype(np.float32))


@pytest.mark.parametrize("M,N,K,stages", [(512, 512, 512, 2), (512, 512, 512, 3), (300, 270, 448, 3),
                                          (257, 513, 200, 2), (33, 1000, 64, 3), (700, 17, 1030, 2)])
def test_f32_against_oracle_full(M, N, K, stages):
    """Every output of ragged shapes (partial M / N tiles, a K tail with two
    stages) within 2e-2 of the fp64 oracle."""
    say("gemm f32", M, N, K, stages)
    A = synthgen.normal_bf16_bits(62, (M, K))
    Bt = synthgen.normal_bf16_bits(63, (N, K))
    C, _ = run_gemm_f32(A, Bt, M, N, K, stages)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_f32(C, ref)


@pytest.mark.parametrize("stages", [2, 3])
def test_f32_8192_sampled(stages):
    """The full-size product, 4096 sampled accumulators within 2e-2."""
    ex = W.GEMM_8192
    M, N, K = ex["M"], ex["N"], ex["K"]
    say("gemm f32 8192^3", stages)
    A = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 1, (M, K))
    Bt = synthgen.normal_bf16_bits(ex["seed"] * 1000 + 2, (N, K))
    C, _ = run_gemm_f32(A, Bt, M, N, K, stages)
    rows, cols = synthgen.sample_pairs(ex["seed"] * 1000 + 3, ex["nsample"], M, N)
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows, cols)
    check_f32(C[rows, cols], ref)
    assert np.isfinite(C).all()


@pytest.mark.parametrize("offset,ldc", [(0, 264), (1, 264), (3, 259)])
def test_f32_c_leading_dimension(offset, ldc):
    """C at any 4-byte offset and any ldc >= N: element stores where 16-byte
    ones do not fit; the padding past N is never written."""
    M, N, K = 300, 250, 128
    A = synthgen.normal_bf16_bits(64, (M, K))
    Bt = synthgen.normal_bf16_bits(65, (N, K))
    C, full = run_gemm_f32(A, Bt, M, N, K, 3, ldc=ldc, offset=offset)
    rows, cols = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref = oracle.gemm_bf16_sample(A, Bt, K, rows.reshape(-1), cols.reshape(-1)).reshape(M, N)
    check_f32(C, ref)
    assert np.isnan(full[:offset]).all()
    assert np.isnan(full[offset:].reshape(M, ldc)[:, N:]).all()


def test_f32_rejects_what_it_does_not_serve():
    """The 32-deep K step and a misaligned C are refused before any launch."""
    A = torch.zeros((256, 64), dtype=torch.int16, device="cuda")
    C = torch.zeros(256 * 256 + 1, dtype=torch.float32, device="cuda")
    m64 = att.tmap_encode("bf16", 2, A.data_ptr(), (64, 256), (128,), (64, 256), None, "128b")
    m32 = att.tmap_encode("bf16", 2, A.data_ptr(), (64, 256), (128,), (32, 256), None, "64b")
    with pytest.raises(att.TmapError):
        att.gemm_bf16_f32(m32, m32, C.data_ptr(), 256, 256, 64, 256, 2, stream())
    with pytest.raises(att.TmapError):
        att.gemm_bf16_f32(m64, m64, C.data_ptr() + 2, 256, 256, 64, 256, 2, stream())
    with pytest.raises(att.TmapError):
        att.gemm_bf16_f32(m64, m64, C.data_ptr(), 256, 256, 64, 256, 4, stream())
    att.gemm_bf16_f32(m64, m64, C.data_ptr(), 256, 256, 64, 256, 3, stream())
    torch.cuda.synchronize()
    assert float(C[:256 * 256].abs().max()) == 0.0
