"""Concurrent calls: two host threads, each on a stream of its own, issue the
tile copy, box loads, an int32 reduce-add and the GEMM at the same time on
buffers of their own (the C ABI's calls are reentrant, and calls on
different streams may overlap as long as their destinations do not).  Every
result is checked afterwards: the copy is the identity, the loads and the
reduction bit-exact against the oracle, the GEMM's sampled outputs within
its tolerance."""
import sys
import threading

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import async_tensor_tile_amd as att  # noqa: E402
import oracle  # noqa: E402
import synthgen  # noqa: E402

from gpu_util import encode, require_native, to_dev, to_host  # noqa: E402

pytestmark = pytest.mark.gpu


def setup_module(module):
    require_native()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


ITERS = 3
NLOAD, NRED = 64, 256
GM = 512                      # GEMM M = N = K


def make_case(k):
    """Host inputs and device buffers of thread k (made on the main thread)."""
    c = {}
    c["src"] = synthgen.u16_bits(71000 + k, (1024, 2048))                # bf16 bits, 1024 rows of 2048
    g = synthgen.rng(71100 + k)
    c["lcoords"] = np.stack([g.integers(-8, 2048, NLOAD), g.integers(-8, 1024, NLOAD)], axis=1).astype(np.int32)
    c["racc"] = synthgen.int32_range(71200 + k, (1024, 1024), -(1 << 20), 1 << 20)
    c["rcoords"] = np.stack([g.integers(-16, 1000, NRED), g.integers(-16, 1000, NRED)], axis=1).astype(np.int32)
    c["rimgs"] = synthgen.int32_range(71300 + k, (NRED, 64, 64), -(1 << 20), 1 << 20)
    c["A"] = synthgen.normal_bf16_bits(71400 + k, (GM, GM))
    c["Bt"] = synthgen.normal_bf16_bits(71500 + k, (GM, GM))
    d = {"src": to_dev(c["src"]), "lcoords": to_dev(c["lcoords"]), "rcoords": to_dev(c["rcoords"]),
         "rimgs": to_dev(c["rimgs"]), "A": to_dev(c["A"]), "Bt": to_dev(c["Bt"])}
    d["dst"] = [torch.full((c["src"].nbytes,), 0x33, dtype=torch.uint8, device="cuda") for _ in range(ITERS)]
    d["limg"] = [torch.full((NLOAD * 128 * 16,), 0x5A, dtype=torch.uint8, device="cuda") for _ in range(ITERS)]
    d["racc"] = [to_dev(c["racc"]) for _ in range(ITERS)]
    d["C"] = [torch.full((GM * GM * 2,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(ITERS)]
    return c, d


def worker(k, c, d, start, errors):
    try:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.default_stream())
        sp = s.cuda_stream
        ms = encode(d["src"], "bf16", (2048, 1024), (4096,), (64, 128), swizzle="128b")
        ml = encode(d["src"], "bf16", (2048, 1024), (4096,), (64, 16), swizzle="128b", fill="nan")
        mA = att.tmap_encode("bf16", 2, d["A"].data_ptr(), (GM, GM), (GM * 2,), (64, 256), None, "128b_k256")
        mB = att.tmap_encode("bf16", 2, d["Bt"].data_ptr(), (GM, GM), (GM * 2,), (64, 256), None, "128b_k256")
        start.wait(timeout=60)
        for it in range(ITERS):
            md = encode(d["dst"][it], "bf16", (2048, 1024), (4096,), (64, 128), swizzle="128b")
            att.tile_copy(ms, md, 2, sp)
            att.tile_load(ml, d["lcoords"], NLOAD, d["limg"][it], sp)
            mr = encode(d["racc"][it], "i32", (1024, 1024), (4096,), (64, 64))
            att.tile_reduce_add(mr, d["rcoords"], NRED, d["rimgs"], sp)
            att.gemm_bf16_ex(mA, mB, d["C"][it].data_ptr(), GM, GM, GM, GM, 3, 0, 1, sp, 16)
        s.synchronize()
    except Exception as e:  # reported on the main thread
        errors.append((k, repr(e)))


def test_two_threads_two_streams():
    cases = [make_case(k) for k in range(2)]
    torch.cuda.synchronize()
    start = threading.Barrier(2)
    errors = []
    threads = [threading.Thread(target=worker, args=(k, c, d, start, errors), daemon=True)
               for k, (c, d) in enumerate(cases)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for k, (c, d) in enumerate(cases):
        say("thread", k, "results")
        ol = oracle.Map("bf16", (2048, 1024), (4096,), (64, 16), swizzle="128b", fill="nan")
        want_load = ol.load(c["src"], c["lcoords"])
        want_red = c["racc"].copy()
        oracle.Map("i32", (1024, 1024), (4096,), (64, 64)).reduce_add(want_red, c["rcoords"], c["rimgs"])
        g = synthgen.rng(71600 + k)
        rows, cols = g.integers(0, GM, 512), g.integers(0, GM, 512)
        ref = oracle.gemm_bf16_sample(c["A"], c["Bt"], GM, rows, cols)
        for it in range(ITERS):
            np.testing.assert_array_equal(to_host(d["dst"][it]), c["src"].view(np.uint8).reshape(-1))
            np.testing.assert_array_equal(to_host(d["limg"][it]).reshape(NLOAD, -1), want_load)
            np.testing.assert_array_equal(to_host(d["racc"][it]).view(np.int32).reshape(1024, 1024), want_red)
            C = to_host(d["C"][it]).view(np.uint16).reshape(GM, GM)
            got = bf16_to_f64(C[rows, cols])
            assert (np.abs(got - ref) <= 2e-2 + 2.0 ** -8 * np.abs(ref)).all(), f"thread {k} GEMM {it}"
