#!/usr/bin/env python3
"""Benchmark: tiled box copy of a bf16 8192 x 8192 tensor through LDS.

One step = one full-grid round trip (8192 boxes of 128 rows x 64 columns,
128-byte swizzle, two LDS stages per workgroup: one wave issues the copies,
four store each part as it lands): every box is loaded global -> LDS with
the swizzle applied on write and stored LDS -> global through a second
map.  Algorithmic bytes per step: 128 MiB read + 128 MiB
written = 268,435,456 B.  Four source/destination pairs (1 GiB) rotate so
the 256 MB last-level cache cannot serve the working set.

Prints one JSON line (rank 0).  Secondary workloads (rank-5 load, reduce-add
store, GEMM mainloop) are timed after the copy and reported under "extra"
(--no-extra skips them).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

BYTES_PER_STEP = 2 * 8192 * 8192 * 2
HBM_PEAK_GBS = 8000.0
PROFILE_DIR = os.path.join(ROOT, "profiles")
COUNTERS_FILE = os.path.join(PROFILE_DIR, "tile_copy_bf16_8192_counters.json")
KERNEL_SOURCES = ("async_tensor_tile_amd/csrc/kernel_copy.hip", "include/att/tile_device.hpp",
                  "include/att/tmap_impl.hpp")


GEMM_COUNTERS_FILE = os.path.join(PROFILE_DIR, "gemm_bf16_8192_counters.json")
GEMM_SOURCES = ("async_tensor_tile_amd/csrc/kernel_gemm.hip", "include/att/tile_device.hpp", "include/tile.hpp",
                "include/att/tmap_impl.hpp")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_counters(path=COUNTERS_FILE, sources=KERNEL_SOURCES):
    """HBM traffic (and, for the copy, LDS bank conflicts) measured by
    rocprofv3 for this exact kernel source; None once the kernel has changed
    since."""
    try:
        with open(path) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_sha") != kernel_source_hash(sources):
        return None
    return c


def gemm_traffic():
    """HBM bytes per launch of the default GEMM (FETCH_SIZE and WRITE_SIZE,
    calibrated like the copy's), or None once its sources have changed."""
    c = committed_counters(GEMM_COUNTERS_FILE, GEMM_SOURCES)
    return c.get("hbm_bytes_per_launch") if c else None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        return "unknown"


def cpu_baseline(min_seconds: float = 10.0, max_passes: int = 8, max_threads: int = 16):
    """The oracle (plain single-threaded C, as it stands) doing the same work
    on the host, timed beside the GPU:

    - the round trip: every box of the 8192-box grid loaded into an LDS image
      and stored back, full passes until min_seconds have elapsed, first on
      one thread, then split by boxes over the host's cores (threads calling
      the oracle on disjoint box ranges; the C calls release the GIL);
    - the GEMM sample: 4096 sampled outputs of the 8192^3 bf16 product as
      float64 dot products (2 * 4096 * 8192 flop), on one thread and split by
      samples over the same threads; the full product's CPU time is only
      extrapolated from that rate."""
    import concurrent.futures as cf

    import numpy as np

    import oracle
    import synthgen
    from synthgen import workloads as W

    src = synthgen.u16_bits(2, (8192, 8192))
    dst = np.zeros_like(src)
    m = oracle.Map("bf16", (8192, 8192), (16384,), (64, 128), swizzle="128b")
    coords = np.array([[64 * (t % 128), 128 * (t // 128)] for t in range(8192)], dtype=np.int32)

    def boxes(b0, b1):
        for a in range(b0, b1, 256):
            e = min(b1, a + 256)
            m.store(dst, coords[a:e], m.load(src, coords[a:e]))

    passes, t0 = 0, time.perf_counter()
    while passes < max_passes:
        boxes(0, 8192)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt1 = time.perf_counter() - t0
    ok = bool(np.array_equal(dst, src))

    avail = len(os.sched_getaffinity(0))
    threads = max(1, min(avail, max_threads))
    dst[...] = 0
    per = (8192 + threads - 1) // threads
    passes_mt, t0 = 0, time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        while passes_mt < 4 * max_passes:
            list(ex.map(lambda w: boxes(w * per, min(8192, (w + 1) * per)), range(threads)))
            passes_mt += 1
            if time.perf_counter() - t0 >= min_seconds / 2:
                break
    dtm = time.perf_counter() - t0
    ok = ok and bool(np.array_equal(dst, src))

    ex_g = W.GEMM_8192
    M, N, K = ex_g["M"], ex_g["N"], ex_g["K"]
    A = synthgen.normal_bf16_bits(ex_g["seed"] * 1000 + 1, (M, K))
    Bt = synthgen.normal_bf16_bits(ex_g["seed"] * 1000 + 2, (N, K))
    rows, cols = synthgen.sample_pairs(ex_g["seed"] * 1000 + 3, ex_g["nsample"], M, N)
    flop = 2.0 * len(rows) * K
    t0 = time.perf_counter()
    ref1 = oracle.gemm_bf16_sample(A, Bt, K, rows, cols)
    g1 = time.perf_counter() - t0
    parts = np.array_split(np.arange(len(rows)), threads)
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        refs = list(ex.map(lambda ix: oracle.gemm_bf16_sample(A, Bt, K, rows[ix], cols[ix]), parts))
    gm = time.perf_counter() - t0
    ok = ok and bool(np.array_equal(np.concatenate(refs), ref1))
    gflops_mt = flop / gm / 1e9
    return {"value": round(passes * BYTES_PER_STEP / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "verified": ok, "cpu_model": cpu_model(),
            "sample": f"{passes} full pass(es) of the 8192-box bf16 8192x8192 round trip "
                      f"(load to LDS image + store), {dt1:.1f} s on one host thread",
            "all_cores": {"value": round(passes_mt * BYTES_PER_STEP / dtm / 1e9, 4), "unit": "GB/s",
                          "cores": threads, "cores_available": avail,
                          "sample": f"{passes_mt} full pass(es) of the same round trip, boxes split over "
                                    f"{threads} threads, {dtm:.1f} s"},
            "gemm_sample": {"what": "4096 sampled outputs of the bf16 8192^3 GEMM as float64 dot products "
                                    "(the oracle's GEMM check)",
                            "GFLOPs_1_thread": round(flop / g1 / 1e9, 3),
                            "GFLOPs_all_cores": round(gflops_mt, 3), "cores": threads,
                            "full_gemm_seconds_extrapolated": round(2.0 * M * N * K / (gflops_mt * 1e9), 1)}}


def run_extra(att, torch, stream, reps: int):
    """Secondary workloads: rank-5 fp32 edge-crossing load, int32 reduce-add
    pass, bf16 GEMM 8192^3.  Each timed with events on the launch stream."""
    import numpy as np

    import synthgen
    from synthgen import workloads as W

    out = {}

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(n):
            fn()
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / n

    # rank-5 fp32, 2048 boxes of 32 KiB, a quarter straddling edges (NaN fill)
    ex = W.RANK5
    dims, strides = ex["dims"], [1040, 134160, 4427280, 30990960]
    vals = synthgen.uniform_f32(ex["seed"], strides[-1] * dims[-1] // 4)
    sd = torch.from_numpy(vals.view(np.uint8)).cuda()
    coords = synthgen.edge_mix_coords(ex["seed"] * 1000, dims, [32, 16, 8, 2, 1], ex["estride"], ex["nbox"])
    cd = torch.from_numpy(coords).cuda()
    img = torch.empty(ex["nbox"] * 32768, dtype=torch.uint8, device="cuda")
    m = att.tmap_encode("f32", 5, sd.data_ptr(), dims, strides, ex["box"], ex["estride"], "128b", "nan")
    ms = timed(lambda: att.tile_load(m, cd.data_ptr(), ex["nbox"], img.data_ptr(), stream), reps)
    out["rank5_load_f32"] = {"ms": round(ms, 4), "GBps_lds_image_written": round(ex["nbox"] * 32768 / ms / 1e6, 1)}

    # reduce-add int32: one pass of 1024 boxes of 64x64 into 4096^2
    ex = W.REDUCE_4096
    dst = torch.from_numpy(synthgen.int32_range(ex["seed"], (4096, 4096), -(1 << 20), 1 << 20)).cuda()
    rc = torch.from_numpy(synthgen.uniform_coords(ex["seed"] * 1000 + 10, ex["nbox"], (0, 0), (4032, 4032))).cuda()
    srcs = torch.from_numpy(synthgen.int32_range(ex["seed"] * 1000 + 20, (ex["nbox"], 64, 64), -(1 << 20), 1 << 20)).cuda()
    mr = att.tmap_encode("i32", 2, dst.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, "none")
    ms = timed(lambda: att.tile_reduce_add(mr, rc.data_ptr(), ex["nbox"], srcs.data_ptr(), stream), reps)
    out["reduce_add_i32_pass"] = {"ms": round(ms, 4),
                                  "GBps_algorithmic": round(ex["nbox"] * 16384 * 3 / ms / 1e6, 1)}
    ms = timed(lambda: att.tile_reduce(mr, "min", rc.data_ptr(), ex["nbox"], srcs.data_ptr(), stream), reps)
    out["reduce_min_i32_pass"] = {"ms": round(ms, 4),
                                  "GBps_algorithmic": round(ex["nbox"] * 16384 * 3 / ms / 1e6, 1)}
    # the same pass in fp32 (N(0,1) values, hardware float atomics)
    dstf = torch.from_numpy(synthgen.normal_f32(ex["seed"], (4096, 4096))).cuda()
    srcf = torch.from_numpy(synthgen.normal_f32(ex["seed"] * 1000 + 22, (ex["nbox"], 64, 64))).cuda()
    mf = att.tmap_encode("f32", 2, dstf.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, "none")
    ms = timed(lambda: att.tile_reduce_add(mf, rc.data_ptr(), ex["nbox"], srcf.data_ptr(), stream), reps)
    out["reduce_add_f32_pass"] = {"ms": round(ms, 4),
                                  "GBps_algorithmic": round(ex["nbox"] * 16384 * 3 / ms / 1e6, 1)}
    # the pages' reduce example type: bf16 add (compare-and-swap per element)
    dst16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"], (4096, 4096)).view(np.int16)).cuda()
    src16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"] * 1000 + 21, (ex["nbox"], 64, 64))
                             .view(np.int16)).cuda()
    mb = att.tmap_encode("bf16", 2, dst16.data_ptr(), ex["dims"], (8192,), ex["box"], None, "none")
    ms = timed(lambda: att.tile_reduce(mb, "add", rc.data_ptr(), ex["nbox"], src16.data_ptr(), stream), reps)
    out["reduce_add_bf16_pass"] = {"ms": round(ms, 4),
                                   "GBps_algorithmic": round(ex["nbox"] * 8192 * 3 / ms / 1e6, 1)}

    # im2col: bf16 NHWC 8 x 56 x 56 x 64, 3 x 3 window, padding 1 -- every tap
    # over every window in 128-pixel boxes of all 64 channels (128B swizzle)
    N_, H_, W_, C_, P_ = 8, 56, 56, 64, 128
    xi = torch.from_numpy(synthgen.normal_bf16_bits(77, (N_, H_, W_, C_)).view(np.int16)).cuda()
    mi = att.tmap_encode_im2col("bf16", 4, xi.data_ptr(), (C_, W_, H_, N_), (C_ * 2, W_ * C_ * 2, H_ * W_ * C_ * 2),
                                (-1, -1), (-1, -1), C_, P_, None, "128b")
    co, of = [], []
    for L0 in range(0, N_ * H_ * W_, P_):
        for i in range(3):
            for j in range(3):
                co.append((0, -1 + L0 % W_, -1 + (L0 // W_) % H_, L0 // (W_ * H_)))
                of.append((j, i))
    cod = torch.from_numpy(np.asarray(co, dtype=np.int32)).cuda()
    ofd = torch.from_numpy(np.asarray(of, dtype=np.int32)).cuda()
    imgs = torch.empty(len(co) * P_ * C_ * 2, dtype=torch.uint8, device="cuda")
    ms = timed(lambda: att.tile_load_im2col(mi, cod.data_ptr(), ofd.data_ptr(), len(co), imgs.data_ptr(), stream),
               reps)
    out["im2col_conv3x3_bf16"] = {"ms": round(ms, 4), "boxes": len(co),
                                  "GBps_lds_image_written": round(len(co) * P_ * C_ * 2 / ms / 1e6, 1)}

    g = run_gemm(att, torch, stream, max(3, reps // 2), variants=(GEMM_DEFAULT,), vendor=True)
    best = g[g["gemm_best"]]
    best["roofline"] = {"bound": "mfma", "achieved": best["TFLOPs"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(best["TFLOPs"] / BF16_PEAK_TFLOPS, 4), "traffic": gemm_traffic()}
    out.update(g)
    return out


# (K step, operand swizzle, ring stages, MFMA shape: 16 = 16x16x32, 32 = 32x32x16)
GEMM_VARIANTS = ((64, "128b_k256", 3, 16), (64, "128b_k256", 2, 16), (64, "128b_k256", 2, 32), (64, "128b", 2, 16),
                 (32, "64b_k256", 4, 32), (32, "64b_k256", 3, 32), (32, "64b", 4, 32))
GEMM_DEFAULT = (64, "128b_k256", 3, 16)
BF16_PEAK_TFLOPS = 2500.0


# Tile rasterisations of the GEMM (group_m, xcd): plain row-major tile order,
# groups of 8 tile rows in dispatch order (neighbouring workgroups land on
# different XCDs), the same groups with each XCD owning a contiguous range,
# and each XCD owning a 2-D block of tiles.
GEMM_RASTERS = ((1, 0), (8, 0), (8, 1), (4, 2), (8, 2))


def run_gemm_raster(att, torch, stream, reps: int, rounds: int = 3):
    """The default GEMM under each rasterisation: median TFLOP/s over
    `rounds` interleaved rounds.  Under rocprofv3 --pmc the dispatches come
    round by round in GEMM_RASTERS order, reps + 1 per raster and round."""
    from synthgen import workloads as W

    ex = W.GEMM_8192
    M, N, K = ex["M"], ex["N"], ex["K"]
    g = torch.Generator(device="cuda").manual_seed(ex["seed"])
    Ad = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    Bd = torch.randn(N, K, generator=g, device="cuda").to(torch.bfloat16)
    Cd = torch.empty(M, N, dtype=torch.bfloat16, device="cuda")
    bk, sw, stages, _ = GEMM_DEFAULT
    mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (K * 2,), (bk, 256), None, sw)
    mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (K * 2,), (bk, 256), None, sw)
    times = {r: [] for r in GEMM_RASTERS}
    for _ in range(rounds):              # rounds interleave the variants against clock drift
        for gm, xcd in GEMM_RASTERS:
            fn = lambda: att.gemm_bf16_ex(mA, mB, Cd.data_ptr(), M, N, K, N, stages, gm, xcd, stream)  # noqa: E731
            fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                fn()
            e.record()
            torch.cuda.synchronize()
            times[(gm, xcd)].append(s.elapsed_time(e) / reps)
    out = []
    for (gm, xcd), t in times.items():
        ms = sorted(t)[len(t) // 2]
        out.append({"group_m": gm, "xcd": xcd, "ms_median": round(ms, 4),
                    "TFLOPs": round(2.0 * M * N * K / ms / 1e9, 1), "ms_all": [round(x, 4) for x in t]})
    return out


def run_gemm(att, torch, stream, reps: int, variants=GEMM_VARIANTS, warmup: int = 40, warmup_ms: float = 100.0,
             vendor: bool = False, rounds: int = 3, c_f32: bool = False):
    """bf16 GEMM mainloop, M = N = K = 8192, A row-major, B column-major,
    N(0,1) operands; 2*M*N*K flop per launch.  Each variant is timed in
    `rounds` interleaved rounds of `reps` launches (median reported), after
    at least `warmup` launches of each and `warmup_ms` of host time, the
    variants in turn: when MFMA work follows a memory-bound phase the
    shader clock takes some 30-60 ms of sustained load to settle (the first
    launches run 20-40 % slower, for the vendor kernel as for these), and
    the figure wanted is the settled rate.
    With `vendor`, torch's A @ B^T on the same operands joins the rounds.
    With `c_f32`, C is written as the fp32 accumulators (gemm_bf16_f32, no
    LDS staging of C), for counters of the mainloop alone."""
    from synthgen import workloads as W

    ex = W.GEMM_8192
    M, N, K = ex["M"], ex["N"], ex["K"]
    g = torch.Generator(device="cuda").manual_seed(ex["seed"])
    Ad = torch.randn(M, K, generator=g, device="cuda").to(torch.bfloat16)
    Bd = torch.randn(N, K, generator=g, device="cuda").to(torch.bfloat16)
    Cd = torch.empty(M, N, dtype=torch.float32 if c_f32 else torch.bfloat16, device="cuda")
    fns = {}
    keep = []
    for bk, sw, stages, mi in variants:
        mA = att.tmap_encode("bf16", 2, Ad.data_ptr(), (K, M), (K * 2,), (bk, 256), None, sw)
        mB = att.tmap_encode("bf16", 2, Bd.data_ptr(), (K, N), (K * 2,), (bk, 256), None, sw)
        keep.append((mA, mB))
        if c_f32:
            fns[f"gemm_bf16_f32_8192_bk{bk}_{sw}_s{stages}"] = (
                lambda mA=mA, mB=mB, stages=stages: att.gemm_bf16_f32(mA, mB, Cd.data_ptr(), M, N, K, N, stages,
                                                                      stream))
            continue
        fns[f"gemm_bf16_8192_bk{bk}_{sw}_s{stages}_mfma{mi}"] = (
            lambda mA=mA, mB=mB, stages=stages, mi=mi: att.gemm_bf16_ex(mA, mB, Cd.data_ptr(), M, N, K, N, stages,
                                                                        0, 1, stream, mi))
    if vendor:
        Bt = Bd.t()
        fns["vendor_gemm_torch_matmul"] = lambda: torch.matmul(Ad, Bt, out=Cd)
    warm, t_end = 0, time.perf_counter() + warmup_ms / 1e3
    while warm < warmup or time.perf_counter() < t_end:
        for fn in fns.values():
            fn()
        torch.cuda.synchronize()
        warm += 1
    times = {k: [] for k in fns}
    for _ in range(rounds):
        for key, fn in fns.items():
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(reps):
                fn()
            e.record()
            torch.cuda.synchronize()
            times[key].append(s.elapsed_time(e) / reps)
    out, best = {}, None
    for key, t in times.items():
        ms = sorted(t)[len(t) // 2]
        tf = 2.0 * M * N * K / ms / 1e9
        out[key] = {"ms": round(ms, 4), "TFLOPs": round(tf, 1), "pct_of_bf16_peak": round(100 * tf / 2500.0, 2)}
        if key.startswith("gemm_") and (best is None or tf > best[0]):
            best = (tf, key)
    out["gemm_best"] = best[1]
    out["warmup_launches_each"] = warm
    return out


def hbm_ceiling(att, torch, stream, reps: int = 100, sweep: bool = True):
    """What plain streaming kernels (the library's hbm_probe: coalesced
    16-byte loads, non-temporal 16-byte stores) reach on this GPU's HBM with
    the same 128 MiB working sets, 4 rotating buffers so the last-level cache
    cannot serve them: read-only, write-only and a linear copy."""
    n = 8192 * 8192 * 2
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255) for _ in range(4)]
    outs = [torch.empty_like(b) for b in bufs]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def timed(fn):
        for k in range(10):
            fn(k)
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for k in range(reps):
            fn(k)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps

    r = timed(lambda k: att.hbm_probe("read", bufs[k % 4], sink, n, stream))
    w = timed(lambda k: att.hbm_probe("write", None, outs[k % 4], n, stream))
    c = timed(lambda k: att.hbm_probe("copy", bufs[k % 4], outs[k % 4], n, stream))
    ok = all(torch.equal(a, b) for a, b in zip(bufs, outs))
    out = {"read_only_GBps": round(n / r / 1e6, 1), "write_only_GBps": round(n / w / 1e6, 1),
           "copy_GBps": round(2 * n / c / 1e6, 1), "copy_verified": ok, "bytes_per_buffer": n,
           "what": "hbm_probe read / write / copy over 4 rotating 128 MiB buffers"}
    if sweep:
        # the best plain copy this GPU runs: every launch shape of
        # hbm_probe_copy_ex (vectors per thread, store kind, order) at 1 to
        # 16 workgroups per CU; the best is checked for correctness
        best = None
        for variant in range(16):
            for wpc in (1, 2, 4, 8, 16):
                t = timed(lambda k, v=variant, g=wpc: att.hbm_probe_copy_ex(bufs[k % 4], outs[k % 4], n, v, g,
                                                                            stream))
                if best is None or t < best[0]:
                    best = (t, variant, wpc)
        for o in outs:
            o.zero_()
        for k in range(4):
            att.hbm_probe_copy_ex(bufs[k], outs[k], n, best[1], best[2], stream)
        ok2 = all(torch.equal(a, b) for a, b in zip(bufs, outs))
        u = 1 << (best[1] & 3)
        out["copy_sweep_best"] = {"GBps": round(2 * n / best[0] / 1e6, 1), "verified": ok2,
                                  "vectors_per_thread": u, "nontemporal_stores": bool(best[1] & 4),
                                  "order": "slice per workgroup" if best[1] & 8 else "grid-stride",
                                  "workgroups_per_cu": best[2], "configs": 80}
        # the same bytes in the tile copy's access shape (8 rows x 128 bytes
        # of one 128 x 128-byte box per wave instruction) through registers:
        # what the box shape itself allows, apart from the LDS staging
        bbest = None
        for nbx in (1, 2, 4, 8):
            for variant in list(range(8)) + [v | 32 for v in range(8)]:
                t = timed(lambda k, v=variant, b=nbx: att.hbm_probe_box_copy(bufs[k % 4], outs[k % 4], 16384, 8192, b,
                                                                             v, stream))
                if bbest is None or t < bbest[0]:
                    bbest = (t, nbx, variant)
        for o in outs:
            o.zero_()
        for k in range(4):
            att.hbm_probe_box_copy(bufs[k], outs[k], 16384, 8192, bbest[1], bbest[2], stream)
        ok3 = all(torch.equal(a, b) for a, b in zip(bufs, outs))
        out["box_copy_sweep_best"] = {"GBps": round(2 * n / bbest[0] / 1e6, 1), "verified": ok3,
                                      "boxes_per_workgroup": bbest[1], "nontemporal_stores": bool(bbest[2] & 1),
                                      "xcd_contiguous": bool(bbest[2] & 2),
                                      "issue": "box-major" if bbest[2] & 4 else "row-group-major",
                                      "rotated_row_walk": bool(bbest[2] & 32), "configs": 64,
                                      "what": "register copy with the tile copy's access shape: one 16-byte "
                                              "vector per lane, 8 rows x 128 bytes of a 128 x 128-byte box "
                                              "per wave instruction"}
    return out


def run_copy_compare(att, torch, stream, reps: int = 20, rounds: int = 3):
    """The tile copy beside the plain copies it is measured against, on the
    same four rotating 128 MiB pairs, for counter runs: per round, `reps`
    dispatches each of the default tile copy, the best plain copy of the
    sweep (16-byte vectors, non-temporal stores, grid-stride, 4 workgroups
    per CU), the register copy in the tile copy's access shape (2 boxes per
    workgroup, non-temporal stores, the tile copy's rotated row walk) and the
    default hbm_probe copy, in that order.  Returns the median GB/s of each
    over the rounds."""
    import numpy as np

    import synthgen
    from synthgen import workloads as W

    ex = W.COPY_8192
    n = 8192 * 8192 * 2
    src_host = torch.from_numpy(synthgen.u16_bits(ex["seed"], (8192, 8192)).view(np.uint8).reshape(-1))
    pairs = []
    for _ in range(4):
        a = src_host.to("cuda")
        b = torch.empty_like(a)
        ma = att.tmap_encode("bf16", 2, a.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, ex["swizzle"])
        mb = att.tmap_encode("bf16", 2, b.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, ex["swizzle"])
        pairs.append((a, b, ma, mb))
    kinds = {
        "tile_copy": lambda a, b, ma, mb: att.tile_copy(ma, mb, 2, stream),
        "plain_copy_best": lambda a, b, ma, mb: att.hbm_probe_copy_ex(a, b, n, 4, 4, stream),
        "box_shaped_register_copy": lambda a, b, ma, mb: att.hbm_probe_box_copy(a, b, 16384, 8192, 2, 33, stream),
        "hbm_probe_copy": lambda a, b, ma, mb: att.hbm_probe("copy", a, b, n, stream),
    }
    times = {k: [] for k in kinds}
    for _ in range(rounds):
        for key, fn in kinds.items():
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for k in range(reps):
                fn(*pairs[k % 4])
            e.record()
            torch.cuda.synchronize()
            times[key].append(s.elapsed_time(e) / reps)
    ok = all(torch.equal(a, b) for a, b, _, _ in pairs)
    return {"order": list(kinds), "rounds": rounds, "dispatches_per_kind_and_round": reps, "verified": ok,
            "GBps_median": {k: round(2 * n / sorted(t)[len(t) // 2] / 1e6, 1) for k, t in times.items()}}


def run_reduce_compare(att, torch, stream, reps: int = 10):
    """The reduce-add pass of 1024 boxes of 64 x 64 into a 4096 x 4096
    destination in int32 and then in bf16, one untimed and `reps` timed
    dispatches each (in that order, for counter runs); algorithmic bytes
    3 x box bytes per box."""
    import numpy as np

    import synthgen
    from synthgen import workloads as W

    ex = W.REDUCE_4096
    rc = torch.from_numpy(synthgen.uniform_coords(ex["seed"] * 1000 + 10, ex["nbox"], (0, 0), (4032, 4032))).cuda()
    dst = torch.from_numpy(synthgen.int32_range(ex["seed"], (4096, 4096), -(1 << 20), 1 << 20)).cuda()
    src = torch.from_numpy(synthgen.int32_range(ex["seed"] * 1000 + 20, (ex["nbox"], 64, 64), -(1 << 20),
                                                1 << 20)).cuda()
    mi = att.tmap_encode("i32", 2, dst.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, "none")
    d16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"], (4096, 4096)).view(np.int16)).cuda()
    s16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"] * 1000 + 21, (ex["nbox"], 64, 64))
                           .view(np.int16)).cuda()
    mb = att.tmap_encode("bf16", 2, d16.data_ptr(), ex["dims"], (8192,), ex["box"], None, "none")
    out = {}
    for key, fn, box_bytes in (("int32", lambda: att.tile_reduce_add(mi, rc.data_ptr(), ex["nbox"], src.data_ptr(),
                                                                      stream), 16384),
                               ("bf16", lambda: att.tile_reduce(mb, "add", rc.data_ptr(), ex["nbox"], s16.data_ptr(),
                                                                stream), 8192)):
        fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        out[key] = {"us": round(ms * 1e3, 2), "GBps_algorithmic": round(ex["nbox"] * box_bytes * 3 / ms / 1e6, 1)}
    out["bf16_per_byte_vs_int32"] = round(out["int32"]["GBps_algorithmic"] / out["bf16"]["GBps_algorithmic"], 3)
    return out


def run_reduce_scale(att, torch, stream, reps: int = 10, rounds: int = 3):
    """The reduce-add pass (64 x 64 boxes at uniform origins in [0, 4032]^2
    of a 4096 x 4096 destination) at 128 to 8192 boxes, int32 and bf16
    interleaved per round; the median per pass over `rounds` rounds of
    `reps` dispatches.  Separates the pass's fixed latency (below about
    1000 boxes every workgroup is resident at once) from its per-byte cost."""
    import numpy as np

    import synthgen
    from synthgen import workloads as W

    ex = W.REDUCE_4096
    counts = (128, 256, 512, 1024, 2048, 4096, 8192)
    nmax = counts[-1]
    rc = torch.from_numpy(synthgen.uniform_coords(ex["seed"] * 1000 + 30, nmax, (0, 0), (4032, 4032))).cuda()
    dst = torch.from_numpy(synthgen.int32_range(ex["seed"], (4096, 4096), -(1 << 20), 1 << 20)).cuda()
    src = torch.from_numpy(synthgen.int32_range(ex["seed"] * 1000 + 31, (nmax, 64, 64), -(1 << 20), 1 << 20)).cuda()
    mi = att.tmap_encode("i32", 2, dst.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, "none")
    d16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"], (4096, 4096)).view(np.int16)).cuda()
    s16 = torch.from_numpy(synthgen.normal_bf16_bits(ex["seed"] * 1000 + 32, (nmax, 64, 64)).view(np.int16)).cuda()
    mb = att.tmap_encode("bf16", 2, d16.data_ptr(), ex["dims"], (8192,), ex["box"], None, "none")
    times = {}
    for _ in range(rounds):
        for n in counts:
            for key, fn in (("int32", lambda n=n: att.tile_reduce_add(mi, rc.data_ptr(), n, src.data_ptr(), stream)),
                            ("bf16", lambda n=n: att.tile_reduce(mb, "add", rc.data_ptr(), n, s16.data_ptr(),
                                                                 stream))):
                fn()
                torch.cuda.synchronize()
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                for _ in range(reps):
                    fn()
                e.record()
                torch.cuda.synchronize()
                times.setdefault((key, n), []).append(s.elapsed_time(e) / reps)
    out = []
    for n in counts:
        row = {"boxes": n}
        for key, bb in (("int32", 16384), ("bf16", 8192)):
            ms = sorted(times[(key, n)])[len(times[(key, n)]) // 2]
            row[key + "_us"] = round(ms * 1e3, 2)
            row[key + "_GBps"] = round(n * bb * 3 / ms / 1e6, 1)
        row["bf16_per_byte_vs_int32"] = round(row["int32_GBps"] / row["bf16_GBps"], 3)
        out.append(row)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--stages", type=int, default=2)
    ap.add_argument("--variant", type=int, default=-1, help="-1: tile_copy defaults")
    ap.add_argument("--grid", type=int, default=0)
    ap.add_argument("--pairs", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary workloads (rank-5 load, reduce-add pass, GEMM 8192^3)")
    ap.add_argument("--only", choices=["copy", "gemm", "gemm-raster", "lds-probe", "copy-compare", "reduce",
                                       "reduce-scale"],
                    default="copy",
                    help="gemm: time only the GEMM mainloop; gemm-raster: the default GEMM under each tile "
                         "rasterisation; lds-probe: run the LDS bank probe layouts; copy-compare: the tile copy "
                         "beside the plain and box-shaped copies; reduce: the int32 and bf16 reduce-add passes "
                         "(profiling runs); reduce-scale: those passes at 128 to 8192 boxes")
    ap.add_argument("--gemm-variant", default="all",
                    help="bk,stages[,k256][,mfma] e.g. 32,4,k256 or 64,2,k256,32 (with --only gemm)")
    ap.add_argument("--gemm-c-f32", action="store_true",
                    help="with --only gemm: write C as the fp32 accumulators (gemm_bf16_f32; 64-deep K step)")
    ap.add_argument("--ref-copy", action="store_true",
                    help="also time a plain device-to-device copy of the same bytes")
    ap.add_argument("--ceiling", action="store_true", help="time the HBM ceiling too (the default)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip timing plain read-only, write-only and copy kernels over the same working sets")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import async_tensor_tile_amd as att
    import synthgen
    from synthgen import workloads as W

    att.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream().cuda_stream
    if args.only == "lds-probe":
        # one dispatch per layout: the pages' grouped / 256-byte-stride sector
        # reads (0, 1), an MFMA 32x32 operand fragment under 128B (2) and
        # 128B_K256 (3), and the GEMM epilogue's C staging writes (4: 128B_K256,
        # 6: 128B) and reads (5), each repeated 1000 times for the LDS counters
        h = torch.zeros(9 * 16 * 8, dtype=torch.int32, device="cuda")
        for layout in range(7):
            att.lds_bank_probe(layout, 1000, h.data_ptr(), stream)
        torch.cuda.synchronize()
        print(json.dumps({"lds_probe_layouts": 7, "iters": 1000}), flush=True)
        return
    if args.only == "copy-compare":
        print(json.dumps({"copy_compare": run_copy_compare(att, torch, stream)}), flush=True)
        return
    if args.only == "reduce":
        print(json.dumps({"reduce_compare": run_reduce_compare(att, torch, stream)}), flush=True)
        return
    if args.only == "reduce-scale":
        print(json.dumps({"reduce_scale": run_reduce_scale(att, torch, stream)}), flush=True)
        return
    if args.only == "gemm-raster":
        print(json.dumps({"gemm_raster": run_gemm_raster(att, torch, stream, args.steps),
                          "order": [list(r) for r in GEMM_RASTERS], "rounds": 3,
                          "dispatches_per_raster_and_round": args.steps + 1}), flush=True)
        return
    if args.only == "gemm":
        variants = GEMM_VARIANTS
        if args.gemm_variant != "all":
            bk, st, *rest = args.gemm_variant.split(",")
            bk, st = int(bk), int(st)
            k256 = "k256" in rest
            mi = [int(x) for x in rest if x.isdigit()]
            mi = mi[0] if mi else (16 if bk == 64 else 32)
            variants = ((bk, ("128b" if bk == 64 else "64b") + ("_k256" if k256 else ""), st, mi),)
        if args.gemm_c_f32:
            variants = tuple(v for v in variants if v[0] == 64 and v[3] == 16)
        res = run_gemm(att, torch, stream, args.steps, variants, vendor=not args.gemm_c_f32,
                       c_f32=args.gemm_c_f32)
        best = res[res["gemm_best"]]
        workload = "bf16 GEMM M=N=K=8192" + (", fp32 C" if args.gemm_c_f32 else "")
        print(json.dumps({"metric": "bf16 GEMM 8192^3 TFLOP/s", "value": best["TFLOPs"], "unit": "TFLOP/s",
                          "n_gpus": 1, "steps": args.steps, "higher_is_better": True, "dtype": "bf16",
                          "data": "synthetic", "config": {"workload": workload},
                          "roofline": {"bound": "mfma", "achieved": best["TFLOPs"], "peak": 2500.0,
                                       "unit": "TFLOP/s", "frac": round(best["TFLOPs"] / 2500.0, 4),
                                       "traffic": gemm_traffic() if (variants == (GEMM_DEFAULT,)
                                                                     and not args.gemm_c_f32) else None},
                          "detail": res}), flush=True)
        return
    ex = W.COPY_8192
    src_host = torch.from_numpy(synthgen.u16_bits(ex["seed"], (8192, 8192)).view(np.uint8).reshape(-1))
    pairs = []
    for p in range(args.pairs):
        s = src_host.to("cuda")
        d = torch.empty_like(s)
        ms_ = att.tmap_encode("bf16", 2, s.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, ex["swizzle"])
        md_ = att.tmap_encode("bf16", 2, d.data_ptr(), ex["dims"], ex["strides"], ex["box"], None, ex["swizzle"])
        pairs.append((s, d, ms_, md_))

    def step(k):
        _, _, ms_, md_ = pairs[k % len(pairs)]
        if args.variant < 0:
            att.tile_copy(ms_, md_, args.stages, stream)
        else:
            att.tile_copy_ex(ms_, md_, args.stages, args.grid, args.variant, stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for k in range(args.steps):
        step(k)
    end.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / args.steps
    gbs = BYTES_PER_STEP / (ms_step / 1e3) / 1e9

    verified = all(torch.equal(s, d) for s, d, _, _ in pairs)

    ref_copy = None
    if args.ref_copy:
        def ref_step(k):
            s_, d_, _, _ = pairs[k % len(pairs)]
            d_.copy_(s_)
        for k in range(args.warmup):
            ref_step(k)
        torch.cuda.synchronize()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a_.record()
        for k in range(args.steps):
            ref_step(k)
        b_.record()
        torch.cuda.synchronize()
        rms = a_.elapsed_time(b_) / args.steps
        ref_copy = {"what": "torch copy_ of the same 128 MiB pairs (plain device copy)",
                    "GBps": round(BYTES_PER_STEP / rms / 1e6, 1), "ms": round(rms, 5)}

    ctr = committed_counters()
    traffic = None
    conflicts = None
    if ctr:
        traffic = ctr.get("hbm_bytes_per_launch")
        conflicts = ctr.get("lds_bank_conflict_cycles_per_tile")

    result = {
        "metric": "tiled box copy GB/s (% of 8 TB/s HBM) bf16 8192^2, LDS bank conflicts/tile",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bf16 8192x8192 tile round trip global->LDS->global, box 128x64, "
                               "128B swizzle, 2 stages per workgroup (producer / consumer waves)",
                   "box": [64, 128], "tiles": 8192, "stages": args.stages, "variant": args.variant,
                   "grid": args.grid or "auto", "buffer_pairs": args.pairs},
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "lds_bank_conflicts_per_tile": conflicts,
        "verified_bit_exact": verified,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if ref_copy:
        result["reference_copy"] = ref_copy
    if not args.no_ceiling:
        ceil = hbm_ceiling(att, torch, stream)
        result["hbm_ceiling"] = ceil
        result["frac_of_linear_copy"] = round(gbs / ceil["copy_GBps"], 4)
        best_copy = max(ceil["copy_GBps"], ceil.get("copy_sweep_best", {}).get("GBps", 0.0))
        result["frac_of_best_plain_copy"] = round(gbs / best_copy, 4)
        if "box_copy_sweep_best" in ceil:
            result["frac_of_box_shaped_copy"] = round(gbs / ceil["box_copy_sweep_best"]["GBps"], 4)
    if not args.no_extra:
        result["extra"] = run_extra(att, torch, stream, 20)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
