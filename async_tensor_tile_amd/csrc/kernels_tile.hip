// kernels_tile.hip -- batch load / store / reduce-add kernels, the
// byte-counted barrier self-test and the LDS bank-sector probe, with their
// C-ABI launchers.  The batch kernels are written against the public device
// API (tile.hpp) and take the host's 128-byte map by value.
//
// Batch kernels run one workgroup (4 waves) per box: the box goes through a
// real LDS image, exactly as a single copy of [HPC] "single-tile load" /
// "TMA store" / "TMA reduce" would, and the image is dumped or consumed.
#include <hip/hip_runtime.h>

#include <cstring>

#include "host_util.hpp"
#include "tile.hpp"
#include "tmap.h"

namespace att {

constexpr uint32_t kBatchThreads = 256;

// Error bits the batch kernels record instead of trapping: a bounded barrier
// wait gave up (the box it guarded is not valid), and, in builds with
// ATT_DEBUG, a box whose waves issued other than its byte count or a barrier
// found in the wrong state when its box was consumed.  Read and cleared by
// tile_device_status.
enum : uint32_t { DEVERR_TIMEOUT = 1u, DEVERR_BYTES = 2u, DEVERR_PHASE = 4u };
static __device__ uint32_t g_dev_error;

__device__ __forceinline__ void record_error(uint32_t bits) {
    __hip_atomic_fetch_or(&g_dev_error, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Consume-side check of a barrier that completed phase 0: its state must be
// re-armed (arrivals = count, pending 0) with the phase flipped, unless a
// wait timed out (already recorded).  Debug builds only.
__device__ __forceinline__ void check_consumed(TxBar* bar, bool ok) {
    if (!ok) {
        if (threadIdx.x % 64u == 0) record_error(DEVERR_TIMEOUT);
        return;
    }
#ifdef ATT_DEBUG
    const int64_t st = __hip_atomic_load(&bar->state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t ph = __hip_atomic_load(&bar->phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (threadIdx.x == 0 && (st != ((int64_t)bar->expected << 32) || ph != 1u)) record_error(DEVERR_PHASE);
#else
    (void)bar;
#endif
}

#ifdef ATT_DEBUG
// Debug builds poison an LDS image before it is loaded (a consumer that
// reads before the copies land then sees the pattern, not stale data) and
// add up the bytes the waves issued, which must equal the box bytes.
constexpr uint32_t kPoison = 0xDBDBDBDBu;
__device__ __forceinline__ void poison_image(uint8_t* img, uint32_t bytes) {
    for (uint32_t i = threadIdx.x; i < bytes / 16u; i += blockDim.x)
        reinterpret_cast<u32x4*>(img)[i] = u32x4{kPoison, kPoison, kPoison, kPoison};
}
#endif

__device__ __forceinline__ void read_coords(const TmapImpl& m, const int32_t* __restrict__ coords,
                                            uint32_t b, int32_t c[5]) {
#pragma unroll
    for (int d = 0; d < 5; ++d) c[d] = d < m.rank ? coords[(size_t)b * m.rank + d] : 0;
}

// Load box b into LDS with the byte-counted barrier, then dump the image.
__global__ __launch_bounds__(kBatchThreads) void k_tile_load(tmap_t map, const int32_t* __restrict__ coords,
                                                            uint8_t* __restrict__ out, uint32_t bar_off) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    TxBar* bar = reinterpret_cast<TxBar*>(smem + bar_off);
    const TmapImpl m = tmap_tiled_uniform(map);
    const uint32_t b = blockIdx.x;
    const uint32_t tid = threadIdx.x, wave = tid >> 6, nwaves = blockDim.x >> 6;
    int32_t c[5];
    read_coords(m, coords, b, c);
#ifdef ATT_DEBUG
    uint32_t* issued = reinterpret_cast<uint32_t*>(smem + bar_off + sizeof(TxBar));
    poison_image(smem, m.box_bytes);
    if (tid == 0) *issued = 0;
#endif
    if (tid == 0) {
        txbar_init(bar, 1);
        txbar_arrive_expect_tx(bar, (int32_t)tile_box_bytes(map));   // expect before any copy is issued
    }
    __syncthreads();
    // the barrier form: each wave's share completes on `bar` once landed
    const uint32_t bytes = tile_load_async(map, c, smem, bar, wave, nwaves);
#ifdef ATT_DEBUG
    if (lane_id() == 0) atomicAdd(issued, bytes);
#endif
    check_consumed(bar, txbar_wait(bar, 0));
#ifdef ATT_DEBUG
    __syncthreads();
    if (tid == 0 && *issued != m.box_bytes) record_error(DEVERR_BYTES);
#else
    (void)bytes;
#endif
    const uint32_t nchunk = m.box_bytes >> 4;
    uint8_t* dst = out + (size_t)b * m.box_bytes;
    for (uint32_t i = tid; i < nchunk; i += blockDim.x)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(smem + i * 16u), reinterpret_cast<u32x4*>(dst + i * 16u));
}

// Load box b of an im2col map into LDS (swizzle on write, byte-counted
// completion as in the tiled load), then dump the image.
__global__ __launch_bounds__(kBatchThreads) void k_tile_load_im2col(tmap_t map, const int32_t* __restrict__ coords,
                                                                   const int32_t* __restrict__ offsets,
                                                                   uint8_t* __restrict__ out, uint32_t bar_off) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    TxBar* bar = reinterpret_cast<TxBar*>(smem + bar_off);
    const Im2colImpl& m = tmap_im2col(map);
    const uint32_t b = blockIdx.x;
    const uint32_t tid = threadIdx.x, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const int R = m.rank, S = R - 2;
    int32_t c[5] = {0, 0, 0, 0, 0};
    int32_t off[3] = {0, 0, 0};
#pragma unroll
    for (int d = 0; d < 5; ++d)
        if (d < R) c[d] = coords[(size_t)b * R + d];
#pragma unroll
    for (int s = 0; s < 3; ++s)
        if (s < S) off[s] = offsets[(size_t)b * S + s];
#ifdef ATT_DEBUG
    poison_image(smem, m.box_bytes);
#endif
    if (tid == 0) {
        txbar_init(bar, 1);
        txbar_arrive_expect_tx(bar, (int32_t)m.box_bytes);
    }
    __syncthreads();
    const uint32_t bytes = tile_load_im2col_async(map, c, off, smem, wave, nwaves);
    tile_load_arrive(bar, bytes);
    check_consumed(bar, txbar_wait(bar, 0));
    const uint32_t nchunk = m.box_bytes >> 4;
    uint8_t* dst = out + (size_t)b * m.box_bytes;
    for (uint32_t i = tid; i < nchunk; i += blockDim.x)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(smem + i * 16u), reinterpret_cast<u32x4*>(dst + i * 16u));
}

// Stage the raw image of box b into LDS, then store / reduce it through the map.
template <int OP>
__global__ __launch_bounds__(kBatchThreads) void k_tile_store(tmap_t map, const int32_t* __restrict__ coords,
                                                             const uint8_t* __restrict__ in) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const TmapImpl m = tmap_tiled_uniform(map);
    const uint32_t b = blockIdx.x;
    const uint32_t tid = threadIdx.x, wave = tid >> 6, nwaves = blockDim.x >> 6;
    const uint32_t nchunk = m.box_bytes >> 4;
    const uint8_t* src = in + (size_t)b * m.box_bytes;
    for (uint32_t grp = wave; grp * 64u < nchunk; grp += nwaves) {
        const uint32_t p = grp * 64u + lane_id();
        if (p < nchunk) dma16(src + p * 16u, smem + grp * 1024u);
    }
    // the box origin is fetched once the image copies are in flight (its
    // scalar load would otherwise hold them up)
    int32_t c[5];
    read_coords(m, coords, b, c);
    wait_vmcnt<0>();
    __syncthreads();
    if constexpr (OP == ST_STORE) tile_store_async(map, c, smem, wave, nwaves);
    else if constexpr (OP == ST_ADD) tile_reduce_async<TMAP_REDUCE_ADD>(map, c, smem, wave, nwaves);
    else if constexpr (OP == ST_MIN) tile_reduce_async<TMAP_REDUCE_MIN>(map, c, smem, wave, nwaves);
    else tile_reduce_async<TMAP_REDUCE_MAX>(map, c, smem, wave, nwaves);
}

// Byte-counted barrier self-test: one barrier (arrival count 1) completes
// after `ntile` copies signal their own byte counts.  Trace records are
// (who, arrivals_left, pending, phase); who = -1 init, -2 arrive.expect_tx,
// t >= 0 the complete-tx of tile t.
__global__ __launch_bounds__(kBatchThreads) void k_txbar_selftest(tmap_t map, const int32_t* __restrict__ coords,
                                                                 uint32_t ntile, int32_t* __restrict__ trace,
                                                                 uint8_t* __restrict__ out, uint32_t img_stride,
                                                                 uint32_t bar_off, uint32_t extra_bytes,
                                                                 uint32_t max_polls) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    TxBar* bar = reinterpret_cast<TxBar*>(smem + bar_off);
    uint32_t* counter = reinterpret_cast<uint32_t*>(smem + bar_off + sizeof(TxBar));
    const TmapImpl m = tmap_tiled_uniform(map);
    const uint32_t tid = threadIdx.x, wave = tid >> 6, nwaves = blockDim.x >> 6;
    if (tid == 0) {
        txbar_init(bar, 1);
        trace[0] = -1; trace[1] = bar->expected; trace[2] = 0; trace[3] = 0;
        const TxState s = txbar_arrive_expect_tx(bar, (int32_t)(tile_box_bytes(map) * ntile + extra_bytes));
        trace[4] = -2; trace[5] = s.arrivals_left; trace[6] = s.pending; trace[7] = (int32_t)s.phase;
        *counter = 0;
    }
    __syncthreads();
    for (uint32_t t = wave; t < ntile; t += nwaves) {
        int32_t c[5];
        read_coords(m, coords, t, c);
        // one wave issues the whole box, then reports its bytes itself so the
        // state after each complete-tx can be recorded
        const uint32_t bytes = tile_load_async(map, c, smem + t * img_stride, 0, 1);
        wait_vmcnt<0>();
        wait_lgkm0();
        if (lane_id() == 0) {
            const TxState s = txbar_complete_tx(bar, (int32_t)bytes);
            const uint32_t slot = 2u + atomicAdd(counter, 1u);
            trace[slot * 4 + 0] = (int32_t)t;
            trace[slot * 4 + 1] = s.arrivals_left;
            trace[slot * 4 + 2] = s.pending;
            trace[slot * 4 + 3] = (int32_t)s.phase;
        }
    }
    const bool ok = txbar_wait(bar, 0, max_polls);
    if (extra_bytes == 0) check_consumed(bar, ok);
    else if (!ok && tid == 0) record_error(DEVERR_TIMEOUT);
    for (uint32_t t = 0; t < ntile; ++t) {
        const uint32_t nchunk = m.box_bytes >> 4;
        for (uint32_t i = tid; i < nchunk; i += blockDim.x)
            *reinterpret_cast<u32x4*>(out + (size_t)t * m.box_bytes + i * 16u) =
                *reinterpret_cast<const u32x4*>(smem + t * img_stride + i * 16u);
    }
}

// Physical LDS address (bytes) of the 16-byte sector (row r, column col) of
// the 16 x 256-byte grid under the 128-byte swizzle.
//   layout 1: grouped as a (group, row, col) box of 2 x 16 x 128 bytes.
//   layout 0: kept at a 256-byte row stride (a reference layout only).
__device__ __forceinline__ uint32_t probe_addr(int32_t layout, uint32_t r, uint32_t col) {
    const uint32_t q = layout == 1 ? ((col >> 3) * 16u + r) * 8u + (col & 7u) : r * 16u + col;
    return swz_chunk(q, TMAP_SWIZZLE_128B) * 16u;
}

__global__ __launch_bounds__(64) void k_lds_bank_probe(int32_t layout, uint32_t iters, int32_t* __restrict__ hist) {
    __shared__ __attribute__((aligned(1024))) uint8_t grid[4096];
    const uint32_t lane = threadIdx.x;
    for (uint32_t i = lane; i < 256; i += 64) reinterpret_cast<u32x4*>(grid)[i] = u32x4{i, i, i, i};
    __syncthreads();
    uint32_t sink = 0;
    if (layout >= 4) {
        // The GEMM epilogue's C staging into 128-byte-row box images of the
        // C map: layout 4 (128B_K256) and 6 (128B) write as the epilogue's
        // first ds_write_b64 does (lane l: row l % 16, four bf16 columns at
        // 4 * (l / 16)); layout 5 reads as its first ds_read_b128 does
        // (lane l: row l / 8, logical chunk l % 8) under 128B_K256.
        const uint32_t sw = layout == 6 ? TMAP_SWIZZLE_128B : TMAP_SWIZZLE_128B_K256;
        uint32_t a;
        if (layout == 5) {
            a = swz_chunk(lane, sw) * 16u;
        } else {
            const uint32_t row = lane & 15u, col = (lane >> 4) * 4u;
            a = (swz_chunk(row * 8u + (col >> 3), sw) << 4) + (col & 7u) * 2u;
        }
        const uint32_t la = lds_addr_of(grid) + a;
        for (uint32_t it = 0; it < iters; ++it) {
            if (layout == 5) {
                const u32x4 v = lds_read16(la);
                wait_lgkm0();
                sink ^= v.x;
            } else {
                asm volatile("ds_write_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(la), "v"(uint2{it, lane}) : "memory");
            }
        }
        hist[lane] = (int32_t)a;
        if (sink == 0xFFFFFFFFu) hist[64] = -1;
        return;
    }
    if (layout >= 2) {
        // One MFMA 32x32x16 operand fragment from a 32-row x 128-byte box:
        // lane l reads row l % 32, logical chunk l / 32, at the physical
        // chunk the swizzle gives (layout 2: 128B, layout 3: 128B_K256).
        const uint32_t sw = layout == 2 ? TMAP_SWIZZLE_128B : TMAP_SWIZZLE_128B_K256;
        const uint32_t a = swz_chunk((lane & 31u) * 8u + (lane >> 5), sw) * 16u;
        const uint32_t la = lds_addr_of(grid) + a;
        for (uint32_t it = 0; it < iters; ++it) {
            const u32x4 v = lds_read16(la);
            wait_lgkm0();
            sink ^= v.x;
        }
        hist[lane] = (int32_t)a;
        if (sink == 0xFFFFFFFFu) hist[64] = -1;
        return;
    }
    for (uint32_t row0 = 0; row0 <= 8; ++row0) {
        for (uint32_t col = 0; col < 16; ++col) {
            const uint32_t a = probe_addr(layout, row0 + (lane & 7u), col);
            const uint32_t sector = (a >> 4) & 7u;
            if (lane < 8) {
                const uint32_t la = lds_addr_of(grid) + a;
                for (uint32_t it = 0; it < iters; ++it) {
                    const u32x4 v = lds_read16(la);
                    wait_lgkm0();
                    sink ^= v.x;
                }
            }
            for (uint32_t s = 0; s < 8; ++s) {
                const uint64_t hit = __ballot(lane < 8 && sector == s);
                if (lane == 0) hist[(row0 * 16 + col) * 8 + s] = (int32_t)__popcll(hit);
            }
        }
    }
    if (sink == 0xFFFFFFFFu) hist[0] = -1;   // keeps the timed reads alive
}

// The caller's descriptor by value for a kernel argument; copied bytewise,
// since the caller's 128 bytes need not sit at tmap_t's 64-byte alignment.
static tmap_t map_value(const tmap_t* m) {
    tmap_t v;
    std::memcpy(&v, m, sizeof(v));
    return v;
}

static tmap_status prepare_dynamic_lds(const void* fn, uint32_t bytes) {
    uint32_t limit = 0;
    tmap_status st = device_lds_limit(&limit);
    if (st) return st;
    if (bytes > limit) return TMAP_ERR_LDS_CAPACITY;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    return TMAP_OK;
}

}  // namespace att

using namespace att;

extern "C" tmap_status tile_load(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                                 void* d_lds_image_out, void* stream) {
    if (!m) return TMAP_ERR_NULL;
    const TmapImpl t = load_map(m);
    if (is_im2col(t)) return TMAP_ERR_UNSUPPORTED;
    if (nbox == 0) return TMAP_OK;
    if (!d_coords || !d_lds_image_out) return TMAP_ERR_NULL;
    const uint32_t bar_off = round_up(t.box_bytes, 1024u);
    const uint32_t lds = bar_off + 64u;
    tmap_status st = prepare_dynamic_lds((const void*)k_tile_load, lds);
    if (st) return st;
    hipLaunchKernelGGL(k_tile_load, dim3(nbox), dim3(kBatchThreads), lds, as_stream(stream), map_value(m), d_coords,
                       static_cast<uint8_t*>(d_lds_image_out), bar_off);
    return check_launch("tile_load");
}

template <int OP>
static tmap_status launch_store(const tmap_t* m, const int32_t* d_coords, uint32_t nbox, const void* d_in,
                                void* stream, const char* name) {
    if (!m) return TMAP_ERR_NULL;
    const TmapImpl t = load_map(m);
    if (is_im2col(t)) return TMAP_ERR_UNSUPPORTED;
    if (nbox == 0) return TMAP_OK;
    if (!d_coords || !d_in) return TMAP_ERR_NULL;
    const uint32_t lds = round_up(t.box_bytes, 1024u);
    tmap_status st = prepare_dynamic_lds((const void*)k_tile_store<OP>, lds);
    if (st) return st;
    hipLaunchKernelGGL(k_tile_store<OP>, dim3(nbox), dim3(kBatchThreads), lds, as_stream(stream), map_value(m),
                       d_coords, static_cast<const uint8_t*>(d_in));
    return check_launch(name);
}

extern "C" tmap_status tile_store(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                                  const void* d_lds_image_in, void* stream) {
    return launch_store<ST_STORE>(m, d_coords, nbox, d_lds_image_in, stream, "tile_store");
}

extern "C" tmap_status tile_reduce_add(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                                       const void* d_lds_image_in, void* stream) {
    return launch_store<ST_ADD>(m, d_coords, nbox, d_lds_image_in, stream, "tile_reduce_add");
}

extern "C" tmap_status tile_reduce(const tmap_t* m, int32_t op, const int32_t* d_coords, uint32_t nbox,
                                   const void* d_lds_image_in, void* stream) {
    switch (op) {
    case TMAP_REDUCE_ADD: return launch_store<ST_ADD>(m, d_coords, nbox, d_lds_image_in, stream, "tile_reduce");
    case TMAP_REDUCE_MIN: return launch_store<ST_MIN>(m, d_coords, nbox, d_lds_image_in, stream, "tile_reduce");
    case TMAP_REDUCE_MAX: return launch_store<ST_MAX>(m, d_coords, nbox, d_lds_image_in, stream, "tile_reduce");
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

extern "C" tmap_status tile_load_im2col(const tmap_t* m, const int32_t* d_coords, const int32_t* d_offsets,
                                        uint32_t nbox, void* d_lds_image_out, void* stream) {
    if (!m) return TMAP_ERR_NULL;
    Im2colImpl t;
    std::memcpy(&t, m, sizeof(t));
    if (!(t.oob & OOB_IM2COL_FLAG) || t.rank < 3 || t.rank > 5) return TMAP_ERR_UNSUPPORTED;
    if (nbox == 0) return TMAP_OK;
    if (!d_coords || !d_offsets || !d_lds_image_out) return TMAP_ERR_NULL;
    const uint32_t bar_off = round_up(t.box_bytes, 1024u);
    const uint32_t lds = bar_off + 64u;
    tmap_status st = prepare_dynamic_lds((const void*)k_tile_load_im2col, lds);
    if (st) return st;
    hipLaunchKernelGGL(k_tile_load_im2col, dim3(nbox), dim3(kBatchThreads), lds, as_stream(stream), map_value(m), d_coords,
                       d_offsets, static_cast<uint8_t*>(d_lds_image_out), bar_off);
    return check_launch("tile_load_im2col");
}

extern "C" tmap_status txbar_selftest_ex(const tmap_t* m, const int32_t* d_coords, uint32_t ntile,
                                         uint32_t extra_bytes, uint32_t max_polls, int32_t* d_trace,
                                         void* d_lds_image_out, void* stream) {
    if (!m || !d_coords || !d_trace || !d_lds_image_out) return TMAP_ERR_NULL;
    if (ntile < 1 || ntile > 8) return TMAP_ERR_UNSUPPORTED;
    const TmapImpl t = load_map(m);
    if (is_im2col(t)) return TMAP_ERR_UNSUPPORTED;
    if ((uint64_t)t.box_bytes * ntile > (1u << 30)) return TMAP_ERR_LDS_CAPACITY;
    const uint32_t img_stride = round_up(t.box_bytes, 1024u);
    const uint32_t bar_off = img_stride * ntile;
    const uint32_t lds = bar_off + 64u;
    tmap_status st = prepare_dynamic_lds((const void*)k_txbar_selftest, lds);
    if (st) return st;
    if (extra_bytes >= (1u << 30) || max_polls == 0) return TMAP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_txbar_selftest, dim3(1), dim3(kBatchThreads), lds, as_stream(stream), map_value(m), d_coords, ntile,
                       d_trace, static_cast<uint8_t*>(d_lds_image_out), img_stride, bar_off, extra_bytes, max_polls);
    return check_launch("txbar_selftest");
}

extern "C" tmap_status txbar_selftest(const tmap_t* m, const int32_t* d_coords, uint32_t ntile,
                                      int32_t* d_trace, void* d_lds_image_out, void* stream) {
    return txbar_selftest_ex(m, d_coords, ntile, 0u, 1u << 22, d_trace, d_lds_image_out, stream);
}

extern "C" tmap_status tile_device_status(void* stream) {
    hipError_t e = hipStreamSynchronize(as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    uint32_t bits = 0;
    e = hipMemcpyFromSymbol(&bits, HIP_SYMBOL(g_dev_error), sizeof(bits), 0, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyFromSymbol");
    if (bits == 0) return TMAP_OK;
    const uint32_t zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_dev_error), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyToSymbol");
    return (bits & DEVERR_TIMEOUT) ? TMAP_ERR_TIMEOUT : TMAP_ERR_DEVICE_CHECK;
}

extern "C" tmap_status lds_bank_probe(int32_t layout, uint32_t iters, int32_t* d_hist, void* stream) {
    if (!d_hist) return TMAP_ERR_NULL;
    if (layout < 0 || layout > 6) return TMAP_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(k_lds_bank_probe, dim3(1), dim3(64), 0, as_stream(stream), layout, iters, d_hist);
    return check_launch("lds_bank_probe");
}
