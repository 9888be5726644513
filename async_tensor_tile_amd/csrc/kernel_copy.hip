// kernel_copy.hip -- full-grid round trip global -> LDS -> global through two
// tensor maps, with a multi-stage LDS ring ([MLC] "TMA in a pipeline": fill
// stage k+1 while stage k is consumed).
//
// Design for gfx950.  A box of B bytes is split into 1 KiB groups (64 lanes x
// 16 bytes, one global_load_lds_dwordx4 each).  The swizzle only permutes
// chunks inside a 128-byte unit, so the wave that loads a group holds every
// chunk it later stores: each wave owns GPW groups of every box and runs its
// own S-deep ring without any workgroup barrier.  Completion of a stage is the
// wave's s_waitcnt vmcnt, counted in DMA instructions issued after that stage;
// LDS reads are inline-asm ds_read_b128 at the swizzled address and go out as
// coalesced global_store_dwordx4 in logical order.  The producer / consumer
// form (the default for two stages) splits the roles instead: one wave
// issues every copy of the workgroup's boxes and four waves store them.
// Edge tiles, element strides or shapes that do not split evenly take the
// generic path: one workgroup per box through tile_load_issue /
// tile_store_issue.
#include <hip/hip_runtime.h>

#include <type_traits>
#include <utility>

#include "host_util.hpp"
#include "att/tile_device.hpp"
#include "tmap.h"

namespace att {

struct CopyArgs {
    TmapImpl src;
    TmapImpl dst;
    uint32_t ntiles;
    uint32_t nt[5];     // tiles per dimension
    uint32_t chunked;   // 1: workgroup b owns tiles [b*per, b*per + per); 0: tiles b + n*grid
    uint32_t xcd;       // 1: renumber workgroups so each XCD owns one contiguous range
    // Maps of rank 1 or 2: what the fast paths read, each field 4- or
    // 8-byte aligned so that it comes in through a scalar load.  Several
    // descriptor fields are single bytes at offsets that are not multiples of
    // four, which the compiler fetches with a vector-memory load at the start
    // of every workgroup: a memory round trip before its first copy.
    uint64_t r2_sbase, r2_dbase, r2_sstride, r2_dstride;
    uint32_t r2_box0, r2_box1, r2_sesize, r2_desize, r2_swizzle, r2_cpr, r2_magic_cpr;
};

// Copy variant flags (tile_copy_ex `variant`).
// Bits 4..5 select how many consecutive boxes share one ring stage (1, 2, 4, 8).
enum : uint32_t {
    CV_NT_STORE = 1u, CV_GENERIC = 2u, CV_CHUNKED = 4u, CV_XCD = 8u, CV_NB_SHIFT = 4u, CV_BATCH = 64u, CV_ROWMAJOR = 128u,
    CV_REGLOAD = 256u, CV_PC = 512u
};
constexpr uint32_t kNumXcd = 8;

constexpr uint32_t kCopyWaves = 4;

// Box t of a rank 1 or 2 map from the aligned fields only: byte offsets of
// its origin in src and dst.  Box row t1 is walked starting t1 boxes along
// dim 0, as in tile_origin.
__device__ __forceinline__ void tile_origin_r2(const CopyArgs& a, uint32_t t, uint64_t& so, uint64_t& dof) {
    const uint32_t t1 = t / a.nt[0];
    uint32_t t0 = t - t1 * a.nt[0] + t1 % a.nt[0];
    if (t0 >= a.nt[0]) t0 -= a.nt[0];
    const uint64_t c0 = (uint64_t)t0 * a.r2_box0, c1 = (uint64_t)t1 * a.r2_box1;
    so = c0 * a.r2_sesize + c1 * a.r2_sstride;
    dof = c0 * a.r2_desize + c1 * a.r2_dstride;
}

// Byte offsets of tile t's origin in src and dst (tiles innermost first).
__device__ __forceinline__ void tile_origin(const CopyArgs& a, uint32_t t, uint64_t& so, uint64_t& dof,
                                            int32_t c[5]) {
    if (a.src.rank <= 2) {
        // one division instead of five (the short-lived workgroups pay this
        // per box).  Box row t1 is walked starting t1 boxes along dim 0 (a
        // rotation of each row, so every box is still visited once): the
        // workgroups in flight together, which straddle neighbouring box
        // rows, then sit at different dim-0 offsets.  Measured on the bf16
        // 8192^2 round trip in 128 x 64 boxes: 2 % faster than the plain
        // row-major walk (and as fast as an XOR of the row into the column).
        const uint32_t t1 = t / a.nt[0];
        uint32_t t0 = t - t1 * a.nt[0] + t1 % a.nt[0];
        if (t0 >= a.nt[0]) t0 -= a.nt[0];
        c[0] = (int32_t)(t0 * (a.src.box_m1[0] + 1u));
        c[1] = (int32_t)(t1 * (a.src.box_m1[1] + 1u));
        c[2] = c[3] = c[4] = 0;
        so = (uint64_t)c[0] * a.src.esize + (uint64_t)c[1] * a.src.stride[0];
        dof = (uint64_t)c[0] * a.dst.esize + (uint64_t)c[1] * a.dst.stride[0];
        return;
    }
    so = 0;
    dof = 0;
#pragma unroll
    for (int d = 0; d < 5; ++d) {
        const uint32_t n = a.nt[d];
        const uint32_t td = t % n;
        t /= n;
        c[d] = (int32_t)(td * (a.src.box_m1[d] + 1u));
        const uint64_t e = (uint64_t)c[d];
        so += d == 0 ? e * a.src.esize : e * a.src.stride[d - 1];
        dof += d == 0 ? e * a.dst.esize : e * a.dst.stride[d - 1];
    }
}

template <int GPW>
__device__ __forceinline__ void lds_read_group(const uint32_t (&addr)[GPW], u32x4 (&v)[GPW]);

template <>
__device__ __forceinline__ void lds_read_group<1>(const uint32_t (&a)[1], u32x4 (&v)[1]) {
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v[0]) : "v"(a[0]) : "memory");
}
template <>
__device__ __forceinline__ void lds_read_group<2>(const uint32_t (&a)[2], u32x4 (&v)[2]) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]) : "v"(a[0]), "v"(a[1]) : "memory");
}
template <>
__device__ __forceinline__ void lds_read_group<4>(const uint32_t (&a)[4], u32x4 (&v)[4]) {
    asm volatile("ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\t"
                 "ds_read_b128 %3, %7\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]) : "memory");
}
template <>
__device__ __forceinline__ void lds_read_group<8>(const uint32_t (&a)[8], u32x4 (&v)[8]) {
    asm volatile("ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\t"
                 "ds_read_b128 %3, %11\n\tds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\t"
                 "ds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]),
                   "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
                 : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]),
                   "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]) : "memory");
}

// Per-lane constants of a wave's GPW groups, identical for every box: where
// the chunk this lane loads comes from (its logical chunk swz(p)), where the
// chunk it stores goes (logical chunk p) and the LDS address of the slot
// holding the latter.  Maps of rank 1 or 2 take a few integer operations per
// chunk (box row = chunk / chunks-per-row) instead of the general rank-5
// address generator.
template <int GPW>
__device__ __forceinline__ void copy_lane_offsets(const CopyArgs& a, uint32_t wave, uint32_t lane, uint32_t lds0,
                                                  uint64_t (&ld_off)[GPW], uint64_t (&st_off)[GPW], uint32_t (&rd)[GPW]) {
    const uint32_t sw = a.src.swizzle;
    const int32_t zero[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < GPW; ++j) {
        const uint32_t p = (wave * GPW + j) * 64u + lane;
        const uint32_t q = swz_chunk(p, sw);
        rd[j] = lds0 + q * 16u;
        if (a.src.rank <= 2) {
            const uint32_t rq = fdiv(q, a.src.magic_cpr), rp = fdiv(p, a.src.magic_cpr);
            ld_off[j] = (uint64_t)rq * a.src.stride[0] + (q - rq * a.src.cpr) * 16u;
            st_off[j] = (uint64_t)rp * a.dst.stride[0] + (p - rp * a.src.cpr) * 16u;
        } else {
            const ChunkLoc ls = chunk_locate(a.src, zero, q);
            ld_off[j] = (uint64_t)(ls.g0 * a.src.esize + ls.rest_off);
            const ChunkLoc ld = chunk_locate(a.dst, zero, p);
            st_off[j] = (uint64_t)(ld.g0 * a.dst.esize + ld.rest_off);
        }
    }
}

// One stage holds NB consecutive boxes (each its own dense LDS image).  The
// wave issues its DMA instructions row-group major, box minor, so that
// back-to-back requests cover NB neighbouring 128-byte segments of the same
// rows: with 128-byte-wide boxes that is what keeps HBM pages busy.
template <int GPW, int S, int NB>
__global__ __launch_bounds__(kCopyWaves * 64) void k_tile_copy_ring(CopyArgs a_arg, uint32_t nt_store) {
    const CopyArgs a = uniform_copy(a_arg);
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    const uint32_t B = a.src.box_bytes;
    uint64_t ld_off[GPW], st_off[GPW];
    uint32_t rd[GPW];
    const uint32_t lds0 = lds_addr_of(smem);
    copy_lane_offsets<GPW>(a, wave, lane, lds0, ld_off, st_off, rd);

    // Units of NB boxes.  Workgroups are dispatched round-robin over the
    // XCDs; with `xcd` the ones sharing an XCD get neighbouring unit ranges.
    const uint32_t U = a.ntiles / NB;
    const uint32_t G = gridDim.x;
    const uint32_t b = a.xcd ? (blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd : blockIdx.x;
    const uint32_t per = (U + G - 1) / G;
    const uint32_t first = a.chunked ? b * per : b;
    const uint32_t step = a.chunked ? 1u : G;
    if (first >= U) return;
    const uint32_t nmine = a.chunked ? (U - first < per ? U - first : per) : (U - 1 - first) / G + 1;

    auto issue = [&](uint32_t n) {
        const uint32_t t0 = (first + n * step) * NB;
        uint8_t* stage = smem + (n % S) * (NB * B);
        uint64_t sb[NB];
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            uint64_t so, dof;
            int32_t c[5];
            tile_origin(a, t0 + x, so, dof, c);
            sb[x] = a.src.base + so;
        }
#ifdef ATT_DEBUG
        // debug builds poison the wave's groups of the stage before refilling
        // them, so a read ahead of its copies sees the pattern
#pragma unroll
        for (int j = 0; j < GPW; ++j)
#pragma unroll
            for (int x = 0; x < NB; ++x)
                *reinterpret_cast<u32x4*>(stage + x * B + (wave * GPW + j) * 1024u + lane * 16u) =
                    u32x4{0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu};
        wait_lgkm0();
#endif
#pragma unroll
        for (int j = 0; j < GPW; ++j)
#pragma unroll
            for (int x = 0; x < NB; ++x)
                dma16((const void*)(uintptr_t)(sb[x] + ld_off[j]), stage + x * B + (wave * GPW + j) * 1024u);
    };

#pragma unroll
    for (int s = 0; s < S - 1; ++s)
        if ((uint32_t)s < nmine) issue(s);

    for (uint32_t n = 0; n < nmine; ++n) {
        if (n + S - 1 < nmine) issue(n + S - 1);
        const uint32_t left = nmine - 1 - n;
        wait_stage<GPW * NB, S - 1>(left < (uint32_t)(S - 1) ? left : (uint32_t)(S - 1));
        const uint32_t t0 = (first + n * step) * NB;
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            uint32_t addr[GPW];
            const uint32_t soff = (n % S) * (NB * B) + x * B;
#pragma unroll
            for (int j = 0; j < GPW; ++j) addr[j] = rd[j] + soff;
            u32x4 v[GPW];
            lds_read_group<GPW>(addr, v);
            uint64_t so, dof;
            int32_t c[5];
            tile_origin(a, t0 + x, so, dof, c);
            gbyte* db = gptr(a.dst.base + dof);
#pragma unroll
            for (int j = 0; j < GPW; ++j) {
                ATT_GLOBAL u32x4* p = (ATT_GLOBAL u32x4*)(db + st_off[j]);
                if (nt_store) __builtin_nontemporal_store(v[j], p);
                else *p = v[j];
            }
        }
    }
}

// Batch round trip: workgroup b owns NBOX consecutive boxes and gives each
// its own LDS stage.  Every wave issues all its copies up front, then takes
// the stages in order -- waiting only for that stage's copies (loads
// complete in issue order; no store has been issued yet, so vmcnt counts
// copies alone) and reading its chunks into registers -- and stores all of
// them at the end.  No wait ever covers a store, so the end of one box's
// stores is never on the path to the next box, and the workgroup retires as
// soon as its stores are issued.
template <int GPW, int NBOX, bool ROWMAJOR, bool REGLOAD>
__global__ __launch_bounds__(kCopyWaves * 64) void k_tile_copy_batch(CopyArgs a_arg, uint32_t nt_store) {
    const CopyArgs a = uniform_copy(a_arg);
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    const uint32_t B = a.src.box_bytes;
    const uint32_t G = gridDim.x;
    const uint32_t b = a.xcd ? (blockIdx.x % kNumXcd) * (G / kNumXcd) + blockIdx.x / kNumXcd : blockIdx.x;
    const uint32_t t0 = b * NBOX;
    if (t0 >= a.ntiles) return;
    const uint32_t lds0 = lds_addr_of(smem);
    uint64_t ld_off[GPW], st_off[GPW];
    uint32_t rd[GPW];
    copy_lane_offsets<GPW>(a, wave, lane, lds0, ld_off, st_off, rd);
    uint64_t sof[NBOX], dof[NBOX];
#pragma unroll
    for (int x = 0; x < NBOX; ++x) {
        int32_t c[5];
        tile_origin(a, t0 + x, sof[x], dof[x], c);
#ifdef ATT_DEBUG
#pragma unroll
        for (int j = 0; j < GPW; ++j)
            *reinterpret_cast<u32x4*>(smem + x * B + (wave * GPW + j) * 1024u + lane * 16u) =
                u32x4{0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu};
#endif
    }
#ifdef ATT_DEBUG
    wait_lgkm0();
#endif
    // ROWMAJOR: copy j of every box, then copy j+1 (the boxes sit side by
    // side, so back-to-back requests cover the same rows NBOX x 128 bytes
    // wide); else box by box.
    u32x4 v[NBOX][GPW];
    if constexpr (REGLOAD) {
        // the loads go to registers and each lane writes its chunk to the
        // slot the copy engine form would (the same LDS image); the wave
        // reads back only chunks it wrote itself, so LDS order suffices
#pragma unroll
        for (int o = 0; o < NBOX * GPW; ++o) {
            const int x = ROWMAJOR ? o % NBOX : o / GPW, j = ROWMAJOR ? o / NBOX : o % GPW;
            v[x][j] = *(const ATT_GLOBAL u32x4*)gptr(a.src.base + sof[x] + ld_off[j]);
        }
#pragma unroll
        for (int o = 0; o < NBOX * GPW; ++o) {
            const int x = ROWMAJOR ? o % NBOX : o / GPW, j = ROWMAJOR ? o / NBOX : o % GPW;
            *reinterpret_cast<u32x4*>(smem + x * B + (wave * GPW + j) * 1024u + lane * 16u) = v[x][j];
        }
    } else {
#pragma unroll
        for (int o = 0; o < NBOX * GPW; ++o) {
            const int x = ROWMAJOR ? o % NBOX : o / GPW, j = ROWMAJOR ? o / NBOX : o % GPW;
            dma16((const void*)(uintptr_t)(a.src.base + sof[x] + ld_off[j]), smem + x * B + (wave * GPW + j) * 1024u);
        }
        // every copy of the workgroup's boxes has landed (the wave only
        // reads chunks it copied itself)
        wait_vmcnt<0>();
    }
    // all stages read with ordinary LDS loads (one wait for all of them),
    // then every chunk stored, in the order the loads went out
#pragma unroll
    for (int x = 0; x < NBOX; ++x)
#pragma unroll
        for (int j = 0; j < GPW; ++j)
            v[x][j] = *reinterpret_cast<const u32x4*>(smem + x * B + (rd[j] - lds0));
#pragma unroll
    for (int o = 0; o < NBOX * GPW; ++o) {
        const int x = ROWMAJOR ? o % NBOX : o / GPW, j = ROWMAJOR ? o / NBOX : o % GPW;
        ATT_GLOBAL u32x4* p = (ATT_GLOBAL u32x4*)(gptr(a.dst.base + dof[x]) + st_off[j]);
        if (nt_store) __builtin_nontemporal_store(v[x][j], p);
        else *p = v[x][j];
    }
}

// Per-lane constants of group g of a box: the global offset of the logical
// chunk its DMA lane copies (ld), the offset the chunk its store lane writes
// goes to (st) and the LDS byte offset holding the latter (rd).
template <bool R2>
__device__ __forceinline__ void group_lane_offsets(const CopyArgs& a, uint32_t g, uint32_t lane, uint64_t& ld,
                                                   uint64_t& st, uint32_t& rd) {
    const uint32_t p = g * 64u + lane;
    if constexpr (R2) {
        const uint32_t q = swz_chunk(p, a.r2_swizzle);
        rd = q * 16u;
        const uint32_t rq = fdiv(q, a.r2_magic_cpr), rp = fdiv(p, a.r2_magic_cpr);
        ld = (uint64_t)rq * a.r2_sstride + (q - rq * a.r2_cpr) * 16u;
        st = (uint64_t)rp * a.r2_dstride + (p - rp * a.r2_cpr) * 16u;
        return;
    }
    const uint32_t q = swz_chunk(p, a.src.swizzle);
    rd = q * 16u;
    if (a.src.rank <= 2) {
        const uint32_t rq = fdiv(q, a.src.magic_cpr), rp = fdiv(p, a.src.magic_cpr);
        ld = (uint64_t)rq * a.src.stride[0] + (q - rq * a.src.cpr) * 16u;
        st = (uint64_t)rp * a.dst.stride[0] + (p - rp * a.src.cpr) * 16u;
    } else {
        const int32_t zero[5] = {0, 0, 0, 0, 0};
        const ChunkLoc ls = chunk_locate(a.src, zero, q);
        ld = (uint64_t)(ls.g0 * a.src.esize + ls.rest_off);
        const ChunkLoc ldst = chunk_locate(a.dst, zero, p);
        st = (uint64_t)(ldst.g0 * a.dst.esize + ldst.rest_off);
    }
}

// Producer / consumer round trip, the pages' division of labour between the
// thread that issues the copies and the threads that consume the staged
// tile: wave 0 of a workgroup issues every LDS-DMA copy of its NB boxes (G
// 1 KiB groups each) and then, as the groups land in order, releases them
// kPcCons at a time with a workgroup barrier; each of the kPcCons consumer
// waves reads one released group from LDS and stores it.  The producer only
// ever has copies outstanding, so its vmcnt waits are exact and follow the
// copies one step at a time; the consumers never wait on their stores, so
// a store is issued as soon as its group has landed.  Every wave passes the
// same NB * G / kPcCons barriers.
constexpr uint32_t kPcCons = 4;

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>)
template <typename F, int... I>
__device__ __forceinline__ void unroll_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll_for(F&& f) {
    unroll_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int G, int NB, bool R2>
__global__ __launch_bounds__((kPcCons + 1) * 64) void k_tile_copy_pc(CopyArgs a_arg, uint32_t nt_store) {
    const CopyArgs a = uniform_copy(a_arg);
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr int K = G * NB;                          // groups per workgroup
    constexpr int STEPS = K / (int)kPcCons;
    static_assert(K % (int)kPcCons == 0 && K <= 64, "whole steps; vmcnt range");
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    const uint32_t B = a.src.box_bytes;
    const uint32_t t0 = blockIdx.x * NB;
    if (wave == 0) {
        uint64_t ld[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            uint64_t st;
            uint32_t rd;
            group_lane_offsets<R2>(a, (uint32_t)g, lane, ld[g], st, rd);
        }
        const uint64_t sbase = R2 ? a.r2_sbase : a.src.base;
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            uint64_t so, dof;
            if constexpr (R2) {
                tile_origin_r2(a, t0 + x, so, dof);
            } else {
                int32_t c[5];
                tile_origin(a, t0 + x, so, dof, c);
            }
#ifdef ATT_DEBUG
#pragma unroll
            for (int g = 0; g < G; ++g)
                *reinterpret_cast<u32x4*>(smem + x * B + g * 1024u + lane * 16u) =
                    u32x4{0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu};
            wait_lgkm0();
#endif
#pragma unroll
            for (int g = 0; g < G; ++g) dma16((const void*)(uintptr_t)(sbase + so + ld[g]), smem + x * B + g * 1024u);
        }
        // step s releases groups [s * kPcCons, (s + 1) * kPcCons): they have
        // landed once at most K - (s + 1) * kPcCons copies are outstanding
        unroll_for<STEPS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            wait_vmcnt<K - (s + 1) * (int)kPcCons>();
            wg_barrier();
        });
    } else {
        const uint32_t cw = wave - 1u;                 // consumer index: group cw of every step
        uint64_t st[G / kPcCons], dof[NB];
        uint32_t rd[G / kPcCons];
#pragma unroll
        for (int i = 0; i < G / (int)kPcCons; ++i) {
            uint64_t ld;
            group_lane_offsets<R2>(a, cw + (uint32_t)i * kPcCons, lane, ld, st[i], rd[i]);
        }
#pragma unroll
        for (int x = 0; x < NB; ++x) {
            uint64_t so;
            if constexpr (R2) {
                tile_origin_r2(a, t0 + x, so, dof[x]);
            } else {
                int32_t c[5];
                tile_origin(a, t0 + x, so, dof[x], c);
            }
        }
        const uint64_t dbase = R2 ? a.r2_dbase : a.dst.base;
        const uint32_t lds0 = lds_addr_of(smem);
        unroll_for<STEPS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            constexpr int k0 = s * (int)kPcCons;       // first group of the step
            constexpr int x = k0 / G, i = (k0 % G) / (int)kPcCons;
            wg_barrier();
            u32x4 v[1];
            const uint32_t addr[1] = {lds0 + x * B + rd[i]};
            lds_read_group<1>(addr, v);
            ATT_GLOBAL u32x4* p = (ATT_GLOBAL u32x4*)(gptr(dbase + dof[x]) + st[i]);
            if (nt_store) __builtin_nontemporal_store(v[0], p);
            else *p = v[0];
        });
    }
}

// Generic round trip: one workgroup per tile, any geometry.
__global__ __launch_bounds__(kCopyWaves * 64) void k_tile_copy_generic(CopyArgs a_arg) {
    const CopyArgs a = uniform_copy(a_arg);
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    const uint32_t wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    uint64_t so, dof;
    int32_t c[5];
    tile_origin(a, blockIdx.x, so, dof, c);
    tile_load_issue(a.src, c, smem, wave, nwaves);
    wait_vmcnt<0>();
    wait_lgkm0();
    __syncthreads();
    tile_store_issue<ST_STORE>(a.dst, c, smem, wave, nwaves);
}

template <int GPW, int NBOX, bool ROWMAJOR, bool REGLOAD>
static tmap_status launch_batch(const CopyArgs& a, uint32_t nt, hipStream_t st) {
    if constexpr (GPW * (NBOX - 1) > 63 || GPW * NBOX > 32) {
        return TMAP_ERR_UNSUPPORTED;           // vmcnt range; registers for every chunk
    } else {
        const uint32_t lds = (uint32_t)NBOX * a.src.box_bytes;
        hipError_t e = hipFuncSetAttribute((const void*)k_tile_copy_batch<GPW, NBOX, ROWMAJOR, REGLOAD>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
        const uint32_t grid = a.ntiles / NBOX;
        hipLaunchKernelGGL((k_tile_copy_batch<GPW, NBOX, ROWMAJOR, REGLOAD>), dim3(grid), dim3(kCopyWaves * 64), lds, st,
                           a, nt);
        return check_launch("tile_copy");
    }
}

template <int GPW, bool REGLOAD>
static tmap_status launch_batch_n(const CopyArgs& a, uint32_t nbox, bool rowmajor, uint32_t nt, hipStream_t st) {
    switch (nbox * 2 + (rowmajor ? 1 : 0)) {
    case 4: return launch_batch<GPW, 2, false, REGLOAD>(a, nt, st);
    case 5: return launch_batch<GPW, 2, true, REGLOAD>(a, nt, st);
    case 6: return launch_batch<GPW, 3, false, REGLOAD>(a, nt, st);
    case 7: return launch_batch<GPW, 3, true, REGLOAD>(a, nt, st);
    case 8: return launch_batch<GPW, 4, false, REGLOAD>(a, nt, st);
    case 9: return launch_batch<GPW, 4, true, REGLOAD>(a, nt, st);
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

template <int GPW>
static tmap_status launch_batch_r(const CopyArgs& a, uint32_t nbox, bool rowmajor, bool regload, uint32_t nt,
                                  hipStream_t st) {
    return regload ? launch_batch_n<GPW, true>(a, nbox, rowmajor, nt, st)
                   : launch_batch_n<GPW, false>(a, nbox, rowmajor, nt, st);
}

template <int G, int NB>
static tmap_status launch_pc(const CopyArgs& a, uint32_t nt, hipStream_t st) {
    if constexpr (G * NB > 64 || (G * NB) % (int)kPcCons != 0 || G < (int)kPcCons) {
        return TMAP_ERR_UNSUPPORTED;
    } else {
        const uint32_t lds = (uint32_t)NB * a.src.box_bytes;
        const void* fn = a.src.rank <= 2 ? (const void*)k_tile_copy_pc<G, NB, true> : (const void*)k_tile_copy_pc<G, NB, false>;
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
        if (a.src.rank <= 2)
            hipLaunchKernelGGL((k_tile_copy_pc<G, NB, true>), dim3(a.ntiles / NB), dim3((kPcCons + 1) * 64), lds, st, a, nt);
        else
            hipLaunchKernelGGL((k_tile_copy_pc<G, NB, false>), dim3(a.ntiles / NB), dim3((kPcCons + 1) * 64), lds, st, a, nt);
        return check_launch("tile_copy");
    }
}

template <int G>
static tmap_status launch_pc_nb(const CopyArgs& a, uint32_t nb, uint32_t nt, hipStream_t st) {
    switch (nb) {
    case 1: return launch_pc<G, 1>(a, nt, st);
    case 2: return launch_pc<G, 2>(a, nt, st);
    case 4: return launch_pc<G, 4>(a, nt, st);
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

template <int GPW, int S, int NB>
static tmap_status launch_ring(const CopyArgs& a, uint32_t grid, uint32_t nt, hipStream_t st) {
    if constexpr (GPW * NB * (S - 1) > 63) {
        return TMAP_ERR_UNSUPPORTED;       // more DMA instructions in flight than vmcnt counts
    } else {
        const uint32_t lds = (uint32_t)S * NB * a.src.box_bytes;
        hipError_t e = hipFuncSetAttribute((const void*)k_tile_copy_ring<GPW, S, NB>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
        hipLaunchKernelGGL((k_tile_copy_ring<GPW, S, NB>), dim3(grid), dim3(kCopyWaves * 64), lds, st, a, nt);
        return check_launch("tile_copy");
    }
}

template <int GPW, int NB>
static tmap_status launch_ring_s(const CopyArgs& a, uint32_t stages, uint32_t grid, uint32_t nt, hipStream_t st) {
    switch (stages) {
    case 1: return launch_ring<GPW, 1, NB>(a, grid, nt, st);
    case 2: return launch_ring<GPW, 2, NB>(a, grid, nt, st);
    case 3: return launch_ring<GPW, 3, NB>(a, grid, nt, st);
    case 4: return launch_ring<GPW, 4, NB>(a, grid, nt, st);
    case 6: return launch_ring<GPW, 6, NB>(a, grid, nt, st);
    case 8: return launch_ring<GPW, 8, NB>(a, grid, nt, st);
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

template <int GPW>
static tmap_status launch_ring_nb(const CopyArgs& a, uint32_t nb, uint32_t stages, uint32_t grid, uint32_t nt,
                                  hipStream_t st) {
    switch (nb) {
    case 1: return launch_ring_s<GPW, 1>(a, stages, grid, nt, st);
    case 2: return launch_ring_s<GPW, 2>(a, stages, grid, nt, st);
    case 4: return launch_ring_s<GPW, 4>(a, stages, grid, nt, st);
    default: return launch_ring_s<GPW, 8>(a, stages, grid, nt, st);
    }
}

static tmap_status launch_ring_g(const CopyArgs& a, uint32_t gpw, uint32_t nb, uint32_t stages, uint32_t grid,
                                 uint32_t nt, hipStream_t st) {
    switch (gpw) {
    case 1: return launch_ring_nb<1>(a, nb, stages, grid, nt, st);
    case 2: return launch_ring_nb<2>(a, nb, stages, grid, nt, st);
    case 4: return launch_ring_nb<4>(a, nb, stages, grid, nt, st);
    default: return launch_ring_nb<8>(a, nb, stages, grid, nt, st);
    }
}

// Persistent grid: workgroups per CU chosen to minimise the tail of the last
// round of tiles, within what LDS allows.
static uint32_t auto_grid(uint32_t ntiles, uint32_t cus, uint32_t lds_per_wg) {
    uint32_t max_k = lds_per_wg ? (uint32_t)(TMAP_LDS_CAPACITY / lds_per_wg) : 8u;
    if (max_k > 8) max_k = 8;
    if (max_k < 1) max_k = 1;
    uint32_t best = cus, best_k = 1;
    double best_eff = -1.0;
    for (uint32_t k = 1; k <= max_k; ++k) {
        const uint64_t g = (uint64_t)cus * k;
        const uint64_t per = (ntiles + g - 1) / g;
        const double eff = (double)ntiles / (double)(g * per);
        if (eff > best_eff + 1e-9 || (eff > best_eff - 1e-9 && k > best_k)) {
            best_eff = eff;
            best = (uint32_t)g;
            best_k = k;
        }
    }
    return best < ntiles ? best : ntiles;
}

}  // namespace att

using namespace att;

extern "C" tmap_status tile_copy_ex(const tmap_t* src, const tmap_t* dst, uint32_t stages, uint32_t grid,
                                    uint32_t variant, void* stream) {
    if (!src || !dst) return TMAP_ERR_NULL;
    if (stages < 1 || stages > 8 || variant > 1023) return TMAP_ERR_UNSUPPORTED;
    CopyArgs a;
    a.src = load_map(src);
    a.dst = load_map(dst);
    if (is_im2col(a.src) || is_im2col(a.dst)) return TMAP_ERR_UNSUPPORTED;
    if (a.src.dtype != a.dst.dtype || a.src.rank != a.dst.rank || a.src.swizzle != a.dst.swizzle)
        return TMAP_ERR_UNSUPPORTED;
    bool even = true;
    uint64_t T = 1;
    for (int d = 0; d < 5; ++d) {
        if (a.src.dim[d] != a.dst.dim[d] || a.src.L[d] != a.dst.L[d] || a.src.es[d] != 1 || a.dst.es[d] != 1)
            return TMAP_ERR_UNSUPPORTED;
        const uint64_t bx = (uint64_t)a.src.box_m1[d] + 1u;
        const uint64_t n = ((uint64_t)a.src.dim[d] + bx - 1) / bx;
        a.nt[d] = (uint32_t)n;
        even = even && ((uint64_t)a.src.dim[d] % bx == 0);
        T *= n;
    }
    if (T == 0 || T > 0x7FFFFFFFull) return TMAP_ERR_UNSUPPORTED;
    a.ntiles = (uint32_t)T;
    a.chunked = (variant & CV_CHUNKED) ? 1u : 0u;
    a.xcd = 0u;
    a.r2_sbase = a.src.base;
    a.r2_dbase = a.dst.base;
    a.r2_sstride = a.src.rank >= 2 ? a.src.stride[0] : 0u;
    a.r2_dstride = a.dst.rank >= 2 ? a.dst.stride[0] : 0u;
    a.r2_box0 = (uint32_t)a.src.box_m1[0] + 1u;
    a.r2_box1 = (uint32_t)a.src.box_m1[1] + 1u;
    a.r2_sesize = a.src.esize;
    a.r2_desize = a.dst.esize;
    a.r2_swizzle = a.src.swizzle;
    a.r2_cpr = a.src.cpr;
    a.r2_magic_cpr = a.src.magic_cpr;
    uint32_t limit = 0, cus = 0;
    tmap_status st = device_lds_limit(&limit);
    if (st) return st;
    st = device_cu_count(&cus);
    if (st) return st;
    const uint32_t B = a.src.box_bytes;
    const uint32_t groups = B / 1024u;
    const uint32_t gpw = (B % 1024u == 0) ? groups / kCopyWaves : 0u;
    uint32_t nb = 1u << ((variant >> CV_NB_SHIFT) & 3u);
    if (a.ntiles % nb != 0) nb = 1;
    const bool ring_ok = even && !(variant & CV_GENERIC) && gpw * kCopyWaves == groups &&
                         (gpw == 1 || gpw == 2 || gpw == 4 || gpw == 8) && stages * nb * B <= limit &&
                         gpw * nb * (stages - 1) <= 63 && stages != 5 && stages != 7;
    hipStream_t s = as_stream(stream);
    // batch mode: `stages` boxes per workgroup, one stage each
    const bool batch_ok = (variant & CV_BATCH) && even && !(variant & CV_GENERIC) && gpw * kCopyWaves == groups &&
                          (gpw == 1 || gpw == 2 || gpw == 4 || gpw == 8) && stages >= 2 && stages <= 4 &&
                          stages * B <= limit && a.ntiles % stages == 0 && gpw * (stages - 1) <= 63;
    // producer / consumer mode: `stages` boxes per workgroup (1, 2 or 4),
    // one stage each, boxes of 4, 8, 16 or 32 KiB
    const bool pc_ok = (variant & CV_PC) && even && !(variant & CV_GENERIC) && B % 4096u == 0 && B <= 32768u &&
                       (stages == 1 || stages == 2 || stages == 4) && stages * (B / 1024u) <= 64 &&
                       a.ntiles % stages == 0 && stages * B <= limit;
    if (pc_ok) {
        const uint32_t nt = (variant & CV_NT_STORE) ? 1u : 0u;
        switch (B / 1024u) {
        case 4: return launch_pc_nb<4>(a, stages, nt, s);
        case 8: return launch_pc_nb<8>(a, stages, nt, s);
        case 16: return launch_pc_nb<16>(a, stages, nt, s);
        default: return launch_pc_nb<32>(a, stages, nt, s);
        }
    }
    if (batch_ok) {
        const uint32_t g = a.ntiles / stages;
        a.xcd = ((variant & CV_XCD) && g % kNumXcd == 0) ? 1u : 0u;
        const uint32_t nt = (variant & CV_NT_STORE) ? 1u : 0u;
        const bool rm = (variant & CV_ROWMAJOR) != 0, rl = (variant & CV_REGLOAD) != 0;
        switch (gpw) {
        case 1: return launch_batch_r<1>(a, stages, rm, rl, nt, s);
        case 2: return launch_batch_r<2>(a, stages, rm, rl, nt, s);
        case 4: return launch_batch_r<4>(a, stages, rm, rl, nt, s);
        default: return launch_batch_r<8>(a, stages, rm, rl, nt, s);
        }
    }
    if (ring_ok) {
        const uint32_t units = a.ntiles / nb;
        const uint32_t g = grid ? grid : auto_grid(units, cus, stages * nb * B);
        a.xcd = ((variant & CV_XCD) && g % kNumXcd == 0) ? 1u : 0u;
        return launch_ring_g(a, gpw, nb, stages, g, (variant & CV_NT_STORE) ? 1u : 0u, s);
    }
    const uint32_t lds = round_up(B, 1024u);
    if (lds > limit) return TMAP_ERR_LDS_CAPACITY;
    hipError_t e = hipFuncSetAttribute((const void*)k_tile_copy_generic, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    hipLaunchKernelGGL(k_tile_copy_generic, dim3(a.ntiles), dim3(kCopyWaves * 64), lds, s, a);
    return check_launch("tile_copy");
}

// Default launch: non-temporal stores, workgroups owning neighbouring boxes,
// two ring stages' worth of boxes per workgroup so that LDS, not the grid,
// bounds how many workgroups share a CU.  With two stages the producer /
// consumer form takes the two boxes where the box size allows it (measured
// on the bf16 8192^2 round trip: 49.7-49.8 us against the ring's 50.1).
extern "C" tmap_status tile_copy(const tmap_t* src, const tmap_t* dst, uint32_t stages, void* stream) {
    if (!src) return TMAP_ERR_NULL;
    const TmapImpl s = load_map(src);
    uint64_t T = 1;
    for (int d = 0; d < 5; ++d) {
        const uint64_t bx = (uint64_t)s.box_m1[d] + 1u;
        T *= ((uint64_t)s.dim[d] + bx - 1) / bx;
    }
    const uint32_t grid = T >= 2 ? (uint32_t)((T + 1) / 2) : 1u;
    return tile_copy_ex(src, dst, stages, grid, CV_NT_STORE | CV_CHUNKED | (stages == 2 ? CV_PC : 0u), stream);
}
