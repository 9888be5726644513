// kernel_gemm.hip -- bf16 GEMM mainloop fed by the tile loader: the consumer
// the reference pages motivate ([MLC] overview: the matrix unit must not wait
// for the next A / B tiles; "TMA in a pipeline": fill one stage while the
// other is consumed).
//
// C[M,N] = A[M,K] * B[K,N]; A row-major (map dims {K, M}), B column-major
// (map dims {K, N}); both are K-contiguous, so every 16-byte LDS chunk holds 8
// consecutive K values of one row -- exactly one MFMA operand per lane.
//
// Workgroup tile 256 x 256, K-step BK (the box's inner extent: 64 bf16 =
// 128-byte rows under the 128-byte swizzle, or 32 bf16 = 64-byte rows under
// the 64-byte swizzle), S-stage LDS ring.  Four waves in a 2 x 2 layout each
// own a 128 x 128 block of C held as 4 x 4 tiles of v_mfma_f32_32x32x16_bf16
// accumulators.  Per stage every wave copies its quarter of the A and B boxes
// with global_load_lds_dwordx4 (swizzle applied on the source side, as in the
// loader), waits vmcnt, and one s_barrier publishes the stage.  Fragment
// reads use the same swizzle: lane l of a 32 x 16 operand reads row l % 32,
// logical chunk 2*kk + l / 32, at the physical chunk the map's swizzle gives.
// With the pages' 8-row key those reads hit every LDS bank twice on gfx950
// (16 lanes x 16 bytes per clock); the _K256 modes' 16-row key removes that.
#include <hip/hip_runtime.h>

#include <cstring>
#include <type_traits>
#include <utility>

#include "host_util.hpp"
#include "tile.hpp"
#include "tmap.h"

namespace att {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kTM = 256, kTN = 256;
constexpr int kGemmThreads = 256;

struct GemmArgs {
    TmapImpl A;          // dims {K, M}, box {BK, 256}
    TmapImpl B;          // dims {K, N}, box {BK, 256}
    uint64_t C;          // bf16, row-major, leading dimension ldc elements
    uint32_t M, N, K, ldc;
    uint32_t tiles_m, tiles_n;
    uint32_t group_m;    // tile rows per rasterisation group
    uint32_t xcd;        // 0: plain order, 1: contiguous ranges per XCD, 2: a 2-D block of tiles per XCD
    uint32_t blk_m, blk_n;   // xcd == 2: tile rows / columns of each XCD's block
    uint32_t c_staged;       // 1: C written back through Cm (LDS image + tile store)
    TmapImpl Cm;             // C map: dims {N, M}, box {64, 256}, 128B swizzle
};

// Swizzle of the staged epilogue's C box images: the 128-byte mode, whose
// key (row % 8) differs across any 8 consecutive rows, so the 16-byte writes
// of 8 lanes holding one chunk column of 8 consecutive rows hit 8 distinct
// bank groups.
constexpr uint32_t kCSwizzle = TMAP_SWIZZLE_128B;

// The C map of the staged epilogue: dims {N, M} with a row stride of
// ld_bytes, box {64, 256}, bf16, 128B swizzle, zero fill -- exactly
// what tmap_encode makes of those arguments (the host compares the two
// before choosing the staged epilogue).  Built here from constants but the
// base, stride and dims, so the box store inlined into the epilogue folds
// its per-map fields instead of keeping them in scalar registers.
__host__ __device__ __forceinline__ TmapImpl gemm_c_box_map(uint64_t base, uint64_t ld_bytes, uint32_t N,
                                                           uint32_t M) {
    TmapImpl t;
    t.base = base;
    t.stride[0] = ld_bytes;
    t.stride[1] = t.stride[2] = t.stride[3] = 0;
    t.dim[0] = N;
    t.dim[1] = M;
    t.dim[2] = t.dim[3] = t.dim[4] = 1;
    t.L[0] = 64;
    t.L[1] = 256;
    t.L[2] = t.L[3] = t.L[4] = 1;
    t.box_m1[0] = 63;
    t.box_m1[1] = 255;
    t.box_m1[2] = t.box_m1[3] = t.box_m1[4] = 0;
    t.es[0] = t.es[1] = t.es[2] = t.es[3] = t.es[4] = 1;
    t.rank = 2;
    t.dtype = TMAP_BF16;
    t.esize = 2;
    t.swizzle = kCSwizzle;
    t.oob = TMAP_OOB_ZERO;
    t.fill_idx = FILL_ZERO;
    t.cpr = 8;
    t.box_bytes = 32768;
    t.magic_cpr = 0x20000000u;      // ceil(2^32 / 8)
    t.magic_L[0] = 0x01000000u;     // ceil(2^32 / 256)
    t.magic_L[1] = t.magic_L[2] = 0;
    return t;
}

// One iteration of the main loop as a fixed sequence of MFMA slots (see the
// kernel): which MFMA each slot runs, which fragment read follows it, and the
// lgkmcnt the slot must wait for before its MFMA.  A wave's C block is NI x
// NJ MFMA tiles; one sub-step (one MFMA K extent) needs NI A and NJ B
// fragments and runs SUB = NI * NJ MFMAs; an iteration covers KK sub-steps.
// The last AR accumulator rows of the previous tile's last sub-step run at
// the start of the next iteration, under the reads of its first sub-step.
// Fragment reads are issued as inline asm (so the compiler's LDS-DMA alias
// tracking adds no vmcnt waits) and complete in issue order, so the wait is
// exact (clamped to the counter's 4 bits, which only waits longer).
// The 16 x 16 MFMAs here are inline asm, so the compiler does not know their
// latency: code it generates next to them (accumulator copies at control-
// flow joins, spills, the epilogue's reads) could read a result that has not
// landed, or write an accumulator a queued MFMA still reads.  Issued MFMAs
// queue behind each other for well over a hundred cycles, so the drain is
// 32 x 8 wait states; it runs once per tile, after the last MFMA.
// acc_fence() then hands every accumulator through an empty asm statement
// ordered after the drain, so that no compiler copy of a final value can be
// placed before it; at the start it pins the zeroed accumulators in AGPRs
// before the first MFMA.
template <typename AccT, int NI, int NJ>
__device__ __forceinline__ void acc_fence(AccT (&acc)[NI][NJ]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
}

__device__ __forceinline__ void mfma_drain() {
    asm volatile(
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
        "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

template <int NI, int NJ, int KK, int AR = NI / 2>
struct GemmSched {
    static constexpr int NA = NI;                     // A fragments (ids 0..NA-1; B fragments follow)
    static constexpr int SUB = NI * NJ;
    static constexpr int HALF = AR * NJ;              // slots of rows NI-AR.. of the last sub-step
    static constexpr int NF = NI + NJ;                // fragments per sub-step
    static constexpr int RA = HALF / NF;              // read spacing while finishing the previous tile
    static constexpr int RB = SUB / NF;               // read spacing inside a sub-step
    static constexpr int SLOTS = SUB * KK;
    static constexpr int B_END = HALF + SUB * (KK - 1);
    static_assert(RA >= 1 && RB >= 1 && HALF % NF == 0 && SUB % NF == 0, "read spacing");
    // MFMA of slot m: accumulator row i, column j, fragment buffer.
    static constexpr int mi(int m) {
        return m < HALF ? NI - AR + m / NJ : (m < B_END ? ((m - HALF) % SUB) / NJ : (m - B_END) / NJ);
    }
    static constexpr int mj(int m) { return m < HALF ? m % NJ : (m < B_END ? (m - HALF) % NJ : (m - B_END) % NJ); }
    static constexpr int mbuf(int m) { return m < HALF ? 1 : (m < B_END ? ((m - HALF) / SUB) & 1 : 1); }
    // Read order inside a sub-step: A0 and B0..B(NJ-1) first, since the
    // following MFMAs start with accumulator row 0; fragment ids 0..NI-1 are
    // A rows, NI.. B columns.
    static constexpr int order(int p) { return p == 0 ? 0 : (p <= NJ ? NI + p - 1 : p - NJ); }
    // Fragment read after slot m's MFMA, or -1; its sub-step and buffer.
    static constexpr int rfrag(int m) {
        return m < HALF ? (m % RA == 0 ? order(m / RA) : -1)
                        : (m < B_END && ((m - HALF) % RB) == 0 ? order(((m - HALF) % SUB) / RB) : -1);
    }
    static constexpr int rkk(int m) { return m < HALF ? 0 : (m - HALF) / SUB + 1; }
    static constexpr int rbuf(int m) { return rkk(m) & 1; }
    static constexpr int reads_before(int m) {
        int n = 0;
        for (int x = 0; x < m; ++x) n += rfrag(x) >= 0;
        return n;
    }
    // Issue index (within the iteration) of the read that filled fragment f
    // of the buffer slot m consumes; -1 if it was read in an earlier
    // iteration (complete at the barrier).
    static constexpr int producer(int m, int f) {
        for (int x = m - 1; x >= 0; --x)
            if (rfrag(x) == f && rbuf(x) == mbuf(m)) return reads_before(x);
        return -1;
    }
    // lgkmcnt to wait for before slot m's MFMA, or -1 for none.
    static constexpr int lgkm(int m) {
        const int pa = producer(m, mi(m)), pb = producer(m, NI + mj(m));
        const int p = pa > pb ? pa : pb;
        const int w = p < 0 ? -1 : reads_before(m) - p - 1;
        return w > 15 ? 15 : w;
    }
};

// Slot HALF (first MFMA of sub-step 0) needs A0 and B0, the first two of the
// NF reads issued while the previous tile finishes.
static_assert(GemmSched<4, 4, 2>::lgkm(8) == 6 && GemmSched<4, 4, 4>::lgkm(8) == 6, "schedule");
static_assert(GemmSched<4, 4, 2>::lgkm(0) == -1 && GemmSched<4, 4, 2>::lgkm(31) >= 0, "schedule");
static_assert(GemmSched<8, 8, 2>::lgkm(32) == 14 && GemmSched<8, 8, 2>::SLOTS == 128, "schedule");
static_assert(GemmSched<8, 8, 2, 6>::mi(0) == 2 && GemmSched<8, 8, 2, 6>::mi(47) == 7 && GemmSched<8, 8, 2, 6>::mi(127) == 1,
              "schedule");

// The schedule's lgkmcnt waits with the redundant ones dropped: LDS reads
// complete in issue order, so once a wait has covered read p, a later MFMA
// that needs read p or an earlier one needs no wait of its own (which would
// cost an issue slot and nothing else).  w[m] is the count to wait for before
// slot m's MFMA, or -1 for none; every wait that remains equals Sch::lgkm(m).
template <typename Sch>
struct GemmWaits {
    int w[Sch::SLOTS];
    constexpr GemmWaits() : w() {
        int last[2][Sch::NF] = {};   // index of the latest read of fragment f into buffer b, -1 for none
        for (int b = 0; b < 2; ++b)
            for (int f = 0; f < Sch::NF; ++f) last[b][f] = -1;
        int nread = 0, covered = -1;
        for (int m = 0; m < Sch::SLOTS; ++m) {
            const int b = Sch::mbuf(m);
            const int pa = last[b][Sch::mi(m)], pb = last[b][Sch::NA + Sch::mj(m)];
            const int p = pa > pb ? pa : pb;
            if (p < 0 || p <= covered) {
                w[m] = -1;
            } else {
                const int c = nread - p - 1 > 15 ? 15 : nread - p - 1;
                w[m] = c;
                covered = nread - c - 1;
            }
            const int f = Sch::rfrag(m);
            if (f >= 0) last[Sch::rbuf(m)][f] = nread++;
        }
    }
};
template <typename Sch>
constexpr GemmWaits<Sch> kGemmWaits{};

template <typename Sch>
constexpr bool waits_consistent() {
    int kept = 0;
    for (int m = 0; m < Sch::SLOTS; ++m) {
        const int w = kGemmWaits<Sch>.w[m];
        if (w >= 0 && w != Sch::lgkm(m)) return false;
        if (w < 0 && Sch::lgkm(m) < 0) continue;
        kept += w >= 0;
    }
    return kept > 0;
}
static_assert(waits_consistent<GemmSched<8, 8, 2, 4>>() && waits_consistent<GemmSched<4, 4, 2>>(), "pruned waits");

// The operand ring's copies: dma16_sv with only the one wait state the M0
// write needs.  dma16_sv's four more (for a VALU write of the base SGPRs
// just before) sit on the ring's issue path and cost 5 % of the GEMM.  The
// ring's bases and M0 values come from scalar arithmetic, and its kernels
// spill no SGPRs (a spill restore is a VALU write, v_readlane); the CPU
// suite compiles this file to gfx950 assembly and checks both: no
// SGPR-base DMA of any kernel here has a VALU write of its base or M0 within
// five wait states on any path, and the ring kernels report no SGPR spills.
// Debug builds poison the 1 KiB group before refilling it (a fragment read
// ahead of its copy then sees the pattern) and keep the full wait states.
__device__ __forceinline__ void dma16_sv_ring(uint64_t sbase, uint32_t voff, uint32_t lds_group_addr) {
#ifdef ATT_DEBUG
    typedef __attribute__((address_space(3))) u32x4 lds_u4_t;
    *(lds_u4_t*)(uintptr_t)(lds_group_addr + lane_id() * 16u) =
        u32x4{0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu, 0xDBDBDBDBu};
    wait_lgkm0();
    dma16_sv(sbase, voff, lds_group_addr);
#else
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_group_addr)
                 : "memory");
#endif
}

template <int N>
__device__ __forceinline__ void wait_lgkm() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Tile (tm, tn) of workgroup b: groups of `group_m` tile rows are walked
// column by column so that concurrently running workgroups share A and B
// panels in L2.
__device__ __forceinline__ void gemm_tile_of(const GemmArgs& g, uint32_t b, uint32_t& tm, uint32_t& tn) {
    const uint32_t per_group = g.group_m * g.tiles_n;
    const uint32_t grp = b / per_group;
    const uint32_t first_m = grp * g.group_m;
    const uint32_t rows = (g.tiles_m - first_m) < g.group_m ? (g.tiles_m - first_m) : g.group_m;
    const uint32_t in = b - grp * per_group;
    tm = first_m + in % rows;
    tn = in / rows;
}

// C tile of this workgroup.  Workgroups are dispatched round-robin over the
// 8 XCDs; xcd == 1 renumbers them so that each XCD owns a contiguous range of
// the grouped order, xcd == 2 gives XCD x a blk_m x blk_n block of C tiles
// (blocks 2 wide in n), walked in groups of group_m tile rows, so its L2
// serves blk_m A panels and blk_n B panels instead of whole tile rows.
__device__ __forceinline__ void gemm_block_tile(const GemmArgs& g, uint32_t& tm, uint32_t& tn) {
    const uint32_t G = gridDim.x;
    if (g.xcd == 2) {
        const uint32_t x = blockIdx.x % 8u, local = blockIdx.x / 8u;
        const uint32_t bm0 = (x >> 1) * g.blk_m, bn0 = (x & 1u) * g.blk_n;
        const uint32_t gm = g.group_m < g.blk_m ? g.group_m : g.blk_m;
        const uint32_t per = gm * g.blk_n;
        const uint32_t grp = local / per, in = local % per;
        tm = bm0 + grp * gm + in % gm;
        tn = bn0 + in / gm;
    } else {
        const uint32_t bid = g.xcd ? (blockIdx.x % 8u) * (G / 8u) + blockIdx.x / 8u : blockIdx.x;
        gemm_tile_of(g, bid, tm, tn);
    }
}

// Epilogue of a workgroup's 256 x 256 C tile from the accumulators of its
// four waves (2 x 2 blocks of 128 x 128, NI x NJ tiles of MI x MI each).
template <int MI, bool CF32, typename AccT, int NI, int NJ>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, AccT (&acc)[NI][NJ], uint8_t* smem, uint32_t lds0,
                                              uint32_t wave, uint32_t lane, uint32_t m0, uint32_t n0) {
    // Epilogue.  The MFMAs take B as their first operand, so accumulator
    // (i, j) holds the transposed MI x MI tile: register 4q + r of lane l is C
    // row i*MI + l%MI of the wave's block and column j*MI + q*8 + (l/MI)*4 + r,
    // i.e. four consecutive columns per group of four registers (8 bytes of
    // bf16, converted with round-to-nearest-even); MI*MI/256 groups per tile.
    constexpr int NQ = MI * MI / 256;
    const uint32_t wm = wave >> 1, wn = wave & 1;
    const uint32_t rloc = wm * 128u + (lane % (uint32_t)MI);
    const uint32_t cloc = wn * 128u + (lane / (uint32_t)MI) * 4u;
    if constexpr (CF32) {
        // fp32 C straight from the accumulators: each group of four
        // registers is four consecutive columns of one row, one 16-byte
        // store where C allows it, element stores at the N edge.
        ATT_GLOBAL float* C = (ATT_GLOBAL float*)gptr(g.C);
        const bool vec = (g.C & 15u) == 0 && g.ldc % 4u == 0;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const uint32_t row = m0 + rloc + (uint32_t)i * (uint32_t)MI;
                    const uint32_t col = n0 + cloc + (uint32_t)j * (uint32_t)MI + (uint32_t)q * 8u;
                    if (row >= g.M) continue;
                    ATT_GLOBAL float* dst = C + (uint64_t)row * g.ldc + col;
                    if (vec && col + 4u <= g.N) {
                        *(ATT_GLOBAL f32x4*)dst = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                                        acc[i][j][4 * q + 3]};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (col + (uint32_t)e < g.N) dst[e] = acc[i][j][4 * q + e];
                    }
                }
        return;
    }
    if (g.c_staged) {
        // Registers -> LDS -> global through the tile store, as the pages'
        // epilogue does ([MLC] "waiting for a TMA store": write the output
        // tile to shared memory, store it, wait on the store group, then
        // reuse the buffer).  The 256 x 256 tile is four 256 x 64 boxes of
        // the C map (128-byte rows, 128-byte swizzle).  With 16 x 16 tiles
        // a lane holds four consecutive columns of one row per tile; lanes
        // l and l + 16 swap halves of two neighbouring tiles
        // (v_permlane16_swap), so that each lane holds a whole 16-byte
        // chunk (eight columns of one row) and writes it with one 16-byte
        // LDS store: 8 lanes of a store cover one chunk column of 8
        // consecutive rows, 8 distinct bank groups under the row % 8 key.
        // (With 32 x 32 tiles the lanes write their 8-byte pieces.)  Two
        // LDS stages of one box each are used twice: in pass r the waves of
        // column half wn write box 2*wn + r (their accumulator columns j*MI
        // with j in [r*NJ/2, (r+1)*NJ/2)) into stage wn, then every wave
        // stores its share of both boxes as two store groups; pass 1 refills
        // the stages once those groups no longer read them.  The box store clips
        // at the M / N edges.  The ring is free once every wave has passed
        // the first barrier (all fragment reads completed before the last
        // MFMAs).
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        typedef __attribute__((address_space(3))) u32x2 lds_u2_t;
        typedef __attribute__((address_space(3))) u32x4 lds_u4_t;
        constexpr uint32_t kStage = 256u * 128u;      // one C box image
        const TmapImpl cm = gemm_c_box_map(g.Cm.base, g.Cm.stride[0], (uint32_t)g.Cm.dim[0], (uint32_t)g.Cm.dim[1]);
        const tmap_t& cmap = reinterpret_cast<const tmap_t&>(cm);
        StoreGroups sg;
        store_groups_init(sg);
        wg_barrier();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (r == 1) {
                store_wait_read<0>(sg);               // this wave's stores no longer read either stage
                wg_barrier();                         // ... nor any other wave's
            }
            if constexpr (MI == 16) {
                static_assert(NQ == 1 && NJ % 4 == 0, "16 x 16 tiles, pairs of tiles per pass");
                // Before the swap lane group lg = lane / 16 holds columns
                // 4 lg .. 4 lg + 3 of tiles j0 and j0 + 1; the swap trades the
                // odd groups' pieces of j0 for the even groups' pieces of
                // j0 + 1, after which group lg holds columns 8 (lg >> 1) ..
                // + 7 of tile j0 + (lg & 1): four from the first result (the
                // even group's), four from the second (the odd group's).
                const uint32_t lg = lane >> 4;
                const uint32_t row = rloc;                       // + i * 16 below
                const uint32_t tsel = lg & 1u, half = lg >> 1;
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int jp = 0; jp < NJ / 4; ++jp) {
                        const int j0 = r * (NJ / 2) + 2 * jp;
                        uint32_t t0[2], t1[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            const f32x2 a = {acc[i][j0][2 * h], acc[i][j0][2 * h + 1]};
                            const f32x2 b = {acc[i][j0 + 1][2 * h], acc[i][j0 + 1][2 * h + 1]};
                            t0[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2));
                            t1[h] = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2));
                        }
                        const auto s0 = __builtin_amdgcn_permlane16_swap(t0[0], t1[0], false, false);
                        const auto s1 = __builtin_amdgcn_permlane16_swap(t0[1], t1[1], false, false);
                        const u32x4 v = {s0[0], s1[0], s0[1], s1[1]};
                        const uint32_t rr = row + (uint32_t)i * 16u;
                        const uint32_t col = (uint32_t)(j0 + (int)tsel) * 16u + half * 8u;  // tile-local column
                        const uint32_t chunk = rr * 8u + ((col & 63u) >> 3);
                        const uint32_t addr = lds0 + wn * kStage + (swz_chunk(chunk, kCSwizzle) << 4);
                        *(lds_u4_t*)(uintptr_t)addr = v;
                    }
            } else {
#pragma unroll
                for (int i = 0; i < NI; ++i)
#pragma unroll
                    for (int jj = 0; jj < NJ / 2; ++jj)
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            const int j = r * (NJ / 2) + jj;
                            const uint32_t row = rloc + (uint32_t)i * (uint32_t)MI;
                            const uint32_t col = cloc + (uint32_t)j * (uint32_t)MI + (uint32_t)q * 8u;
                            const uint32_t chunk = row * 8u + ((col & 63u) >> 3);
                            const uint32_t addr = lds0 + wn * kStage + (swz_chunk(chunk, kCSwizzle) << 4) +
                                                  (col & 7u) * 2u;
                            const f32x2 lo = {acc[i][j][4 * q], acc[i][j][4 * q + 1]};
                            const f32x2 hi = {acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            const u32x2 v = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
                            *(lds_u2_t*)(uintptr_t)addr = v;
                        }
            }
            wait_lgkm0();
            wg_barrier();                             // both box images complete
#pragma unroll
            for (uint32_t st = 0; st < 2; ++st) {
                const int32_t cb[5] = {(int32_t)(n0 + (2u * st + (uint32_t)r) * 64u), (int32_t)m0, 0, 0, 0};
                // non-temporal: C is not read back, and the write burst of
                // all workgroups finishing together drains faster without
                // displacing the operand panels from L2
                tile_store_async(cmap, cb, smem + st * kStage, wave, 4u, sg, true);
                store_commit(sg);
            }
        }
        return;
    }
    // C not 16-byte aligned: element stores, masked at the M / N edge.
    ATT_GLOBAL uint16_t* C = (ATT_GLOBAL uint16_t*)gptr(g.C);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint32_t row = m0 + rloc + (uint32_t)i * (uint32_t)MI;
                const uint32_t col = n0 + cloc + (uint32_t)j * (uint32_t)MI + (uint32_t)q * 8u;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (row < g.M && col + e < g.N)
                        C[(uint64_t)row * g.ldc + col + e] = f32_to_bf16_rne(acc[i][j][4 * q + e]);
            }
}

// EDGE = false: K a multiple of BK; copies use precomputed per-lane offsets,
// and in a partial tile the rows past M (N) re-read the last row (they only
// reach C rows / columns the epilogue clips).  EDGE = true: any K; boxes go
// through the general loader with zero fill at the edges.
// SWM: the operands' swizzle mode (64B / 128B, or their _K256 forms).
// MI: the MFMA shape, 32 (v_mfma_f32_32x32x16_bf16, 4 x 4 tiles per wave) or
// 16 (v_mfma_f32_16x16x32_bf16, 8 x 8 tiles).  Both run 1024 flop per clock
// per SIMD; the 16 x 16 form moves less accumulator and operand register
// data per flop, which under the chip's power limit holds a higher clock.
template <int BK, int S, bool EDGE, int SWM, int MI, bool CF32>
__global__ __launch_bounds__(kGemmThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_bf16(GemmArgs g) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr uint32_t ROWB = BK * 2;                 // bytes per LDS row (128 or 64)
    constexpr uint32_t BOX = kTM * ROWB;              // bytes per operand box
    // Ring layout: the S A-box slots first, then the S B-box slots, so that
    // slot s of either operand is s * BOX from slot 0 (with two slots that
    // offset fits a ds_read immediate).
    constexpr uint32_t BREG = (uint32_t)S * BOX;
    constexpr uint32_t GROUPS = BOX / 1024;           // 1 KiB DMA groups per box
    constexpr uint32_t GPW = GROUPS / 4;              // per wave and operand
    constexpr uint32_t SW = SWM & 3;                  // swizzled chunk bits (3 or 2)
    constexpr uint32_t KSH = (SWM & 4) ? 8u : 7u;     // key: 256- or 128-byte unit
    constexpr uint32_t CPR = ROWB / 16;               // chunks per row
    static_assert(MI == 32 || MI == 16, "MFMA shape");
    constexpr int NI = 128 / MI, NJ = 128 / MI;       // MFMA tiles per wave block (rows, columns)
    constexpr int NF = NI + NJ;                       // fragments per sub-step
    constexpr uint32_t KMI = MI == 32 ? 16u : 32u;    // K extent of one MFMA
    typedef std::conditional_t<MI == 32, f32x16, f32x4> AccT;

    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    uint32_t tm, tn;
    gemm_block_tile(g, tm, tn);
    // tile origin, taken to scalar registers once: the operand copies take
    // their bases from scalar arithmetic on these
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(tm * kTM), n0 = __builtin_amdgcn_readfirstlane(tn * kTN);
    const uint32_t nk = (g.K + BK - 1) / BK;
    constexpr bool interior = !EDGE;

    // Per-lane source offsets inside a box (same for every K step): lane l of
    // group j fills physical chunk p = j*64 + l with logical chunk swz(p).
    // Rows past M (or N) in a partial tile re-read the last row instead:
    // they only feed C rows (columns) the epilogue never stores.
    const uint32_t lds0 = lds_addr_of(smem);
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t rowsA = g.M - m0 < kTM ? g.M - m0 : kTM, rowsB = g.N - n0 < kTN ? g.N - n0 : kTN;
    uint32_t offA[GPW], offB[GPW];
#pragma unroll
    for (uint32_t j = 0; j < GPW; ++j) {
        const uint32_t p = (wave * GPW + j) * 64u + lane;
        const uint32_t q = swz_chunk(p, SWM);
        const uint32_t row = q / CPR, ch = q % CPR;
        offA[j] = (row < rowsA ? row : rowsA - 1u) * (uint32_t)g.A.stride[0] + ch * 16u;
        offB[j] = (row < rowsB ? row : rowsB - 1u) * (uint32_t)g.B.stride[0] + ch * 16u;
    }
    const uint64_t baseA = g.A.base + (uint64_t)m0 * g.A.stride[0];
    const uint64_t baseB = g.B.base + (uint64_t)n0 * g.B.stride[0];

    // Whole-tile issue (prologue, and every copy of the general loader).
    // Whole-tile copy through the general loader: zero fill past K (and
    // past M / N).
    auto issue_general = [&](uint32_t kt, uint32_t slot) {
        const int32_t ca[5] = {(int32_t)(kt * BK), (int32_t)m0, 0, 0, 0};
        const int32_t cb[5] = {(int32_t)(kt * BK), (int32_t)n0, 0, 0, 0};
        tile_load_issue(g.A, ca, smem + slot * BOX, wave, 4);
        tile_load_issue(g.B, cb, smem + BREG + slot * BOX, wave, 4);
    };
    // With two slots the fast loader also serves a K that is not a multiple
    // of BK: only the last, partial K tile goes through the general loader
    // (every wait of the two-slot ring is vmcnt(0), so its copy count does
    // not matter).
    const bool ktail = S == 2 && interior && g.K % BK != 0;
    auto issue = [&](uint32_t kt, uint32_t slot) {
        if constexpr (interior) {
            if (ktail && kt + 1u == nk) {
                issue_general(kt, slot);
                return;
            }
            const uint64_t ka = baseA + (uint64_t)kt * ROWB;
            const uint64_t kb = baseB + (uint64_t)kt * ROWB;
            const uint32_t la = lds0 + slot * BOX + wave_u * GPW * 1024u;
#pragma unroll
            for (uint32_t j = 0; j < GPW; ++j) dma16_sv(ka, offA[j], la + j * 1024u);
#pragma unroll
            for (uint32_t j = 0; j < GPW; ++j) dma16_sv(kb, offB[j], la + BREG + j * 1024u);
        } else {
            issue_general(kt, slot);
        }
    };

    AccT acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = AccT{};

    const uint32_t wm = wave >> 1, wn = wave & 1;
    const uint32_t khalf = lane / (uint32_t)MI;      // which 8-element K chunk of the sub-step
    constexpr uint32_t KK = BK / KMI;                 // MFMA sub-steps per stage (even)
    static_assert(KK % 2 == 0, "fragment buffer parity assumes an even sub-step count");

    // LDS address of fragment f (0..NI-1: A rows wm*128 + f*MI + l%MI; NI..:
    // B) for sub-step kk, relative to the ring slot: lane l reads logical chunk
    // (KMI/8)*kk + l/MI of its row at the physical chunk the swizzle gives.
    // Loop invariant, so each read is one add of the slot offset.
    uint32_t fad[KK][NF];
#pragma unroll
    for (uint32_t kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const uint32_t row = (f < NI ? wm : wn) * 128u + (uint32_t)(f % NI) * (uint32_t)MI + (lane % (uint32_t)MI);
            const uint32_t rb = row * ROWB;
            const uint32_t key = (rb >> KSH) & ((1u << SW) - 1u);
            fad[kk][f] = lds0 + (f < NI ? 0u : BREG) + rb + ((((KMI / 8u) * kk + khalf) ^ key) << 4);
        }
    bf16x8 fr[2][NF];                                 // [sub-step parity][A rows, B columns]
#pragma unroll
    for (int f = 0; f < NF; ++f) fr[1][f] = bf16x8{};
    if constexpr (MI == 16) {
        acc_fence(acc);                               // accumulator writes before the first MFMA
        asm volatile("s_nop 7" ::: "memory");
    }

    // One MFMA: B as the first operand, so each accumulator holds the
    // transposed tile (consecutive C columns per lane).  The 16 x 16 form is
    // inline asm with the accumulator tied to the destination: the builtin
    // lets the register allocator split them and copy accumulators around.
    auto mfma = [&](AccT& c, const bf16x8& b, const bf16x8& a) {
        if constexpr (MI == 32) {
            c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c, 0, 0, 0);
        } else {
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
        }
    };

    // One iteration runs from one workgroup barrier to the next:
    //   phase A: accumulator rows NI-AR.. of the previous tile's last
    //            sub-step (fragments already in registers), while reading
    //            sub-step 0 of tile t;
    //   phase B: sub-steps 0 .. KK-2 of tile t, reading the next sub-step;
    //   phase C: rows 0 .. NI-AR-1 of tile t's last sub-step; then wait for
    //            tile t+1's copies, and the barrier.
    // The slot of tile t-1 is free from the start of the iteration (every
    // wave passed the barrier after its last read of it), so tile t+S-1's
    // copies go there, spread evenly over the first SPAN MFMAs: the CU's
    // address unit takes 16 cycles per 1 KiB copy, and issued back to back
    // they would hold the waves' MFMA streams.  Every MFMA slot is pinned by
    // a scheduling barrier.  Iteration 0's phase A multiplies zero fragments
    // into zero accumulators (an exact no-op).
    constexpr int AR = MI == 16 ? 4 : 2;             // rows carried into the next iteration
    typedef GemmSched<NI, NJ, (int)KK, AR> Sch;
    constexpr int SLOTS = Sch::SLOTS;                // MFMAs per wave and iteration
    constexpr int NDMA = 2 * (int)GPW;               // copies per wave and tile
    constexpr int SPAN = S >= 3 ? SLOTS : (SLOTS * 3) / 8;
    // slot_c: the slot of tile t as a compile-time constant (two-slot ring:
    // the fragment reads carry it as an immediate offset, no per-read add),
    // or -1 to add slot_t at run time.
    auto iteration = [&](auto with_copies, auto slot_c, uint32_t t, uint32_t slot_t, uint32_t slot_fill,
                         uint32_t later, bool wait_next) {
        constexpr bool COPY = decltype(with_copies)::value;
        constexpr int SC = decltype(slot_c)::value;
        const uint32_t so = slot_t * BOX;
        const uint64_t ka = baseA + (uint64_t)(t + S - 1) * ROWB;
        const uint64_t kb = baseB + (uint64_t)(t + S - 1) * ROWB;
        const uint32_t la = lds0 + slot_fill * BOX + wave_u * GPW * 1024u;
        static_for<SLOTS>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int W = kGemmWaits<Sch>.w[m];
            if constexpr (W >= 0) {
                wait_lgkm<W>();
                __builtin_amdgcn_sched_barrier(0);
            }
            constexpr int i = Sch::mi(m), j = Sch::mj(m), buf = Sch::mbuf(m);
            mfma(acc[i][j], fr[buf][NI + j], fr[buf][i]);
            constexpr int f = Sch::rfrag(m);
            if constexpr (f >= 0) {
                if constexpr (SC >= 0)
                    fr[Sch::rbuf(m)][f] = __builtin_bit_cast(bf16x8, lds_read16_off<(uint32_t)SC * BOX>(fad[Sch::rkk(m)][f]));
                else
                    fr[Sch::rbuf(m)][f] = __builtin_bit_cast(bf16x8, lds_read16(fad[Sch::rkk(m)][f] + so));
            }
            if constexpr (COPY && interior) {
                static_for<NDMA>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
                    if constexpr ((c * SPAN) / NDMA == m) {
                        if constexpr (c < (int)GPW) dma16_sv(ka, offA[c], la + (uint32_t)c * 1024u);
                        else dma16_sv(kb, offB[c - GPW], la + BREG + (uint32_t)(c - GPW) * 1024u);
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if (wait_next) {
            if constexpr (interior) wait_stage<2 * GPW, S - 2>(later);
            else wait_vmcnt<0>();
            wait_lgkm0();
            wg_barrier();
        } else {
            // Last tile: rows NI-AR.. of its last sub-step, inside the
            // iteration (the accumulators still sit where its MFMAs left
            // them; the fragments come from asm reads the compiler believes
            // complete at issue, hence the wait before any MFMA), then let
            // every MFMA retire before code outside the loop touches them.
            wait_lgkm0();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < Sch::HALF; ++m)
                mfma(acc[NI - AR + m / NJ][m % NJ], fr[1][NI + m % NJ], fr[1][NI - AR + m / NJ]);
            if constexpr (MI == 16) {
                mfma_drain();
                acc_fence(acc);
            }
        }
    };

    // Prologue: tiles 0 .. S-2 in flight; wait for tile 0.
    const uint32_t pro = nk < (uint32_t)(S - 1) ? nk : (uint32_t)(S - 1);
    for (uint32_t s = 0; s < pro; ++s) issue(s, s);
    if constexpr (interior) wait_stage<2 * GPW, S - 2>(pro - 1);
    else wait_vmcnt<0>();
    wait_lgkm0();
    wg_barrier();

    // Iterations whose tile t+S-1 exists copy it into the slot of tile t-1.
    // The general loader issues whole tiles up front and drains before each
    // barrier.
    uint32_t slot_t = 0, slot_fill = S - 1;
    uint32_t t = 0;
    const uint32_t nfull = nk >= (uint32_t)S ? nk - (uint32_t)S + 1u : 0u;
    typedef std::integral_constant<bool, true> with_c;
    typedef std::integral_constant<bool, false> without_c;
    typedef std::integral_constant<int, -1> slot_rt;
    if constexpr (S == 2 && interior) {
        // tile t sits in slot t % 2: unroll by two so each body knows its slot
        const uint32_t nfast = ktail && nfull ? nfull - 1u : nfull;
        for (; t + 2 <= nfast; t += 2) {
            iteration(with_c{}, std::integral_constant<int, 0>{}, t, 0u, 1u, 0u, true);
            iteration(with_c{}, std::integral_constant<int, 1>{}, t + 1, 1u, 0u, 0u, true);
        }
        if (t < nfast) {
            iteration(with_c{}, std::integral_constant<int, 0>{}, t, 0u, 1u, 0u, true);
            ++t;
        }
        if (t < nfull) {
            // the partial last K tile, copied whole before this iteration
            issue_general(t + 1u, (t + 1u) & 1u);
            iteration(without_c{}, slot_rt{}, t, t & 1u, (t + 1u) & 1u, 0u, true);
            ++t;
        }
        slot_t = t & 1u;
        slot_fill = slot_t ^ 1u;
    } else {
        for (; t < nfull; ++t) {
            if constexpr (!interior) issue(t + S - 1, slot_fill);
            iteration(with_c{}, slot_rt{}, t, slot_t, slot_fill, (uint32_t)(S - 2), true);
            slot_fill = slot_t;
            slot_t = slot_t + 1 == (uint32_t)S ? 0u : slot_t + 1;
        }
    }
    // Tiles without copies: the last S-1 (with two slots, only the last).
    if constexpr (S > 2) {
        for (; t + 1 < nk; ++t) {
            // Tiles issued after tile t+1: t+2 .. nk-1.
            iteration(without_c{}, slot_rt{}, t, slot_t, slot_fill, nk - t - 2, true);
            slot_t = slot_t + 1 == (uint32_t)S ? 0u : slot_t + 1;
        }
    }
    iteration(without_c{}, slot_rt{}, t, slot_t, slot_fill, 0u, false);
    gemm_epilogue<MI, CF32>(g, acc, smem, lds0, wave_u, lane, m0, n0);
}

// Operand ring for 64-deep boxes with 16 x 16 x 32 MFMAs: five 32 KiB slots
// (the whole 160 KiB LDS) hold operand boxes, A's box of K-step k as unit 2k
// and B's as unit 2k+1, unit u in slot u % 5.  Iteration t reads A_t and
// B_t; over its first third it copies B_{t+1}, over the rest A_{t+2}, into
// the two slots that A_{t-1} and B_{t-1} left.  A is thus three deep
// and B two deep: the A copies get a whole extra iteration to land, and the
// copies spread over the whole iteration (the CU's address unit takes 16
// cycles per 1 KiB copy, half of the iteration's MFMA time).  The loop is
// unrolled by five, so every body knows its slots.  Fragment reads need one
// base address per (operand, sub-step, 64 KiB window): the 128-byte swizzle
// key of a fragment row depends only on the lane (fragments start on 16-row
// boundaries), so fragment f of a slot sits f * 2048 bytes further and the
// slot offset within the window rides in the ds_read immediate too.  K a
// multiple of 64; partial M / N tiles clamp their rows as k_gemm_bf16 does.
template <int SWM, bool CF32>
__global__ __launch_bounds__(kGemmThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_bf16_ring5(GemmArgs g) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr uint32_t RING = 5;
    constexpr uint32_t ROWB = 128;                    // 64 bf16 per LDS row
    constexpr uint32_t UBOX = kTM * ROWB;             // 32 KiB: one operand box
    constexpr uint32_t GPW = UBOX / 1024 / 4;         // copies per wave and unit
    constexpr uint32_t SW = SWM & 3;
    constexpr uint32_t KSH = (SWM & 4) ? 8u : 7u;
    constexpr uint32_t CPR = ROWB / 16;
    constexpr int MI = 16, NI = 8, NJ = 8, NF = NI + NJ;
    constexpr int NDMA = (int)GPW;
    typedef f32x4 AccT;
    static_assert(SW == 3, "128-byte rows take the 128-byte swizzle");

    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    uint32_t tm, tn;
    gemm_block_tile(g, tm, tn);
    // tile origin, taken to scalar registers once: the operand copies take
    // their bases from scalar arithmetic on these
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(tm * kTM), n0 = __builtin_amdgcn_readfirstlane(tn * kTN);
    const uint32_t NT = g.K / 64u;                   // K-steps
    const uint32_t lds0 = lds_addr_of(smem);
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);

    // rows past M (N) of a partial tile re-read the last row (see k_gemm_bf16)
    const uint32_t rowsA = g.M - m0 < kTM ? g.M - m0 : kTM, rowsB = g.N - n0 < kTN ? g.N - n0 : kTN;
    uint32_t offA[GPW], offB[GPW];
#pragma unroll
    for (uint32_t j = 0; j < GPW; ++j) {
        const uint32_t p = (wave * GPW + j) * 64u + lane;
        const uint32_t q = swz_chunk(p, SWM);
        const uint32_t row = q / CPR, ch = q % CPR;
        offA[j] = (row < rowsA ? row : rowsA - 1u) * (uint32_t)g.A.stride[0] + ch * 16u;
        offB[j] = (row < rowsB ? row : rowsB - 1u) * (uint32_t)g.B.stride[0] + ch * 16u;
    }
    const uint64_t baseA = g.A.base + (uint64_t)m0 * g.A.stride[0];
    const uint64_t baseB = g.B.base + (uint64_t)n0 * g.B.stride[0];
    // K-steps past the last re-read the last one instead (no branch in the
    // MFMA stream): they land in slots no later iteration reads, and the
    // last iteration drains them before the epilogue reuses the LDS.
    const uint32_t klast = NT - 1u;
    auto clamp_k = [&](uint32_t k) { return k < klast ? k : klast; };
    // Copy c (0..NDMA-1) of operand OP's box of K-step k into slot `slot`.
    auto copy_unit = [&](auto opc, uint32_t k, uint32_t slot, int c) {
        constexpr int OP = decltype(opc)::value;
        const uint32_t la = lds0 + slot * UBOX + wave_u * GPW * 1024u + (uint32_t)c * 1024u;
        if constexpr (OP == 0) dma16_sv_ring(baseA + (uint64_t)k * ROWB, offA[c], la);
        else dma16_sv_ring(baseB + (uint64_t)k * ROWB, offB[c], la);
    };
    typedef std::integral_constant<int, 0> opA;
    typedef std::integral_constant<int, 1> opB;

    // Prologue: A_0, B_0, A_1 into slots 0, 1, 2, issued first so that the
    // register set-up below overlaps their latency.
#pragma unroll
    for (int c = 0; c < NDMA; ++c) copy_unit(opA{}, 0u, 0u, c);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) copy_unit(opB{}, 0u, 1u, c);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) copy_unit(opA{}, clamp_k(1u), 2u, c);
    __builtin_amdgcn_sched_barrier(0);

    AccT acc[NI][NJ];
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = AccT{};
    const uint32_t wm = wave >> 1, wn = wave & 1;
    // Lane l reads row l % 16 of each fragment and logical chunk 4kk + l/16
    // of it; base address per operand, sub-step kk and 64 KiB window w.
    uint32_t fa[2][3], fb[2][3];
#pragma unroll
    for (uint32_t kk = 0; kk < 2; ++kk) {
        const uint32_t ra = (wm * 128u + (lane & 15u)) * ROWB, rbb = (wn * 128u + (lane & 15u)) * ROWB;
        const uint32_t ka = (ra >> KSH) & 7u, kb = (rbb >> KSH) & 7u;
        const uint32_t ch = 4u * kk + (lane >> 4);
#pragma unroll
        for (uint32_t w = 0; w < 3; ++w) {
            fa[kk][w] = lds0 + w * 65536u + ra + ((ch ^ ka) << 4);
            fb[kk][w] = lds0 + w * 65536u + rbb + ((ch ^ kb) << 4);
        }
    }
    bf16x8 fr[2][NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) fr[1][f] = bf16x8{};
    acc_fence(acc);
    asm volatile("s_nop 7" ::: "memory");
    auto mfma = [&](AccT& c, const bf16x8& b, const bf16x8& a) {
        asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(b), "v"(a));
    };

    // wait for A_0 and B_0
    wait_vmcnt<NDMA>();
    wait_lgkm0();
    wg_barrier();

    typedef GemmSched<NI, NJ, 2, 4> Sch;
    constexpr int SLOTS = Sch::SLOTS;
    constexpr int BSP = 5, AST = 48, ASP = 10;       // copy placement (MFMA slots)
    static_assert(BSP * NDMA <= AST && AST + ASP * (NDMA - 1) < SLOTS, "copy placement");
    auto body = [&](auto rc, uint32_t t) {
        constexpr int R = decltype(rc)::value;        // t % 5
        constexpr uint32_t SA = (2u * R) % RING, SB = (2u * R + 1u) % RING;
        constexpr uint32_t F1 = (2u * R + 3u) % RING, F2 = (2u * R + 4u) % RING;
        const uint32_t kb1 = clamp_k(t + 1u), ka2 = clamp_k(t + 2u);
        static_for<SLOTS>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int W = kGemmWaits<Sch>.w[m];
            if constexpr (W >= 0) {
                wait_lgkm<W>();
                __builtin_amdgcn_sched_barrier(0);
            }
            constexpr int i = Sch::mi(m), j = Sch::mj(m), buf = Sch::mbuf(m);
            mfma(acc[i][j], fr[buf][NI + j], fr[buf][i]);
            constexpr int f = Sch::rfrag(m);
            if constexpr (f >= 0) {
                constexpr int kk = Sch::rkk(m);
                constexpr uint32_t slot = f < NI ? SA : SB;
                constexpr uint32_t imm = (slot & 1u) * UBOX + (uint32_t)(f % NI) * 16u * ROWB;
                const uint32_t base = f < NI ? fa[kk][slot >> 1] : fb[kk][slot >> 1];
                fr[Sch::rbuf(m)][f] = __builtin_bit_cast(bf16x8, lds_read16_off<imm>(base));
            }
            // B_{t+1} early (it must land by the end of this iteration), one
            // copy every BSP slots; A_{t+2} over the rest, every ASP slots
            if constexpr (m < BSP * NDMA && m % BSP == 0) copy_unit(opB{}, kb1, F1, m / BSP);
            if constexpr (m >= AST && (m - AST) % ASP == 0 && (m - AST) / ASP < NDMA)
                copy_unit(opA{}, ka2, F2, (m - AST) / ASP);
            __builtin_amdgcn_sched_barrier(0);
        });
        // A_{t+1} and B_{t+1} have landed once at most A_{t+2}'s copies
        // (issued last) are in flight
        wait_vmcnt<NDMA>();
        wait_lgkm0();
        wg_barrier();
        // (the layout hints keep the common path free of taken branches:
        // 0.5 % on the 8192^3 GEMM, timed interleaved with the plain form)
        if (__builtin_expect(t + 1u == NT, 0)) {
            // Rows 4.. of the last sub-step, inside the body, where the
            // accumulators still sit; then drain (the clamped copies too)
            // before code outside the loop touches accumulators or LDS.
            wait_vmcnt<0>();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int m = 0; m < Sch::HALF; ++m) mfma(acc[4 + m / NJ][m % NJ], fr[1][NI + m % NJ], fr[1][4 + m / NJ]);
            mfma_drain();
            acc_fence(acc);
        }
    };
    for (uint32_t t = 0; t < NT; t += 5u) {
        body(std::integral_constant<int, 0>{}, t);
        if (__builtin_expect(t + 1u < NT, 1)) body(std::integral_constant<int, 1>{}, t + 1u);
        if (__builtin_expect(t + 2u < NT, 1)) body(std::integral_constant<int, 2>{}, t + 2u);
        if (__builtin_expect(t + 3u < NT, 1)) body(std::integral_constant<int, 3>{}, t + 3u);
        if (__builtin_expect(t + 4u < NT, 1)) body(std::integral_constant<int, 4>{}, t + 4u);
    }
    gemm_epilogue<MI, CF32>(g, acc, smem, lds0, wave_u, lane, m0, n0);
}

template <int SWM, bool CF32 = false>
static tmap_status launch_gemm_ring5(const GemmArgs& g, hipStream_t st) {
    constexpr uint32_t lds = 5u * kTM * 128u;        // 160 KiB: the ring (the C image reuses it)
    uint32_t limit = 0;
    tmap_status s = device_lds_limit(&limit);
    if (s) return s;
    if (lds > limit) return TMAP_ERR_UNSUPPORTED;
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_bf16_ring5<SWM, CF32>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)lds);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    hipLaunchKernelGGL((k_gemm_bf16_ring5<SWM, CF32>), dim3(g.tiles_m * g.tiles_n), dim3(kGemmThreads), lds, st, g);
    return check_launch("gemm_bf16");
}

template <int BK, int S, bool EDGE, int SWM, int MI, bool CF32 = false>
static tmap_status launch_gemm_t(const GemmArgs& g, hipStream_t st) {
    // The ring, or the 128 KiB C staging image if that is larger.
    constexpr uint32_t ring = (uint32_t)S * 2u * kTM * BK * 2u;
    constexpr uint32_t lds = ring > 4u * 32768u ? ring : 4u * 32768u;
    uint32_t limit = 0;
    tmap_status s = device_lds_limit(&limit);
    if (s) return s;
    if (lds > limit) return TMAP_ERR_UNSUPPORTED;
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_bf16<BK, S, EDGE, SWM, MI, CF32>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    hipLaunchKernelGGL((k_gemm_bf16<BK, S, EDGE, SWM, MI, CF32>), dim3(g.tiles_m * g.tiles_n), dim3(kGemmThreads), lds, st,
                       g);
    return check_launch("gemm_bf16");
}

template <int BK, int S, int MI>
static tmap_status launch_gemm_mi(const GemmArgs& g, uint32_t swm, hipStream_t st) {
    // K a multiple of BK, or two slots: the fast loader (partial M / N tiles
    // clamp their rows; with two slots a partial last K tile goes through the
    // general loader); otherwise every copy goes through the general loader.
    constexpr int BASE = BK == 64 ? TMAP_SWIZZLE_128B : TMAP_SWIZZLE_64B;
    if constexpr (S == 2) {
        if (swm & 4u) return launch_gemm_t<BK, S, false, BASE | 4, MI>(g, st);
        return launch_gemm_t<BK, S, false, BASE, MI>(g, st);
    } else {
        const bool even = g.K % BK == 0;
        if (swm & 4u)
            return even ? launch_gemm_t<BK, S, false, BASE | 4, MI>(g, st) : launch_gemm_t<BK, S, true, BASE | 4, MI>(g, st);
        return even ? launch_gemm_t<BK, S, false, BASE, MI>(g, st) : launch_gemm_t<BK, S, true, BASE, MI>(g, st);
    }
}

// The 16 x 16 x 32 form needs an even number of 32-deep sub-steps per stage,
// so it serves the 64-deep K step; the 32-deep step always uses 32 x 32 x 16.
template <int BK, int S>
static tmap_status launch_gemm(const GemmArgs& g, uint32_t swm, uint32_t mfma, hipStream_t st) {
    if constexpr (BK == 64) {
        if (mfma != 32) return launch_gemm_mi<BK, S, 16>(g, swm, st);
    } else {
        if (mfma == 16) return TMAP_ERR_UNSUPPORTED;
    }
    return launch_gemm_mi<BK, S, 32>(g, swm, st);
}

static tmap_status check_operand(const TmapImpl& t, uint32_t rows, uint32_t K, uint32_t* bk, uint32_t* swm) {
    if (t.dtype != TMAP_BF16 || t.rank != 2 || t.oob != TMAP_OOB_ZERO) return TMAP_ERR_UNSUPPORTED;
    if ((uint64_t)t.dim[0] != K || (uint64_t)t.dim[1] != rows) return TMAP_ERR_UNSUPPORTED;
    if (t.es[0] != 1 || t.es[1] != 1 || (uint32_t)t.box_m1[1] + 1u != (uint32_t)kTM) return TMAP_ERR_UNSUPPORTED;
    const uint32_t b0 = (uint32_t)t.box_m1[0] + 1u;
    const uint32_t span = t.swizzle & 3u;
    if (!((b0 == 64 && span == TMAP_SWIZZLE_128B) || (b0 == 32 && span == TMAP_SWIZZLE_64B)))
        return TMAP_ERR_UNSUPPORTED;
    *swm = t.swizzle;
    if (t.stride[0] >= (1ull << 31) / kTM) return TMAP_ERR_UNSUPPORTED;   // 32-bit in-box offsets
    *bk = b0;
    return TMAP_OK;
}

}  // namespace att

using namespace att;

static tmap_status gemm_run(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N, uint32_t K,
                            uint32_t ldc, uint32_t stages, uint32_t group_m, uint32_t xcd, uint32_t mfma,
                            bool c_f32, void* stream) {
    if (mfma != 0 && mfma != 16 && mfma != 32) return TMAP_ERR_UNSUPPORTED;
    if (!A || !B || !d_C) return TMAP_ERR_NULL;
    if (M == 0 || N == 0) return TMAP_OK;
    const uintptr_t calign = c_f32 ? 3u : 1u;
    if (K == 0 || ldc < N || (reinterpret_cast<uintptr_t>(d_C) & calign)) return TMAP_ERR_UNSUPPORTED;
    GemmArgs g;
    g.A = load_map(A);
    g.B = load_map(B);
    uint32_t bka = 0, bkb = 0, swa = 0, swb = 0;
    tmap_status s = check_operand(g.A, M, K, &bka, &swa);
    if (s) return s;
    s = check_operand(g.B, N, K, &bkb, &swb);
    if (s) return s;
    if (bka != bkb || swa != swb) return TMAP_ERR_UNSUPPORTED;
    g.C = reinterpret_cast<uint64_t>(d_C);
    g.M = M; g.N = N; g.K = K; g.ldc = ldc;
    g.tiles_m = (M + kTM - 1) / kTM;
    g.tiles_n = (N + kTN - 1) / kTN;
    g.group_m = group_m ? group_m : 8u;
    const uint32_t G = g.tiles_m * g.tiles_n;
    g.xcd = (xcd && G % 8u == 0) ? 1u : 0u;
    g.blk_m = g.blk_n = 0;
    if (xcd == 2 && g.tiles_m % 4u == 0 && g.tiles_n % 2u == 0) {
        g.xcd = 2;                     // 4 x 2 arrangement of XCD blocks
        g.blk_m = g.tiles_m / 4u;
        g.blk_n = g.tiles_n / 2u;
        if (g.group_m > g.blk_m || g.blk_m % g.group_m) g.group_m = g.blk_m;
    }
    g.c_staged = 0;
    if (!c_f32 && (reinterpret_cast<uintptr_t>(d_C) & 15u) == 0 && ldc % 8u == 0) {
        tmap_t cm;
        const uint64_t cdim[2] = {N, M};
        const uint64_t cstride[1] = {(uint64_t)ldc * 2u};
        const uint32_t cbox[2] = {64u, (uint32_t)kTM};
        if (tmap_encode(&cm, TMAP_BF16, 2, d_C, cdim, cstride, cbox, nullptr, (tmap_swizzle)kCSwizzle,
                        TMAP_OOB_ZERO) == TMAP_OK) {
            g.Cm = load_map(&cm);
            const TmapImpl want = gemm_c_box_map(g.Cm.base, g.Cm.stride[0], N, M);
            g.c_staged = std::memcmp(&want, &g.Cm, sizeof(want)) == 0 ? 1u : 0u;
        }
    }
    hipStream_t st = as_stream(stream);
    if (c_f32) {
        // fp32 C: the 64-deep K step with 16 x 16 x 32 MFMAs
        if (bka != 64 || mfma == 32) return TMAP_ERR_UNSUPPORTED;
        if (stages == 2) {
            if (swa & 4u) return launch_gemm_t<64, 2, false, TMAP_SWIZZLE_128B_K256, 16, true>(g, st);
            return launch_gemm_t<64, 2, false, TMAP_SWIZZLE_128B, 16, true>(g, st);
        }
        if (stages == 3) {
            if (K % 64u) return TMAP_ERR_UNSUPPORTED;
            if (swa & 4u) return launch_gemm_ring5<TMAP_SWIZZLE_128B_K256, true>(g, st);
            return launch_gemm_ring5<TMAP_SWIZZLE_128B, true>(g, st);
        }
        return TMAP_ERR_UNSUPPORTED;
    }
    if (bka == 64) {
        if (stages == 2) return launch_gemm<64, 2>(g, swa, mfma, st);
        if (stages == 3) {
            // A three deep, B two deep in five operand slots: K a multiple
            // of 64, 16 x 16 x 32 MFMAs
            if (mfma == 32 || K % 64u) return TMAP_ERR_UNSUPPORTED;
            if (swa & 4u) return launch_gemm_ring5<TMAP_SWIZZLE_128B_K256>(g, st);
            return launch_gemm_ring5<TMAP_SWIZZLE_128B>(g, st);
        }
        return TMAP_ERR_UNSUPPORTED;
    }
    switch (stages) {
    case 2: return launch_gemm<32, 2>(g, swa, mfma, st);
    case 3: return launch_gemm<32, 3>(g, swa, mfma, st);
    case 4: return launch_gemm<32, 4>(g, swa, mfma, st);
    case 5: return launch_gemm<32, 5>(g, swa, mfma, st);
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

extern "C" tmap_status gemm_bf16_ex(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                                    uint32_t K, uint32_t ldc, uint32_t stages, uint32_t group_m, uint32_t xcd,
                                    uint32_t mfma, void* stream) {
    return gemm_run(A, B, d_C, M, N, K, ldc, stages, group_m, xcd, mfma, false, stream);
}

extern "C" tmap_status gemm_bf16(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N, uint32_t K,
                                 uint32_t ldc, uint32_t stages, void* stream) {
    return gemm_run(A, B, d_C, M, N, K, ldc, stages, 0u, 1u, 0u, false, stream);
}

extern "C" tmap_status gemm_bf16_f32(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                                     uint32_t K, uint32_t ldc, uint32_t stages, void* stream) {
    return gemm_run(A, B, d_C, M, N, K, ldc, stages, 0u, 1u, 0u, true, stream);
}
