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

#include "host_util.hpp"
#include "tile_device.hpp"
#include "tmap.h"

namespace att {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
};

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

// EDGE = false: every box is inside the tensors (M, N multiples of 256, K a
// multiple of BK), copies use precomputed per-lane offsets.  EDGE = true: any
// shape; boxes go through the general loader with zero fill at the edges.
// SWM: the operands' swizzle mode (64B / 128B, or their _K256 forms).
template <int BK, int S, bool EDGE, int SWM>
__global__ __launch_bounds__(kGemmThreads, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_bf16(GemmArgs g) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
    constexpr uint32_t ROWB = BK * 2;                 // bytes per LDS row (128 or 64)
    constexpr uint32_t BOX = kTM * ROWB;              // bytes per operand box
    constexpr uint32_t STAGE = 2 * BOX;
    constexpr uint32_t GROUPS = BOX / 1024;           // 1 KiB DMA groups per box
    constexpr uint32_t GPW = GROUPS / 4;              // per wave and operand
    constexpr uint32_t SW = SWM & 3;                  // swizzled chunk bits (3 or 2)
    constexpr uint32_t KSH = (SWM & 4) ? 8u : 7u;     // key: 256- or 128-byte unit
    constexpr uint32_t CPR = ROWB / 16;               // chunks per row

    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t lane = lane_id();
    const uint32_t G = gridDim.x;
    uint32_t tm, tn;
    if (g.xcd == 2) {
        // Workgroups are dispatched round-robin over the 8 XCDs: XCD x owns a
        // blk_m x blk_n block of C tiles (blocks 2 wide in n), walked in
        // groups of group_m tile rows, so its L2 serves blk_m A panels and
        // blk_n B panels instead of whole tile rows.
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
    const uint32_t m0 = tm * kTM, n0 = tn * kTN;
    const uint32_t nk = (g.K + BK - 1) / BK;
    constexpr bool interior = !EDGE;

    // Per-lane source offsets inside a box (same for every K step): lane l of
    // group j fills physical chunk p = j*64 + l with logical chunk swz(p).
    const uint32_t lds0 = lds_addr_of(smem);
    const uint32_t wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t offA[GPW], offB[GPW];
#pragma unroll
    for (uint32_t j = 0; j < GPW; ++j) {
        const uint32_t p = (wave * GPW + j) * 64u + lane;
        const uint32_t q = swz_chunk(p, SWM);
        const uint32_t row = q / CPR, ch = q % CPR;
        offA[j] = row * (uint32_t)g.A.stride[0] + ch * 16u;
        offB[j] = row * (uint32_t)g.B.stride[0] + ch * 16u;
    }
    const uint64_t baseA = g.A.base + (uint64_t)m0 * g.A.stride[0];
    const uint64_t baseB = g.B.base + (uint64_t)n0 * g.B.stride[0];

    auto issue = [&](uint32_t kt) {
        uint8_t* st = smem + (kt % S) * STAGE;
        if constexpr (interior) {
            const uint64_t ka = baseA + (uint64_t)kt * ROWB;
            const uint64_t kb = baseB + (uint64_t)kt * ROWB;
            const uint32_t la = lds0 + (kt % S) * STAGE + wave_u * GPW * 1024u;
#pragma unroll
            for (uint32_t j = 0; j < GPW; ++j) dma16_sv(ka, offA[j], la + j * 1024u);
#pragma unroll
            for (uint32_t j = 0; j < GPW; ++j) dma16_sv(kb, offB[j], la + BOX + j * 1024u);
        } else {
            const int32_t ca[5] = {(int32_t)(kt * BK), (int32_t)m0, 0, 0, 0};
            const int32_t cb[5] = {(int32_t)(kt * BK), (int32_t)n0, 0, 0, 0};
            tile_load_issue(g.A, ca, st, wave, 4);
            tile_load_issue(g.B, cb, st + BOX, wave, 4);
        }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const uint32_t wm = wave >> 1, wn = wave & 1;
    // LDS byte offset of this lane's operand row inside a box, and its XOR key.
    const uint32_t rowA0 = wm * 128u + (lane & 31u);
    const uint32_t rowB0 = wn * 128u + (lane & 31u);
    const uint32_t khalf = lane >> 5;

    constexpr uint32_t KK = BK / 16;                  // MFMA sub-steps per stage
    // Fragment reads for sub-step kk of the tile held in ring slot `slot`,
    // addressed with 32-bit LDS offsets (row base and XOR key per fragment
    // row are loop invariants).
    typedef __attribute__((address_space(3))) const bf16x8 lds_frag_t;
    uint32_t rbA[4], kyA[4], rbB[4], kyB[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ra = rowA0 + i * 32u, rb = rowB0 + i * 32u;
        rbA[i] = lds0 + ra * ROWB;
        kyA[i] = ((ra * ROWB) >> KSH) & ((1u << SW) - 1u);
        rbB[i] = lds0 + BOX + rb * ROWB;
        kyB[i] = ((rb * ROWB) >> KSH) & ((1u << SW) - 1u);
    }
    auto load_frags = [&](uint32_t slot, uint32_t kk, bf16x8 (&a)[4], bf16x8 (&b)[4]) {
        const uint32_t so = slot * STAGE;
        const uint32_t lc = 2u * kk + khalf;          // logical 16-byte chunk of the row
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = *(lds_frag_t*)(uintptr_t)(rbA[i] + so + ((lc ^ kyA[i]) << 4));
#pragma unroll
        for (int j = 0; j < 4; ++j)
            b[j] = *(lds_frag_t*)(uintptr_t)(rbB[j] + so + ((lc ^ kyB[j]) << 4));
    };

    // Prologue: all S ring slots in flight; wait for the first.
#pragma unroll
    for (int s = 0; s < S; ++s)
        if ((uint32_t)s < nk) issue(s);
    if constexpr (interior) wait_stage<2 * GPW, S - 1>(nk - 1 < (uint32_t)(S - 1) ? nk - 1 : (uint32_t)(S - 1));
    else wait_vmcnt<0>();
    wait_lgkm0();
    wg_barrier();

    // Main loop.  Fragment registers are double-buffered: the reads for
    // sub-step kk+1 are interleaved with the 16 MFMAs of kk (one read per two
    // MFMAs; scheduling-group barriers pin the pattern).  During the last
    // sub-step of a tile the wave has issued every read of that slot: after
    // the first half of its MFMAs it waits for the next tile's copies, joins
    // the workgroup barrier (after which no wave reads the slot any more),
    // refills the slot with tile kt+S, and reads the next tile's first
    // fragments between the remaining MFMAs.
    bf16x8 fa[2][4], fb[2][4];
    load_frags(0, 0, fa[0], fb[0]);
    // MFMAs for accumulator rows [i0, i0 + ni) of sub-step buffer `cur`
    // (constant bounds after unrolling, so acc stays in registers).
    auto mfma_rows = [&](uint32_t cur, int i0, int ni) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i < i0 || i >= i0 + ni) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
        }
    };
    // Accumulator updates stay outside runtime branches (only the copy issue
    // is conditional), so the 256 accumulator registers never meet a join.
    for (uint32_t kt = 0; kt < nk; ++kt) {
        const uint32_t s = kt % S;
#pragma unroll
        for (uint32_t kk = 0; kk < KK; ++kk) {
            const uint32_t cur = kk & 1u;
            if constexpr (true) {
                if (kk + 1 < KK) {
                    load_frags(s, kk + 1, fa[cur ^ 1u], fb[cur ^ 1u]);
                    mfma_rows(cur, 0, 4);
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    continue;
                }
            }
            // last sub-step of the tile
            mfma_rows(cur, 0, 2);
            __builtin_amdgcn_sched_barrier(0);
            const uint32_t rem = nk - 1 - kt;             // tiles after this one
            const uint32_t later = rem == 0 ? 0u : (rem - 1 < (uint32_t)(S - 2) ? rem - 1 : (uint32_t)(S - 2));
            if constexpr (interior) wait_stage<2 * GPW, S - 2>(later);
            else wait_vmcnt<0>();
            wait_lgkm0();
            wg_barrier();
            if (kt + S < nk) issue(kt + S);
            __builtin_amdgcn_sched_barrier(0);
            load_frags((s + 1) % S, 0, fa[cur ^ 1u], fb[cur ^ 1u]);   // unused after the last tile
            mfma_rows(cur, 2, 2);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // Epilogue: fp32 -> bf16 (round to nearest even), masked at the M / N edge.
    // Accumulator register r of lane l holds row (r/4)*8 + (l/32)*4 + r%4 and
    // column l%32 of its 32 x 32 tile.
    ATT_GLOBAL uint16_t* C = (ATT_GLOBAL uint16_t*)gptr(g.C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t col = n0 + wn * 128u + j * 32u + (lane & 31u);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const uint32_t row = m0 + wm * 128u + i * 32u + (r / 4) * 8u + khalf * 4u + (r % 4);
                if (row < g.M && col < g.N) C[(uint64_t)row * g.ldc + col] = f32_to_bf16_rne(acc[i][j][r]);
            }
        }
}

template <int BK, int S, bool EDGE, int SWM>
static tmap_status launch_gemm_t(const GemmArgs& g, hipStream_t st) {
    constexpr uint32_t lds = (uint32_t)S * 2u * kTM * BK * 2u;
    uint32_t limit = 0;
    tmap_status s = device_lds_limit(&limit);
    if (s) return s;
    if (lds > limit) return TMAP_ERR_UNSUPPORTED;
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_bf16<BK, S, EDGE, SWM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return hip_fail(e, "hipFuncSetAttribute");
    hipLaunchKernelGGL((k_gemm_bf16<BK, S, EDGE, SWM>), dim3(g.tiles_m * g.tiles_n), dim3(kGemmThreads), lds, st, g);
    return check_launch("gemm_bf16");
}

template <int BK, int S>
static tmap_status launch_gemm(const GemmArgs& g, uint32_t swm, hipStream_t st) {
    const bool even = g.M % kTM == 0 && g.N % kTN == 0 && g.K % BK == 0;
    constexpr int BASE = BK == 64 ? TMAP_SWIZZLE_128B : TMAP_SWIZZLE_64B;
    if (swm & 4u)
        return even ? launch_gemm_t<BK, S, false, BASE | 4>(g, st) : launch_gemm_t<BK, S, true, BASE | 4>(g, st);
    return even ? launch_gemm_t<BK, S, false, BASE>(g, st) : launch_gemm_t<BK, S, true, BASE>(g, st);
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

extern "C" tmap_status gemm_bf16_ex(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                                    uint32_t K, uint32_t ldc, uint32_t stages, uint32_t group_m, uint32_t xcd,
                                    void* stream) {
    if (!A || !B || !d_C) return TMAP_ERR_NULL;
    if (M == 0 || N == 0) return TMAP_OK;
    if (K == 0 || ldc < N || (reinterpret_cast<uintptr_t>(d_C) & 1u)) return TMAP_ERR_UNSUPPORTED;
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
    hipStream_t st = as_stream(stream);
    if (bka == 64) {
        if (stages == 2) return launch_gemm<64, 2>(g, swa, st);
        return TMAP_ERR_UNSUPPORTED;
    }
    switch (stages) {
    case 2: return launch_gemm<32, 2>(g, swa, st);
    case 3: return launch_gemm<32, 3>(g, swa, st);
    case 4: return launch_gemm<32, 4>(g, swa, st);
    case 5: return launch_gemm<32, 5>(g, swa, st);
    default: return TMAP_ERR_UNSUPPORTED;
    }
}

extern "C" tmap_status gemm_bf16(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N, uint32_t K,
                                 uint32_t ldc, uint32_t stages, void* stream) {
    return gemm_bf16_ex(A, B, d_C, M, N, K, ldc, stages, 0u, 1u, stream);
}
