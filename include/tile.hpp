/*
 * tile.hpp -- device API of the MI355X (gfx950) tile mover: the operations of
 * tmap.h issued from inside a HIP kernel, on LDS the kernel owns, with a map
 * the host encoded by tmap_encode / tmap_encode_im2col and passed to the
 * kernel by value (as a kernel argument, so every field lands in scalar
 * registers; [H200] section 05 passes the descriptor as a const kernel
 * parameter, [HPC] "Tensor descriptor" keeps it in constant memory).
 *
 * Compile with hipcc --offload-arch=gfx950 -I<this directory>; add
 * -munsafe-fp-atomics for the hardware float atomics in the reductions (the
 * library is built so; without it float adds become compare-and-swap
 * loops).  The library's own batch kernels (tile_load, tile_store,
 * tile_reduce, tile_load_im2col, txbar_selftest) are written against these
 * calls.
 *
 * The pages' device operation is one thread describing a whole box to a copy
 * engine that reports its bytes to an LDS barrier ([MLC] "one thread
 * describes the whole tile", "waiting for a TMA load"; [HPC] single-tile load
 * takes LDS destination, map, coordinates and barrier).  gfx950 has no copy
 * engine: the waves of the workgroup are the address generators.  Each wave
 * issues its share of the box (64 chunks of 16 bytes per wave instruction),
 * and after its own copies have landed reports the bytes it wrote to the
 * byte-counted barrier, so a consumer waits on the barrier's phase exactly as
 * on the pages:
 *
 *     __shared__ att::TxBar bar;            // 8-byte aligned LDS
 *     extern __shared__ __attribute__((aligned(1024))) uint8_t img[];
 *     if (threadIdx.x == 0) {
 *         att::txbar_init(&bar, 1);
 *         att::txbar_arrive_expect_tx(&bar, att::tile_box_bytes(map));
 *     }
 *     __syncthreads();
 *     const uint32_t w = threadIdx.x / 64, nw = blockDim.x / 64;
 *     const uint32_t bytes = att::tile_load_async(map, c, img, w, nw);
 *     ...                                   // independent work
 *     att::tile_load_arrive(&bar, bytes);   // this wave's copies landed
 *     att::txbar_wait(&bar, 0);             // the whole box landed
 *
 * Conventions
 *   - Coordinates are box origins in elements, innermost first, five entries
 *     (entries past the map's rank are ignored).  Any int32 is legal: elements
 *     outside the tensor are filled on load (zero or the dtype's quiet NaN, as
 *     encoded) and skipped on store / reduce.  Nothing is checked on the
 *     device; maps are validated once, by the host encoder.
 *   - An LDS image is the box's elements densely packed, innermost fastest,
 *     extents ceil(box_i / elementStride_i), with 16-byte chunks XOR-permuted
 *     by the map's swizzle relative to the image start.  It must be 16-byte
 *     aligned; 1024-byte alignment makes the swizzle's bank pattern the one
 *     the pages describe.  The image is tile_box_bytes(map) bytes.
 *   - `wave` / `nwaves`: every wave in [0, nwaves) of the workgroup calls the
 *     operation with its own index and the same arguments; the box's 64-chunk
 *     groups go round-robin to the waves.  One wave alone uses wave = 0,
 *     nwaves = 1.  Calls are wave-uniform: all 64 lanes of a wave take part.
 *   - Tiled maps go to the tile_* calls, im2col maps to tile_load_im2col_async
 *     only; passing the other kind is undefined.
 *   - Nothing here allocates, blocks without bound or traps: txbar_wait gives
 *     up after a bounded number of polls and returns false.
 */
#ifndef ATT_TILE_HPP
#define ATT_TILE_HPP

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tmap.h"
#include "att/im2col_device.hpp"
#include "att/tile_device.hpp"
#include "att/tmap_impl.hpp"

namespace att {

// The 128 bytes of a tiled map as the device reads them.
__device__ __forceinline__ const TmapImpl& tmap_tiled(const tmap_t& map) {
    return *reinterpret_cast<const TmapImpl*>(&map);
}

// A copy of a map that is the same for the whole wave (a kernel argument,
// as the pages pass descriptors) in scalar registers, read as whole 32-bit
// words: the map's one- and two-byte fields read where they lie would take
// vector-memory loads, a memory round trip before the first copy of every
// workgroup.  Kernels that take a map as an argument start from this.
__device__ __forceinline__ TmapImpl tmap_tiled_uniform(const tmap_t& map) { return uniform_copy(tmap_tiled(map)); }

// The 128 bytes of an im2col map as the device reads them.
__device__ __forceinline__ const Im2colImpl& tmap_im2col(const tmap_t& map) {
    return *reinterpret_cast<const Im2colImpl*>(&map);
}

// The box origin as the address generator takes it: entries past the map's
// rank become 0 (the caller's values there are ignored).
__device__ __forceinline__ void clip_coords(const TmapImpl& m, const int32_t (&c)[5], int32_t (&out)[5]) {
#pragma unroll
    for (int d = 0; d < 5; ++d) out[d] = d < (int)m.rank ? c[d] : 0;
}

// Bytes of one box's LDS image: the expect_tx amount of a whole load, for
// boxes inside, across or wholly outside the tensor alike ([HPC] async
// completion arms the barrier with the full tile size).
__device__ __forceinline__ uint32_t tile_box_bytes(const tmap_t& map) { return tmap_tiled(map).box_bytes; }

// Load, global -> LDS ([HPC] single-tile load; [MLC] "TMA writes swizzled
// layout").  Issues this wave's share of box `c` of a tiled map into the LDS
// image at `lds` and returns the bytes that share writes.  The copies are in
// flight when the call returns; they have landed after tile_load_arrive (or
// the wave's own s_waitcnt vmcnt(0) lgkmcnt(0)).  The bits are copied as
// they are (no float conversion); the swizzle is applied on the source side.
__device__ __forceinline__ uint32_t tile_load_async(const tmap_t& map, const int32_t (&c)[5], void* lds,
                                                    uint32_t wave, uint32_t nwaves) {
    int32_t cc[5];
    clip_coords(tmap_tiled(map), c, cc);
    return tile_load_issue(tmap_tiled(map), cc, static_cast<uint8_t*>(lds), wave, nwaves);
}

// Im2col-mode load ([HPC] closing paragraph names im2col-mode maps): the
// map's pixelsPerColumn pixels from window origin `c` = (channel, spatial...,
// image) and channelsPerPixel channels each, the spatial tap `off` (one entry
// per spatial dimension, W first) added to every pixel's position.  Same
// completion as tile_load_async.
__device__ __forceinline__ uint32_t tile_load_im2col_async(const tmap_t& map, const int32_t (&c)[5],
                                                           const int32_t (&off)[3], void* lds, uint32_t wave,
                                                           uint32_t nwaves) {
    const Im2colImpl& m = tmap_im2col(map);
    int32_t cc[5], oo[3];
#pragma unroll
    for (int d = 0; d < 5; ++d) cc[d] = d < (int)m.rank ? c[d] : 0;
#pragma unroll
    for (int s = 0; s < 3; ++s) oo[s] = s + 2 < (int)m.rank ? off[s] : 0;
    return tile_load_im2col_issue(m, cc, oo, static_cast<uint8_t*>(lds), wave, nwaves);
}

// Completion of a load ([MLC] "waiting for a TMA load": the copy reports the
// bytes it wrote to the barrier).  Waits until this wave's outstanding
// copies have landed, then one lane applies complete_tx(bytes) to `bar`.
// Every wave that issued part of the box calls it with the bytes its
// tile_load_async returned (0 is allowed and reports nothing).
__device__ __forceinline__ void tile_load_arrive(TxBar* bar, uint32_t bytes) {
    wait_vmcnt<0>();
    wait_lgkm0();
    if (lane_id() == 0 && bytes) txbar_complete_tx(bar, (int32_t)bytes);
}

// The pages' form of the load, with the barrier as an argument ([HPC]
// single-tile load: LDS destination, map, coordinates, barrier): this wave's
// share of box `c` is issued and, once it has landed, its bytes are applied
// to `bar` as complete_tx.  gfx950 has no engine to report the bytes later,
// so the wave itself waits for its copies before returning; the two-step
// form (tile_load_async, independent work, tile_load_arrive) keeps the wave
// free in between.  Returns the bytes this wave's share wrote.
__device__ __forceinline__ uint32_t tile_load_async(const tmap_t& map, const int32_t (&c)[5], void* lds, TxBar* bar,
                                                    uint32_t wave, uint32_t nwaves) {
    const uint32_t bytes = tile_load_async(map, c, lds, wave, nwaves);
    tile_load_arrive(bar, bytes);
    return bytes;
}

// Store, LDS -> global, with the inverse swizzle ([HPC] "TMA store").  Writes
// this wave's share of the LDS image at `lds` to box `c`; elements outside
// the tensor are not written.  The image must be complete in LDS (all its
// writers past a workgroup barrier).  When the call returns this wave's LDS
// reads have completed; the global writes are in flight.  Completion goes
// through store groups: pass the wave's StoreGroups to add these stores to
// its open group, then store_commit / store_wait<N> as on the pages
// (tile_store_wait waits for everything).  `streaming` makes the 16-byte
// stores non-temporal (for output not read again soon).
__device__ __forceinline__ void tile_store_async(const tmap_t& map, const int32_t (&c)[5], const void* lds,
                                                 uint32_t wave, uint32_t nwaves) {
    int32_t cc[5];
    clip_coords(tmap_tiled(map), c, cc);
    tile_store_issue<ST_STORE>(tmap_tiled(map), cc, static_cast<const uint8_t*>(lds), wave, nwaves);
}

__device__ __forceinline__ void tile_store_async(const tmap_t& map, const int32_t (&c)[5], const void* lds,
                                                 uint32_t wave, uint32_t nwaves, StoreGroups& groups,
                                                 bool streaming = false) {
    int32_t cc[5];
    clip_coords(tmap_tiled(map), c, cc);
    const uint8_t* img = static_cast<const uint8_t*>(lds);
    groups.open += streaming ? tile_store_issue<ST_STORE, true>(tmap_tiled(map), cc, img, wave, nwaves)
                             : tile_store_issue<ST_STORE, false>(tmap_tiled(map), cc, img, wave, nwaves);
}

// Reduce store ([HPC] "TMA reduce": element-wise add, min or max on write
// back).  OP is TMAP_REDUCE_ADD, TMAP_REDUCE_MIN or TMAP_REDUCE_MAX.  Each
// in-range element of the image is combined atomically with global memory:
// integers add modulo 2^w, a float add rounds the exact sum of the two
// operands once to the element type (round to nearest even); min / max
// compare integers as their type and floats as IEEE minNum / maxNum (a NaN
// operand yields the other one, two NaNs the canonical quiet NaN, -0 below
// +0).  Boxes of one or several workgroups may overlap; no order between
// them is defined.  Completion as tile_store_async.
template <int OP>
__device__ __forceinline__ void tile_reduce_async(const tmap_t& map, const int32_t (&c)[5], const void* lds,
                                                  uint32_t wave, uint32_t nwaves) {
    static_assert(OP == TMAP_REDUCE_ADD || OP == TMAP_REDUCE_MIN || OP == TMAP_REDUCE_MAX, "reduce op");
    constexpr int ST = OP == TMAP_REDUCE_ADD ? ST_ADD : (OP == TMAP_REDUCE_MIN ? ST_MIN : ST_MAX);
    int32_t cc[5];
    clip_coords(tmap_tiled(map), c, cc);
    tile_store_issue<ST>(tmap_tiled(map), cc, static_cast<const uint8_t*>(lds), wave, nwaves);
}

// The same reduction as part of the wave's open store group.
template <int OP>
__device__ __forceinline__ void tile_reduce_async(const tmap_t& map, const int32_t (&c)[5], const void* lds,
                                                  uint32_t wave, uint32_t nwaves, StoreGroups& groups) {
    tile_reduce_async<OP>(map, c, lds, wave, nwaves);
    (void)groups;   // atomics add nothing to the group's lower bound
}

// Wait until this wave's global writes (stores and reductions) have
// completed, e.g. before other workgroups are told to read them.  Also waits
// for this wave's outstanding loads.
__device__ __forceinline__ void tile_store_wait() {
    wait_vmcnt<0>();
    wait_lgkm0();
}

// ---- store groups ([HPC] "TMA store": commit_group / wait_group N; [MLC]
// "waiting for a TMA store": the source tile may be overwritten only after
// the group that stores it has completed) ------------------------------------
//
//     att::StoreGroups sg;
//     att::store_groups_init(sg);
//     att::tile_store_async(map, c0, stage0, w, nw, sg);  att::store_commit(sg);
//     att::tile_store_async(map, c1, stage1, w, nw, sg);  att::store_commit(sg);
//     att::store_wait<1>(sg);        // the first group's writes are done
//     ... every storing wave waits, then a workgroup barrier; stage0 is free
//
// Groups are per wave, like the pages' per-thread groups: a stage stored by
// several waves is free once each of them has waited and the workgroup has
// passed a barrier.

// Close the open group: the stores issued since the last commit.
__device__ __forceinline__ void store_commit(StoreGroups& g) {
#pragma unroll
    for (int i = StoreGroups::kDepth - 1; i > 0; --i) g.cnt[i] = g.cnt[i - 1];
    g.cnt[0] = g.open;
    g.open = 0;
}

// Wait until every committed group except the N most recent has completed
// (its global writes performed), as the pages' wait_group N.  Stores still
// open count as newer than every committed group.
template <int N>
__device__ __forceinline__ void store_wait(StoreGroups& g) {
    static_assert(N >= 0 && N < StoreGroups::kDepth, "store_wait depth");
    uint32_t newer = g.open;
#pragma unroll
    for (int i = 0; i < N; ++i) newer += g.cnt[i];
    wait_vmcnt_le(newer);
}

// The pages' wait_group.read N: the LDS sources of every committed group
// except the N most recent may be overwritten.  On gfx950 a store call's
// LDS reads have completed when it returns, so this only makes sure of that
// (lgkmcnt); the global writes may still be in flight.
template <int N>
__device__ __forceinline__ void store_wait_read(StoreGroups& g) {
    static_assert(N >= 0 && N < StoreGroups::kDepth, "store_wait depth");
    (void)g;
    wait_lgkm0();
}

}  // namespace att

#endif  // ATT_TILE_HPP
