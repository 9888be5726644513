// A kernel written the way a user of the device API would write one: it
// includes only tile.hpp (compiled with include/ as the only include path)
// and moves boxes of host-encoded maps itself.  One workgroup per box: load
// the box of `src` into LDS with byte-counted completion, then store it
// through `dst` and add it into `acc` through the same coordinates.
#include <hip/hip_runtime.h>

#include "tile.hpp"

__global__ __launch_bounds__(256) void user_load_store_reduce(tmap_t src, tmap_t dst, tmap_t acc,
                                                              const int32_t* __restrict__ coords, uint32_t rank,
                                                              uint32_t bar_off, int32_t* __restrict__ landed) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t img[];
    att::TxBar* bar = reinterpret_cast<att::TxBar*>(img + bar_off);
    const uint32_t w = threadIdx.x / 64, nw = blockDim.x / 64;
    int32_t c[5] = {0, 0, 0, 0, 0};
    for (uint32_t d = 0; d < rank; ++d) c[d] = coords[blockIdx.x * rank + d];
    if (threadIdx.x == 0) {
        att::txbar_init(bar, 1);
        att::txbar_arrive_expect_tx(bar, (int32_t)att::tile_box_bytes(src));
    }
    __syncthreads();
    const uint32_t bytes = att::tile_load_async(src, c, img, w, nw);
    att::tile_load_arrive(bar, bytes);
    const bool ok = att::txbar_wait(bar, 0);
    __syncthreads();
    att::tile_store_async(dst, c, img, w, nw);
    att::tile_reduce_async<TMAP_REDUCE_ADD>(acc, c, img, w, nw);
    att::tile_store_wait();
    if (threadIdx.x == 0) landed[blockIdx.x] = ok ? 1 : 0;
}

// Launch: nbox workgroups of 256 threads, the box image plus the barrier in
// dynamic LDS.  Returns a hipError_t.
extern "C" int user_load_store_reduce_launch(const tmap_t* src, const tmap_t* dst, const tmap_t* acc,
                                             const int32_t* d_coords, uint32_t rank, uint32_t nbox,
                                             uint32_t box_bytes, int32_t* d_landed, void* stream) {
    if (nbox == 0) return 0;
    const uint32_t bar_off = (box_bytes + 1023u) / 1024u * 1024u;
    const uint32_t lds = bar_off + 64u;
    hipError_t e = hipFuncSetAttribute((const void*)user_load_store_reduce,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    tmap_t s, d, a;
    __builtin_memcpy(&s, src, sizeof(s));
    __builtin_memcpy(&d, dst, sizeof(d));
    __builtin_memcpy(&a, acc, sizeof(a));
    hipLaunchKernelGGL(user_load_store_reduce, dim3(nbox), dim3(256), lds, (hipStream_t)stream, s, d, a, d_coords,
                       rank, bar_off, d_landed);
    return (int)hipGetLastError();
}

// Store groups with LDS stages reused across boxes: one workgroup copies
// `nbox` boxes of `src` to `dst` through S stages.  Box k is loaded into
// stage k % S with the barrier form of the load and stored as one store
// group; before a stage is refilled, the group that stored from it must have
// completed: with one stage that is the newest group (store_wait<0>), with
// two all but the newest (store_wait<1>).  Wave 0 records the size its
// store_commit gave every group.  The coordinates past the map's rank hold
// junk that every call must ignore.
template <int S>
__global__ __launch_bounds__(256) void user_staged_copy(tmap_t src, tmap_t dst, const int32_t* __restrict__ coords,
                                                        uint32_t rank, uint32_t nbox, uint32_t stage_bytes,
                                                        int32_t* __restrict__ sizes, int32_t* __restrict__ landed) {
    extern __shared__ __attribute__((aligned(1024))) uint8_t lds[];
    att::TxBar* bars = reinterpret_cast<att::TxBar*>(lds + S * stage_bytes);
    const uint32_t w = threadIdx.x / 64, nw = blockDim.x / 64;
    att::StoreGroups sg;
    att::store_groups_init(sg);
    if (threadIdx.x == 0)
        for (int s = 0; s < S; ++s) att::txbar_init(&bars[s], 1);
    __syncthreads();
    bool ok = true;
    for (uint32_t k = 0; k < nbox; ++k) {
        const uint32_t s = k % S;
        if (k >= (uint32_t)S) {
            if constexpr (S == 1) att::store_wait<0>(sg);
            else att::store_wait<1>(sg);
            att::wg_barrier();                 // the stage is free in every wave
        }
        int32_t c[5];
        for (uint32_t d = 0; d < 5; ++d) c[d] = d < rank ? coords[k * rank + d] : (int32_t)(12345 + d);
        uint8_t* stage = lds + s * stage_bytes;
        if (threadIdx.x == 0) att::txbar_arrive_expect_tx(&bars[s], (int32_t)att::tile_box_bytes(src));
        att::wg_barrier();                     // expected before any copy is issued
        att::tile_load_async(src, c, stage, &bars[s], w, nw);
        ok = att::txbar_wait(&bars[s], (k / S) & 1u) && ok;
        att::tile_store_async(dst, c, stage, w, nw, sg);
        att::store_commit(sg);
        if (threadIdx.x == 0) sizes[k] = (int32_t)sg.cnt[0];
    }
    att::store_wait<0>(sg);
    if (att::lane_id() == 0) landed[w] = ok ? 1 : 0;
}

// Launch: one workgroup of 256 threads; S stages of the box image plus a
// barrier per stage in dynamic LDS.  stages 1 or 2.  Returns a hipError_t,
// or -1 for other stage counts.
extern "C" int user_staged_copy_launch(const tmap_t* src, const tmap_t* dst, const int32_t* d_coords, uint32_t rank,
                                       uint32_t nbox, uint32_t stages, uint32_t box_bytes, int32_t* d_sizes,
                                       int32_t* d_landed, void* stream) {
    if (stages != 1 && stages != 2) return -1;
    const uint32_t stage_bytes = (box_bytes + 1023u) / 1024u * 1024u;
    const uint32_t lds = stages * stage_bytes + 64u;
    const void* fn = stages == 1 ? (const void*)user_staged_copy<1> : (const void*)user_staged_copy<2>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    tmap_t s, d;
    __builtin_memcpy(&s, src, sizeof(s));
    __builtin_memcpy(&d, dst, sizeof(d));
    if (stages == 1)
        hipLaunchKernelGGL(user_staged_copy<1>, dim3(1), dim3(256), lds, (hipStream_t)stream, s, d, d_coords, rank, nbox,
                           stage_bytes, d_sizes, d_landed);
    else
        hipLaunchKernelGGL(user_staged_copy<2>, dim3(1), dim3(256), lds, (hipStream_t)stream, s, d, d_coords, rank, nbox,
                           stage_bytes, d_sizes, d_landed);
    return (int)hipGetLastError();
}
