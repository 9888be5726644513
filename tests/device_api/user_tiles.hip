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
