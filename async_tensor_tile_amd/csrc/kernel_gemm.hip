// kernel_gemm.hip -- bf16 GEMM mainloop consuming tiles staged by the tile
// loader (work in progress: the entry point reports TMAP_ERR_UNSUPPORTED).
#include <hip/hip_runtime.h>

#include "host_util.hpp"
#include "tmap.h"

extern "C" tmap_status gemm_bf16(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                                 uint32_t K, uint32_t ldc, uint32_t stages, void* stream) {
    (void)M; (void)N; (void)K; (void)ldc; (void)stages; (void)stream;
    if (!A || !B || !d_C) return TMAP_ERR_NULL;
    return TMAP_ERR_UNSUPPORTED;
}
