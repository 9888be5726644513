// host_util.hpp -- helpers shared by the launch entry points.
#pragma once

#include <hip/hip_runtime.h>

#include "tmap.h"
#include "att/tmap_impl.hpp"

namespace att {

tmap_status hip_fail(hipError_t e, const char* where);
int esize_of(int32_t dtype);
TmapImpl load_map(const tmap_t* m);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// LDS bytes one workgroup may use on the current device.
inline tmap_status device_lds_limit(uint32_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    *out = (uint32_t)v;
    return TMAP_OK;
}

inline tmap_status device_cu_count(uint32_t* out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int v = 0;
    e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    *out = (uint32_t)v;
    return TMAP_OK;
}

inline tmap_status check_launch(const char* where) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, where);
    return TMAP_OK;
}

inline uint32_t round_up(uint32_t x, uint32_t a) { return (x + a - 1) / a * a; }

}  // namespace att
