// tmap_host.hip -- host side of the C ABI: descriptor encoding and
// validation, queries and error text.  Launch entry points live beside their
// kernels.
//
// Constraint sources: [H200] section 03 table (rank, box, strides, base
// alignment), [MLC] "3D TMA" / "grouping requirement" (swizzle span), [H200]
// section 02 table (zero / NaN fill).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>

#include "tmap.h"
#include "att/tmap_impl.hpp"
#include "host_util.hpp"

namespace att {

thread_local char g_last_error[256] = "";

tmap_status hip_fail(hipError_t e, const char* where) {
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
    return TMAP_ERR_HIP;
}

int esize_of(int32_t dtype) {
    switch (dtype) {
    case TMAP_U8: return 1;
    case TMAP_U16: case TMAP_F16: case TMAP_BF16: return 2;
    case TMAP_U32: case TMAP_I32: case TMAP_F32: return 4;
    case TMAP_U64: case TMAP_I64: case TMAP_F64: return 8;
    default: return 0;
    }
}

static bool is_float(int32_t dtype) {
    return dtype == TMAP_F16 || dtype == TMAP_BF16 || dtype == TMAP_F32 || dtype == TMAP_F64;
}

// Caller storage may be less aligned than TmapImpl (e.g. a ctypes buffer), so
// descriptors are always copied bytewise.
TmapImpl load_map(const tmap_t* m) {
    TmapImpl t;
    std::memcpy(&t, m, sizeof(t));
    return t;
}

}  // namespace att

using namespace att;

extern "C" tmap_status tmap_encode(tmap_t* out, int32_t dtype, uint32_t rank, void* gaddr,
                                   const uint64_t* gdim, const uint64_t* gstride,
                                   const uint32_t* box, const uint32_t* estride,
                                   int32_t swizzle, int32_t oob) {
    if (!out) return TMAP_ERR_NULL;
    std::memset(out, 0, sizeof(tmap_t));
    if (!gdim || !box || (rank > 1 && !gstride)) return TMAP_ERR_NULL;
    if (rank < 1 || rank > 5) return TMAP_ERR_RANK;
    const int es = esize_of(dtype);
    if (es == 0) return TMAP_ERR_DTYPE;
    if (swizzle < TMAP_SWIZZLE_NONE || swizzle > TMAP_SWIZZLE_128B_K256 || swizzle == 4) return TMAP_ERR_UNSUPPORTED;
    if (oob != TMAP_OOB_ZERO && oob != TMAP_OOB_NAN) return TMAP_ERR_UNSUPPORTED;
    if (!gaddr) return TMAP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gaddr) % 16 != 0) return TMAP_ERR_ALIGN;
    for (uint32_t d = 0; d < rank; ++d)
        if (gdim[d] < 1 || gdim[d] > (1ull << 32)) return TMAP_ERR_DIM;
    for (uint32_t d = 1; d < rank; ++d) {
        const uint64_t s = gstride[d - 1];
        if (s == 0 || s % 16 != 0 || s >= (1ull << 40)) return TMAP_ERR_STRIDE;
    }
    for (uint32_t d = 0; d < rank; ++d)
        if (box[d] < 1 || box[d] > 256) return TMAP_ERR_BOX;
    if ((uint64_t)box[0] * (uint64_t)es % 16 != 0) return TMAP_ERR_BOX;
    uint32_t L[5] = {1, 1, 1, 1, 1};
    uint32_t esv[5] = {1, 1, 1, 1, 1};
    for (uint32_t d = 0; d < rank; ++d) {
        const uint32_t e = estride ? estride[d] : 1u;
        if (e < 1 || e > 8) return TMAP_ERR_ESTRIDE;
        esv[d] = e;
        L[d] = (box[d] + e - 1) / e;
    }
    const uint32_t row_bytes = L[0] * (uint32_t)es;
    if (row_bytes % 16 != 0) return TMAP_ERR_ESTRIDE;
    if (swizzle != TMAP_SWIZZLE_NONE && row_bytes != (16u << (swizzle & 3))) return TMAP_ERR_SWIZZLE_WIDTH;
    if (oob == TMAP_OOB_NAN && !is_float(dtype)) return TMAP_ERR_OOB_FILL_DTYPE;
    uint64_t bytes = (uint64_t)es;
    for (int d = 0; d < 5; ++d) bytes *= L[d];
    if (bytes > TMAP_LDS_CAPACITY) return TMAP_ERR_LDS_CAPACITY;

    TmapImpl t;
    std::memset(&t, 0, sizeof(t));
    t.base = reinterpret_cast<uint64_t>(gaddr);
    for (int d = 0; d < 5; ++d) {
        t.dim[d] = d < (int)rank ? (int64_t)gdim[d] : 1;
        t.L[d] = (uint16_t)L[d];
        t.box_m1[d] = (uint8_t)(d < (int)rank ? box[d] - 1 : 0);
        t.es[d] = (uint8_t)esv[d];
    }
    for (int d = 1; d < 5; ++d) t.stride[d - 1] = d < (int)rank ? gstride[d - 1] : 0;
    t.rank = (uint8_t)rank;
    t.dtype = (uint8_t)dtype;
    t.esize = (uint8_t)es;
    t.swizzle = (uint8_t)swizzle;
    t.oob = (uint8_t)oob;
    t.fill_idx = FILL_ZERO;
    if (oob == TMAP_OOB_NAN) {
        t.fill_idx = dtype == TMAP_F32 ? FILL_NAN_F32
                   : dtype == TMAP_F16 ? FILL_NAN_F16
                   : dtype == TMAP_BF16 ? FILL_NAN_BF16 : FILL_NAN_F64;
    }
    t.cpr = (uint16_t)(row_bytes / 16);
    t.box_bytes = (uint32_t)bytes;
    t.magic_cpr = magic_for(t.cpr);
    for (int d = 0; d < 3; ++d) t.magic_L[d] = magic_for(L[d + 1]);
    std::memcpy(out, &t, sizeof(t));
    return TMAP_OK;
}

// Im2col-mode map (see tmap.h for the definition).  Same header checks as the
// tiled encoder, then the window grid per spatial dimension.
extern "C" tmap_status tmap_encode_im2col(tmap_t* out, int32_t dtype, uint32_t rank, void* gaddr,
                                          const uint64_t* gdim, const uint64_t* gstride, const int32_t* lower,
                                          const int32_t* upper, uint32_t channels, uint32_t pixels,
                                          const uint32_t* estride, int32_t swizzle, int32_t oob) {
    if (!out) return TMAP_ERR_NULL;
    std::memset(out, 0, sizeof(tmap_t));
    if (!gdim || !gstride || !lower || !upper) return TMAP_ERR_NULL;
    if (rank < 3 || rank > 5) return TMAP_ERR_RANK;
    const int es = esize_of(dtype);
    if (es == 0) return TMAP_ERR_DTYPE;
    if (swizzle < TMAP_SWIZZLE_NONE || swizzle > TMAP_SWIZZLE_128B_K256 || swizzle == 4) return TMAP_ERR_UNSUPPORTED;
    if (oob != TMAP_OOB_ZERO && oob != TMAP_OOB_NAN) return TMAP_ERR_UNSUPPORTED;
    if (!gaddr) return TMAP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gaddr) % 16 != 0) return TMAP_ERR_ALIGN;
    for (uint32_t d = 0; d < rank; ++d)
        if (gdim[d] < 1 || gdim[d] > (1ull << 32)) return TMAP_ERR_DIM;
    for (uint32_t d = 1; d < rank; ++d) {
        const uint64_t st = gstride[d - 1];
        if (st == 0 || st % 16 != 0 || st >= (1ull << 40)) return TMAP_ERR_STRIDE;
    }
    if (channels < 1 || channels > 256 || ((uint64_t)channels * (uint64_t)es) % 16 != 0) return TMAP_ERR_BOX;
    if (pixels < 1 || pixels > 1024) return TMAP_ERR_BOX;
    uint32_t esv[5] = {1, 1, 1, 1, 1};
    for (uint32_t d = 0; d < rank; ++d) esv[d] = estride ? estride[d] : 1u;
    if (esv[0] != 1 || esv[rank - 1] != 1) return TMAP_ERR_ESTRIDE;
    for (uint32_t d = 1; d + 1 < rank; ++d)
        if (esv[d] < 1 || esv[d] > 8) return TMAP_ERR_ESTRIDE;
    const uint32_t S = rank - 2;
    uint64_t npos[3] = {1, 1, 1};
    // the linear window index (image most significant) must fit signed
    // 64-bit arithmetic
    for (uint32_t sd = 0; sd < S; ++sd) {
        if (lower[sd] < -32768 || lower[sd] > 32767 || upper[sd] < -32768 || upper[sd] > 32767) return TMAP_ERR_BOX;
        const int64_t lo = lower[sd];
        const int64_t hi = (int64_t)gdim[sd + 1] - 1 + (int64_t)upper[sd];
        if (hi < lo) return TMAP_ERR_BOX;
        npos[sd] = (uint64_t)((hi - lo) / (int64_t)esv[sd + 1] + 1);
    }
    // checked after every factor (each below 2^34), so the product never
    // wraps the 128-bit counter
    unsigned __int128 total = gdim[rank - 1];
    if (total > ((unsigned __int128)1 << 62)) return TMAP_ERR_DIM;
    for (uint32_t sd = 0; sd < S; ++sd) {
        total *= npos[sd];
        if (total > ((unsigned __int128)1 << 62)) return TMAP_ERR_DIM;
    }
    const uint32_t row_bytes = channels * (uint32_t)es;
    if (swizzle != TMAP_SWIZZLE_NONE && row_bytes != (16u << (swizzle & 3))) return TMAP_ERR_SWIZZLE_WIDTH;
    if (oob == TMAP_OOB_NAN && !is_float(dtype)) return TMAP_ERR_OOB_FILL_DTYPE;
    if ((uint64_t)row_bytes * pixels > TMAP_LDS_CAPACITY) return TMAP_ERR_LDS_CAPACITY;

    Im2colImpl t;
    std::memset(&t, 0, sizeof(t));
    t.base = reinterpret_cast<uint64_t>(gaddr);
    for (int d = 0; d < 5; ++d) {
        t.dim[d] = d < (int)rank ? (int64_t)gdim[d] : 1;
        t.es[d] = (uint8_t)esv[d];
    }
    for (int d = 1; d < 5; ++d) t.stride[d - 1] = d < (int)rank ? gstride[d - 1] : 0;
    for (uint32_t sd = 0; sd < 3; ++sd) {
        t.lower[sd] = (int16_t)(sd < S ? lower[sd] : 0);
        t.upper[sd] = (int16_t)(sd < S ? upper[sd] : 0);
        t.npos[sd] = (uint32_t)npos[sd];
    }
    t.rank = (uint8_t)rank;
    t.dtype = (uint8_t)dtype;
    t.esize = (uint8_t)es;
    t.swizzle = (uint8_t)swizzle;
    t.oob = (uint8_t)(oob | OOB_IM2COL_FLAG);
    t.fill_idx = FILL_ZERO;
    if (oob == TMAP_OOB_NAN) {
        t.fill_idx = dtype == TMAP_F32 ? FILL_NAN_F32
                   : dtype == TMAP_F16 ? FILL_NAN_F16
                   : dtype == TMAP_BF16 ? FILL_NAN_BF16 : FILL_NAN_F64;
    }
    t.cpr = (uint16_t)(row_bytes / 16);
    t.box_bytes = row_bytes * pixels;
    t.channels = (uint16_t)channels;
    t.pixels = (uint16_t)pixels;
    std::memcpy(out, &t, sizeof(t));
    return TMAP_OK;
}

extern "C" tmap_status tmap_replace_address(tmap_t* m, void* gaddr) {
    if (!m || !gaddr) return TMAP_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(gaddr) % 16 != 0) return TMAP_ERR_ALIGN;
    TmapImpl t = load_map(m);
    t.base = reinterpret_cast<uint64_t>(gaddr);
    std::memcpy(m, &t, sizeof(t));
    return TMAP_OK;
}

extern "C" uint32_t tmap_box_bytes(const tmap_t* m) { return m ? load_map(m).box_bytes : 0u; }

extern "C" tmap_status tmap_query(const tmap_t* m, tmap_info_t* info) {
    if (!m || !info) return TMAP_ERR_NULL;
    const TmapImpl tv = load_map(m);
    const TmapImpl* t = &tv;
    std::memset(info, 0, sizeof(*info));
    info->dtype = t->dtype;
    info->rank = t->rank;
    info->esize = t->esize;
    info->swizzle = t->swizzle;
    info->oob = t->oob & (uint8_t)~OOB_IM2COL_FLAG;
    if (is_im2col(*t)) {
        Im2colImpl im;
        std::memcpy(&im, m, sizeof(im));
        info->lds_extent[0] = im.channels;
        info->lds_extent[1] = im.pixels;
        for (int d = 2; d < 5; ++d) info->lds_extent[d] = 1;
    } else {
        for (int d = 0; d < 5; ++d) info->lds_extent[d] = t->L[d];
    }
    info->box_bytes = t->box_bytes;
    info->row_bytes = (uint32_t)t->cpr * 16u;
    info->atom_bytes = t->swizzle ? ((t->swizzle & 4) ? 16u : 8u) * (16u << (t->swizzle & 3)) : 0u;
    info->base = t->base;
    return TMAP_OK;
}

extern "C" const char* tmap_strerror(tmap_status s) {
    switch (s) {
    case TMAP_OK: return "ok";
    case TMAP_ERR_NULL: return "required pointer is NULL";
    case TMAP_ERR_RANK: return "rank must be in [1, 5]";
    case TMAP_ERR_DTYPE: return "unknown element type";
    case TMAP_ERR_ALIGN: return "base address must be 16-byte aligned";
    case TMAP_ERR_DIM: return "globalDim must be in [1, 2^32]";
    case TMAP_ERR_STRIDE: return "global strides must be nonzero multiples of 16 below 2^40";
    case TMAP_ERR_BOX: return "box extents must be in [1, 256] with box[0]*esize a multiple of 16";
    case TMAP_ERR_ESTRIDE: return "element strides must be in [1, 8] and keep LDS rows whole 16-byte chunks";
    case TMAP_ERR_SWIZZLE_WIDTH: return "swizzled LDS row must equal the swizzle span";
    case TMAP_ERR_OOB_FILL_DTYPE: return "NaN fill needs a floating-point element type";
    case TMAP_ERR_LDS_CAPACITY: return "box image exceeds the LDS of one workgroup";
    case TMAP_ERR_UNSUPPORTED: return "unsupported argument for this call";
    case TMAP_ERR_HIP: return "HIP runtime error";
    case TMAP_ERR_TIMEOUT: return "a bounded barrier wait in a kernel gave up; the box it guarded is not valid";
    case TMAP_ERR_DEVICE_CHECK: return "a device-side check of the debug build failed";
    default: return "unknown status";
    }
}

extern "C" const char* tmap_last_error(void) { return g_last_error; }

// Host check of the invariant-division trick the kernels use: for every
// divisor 1..256 and every numerator below 2^20 the quotient is exact.
// Returns the number of mismatches (0 expected).
extern "C" uint64_t tmap_selftest_divide(void) {
    uint64_t bad = 0;
    for (uint32_t d = 1; d <= 256; ++d) {
        const uint32_t mg = magic_for(d);
        for (uint32_t n = 0; n < (1u << 20); ++n) {
            const uint32_t q = mg ? (uint32_t)(((uint64_t)n * mg) >> 32) : n;
            bad += (q != n / d);
        }
    }
    return bad;
}
