// tmap_impl.hpp -- layout of the 128-byte tensor-map descriptor as the host
// encoder writes it and the gfx950 kernels read it (by value, as a kernel
// argument, so every field lands in scalar registers).
//
// The public header exposes tmap_t as 128 opaque bytes; this file is the only
// place that interprets them.
#pragma once

#include <stdint.h>

#include "tmap.h"

namespace att {

struct alignas(64) TmapImpl {
    uint64_t base;          // global base address (16-byte aligned)
    uint64_t stride[4];     // byte strides of dims 1..4 (0 beyond rank)
    int64_t  dim[5];        // globalDim (1 beyond rank)
    uint16_t L[5];          // LDS extent per dim: ceil(box / estride)
    uint8_t  box_m1[5];     // box extent - 1
    uint8_t  es[5];         // element stride per dim
    uint8_t  rank;
    uint8_t  dtype;         // tmap_dtype
    uint8_t  esize;         // 1, 2, 4, 8
    uint8_t  swizzle;       // tmap_swizzle; also the number of XOR bits
    uint8_t  oob;           // tmap_oob
    uint8_t  fill_idx;      // row of the device fill-pattern table
    uint16_t cpr;           // 16-byte chunks per LDS row
    uint32_t box_bytes;     // esize * prod(L)
    // Division by an invariant d < 2^16 for n < 2^24: q = umulhi(n, magic)
    // with magic = ceil(2^32 / d); magic == 0 encodes d == 1 (q = n).
    uint32_t magic_cpr;
    uint32_t magic_L[3];    // for L[1], L[2], L[3]
};

static_assert(sizeof(TmapImpl) == 128, "descriptor must stay 128 bytes");

// Bit 7 of the OOB byte marks an im2col-mode descriptor (Im2colImpl below);
// tiled entry points reject such maps.
constexpr uint8_t OOB_IM2COL_FLAG = 0x80;

// The same 128 bytes for an im2col-mode map: dims (C, W[, H[, D]], N), S =
// rank - 2 spatial dimensions.  Window origins along spatial dimension s run
// over lower[s] + t * es[s+1], t < npos[s] (the grid up to dim - 1 +
// upper[s]).  The header fields shared with TmapImpl sit at the same offsets.
struct alignas(64) Im2colImpl {
    uint64_t base;
    uint64_t stride[4];
    int64_t  dim[5];
    int16_t  lower[3];
    int16_t  upper[3];
    uint8_t  pad0[3];
    uint8_t  es[5];
    uint8_t  rank;
    uint8_t  dtype;
    uint8_t  esize;
    uint8_t  swizzle;
    uint8_t  oob;           // TMAP_OOB_* | OOB_IM2COL_FLAG
    uint8_t  fill_idx;
    uint16_t cpr;           // 16-byte chunks per LDS row (per pixel)
    uint32_t box_bytes;     // pixels * channels * esize
    uint16_t channels;      // channelsPerPixel
    uint16_t pixels;        // pixelsPerColumn
    uint32_t npos[3];       // window positions per spatial dimension
};

static_assert(sizeof(Im2colImpl) == 128, "im2col descriptor must stay 128 bytes");
static_assert(__builtin_offsetof(Im2colImpl, es) == __builtin_offsetof(TmapImpl, es) &&
              __builtin_offsetof(Im2colImpl, rank) == __builtin_offsetof(TmapImpl, rank) &&
              __builtin_offsetof(Im2colImpl, oob) == __builtin_offsetof(TmapImpl, oob) &&
              __builtin_offsetof(Im2colImpl, fill_idx) == __builtin_offsetof(TmapImpl, fill_idx) &&
              __builtin_offsetof(Im2colImpl, cpr) == __builtin_offsetof(TmapImpl, cpr) &&
              __builtin_offsetof(Im2colImpl, box_bytes) == __builtin_offsetof(TmapImpl, box_bytes),
              "shared header fields at the same offsets");

inline bool is_im2col(const TmapImpl& t) { return (t.oob & OOB_IM2COL_FLAG) != 0; }
static_assert(sizeof(tmap_t) == 128, "public descriptor is 128 bytes");

// Rows of the device fill table (16 bytes each): zero, then one quiet-NaN row
// per float element width.
enum : uint8_t { FILL_ZERO = 0, FILL_NAN_F32 = 1, FILL_NAN_F16 = 2, FILL_NAN_BF16 = 3, FILL_NAN_F64 = 4 };

inline uint32_t magic_for(uint32_t d) {
    if (d <= 1) return 0u;
    return (uint32_t)(((1ull << 32) + d - 1) / d);
}

}  // namespace att
