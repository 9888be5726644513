// im2col_device.hpp -- gfx950 device side of im2col-mode loads: one box of
// an im2col map (pixels x channels) into an LDS image, with the swizzle
// applied on write and fill for pixels or channels outside the tensor
// ([HPC] closing paragraph names im2col-mode tensor maps; the window
// semantics are this library's reading of that name).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_device.hpp"

namespace att {

// ---- im2col mode ------------------------------------------------------------
// Window origins form a mixed-radix number (W digit fastest, image index
// last); pixel r of a load is the origin r positions after the one its
// coordinates name (a start between grid points snaps down to the grid).

__device__ __forceinline__ int64_t floor_div64(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

// One pixel row: whether the whole pixel (all spatial dims and the image
// index) lies inside the tensor, and its byte offset without the channel.
struct PixelLoc {
    int64_t off;
    bool in;
};

__device__ __forceinline__ PixelLoc im2col_pixel(const Im2colImpl& m, int64_t L, const int32_t off[3]) {
    const int S = m.rank - 2;
    PixelLoc r;
    r.off = 0;
    r.in = true;
#pragma unroll
    for (int s = 0; s < 3; ++s) {
        if (s < S) {
            const int64_t n = (int64_t)m.npos[s];
            const int64_t q = floor_div64(L, n);
            const int64_t digit = L - q * n;
            L = q;
            const int64_t x = (int64_t)m.lower[s] + digit * (int64_t)m.es[s + 1] + (int64_t)off[s];
            r.in = r.in && x >= 0 && x < m.dim[s + 1];
            r.off += x * (int64_t)m.stride[s];
        }
    }
    r.in = r.in && L >= 0 && L < m.dim[m.rank - 1];
    r.off += L * (int64_t)m.stride[m.rank - 2];
    return r;
}

template <typename T>
__device__ __forceinline__ u32x4 im2col_gather_t(const Im2colImpl& m, const PixelLoc& P, int64_t ch0) {
    constexpr int N = 16 / (int)sizeof(T);
    union { u32x4 v; T e[N]; } u;
    const T fillv = *reinterpret_cast<const T*>(g_fill_rows[m.fill_idx]);
    const ATT_GLOBAL T* row = (const ATT_GLOBAL T*)gptr(m.base + (uint64_t)P.off);
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const int64_t ch = ch0 + e;
        const bool in = P.in && ch >= 0 && ch < m.dim[0];
        u.e[e] = in ? row[ch] : fillv;
    }
    return u.v;
}

__device__ __forceinline__ u32x4 im2col_gather(const Im2colImpl& m, const PixelLoc& P, int64_t ch0) {
    switch (m.esize) {
    case 1: return im2col_gather_t<uint8_t>(m, P, ch0);
    case 2: return im2col_gather_t<uint16_t>(m, P, ch0);
    case 4: return im2col_gather_t<uint32_t>(m, P, ch0);
    default: return im2col_gather_t<uint64_t>(m, P, ch0);
    }
}

// Window-origin index of the first pixel of a load: the mixed-radix number
// whose digits are the spatial origins' grid positions (W fastest) and whose
// last digit is the image index.  c holds (channel, spatial..., image).
__device__ __forceinline__ int64_t im2col_first_pixel(const Im2colImpl& m, const int32_t c[5]) {
    const int R = m.rank;
    int64_t L0 = c[R - 1];
#pragma unroll
    for (int s = 2; s >= 0; --s)
        if (s < R - 2)
            L0 = L0 * (int64_t)m.npos[s] + floor_div64((int64_t)c[s + 1] - m.lower[s], (int64_t)m.es[s + 1]);
    return L0;
}

// This wave's share of one im2col box (64-chunk groups wave, wave + nwaves,
// ...) into the LDS image `lds`; returns the bytes this wave wrote, landed
// once the wave has waited vmcnt(0) and lgkmcnt(0).  Lane l of group grp
// fills physical chunk grp*64 + l with logical chunk swz(p): its pixel row
// and channel block.  Whole in-range 16-byte aligned chunks and wholly
// out-of-range chunks (read from the fill row) go through global_load_lds;
// chunks cut by the channel edge are gathered by their lane.
__device__ __forceinline__ uint32_t tile_load_im2col_issue(const Im2colImpl& m, const int32_t c[5],
                                                           const int32_t off[3], uint8_t* lds, uint32_t wave,
                                                           uint32_t nwaves) {
    const int64_t L0 = im2col_first_pixel(m, c);
    const uint32_t lane = lane_id();
    const uint32_t nchunk = m.box_bytes >> 4;
    const int64_t n_el = 16 / m.esize;
    const bool aligned = (((int64_t)c[0] * m.esize) & 15) == 0;
    const void* fill = g_fill_rows[m.fill_idx];
    uint32_t bytes = 0;
    for (uint32_t grp = wave; grp * 64u < nchunk; grp += nwaves) {
        const uint32_t p = grp * 64u + lane;
        const bool active = p < nchunk;
        const uint32_t rem = nchunk - grp * 64u;
        bytes += 16u * (rem < 64u ? rem : 64u);
        const uint32_t q = active ? swz_chunk(p, m.swizzle) : 0u;
        const uint32_t row = q / m.cpr;
        const uint32_t j = q - row * m.cpr;
        const PixelLoc P = im2col_pixel(m, L0 + (int64_t)row, off);
        const int64_t ch0 = (int64_t)c[0] + (int64_t)j * n_el;
        const bool full_in = P.in && ch0 >= 0 && ch0 + n_el <= m.dim[0];
        const bool full_out = !P.in || ch0 >= m.dim[0] || ch0 + n_el <= 0;
        const bool partial = !aligned || (!full_in && !full_out);
        const void* src = full_in ? (const void*)(uintptr_t)(m.base + (uint64_t)P.off + (uint64_t)ch0 * m.esize) : fill;
        if (active && !partial) dma16(src, lds + grp * 1024u);
        if (active && partial) *reinterpret_cast<u32x4*>(lds + p * 16u) = im2col_gather(m, P, ch0);
    }
    return bytes;
}

}  // namespace att
