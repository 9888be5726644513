// tile_device.hpp -- gfx950 device side of the tile mover.
//
// What the reference pages give to a dedicated copy engine (one thread hands
// a descriptor plus box origin to hardware, [MLC] "one thread describes the
// whole tile") is done here by the wavefront itself: every lane computes the
// global address of one 16-byte chunk of the box and the wave issues
// global_load_lds_dwordx4, which writes lane l's 16 bytes to LDS at
// M0 + 16*l.  Because the LDS side of that instruction is lane-linear, the
// swizzle-on-write ([MLC] "TMA writes swizzled layout") is realised on the
// source side: the lane that fills physical chunk p fetches logical chunk
// swz(p); the XOR swizzle is an involution, so the same function maps both
// ways.  Completion is tracked per wave with s_waitcnt vmcnt; a byte-counted
// LDS barrier (TxBar) gives the expect-tx / complete-tx accounting of [MLC]
// "waiting for TMA load" when several waves share a box.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tmap_impl.hpp"

namespace att {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Global-memory pointers carry address space 1 so that accesses compile to
// global_* instructions rather than flat_* ones.
#define ATT_GLOBAL __attribute__((address_space(1)))
typedef ATT_GLOBAL uint8_t gbyte;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ gbyte* gptr(uint64_t addr) { return (gbyte*)addr; }
__device__ __forceinline__ gbyte* gptr(const void* p) { return (gbyte*)(uintptr_t)p; }

// 16-byte out-of-bounds fill rows, indexed by TmapImpl::fill_idx.
static __device__ __attribute__((aligned(16))) const uint32_t g_fill_rows[5][4] = {
    {0u, 0u, 0u, 0u},
    {0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u},   // f32 quiet NaN
    {0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u},   // f16 quiet NaN
    {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u},   // bf16 quiet NaN
    {0x00000000u, 0x7FF80000u, 0x00000000u, 0x7FF80000u},   // f64 quiet NaN
};

__device__ __forceinline__ uint32_t lane_id() { return __lane_id(); }

// A copy of a struct that is the same for the whole wave (a kernel
// argument), read as aligned 32-bit words into scalar registers.  Reading
// its one- and two-byte fields where they lie takes vector-memory loads
// (there are no sub-word scalar loads): for a kernel argument, a memory
// round trip at the start of every workgroup, before its first copy.  Words
// the caller never uses are dropped by the compiler.
template <typename T>
__device__ __forceinline__ T uniform_copy(const T& x) {
    static_assert(sizeof(T) % 4 == 0 && alignof(T) >= 4, "whole 32-bit words");
    union {
        uint32_t u[sizeof(T) / 4];
        T t;
    } r;
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&x);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) r.u[i] = __builtin_amdgcn_readfirstlane(w[i]);
    return r.t;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, uint32_t magic) {
    return magic ? __umulhi(n, magic) : n;
}

// Physical <-> logical 16-byte chunk inside a box image.  The low (sw & 3)
// chunk bits (3 for 128B, 2 for 64B, 1 for 32B, 0 for NONE) are XORed with
// the 128-byte unit index (chunk bits 3..), or with the 256-byte unit index
// (chunk bits 4..) for the _K256 modes.
__device__ __forceinline__ uint32_t swz_chunk(uint32_t c, uint32_t sw) {
    return c ^ ((c >> (3u + ((sw >> 2) & 1u))) & ((1u << (sw & 3u)) - 1u));
}

// Box coordinates of logical chunk q: k[0] is the first element's index in
// dimension 0, k[1..4] the LDS row's coordinates.
__device__ __forceinline__ void chunk_box_coords(const TmapImpl& m, uint32_t q, uint32_t k[5]) {
    const uint32_t row = fdiv(q, m.magic_cpr);
    const uint32_t j = q - row * m.cpr;
    k[0] = j * (16u / m.esize);
    const uint32_t r1 = fdiv(row, m.magic_L[0]);
    k[1] = row - r1 * m.L[1];
    const uint32_t r2 = fdiv(r1, m.magic_L[1]);
    k[2] = r1 - r2 * m.L[2];
    const uint32_t r3 = fdiv(r2, m.magic_L[2]);
    k[3] = r2 - r3 * m.L[3];
    k[4] = r3;
}

// Byte offset of the box element k (k[0] along dim 0) from the box origin's
// address (origin given separately), and whether dims 1..4 are in range.
struct ChunkLoc {
    int64_t g0;        // global index of the chunk's first element in dim 0
    int64_t rest_off;  // sum over dims >= 1 of g_i * stride_i (bytes)
    bool rest_in;      // dims >= 1 inside the tensor
};

__device__ __forceinline__ ChunkLoc chunk_locate(const TmapImpl& m, const int32_t c[5], uint32_t q) {
    uint32_t k[5];
    chunk_box_coords(m, q, k);
    ChunkLoc r;
    r.g0 = (int64_t)c[0] + (int64_t)k[0] * m.es[0];
    r.rest_off = 0;
    r.rest_in = true;
#pragma unroll
    for (int d = 1; d < 5; ++d) {
        const int64_t g = (int64_t)c[d] + (int64_t)k[d] * m.es[d];
        r.rest_in = r.rest_in && (g >= 0) && (g < m.dim[d]);
        r.rest_off += g * (int64_t)m.stride[d - 1];
    }
    return r;
}

// chunk_locate for maps of rank 1 or 2 (dims 2..4 of extent 1, coordinate 0):
// the row of the LDS image is the box coordinate in dim 1.
__device__ __forceinline__ ChunkLoc chunk_locate_2d(const TmapImpl& m, const int32_t c[5], uint32_t q) {
    const uint32_t row = fdiv(q, m.magic_cpr);
    const uint32_t j = q - row * m.cpr;
    ChunkLoc r;
    r.g0 = (int64_t)c[0] + (int64_t)(j * (16u / m.esize)) * m.es[0];
    const int64_t g1 = (int64_t)c[1] + (int64_t)row * m.es[1];
    r.rest_in = g1 >= 0 && g1 < m.dim[1];
    r.rest_off = g1 * (int64_t)m.stride[0];
    return r;
}

// Gather one 16-byte chunk element by element (element stride in dim 0,
// unaligned origin, or a chunk cut by the tensor edge).  Out-of-range
// elements take the fill pattern and are never read.
template <typename T>
__device__ __forceinline__ u32x4 gather_chunk_t(const TmapImpl& m, const ChunkLoc& L) {
    constexpr int N = 16 / (int)sizeof(T);
    union { u32x4 v; T e[N]; } u;
    const T fillv = *reinterpret_cast<const T*>(g_fill_rows[m.fill_idx]);
    const ATT_GLOBAL T* row = (const ATT_GLOBAL T*)gptr(m.base + (uint64_t)L.rest_off);
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const int64_t g = L.g0 + (int64_t)e * m.es[0];
        const bool in = L.rest_in && g >= 0 && g < m.dim[0];
        u.e[e] = in ? row[g] : fillv;
    }
    return u.v;
}

__device__ __forceinline__ u32x4 gather_chunk(const TmapImpl& m, const ChunkLoc& L) {
    switch (m.esize) {
    case 1: return gather_chunk_t<uint8_t>(m, L);
    case 2: return gather_chunk_t<uint16_t>(m, L);
    case 4: return gather_chunk_t<uint32_t>(m, L);
    default: return gather_chunk_t<uint64_t>(m, L);
    }
}

// One async 16-byte global->LDS copy per active lane; `lds_group` is the
// wave-uniform LDS address of lane 0's slot.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_group) {
    __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)lds_group, 16, 0, 0);
}

// The same 16-byte copy with a wave-uniform 64-bit base (SGPRs), a per-lane
// 32-bit offset and the LDS group address in M0, issued as inline asm so the
// compiler's LDS alias tracking does not see it: the caller orders it against
// LDS reads with its own vmcnt waits and barriers.
// The compiler's hazard recogniser does not look inside inline asm, so the
// asm provides its own wait states: a vector-memory instruction must come at
// least five wait states after a VALU instruction that wrote one of the
// SGPRs it reads (here the base, which the compiler may produce with
// v_readfirstlane), and an LDS-DMA one after the write of M0.  s_nop 4 gives
// five, whatever the compiler placed just before the asm.
__device__ __forceinline__ void dma16_sv(uint64_t sbase, uint32_t voff, uint32_t lds_group_addr) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(voff), "s"(sbase), "{m0}"(lds_group_addr)
                 : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Retire the copies of the stage about to be read when `later` stages of
// PER DMA instructions each were issued after it.  Loads complete in issue
// order, so vmcnt <= later * PER means that stage has landed in LDS.
template <int PER, int K>
__device__ __forceinline__ void wait_stage(uint32_t later) {
    if constexpr (K > 0) {
        if (later >= (uint32_t)K) {
            wait_vmcnt<K * PER>();
            return;
        }
        wait_stage<PER, K - 1>(later);
    } else {
        wait_vmcnt<0>();
    }
}

// Workgroup barrier that also stops the compiler from moving memory
// accesses across it (the raw s_barrier builtin alone does not).
__device__ __forceinline__ void wg_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// ds_read_b128 issued as inline asm: the compiler's own LDS-DMA alias
// tracking would otherwise put vmcnt(0) in front of every LDS read and
// serialise the staging ring.  The caller waits lgkmcnt before use.
__device__ __forceinline__ u32x4 lds_read16(uint32_t lds_addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr) : "memory");
    return v;
}

// The same read with a compile-time byte offset in the instruction's
// immediate field (no address arithmetic at the call site).
template <uint32_t OFF>
__device__ __forceinline__ u32x4 lds_read16_off(uint32_t lds_addr) {
    static_assert(OFF < 65536u, "ds_read offset field is 16 bits");
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(lds_addr), "n"(OFF) : "memory");
    return v;
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

// Load one box into LDS image `lds` (this wave's share of the 64-chunk
// groups grp = wave, wave + nwaves, ...).  Returns the bytes this wave wrote
// to LDS; they have landed once the wave has waited vmcnt(0) and lgkmcnt(0).
//
// Fast path (dim-0 element stride 1 and a 16-byte-aligned dim-0 origin, so
// every chunk is one aligned 16-byte global read): in-range chunks and
// wholly out-of-range chunks (redirected to the fill row) go through
// global_load_lds; chunks cut by the dim-0 edge are gathered per element and
// written with ds_write_b128 by their lane, which sits out the DMA.
__device__ __forceinline__ uint32_t tile_load_issue(const TmapImpl& m, const int32_t c[5], uint8_t* lds,
                                                    uint32_t wave, uint32_t nwaves) {
    const uint32_t lane = lane_id();
    const uint32_t nchunk = m.box_bytes >> 4;
    const bool fast = (m.es[0] == 1) && ((((int64_t)c[0] * m.esize) & 15) == 0);
    const int64_t n_el = 16 / m.esize;
    const void* fill = g_fill_rows[m.fill_idx];
    uint32_t bytes = 0;
    for (uint32_t grp = wave; grp * 64u < nchunk; grp += nwaves) {
        const uint32_t p = grp * 64u + lane;
        const bool active = p < nchunk;
        const uint32_t rem = nchunk - grp * 64u;
        bytes += 16u * (rem < 64u ? rem : 64u);
        const uint32_t q = swz_chunk(p, m.swizzle);
        const ChunkLoc L = chunk_locate(m, c, active ? q : 0u);
        bool partial = !fast;
        const void* src = fill;
        if (fast) {
            const bool full_in = L.rest_in && L.g0 >= 0 && L.g0 + n_el <= m.dim[0];
            const bool full_out = !L.rest_in || L.g0 >= m.dim[0] || L.g0 + n_el <= 0;
            partial = !full_in && !full_out;
            if (full_in) src = (const void*)(uintptr_t)(m.base + (uint64_t)(L.g0 * m.esize + L.rest_off));
        }
        if (active && !partial) dma16(src, lds + grp * 1024u);
        if (active && partial) {
            const u32x4 v = gather_chunk(m, L);
            *reinterpret_cast<u32x4*>(lds + p * 16u) = v;
        }
    }
    return bytes;
}

// ---- reduce-add element helpers ------------------------------------------

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// 8- and 16-bit lanes of a 32-bit word updated with compare-and-swap.  The
// aligned word never leaves the page that holds the element.
template <typename F>
__device__ __forceinline__ void cas_update_sub(gbyte* addr, int bits, F f) {
    const uint64_t a = (uint64_t)(uintptr_t)addr;
    ATT_GLOBAL uint32_t* w = (ATT_GLOBAL uint32_t*)(a & ~(uint64_t)3);
    const uint32_t shift = (uint32_t)(a & 3u) * 8u;
    const uint32_t mask = (bits == 8 ? 0xFFu : 0xFFFFu) << shift;
    uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (true) {
        const uint32_t cur = (old & mask) >> shift;
        const uint32_t nw = (old & ~mask) | ((f(cur) << shift) & mask);
        if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            break;
    }
}

template <typename T>
__device__ __forceinline__ void atomic_add_g(gbyte* dst, T v) {
    __hip_atomic_fetch_add((ATT_GLOBAL T*)dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// IEEE addition of a 4- or 8-byte float `bits` into global memory, rounded
// to nearest even.  The hardware float atomic rounds that way, but an L2
// adder may treat subnormal operands or results as zero.  That can change
// the sum only when the added value is zero, not finite, or tiny: for
// |v| >= 2^(emin + p + 2) (exponent field >= p + 3, p the significand bits)
// a subnormal other operand is below a quarter ulp of v, so the correctly
// rounded sum is v either way, and a cancellation cannot end in the
// subnormal range (both operands are then multiples of 2^(emin + 2)).  Those
// values take the hardware atomic; the rest a compare-and-swap loop whose
// sum the VALU forms with subnormals kept.  A NaN result is a quiet NaN
// whose payload is not fixed (IEEE 754 leaves it open).
template <typename F, typename U>
__device__ __forceinline__ void float_add_atomic(gbyte* dst, U bits) {
    constexpr int MB = sizeof(F) == 4 ? 23 : 52;              // stored significand bits
    constexpr U EMAX = sizeof(F) == 4 ? 0xFFu : 0x7FFu;        // exponent field of inf / NaN
    const U e = (bits >> MB) & EMAX;
    if (e >= (U)(MB + 4) && e < EMAX) {
        __hip_atomic_fetch_add((ATT_GLOBAL F*)dst, __builtin_bit_cast(F, bits), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    ATT_GLOBAL U* w = (ATT_GLOBAL U*)dst;
    U old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (true) {
        const U nw = __builtin_bit_cast(U, __builtin_bit_cast(F, old) + __builtin_bit_cast(F, bits));
        if (nw == old) return;
        if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

// Element `bits` (the low esize bytes hold it) added into dst.
__device__ __forceinline__ void reduce_add_element(uint8_t dtype, gbyte* dst, uint64_t bits) {
    switch (dtype) {
    case TMAP_U32: case TMAP_I32:
        atomic_add_g<uint32_t>(dst, (uint32_t)bits);
        break;
    case TMAP_U64: case TMAP_I64:
        atomic_add_g<uint64_t>(dst, bits);
        break;
    case TMAP_F32:
        float_add_atomic<float, uint32_t>(dst, (uint32_t)bits);
        break;
    case TMAP_F64:
        float_add_atomic<double, uint64_t>(dst, bits);
        break;
    case TMAP_U8: {
        const uint32_t v = (uint32_t)bits & 0xFFu;
        cas_update_sub(dst, 8, [v](uint32_t cur) { return (cur + v) & 0xFFu; });
        break;
    }
    case TMAP_U16: {
        const uint32_t v = (uint32_t)bits & 0xFFFFu;
        cas_update_sub(dst, 16, [v](uint32_t cur) { return (cur + v) & 0xFFFFu; });
        break;
    }
    case TMAP_BF16: {
        const float v = bf16_to_f32((uint16_t)bits);
        cas_update_sub(dst, 16, [v](uint32_t cur) {
            return (uint32_t)f32_to_bf16_rne(bf16_to_f32((uint16_t)cur) + v);
        });
        break;
    }
    case TMAP_F16: {
        const float v = (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
        cas_update_sub(dst, 16, [v](uint32_t cur) {
            const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)cur) + v;
            return s != s ? 0x7E00u : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)s);
        });
        break;
    }
    default: break;
    }
}

// What a box store does with each in-bounds element.
enum : int { ST_STORE = 0, ST_ADD = 1, ST_MIN = 2, ST_MAX = 3 };

// min / max of two floating-point values given as raw bits ([HPC] "TMA
// reduce" names add and min; the readings): a NaN operand yields the other,
// two NaNs the canonical quiet NaN, -0 orders below +0, and the winner's
// bits are returned unchanged.  F is float (f32, or f16 / bf16 widened
// exactly) or double.
template <bool MAX, typename F>
__device__ __forceinline__ bool float_take_new(F cur, F v) {
    const bool nc = cur != cur, nv = v != v;
    if (nv) return false;
    if (nc) return true;
    const bool v_less = v < cur || (v == cur && v == F(0) && __builtin_signbit(v) && !__builtin_signbit(cur));
    const bool c_less = cur < v || (v == cur && v == F(0) && __builtin_signbit(cur) && !__builtin_signbit(v));
    return MAX ? c_less : v_less;
}

__device__ __forceinline__ float half_bits_to_f32(uint8_t dtype, uint32_t h) {
    return dtype == TMAP_BF16 ? __builtin_bit_cast(float, h << 16)
                              : (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// New bits of a min / max update of `cur` by `v` (both raw, esize bytes).
template <bool MAX>
__device__ __forceinline__ uint64_t minmax_bits(uint8_t dtype, uint64_t cur, uint64_t v) {
    switch (dtype) {
    case TMAP_F32: {
        const float a = __builtin_bit_cast(float, (uint32_t)cur), b = __builtin_bit_cast(float, (uint32_t)v);
        if (a != a && b != b) return 0x7FC00000u;
        return float_take_new<MAX>(a, b) ? v : cur;
    }
    case TMAP_F64: {
        const double a = __builtin_bit_cast(double, cur), b = __builtin_bit_cast(double, v);
        if (a != a && b != b) return 0x7FF8000000000000ull;
        return float_take_new<MAX>(a, b) ? v : cur;
    }
    case TMAP_F16: case TMAP_BF16: {
        const float a = half_bits_to_f32(dtype, (uint32_t)cur), b = half_bits_to_f32(dtype, (uint32_t)v);
        if (a != a && b != b) return dtype == TMAP_BF16 ? 0x7FC0u : 0x7E00u;
        return float_take_new<MAX>(a, b) ? v : cur;
    }
    case TMAP_U8: case TMAP_U16: case TMAP_U32: case TMAP_U64:
        return MAX ? (v > cur ? v : cur) : (v < cur ? v : cur);
    case TMAP_I32: {
        const int32_t a = (int32_t)(uint32_t)cur, b = (int32_t)(uint32_t)v;
        return (MAX ? b > a : b < a) ? v : cur;
    }
    default: {   // TMAP_I64
        const int64_t a = (int64_t)cur, b = (int64_t)v;
        return (MAX ? b > a : b < a) ? v : cur;
    }
    }
}

// Atomic min / max of element `bits` into dst: hardware integer min / max
// for 32- and 64-bit integers, compare-and-swap otherwise.  A value that
// would not change memory is not written (min only lowers and max only
// raises the stored value in the order above, so it never would later).
template <bool MAX>
__device__ __forceinline__ void reduce_minmax_element(uint8_t dtype, gbyte* dst, uint64_t bits) {
    switch (dtype) {
    case TMAP_I32:
        if (MAX) __hip_atomic_fetch_max((ATT_GLOBAL int32_t*)dst, (int32_t)(uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_fetch_min((ATT_GLOBAL int32_t*)dst, (int32_t)(uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    case TMAP_U32:
        if (MAX) __hip_atomic_fetch_max((ATT_GLOBAL uint32_t*)dst, (uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_fetch_min((ATT_GLOBAL uint32_t*)dst, (uint32_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    case TMAP_I64:
        if (MAX) __hip_atomic_fetch_max((ATT_GLOBAL int64_t*)dst, (int64_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_fetch_min((ATT_GLOBAL int64_t*)dst, (int64_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    case TMAP_U64:
        if (MAX) __hip_atomic_fetch_max((ATT_GLOBAL uint64_t*)dst, (uint64_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_fetch_min((ATT_GLOBAL uint64_t*)dst, (uint64_t)bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    case TMAP_F32: {
        ATT_GLOBAL uint32_t* w = (ATT_GLOBAL uint32_t*)dst;
        uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (true) {
            const uint32_t nw = (uint32_t)minmax_bits<MAX>(dtype, old, bits);
            if (nw == old) return;
            if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                return;
        }
    }
    case TMAP_F64: {
        ATT_GLOBAL uint64_t* w = (ATT_GLOBAL uint64_t*)dst;
        uint64_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (true) {
            const uint64_t nw = minmax_bits<MAX>(dtype, old, bits);
            if (nw == old) return;
            if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT))
                return;
        }
    }
    case TMAP_U8:
        cas_update_sub(dst, 8, [dtype, bits](uint32_t cur) { return (uint32_t)minmax_bits<MAX>(dtype, cur, bits & 0xFFu); });
        return;
    default:   // U16, F16, BF16
        cas_update_sub(dst, 16, [dtype, bits](uint32_t cur) { return (uint32_t)minmax_bits<MAX>(dtype, cur, bits & 0xFFFFu); });
        return;
    }
}

// One 8- or 16-bit element of a reduction, raw bits in and out: the same
// arithmetic as reduce_add_element / reduce_minmax_element.
template <int OP>
__device__ __forceinline__ uint32_t reduce_sub_value(uint8_t dtype, uint32_t cur, uint32_t v) {
    if constexpr (OP == ST_ADD) {
        switch (dtype) {
        case TMAP_U8: return (cur + v) & 0xFFu;
        case TMAP_U16: return (cur + v) & 0xFFFFu;
        case TMAP_BF16: return (uint32_t)f32_to_bf16_rne(bf16_to_f32((uint16_t)cur) + bf16_to_f32((uint16_t)v));
        default: {   // F16
            const float sum = (float)__builtin_bit_cast(_Float16, (uint16_t)cur) +
                              (float)__builtin_bit_cast(_Float16, (uint16_t)v);
            return sum != sum ? 0x7E00u : (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sum);
        }
        }
    } else {
        return (uint32_t)minmax_bits<OP == ST_MAX>(dtype, cur, v);
    }
}

// A reduction of the 8- or 16-bit elements of one aligned 32-bit word at
// once (element i of the word takes part if bit i of `inb` is set), by
// compare-and-swap: one atomic per word instead of one per element, and no
// two lanes of an instruction contend for the same word.
template <int OP>
__device__ __forceinline__ void reduce_word(uint8_t dtype, uint32_t esize, ATT_GLOBAL uint32_t* w, uint32_t vw,
                                            uint32_t inb) {
    const uint32_t bits = esize * 8u, epw = 4u / esize;
    const uint32_t em = esize == 1 ? 0xFFu : 0xFFFFu;
    uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (true) {
        uint32_t nw = old;
        for (uint32_t i = 0; i < epw; ++i) {
            if (!((inb >> i) & 1u)) continue;
            const uint32_t sh = i * bits;
            const uint32_t nv = reduce_sub_value<OP>(dtype, (old >> sh) & em, (vw >> sh) & em) & em;
            nw = (nw & ~(em << sh)) | (nv << sh);
        }
        if (nw == old) return;
        if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

// Whether the 16-bit float sum a + b (low halves of the arguments, bf16 or
// f16) is a NaN: an operand is one, or they are infinities of opposite sign.
__device__ __forceinline__ bool half_sum_nan(bool bf, uint32_t a, uint32_t b) {
    const uint32_t inf = bf ? 0x7F80u : 0x7C00u;
    const uint32_t ma = a & 0x7FFFu, mb = b & 0x7FFFu;
    return ma > inf || mb > inf || (ma == inf && mb == inf && ((a ^ b) & 0x8000u));
}

// The halves of the word selected by `halves` (bit 0 low, bit 1 high) that
// hold a NaN become the canonical quiet NaN; the rest of the word is left
// as it is, whatever concurrent updates do to it.
__device__ __forceinline__ void canon_nan_halves(bool bf, ATT_GLOBAL uint32_t* w, uint32_t halves) {
    const uint32_t inf = bf ? 0x7F80u : 0x7C00u, canon = bf ? 0x7FC0u : 0x7E00u;
    uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (true) {
        uint32_t nw = old;
        if ((halves & 1u) && (old & 0x7FFFu) > inf) nw = (nw & 0xFFFF0000u) | canon;
        if ((halves & 2u) && ((old >> 16) & 0x7FFFu) > inf) nw = (nw & 0x0000FFFFu) | (canon << 16);
        if (nw == old) return;
        if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

// The packed adds quiet a signalling NaN and return every other value of a
// half they add -0 to unchanged.  A half outside the box that held a
// signalling NaN `orig` is put back, unless it no longer holds the quieted
// value (another reduction into that element has changed it since, and its
// result stands).
__device__ __forceinline__ bool half_is_snan(bool bf, uint32_t h) {
    return bf ? ((h & 0x7F80u) == 0x7F80u && (h & 0x7Fu) != 0 && !(h & 0x40u))
              : ((h & 0x7C00u) == 0x7C00u && (h & 0x3FFu) != 0 && !(h & 0x200u));
}

__device__ __forceinline__ void restore_half(bool bf, ATT_GLOBAL uint32_t* w, uint32_t shift, uint32_t orig) {
    const uint32_t quieted = orig | (bf ? 0x40u : 0x200u);
    uint32_t old = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (((old >> shift) & 0xFFFFu) == quieted) {
        const uint32_t nw = (old & ~(0xFFFFu << shift)) | (orig << shift);
        if (__hip_atomic_compare_exchange_strong(w, &old, nw, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return;
    }
}

// The esize bytes at byte offset `off` of a 16-byte chunk (off a multiple of
// esize), selected with shifts so that no per-lane array is indexed at run
// time (that would live in scratch memory).
__device__ __forceinline__ uint64_t chunk_element(const u32x4 v, uint32_t off, uint32_t esize) {
    const uint32_t w = off >> 2;
    const uint32_t lo = w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
    if (esize == 8) return ((uint64_t)(w == 0 ? v.y : v.w) << 32) | lo;
    const uint32_t x = lo >> ((off & 3u) * 8u);
    return esize == 4 ? x : (esize == 2 ? (x & 0xFFFFu) : (x & 0xFFu));
}

// Write one box from LDS image `lds` back through the map (inverse swizzle).
// Every in-bounds element of a box image with element stride 1 in dim 0,
// element-major: lane l of a wave takes element l of each run of 64
// consecutive box elements and passes its global address and bits to f, so
// that a wave's accesses to one row fall on consecutive addresses whatever
// the row's alignment.  The rows of rank-1 and rank-2 maps are located with
// one multiply-high per element.
template <typename F>
__device__ __forceinline__ void box_elements(const TmapImpl& m, const int32_t c[5], const uint8_t* lds, uint32_t nchunk,
                                             uint32_t wave, uint32_t nwaves, F&& f) {
    const uint32_t lane = lane_id();
    const uint32_t sh = m.esize == 1 ? 4u : m.esize == 2 ? 3u : m.esize == 4 ? 2u : 1u;   // log2 of elements per chunk
    const uint32_t nel = nchunk << sh;
    const uint32_t rowel = m.cpr << sh;                       // elements per LDS row
    const bool two_d = m.rank <= 2;
    for (uint32_t e0 = wave * 64u; e0 < nel; e0 += nwaves * 64u) {
        const uint32_t E = e0 + lane;
        if (E >= nel) continue;
        const uint32_t q = E >> sh, eo = E & ((1u << sh) - 1u);
        int64_t g, rest_off;
        if (two_d) {
            const uint32_t row = fdiv(q, m.magic_cpr);
            g = (int64_t)c[0] + (int64_t)(E - row * rowel);
            const int64_t g1 = (int64_t)c[1] + (int64_t)row * m.es[1];
            if (g1 < 0 || g1 >= m.dim[1]) continue;
            rest_off = g1 * (int64_t)m.stride[0];
        } else {
            const ChunkLoc L = chunk_locate(m, c, q);
            if (!L.rest_in) continue;
            g = L.g0 + (int64_t)eo;
            rest_off = L.rest_off;
        }
        if (g < 0 || g >= m.dim[0]) continue;
        const uint8_t* src = lds + swz_chunk(q, m.swizzle) * 16u + (eo << (4u - sh));
        const uint64_t bits = sh == 4u ? (uint64_t)*src
                            : sh == 3u ? (uint64_t)*reinterpret_cast<const uint16_t*>(src)
                            : sh == 2u ? (uint64_t)*reinterpret_cast<const uint32_t*>(src)
                                       : *reinterpret_cast<const uint64_t*>(src);
        f(gptr(m.base + (uint64_t)rest_off) + g * m.esize, bits);
    }
}

// Reductions on 8- and 16-bit elements with element stride 1 in dim 0:
// lane l takes one aligned 32-bit word of global memory, so that one atomic
// updates all its elements.  A box row of L0 elements starting at c0 touches
// words floor(c0 / EPW) .. floor((c0 + L0 - 1) / EPW); with an origin that is
// not word-aligned a word's elements come from two neighbouring box
// elements, read from LDS one by one.  Elements past either end of the box
// row or of dim 0 are left alone.  For maps of rank 1 or 2 the rows and
// elements inside the tensor are worked out once per box, so a word costs a
// multiply-high and a few 32-bit operations; higher ranks locate each
// word's row with chunk_locate.
template <int OP, uint32_t ESZ, bool TWO_D>
__device__ __forceinline__ void reduce_words(const TmapImpl& m, const int32_t c[5], const uint8_t* lds,
                                             uint32_t nchunk, uint32_t wave, uint32_t nwaves) {
    constexpr uint32_t EPW = 4u / ESZ;                          // elements per word
    const uint32_t lane = lane_id();
    const uint32_t L0 = m.L[0], cpr = m.cpr;
    const int64_t c0 = c[0];
    const int64_t w_first = c0 >= 0 ? c0 / EPW : -((-c0 + EPW - 1) / EPW);
    const uint32_t head = (uint32_t)(c0 - w_first * (int64_t)EPW);     // 0 .. EPW-1
    const uint32_t wpr = (head + L0 + EPW - 1u) / EPW;                 // words per box row
    const uint32_t nrow = fdiv(nchunk, m.magic_cpr);
    const uint32_t nwd = nrow * wpr;
    // ceil(2^32 / wpr) for fdiv, from 32-bit arithmetic (a 64-bit division
    // here is a long software routine run by every wave)
    const uint32_t magic_wpr = wpr == 1u ? 0u : 0xFFFFFFFFu / wpr + 1u;
    // box elements of a row inside dim 0: [e_lo, e_hi)
    const int64_t elo = c0 < 0 ? (-c0 < (int64_t)L0 ? -c0 : (int64_t)L0) : 0;
    int64_t ehi = m.dim[0] - c0;
    if (ehi > (int64_t)L0) ehi = L0;
    if (ehi < elo) ehi = elo;
    const int32_t e_lo = (int32_t)elo, e_hi = (int32_t)ehi;
    // rank <= 2: image rows inside dim 1, [r_lo, r_hi), and row r's address
    uint32_t r_lo = 0, r_hi = nrow;
    int64_t rb0 = 0, rstep = 0;
    if constexpr (TWO_D) {
        // row r is inside iff 0 <= c1 + r * es1 < dim1; 32-bit divisions
        // only, the upper bound clamped to the image first
        const int64_t c1 = c[1];
        const uint32_t es1 = m.es[1];
        const int64_t below = c1 < 0 ? -c1 : 0;                       // rows needed to reach 0
        const uint64_t lo = below >= (int64_t)nrow * es1 ? nrow : ((uint32_t)below + es1 - 1u) / es1;
        const int64_t avail = m.dim[1] - c1;                          // coordinates left in dim 1
        const uint64_t hi = avail <= 0 ? 0u
                          : (avail >= (int64_t)nrow * es1 ? nrow : ((uint32_t)avail + es1 - 1u) / es1);
        r_hi = (uint32_t)hi;
        r_lo = (uint32_t)(lo < hi ? lo : hi);
        rb0 = (int64_t)m.base + c1 * (int64_t)m.stride[0] + w_first * 4;
        rstep = (int64_t)es1 * (int64_t)m.stride[0];
    }
    // Word W of the box image (W < nwd): its address, its box elements
    // packed into a word and which of them the box covers (inb bit h for
    // element h); inb == 0 if none is inside.
    auto word_at = [&](uint32_t W, ATT_GLOBAL uint32_t*& wp, uint32_t& vw, uint32_t& inb) {
        if constexpr (TWO_D) {
            // no branch on W: a word past the image or in a row outside the
            // tensor is computed from clamped indices and gets inb == 0
            const uint32_t Wc = W < nwd ? W : nwd - 1u;
            const uint32_t row = fdiv(Wc, magic_wpr), wi = Wc - row * wpr;
            const uint32_t q_row = row * cpr;
            const int32_t e0 = (int32_t)(wi * EPW) - (int32_t)head;    // box element of the word's element 0
            const int32_t lo = e_lo - e0 > 0 ? e_lo - e0 : 0;
            const int32_t hi = e_hi - e0 < (int32_t)EPW ? (e_hi - e0 > 0 ? e_hi - e0 : 0) : (int32_t)EPW;
            const uint32_t span = hi > lo ? ((1u << hi) - 1u) & ~((1u << lo) - 1u) : 0u;
            inb = (W < nwd && row >= r_lo && row < r_hi) ? span : 0u;
            uint32_t keep = 0;
#pragma unroll
            for (uint32_t h = 0; h < EPW; ++h) keep |= ((inb >> h) & 1u) * ((ESZ == 2 ? 0xFFFFu : 0xFFu) << (h * ESZ * 8u));
            if (head == 0) {
                // a word-aligned row: the word's elements sit in one 16-byte chunk
                const uint32_t eb = (uint32_t)e0 * ESZ;
                vw = *reinterpret_cast<const uint32_t*>(lds + swz_chunk(q_row + (eb >> 4), m.swizzle) * 16u + (eb & 15u)) &
                     keep;
            } else {
                uint32_t v = 0;
#pragma unroll
                for (uint32_t h = 0; h < EPW; ++h) {
                    int32_t e = e0 + (int32_t)h;
                    e = e < 0 ? 0 : (e >= (int32_t)L0 ? (int32_t)L0 - 1 : e);
                    const uint32_t eb = (uint32_t)e * ESZ;
                    const uint8_t* src = lds + swz_chunk(q_row + (eb >> 4), m.swizzle) * 16u + (eb & 15u);
                    v |= (ESZ == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(src) : (uint32_t)*src) << (h * ESZ * 8u);
                }
                vw = v & keep;
            }
            wp = (ATT_GLOBAL uint32_t*)gptr((uint64_t)(rb0 + (int64_t)row * rstep + (int64_t)wi * 4));
        } else {
            wp = nullptr;
            vw = 0;
            inb = 0;
            if (W >= nwd) return;
            const uint32_t row = fdiv(W, magic_wpr), wi = W - row * wpr;
            const uint32_t q_row = row * cpr;
            const int32_t e0 = (int32_t)(wi * EPW) - (int32_t)head;
            const ChunkLoc L = chunk_locate(m, c, q_row);
            if (!L.rest_in) return;
#pragma unroll
            for (uint32_t h = 0; h < EPW; ++h) {
                const int32_t e = e0 + (int32_t)h;
                if (e >= e_lo && e < e_hi) inb |= 1u << h;
            }
            if (!inb) return;
#pragma unroll
            for (uint32_t h = 0; h < EPW; ++h) {
                if (!(inb & (1u << h))) continue;
                const uint32_t eb = (uint32_t)(e0 + (int32_t)h) * ESZ;
                const uint8_t* src = lds + swz_chunk(q_row + (eb >> 4), m.swizzle) * 16u + (eb & 15u);
                const uint32_t v = ESZ == 2 ? (uint32_t)*reinterpret_cast<const uint16_t*>(src) : (uint32_t)*src;
                vw |= v << (h * ESZ * 8u);
            }
            wp = (ATT_GLOBAL uint32_t*)gptr((uint64_t)((int64_t)m.base + L.rest_off + (w_first + (int64_t)wi) * 4));
        }
    };
    // WB words per lane per step: their LDS reads, then their atomics, are
    // in flight together (the packed adds return the old value, which is
    // only looked at after all of them have been issued).  Measured on the
    // 4096^2 bf16 pass: two words per lane run 4-6 % faster than four and
    // 20-50 % faster than 8-16 (the returning adds queue at the L2), at 1024
    // to 8192 boxes.
    constexpr uint32_t WB = 2;
    if constexpr (OP == ST_ADD && ESZ == 2) {
        if (m.dtype == TMAP_BF16 || m.dtype == TMAP_F16) {
            // The packed hardware add, which rounds the exact sum once to
            // nearest even like the f32-then-round definition (f32 carries
            // more than 2p + 2 bits); a half outside the box (a word cut by
            // the box row's ends) gets -0 added, which leaves it as it was.
            // A NaN sum keeps an operand's payload or sign there; the old
            // value the add returns tells when that happened, and that half
            // is then set to the canonical NaN.  It also tells whether a half
            // outside the box held a signalling NaN (the add quiets it), to
            // put it back.
            const bool bf = m.dtype == TMAP_BF16;
            for (uint32_t w0 = wave * 64u * WB; w0 < nwd; w0 += nwaves * 64u * WB) {
                ATT_GLOBAL uint32_t* wp[WB];
                uint32_t vw[WB], inb[WB], old[WB];
#pragma unroll
                for (uint32_t b = 0; b < WB; ++b) word_at(w0 + b * 64u + lane, wp[b], vw[b], inb[b]);
#pragma unroll
                for (uint32_t b = 0; b < WB; ++b) {
                    old[b] = 0;
                    if (!inb[b]) continue;
                    const uint32_t v = vw[b] | ((inb[b] & 1u) ? 0u : 0x8000u) | ((inb[b] & 2u) ? 0u : 0x80000000u);
                    old[b] = bf ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_global_atomic_fadd_v2bf16(
                                                                   (ATT_GLOBAL bf16x2_t*)wp[b], __builtin_bit_cast(bf16x2_t, v)))
                                : __builtin_bit_cast(uint32_t, __builtin_amdgcn_global_atomic_fadd_v2f16(
                                                                   (ATT_GLOBAL f16x2_t*)wp[b], __builtin_bit_cast(f16x2_t, v)));
                }
#pragma unroll
                for (uint32_t b = 0; b < WB; ++b) {
                    if (!inb[b]) continue;
                    const uint32_t nan = ((inb[b] & 1u) && half_sum_nan(bf, old[b], vw[b]) ? 1u : 0u) |
                                         ((inb[b] & 2u) && half_sum_nan(bf, old[b] >> 16, vw[b] >> 16) ? 2u : 0u);
                    if (nan) canon_nan_halves(bf, wp[b], nan);
                    if (inb[b] == 1u && half_is_snan(bf, old[b] >> 16)) restore_half(bf, wp[b], 16u, old[b] >> 16);
                    if (inb[b] == 2u && half_is_snan(bf, old[b] & 0xFFFFu)) restore_half(bf, wp[b], 0u, old[b] & 0xFFFFu);
                }
            }
            return;
        }
    }
    for (uint32_t w0 = wave * 64u * WB; w0 < nwd; w0 += nwaves * 64u * WB) {
        ATT_GLOBAL uint32_t* wp[WB];
        uint32_t vw[WB], inb[WB];
#pragma unroll
        for (uint32_t b = 0; b < WB; ++b) word_at(w0 + b * 64u + lane, wp[b], vw[b], inb[b]);
#pragma unroll
        for (uint32_t b = 0; b < WB; ++b)
            if (inb[b]) reduce_word<OP>(m.dtype, ESZ, wp[b], vw[b], inb[b]);
    }
}

// Lane l of group grp handles logical chunk grp*64 + l so that global writes
// are in address order; it reads the chunk's physical LDS slot.  Elements
// outside the tensor are skipped; OP (ST_STORE, ST_ADD, ST_MIN, ST_MAX)
// stores, or combines atomically with what global memory holds; NT makes
// the 16-byte stores non-temporal.  Returns a lower bound of the vector-
// memory instructions this wave issued (the whole-chunk stores; reductions
// and element stores count 0), which store groups use to bound vmcnt.  Every
// LDS read of the call has completed when it returns.
template <int OP, bool NT = false>
__device__ __forceinline__ uint32_t tile_store_issue(const TmapImpl& m, const int32_t c[5], const uint8_t* lds,
                                                     uint32_t wave, uint32_t nwaves) {
    const uint32_t lane = lane_id();
    const uint32_t nchunk = m.box_bytes >> 4;
    if constexpr (OP != ST_STORE) {
        if (m.esize >= 4 && m.es[0] == 1) {
            // Reductions on 4- and 8-byte elements go element-major: lane l
            // of an atomic instruction takes element l of a run of 64
            // consecutive box elements, so one instruction updates whole
            // cache lines instead of one element in each of 64 chunks 16
            // bytes apart (the L2 then merges a line's atomics into one
            // request).  The result is the same: integer and min / max
            // updates commute, and float adds are unordered across boxes
            // anyway.  Each element type gets a loop of its own: with
            // nothing but non-returning atomics in it (integer add, min and
            // max; float add outside its rare compare-and-swap cases), no
            // iteration waits for the previous one's atomics to complete,
            // as one loop holding every type's compare-and-swap paths did.
            if constexpr (OP == ST_ADD) {
                switch (m.dtype) {
                case TMAP_U32: case TMAP_I32:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { atomic_add_g<uint32_t>(dst, (uint32_t)bits); });
                    break;
                case TMAP_U64: case TMAP_I64:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { atomic_add_g<uint64_t>(dst, bits); });
                    break;
                case TMAP_F32:
                    box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* dst, uint64_t bits) {
                        float_add_atomic<float, uint32_t>(dst, (uint32_t)bits);
                    });
                    break;
                default:
                    box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* dst, uint64_t bits) {
                        float_add_atomic<double, uint64_t>(dst, bits);
                    });
                    break;
                }
            } else {
                constexpr bool MX = OP == ST_MAX;
                switch (m.dtype) {
                case TMAP_I32:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { reduce_minmax_element<MX>(TMAP_I32, dst, bits); });
                    break;
                case TMAP_U32:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { reduce_minmax_element<MX>(TMAP_U32, dst, bits); });
                    break;
                case TMAP_I64:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { reduce_minmax_element<MX>(TMAP_I64, dst, bits); });
                    break;
                case TMAP_U64:
                    box_elements(m, c, lds, nchunk, wave, nwaves,
                                 [](gbyte* dst, uint64_t bits) { reduce_minmax_element<MX>(TMAP_U64, dst, bits); });
                    break;
                default:
                    box_elements(m, c, lds, nchunk, wave, nwaves, [&m](gbyte* dst, uint64_t bits) {
                        reduce_minmax_element<MX>(m.dtype, dst, bits);
                    });
                    break;
                }
            }
            wait_lgkm0();
            return 0;
        }
        if (m.es[0] == 1) {
            if (m.esize == 2) {
                if (m.rank <= 2) reduce_words<OP, 2, true>(m, c, lds, nchunk, wave, nwaves);
                else reduce_words<OP, 2, false>(m, c, lds, nchunk, wave, nwaves);
            } else {
                if (m.rank <= 2) reduce_words<OP, 1, true>(m, c, lds, nchunk, wave, nwaves);
                else reduce_words<OP, 1, false>(m, c, lds, nchunk, wave, nwaves);
            }
            wait_lgkm0();
            return 0;
        }
    }
    // A store whose rows do not start on a 16-byte boundary: one element per
    // lane, consecutive lanes on consecutive addresses, rather than a
    // 16-byte chunk per lane written an element at a time.
    if constexpr (OP == ST_STORE) {
        if (m.es[0] == 1 && (((int64_t)c[0] * m.esize) & 15) != 0) {
            switch (m.esize) {
            case 1: box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* d, uint64_t b) { *d = (uint8_t)b; }); break;
            case 2: box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* d, uint64_t b) { *(ATT_GLOBAL uint16_t*)d = (uint16_t)b; }); break;
            case 4: box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* d, uint64_t b) { *(ATT_GLOBAL uint32_t*)d = (uint32_t)b; }); break;
            default: box_elements(m, c, lds, nchunk, wave, nwaves, [](gbyte* d, uint64_t b) { *(ATT_GLOBAL uint64_t*)d = b; }); break;
            }
            wait_lgkm0();
            return 0;
        }
    }
    // Chunk-major: SB of this wave's 64-chunk groups per step, their LDS
    // reads issued together ahead of the writes.
    const bool fast = (m.es[0] == 1) && ((((int64_t)c[0] * m.esize) & 15) == 0);
    const bool two_d = m.rank <= 2;
    const int64_t n_el = 16 / m.esize;
    constexpr uint32_t SB = 4;
    uint32_t issued = 0;
    for (uint32_t g0 = wave; g0 * 64u < nchunk; g0 += SB * nwaves) {
        u32x4 v[SB];
#pragma unroll
        for (uint32_t b = 0; b < SB; ++b) {
            const uint32_t q = (g0 + b * nwaves) * 64u + lane;
            v[b] = q < nchunk ? *reinterpret_cast<const u32x4*>(lds + swz_chunk(q, m.swizzle) * 16u) : u32x4{};
        }
#pragma unroll
        for (uint32_t b = 0; b < SB; ++b) {
            const uint32_t q = (g0 + b * nwaves) * 64u + lane;
            bool whole = false;
            if (q < nchunk) {
                const ChunkLoc L = two_d ? chunk_locate_2d(m, c, q) : chunk_locate(m, c, q);
                if (L.rest_in) {
                    gbyte* rowp = gptr(m.base + (uint64_t)L.rest_off);
                    whole = OP == ST_STORE && fast && L.g0 >= 0 && L.g0 + n_el <= m.dim[0];
                    if (whole) {
                        ATT_GLOBAL u32x4* dst = (ATT_GLOBAL u32x4*)(rowp + L.g0 * m.esize);
                        if constexpr (NT) __builtin_nontemporal_store(v[b], dst);
                        else *dst = v[b];
                    } else {
                        for (int64_t e = 0; e < n_el; ++e) {
                            const int64_t g = L.g0 + e * m.es[0];
                            if (g < 0 || g >= m.dim[0]) continue;
                            gbyte* dst = rowp + g * m.esize;
                            const uint64_t bits = chunk_element(v[b], (uint32_t)e * m.esize, m.esize);
                            if constexpr (OP == ST_ADD) {
                                reduce_add_element(m.dtype, dst, bits);
                            } else if constexpr (OP == ST_MIN || OP == ST_MAX) {
                                reduce_minmax_element<OP == ST_MAX>(m.dtype, dst, bits);
                            } else {
                                switch (m.esize) {
                                case 1: *dst = (uint8_t)bits; break;
                                case 2: *(ATT_GLOBAL uint16_t*)dst = (uint16_t)bits; break;
                                case 4: *(ATT_GLOBAL uint32_t*)dst = (uint32_t)bits; break;
                                default: *(ATT_GLOBAL uint64_t*)dst = bits; break;
                                }
                            }
                        }
                    }
                }
            }
            // one 16-byte store instruction ran if any lane took it
            if constexpr (OP == ST_STORE) issued += __ballot(whole) != 0 ? 1u : 0u;
        }
    }
    wait_lgkm0();
    return issued;
}

// ---- store groups --------------------------------------------------------
// Wait until at most x of this wave's vector-memory instructions are
// outstanding (x clamped to the counter's 63, which only waits longer).
template <int LO, int HI>
__device__ __forceinline__ void wait_vmcnt_range(uint32_t x) {
    if constexpr (LO == HI) {
        wait_vmcnt<LO>();
    } else {
        constexpr int MID = (LO + HI + 1) / 2;
        if (x >= (uint32_t)MID) wait_vmcnt_range<MID, HI>(x);
        else wait_vmcnt_range<LO, MID - 1>(x);
    }
}

__device__ __forceinline__ void wait_vmcnt_le(uint32_t x) { wait_vmcnt_range<0, 63>(x < 63u ? x : 63u); }

// A wave's committed store groups ([HPC] "TMA store": commit_group, then
// wait_group N; [MLC] "waiting for a TMA store").  Held per wave in scalar
// registers: the stores issued since the last commit (`open`) and, newest
// first, the sizes of the last kDepth committed groups, each a lower bound
// of the vector-memory instructions the group issued.  A group's stores have
// completed once the wave has at most as many instructions outstanding as
// it issued after them; stores complete in issue order, and loads issued in
// between only make the wait longer.
struct StoreGroups {
    static constexpr int kDepth = 4;
    uint32_t open;
    uint32_t cnt[kDepth];
};

__device__ __forceinline__ void store_groups_init(StoreGroups& g) {
    g.open = 0;
#pragma unroll
    for (int i = 0; i < StoreGroups::kDepth; ++i) g.cnt[i] = 0;
}

// ---- byte-counted LDS barrier -----------------------------------------------
// state = arrivals_left * 2^32 + pending_bytes (pending signed, |pending| <
// 2^31), so one 64-bit LDS atomic applies an arrival and a byte count
// together and "both zero" is state == 0.  The operation that brings the
// state to zero re-arms the arrival count and flips the phase ([MLC]
// "waiting for TMA load"; [HPC] async completion: a phase needs its arrivals
// and its transaction bytes).
struct TxBar {
    int64_t state;
    uint32_t phase;
    int32_t expected;
};

struct TxState { int32_t arrivals_left; int32_t pending; uint32_t phase; };

__device__ __forceinline__ void txbar_init(TxBar* b, int32_t count) {
    b->state = (int64_t)count << 32;
    b->phase = 0u;
    b->expected = count;
}

// Applies (d_arrivals, d_bytes); returns the state right after this
// operation (phase already flipped if it completed the phase).
__device__ __forceinline__ TxState txbar_op(TxBar* b, int32_t d_arrivals, int32_t d_bytes) {
    const int64_t delta = ((int64_t)d_arrivals << 32) + (int64_t)d_bytes;
    const int64_t old = __hip_atomic_fetch_add(&b->state, delta, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
    const int64_t now = old + delta;
    TxState s;
    if (now == 0) {
        const int32_t exp = __hip_atomic_load(&b->expected, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        __hip_atomic_fetch_add(&b->state, (int64_t)exp << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        const uint32_t ph = __hip_atomic_fetch_xor(&b->phase, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        s.arrivals_left = exp;
        s.pending = 0;
        s.phase = ph ^ 1u;
    } else {
        s.pending = (int32_t)(uint32_t)(uint64_t)now;
        s.arrivals_left = (int32_t)((now - (int64_t)s.pending) >> 32);
        s.phase = __hip_atomic_load(&b->phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    return s;
}

__device__ __forceinline__ TxState txbar_expect_tx(TxBar* b, int32_t bytes) { return txbar_op(b, 0, bytes); }
__device__ __forceinline__ TxState txbar_arrive(TxBar* b, int32_t count) { return txbar_op(b, -count, 0); }
__device__ __forceinline__ TxState txbar_arrive_expect_tx(TxBar* b, int32_t bytes) { return txbar_op(b, -1, bytes); }
__device__ __forceinline__ TxState txbar_complete_tx(TxBar* b, int32_t bytes) { return txbar_op(b, 0, -bytes); }

__device__ __forceinline__ bool txbar_try_wait(TxBar* b, uint32_t parity) {
    return __hip_atomic_load(&b->phase, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) != (parity & 1u);
}

// Bounded wait: returns false if the phase did not complete within
// `max_polls` polls (the caller's data is then not valid), so that a broken
// accounting can never hang the GPU.
__device__ __forceinline__ bool txbar_wait(TxBar* b, uint32_t parity, uint32_t max_polls = 1u << 22) {
    for (uint32_t i = 0; i < max_polls; ++i) {
        if (txbar_try_wait(b, parity)) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

}  // namespace att
