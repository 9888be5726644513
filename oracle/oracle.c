/*
 * oracle.c -- plain CPU reference for descriptor-driven tile movement.
 *
 * TEST INFRASTRUCTURE ONLY: called by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  No blocking,
 * no vectorisation, no shortcuts: each function is the definition written out
 * as nested scalar loops, so that it can be checked against the reference
 * pages by eye.
 *
 * Page keys used in the comments below:
 *   [MLC]  Modern GPU Programming for MLSys (zh), chapter "TMA".
 *   [H200] blog.coolgpu.cn, "H200 // TMA" feature card.
 *   [HPC]  gpu-hpc-book, chapter 08 "Cuda TMA".
 *
 * Parity status per function (what pins it is listed in the test suite):
 *   orc_validate        pinned by [H200] section 03's constraint table.
 *   orc_swizzle 128B    pinned by [MLC] "TMA writes swizzled layout" and
 *                       "3D TMA for several swizzle atoms" worked examples.
 *   orc_swizzle 32B/64B the pages only name the narrower modes ([MLC]
 *                       "grouping requirement" closing paragraph); the key
 *                       is read as the 128-byte unit index, as in that
 *                       section's 256-byte-row formula.  Pinned by that
 *                       section's bank-sector criterion (one 16-byte column
 *                       of an 8-row atom hits 8 distinct sectors; the
 *                       row-index key fails it), the shared key of the rows
 *                       of one 128-byte unit, and the key sequences.
 *   orc_swizzle *_K256  not on the pages (this library's gfx950 modes: the
 *                       key one address bit higher); pinned relative to the
 *                       base modes (key of row r = base key of row r / 2)
 *                       and by 16 distinct sectors of a 64-bank model.
 *   orc_load/store      pinned against an independent NumPy pad-and-slice
 *                       formulation and the worked examples above.
 *   orc_reduce_add      pinned by closed forms (integer wrap, IEEE sums).
 *   orc_reduce_minmax   pinned by NumPy minimum / maximum / fmin / fmax per
 *                       type and hand-listed NaN / signed-zero cases.
 *   orc_im2col_*        the pages only name im2col encoding: the definition is
 *                       a reading, pinned against torch's unfold (1-D and
 *                       2-D convolutions) and a NumPy pad-and-slice 3-D case.
 *   orc_txbar_*         pinned by [MLC] "waiting for TMA load" 4096-byte trace.
 *   orc_bank_sector_*   pinned by [MLC] "128-byte swizzle grouping" counts.
 *   orc_gemm_*          pinned by exact special cases and a library matmul.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

int orc_esize(int dtype)
{
    switch (dtype) {
    case ORC_U8: return 1;
    case ORC_U16: case ORC_F16: case ORC_BF16: return 2;
    case ORC_U32: case ORC_I32: case ORC_F32: return 4;
    case ORC_U64: case ORC_I64: case ORC_F64: return 8;
    default: return 0;
    }
}

static int is_float(int dtype)
{
    return dtype == ORC_F16 || dtype == ORC_BF16 || dtype == ORC_F32 || dtype == ORC_F64;
}

/* LDS extent of one box dimension: every estride-th element of the box is
 * taken, so ceil(box / estride) elements land on chip ([HPC] CUtensorMap
 * field list, elementStrides; read as a traversal stride). */
uint32_t orc_lds_extent(const orc_map* m, int d)
{
    if (d >= m->rank) return 1;
    return (m->box[d] + m->estride[d] - 1) / m->estride[d];
}

uint32_t orc_box_bytes(const orc_map* m)
{
    uint64_t n = (uint64_t)orc_esize(m->dtype);
    for (int d = 0; d < m->rank; ++d) n *= orc_lds_extent(m, d);
    return (uint32_t)n;
}

/* Descriptor constraints, [H200] section 03 table and section 05 list:
 * rank <= 5, boxDim <= 256 per dimension, boxDim[0]*esize a multiple of 16,
 * globalStrides multiples of 16 below 2^40, base 16-byte aligned.  [MLC]
 * "3D TMA" and "grouping requirement": a swizzled box's contiguous extent is
 * at most the atom width and at least the atom width, i.e. equal to it. */
int orc_validate(const orc_map* m)
{
    if (!m) return ORC_ERR_NULL;
    if (m->rank < 1 || m->rank > 5) return ORC_ERR_RANK;
    int es = orc_esize(m->dtype);
    if (es == 0) return ORC_ERR_DTYPE;
    if (m->swizzle < ORC_SW_NONE || m->swizzle > ORC_SW_128B_K256 || m->swizzle == 4) return ORC_ERR_UNSUPPORTED;
    if (m->fill != ORC_FILL_ZERO && m->fill != ORC_FILL_NAN) return ORC_ERR_UNSUPPORTED;
    if (m->base_addr == 0) return ORC_ERR_NULL;
    if (m->base_addr % 16 != 0) return ORC_ERR_ALIGN;
    for (int d = 0; d < m->rank; ++d)
        if (m->dim[d] < 1 || m->dim[d] > (1ull << 32)) return ORC_ERR_DIM;
    for (int d = 1; d < m->rank; ++d) {
        if (m->stride[d] == 0 || m->stride[d] % 16 != 0) return ORC_ERR_STRIDE;
        if (m->stride[d] >= (1ull << 40)) return ORC_ERR_STRIDE;
    }
    for (int d = 0; d < m->rank; ++d)
        if (m->box[d] < 1 || m->box[d] > 256) return ORC_ERR_BOX;
    if (((uint64_t)m->box[0] * (uint64_t)es) % 16 != 0) return ORC_ERR_BOX;
    for (int d = 0; d < m->rank; ++d)
        if (m->estride[d] < 1 || m->estride[d] > 8) return ORC_ERR_ESTRIDE;
    uint32_t row_bytes = orc_lds_extent(m, 0) * (uint32_t)es;
    if (row_bytes % 16 != 0) return ORC_ERR_ESTRIDE;
    if (m->swizzle != ORC_SW_NONE) {
        uint32_t span = 16u << (m->swizzle & 3);   /* 32, 64, 128 bytes */
        if (row_bytes != span) return ORC_ERR_SWIZZLE_WIDTH;
    }
    if (m->fill == ORC_FILL_NAN && !is_float(m->dtype)) return ORC_ERR_OOB_FILL_DTYPE;
    uint64_t bytes = (uint64_t)es;
    for (int d = 0; d < m->rank; ++d) bytes *= orc_lds_extent(m, d);
    if (bytes > ORC_LDS_CAPACITY) return ORC_ERR_LDS_CAPACITY;
    return ORC_OK;
}

/* Swizzle on the LDS byte offset.  [MLC] "TMA writes swizzled layout": with
 * 128-byte rows, the 16-byte sector `col` of row `row` lands at sector
 * col XOR row, repeating every 8 rows (one 8 x 128-byte atom).  Written on
 * the byte offset: bits 4..6 (sector within a 128-byte unit) are XORed with
 * bits 7..9 (the 128-byte unit index modulo 8).  For 64- and 32-byte spans
 * only the low 2 or 1 sector bits take part. */
uint32_t orc_swizzle(uint32_t off, int swizzle)
{
    if (swizzle == ORC_SW_NONE) return off;
    uint32_t nbits = (uint32_t)(swizzle & 3);     /* 1, 2, 3 */
    uint32_t mask = (1u << nbits) - 1u;
    uint32_t shift = (swizzle & 4) ? 8u : 7u;     /* 256- or 128-byte unit */
    uint32_t unit = (off >> shift) & mask;
    return off ^ (unit << 4);
}

static void fill_bits(int dtype, int fill, uint8_t* out)
{
    int es = orc_esize(dtype);
    memset(out, 0, (size_t)es);
    if (fill != ORC_FILL_NAN) return;
    /* canonical quiet NaN of each float type, little-endian */
    if (dtype == ORC_F32) { uint32_t v = 0x7FC00000u; memcpy(out, &v, 4); }
    if (dtype == ORC_F64) { uint64_t v = 0x7FF8000000000000ull; memcpy(out, &v, 8); }
    if (dtype == ORC_F16) { uint16_t v = 0x7E00u; memcpy(out, &v, 2); }
    if (dtype == ORC_BF16) { uint16_t v = 0x7FC0u; memcpy(out, &v, 2); }
}

/* One element of the box: its LDS linear index (innermost fastest) and, when
 * every coordinate is inside the tensor, its byte offset from base. */
static int element_address(const orc_map* m, const int32_t* coords, const uint32_t* k,
                           uint64_t* lin_out, uint64_t* byte_off_out)
{
    int es = orc_esize(m->dtype);
    uint64_t lin = 0;
    for (int d = m->rank - 1; d >= 0; --d)
        lin = lin * orc_lds_extent(m, d) + k[d];
    *lin_out = lin;

    int inb = 1;
    uint64_t off = 0;
    for (int d = 0; d < m->rank; ++d) {
        int64_t g = (int64_t)coords[d] + (int64_t)k[d] * (int64_t)m->estride[d];
        if (g < 0 || (uint64_t)g >= m->dim[d]) { inb = 0; continue; }
        if (d == 0) off += (uint64_t)g * (uint64_t)es;
        else off += (uint64_t)g * m->stride[d];
    }
    *byte_off_out = off;
    return inb;
}

/* Advance the 5-digit box counter k (innermost fastest); returns 0 at end. */
static int next_k(const orc_map* m, uint32_t* k)
{
    for (int d = 0; d < m->rank; ++d) {
        if (++k[d] < orc_lds_extent(m, d)) return 1;
        k[d] = 0;
    }
    return 0;
}

/* Load, [MLC] "one thread describes the whole tile" and "TMA writes swizzled
 * layout"; out-of-range elements take the fill pattern ([H200] section 02
 * table, last row).  The element's bits are copied untouched. */
void orc_load(const orc_map* m, const uint8_t* gmem, const int32_t* coords, uint8_t* lds)
{
    int es = orc_esize(m->dtype);
    uint8_t fill[8];
    fill_bits(m->dtype, m->fill, fill);
    uint32_t k[5] = {0, 0, 0, 0, 0};
    do {
        uint64_t lin, off;
        int inb = element_address(m, coords, k, &lin, &off);
        uint32_t phys = orc_swizzle((uint32_t)(lin * (uint64_t)es), m->swizzle);
        if (inb) memcpy(lds + phys, gmem + off, (size_t)es);
        else memcpy(lds + phys, fill, (size_t)es);
    } while (next_k(m, k));
}

/* ---- im2col mode ------------------------------------------------------------
 * (see oracle.h for the reading).  Window origins along spatial dimension s
 * form a grid of n_s positions; a pixel's position is a mixed-radix number
 * (W digit fastest, image index last) counted from the load's start. */

static int64_t floor_div(int64_t a, int64_t b)
{
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

/* The same floor division on 128-bit integers: a window's linear index is a
 * mixed-radix number whose digits may each be close to 2^32, so it is kept
 * exact at any tensor size. */
static __int128 floor_div128(__int128 a, __int128 b)
{
    __int128 q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

static int64_t im2col_positions(const orc_im2col* m, int s)
{
    int64_t lo = m->lower[s];
    int64_t hi = (int64_t)m->t.dim[s + 1] - 1 + (int64_t)m->upper[s];
    if (hi < lo) return 0;
    return (hi - lo) / (int64_t)m->t.estride[s + 1] + 1;
}

int orc_im2col_validate(const orc_im2col* m)
{
    if (!m) return ORC_ERR_NULL;
    const orc_map* t = &m->t;
    if (t->rank < 3 || t->rank > 5) return ORC_ERR_RANK;
    int es = orc_esize(t->dtype);
    if (es == 0) return ORC_ERR_DTYPE;
    if (t->swizzle < ORC_SW_NONE || t->swizzle > ORC_SW_128B_K256 || t->swizzle == 4) return ORC_ERR_UNSUPPORTED;
    if (t->fill != ORC_FILL_ZERO && t->fill != ORC_FILL_NAN) return ORC_ERR_UNSUPPORTED;
    if (t->base_addr == 0) return ORC_ERR_NULL;
    if (t->base_addr % 16 != 0) return ORC_ERR_ALIGN;
    for (int d = 0; d < t->rank; ++d)
        if (t->dim[d] < 1 || t->dim[d] > (1ull << 32)) return ORC_ERR_DIM;
    for (int d = 1; d < t->rank; ++d)
        if (t->stride[d] == 0 || t->stride[d] % 16 != 0 || t->stride[d] >= (1ull << 40)) return ORC_ERR_STRIDE;
    if (m->channels < 1 || m->channels > 256) return ORC_ERR_BOX;
    if (((uint64_t)m->channels * (uint64_t)es) % 16 != 0) return ORC_ERR_BOX;
    if (m->pixels < 1 || m->pixels > 1024) return ORC_ERR_BOX;
    if (t->estride[0] != 1 || t->estride[t->rank - 1] != 1) return ORC_ERR_ESTRIDE;
    for (int d = 1; d < t->rank - 1; ++d)
        if (t->estride[d] < 1 || t->estride[d] > 8) return ORC_ERR_ESTRIDE;
    for (int s = 0; s < t->rank - 2; ++s) {
        if (m->lower[s] < -32768 || m->lower[s] > 32767) return ORC_ERR_BOX;
        if (m->upper[s] < -32768 || m->upper[s] > 32767) return ORC_ERR_BOX;
        if (im2col_positions(m, s) < 1) return ORC_ERR_BOX;
    }
    uint32_t row_bytes = m->channels * (uint32_t)es;
    if (t->swizzle != ORC_SW_NONE && row_bytes != (16u << (t->swizzle & 3))) return ORC_ERR_SWIZZLE_WIDTH;
    if (t->fill == ORC_FILL_NAN && !is_float(t->dtype)) return ORC_ERR_OOB_FILL_DTYPE;
    if ((uint64_t)row_bytes * m->pixels > ORC_LDS_CAPACITY) return ORC_ERR_LDS_CAPACITY;
    return ORC_OK;
}

uint32_t orc_im2col_box_bytes(const orc_im2col* m)
{
    return m->pixels * m->channels * (uint32_t)orc_esize(m->t.dtype);
}

void orc_im2col_load(const orc_im2col* m, const uint8_t* gmem, const int32_t* coords,
                     const int32_t* offsets, uint8_t* lds)
{
    const orc_map* t = &m->t;
    int es = orc_esize(t->dtype);
    int S = t->rank - 2;
    uint8_t fill[8];
    fill_bits(t->dtype, t->fill, fill);
    int64_t npos[3];
    for (int s = 0; s < S; ++s) npos[s] = im2col_positions(m, s);
    /* linear index of the start: image index is the most significant digit */
    __int128 L0 = coords[t->rank - 1];
    for (int s = S - 1; s >= 0; --s)
        L0 = L0 * npos[s] + floor_div((int64_t)coords[s + 1] - m->lower[s], (int64_t)t->estride[s + 1]);
    for (uint32_t p = 0; p < m->pixels; ++p) {
        __int128 L = L0 + (__int128)p;
        int64_t x[3];
        for (int s = 0; s < S; ++s) {
            __int128 q = floor_div128(L, npos[s]);
            int64_t digit = (int64_t)(L - q * npos[s]);
            x[s] = (int64_t)m->lower[s] + digit * (int64_t)t->estride[s + 1] + (int64_t)offsets[s];
            L = q;
        }
        __int128 img = L;
        int inb_pix = img >= 0 && img < (__int128)t->dim[t->rank - 1];
        uint64_t pix_off = inb_pix ? (uint64_t)img * t->stride[t->rank - 1] : 0;
        for (int s = 0; s < S; ++s) {
            if (x[s] < 0 || (uint64_t)x[s] >= t->dim[s + 1]) inb_pix = 0;
            else pix_off += (uint64_t)x[s] * t->stride[s + 1];
        }
        for (uint32_t k = 0; k < m->channels; ++k) {
            int64_t ch = (int64_t)coords[0] + (int64_t)k;
            int inb = inb_pix && ch >= 0 && (uint64_t)ch < t->dim[0];
            uint32_t phys = orc_swizzle((p * m->channels + k) * (uint32_t)es, t->swizzle);
            if (inb) memcpy(lds + phys, gmem + pix_off + (uint64_t)ch * (uint64_t)es, (size_t)es);
            else memcpy(lds + phys, fill, (size_t)es);
        }
    }
}

void orc_im2col_load_batch(const orc_im2col* m, const uint8_t* gmem, const int32_t* coords,
                           const int32_t* offsets, uint32_t nbox, uint8_t* lds)
{
    uint32_t bb = orc_im2col_box_bytes(m);
    int r = m->t.rank;
    for (uint32_t b = 0; b < nbox; ++b)
        orc_im2col_load(m, gmem, coords + (size_t)b * (size_t)r, offsets + (size_t)b * (size_t)(r - 2),
                        lds + (size_t)b * bb);
}

/* Store, [HPC] "TMA store": the box's LDS image is written back through the
 * same map; elements outside the tensor are not written. */
void orc_store(const orc_map* m, uint8_t* gmem, const int32_t* coords, const uint8_t* lds)
{
    int es = orc_esize(m->dtype);
    uint32_t k[5] = {0, 0, 0, 0, 0};
    do {
        uint64_t lin, off;
        int inb = element_address(m, coords, k, &lin, &off);
        uint32_t phys = orc_swizzle((uint32_t)(lin * (uint64_t)es), m->swizzle);
        if (inb) memcpy(gmem + off, lds + phys, (size_t)es);
    } while (next_k(m, k));
}

/* ---- scalar conversions for the 16-bit float types ------------------------ */

double orc_bf16_to_f64(uint16_t bits)
{
    uint32_t w = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &w, 4);
    return (double)f;
}

double orc_f16_to_f64(uint16_t bits)
{
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1F;
    int man = bits & 0x3FF;
    double v;
    if (e == 0) v = ldexp((double)man, -24);
    else if (e == 31) v = man ? NAN : INFINITY;
    else v = ldexp((double)(1024 + man), e - 25);
    return sign ? -v : v;
}

/* Round x to a binary format with p significand bits, minimum normal
 * exponent emin and maximum exponent emax, ties to even.  Returns +-inf on
 * overflow.  Exactness: scaling by powers of two is exact here and rint()
 * rounds to nearest-even in the default rounding mode. */
static double round_to_format(double x, int p, int emin, int emax)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    (void)frexp(fabs(x), &e);
    int lead = e - 1;                       /* exponent of the leading bit */
    if (lead < emin) lead = emin;           /* subnormal range: fixed quantum */
    int q = lead - (p - 1);
    double r = ldexp(rint(ldexp(x, -q)), q);
    if (fabs(r) >= ldexp(1.0, emax + 1)) return x > 0 ? INFINITY : -INFINITY;
    return r;
}

uint16_t orc_f64_to_bf16(double x)
{
    if (isnan(x)) return 0x7FC0u;
    double r = round_to_format(x, 8, -126, 127);
    float f = (float)r;                     /* exact: r has <= 8 significand bits */
    uint32_t w;
    memcpy(&w, &f, 4);
    return (uint16_t)(w >> 16);
}

uint16_t orc_f64_to_f16(double x)
{
    if (isnan(x)) return 0x7E00u;
    double r = round_to_format(x, 11, -14, 15);
    uint16_t sign = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) return (uint16_t)(sign | (uint16_t)ldexp(a, 24));
    int e;
    (void)frexp(a, &e);
    int lead = e - 1;
    uint16_t man = (uint16_t)(ldexp(a, 10 - lead) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((lead + 15) << 10) | man);
}

/* IEEE addition of two values of the element type, rounded once to that type.
 * The sum is formed in float64 first; for f32, f16 and bf16 operands float64
 * carries at least 2p+2 significand bits, so that intermediate rounding cannot
 * change the final correctly rounded result (Figueroa, "When is double
 * rounding innocuous?", 1995). */
static void add_element(int dtype, uint8_t* dst, const uint8_t* src)
{
    switch (dtype) {
    case ORC_U8: { uint8_t a, b; memcpy(&a, dst, 1); memcpy(&b, src, 1); a = (uint8_t)(a + b); memcpy(dst, &a, 1); break; }
    case ORC_U16: { uint16_t a, b; memcpy(&a, dst, 2); memcpy(&b, src, 2); a = (uint16_t)(a + b); memcpy(dst, &a, 2); break; }
    case ORC_U32: case ORC_I32: { uint32_t a, b; memcpy(&a, dst, 4); memcpy(&b, src, 4); a += b; memcpy(dst, &a, 4); break; }
    case ORC_U64: case ORC_I64: { uint64_t a, b; memcpy(&a, dst, 8); memcpy(&b, src, 8); a += b; memcpy(dst, &a, 8); break; }
    case ORC_F32: { float a, b; memcpy(&a, dst, 4); memcpy(&b, src, 4); a = (float)((double)a + (double)b); memcpy(dst, &a, 4); break; }
    case ORC_F64: { double a, b; memcpy(&a, dst, 8); memcpy(&b, src, 8); a = a + b; memcpy(dst, &a, 8); break; }
    case ORC_BF16: { uint16_t a, b; memcpy(&a, dst, 2); memcpy(&b, src, 2);
        a = orc_f64_to_bf16(orc_bf16_to_f64(a) + orc_bf16_to_f64(b)); memcpy(dst, &a, 2); break; }
    case ORC_F16: { uint16_t a, b; memcpy(&a, dst, 2); memcpy(&b, src, 2);
        a = orc_f64_to_f16(orc_f16_to_f64(a) + orc_f16_to_f64(b)); memcpy(dst, &a, 2); break; }
    default: break;
    }
}

/* Reduce-add store, [HPC] "TMA reduce": like the store, but each in-bounds
 * element is added to what global memory already holds. */
void orc_reduce_add(const orc_map* m, uint8_t* gmem, const int32_t* coords, const uint8_t* lds)
{
    int es = orc_esize(m->dtype);
    uint32_t k[5] = {0, 0, 0, 0, 0};
    do {
        uint64_t lin, off;
        int inb = element_address(m, coords, k, &lin, &off);
        uint32_t phys = orc_swizzle((uint32_t)(lin * (uint64_t)es), m->swizzle);
        if (inb) add_element(m->dtype, gmem + off, lds + phys);
    } while (next_k(m, k));
}

static double element_as_f64(int dtype, const uint8_t* p)
{
    switch (dtype) {
    case ORC_F32: { float v; memcpy(&v, p, 4); return (double)v; }
    case ORC_F64: { double v; memcpy(&v, p, 8); return v; }
    case ORC_BF16: { uint16_t v; memcpy(&v, p, 2); return orc_bf16_to_f64(v); }
    case ORC_F16: { uint16_t v; memcpy(&v, p, 2); return orc_f16_to_f64(v); }
    default: return 0.0;
    }
}

/* ---- min / max reduce ------------------------------------------------------
 * Readings (the pages name "add, min and the like" without defining them):
 *   integers compare as their type, signed for I32 / I64, unsigned otherwise;
 *   floats follow IEEE 754 minNum / maxNum: a NaN operand yields the other
 *   operand, two NaNs give the type's canonical quiet NaN; -0 is ordered
 *   below +0; otherwise the chosen operand's bits are kept unchanged
 *   (subnormals and infinities included).  Under these rules the result does
 *   not depend on the order in which contributions arrive. */
static int element_is_nan(int dtype, const uint8_t* p)
{
    return is_float(dtype) && isnan(element_as_f64(dtype, p));
}

/* 1 if a orders strictly below b (both non-NaN floats, or integers). */
static int element_less(int dtype, const uint8_t* a, const uint8_t* b)
{
    switch (dtype) {
    case ORC_U8: return a[0] < b[0];
    case ORC_U16: { uint16_t x, y; memcpy(&x, a, 2); memcpy(&y, b, 2); return x < y; }
    case ORC_U32: { uint32_t x, y; memcpy(&x, a, 4); memcpy(&y, b, 4); return x < y; }
    case ORC_I32: { int32_t x, y; memcpy(&x, a, 4); memcpy(&y, b, 4); return x < y; }
    case ORC_U64: { uint64_t x, y; memcpy(&x, a, 8); memcpy(&y, b, 8); return x < y; }
    case ORC_I64: { int64_t x, y; memcpy(&x, a, 8); memcpy(&y, b, 8); return x < y; }
    default: {
        double x = element_as_f64(dtype, a), y = element_as_f64(dtype, b);
        if (x == 0.0 && y == 0.0) return signbit(x) && !signbit(y);
        return x < y;
    }
    }
}

static void canonical_nan(int dtype, uint8_t* dst)
{
    switch (dtype) {
    case ORC_F32: { uint32_t v = 0x7FC00000u; memcpy(dst, &v, 4); break; }
    case ORC_F64: { uint64_t v = 0x7FF8000000000000ull; memcpy(dst, &v, 8); break; }
    case ORC_BF16: { uint16_t v = 0x7FC0u; memcpy(dst, &v, 2); break; }
    case ORC_F16: { uint16_t v = 0x7E00u; memcpy(dst, &v, 2); break; }
    default: break;
    }
}

static void minmax_element(int dtype, int op, uint8_t* dst, const uint8_t* src)
{
    int es = orc_esize(dtype);
    int nd = element_is_nan(dtype, dst), ns = element_is_nan(dtype, src);
    if (nd && ns) { canonical_nan(dtype, dst); return; }
    if (ns) return;                                   /* keep dst */
    if (nd) { memcpy(dst, src, (size_t)es); return; }
    int take_src = op == ORC_RED_MIN ? element_less(dtype, src, dst) : element_less(dtype, dst, src);
    if (take_src) memcpy(dst, src, (size_t)es);
}

void orc_reduce_minmax(const orc_map* m, int op, uint8_t* gmem, const int32_t* coords, const uint8_t* lds)
{
    int es = orc_esize(m->dtype);
    uint32_t k[5] = {0, 0, 0, 0, 0};
    do {
        uint64_t lin, off;
        int inb = element_address(m, coords, k, &lin, &off);
        uint32_t phys = orc_swizzle((uint32_t)(lin * (uint64_t)es), m->swizzle);
        if (inb) minmax_element(m->dtype, op, gmem + off, lds + phys);
    } while (next_k(m, k));
}

void orc_reduce_minmax_batch(const orc_map* m, int op, uint8_t* gmem, const int32_t* coords,
                             uint32_t nbox, const uint8_t* lds)
{
    uint32_t bb = orc_box_bytes(m);
    for (uint32_t b = 0; b < nbox; ++b)
        orc_reduce_minmax(m, op, gmem, coords + (size_t)b * (size_t)m->rank, lds + (size_t)b * bb);
}

void orc_load_batch(const orc_map* m, const uint8_t* gmem, const int32_t* coords,
                    uint32_t nbox, uint8_t* lds)
{
    uint32_t bb = orc_box_bytes(m);
    for (uint32_t b = 0; b < nbox; ++b)
        orc_load(m, gmem, coords + (size_t)b * (size_t)m->rank, lds + (size_t)b * bb);
}

void orc_store_batch(const orc_map* m, uint8_t* gmem, const int32_t* coords,
                     uint32_t nbox, const uint8_t* lds)
{
    uint32_t bb = orc_box_bytes(m);
    for (uint32_t b = 0; b < nbox; ++b)
        orc_store(m, gmem, coords + (size_t)b * (size_t)m->rank, lds + (size_t)b * bb);
}

void orc_reduce_add_batch(const orc_map* m, uint8_t* gmem, const int32_t* coords,
                          uint32_t nbox, const uint8_t* lds)
{
    uint32_t bb = orc_box_bytes(m);
    for (uint32_t b = 0; b < nbox; ++b)
        orc_reduce_add(m, gmem, coords + (size_t)b * (size_t)m->rank, lds + (size_t)b * bb);
}

void orc_reduce_add_f64_accumulate(const orc_map* m, double* acc, double* mag,
                                   const int32_t* coords, uint32_t nbox,
                                   const uint8_t* lds)
{
    int es = orc_esize(m->dtype);
    uint32_t bb = orc_box_bytes(m);
    for (uint32_t b = 0; b < nbox; ++b) {
        const int32_t* c = coords + (size_t)b * (size_t)m->rank;
        const uint8_t* img = lds + (size_t)b * bb;
        uint32_t k[5] = {0, 0, 0, 0, 0};
        do {
            uint64_t lin, off;
            int inb = element_address(m, c, k, &lin, &off);
            uint32_t phys = orc_swizzle((uint32_t)(lin * (uint64_t)es), m->swizzle);
            if (inb) {
                double v = element_as_f64(m->dtype, img + phys);
                acc[off / (uint64_t)es] += v;
                mag[off / (uint64_t)es] += fabs(v);
            }
        } while (next_k(m, k));
    }
}

/* ---- transaction-count barrier ([MLC] "waiting for TMA load"; [HPC]
 * "TMA async completion") ------------------------------------------------- */

static void txbar_check_phase(orc_txbar* b)
{
    if (b->arrivals_left == 0 && b->pending_bytes == 0) {
        b->phase ^= 1;
        b->arrivals_left = b->expected_arrivals;
    }
}

void orc_txbar_init(orc_txbar* b, int32_t count)
{
    b->expected_arrivals = count;
    b->arrivals_left = count;
    b->pending_bytes = 0;
    b->phase = 0;
}

void orc_txbar_expect_tx(orc_txbar* b, int64_t bytes)
{
    b->pending_bytes += bytes;
    txbar_check_phase(b);
}

void orc_txbar_arrive(orc_txbar* b, int32_t count)
{
    b->arrivals_left -= count;
    txbar_check_phase(b);
}

void orc_txbar_arrive_expect_tx(orc_txbar* b, int64_t bytes)
{
    b->pending_bytes += bytes;
    b->arrivals_left -= 1;
    txbar_check_phase(b);
}

void orc_txbar_complete_tx(orc_txbar* b, int64_t bytes)
{
    b->pending_bytes -= bytes;
    txbar_check_phase(b);
}

/* The waiter holds the parity of the phase it waits for; that phase is over
 * once the barrier's current phase differs from it. */
int orc_txbar_try_wait(const orc_txbar* b, int32_t parity)
{
    return b->phase != (parity & 1);
}

/* ---- bank sectors ([MLC] "128-byte swizzle grouping requirement") ------- */

void orc_bank_sector_hist(int grouped, int row0, int col, int32_t hist[8])
{
    for (int s = 0; s < 8; ++s) hist[s] = 0;
    for (int r = row0; r < row0 + 8; ++r) {
        uint32_t off;
        if (grouped) {
            /* (group, row, col) box: group = col / 8 selects one of two
             * 16-row x 128-byte groups laid out one after the other. */
            off = (uint32_t)(col / 8) * 16u * 128u + (uint32_t)r * 128u + (uint32_t)(col % 8) * 16u;
        } else {
            off = (uint32_t)r * 256u + (uint32_t)col * 16u;
        }
        uint32_t phys = orc_swizzle(off, ORC_SW_128B);
        hist[(phys >> 4) & 7u] += 1;   /* 4 banks x 4 bytes per sector */
    }
}

/* ---- GEMM sampled reference --------------------------------------------- */

void orc_gemm_bf16_sample(const uint16_t* A, const uint16_t* B, uint32_t K,
                          const uint32_t* rows, const uint32_t* cols,
                          uint32_t nsample, double* out)
{
    for (uint32_t s = 0; s < nsample; ++s) {
        const uint16_t* a = A + (size_t)rows[s] * K;
        const uint16_t* b = B + (size_t)cols[s] * K;
        double acc = 0.0;
        for (uint32_t k = 0; k < K; ++k)
            acc += orc_bf16_to_f64(a[k]) * orc_bf16_to_f64(b[k]);
        out[s] = acc;
    }
}
