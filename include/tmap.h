/*
 * tmap.h -- C ABI of the MI355X (gfx950) descriptor-driven tile mover.
 *
 * A tensor map (tmap_t) describes how a tensor lies in device memory and
 * which box a single copy moves; per-call box origins then drive
 * global->LDS loads (with the swizzle applied on write), LDS->global stores
 * and reduce-add stores.  Everything runs in hand-written HIP kernels for
 * gfx950; this header exposes only plain pointers, sizes and integers.
 *
 * Reference pages cited below:
 *   [MLC]  Modern GPU Programming for MLSys (zh), chapter "TMA".
 *   [H200] blog.coolgpu.cn, "H200 // TMA" feature card.
 *   [HPC]  gpu-hpc-book, chapter 08 "Cuda TMA".
 *
 * Conventions shared by every call
 *   - Dimensions, strides, box extents and coordinates are listed innermost
 *     (fastest varying) first, as on the pages ([H200] section 04 example 1).
 *   - "d_" pointers are device (HBM) addresses; all other pointers are host
 *     addresses read before the call returns.  The library never allocates
 *     per call and never frees caller memory.
 *   - Launch calls are asynchronous and ordered on `stream` (a hipStream_t;
 *     NULL = the null stream).  No call synchronises implicitly.
 *   - Errors are returned as tmap_status; nothing aborts or throws across the
 *     ABI.  Launch-time failures return TMAP_ERR_HIP and keep the HIP error
 *     text for tmap_last_error().
 *   - Calls are reentrant; concurrent calls on different streams are safe as
 *     long as their destination memory does not overlap.
 *
 * Kernels that move tiles themselves use the device API in tile.hpp with the
 * same maps, passed to the kernel by value.
 */
#ifndef ATT_TMAP_H
#define ATT_TMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- types ---------------------------------------------------------------- */

/* Opaque 128-byte descriptor, 64-byte aligned, copyable by value.  Created on
 * the host only ([H200] section 05: build the map on the host, rebase it with
 * an address replacement rather than rebuilding it on the device). */
typedef struct tmap_t {
    uint8_t opaque[128];
} __attribute__((aligned(64))) tmap_t;

typedef enum {
    TMAP_U8 = 0, TMAP_U16 = 1, TMAP_U32 = 2, TMAP_I32 = 3, TMAP_U64 = 4,
    TMAP_I64 = 5, TMAP_F16 = 6, TMAP_BF16 = 7, TMAP_F32 = 8, TMAP_F64 = 9
} tmap_dtype;

/* XOR swizzle applied on the LDS byte offset relative to the box image:
 * bits 4..(3+b) of the offset are XORed with bits 7..(6+b), b = 1, 2, 3 for
 * the 32-, 64- and 128-byte spans.  With 128-byte rows the 128-byte mode puts
 * logical 16-byte sector c of row r at physical sector c XOR (r % 8) ([MLC]
 * "TMA writes swizzled layout"; atoms of 8 rows, [MLC] "3D TMA").  The pages
 * only name the 32- and 64-byte modes; their bit pattern is this library's
 * reading.
 * The _K256 modes are this library's addition for gfx950, whose LDS serves
 * ds_read_b128 at 256 bytes per clock: the key is taken from bits
 * 8..(7+b) (the 256-byte unit index), giving 16-row atoms, so that one
 * 16-byte column read across 32 rows (an MFMA 32x32 operand fragment) hits
 * every bank once where the 8-row pattern hits each bank twice. */
typedef enum {
    TMAP_SWIZZLE_NONE = 0, TMAP_SWIZZLE_32B = 1, TMAP_SWIZZLE_64B = 2, TMAP_SWIZZLE_128B = 3,
    TMAP_SWIZZLE_32B_K256 = 5, TMAP_SWIZZLE_64B_K256 = 6, TMAP_SWIZZLE_128B_K256 = 7
} tmap_swizzle;

/* Out-of-bounds fill for loads ([H200] section 02 table: zero or NaN).
 * NAN writes the type's canonical quiet NaN (f32 0x7FC00000, f16 0x7E00,
 * bf16 0x7FC0, f64 0x7FF8000000000000) and is accepted for float types only. */
typedef enum { TMAP_OOB_ZERO = 0, TMAP_OOB_NAN = 1 } tmap_oob;

typedef int32_t tmap_status;
enum {
    TMAP_OK = 0,
    TMAP_ERR_NULL = 1,            /* a required pointer is NULL               */
    TMAP_ERR_RANK = 2,            /* rank outside [1, 5]                      */
    TMAP_ERR_DTYPE = 3,           /* unknown element type                     */
    TMAP_ERR_ALIGN = 4,           /* base address not 16-byte aligned         */
    TMAP_ERR_DIM = 5,             /* globalDim outside [1, 2^32]              */
    TMAP_ERR_STRIDE = 6,          /* stride 0, not a multiple of 16, >= 2^40  */
    TMAP_ERR_BOX = 7,             /* box outside [1, 256] or box[0]*esize%16  */
    TMAP_ERR_ESTRIDE = 8,         /* element stride outside [1, 8], or the
                                     LDS row ceil(box0/es0)*esize not a
                                     multiple of 16 bytes                     */
    TMAP_ERR_SWIZZLE_WIDTH = 9,   /* swizzled LDS row bytes != span           */
    TMAP_ERR_OOB_FILL_DTYPE = 10, /* NaN fill requested for an integer type   */
    TMAP_ERR_LDS_CAPACITY = 11,   /* box image larger than one workgroup's LDS*/
    TMAP_ERR_UNSUPPORTED = 12,    /* enum value or shape this call cannot do  */
    TMAP_ERR_HIP = 13,            /* HIP runtime error; see tmap_last_error() */
    TMAP_ERR_TIMEOUT = 14,        /* a bounded barrier wait inside a kernel
                                     gave up: the box it guarded is not valid
                                     (reported by tile_device_status)        */
    TMAP_ERR_DEVICE_CHECK = 15    /* a check of a debug build failed on the
                                     device (tile_device_status)             */
};

/* Largest box image (bytes) a map may describe: the 160 KiB of LDS per CU
 * less 1 KiB kept for the completion barrier beside the image. */
#define TMAP_LDS_CAPACITY 162816u

typedef struct {
    int32_t  dtype;          /* tmap_dtype                                  */
    int32_t  rank;
    int32_t  esize;          /* bytes per element                           */
    int32_t  swizzle;        /* tmap_swizzle                                */
    int32_t  oob;            /* tmap_oob                                    */
    uint32_t lds_extent[5];  /* ceil(box[i] / estride[i]); 1 beyond rank    */
    uint32_t box_bytes;      /* esize * prod(lds_extent): expect_tx amount  */
    uint32_t row_bytes;      /* lds_extent[0] * esize                       */
    uint32_t atom_bytes;     /* one period of the XOR key: 8 rows (16 rows
                                for _K256) of the span; 0 for NONE          */
    uint64_t base;           /* current global base address                 */
} tmap_info_t;

/* ---- host-only descriptor calls --------------------------------------------- */

/* Encode and validate a tensor map ([H200] section 03 constraint table and
 * section 04 example 1; [HPC] "Tensor descriptor" field list).
 *   out            receives the descriptor (caller-owned storage).
 *   dtype          tmap_dtype.
 *   rank           1..5.
 *   gaddr          device base address, 16-byte aligned.
 *   gdim[rank]     globalDim, each in [1, 2^32].
 *   gstride[rank-1] byte strides of dims 1..rank-1: multiples of 16, nonzero,
 *                  below 2^40, in any order (may be NULL when rank == 1).
 *   box[rank]      box extents, each in [1, 256]; box[0]*esize % 16 == 0.
 *   estride[rank]  element strides in [1, 8] (NULL = all 1).  The box reads
 *                  elements c + k*estride for k < ceil(box/estride); the LDS
 *                  image is dense ([HPC] field list; this library's reading of
 *                  a garbled passage).
 *   swizzle        tmap_swizzle; when not NONE the LDS row
 *                  ceil(box0/estride0)*esize must equal the span exactly
 *                  ([MLC] "3D TMA" and "grouping requirement").
 *   oob            tmap_oob.
 * Validation order (first failure is reported): NULL, RANK, DTYPE,
 * UNSUPPORTED (enums), NULL/ALIGN (base), DIM, STRIDE, BOX, ESTRIDE,
 * SWIZZLE_WIDTH, OOB_FILL_DTYPE, LDS_CAPACITY.  On error *out is zeroed. */
tmap_status tmap_encode(tmap_t* out, int32_t dtype, uint32_t rank, void* gaddr,
                        const uint64_t* gdim, const uint64_t* gstride,
                        const uint32_t* box, const uint32_t* estride,
                        int32_t swizzle, int32_t oob);

/* Point an encoded map at another base address of identical layout ([H200]
 * sections 03 and 05: runtime rebasing).  Errors: NULL, ALIGN. */
tmap_status tmap_replace_address(tmap_t* m, void* gaddr);

/* Bytes one box occupies on chip: the amount a load expects ([MLC] "waiting
 * for TMA load"); 0 for a NULL map. */
uint32_t tmap_box_bytes(const tmap_t* m);

/* Fill *info from an encoded map.  Errors: NULL. */
tmap_status tmap_query(const tmap_t* m, tmap_info_t* info);

/* Static text for a status code. */
const char* tmap_strerror(tmap_status s);

/* Text of the last TMAP_ERR_HIP on the calling thread ("" if none). */
const char* tmap_last_error(void);

/* ---- launches (asynchronous, stream-ordered) ------------------------------ */

/* Im2col-mode tensor map ([HPC] closing paragraph: im2col encoding exists,
 * with its own swizzle parameter; the pages define nothing further, so the
 * following is this library's reading).  The tensor is channel-innermost:
 * gdim = (C, W[, H[, D]], N), rank 3..5, byte strides as for tmap_encode.
 * Along spatial dimension s (gdim[s+1]) window origins form the grid
 * lower[s], lower[s] + es, ... up to gdim[s+1] - 1 + upper[s] (lower counted
 * from the start and upper from the end of the dimension; es = estride[s+1],
 * the convolution stride).  One load (tile_load_im2col) reads
 * pixels_per_column consecutive window origins -- W fastest, then H, D and
 * the image index -- starting at the origin named by its coordinates, and
 * for each origin channels_per_pixel channels from the channel coordinate
 * on, at the origin plus the load's per-dimension offsets (the filter tap).
 * Elements outside the tensor take the OOB fill.  The LDS image is
 * pixels_per_column rows of channels_per_pixel elements, swizzled like a
 * tiled box.  Limits: channels_per_pixel 1..256 with channels * esize a
 * multiple of 16 (equal to the swizzle span when swizzled),
 * pixels_per_column 1..1024, corners in [-32768, 32767] with a non-empty
 * grid, estride 1 on C and N and 1..8 on spatial dimensions (NULL = all 1),
 * at most 2^62 windows in total (a limit of this library: a window is
 * located through a signed 64-bit linear index; the pages set no bound).
 * Errors as tmap_encode (ERR_BOX for the
 * pixel / channel / corner limits, ERR_DIM for the window count).  The
 * result is a tmap_t usable only with tile_load_im2col (tiled entry points
 * return ERR_UNSUPPORTED for it); tmap_query reports lds_extent =
 * {channels, pixels, 1, 1, 1}. */
tmap_status tmap_encode_im2col(tmap_t* out, int32_t dtype, uint32_t rank, void* gaddr,
                               const uint64_t* gdim, const uint64_t* gstride_bytes,
                               const int32_t* lower, const int32_t* upper,
                               uint32_t channels_per_pixel, uint32_t pixels_per_column,
                               const uint32_t* estride, int32_t swizzle, int32_t oob);

/* Load nbox im2col boxes and dump each raw LDS image (swizzle included) to
 * d_lds_image_out + b * tmap_box_bytes(m).  Box b's coordinates are
 * d_coords[b*rank ..] = (channel, spatial origin..., image) and its
 * filter-tap offsets d_offsets[b*(rank-2) ..] (int32, one per spatial
 * dimension, W first); any values are legal (elements outside the tensor
 * take the fill).  Completion inside the kernel is byte-counted.  Errors:
 * NULL, UNSUPPORTED (not an im2col map), LDS_CAPACITY, HIP.  nbox == 0 is a
 * no-op. */
tmap_status tile_load_im2col(const tmap_t* m, const int32_t* d_coords, const int32_t* d_offsets,
                             uint32_t nbox, void* d_lds_image_out, void* stream);

/* Load nbox boxes global->LDS and dump each box's raw LDS image.
 * [MLC] "one thread describes the whole tile", "TMA writes swizzled layout";
 * [HPC] single-tile load.  Box b starts at d_coords[b*rank .. b*rank+rank-1]
 * (int32, any value: elements outside the tensor take the OOB fill).  The
 * image of box b (physical LDS bytes, swizzle included) is written to
 * d_lds_image_out + b * tmap_box_bytes(m).  Completion inside the kernel is
 * byte-counted.  Errors: NULL, LDS_CAPACITY (image larger than the device's
 * per-workgroup LDS), HIP.  nbox == 0 is a no-op. */
tmap_status tile_load(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                      void* d_lds_image_out, void* stream);

/* Store nbox boxes LDS->global ([HPC] "TMA store").  The raw LDS image of box
 * b is read from d_lds_image_in + b * tmap_box_bytes(m), staged in LDS, and
 * each element inside the tensor is written through the map (inverse
 * swizzle); elements outside are skipped.  Boxes that overlap race (last
 * writer unspecified).  Errors as tile_load. */
tmap_status tile_store(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                       const void* d_lds_image_in, void* stream);

/* Reduce-add store ([HPC] "TMA reduce"): like tile_store but every in-bounds
 * element is added to global memory atomically.  Integer types wrap modulo
 * 2^w; f32/f64 use IEEE addition (round to nearest even; a NaN result's
 * payload is not fixed), f16/bf16 add in f32 and round once to nearest
 * even, a NaN result being the type's canonical quiet NaN (0x7E00 /
 * 0x7FC0).  Elements outside the box that share a 32-bit word with a 16- or
 * 8-bit element inside it are left as they were.  Overlapping boxes are
 * applied in an unspecified order (bit-exact for integers).  Errors as
 * tile_load. */
tmap_status tile_reduce_add(const tmap_t* m, const int32_t* d_coords, uint32_t nbox,
                            const void* d_lds_image_in, void* stream);

/* Reduce store with a chosen element-wise operation ([HPC] "TMA reduce":
 * the write-back combines with what global memory holds, "add, min and the
 * like").  op TMAP_REDUCE_ADD is tile_reduce_add.  TMAP_REDUCE_MIN / _MAX:
 * integers compare as their type (signed for I32 / I64, unsigned
 * otherwise); floating types follow IEEE minNum / maxNum -- a NaN operand
 * yields the other operand, two NaNs the type's canonical quiet NaN -- with
 * -0 ordered below +0, and the winning operand's bits are stored unchanged.
 * Each element update is atomic; min / max results do not depend on the
 * order of overlapping boxes.  Errors as tile_load, plus UNSUPPORTED for an
 * unknown op. */
enum { TMAP_REDUCE_ADD = 0, TMAP_REDUCE_MIN = 1, TMAP_REDUCE_MAX = 2 };
tmap_status tile_reduce(const tmap_t* m, int32_t op, const int32_t* d_coords, uint32_t nbox,
                        const void* d_lds_image_in, void* stream);

/* Full-grid round trip: every box of the grid covering `src` (origins at
 * multiples of box[i]) is loaded global->LDS through `src` and stored
 * LDS->global through `dst`, with `stages` LDS buffers per workgroup
 * ([MLC] "TMA in a pipeline": fill one stage while another is consumed;
 * with two stages and boxes of 4 to 32 KiB one wave issues the copies and
 * four others store each part as it lands).  src and dst must have
 * the same dtype, rank, dims, box and swizzle, all element strides 1, and
 * must not overlap.  stages in [1, 8].  Errors: NULL, UNSUPPORTED (geometry
 * mismatch, stages, element strides), LDS_CAPACITY, HIP. */
tmap_status tile_copy(const tmap_t* src, const tmap_t* dst, uint32_t stages, void* stream);

/* Same as tile_copy with an explicit grid size (0 = automatic) and launch
 * variant bits, for tuning sweeps: 1 non-temporal stores, 2 force the
 * generic one-workgroup-per-box path, 4 workgroups own contiguous box
 * ranges (else strided), 8 XCD-aware workgroup numbering, bits 4..5 boxes
 * per ring stage (1, 2, 4, 8), 64 batch mode: each workgroup owns `stages`
 * (2..4) consecutive boxes, one LDS stage each, loads all of them, reads
 * each stage once its copies have landed and stores them all at the end
 * (grid ignored; the box count must divide by `stages`), 128 with 64: the
 * workgroup's boxes are neighbours in dim 0 and each wave issues its first
 * copy of every box, then its second, ... (back-to-back requests cover the
 * same rows several boxes wide), 256 with 64: loads through registers and
 * ds_write instead of the LDS-DMA, 512 producer / consumer form: each
 * workgroup owns `stages` (1, 2 or 4) consecutive boxes of 4, 8, 16 or 32
 * KiB (at most 64 KiB of copies), one stage each; one wave issues every
 * copy and releases the landed 1 KiB groups four at a time with a barrier,
 * four consumer waves read and store them (grid ignored; other shapes fall
 * back to the modes above).  tile_copy uses 1|4|512 with two boxes per
 * workgroup for stages = 2, 1|4 otherwise.  Ring depths 5 and 7 take the
 * generic path. */
tmap_status tile_copy_ex(const tmap_t* src, const tmap_t* dst, uint32_t stages,
                         uint32_t grid, uint32_t variant, void* stream);

/* Byte-counted barrier self-test ([MLC] "waiting for TMA load": several tile
 * copies complete one barrier phase by byte count).  One workgroup initialises a barrier
 * with arrival count 1, performs arrive.expect_tx(sum of tile bytes), then
 * loads `ntile` boxes of map `m` (origins d_coords) and lets each copy signal
 * complete-tx with its own byte count as it lands.  After every barrier
 * operation the state (arrivals_left, pending_bytes, phase) is appended to
 * d_trace (int32 triples, 3 * (2 + ntile) entries: after init, after
 * arrive.expect_tx, after each complete-tx, in completion order); the loaded
 * images are written to d_lds_image_out.  ntile in [1, 8]; the images must
 * fit LDS together.  Errors: NULL, UNSUPPORTED, LDS_CAPACITY, HIP. */
tmap_status txbar_selftest(const tmap_t* m, const int32_t* d_coords, uint32_t ntile,
                           int32_t* d_trace, void* d_lds_image_out, void* stream);

/* txbar_selftest with two more inputs: the barrier expects `extra_bytes`
 * beyond the tiles' bytes (0 in txbar_selftest), and its final wait gives up
 * after `max_polls` polls (each about a 64-cycle sleep; txbar_selftest uses
 * 2^22).  With extra_bytes > 0 the phase never completes, so the wait times
 * out and the kernel records TMAP_ERR_TIMEOUT for tile_device_status while
 * still exiting normally: the host-forced failure path of the bounded wait.
 * extra_bytes < 2^30, max_polls >= 1, else UNSUPPORTED; other errors as
 * txbar_selftest. */
tmap_status txbar_selftest_ex(const tmap_t* m, const int32_t* d_coords, uint32_t ntile,
                              uint32_t extra_bytes, uint32_t max_polls, int32_t* d_trace,
                              void* d_lds_image_out, void* stream);

/* Device-side status of the batch calls (tile_load, tile_load_im2col,
 * txbar_selftest[_ex]): their kernels never trap; a barrier wait that gives
 * up (a box whose bytes never all arrived) or, in a debug build (ATT_DEBUG),
 * a failed device check is recorded in a per-device error word instead.
 * This call synchronises `stream`, reads that word on the current device
 * and clears it: TMAP_OK if nothing was recorded since the last call,
 * TMAP_ERR_TIMEOUT if a wait gave up, TMAP_ERR_DEVICE_CHECK for a debug
 * check, TMAP_ERR_HIP on a runtime error.  Not for use under graph
 * capture (it synchronises). */
tmap_status tile_device_status(void* stream);

/* LDS bank-sector probe ([MLC] "128-byte swizzle grouping requirement").
 * For a 16 x 256-byte sector grid laid out in LDS either grouped (two
 * 128-byte groups per row, a 3-D box, layout 1) or with a 256-byte row
 * stride (layout 0), both under the 128-byte swizzle, eight lanes read one
 * 16-byte column of eight consecutive rows with ds_read_b128 at the
 * swizzled addresses the device address generator produces.  For row0 in
 * 0..8 and col in 0..15 the kernel writes the hit count of each bank sector
 * ((addr >> 4) & 7) to d_hist[(row0*16 + col)*8 + s], and repeats the reads
 * `iters` times so hardware counters can be sampled.
 * Layouts 2 and 3 instead read one MFMA 32x32x16 operand fragment of a
 * 32-row x 128-byte box (lane l: row l % 32, logical chunk l / 32) under
 * TMAP_SWIZZLE_128B (2) or TMAP_SWIZZLE_128B_K256 (3), `iters` times, and
 * write each lane's physical LDS byte offset to d_hist[l] (64 entries).
 * Layouts 4 to 6 replay the GEMM epilogue's C staging in a 128-byte-row box
 * image: 4 and 6 its 8-byte writes (lane l: row l % 16, four bf16 columns
 * from 4 * (l / 16)) under TMAP_SWIZZLE_128B_K256 (4) or TMAP_SWIZZLE_128B
 * (6), 5 its 16-byte reads (lane l: row l / 8, logical chunk l % 8) under
 * TMAP_SWIZZLE_128B_K256; d_hist[l] as for layouts 2 and 3.
 * Errors: NULL, UNSUPPORTED (layout), HIP. */
tmap_status lds_bank_probe(int32_t layout, uint32_t iters, int32_t* d_hist, void* stream);

/* HBM streaming probe (a measurement aid, not an operation of the pages):
 * moves `bytes` (a multiple of 16) with plain fully coalesced 16-byte vector
 * accesses, non-temporal stores, about eight 256-thread workgroups per CU,
 * so that a benchmark can report what this GPU's memory system delivers to
 * simple streams beside the tile copy.  kind 0: read d_src only (d_dst is a
 * sink of at least 4 bytes that may receive one word); kind 1: write d_dst
 * only (d_src ignored, may be NULL); kind 2: copy d_src -> d_dst.  Device
 * pointers, 16-byte aligned, caller-owned.  Asynchronous on `stream`.
 * Errors: NULL, ALIGN, UNSUPPORTED (kind, bytes not a multiple of 16), HIP.
 * bytes == 0 is a no-op. */
tmap_status hbm_probe(int32_t kind, const void* d_src, void* d_dst, uint64_t bytes, void* stream);

/* The copy of hbm_probe in other launch shapes, for a sweep that finds the
 * best plain copy this GPU runs (the measured ceiling reported beside the
 * tile copy): variant bits 0..1 select 1, 2, 4 or 8 16-byte vectors per
 * thread and step, bit 2 non-temporal stores, bit 3 one contiguous slice per
 * workgroup (else grid-stride order); wg_per_cu 1..32 workgroups of 256
 * threads per CU (fewer if the data needs fewer).  Pointers and errors as
 * hbm_probe (kind 2); variant > 15 or wg_per_cu outside 1..32 is
 * UNSUPPORTED. */
tmap_status hbm_probe_copy_ex(const void* d_src, void* d_dst, uint64_t bytes, uint32_t variant,
                              uint32_t wg_per_cu, void* stream);

/* Box-shaped copy without LDS (a measurement aid): copies a row-major byte
 * matrix of `height` rows of `width` bytes (both multiples of 128) in boxes
 * of 128 rows x 128 bytes with the tile copy's access shape -- each wave
 * instruction moves 8 rows x 128 bytes of one box -- through registers,
 * `boxes_per_wg` (1, 2, 4, 8; dividing width / 128) neighbouring boxes per
 * 256-thread workgroup, all loads of a workgroup before its stores.  variant
 * bit 0 non-temporal stores, bit 1 XCD-contiguous workgroup numbering (the
 * workgroup count must divide by 8), bit 2 box-major instead of row-group-
 * major issue, bits 3..4 = k > 0: reserve 16 KiB << (k - 1) of LDS per
 * workgroup (unused; it bounds the workgroups per CU as the tile copy's
 * stages do), bit 5 box row r walked starting r boxes along (as the tile
 * copy walks it).  Shows what the box shape costs apart from the LDS staging.
 * Errors: NULL, ALIGN (16 bytes), UNSUPPORTED (shape, variant > 63), HIP. */
tmap_status hbm_probe_box_copy(const void* d_src, void* d_dst, uint32_t width, uint32_t height,
                               uint32_t boxes_per_wg, uint32_t variant, void* stream);

/* Consumer: bf16 GEMM mainloop C = A * B ([MLC] overview and "TMA in a
 * pipeline"; [H200] section 02 result).  A is M x K row-major (map dims
 * {K, M}), B is K x N column-major (map dims {K, N}), both bf16 with box
 * {64, 256} and TMAP_SWIZZLE_128B or TMAP_SWIZZLE_128B_K256 (or the 32-deep
 * box that gemm_bf16_ex describes); tiles are staged by the tile loader into a
 * `stages`-deep LDS ring and consumed by MFMA bf16 with fp32 accumulation.
 * d_C is M x N row-major bf16 (round to nearest even), leading dimension
 * ldc >= N elements.  Any M and N, and any K >= 1 (the maps' dim 0 is K,
 * and a map dimension is at least 1): partial tiles in M and N are clipped
 * by the epilogue, and a K that is not a multiple of the box depth is zero-
 * filled through the maps' OOB fill (with stages = 2 only the last K tile
 * takes that slower loader, with more stages every tile).  For the 64-deep K step, stages
 * = 2 is the double buffer (two 64 KiB stages; three do not fit the 160 KiB
 * LDS) and stages = 3 the operand ring: five 32 KiB slots holding A and B
 * boxes in turn, so that A runs three deep and B two deep; it takes K a
 * multiple of 64.  Errors: NULL, UNSUPPORTED (map shape, dtype, box,
 * swizzle, OOB fill other than zero, stages, K for stages = 3, K == 0,
 * ldc < N), HIP.  M == 0 or N == 0 is a no-op. */
tmap_status gemm_bf16(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                      uint32_t K, uint32_t ldc, uint32_t stages, void* stream);

/* gemm_bf16 with tuning knobs: `group_m` tile rows per rasterisation group
 * (0 = 8) and `xcd` (0 = plain order, 1 = each XCD a contiguous range of
 * tiles, 2 = each XCD a 2-D block of tiles in a 4 x 2 arrangement when the
 * tile grid divides).  Maps
 * with box {32, 256} and TMAP_SWIZZLE_64B or TMAP_SWIZZLE_64B_K256 select the
 * 32-deep K step, for which stages may be 2 to 5; box {64, 256} takes
 * stages 2 or 3 as above.  `mfma` picks the matrix instruction: 16 (16x16x32
 * tiles, the default for the 64-deep step and the only form of its operand
 * ring), 32 (32x32x16 tiles, the only form for the 32-deep step) or 0 for
 * the default; others return ERR_UNSUPPORTED. */
tmap_status gemm_bf16_ex(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                         uint32_t K, uint32_t ldc, uint32_t stages, uint32_t group_m, uint32_t xcd,
                         uint32_t mfma, void* stream);

/* gemm_bf16 with C written as fp32: the accumulators as the mainloop leaves
 * them, before any rounding to bf16, so that the mainloop's own accuracy can
 * be checked.  d_C is M x N row-major fp32, leading dimension ldc >= N
 * elements, 4-byte aligned (16-byte stores where C and ldc allow them,
 * element stores otherwise).  Maps with box {64, 256} only (the 64-deep K
 * step, 16x16x32 MFMAs), stages 2 or 3 as in gemm_bf16; other maps or
 * stages return ERR_UNSUPPORTED, and errors are otherwise as gemm_bf16. */
tmap_status gemm_bf16_f32(const tmap_t* A, const tmap_t* B, void* d_C, uint32_t M, uint32_t N,
                          uint32_t K, uint32_t ldc, uint32_t stages, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ATT_TMAP_H */
