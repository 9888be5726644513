/*
 * oracle.h -- CPU oracle for descriptor-driven tile movement.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes this
 * header or links this code; only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg call it.  It shares no code with the HIP path.
 *
 * Every routine is a plain scalar loop written from the reference pages'
 * definitions (Modern GPU Programming for MLSys, chapter "TMA"; the H200 TMA
 * feature card; gpu-hpc-book chapter 08 "Cuda TMA").  Dimensions, box extents
 * and coordinates are listed innermost first, as on those pages.
 */
#ifndef ATT_ORACLE_H
#define ATT_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  Integer codes are private to the oracle. */
enum {
    ORC_U8 = 0, ORC_U16 = 1, ORC_U32 = 2, ORC_I32 = 3, ORC_U64 = 4,
    ORC_I64 = 5, ORC_F16 = 6, ORC_BF16 = 7, ORC_F32 = 8, ORC_F64 = 9
};

/* Swizzle modes: NONE, and XOR patterns whose span is 32, 64 or 128 bytes.
 * The _K256 modes take the XOR key from the 256-byte unit index instead of
 * the 128-byte one (16-row atoms for 128-byte rows); they are not on the
 * pages and exist for LDS that serves 256 bytes per clock. */
enum { ORC_SW_NONE = 0, ORC_SW_32B = 1, ORC_SW_64B = 2, ORC_SW_128B = 3,
       ORC_SW_32B_K256 = 5, ORC_SW_64B_K256 = 6, ORC_SW_128B_K256 = 7 };

/* Out-of-bounds fill: all-zero bits, or the element type's quiet NaN. */
enum { ORC_FILL_ZERO = 0, ORC_FILL_NAN = 1 };

/* Validation outcomes (0 = accepted). */
enum {
    ORC_OK = 0, ORC_ERR_NULL = 1, ORC_ERR_RANK = 2, ORC_ERR_DTYPE = 3,
    ORC_ERR_ALIGN = 4, ORC_ERR_DIM = 5, ORC_ERR_STRIDE = 6, ORC_ERR_BOX = 7,
    ORC_ERR_ESTRIDE = 8, ORC_ERR_SWIZZLE_WIDTH = 9, ORC_ERR_OOB_FILL_DTYPE = 10,
    ORC_ERR_LDS_CAPACITY = 11, ORC_ERR_UNSUPPORTED = 12
};

/* Largest LDS box image the oracle accepts: 160 KiB of on-chip memory per
 * CU less 1 KiB kept for the completion barrier (a reading: the pages only
 * imply that a box must fit in shared memory). */
#define ORC_LDS_CAPACITY 162816u

/* A tensor map as the oracle sees it.  stride[0] is unused (the element size
 * is implied by dtype); stride[i] for i >= 1 is the byte distance between
 * consecutive indices of dimension i. */
typedef struct {
    int32_t  dtype;
    int32_t  rank;
    uint64_t base_addr;     /* only its alignment is inspected */
    uint64_t dim[5];
    uint64_t stride[5];
    uint32_t box[5];
    uint32_t estride[5];
    int32_t  swizzle;
    int32_t  fill;
} orc_map;

int      orc_esize(int dtype);
int      orc_validate(const orc_map* m);
uint32_t orc_lds_extent(const orc_map* m, int dim);
uint32_t orc_box_bytes(const orc_map* m);
uint32_t orc_swizzle(uint32_t lds_offset, int swizzle);

/* gmem points at the tensor's base address; the tensor's footprint must be
 * readable / writable.  lds is the box's on-chip image, orc_box_bytes long. */
void orc_load(const orc_map* m, const uint8_t* gmem, const int32_t* coords, uint8_t* lds);
void orc_store(const orc_map* m, uint8_t* gmem, const int32_t* coords, const uint8_t* lds);
void orc_reduce_add(const orc_map* m, uint8_t* gmem, const int32_t* coords, const uint8_t* lds);

/* Batched forms: box b uses coords[b*rank ...] and image lds + b*box_bytes.
 * Boxes are applied in index order. */
void orc_load_batch(const orc_map* m, const uint8_t* gmem, const int32_t* coords,
                    uint32_t nbox, uint8_t* lds);
void orc_store_batch(const orc_map* m, uint8_t* gmem, const int32_t* coords,
                     uint32_t nbox, const uint8_t* lds);
void orc_reduce_add_batch(const orc_map* m, uint8_t* gmem, const int32_t* coords,
                          uint32_t nbox, const uint8_t* lds);

/* Reduce store with an element-wise operation other than add ([HPC] "TMA
 * reduce": the write-back may combine with what global memory holds, add,
 * min and the like).  op: ORC_RED_MIN or ORC_RED_MAX (ORC_RED_ADD is
 * orc_reduce_add).  Boxes are applied in index order. */
enum { ORC_RED_ADD = 0, ORC_RED_MIN = 1, ORC_RED_MAX = 2 };
void orc_reduce_minmax(const orc_map* m, int op, uint8_t* gmem, const int32_t* coords, const uint8_t* lds);
void orc_reduce_minmax_batch(const orc_map* m, int op, uint8_t* gmem, const int32_t* coords,
                             uint32_t nbox, const uint8_t* lds);

/* Order-free reference for float reductions.  acc and mag are float64 arrays
 * indexed by (element byte offset from base) / esize; acc must already hold
 * the destination's initial values (and mag their magnitudes).  Every
 * in-bounds contribution of every box is added to acc in float64 without
 * rounding to the element type, and its magnitude to mag. */
void orc_reduce_add_f64_accumulate(const orc_map* m, double* acc, double* mag,
                                   const int32_t* coords, uint32_t nbox,
                                   const uint8_t* lds);

/* Im2col-mode map (the pages name im2col tensor-map encoding, with its own
 * swizzle parameter, and nothing more; the definition below is a reading).
 * The tensor is channel-innermost: dims (C, W[, H[, D]], N), rank 3..5, so
 * S = rank - 2 spatial dimensions.  t.box is unused; t.estride[0] and
 * t.estride[rank-1] must be 1 and the spatial element strides are the
 * convolution strides.  Along spatial dimension s (tensor dim s+1) window
 * origins run over lower[s], lower[s] + es, ... up to dim - 1 + upper[s]
 * (lower counted from the start, upper from the end of the dimension).  A
 * load reads `pixels` consecutive window origins -- W fastest, then H, D and
 * the image index N -- starting at the origin named by its coordinates, and
 * for each takes `channels` channels from the channel coordinate on, at the
 * origin shifted by the load's per-dimension offsets (the filter tap).
 * Elements outside the tensor take the fill.  The LDS image is `pixels` rows
 * of channels * esize bytes, swizzled like a tiled box. */
typedef struct {
    orc_map  t;
    int32_t  lower[3];
    int32_t  upper[3];
    uint32_t channels;
    uint32_t pixels;
} orc_im2col;

int      orc_im2col_validate(const orc_im2col* m);
uint32_t orc_im2col_box_bytes(const orc_im2col* m);
/* coords: rank values (channel, spatial..., image); offsets: rank-2 values. */
void orc_im2col_load(const orc_im2col* m, const uint8_t* gmem, const int32_t* coords,
                     const int32_t* offsets, uint8_t* lds);
void orc_im2col_load_batch(const orc_im2col* m, const uint8_t* gmem, const int32_t* coords,
                           const int32_t* offsets, uint32_t nbox, uint8_t* lds);

/* Transaction-count barrier model. */
typedef struct {
    int32_t expected_arrivals;
    int32_t arrivals_left;
    int64_t pending_bytes;
    int32_t phase;
} orc_txbar;

void orc_txbar_init(orc_txbar* b, int32_t count);
void orc_txbar_expect_tx(orc_txbar* b, int64_t bytes);
void orc_txbar_arrive(orc_txbar* b, int32_t count);
void orc_txbar_arrive_expect_tx(orc_txbar* b, int64_t bytes);
void orc_txbar_complete_tx(orc_txbar* b, int64_t bytes);
int  orc_txbar_try_wait(const orc_txbar* b, int32_t parity);

/* Bank-sector model: 32 banks of 4 bytes grouped into 8 sectors of 16 bytes.
 * For eight consecutive rows starting at row0 and one 16-byte column col of a
 * 16 x 16 sector grid (256-byte rows), fill hist[8] with how many of the eight
 * accesses land in each sector.  grouped != 0 splits each row into two
 * 128-byte groups (a three-dimensional box); grouped == 0 keeps the 256-byte
 * row stride. */
void orc_bank_sector_hist(int grouped, int row0, int col, int32_t hist[8]);

/* Sampled GEMM reference: C[i,j] = sum_k A[i,k] * B[k,j] in float64 from
 * bfloat16 bits.  A is row-major M x K; B is column-major K x N (element
 * (k, j) at j*K + k). */
void orc_gemm_bf16_sample(const uint16_t* A, const uint16_t* B, uint32_t K,
                          const uint32_t* rows, const uint32_t* cols,
                          uint32_t nsample, double* out);

/* Round-trip helpers used by the reduce definition; exposed for pinning. */
double   orc_bf16_to_f64(uint16_t bits);
double   orc_f16_to_f64(uint16_t bits);
uint16_t orc_f64_to_bf16(double x);
uint16_t orc_f64_to_f16(double x);

#ifdef __cplusplus
}
#endif
#endif
