/*
 * tf_exl3.h - C ABI of the MI355X (gfx950) EXL3 decode-row projection.
 *
 * The projection is the one described on the TensorFold pull request
 * "hip exl3: the input rotation and trellis linear for decode rows, under the
 * kernel contract", section "What this changes":
 *
 *   rot_in:  z = RN16( H128(x * suh) * s )      per 128-wide block of each row
 *   linear:  y = cast( svh * ( H128(z . W) * s ) ) per 128-wide block of outputs
 *
 * where H128 is the unscaled 128-point Walsh-Hadamard transform, s is the fp32
 * value of 1/sqrt(128) (multiplied, not divided), and W is an in_dim x out_dim
 * weight matrix stored as a K-bit shift-register trellis over 16 x 16 tiles and
 * decoded in registers through a multiplicative-hash codebook. The stream format
 * (bit order, window, value order, tile order, codebook constants) is fixed in
 * the comments of tf_exl3_linear below.
 *
 * Conventions for every call:
 *  - Data pointers are DEVICE pointers owned by the caller. The library
 *    allocates nothing, frees nothing and keeps no mutable global state; calls
 *    are thread-safe.
 *  - `stream` is a hipStream_t (NULL = the default stream). Launches are
 *    asynchronous; the caller synchronizes.
 *  - Arguments are checked on the host before anything is launched. On a
 *    refusal (negative status) nothing is launched and nothing is written.
 *  - No C++ exception crosses this interface.
 */
#ifndef TF_EXL3_H
#define TF_EXL3_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of rows and outputs. */
enum {
  TF_DT_F32 = 0,  /* IEEE binary32 */
  TF_DT_F16 = 1,  /* IEEE binary16 */
  TF_DT_BF16 = 2  /* bfloat16 (top half of binary32) */
};

/* Status codes. */
enum {
  TF_OK = 0,
  TF_E_BITS = -1,   /* bits not in {2, 3, 4, 5, 6, 8} */
  TF_E_SHAPE = -2,  /* a dimension < 128, not a multiple of 128, or a stream >= 4 GiB */
  TF_E_ROWS = -3,   /* rows < 0, or more than the launch grid holds: 1048560 for the linear (65535
                       passes of 16), fewer for project, rows * in_dim / 128 below 2^33 for rot_in */
  TF_E_DTYPE = -4,  /* element type outside the table above */
  TF_E_NULL = -5,   /* a required pointer is NULL */
  TF_E_ALIGN = -6,  /* trellis or z not 16-byte aligned, or a row buffer not element-aligned */
  TF_E_ALIAS = -7,  /* an output overlaps an input */
  TF_E_WAVES = -8,  /* waves not in {0, 4, 8} */
  TF_E_LAUNCH = -9  /* the HIP runtime reported an error at launch */
};

/*
 * rot_in: the input rotation ("What this changes", first item; the rounding
 * rules are the ones the page's "Checks on this head" section tests).
 *
 * For each row r and each 128-block b of in_dim:
 *   p_i = RN32(f32(x[r][128b+i]) * f32(suh[128b+i]))
 *   butterflies over p in stages h = 1, 2, 4, ..., 64: (p_i, p_i+h) <- (RN32(p_i + p_i+h),
 *     RN32(p_i - p_i+h)) for every i with (i & h) == 0
 *   z[r][128b+i] = RN16(RN32(p_i * s)),  s = RN32(1/sqrt(128)) = 0x3DB504F3
 * Two roundings at the end (fp32 product, then fp16), never one fused rounding.
 * RN is round-to-nearest-even; fp16 subnormals are kept; overflow gives inf.
 *
 *  x      [rows][in_dim], row-major, element type x_dtype (TF_DT_F32/F16/BF16)
 *  suh    [in_dim] fp16 input signs/scales
 *  z      [rows][in_dim] fp16 output, row-major, 16-byte aligned, must not overlap x
 *  rows   >= 0 (0 launches nothing); rows * in_dim / 128 below 2^33 (TF_E_ROWS)
 *  in_dim multiple of 128
 */
int tf_exl3_rot_in(const void* x, int x_dtype, const uint16_t* suh, uint16_t* z,
                   int rows, int in_dim, void* stream);

/*
 * linear: the trellis linear ("What this changes", second item).
 *
 *   acc[r][n] = sum over k of z[r][k] * W[k][n], fp16 products summed in fp32
 *   y[r][128c+j] = cast_y( RN32( RN32(H128(acc[r][128c..])_j * s) * f32(svh[128c+j]) ) )
 *
 * A row's sum is a chain of v_dot2_f32_f16 over (k, k+1) pairs in a fixed
 * order that depends only on (in_dim, waves), never on how many rows share the
 * launch: a row's output bits are the same alone, in any window of rows and in
 * any pass. Rows are processed 16 per pass; rows > 16 run ceil(rows/16) passes.
 *
 * Stream format (tile layout). W is in_dim x out_dim; tile (kt, nt) holds
 * W[16kt .. 16kt+15][16nt .. 16nt+15] and is 8*bits little-endian uint32 words
 * starting at word (kt * out_dim/16 + nt) * 8*bits. Bit i of a tile is
 * (word[i >> 5] >> (i & 31)) & 1. Value j = 0..255 of a tile sits at k = j % 16,
 * n = j / 16, and its state is the 16-bit window of tile bits j*bits .. j*bits+15
 * (bit t of the state = tile bit (j*bits + t) mod 256*bits; the window wraps).
 * Codebook: x = (state * 0x9E3779) mod 2^32; h = sum of the four bytes of x;
 * w = RN16((1024 + h) * A + B) in one fused multiply-add, A = fp16 0x1EEE,
 * B = fp16 0xC931.
 *
 *  bits     2, 3, 4, 5, 6 or 8
 *  rows     >= 0 (0 launches nothing)
 *  in_dim, out_dim  multiples of 128; in_dim*out_dim*bits/8 < 2^32
 *  z        [rows][in_dim] fp16 (rot_in's output), 16-byte aligned
 *  trellis  tf_exl3_trellis_bytes(bits, in_dim, out_dim) bytes, 16-byte aligned
 *  svh      [out_dim] fp16 output signs/scales
 *  y        [rows][out_dim], element type y_dtype; must not overlap z, trellis or svh
 *  waves    waves per 128-column block: 0 = planner's choice (8 if out_dim >= 8192,
 *           else 4), or 4, or 8. The wave count fixes the summation order.
 */
int tf_exl3_linear(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                   const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                   int waves, void* stream);

/*
 * linear_strips: tf_exl3_linear on a stream in the strips layout (TensorFold
 * pull request "hip exl3: the input rotation and trellis linear for decode
 * rows", "Checks on this head": the identity check runs on the checkpoint's tile
 * layout at 4 waves and on a strips layout at 8). The strips layout holds the same tiles ordered strip
 * by strip: tile (kt, nt) starts at word ((nt / 8) * in_dim/16 + kt) * 8 + nt % 8,
 * times 8*bits, so each 128-column strip is one contiguous stream of
 * in_dim/16 * 256*bits bytes. Same arguments, refusals, waves and summation
 * order as tf_exl3_linear; for a stream and its tf_exl3_repack_strips image the
 * outputs are bit-identical.
 */
int tf_exl3_linear_strips(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                          const uint32_t* strips, const uint16_t* svh, void* y, int y_dtype,
                          int waves, void* stream);

/*
 * repack_strips: writes the strips-layout image of a tile-layout stream
 * (tf_exl3_trellis_bytes(bits, in_dim, out_dim) bytes each; both device, 16-byte
 * aligned, not overlapping; asynchronous on `stream`). Refusals: TF_E_BITS,
 * TF_E_SHAPE, TF_E_NULL, TF_E_ALIGN, TF_E_ALIAS (the buffers overlap; the repack
 * is not in place), TF_E_LAUNCH.
 */
int tf_exl3_repack_strips(int bits, int in_dim, int out_dim, const uint32_t* tiles, uint32_t* strips,
                          void* stream);

/*
 * linear_prompt: the prompt path, bit-equal to tf_exl3_linear (TensorFold pull
 * request "hip exl3: the input rotation and trellis linear for decode rows",
 * "Known limits": the prompt path that follows the decode rows is to give the
 * same bits as this linear). Same arguments, refusals, stream format, waves and
 * summation order as tf_exl3_linear; full passes carry 32 rows instead of 16,
 * so each tile row is decoded once for twice the rows, and the remaining
 * rows % 32 run as tf_exl3_linear's passes. Every output row is bit-identical
 * to tf_exl3_linear's for the same (z row, trellis, svh, waves).
 */
int tf_exl3_linear_prompt(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                          const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                          int waves, void* stream);

/*
 * linear_mfma: the same projection with the same arguments, refusals, stream
 * format and finish, but the sums over k run on the matrix cores
 * (v_mfma_f32_16x16x32_f16 over pairs of tile rows, one instruction shape for
 * every pass of 1 to 16 rows) instead of v_dot2 chains, so the vector ALUs only
 * decode and the time grows slowly with the rows. At 4 waves, a matrix with
 * fewer than 256 strips runs a column-split form (twice the waves per strip, the
 * same MFMAs per column, the same bits). Its k order per
 * output is fixed by (in_dim, waves) and never depends on the rows sharing the
 * launch; it is a different fixed order from tf_exl3_linear's, so the two agree
 * to the float64 gate, not bit for bit. (The page's "Known limits" and the
 * multi-row work it announces are the use; the page's own kernels sum with dot2.)
 */
int tf_exl3_linear_mfma(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                        const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                        int waves, void* stream);

/*
 * project: rot_in and the linear in one launch, y = linear(rot_in(x)).
 * Source: the same page, "What this changes": the projection is the two calls in
 * sequence, rot_in's fp16 rows feeding the linear; this entry runs both as one
 * launch with rot_in's arithmetic unchanged. Every workgroup rotates its pass's rows into LDS with the same arithmetic as
 * tf_exl3_rot_in and then runs tf_exl3_linear's own tile-row walk, so y is bit
 * for bit what tf_exl3_rot_in followed by tf_exl3_linear gives, with one launch
 * and no z buffer. Each workgroup recomputes the rotation of its rows (about 5%
 * more vector work than the linear for one 5120-wide row: on the LM head about what
 * the saved launch is worth; on a one-strip layer, whose step is mostly launch
 * latency, the single launch is the faster route). Passes hold as many rows as fit in 48 KiB
 * of LDS (tf_exl3_project_pass_rows: 2 at in_dim 5120) and each pass streams the
 * weights once, so beyond a pass's rows tf_exl3_rot_in + tf_exl3_linear, which
 * stream them once per 16 rows, are the faster route.
 *
 *  x       [rows][in_dim], element type x_dtype; suh [in_dim] fp16
 *  trellis, svh, y, y_dtype, waves: as tf_exl3_linear; y must not overlap any input
 */
int tf_exl3_project(int bits, int rows, int in_dim, int out_dim, const void* x, int x_dtype,
                    const uint16_t* suh, const uint32_t* trellis, const uint16_t* svh, void* y,
                    int y_dtype, int waves, void* stream);

/* Rows per pass tf_exl3_project uses for these arguments (host only), or a refusal:
 * TF_E_SHAPE if even one row does not fit, TF_E_ROWS, TF_E_WAVES. The pass size is
 * the single launch's own planning (its LDS holds a pass's rotated rows); the rows
 * per pass of the page's linear ("What this changes": 1 to 16 rows a pass) bound it. */
int tf_exl3_project_pass_rows(int rows, int in_dim, int out_dim, int waves);

/*
 * Launch plan the linear would use (host only; no GPU needed). Source: the same
 * page, "What this changes" (the launches refuse the shapes they cannot run
 * ("fits"), map the width to a kernel ("widthIndex") and choose the wave count,
 * with no K split, all host-tested) and "Kernel contract" (the plan's 8-wave edge:
 * 8192 output columns by 1024 run on 8 waves, 8064 by 1024 on 4).
 */
typedef struct {
  int width_index;    /* position of bits in {2, 3, 4, 5, 6, 8} */
  int waves;          /* waves per block */
  int threads;        /* threads per block (64 * waves) */
  int grid_x;         /* blocks per pass = out_dim / 128 */
  int passes;         /* ceil(rows / 16) */
  int rows_last_pass; /* rows in the last pass (1..16), 0 when rows == 0 */
  int rows_kernel;    /* row capacity of the variant for the first launch: 1, 2, 4, 8, 12 or 16
                         (up to 4 rows z arrives through scalar loads, above through LDS) */
  int lds_bytes;      /* LDS per block of that launch: partial sums waves * min(rows_kernel, 16)
                         * 512 bytes, plus z slots (w * 2 * rows_kernel * 16 bytes, w = the block's
                         waves) above 4 rows or when column_split */
  int column_split;   /* 1 if that launch runs the column-split variant: a launch with fewer than
                         2048 waves in flight gets twice the waves per block (threads = 128 *
                         waves), each lane one column, with the same sums in the same order */
} tf_exl3_plan;

/* Fills *out with the plan for these arguments, or returns the refusal the linear
 * would return (TF_E_BITS, TF_E_SHAPE, TF_E_ROWS, TF_E_WAVES, TF_E_NULL if out is NULL). */
int tf_exl3_linear_plan(int bits, int rows, int in_dim, int out_dim, int waves,
                        tf_exl3_plan* out);

/* Bytes of a trellis stream: in_dim * out_dim * bits / 8 (0 for a refused shape).
 * Source: the same page, "Kernel contract": the linear's static LDS records hold
 * eight tiles per wave, 32 * bits bytes per 16 x 16 tile, i.e. bits bits per weight. */
size_t tf_exl3_trellis_bytes(int bits, int in_dim, int out_dim);

/* Static text for a status code (never NULL). The refusals are the planner's
 * ("What this changes": fits, widthIndex, waves) and this interface's own pointer,
 * alignment and overlap checks. */
const char* tf_exl3_status_string(int status);

/*
 * Test entry points. They run the same device decode functions as the linear.
 * Source: the same page, "Checks on this head": the linear's kernel test decodes
 * every width's weights bit for bit as the format's unpack does, and its window
 * test compares a row's bits across launches; these entries expose the decode
 * and the variant choice so the tests can check both against the oracle.
 *
 * debug_decode_states: w[i] = codebook(states[i]) as fp16 bits, i < n.
 *   states, w: device arrays of n uint16; n >= 0.
 * debug_decode_tiles: W[k][n] (fp16 bits, [in_dim][out_dim] row-major) decoded from
 *   a tile-layout stream through the linear's own load, window and codebook path.
 */
int tf_exl3_debug_decode_states(const uint16_t* states, uint16_t* w, int n, void* stream);
/* debug_linear_split: tf_exl3_linear with the variant forced for every launch
 * (split 0: the regular kernels, 1: the column-split ones), so the two can be
 * compared bit for bit on the same shape; split outside {0, 1} is TF_E_SHAPE. */
int tf_exl3_debug_linear_split(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                               const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                               int waves, int split, void* stream);
int tf_exl3_debug_decode_tiles(int bits, int in_dim, int out_dim, const uint32_t* trellis,
                               uint16_t* w, void* stream);
/* debug_linear_mfma_split: tf_exl3_linear_mfma with its form forced at 4 waves (split 0:
 * each strip's 8 column tiles on every wave, 1: in halves over twice the waves); at 8 waves
 * split must be 0. Both forms give the same bits, which the tests check; split outside
 * {0, 1}, or 1 at 8 waves, is TF_E_SHAPE. */
int tf_exl3_debug_linear_mfma_split(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                                    const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                    int waves, int split, void* stream);

/*
 * Calibration entry points for measurement (not part of the projection, and
 * defined by no page: they give the device's own copy and read rates, against
 * which the linear's HBM traffic counters and bandwidth are scaled). Both
 * move 16 bytes per lane in wave-contiguous 1 KiB runs, the access form of the
 * linear's weight stream.
 *
 * calib_copy: dst[0 .. bytes) = src[0 .. bytes); bytes a multiple of 16, both
 *   16-byte aligned and disjoint; `blocks` workgroups of 256 threads (>= 1).
 * calib_stream_read: reads src[0 .. bytes) and writes one XOR word per thread
 *   to out, which must hold blocks * 256 uint32 and not overlap src.
 */
int tf_exl3_calib_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream);
int tf_exl3_calib_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TF_EXL3_H */
