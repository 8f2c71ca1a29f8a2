// C ABI of the EXL3 decode-row projection: argument checks, the launch planner
// and status strings. Host code only; the kernels live in the .hip files.
//
// The planner follows the TensorFold pull request "hip exl3: the input rotation
// and trellis linear for decode rows": "What this changes" (launches refuse the
// shapes they cannot run, map the width to a kernel and choose the wave count;
// dense plan, no K split) and "Kernel contract" (8 waves from 8192 output
// columns up, 4 waves below: 8064 x 1024 runs on 4, 8192 x 1024 on 8).
#include <stddef.h>
#include <stdint.h>

#include "exl3_launch.hpp"
#include "tf_exl3.h"

namespace {

constexpr int kMaxRowsPerPass = 16;
// Passes are the grid's second dimension (at most 65535 workgroups).
constexpr int kMaxPasses = 65535;
constexpr int kMaxRows = kMaxPasses * kMaxRowsPerPass;
constexpr int kWaveEdgeColumns = 8192;

int width_index(int bits) {
  switch (bits) {
    case 2: return 0;
    case 3: return 1;
    case 4: return 2;
    case 5: return 3;
    case 6: return 4;
    case 8: return 5;
    default: return -1;
  }
}

bool dim_ok(int d) { return d >= 128 && d % 128 == 0; }

// Stream bytes, or 0 when the shape is refused.
uint64_t stream_bytes(int bits, int in_dim, int out_dim) {
  if (width_index(bits) < 0 || !dim_ok(in_dim) || !dim_ok(out_dim)) return 0;
  const uint64_t b = (uint64_t)in_dim * (uint64_t)out_dim * (uint64_t)bits / 8u;
  return b < (1ull << 32) ? b : 0;
}

int plan_waves(int out_dim, int waves) {
  if (waves == 0) return out_dim >= kWaveEdgeColumns ? 8 : 4;
  return (waves == 4 || waves == 8) ? waves : -1;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (na == 0 || nb == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

size_t elem_size(int dt) { return dt == TF_DT_F32 ? 4 : 2; }

bool dtype_ok(int dt) { return dt == TF_DT_F32 || dt == TF_DT_F16 || dt == TF_DT_BF16; }

}  // namespace

extern "C" {

size_t tf_exl3_trellis_bytes(int bits, int in_dim, int out_dim) {
  return (size_t)stream_bytes(bits, in_dim, out_dim);
}

const char* tf_exl3_status_string(int status) {
  switch (status) {
    case TF_OK: return "ok";
    case TF_E_BITS: return "bits must be 2, 3, 4, 5, 6 or 8 (widthIndex)";
    case TF_E_SHAPE: return "in_dim and out_dim must be multiples of 128, and the stream under 4 GiB (fits)";
    case TF_E_ROWS:
      return "rows must be >= 0 and fit the launch grid (at most 1048560 = 65535 passes of 16 rows for the linear)";
    case TF_E_DTYPE: return "element type must be TF_DT_F32, TF_DT_F16 or TF_DT_BF16";
    case TF_E_NULL: return "a required pointer is NULL";
    case TF_E_ALIGN: return "trellis and z must be 16-byte aligned and row buffers element-aligned";
    case TF_E_ALIAS: return "an output buffer overlaps an input buffer";
    case TF_E_WAVES: return "waves must be 0 (auto), 4 or 8";
    case TF_E_LAUNCH: return "the HIP runtime reported an error at launch";
    default: return "unknown status";
  }
}

int tf_exl3_linear_plan(int bits, int rows, int in_dim, int out_dim, int waves, tf_exl3_plan* out) {
  if (out == nullptr) return TF_E_NULL;
  const int wi = width_index(bits);
  if (wi < 0) return TF_E_BITS;
  if (stream_bytes(bits, in_dim, out_dim) == 0) return TF_E_SHAPE;
  if (rows < 0 || rows > kMaxRows) return TF_E_ROWS;
  const int w = plan_waves(out_dim, waves);
  if (w < 0) return TF_E_WAVES;
  tf_exl3_plan p;
  p.width_index = wi;
  p.waves = w;
  p.threads = 64 * w;
  p.grid_x = out_dim / 128;
  p.passes = (rows + kMaxRowsPerPass - 1) / kMaxRowsPerPass;
  p.rows_last_pass = rows == 0 ? 0 : rows - (p.passes - 1) * kMaxRowsPerPass;
  p.rows_kernel = rows == 0 ? 0 : tf_exl3::rows_bucket(rows >= kMaxRowsPerPass ? kMaxRowsPerPass : rows);
  // The first launch: the full passes, or the one pass of the remaining rows.
  const int first_passes = rows >= kMaxRowsPerPass ? rows / kMaxRowsPerPass : 1;
  p.column_split = rows == 0 ? 0 : (tf_exl3::column_split(out_dim, first_passes, w) ? 1 : 0);
  p.lds_bytes = rows == 0 ? 0
                : p.column_split ? tf_exl3::linear_cs_lds_bytes(w, p.rows_kernel)
                                 : tf_exl3::linear_lds_bytes(w, p.rows_kernel);
  p.threads = (p.column_split ? 128 : 64) * w;
  *out = p;
  return TF_OK;
}

int tf_exl3_rot_in(const void* x, int x_dtype, const uint16_t* suh, uint16_t* z, int rows, int in_dim,
                   void* stream) {
  if (!dtype_ok(x_dtype)) return TF_E_DTYPE;
  if (!dim_ok(in_dim)) return TF_E_SHAPE;
  if (rows < 0) return TF_E_ROWS;
  // One wave per 128-block, four per workgroup: the grid must stay below 2^31 workgroups.
  if ((long long)rows * (in_dim / 128) > 4LL * 0x7FFFFFFFLL) return TF_E_ROWS;
  if (rows == 0) return TF_OK;
  if (x == nullptr || suh == nullptr || z == nullptr) return TF_E_NULL;
  if (!aligned(z, 16) || !aligned(x, elem_size(x_dtype)) || !aligned(suh, 2)) return TF_E_ALIGN;
  const size_t n = (size_t)rows * (size_t)in_dim;
  if (overlap(x, n * elem_size(x_dtype), z, n * 2) || overlap(suh, (size_t)in_dim * 2, z, n * 2))
    return TF_E_ALIAS;
  const hipError_t e =
      tf_exl3::launch_rot_in(x, x_dtype, suh, z, rows, in_dim, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

namespace {

// Checks shared by both engines; TF_OK means the launch may proceed (rows > 0).
int linear_checks(int bits, int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                  const uint16_t* svh, void* y, int y_dtype, int waves, tf_exl3_plan* plan) {
  const int st = tf_exl3_linear_plan(bits, rows, in_dim, out_dim, waves, plan);
  if (st != TF_OK) return st;
  if (!dtype_ok(y_dtype)) return TF_E_DTYPE;
  if (rows == 0) return TF_OK;
  if (z == nullptr || trellis == nullptr || svh == nullptr || y == nullptr) return TF_E_NULL;
  if (!aligned(z, 16) || !aligned(trellis, 16) || !aligned(svh, 2) || !aligned(y, elem_size(y_dtype)))
    return TF_E_ALIGN;
  const size_t ny = (size_t)rows * (size_t)out_dim * elem_size(y_dtype);
  if (overlap(y, ny, z, (size_t)rows * in_dim * 2) ||
      overlap(y, ny, trellis, (size_t)stream_bytes(bits, in_dim, out_dim)) ||
      overlap(y, ny, svh, (size_t)out_dim * 2))
    return TF_E_ALIAS;
  return TF_OK;
}

}  // namespace

int tf_exl3_linear(int bits, int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                   const uint16_t* svh, void* y, int y_dtype, int waves, void* stream) {
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK || rows == 0) return st;
  const hipError_t e = tf_exl3::launch_linear(bits, plan.waves, rows, in_dim, out_dim, z, trellis, svh, y,
                                              y_dtype, 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_debug_linear_split(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                               const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int waves,
                               int split, void* stream) {
  if (split != 0 && split != 1) return TF_E_SHAPE;
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK || rows == 0) return st;
  const hipError_t e = tf_exl3::launch_linear(bits, plan.waves, rows, in_dim, out_dim, z, trellis, svh, y,
                                              y_dtype, 0, static_cast<hipStream_t>(stream), split);
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_debug_linear_mfma_split(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                                    const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int waves,
                                    int split, void* stream) {
  if (split != 0 && split != 1) return TF_E_SHAPE;
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK) return st;
  if (split != 0 && plan.waves != 4) return TF_E_SHAPE;
  if (rows == 0) return TF_OK;
  const hipError_t e = tf_exl3::launch_linear_mfma(bits, plan.waves, rows, in_dim, out_dim, z, trellis, svh, y,
                                                   y_dtype, static_cast<hipStream_t>(stream), split);
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_linear_strips(int bits, int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* strips,
                          const uint16_t* svh, void* y, int y_dtype, int waves, void* stream) {
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, strips, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK || rows == 0) return st;
  const hipError_t e = tf_exl3::launch_linear(bits, plan.waves, rows, in_dim, out_dim, z, strips, svh, y,
                                              y_dtype, 1, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_repack_strips(int bits, int in_dim, int out_dim, const uint32_t* tiles, uint32_t* strips,
                          void* stream) {
  if (width_index(bits) < 0) return TF_E_BITS;
  const uint64_t n = stream_bytes(bits, in_dim, out_dim);
  if (n == 0) return TF_E_SHAPE;
  if (tiles == nullptr || strips == nullptr) return TF_E_NULL;
  if (!aligned(tiles, 16) || !aligned(strips, 16)) return TF_E_ALIGN;
  if (overlap(tiles, (size_t)n, strips, (size_t)n)) return TF_E_ALIAS;
  const hipError_t e =
      tf_exl3::launch_repack_strips(bits, in_dim, out_dim, tiles, strips, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_linear_prompt(int bits, int rows, int in_dim, int out_dim, const uint16_t* z,
                          const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int waves,
                          void* stream) {
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK || rows == 0) return st;
  const hipError_t e = tf_exl3::launch_linear_prompt(bits, plan.waves, rows, in_dim, out_dim, z, trellis, svh,
                                                     y, y_dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_linear_mfma(int bits, int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                        const uint16_t* svh, void* y, int y_dtype, int waves, void* stream) {
  tf_exl3_plan plan;
  const int st = linear_checks(bits, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, waves, &plan);
  if (st != TF_OK || rows == 0) return st;
  const hipError_t e = tf_exl3::launch_linear_mfma(bits, plan.waves, rows, in_dim, out_dim, z, trellis, svh,
                                                   y, y_dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_project_pass_rows(int rows, int in_dim, int out_dim, int waves) {
  if (!dim_ok(in_dim) || !dim_ok(out_dim)) return TF_E_SHAPE;
  if (rows < 0) return TF_E_ROWS;
  const int w = plan_waves(out_dim, waves);
  if (w < 0) return TF_E_WAVES;
  const int p = tf_exl3::project_pass_rows(rows, w, in_dim);
  return p > 0 ? p : TF_E_SHAPE;
}

int tf_exl3_project(int bits, int rows, int in_dim, int out_dim, const void* x, int x_dtype, const uint16_t* suh,
                    const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int waves, void* stream) {
  tf_exl3_plan plan;
  const int st = tf_exl3_linear_plan(bits, rows, in_dim, out_dim, waves, &plan);
  if (st != TF_OK) return st;
  if (!dtype_ok(x_dtype) || !dtype_ok(y_dtype)) return TF_E_DTYPE;
  const int pass_rows = tf_exl3::project_pass_rows(rows, plan.waves, in_dim);
  if (pass_rows == 0) return TF_E_SHAPE;
  if (rows > 0 && (rows - 1) / pass_rows + 1 > kMaxPasses) return TF_E_ROWS;
  if (rows == 0) return TF_OK;
  if (x == nullptr || suh == nullptr || trellis == nullptr || svh == nullptr || y == nullptr) return TF_E_NULL;
  if (!aligned(x, elem_size(x_dtype)) || !aligned(suh, 2) || !aligned(trellis, 16) || !aligned(svh, 2) ||
      !aligned(y, elem_size(y_dtype)))
    return TF_E_ALIGN;
  const size_t ny = (size_t)rows * (size_t)out_dim * elem_size(y_dtype);
  if (overlap(y, ny, x, (size_t)rows * in_dim * elem_size(x_dtype)) || overlap(y, ny, suh, (size_t)in_dim * 2) ||
      overlap(y, ny, trellis, (size_t)stream_bytes(bits, in_dim, out_dim)) ||
      overlap(y, ny, svh, (size_t)out_dim * 2))
    return TF_E_ALIAS;
  const hipError_t e = tf_exl3::launch_project(bits, plan.waves, pass_rows, rows, in_dim, out_dim, x, x_dtype, suh,
                                               trellis, svh, y, y_dtype, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_debug_decode_states(const uint16_t* states, uint16_t* w, int n, void* stream) {
  if (n < 0) return TF_E_SHAPE;
  if (n == 0) return TF_OK;
  if (states == nullptr || w == nullptr) return TF_E_NULL;
  if (!aligned(states, 2) || !aligned(w, 2)) return TF_E_ALIGN;
  if (overlap(states, (size_t)n * 2, w, (size_t)n * 2)) return TF_E_ALIAS;
  const hipError_t e = tf_exl3::launch_decode_states(states, w, n, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_debug_decode_tiles(int bits, int in_dim, int out_dim, const uint32_t* trellis, uint16_t* w,
                               void* stream) {
  if (width_index(bits) < 0) return TF_E_BITS;
  const uint64_t nb = stream_bytes(bits, in_dim, out_dim);
  if (nb == 0) return TF_E_SHAPE;
  if (trellis == nullptr || w == nullptr) return TF_E_NULL;
  if (!aligned(trellis, 16) || !aligned(w, 2)) return TF_E_ALIGN;
  if (overlap(trellis, (size_t)nb, w, (size_t)in_dim * out_dim * 2)) return TF_E_ALIAS;
  const hipError_t e =
      tf_exl3::launch_decode_tiles(bits, in_dim, out_dim, trellis, w, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_calib_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (bytes % 16 != 0) return TF_E_SHAPE;
  if (blocks < 1) return TF_E_SHAPE;
  if (bytes == 0) return TF_OK;
  if (src == nullptr || dst == nullptr) return TF_E_NULL;
  if (!aligned(src, 16) || !aligned(dst, 16)) return TF_E_ALIGN;
  if (overlap(src, bytes, dst, bytes)) return TF_E_ALIAS;
  const hipError_t e = tf_exl3::launch_copy(src, dst, bytes, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

int tf_exl3_calib_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, void* stream) {
  if (bytes % 16 != 0) return TF_E_SHAPE;
  if (blocks < 1) return TF_E_SHAPE;
  if (src == nullptr || out == nullptr) return TF_E_NULL;
  if (!aligned(src, 16) || !aligned(out, 4)) return TF_E_ALIGN;
  if (overlap(src, bytes, out, (size_t)blocks * 256 * 4)) return TF_E_ALIAS;
  const hipError_t e = tf_exl3::launch_stream_read(src, bytes, out, blocks, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? TF_OK : TF_E_LAUNCH;
}

}  // extern "C"
