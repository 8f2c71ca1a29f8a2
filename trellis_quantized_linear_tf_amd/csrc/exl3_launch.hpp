// Internal launch interface between the C ABI (exl3_abi.cpp) and the kernels.
// Arguments reaching these functions have already been checked by the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace tf_exl3 {

// Row capacity of the linear kernel variant that serves `rows` (1..16) rows.
inline int rows_bucket(int rows) {
  return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : rows <= 12 ? 12 : 16;
}

// Up to this many rows a pass takes z through scalar loads; above it, through
// a wave-private LDS slot (one vector load per lane per tile row).
constexpr int kScalarZRows = 4;

// LDS bytes of one linear block: the waves' partial sums [waves][min(rows, 16)][128]
// fp32, plus the z slots [waves][2 * rows] of 16 bytes when z goes through LDS.
inline int linear_lds_bytes(int waves, int rows_cap) {
  const int fr = rows_cap < 16 ? rows_cap : 16;
  return waves * fr * 128 * 4 + (rows_cap > kScalarZRows ? waves * 2 * rows_cap * 16 : 0);
}

// Row capacity of the fused projection's variant for `rows` rows (powers of two).
inline int pow2_bucket(int rows) { return rows <= 1 ? 1 : rows <= 2 ? 2 : rows <= 4 ? 4 : rows <= 8 ? 8 : 16; }

// Fused projection: LDS of one workgroup holds its pass's z rows (fp16) and the
// waves' partial sums; passes carry as many rows (1, 2, 4, 8 or 16) as fit in
// kProjectLdsBudget, so several workgroups still share a CU.
constexpr size_t kProjectLdsBudget = 48 * 1024;

inline size_t project_lds_bytes(int waves, int rows_cap, int in_dim) {
  return (size_t)rows_cap * in_dim * 2 + (size_t)waves * rows_cap * 128 * 4;
}

// Rows per pass of the fused projection for `rows` rows (0 if even one row does not fit).
inline int project_pass_rows(int rows, int waves, int in_dim) {
  int cap = 0;
  for (int nr = 16; nr >= 1; nr /= 2) {
    if (project_lds_bytes(waves, nr, in_dim) <= kProjectLdsBudget) {
      cap = nr;
      break;
    }
  }
  if (cap == 0 || rows <= 0) return cap;
  const int want = pow2_bucket(rows < cap ? rows : cap);
  return want < cap ? want : cap;
}

hipError_t launch_project(int bits, int waves, int nr_cap, int rows, int in_dim, int out_dim, const void* x,
                          int x_dtype, const uint16_t* suh, const uint32_t* trellis, const uint16_t* svh, void* y,
                          int y_dtype, hipStream_t stream);

hipError_t launch_rot_in(const void* x, int x_dtype, const uint16_t* suh, uint16_t* z, int rows,
                         int in_dim, hipStream_t stream);

// A launch of the linear with fewer than this many waves in flight runs the
// column-split variant (twice the waves, the same bits): two waves per SIMD.
constexpr long long kSplitBelowWaves = 2048;

inline bool column_split(int out_dim, int passes, int waves) {
  return (long long)(out_dim / 128) * passes * waves < kSplitBelowWaves;
}

// LDS bytes of one column-split block (partial sums and the z slots of 2 * waves waves).
inline int linear_cs_lds_bytes(int waves, int rows_cap) {
  const int fr = rows_cap < 16 ? rows_cap : 16;
  return waves * fr * 128 * 4 + 2 * waves * 2 * rows_cap * 16;
}

// layout: 0 = tile layout, 1 = strips layout (kLayoutTiles / kLayoutStrips).
// split: -1 = by column_split(), 0 = never, 1 = always (a test hook: both give the same bits).
hipError_t launch_linear(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                         const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int layout,
                         hipStream_t stream, int split = -1);

// One launch of the column-split variant: grid (strips, passes) of row capacity nr_cap.
void launch_linear_cs(int bits, int waves, int nr_cap, dim3 grid, const uint16_t* z, const uint32_t* trellis,
                      const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim, int out_dim, int layout,
                      hipStream_t stream);

hipError_t launch_repack_strips(int bits, int in_dim, int out_dim, const uint32_t* tiles, uint32_t* strips,
                                hipStream_t stream);

// Rows per full pass of the prompt path (the rest runs as decode passes).
constexpr int kPromptRowsPerPass = 32;

hipError_t launch_linear_prompt(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                                const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                hipStream_t stream);

// The matrix-core linear at 4 waves runs its column-split form (each strip's
// columns in two halves over twice the waves, the same bits) where the first form
// would put fewer waves than SIMDs in flight.
constexpr long long kMfmaSplitBelowWaves = 1024;

inline int mfma_column_parts(int out_dim, int waves) {
  return waves == 4 && (long long)(out_dim / 128) * waves < kMfmaSplitBelowWaves ? 2 : 1;
}

// split: -1 = by mfma_column_parts(), 0 = the first form, 1 = halves (4 waves only).
hipError_t launch_linear_mfma(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                              const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                              hipStream_t stream, int split = -1);

hipError_t launch_decode_states(const uint16_t* states, uint16_t* w, int n, hipStream_t stream);

hipError_t launch_decode_tiles(int bits, int in_dim, int out_dim, const uint32_t* trellis,
                               uint16_t* w, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream);

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t stream);

}  // namespace tf_exl3
