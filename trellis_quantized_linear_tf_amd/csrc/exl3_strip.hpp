// Pieces shared by the linear kernels: the stream share load, the output
// store, and the strip finish (cross-wave sums, output butterflies, scale, svh).
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "What this changes": the waves' sums, the output rotation and
// svh follow the finish of the reference path.
#pragma once

#include "exl3_device.hpp"
#include "tf_exl3.h"

namespace tf_exl3 {

// Tile rows in flight per wave: about 4 KiB of stream per wave.
template <int BITS>
constexpr int prefetch_depth() {
  return BITS == 2 ? 8 : BITS == 3 ? 5 : BITS == 4 ? 4 : BITS == 8 ? 2 : 3;
}

// A lane's share of a tile row plus the first dword of the next lane's share,
// which completes the last windows (it lies in cache lines the wave loads
// anyway). The stream is read once, so the loads are nontemporal. `p` is the
// wave-uniform start of the strip's tile row (an SGPR pair), `off` the lane's
// dword offset and `nb` the next lane's (wrapping inside the tile), so the
// loads take the scalar-base + vector-offset form.
template <int BITS>
__device__ __forceinline__ void load_share(uint32_t (&dst)[BITS + 1], const uint32_t* __restrict__ p, int off,
                                           int nb) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) dst[i] = __builtin_nontemporal_load(p + off + i);
  dst[BITS] = __builtin_nontemporal_load(p + nb);
}

__device__ __forceinline__ void store_out(void* __restrict__ y, int y_dtype, size_t i, float v) {
  if (y_dtype == TF_DT_F32) {
    static_cast<float*>(y)[i] = v;
  } else if (y_dtype == TF_DT_F16) {
    static_cast<uint16_t*>(y)[i] = f32_to_f16_bits(v);
  } else {
    static_cast<uint16_t*>(y)[i] = f32_to_bf16_bits(v);
  }
}

// partial[(w * rstride + r) * 128 + col] holds wave w's sum for row r of the
// pass; after a barrier, wave w finishes rows r = w, w + WAVES, ... < nr:
// the waves' sums in wave order 0..WAVES-1, the fp32 output butterflies,
// RN32(. * s), RN32(. * svh), then the cast and store of y[r0 + r][strip cols].
template <int WAVES>
__device__ __forceinline__ void finish_strip(const float* partial, int rstride, int wave, int lane, int nr,
                                             int r0, int strip, int out_dim, const uint16_t* __restrict__ svh,
                                             void* __restrict__ y, int y_dtype) {
  const float s = bits_to_f32(kScaleBits);
  const int col = strip * kBlock + lane;
  const float g0 = f16_bits_to_f32(svh[col]);
  const float g1 = f16_bits_to_f32(svh[col + 64]);
  for (int r = wave; r < nr; r += WAVES) {
    float v0 = partial[r * kBlock + lane];
    float v1 = partial[r * kBlock + lane + 64];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      v0 = v0 + partial[(w * rstride + r) * kBlock + lane];
      v1 = v1 + partial[(w * rstride + r) * kBlock + lane + 64];
    }
    fwht128_wave(v0, v1);
    v0 = opaque(v0 * s);
    v1 = opaque(v1 * s);
    v0 = opaque(v0 * g0);
    v1 = opaque(v1 * g1);
    const size_t o = (size_t)(r0 + r) * out_dim + col;
    store_out(y, y_dtype, o, v0);
    store_out(y, y_dtype, o + 64, v1);
  }
}

}  // namespace tf_exl3
