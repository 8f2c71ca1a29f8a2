// Pieces shared by the linear kernels: the stream share load, the output
// store, and the strip finish (cross-wave sums, output butterflies, scale, svh).
//
// Source: TensorFold pull request "hip exl3: the input rotation and trellis
// linear for decode rows", section "What this changes" (the block's finish: the
// wave partials are added, then rotated, scaled and multiplied by svh in the
// same order as the input rotation's arithmetic).
#pragma once

#include <type_traits>

#include "exl3_device.hpp"
#include "tf_exl3.h"

namespace tf_exl3 {

// Stream layouts. Both store a strip's tile row (its 8 tiles, 64 * BITS words)
// contiguously; the tile layout puts whole tile rows (every strip) one after
// another, the strips layout puts each strip's tile rows together, so a strip
// is one contiguous stream.
constexpr int kLayoutTiles = 0;
constexpr int kLayoutStrips = 1;

struct StreamStrides {
  size_t row;    // words from a strip's tile row kt to kt + 1
  size_t strip;  // words from strip s's tile row kt to strip s + 1's
};

template <int BITS>
__device__ __forceinline__ StreamStrides stream_strides(int layout, int in_dim, int out_dim) {
  const size_t unit = 64 * BITS;
  if (layout == kLayoutStrips) return {unit, (size_t)(in_dim / 16) * unit};
  return {(size_t)(out_dim / 128) * unit, unit};
}

// Tile rows in flight per wave: about 4 KiB of stream per wave.
template <int BITS>
constexpr int prefetch_depth() {
  return BITS == 2 ? 8 : BITS == 3 ? 5 : BITS == 4 ? 4 : BITS == 8 ? 2 : 3;
}

// A lane's share of a tile row: BITS dwords (decode_lane fetches the next
// lane's first dword from that lane). The stream is read once, so the loads are
// nontemporal. `p` is the wave-uniform start of the strip's tile row (an SGPR
// pair) and `off` the lane's dword offset, so the loads take the scalar-base +
// vector-offset form.
template <int BITS>
__device__ __forceinline__ void load_share(uint32_t (&dst)[BITS], const uint32_t* __restrict__ p, int off) {
#pragma unroll
  for (int i = 0; i < BITS; ++i) dst[i] = __builtin_nontemporal_load(p + off + i);
}

// One tile row of the strip for one wave: decode 32 weights per lane and chain
// the dot products of every row.
template <int BITS, int WAVES, int NR>
__device__ __forceinline__ void tile_row_step(const uint32_t (&w)[BITS], int i,
                                              const uint32_t* const (&zrow)[NR], float (&acc)[NR][2]) {
  half2_t wp[2][8];
  decode_lane<BITS>(w, wp);
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const uint32_t* zp = zrow[r] + i * (WAVES * 8);
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const half2_t zz = __builtin_bit_cast(half2_t, zp[p]);
      acc[r][0] = __builtin_amdgcn_fdot2(zz, wp[0][p], acc[r][0], false);
      acc[r][1] = __builtin_amdgcn_fdot2(zz, wp[1][p], acc[r][1], false);
    }
  }
}

// The wave's walk over its tile rows for the v_dot2 engine. Step i (0 <= i <
// iters) is tile row kt = wave + i * WAVES. A ring of PF + 1 slots keeps PF steps
// in flight: step i decodes slot i % (PF + 1) while the load for step i + PF goes
// to the slot step i - 1 has just freed. Addresses past the last step are
// clamped to it, so the ring needs no branches and the wait counts stay exact.
// prime() issues the first PF loads; run() walks all steps. zrow[r] points at
// row r's inputs as (k, k+1) dword pairs, offset to this wave's first tile row
// (global memory or LDS).
template <int BITS, int WAVES, int NR>
struct StreamWalk {
  static constexpr int PF = prefetch_depth<BITS>();
  static constexpr int RING = PF + 1;
  const uint32_t* __restrict__ tp;
  size_t step_words;
  int off, iters;
  uint32_t ring[RING][BITS];

  __device__ __forceinline__ const uint32_t* share(int i) const {
    return tp + (size_t)min(i, iters - 1) * step_words;
  }

  __device__ __forceinline__ void prime() {
#pragma unroll
    for (int d = 0; d < PF; ++d) load_share<BITS>(ring[d], share(d), off);
  }

  __device__ __forceinline__ void run(const uint32_t* const (&zrow)[NR], float (&acc)[NR][2]) {
    int it = 0;
    for (; it + RING <= iters; it += RING) {
#pragma unroll
      for (int d = 0; d < RING; ++d) {
        load_share<BITS>(ring[(d + PF) % RING], share(it + d + PF), off);
        tile_row_step<BITS, WAVES, NR>(ring[d], it + d, zrow, acc);
      }
    }
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      if (it + d < iters) tile_row_step<BITS, WAVES, NR>(ring[d], it + d, zrow, acc);
    }
  }
};

// Runs step(slot, i) for i = 0 .. iters - 1, where slot = i % RING arrives as a
// std::integral_constant, so register rings indexed by it stay in registers.
template <int D, int RING, class F>
__device__ __forceinline__ void steps_from(F& step, int it, int iters, bool tail) {
  if constexpr (D < RING) {
    if (!tail || it + D < iters) step(std::integral_constant<int, D>{}, it + D);
    steps_from<D + 1, RING>(step, it, iters, tail);
  }
}

template <int RING, class F>
__device__ __forceinline__ void step_loop(int iters, F& step) {
  int it = 0;
  for (; it + RING <= iters; it += RING) steps_from<0, RING>(step, it, iters, false);
  steps_from<0, RING>(step, it, iters, true);
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
// pass; after a barrier, wave w finishes rows r = w, w + STRIDE, ... < nr:
// the waves' sums in wave order 0..WAVES-1, the fp32 output butterflies,
// RN32(. * s), RN32(. * svh), then the cast and store of y[r0 + r][strip cols].
// STRIDE is the number of waves that share the rows (WAVES unless the workgroup
// has more waves than partial sums per row).
template <int WAVES, int STRIDE = WAVES>
__device__ __forceinline__ void finish_strip(const float* partial, int rstride, int wave, int lane, int nr,
                                             int r0, int strip, int out_dim, const uint16_t* __restrict__ svh,
                                             void* __restrict__ y, int y_dtype) {
  const float s = bits_to_f32(kScaleBits);
  const int col = strip * kBlock + lane;
  const float g0 = f16_bits_to_f32(svh[col]);
  const float g1 = f16_bits_to_f32(svh[col + 64]);
  for (int r = wave; r < nr; r += STRIDE) {
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

// The end of a pass: the waves' sums (acc[r][c] = strip column 2*lane + c of
// pass row r) through LDS and finish_strip, FR = min(NR, 16) rows per round so
// `partial` ([WAVES][FR][128] fp32) stays at most 64 KiB.
template <int WAVES, int NR>
__device__ __forceinline__ void finish_pass(const float (&acc)[NR][2], float* partial, int wave, int lane,
                                            int nr, int r0, int strip, int out_dim,
                                            const uint16_t* __restrict__ svh, void* __restrict__ y,
                                            int y_dtype) {
  constexpr int FR = NR < kRowsPerPass ? NR : kRowsPerPass;
#pragma unroll
  for (int c = 0; c < NR; c += FR) {
    if (c >= nr) break;  // block-uniform
    if (c > 0) __syncthreads();  // the previous round has read partial
#pragma unroll
    for (int r = 0; r < FR; ++r) {
      float2 v;
      v.x = acc[c + r][0];
      v.y = acc[c + r][1];
      *reinterpret_cast<float2*>(&partial[(wave * FR + r) * kBlock + 2 * lane]) = v;
    }
    __syncthreads();
    finish_strip<WAVES>(partial, FR, wave, lane, min(FR, nr - c), r0 + c, strip, out_dim, svh, y, y_dtype);
  }
}

}  // namespace tf_exl3
