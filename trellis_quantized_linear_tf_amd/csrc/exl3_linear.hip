// The trellis linear for 1..16 decode rows per pass.
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "What this changes": a lane decodes its 16 x 16 tile values with
// one fp16 fma each; a row's sums are v_dot2_f32_f16 chains in a fixed order, so
// a row's bits do not depend on the rows sharing its launch; the waves' partial
// sums, the output rotation and svh finish the block; no K split, no bias.
//
// Work layout on gfx950:
//  - one workgroup per (128-column strip, pass of up to 16 rows);
//  - the strip's tile row kt is 8 contiguous tiles = 256*BITS bytes, read by one
//    wave as one coalesced load (BITS dwords per lane); lane l owns strip
//    columns 2l and 2l+1;
//  - wave w takes tile rows kt = w, w + WAVES, ... (in_dim/16 is a multiple of
//    8, so every wave gets the same count), with a register ring of PF tile rows
//    in flight;
//  - z pairs are wave-uniform and come in through scalar loads, feeding
//    v_dot2_f32_f16 as the SGPR operand;
//  - the partial sums go through LDS and are added in wave order 0..WAVES-1;
//    one wave per row then runs the 128-point butterflies, the scale and svh.
// A row's chain is: for each of its wave's tile rows in ascending kt, the pairs
// p = 0..7 in ascending k; it is the same in every row-capacity variant.
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

template <int BITS, int WAVES, int NR>
__global__ __launch_bounds__(kWave* WAVES) void linear_kernel(const uint16_t* __restrict__ z,
                                                              const uint32_t* __restrict__ trellis,
                                                              const uint16_t* __restrict__ svh,
                                                              void* __restrict__ y, int y_dtype,
                                                              int rows, int in_dim, int out_dim) {
  __shared__ float partial[WAVES * NR * kBlock];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * kRowsPerPass;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  // Stream words of one tile row across the whole matrix, and this lane's share
  // of tile row kt = wave in this strip.
  const size_t row_words = (size_t)(out_dim / 16) * 8 * BITS;
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * row_words + (size_t)strip * 64 * BITS;
  const size_t step_words = (size_t)WAVES * row_words;
  const int off = lane * BITS;
  const int nb = next_lane_in_tile(lane) * BITS;

  // Row r of this pass reads z as dword pairs; padded rows (r >= nr) repeat the
  // last real row and are never stored.
  const uint32_t* zrow_m[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rr = r0 + (r < nr ? r : nr - 1);
    zrow_m[r] = reinterpret_cast<const uint32_t*>(z + (size_t)rr * in_dim) + wave * 8;
  }
  const uint32_t* const(&zrow)[NR] = zrow_m;

  float acc[NR][2];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r][0] = acc[r][1] = 0.0f;

  StreamWalk<BITS, WAVES, NR> walk{tp, step_words, off, nb, iters};
  walk.prime();
  walk.run(zrow, acc);

  // Cross-wave sums in wave order, then the output rotation, scale and svh.
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    float2 v;
    v.x = acc[r][0];
    v.y = acc[r][1];
    *reinterpret_cast<float2*>(&partial[(wave * NR + r) * kBlock + 2 * lane]) = v;
  }
  __syncthreads();

  finish_strip<WAVES>(partial, NR, wave, lane, nr, r0, strip, out_dim, svh, y, y_dtype);
}

template <int BITS, int WAVES>
static hipError_t launch_bw(int rows, int in_dim, int out_dim, const uint16_t* z,
                            const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                            hipStream_t stream) {
  const int full = rows / kRowsPerPass;
  const int rest = rows % kRowsPerPass;
  const dim3 block(kWave * WAVES);
  if (full > 0) {
    hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 16>), dim3(out_dim / kBlock, full), block, 0,
                       stream, z, trellis, svh, y, y_dtype, full * kRowsPerPass, in_dim, out_dim);
  }
  if (rest > 0) {
    const size_t off = (size_t)full * kRowsPerPass;
    const uint16_t* zr = z + off * in_dim;
    void* yr = (y_dtype == TF_DT_F32) ? (void*)(static_cast<float*>(y) + off * out_dim)
                                      : (void*)(static_cast<uint16_t*>(y) + off * out_dim);
    const dim3 grid(out_dim / kBlock, 1);
    switch (rows_bucket(rest)) {
      case 1:
        hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 1>), grid, block, 0, stream, zr, trellis, svh,
                           yr, y_dtype, rest, in_dim, out_dim);
        break;
      case 2:
        hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 2>), grid, block, 0, stream, zr, trellis, svh,
                           yr, y_dtype, rest, in_dim, out_dim);
        break;
      case 4:
        hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 4>), grid, block, 0, stream, zr, trellis, svh,
                           yr, y_dtype, rest, in_dim, out_dim);
        break;
      case 8:
        hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 8>), grid, block, 0, stream, zr, trellis, svh,
                           yr, y_dtype, rest, in_dim, out_dim);
        break;
      default:
        hipLaunchKernelGGL((linear_kernel<BITS, WAVES, 16>), grid, block, 0, stream, zr, trellis,
                           svh, yr, y_dtype, rest, in_dim, out_dim);
        break;
    }
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_b(int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                           const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                           hipStream_t stream) {
  if (waves == 8) return launch_bw<BITS, 8>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  return launch_bw<BITS, 4>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
}

hipError_t launch_linear(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                         const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                         hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_b<2>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 3: return launch_b<3>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 4: return launch_b<4>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 5: return launch_b<5>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 6: return launch_b<6>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    default: return launch_b<8>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  }
}

// ---------------------------------------------------------------------------
// Test kernels on the same device decode path.

__global__ __launch_bounds__(256) void decode_states_kernel(const uint16_t* __restrict__ states,
                                                             uint16_t* __restrict__ w, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t s = states[i];
  w[i] = (uint16_t)(__builtin_bit_cast(uint32_t, decode_pair(s, s)) & 0xFFFFu);
}

// One wave per (strip, tile row): the linear's share load, neighbour exchange and
// decode_lane, then the 32 weights of each lane are written out as W[k][n].
template <int BITS>
__global__ __launch_bounds__(kWave) void decode_tiles_kernel(const uint32_t* __restrict__ trellis,
                                                              uint16_t* __restrict__ w_out,
                                                              int out_dim) {
  const int lane = __lane_id();
  const int strip = blockIdx.x;
  const int kt = blockIdx.y;
  const size_t row_words = (size_t)(out_dim / 16) * 8 * BITS;
  const uint32_t* tp = trellis + (size_t)kt * row_words + (size_t)strip * 64 * BITS;
  uint32_t w[BITS + 1];
  load_share<BITS>(w, tp, lane * BITS, next_lane_in_tile(lane) * BITS);
  half2_t wp[2][8];
  decode_lane<BITS>(w, wp);
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const size_t n = (size_t)strip * kBlock + 2 * lane + c;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      // Halves through the packed dword (bit-casting a vector element directly
      // is lowered as element 0 by this compiler).
      const uint32_t u = __builtin_bit_cast(uint32_t, wp[c][p]);
      w_out[(size_t)(16 * kt + 2 * p) * out_dim + n] = (uint16_t)(u & 0xFFFFu);
      w_out[(size_t)(16 * kt + 2 * p + 1) * out_dim + n] = (uint16_t)(u >> 16);
    }
  }
}

hipError_t launch_decode_states(const uint16_t* states, uint16_t* w, int n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(decode_states_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, states, w, n);
  return hipGetLastError();
}

hipError_t launch_decode_tiles(int bits, int in_dim, int out_dim, const uint32_t* trellis,
                               uint16_t* w, hipStream_t stream) {
  const dim3 grid(out_dim / kBlock, in_dim / 16);
  switch (bits) {
    case 2: hipLaunchKernelGGL(decode_tiles_kernel<2>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
    case 3: hipLaunchKernelGGL(decode_tiles_kernel<3>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
    case 4: hipLaunchKernelGGL(decode_tiles_kernel<4>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
    case 5: hipLaunchKernelGGL(decode_tiles_kernel<5>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
    case 6: hipLaunchKernelGGL(decode_tiles_kernel<6>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
    default: hipLaunchKernelGGL(decode_tiles_kernel<8>, grid, dim3(kWave), 0, stream, trellis, w, out_dim); break;
  }
  return hipGetLastError();
}

}  // namespace tf_exl3
