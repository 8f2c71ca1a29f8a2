// The trellis linear with the row-by-weight products on the matrix cores.
//
// Same projection, stream walk, decode and finish as the v_dot2 linear (TensorFold
// pull request "hip exl3: the input rotation and trellis linear for decode
// rows", "What this changes"); only the sums over k move from v_dot2_f32_f16
// chains to v_mfma_f32_32x32x16_f16, so the vector ALUs spend their cycles on
// decoding alone and the cost no longer grows with the number of rows.
//
// Operand mapping (per wave, per tile row kt, k-half q in {0, 1}, column
// parity c in {0, 1}). Lane l = 32h + j decodes strip columns 2l and 2l+1 for
// the 16 k of the tile row, as packed (k, k+1) pairs wp[c][0..7]:
//  - B (32 k x 32 n): lane l supplies B[8h + t][j] = W[16kt + 8q + t][2l + c],
//    t = 0..7, i.e. the four pairs wp[c][4q .. 4q+3], unchanged;
//  - A (32 m x 32 k): row m = 2r + g carries row r's inputs z[r][16kt + 8q + t]
//    in k-half g only (zeros in the other half), so column j of the product
//    sums exactly the weights of strip column 64g + 2j + c for row r; lane
//    l = 32h + i holds A[i][8h .. 8h+7], non-zero iff i % 2 == h;
//  - D (32 x 32 fp32, two accumulators, c = 0 and 1): lane l holds rows
//    m = 8(v/4) + 4h + v%4 of column j, v = 0..15.
// The zeros come free: A is read with raw buffer loads whose range is this
// pass's rows, and lanes that must see zeros (the other k-half, rows past the
// pass) get an offset outside the range.
// A row's sums therefore accumulate, for each tile row in the wave's order,
// q = 0 then 1, inside D entries that depend only on that row's inputs; the
// row's bits do not depend on the rows that share the launch.
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kRawBufferWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit elements
constexpr uint32_t kOutOfRange = 0x80000000u;

// Tile rows in flight per wave, and how many steps ahead the A operands load;
// the ring's PF + 1 slots must be a multiple of the A ring's ZD + 1 slots.
template <int BITS>
constexpr int mfma_prefetch() {
  return BITS == 3 || BITS == 5 ? 5 : 3;
}
template <int BITS>
constexpr int mfma_a_ahead() {
  return mfma_prefetch<BITS>() == 5 ? 2 : 1;
}

__device__ __forceinline__ half8_t pairs_to_half8(half2_t a, half2_t b, half2_t c, half2_t d) {
  u32x4 u;
  u.x = __builtin_bit_cast(uint32_t, a);
  u.y = __builtin_bit_cast(uint32_t, b);
  u.z = __builtin_bit_cast(uint32_t, c);
  u.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(half8_t, u);
}

template <int BITS>
__device__ __forceinline__ void mfma_step(const uint32_t (&w)[BITS + 1], const u32x4 (&za)[2],
                                          f32x16 (&acc)[2]) {
  half2_t wp[2][8];
  decode_lane<BITS>(w, wp);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const half8_t a = __builtin_bit_cast(half8_t, za[q]);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const half8_t b = pairs_to_half8(wp[c][4 * q], wp[c][4 * q + 1], wp[c][4 * q + 2], wp[c][4 * q + 3]);
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void load_a(u32x4 (&za)[2], __amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  za[0] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0);
  za[1] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, off + 16, 0, 0);
}

// Waves per SIMD the register budget aims at: five (96 registers) where the
// kernel fits without spilling, else four (128).
template <int BITS>
constexpr int mfma_waves_per_simd() {
  return BITS == 2 || BITS == 4 ? 5 : 4;
}

template <int BITS, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) __attribute__((amdgpu_waves_per_eu(mfma_waves_per_simd<BITS>()))) void linear_mfma_kernel(
    const uint16_t* __restrict__ z, const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh,
    void* __restrict__ y, int y_dtype, int rows, int in_dim, int out_dim) {
  constexpr int PF = mfma_prefetch<BITS>();
  constexpr int RING = PF + 1;
  constexpr int ZD = mfma_a_ahead<BITS>();
  constexpr int ZR = ZD + 1;
  static_assert(RING % ZR == 0, "the A ring must line up with the stream ring");
  extern __shared__ float partial[];  // [WAVES][nr][128]

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * kRowsPerPass;
  const int nr = min(kRowsPerPass, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  const size_t row_words = (size_t)(out_dim / 16) * 8 * BITS;
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * row_words + (size_t)strip * 64 * BITS;
  const size_t step_words = (size_t)WAVES * row_words;
  const int off = lane * BITS;
  const int nb = next_lane_in_tile(lane) * BITS;

  // A operand source: this pass's rows as a raw buffer of nr * in_dim fp16.
  const int ai = lane & 31;
  const int ah = lane >> 5;
  const __amdgpu_buffer_rsrc_t zr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(z + (size_t)r0 * in_dim), (short)0, nr * in_dim * 2, kRawBufferWord3);
  const uint32_t a_row = (uint32_t)((ai >> 1) * in_dim + wave * 16) * 2u;  // bytes, step 0
  const uint32_t a_base = ((ai & 1) == ah) ? a_row : kOutOfRange;
  const uint32_t a_step = (uint32_t)WAVES * 32u;  // bytes between a wave's tile rows

  f32x16 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;

  auto share = [&](int i) { return tp + (size_t)min(i, iters - 1) * step_words; };
  uint32_t ring[RING][BITS + 1];
#pragma unroll
  for (int d = 0; d < PF; ++d) load_share<BITS>(ring[d], share(d), off, nb);
  u32x4 za[ZR][2];
#pragma unroll
  for (int d = 0; d < ZD; ++d) load_a(za[d], zr, a_base + (uint32_t)d * a_step);

  int it = 0;
  for (; it + RING <= iters; it += RING) {
#pragma unroll
    for (int d = 0; d < RING; ++d) {
      // A goes out before the stream load: loads complete in issue order, so
      // waiting for an A operand never waits for a younger stream load.
      load_a(za[(d + ZD) % ZR], zr, a_base + (uint32_t)(it + d + ZD) * a_step);
      load_share<BITS>(ring[(d + PF) % RING], share(it + d + PF), off, nb);
      mfma_step<BITS>(ring[d], za[d % ZR], acc);
    }
  }
#pragma unroll
  for (int d = 0; d < RING; ++d) {
    if (it + d < iters) {
      load_a(za[(d + ZD) % ZR], zr, a_base + (uint32_t)(it + d + ZD) * a_step);
      mfma_step<BITS>(ring[d], za[d % ZR], acc);
    }
  }

  // D entry v of accumulator c: row m = 8(v/4) + 4h + v%4 (pass row m/2, k-half
  // g = m%2), strip column 64g + 2j + c.
  const int j = lane & 31;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = 8 * (v >> 2) + 4 * ah + (v & 3);
      const int r = m >> 1;
      if (r < nr) partial[(wave * nr + r) * kBlock + 64 * (m & 1) + 2 * j + c] = acc[c][v];
    }
  }
  __syncthreads();
  finish_strip<WAVES>(partial, nr, wave, lane, nr, r0, strip, out_dim, svh, y, y_dtype);
}

template <int BITS, int WAVES>
static hipError_t launch_mfma_bw(int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                                 const uint16_t* svh, void* y, int y_dtype, hipStream_t stream) {
  const int passes = (rows + kRowsPerPass - 1) / kRowsPerPass;
  const int nr_max = rows < kRowsPerPass ? rows : kRowsPerPass;
  const size_t lds = (size_t)WAVES * nr_max * kBlock * sizeof(float);
  hipLaunchKernelGGL((linear_mfma_kernel<BITS, WAVES>), dim3(out_dim / kBlock, passes), dim3(kWave * WAVES),
                     lds, stream, z, trellis, svh, y, y_dtype, rows, in_dim, out_dim);
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_mfma_b(int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                                const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                hipStream_t stream) {
  if (waves == 8) return launch_mfma_bw<BITS, 8>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  return launch_mfma_bw<BITS, 4>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
}

hipError_t launch_linear_mfma(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                              const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                              hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_mfma_b<2>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 3: return launch_mfma_b<3>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 4: return launch_mfma_b<4>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 5: return launch_mfma_b<5>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 6: return launch_mfma_b<6>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    default: return launch_mfma_b<8>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  }
}

}  // namespace tf_exl3
