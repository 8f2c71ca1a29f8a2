// The trellis linear with the row-by-weight products on the matrix cores.
//
// Same projection, stream walk, decode and finish as the v_dot2 linear (TensorFold
// pull request "hip exl3: the input rotation and trellis linear for decode
// rows", "What this changes"); only the sums over k move from v_dot2_f32_f16
// chains to the matrix cores, so the vector ALUs spend their cycles on decoding
// and the cost grows slowly with the number of rows.
//
// Lane l decodes strip columns 2l and 2l+1 for the 16 k of a tile row kt, as
// packed (k, k+1) pairs wp[c][0..7] (column parity c). For each k-half q the
// four pairs wp[c][4q .. 4q+3] (8 k of one column) are the lane's B operand,
// unchanged. B's k-groups therefore mix strip columns; the A operand undoes the
// mix by carrying a row's inputs only in the k-group of the columns it sums:
//
// Passes of up to 4 rows, v_mfma_f32_16x16x32_f16 (lane l = 16G + n):
//  - B (32 k x 16 n): B[8G + t][n] = W[16kt + 8q + t][2l + c]: column 32G + 2n + c;
//  - A (16 m x 32 k): row m = 4r + g holds pass row r's z[16kt + 8q + t] in
//    k-group g only, so D[4r + g][n] sums strip column 32g + 2n + c of row r;
//    lane 16G + m holds A[m][8G .. 8G+7], non-zero iff m % 4 == G;
//  - D: lane l holds D[4G + i][n], i = 0..3: row G, strip column 32i + 2n + c.
// Passes of 5 to 16 rows, v_mfma_f32_32x32x16_f16 (lane l = 32h + j):
//  - B (16 k x 32 n): B[8h + t][j] = W[16kt + 8q + t][2l + c]: column 64h + 2j + c;
//  - A (32 m x 16 k): row m = 2r + g holds row r's z in k-half g only; lane
//    32h + i holds A[i][8h .. 8h+7], non-zero iff i % 2 == h;
//  - D: lane l holds rows m = 8(v/4) + 4h + v%4, v = 0..15 (row m/2, strip
//    column 64(m%2) + 2j + c).
// The row inputs of a step (rows x 16 k) come in with one 16-byte vector load
// per lane, one step ahead and ahead of the stream load (loads complete in
// order), into a wave-private LDS slot; each lane reads its A operand from there,
// and lanes whose A is zero read a zero entry. Every output sums the same eight
// non-zero products per instruction, in the same k order (tile rows in the
// wave's order, q = 0 then 1), and a row's D entries depend only on its own A
// row; the two instruction shapes give the same bits (tested with rows alone,
// in windows and in multi-pass launches), so a row's bits never depend on the
// rows that share the launch.
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half8_t pairs_to_half8(half2_t a, half2_t b, half2_t c, half2_t d) {
  uint4 u;
  u.x = __builtin_bit_cast(uint32_t, a);
  u.y = __builtin_bit_cast(uint32_t, b);
  u.z = __builtin_bit_cast(uint32_t, c);
  u.w = __builtin_bit_cast(uint32_t, d);
  return __builtin_bit_cast(half8_t, u);
}

// Passes of up to 4 rows on v_mfma_f32_16x16x32_f16.
template <int BITS, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) __attribute__((amdgpu_waves_per_eu(5))) void linear_mfma_kernel(
    const uint16_t* __restrict__ z, const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh,
    void* __restrict__ y, int y_dtype, int rows, int in_dim, int out_dim) {
  constexpr int NR = 4;
  constexpr int PF = prefetch_depth<BITS>();
  constexpr int RING = PF + 1;
  __shared__ float partial[WAVES * NR * kBlock];
  __shared__ uint4 zslot[WAVES][2 * NR + 1];  // row r, k-half h at [2r + h]; [2 * NR] stays zero

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int nr = min(NR, rows);
  const int iters = in_dim / 16 / WAVES;

  const StreamStrides st = stream_strides<BITS>(kLayoutTiles, in_dim, out_dim);
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * st.row + (size_t)strip * st.strip;
  const size_t step_words = (size_t)WAVES * st.row;
  const int off = lane * BITS;
  auto share = [&](int i) { return tp + (size_t)min(i, iters - 1) * step_words; };

  // z staging: lane l < 8 loads row min(l / 2, nr - 1), k-half l % 2.
  const bool stager = lane < 2 * NR;
  const uint4* __restrict__ zsrc = reinterpret_cast<const uint4*>(
      z + (size_t)min(lane >> 1, nr - 1) * in_dim + wave * 16 + (lane & 1) * 8);
  auto zload = [&](int i) { return zsrc[(size_t)min(i, iters - 1) * (WAVES * 2)]; };
  if (lane == 0) zslot[wave][2 * NR] = make_uint4(0u, 0u, 0u, 0u);

  // A address: lane 16G + m reads row min(m / 4, nr - 1) iff m % 4 == G.
  const int m = lane & 15;
  const bool part = (m & 3) == (lane >> 4);
  const int abase = part ? 2 * min(m >> 2, nr - 1) : 2 * NR;
  const int aq = part ? 1 : 0;

  f32x4 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  uint32_t ring[RING][BITS];
  uint4 zn = zload(0);
#pragma unroll
  for (int d = 0; d < PF; ++d) load_share<BITS>(ring[d], share(d), off);

  auto step = [&](auto dc, int i) __attribute__((always_inline)) {
    constexpr int D = decltype(dc)::value;
    const uint4 zc = zn;
    zn = zload(i + 1);  // issued before the next stream load: loads complete in order
    load_share<BITS>(ring[(D + PF) % RING], share(i + PF), off);
    if (stager) zslot[wave][lane] = zc;
    half2_t wp[2][8];
    decode_lane<BITS>(ring[D], wp);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const half8_t a = __builtin_bit_cast(half8_t, zslot[wave][abase + q * aq]);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const half8_t b = pairs_to_half8(wp[c][4 * q], wp[c][4 * q + 1], wp[c][4 * q + 2], wp[c][4 * q + 3]);
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
      }
    }
  };
  step_loop<RING>(iters, step);

  // D entry i of acc[c]: pass row G, strip column 32i + 2n + c.
  const int n = lane & 15;
  const int r = lane >> 4;
  if (r < nr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float2 v;
      v.x = acc[0][i];
      v.y = acc[1][i];
      *reinterpret_cast<float2*>(&partial[(wave * NR + r) * kBlock + 32 * i + 2 * n]) = v;
    }
  }
  __syncthreads();
  finish_strip<WAVES>(partial, NR, wave, lane, nr, 0, strip, out_dim, svh, y, y_dtype);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Passes of up to 16 rows on v_mfma_f32_32x32x16_f16. Pipeline per step i: the
// loads for step i + PF (z slice, then stream share: z never waits behind a
// younger stream load), the z slice of step i + 1 into LDS slot (i + 1) % 2,
// the decode of step i, its MFMAs with the A operands read at the end of step
// i - 1, then the A operands of step i + 1 (their latency hides behind the next
// step's loads and decode).
template <int BITS, int WAVES>
__global__ __launch_bounds__(kWave* WAVES) __attribute__((amdgpu_waves_per_eu(4))) void linear_mfma32_kernel(
    const uint16_t* __restrict__ z, const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh,
    void* __restrict__ y, int y_dtype, int rows, int in_dim, int out_dim) {
  constexpr int NR = kRowsPerPass;
  constexpr int PF = prefetch_depth<BITS>() < 4 ? prefetch_depth<BITS>() : 4;  // z rides in the ring too
  constexpr int RING = PF + 1;
  constexpr int FR = 8;  // rows per finish round: 32 KiB of partial sums at 8 waves
  constexpr int SLOT = 2 * NR + 1;  // row r, k-half h at [2r + h]; [2 * NR] stays zero
  __shared__ float partial[WAVES * FR * kBlock];
  __shared__ uint4 zslot[WAVES][2][SLOT];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  const StreamStrides st = stream_strides<BITS>(kLayoutTiles, in_dim, out_dim);
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * st.row + (size_t)strip * st.strip;
  const size_t step_words = (size_t)WAVES * st.row;
  const int off = lane * BITS;
  auto share = [&](int i) { return tp + (size_t)min(i, iters - 1) * step_words; };

  // z staging: lane l < 32 loads row min(l / 2, nr - 1), k-half l % 2.
  const bool stager = lane < 2 * NR;
  const uint4* __restrict__ zsrc = reinterpret_cast<const uint4*>(
      z + (size_t)(r0 + min(lane >> 1, nr - 1)) * in_dim + wave * 16 + (lane & 1) * 8);
  auto zload = [&](int i) { return zsrc[(size_t)min(i, iters - 1) * (WAVES * 2)]; };
  if (lane == 0) {
    zslot[wave][0][2 * NR] = make_uint4(0u, 0u, 0u, 0u);
    zslot[wave][1][2 * NR] = make_uint4(0u, 0u, 0u, 0u);
  }

  // A address: lane 32h + i reads row min(i / 2, nr - 1) iff i % 2 == h.
  const int ai = lane & 31;
  const int ah = lane >> 5;
  const bool part = (ai & 1) == ah;
  const int abase = part ? 2 * min(ai >> 1, nr - 1) : 2 * NR;
  const int aq = part ? 1 : 0;

  f32x16 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.0f;

  uint32_t ring[RING][BITS];
  uint4 zr[RING];  // z slice of step i travels in ring slot i % RING
#pragma unroll
  for (int d = 0; d < PF; ++d) {
    zr[d] = zload(d);
    load_share<BITS>(ring[d], share(d), off);
  }
  if (stager) zslot[wave][0][lane] = zr[0];
  half8_t a[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) a[q] = __builtin_bit_cast(half8_t, zslot[wave][0][abase + q * aq]);

  auto step = [&](auto dc, int i) __attribute__((always_inline)) {
    constexpr int D = decltype(dc)::value;
    zr[(D + PF) % RING] = zload(i + PF);
    load_share<BITS>(ring[(D + PF) % RING], share(i + PF), off);
    uint4* next = zslot[wave][(i + 1) & 1];
    if (stager) next[lane] = zr[(D + 1) % RING];
    half2_t wp[2][8];
    decode_lane<BITS>(ring[D], wp);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const half8_t b = pairs_to_half8(wp[c][4 * q], wp[c][4 * q + 1], wp[c][4 * q + 2], wp[c][4 * q + 3]);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[q], b, acc[c], 0, 0, 0);
      }
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) a[q] = __builtin_bit_cast(half8_t, next[abase + q * aq]);
  };
  step_loop<RING>(iters, step);

  // D entry v of acc[c]: row m = 8(v/4) + 4h + v%4 (pass row m/2, k-half g = m%2),
  // strip column 64g + 2j + c. Rows 8 at a time: v/4 = 2 * round + {0, 1}.
  const int j = lane & 31;
#pragma unroll
  for (int round = 0; round < NR / FR; ++round) {
    if (round * FR >= nr) break;  // block-uniform
    if (round > 0) __syncthreads();  // the previous round has read partial
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int v = 8 * round; v < 8 * round + 8; ++v) {
        const int m = 8 * (v >> 2) + 4 * ah + (v & 3);
        const int r = m >> 1;
        if (r < nr) partial[(wave * FR + r - FR * round) * kBlock + 64 * (m & 1) + 2 * j + c] = acc[c][v];
      }
    }
    __syncthreads();
    finish_strip<WAVES>(partial, FR, wave, lane, min(FR, nr - FR * round), r0 + FR * round, strip, out_dim, svh,
                        y, y_dtype);
  }
}

template <int BITS, int WAVES>
static void launch_4(int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                     const uint16_t* svh, void* y, int y_dtype, hipStream_t stream) {
  hipLaunchKernelGGL((linear_mfma_kernel<BITS, WAVES>), dim3(out_dim / kBlock), dim3(kWave * WAVES), 0, stream, z,
                     trellis, svh, y, y_dtype, rows, in_dim, out_dim);
}

template <int BITS, int WAVES>
static void launch_32(dim3 grid, int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                      const uint16_t* svh, void* y, int y_dtype, hipStream_t stream) {
  hipLaunchKernelGGL((linear_mfma32_kernel<BITS, WAVES>), grid, dim3(kWave * WAVES), 0, stream, z, trellis, svh, y,
                     y_dtype, rows, in_dim, out_dim);
}

template <int BITS, int WAVES>
static hipError_t launch_mfma_bw(int rows, int in_dim, int out_dim, const uint16_t* z, const uint32_t* trellis,
                                 const uint16_t* svh, void* y, int y_dtype, hipStream_t stream) {
  const int full = rows / kRowsPerPass;
  const int rest = rows % kRowsPerPass;
  const int strips = out_dim / kBlock;
  if (full > 0)
    launch_32<BITS, WAVES>(dim3(strips, full), full * kRowsPerPass, in_dim, out_dim, z, trellis, svh, y, y_dtype,
                           stream);
  if (rest > 0) {
    const size_t off = (size_t)full * kRowsPerPass;
    const uint16_t* zr = z + off * in_dim;
    void* yr = (y_dtype == TF_DT_F32) ? (void*)(static_cast<float*>(y) + off * out_dim)
                                      : (void*)(static_cast<uint16_t*>(y) + off * out_dim);
    const dim3 grid(strips, 1);
    if (rest <= 4) {
      launch_4<BITS, WAVES>(rest, in_dim, out_dim, zr, trellis, svh, yr, y_dtype, stream);
    } else {
      launch_32<BITS, WAVES>(grid, rest, in_dim, out_dim, zr, trellis, svh, yr, y_dtype, stream);
    }
  }
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
