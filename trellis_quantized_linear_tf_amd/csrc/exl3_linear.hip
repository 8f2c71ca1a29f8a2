// The trellis linear: 1..16 decode rows per pass, and the prompt path's 32-row
// passes.
//
// Source: TensorFold pull request "hip exl3: the input rotation and trellis
// linear for decode rows", section "What this changes". Each weight costs one
// fp16 fused multiply-add in the codebook; every output's sum over k is a chain
// of v_dot2_f32_f16 whose order is fixed by the shape alone, which is what keeps
// an output row's bits independent of its launch-mates. After the k sums, the
// per-wave partials are added, the 128-point output rotation and the svh scale
// are applied. The k range is never split across workgroups and there is no bias.
//
// Work layout on gfx950:
//  - one workgroup per (128-column strip, pass of rows);
//  - the strip's tile row kt is 8 contiguous tiles = 256*BITS bytes, read by one
//    wave as one coalesced load (BITS dwords per lane); lane l owns strip
//    columns 2l and 2l+1;
//  - wave w takes tile rows kt = w, w + WAVES, ... (in_dim/16 is a multiple of
//    8, so every wave gets the same count), with a register ring of tile rows in
//    flight;
//  - z pairs are wave-uniform. For up to 4 rows a pass (linear_kernel) they come
//    in through scalar loads and feed v_dot2_f32_f16 as the SGPR operand. For 8,
//    12, 16 and 32 rows (linear_lds_kernel) a step's z (rows x 16 k) needs more
//    scalar registers than a wave has, so each lane brings 16 bytes of it in
//    with one vector load, one step ahead and ahead of the stream loads, the
//    wave parks the slice in a private LDS slot and reads each row back as a
//    broadcast;
//  - the partial sums go through LDS and are added in wave order 0..WAVES-1;
//    one wave per row then runs the 128-point butterflies, the scale and svh
//    (16 rows per round, so a 32-row pass keeps 64 KiB of partial sums).
// A row's chain is: for each of its wave's tile rows in ascending kt, the pairs
// p = 0..7 in ascending k; it is the same in every variant, whichever way z
// arrives, so a row's bits never depend on the variant. A launch that would put
// fewer than 2048 waves in flight (narrow matrices) runs the column-split form
// in exl3_linear_cs.hip instead, with the same chains.
//
// Prompt path (the same page, "Known limits": the prompt path that follows must
// reproduce the decode linear's bits): full passes of 32 rows decode each tile row once
// for twice the rows; the remainder runs as decode passes.
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

template <int BITS, int WAVES, int NR>
__global__ __launch_bounds__(kWave* WAVES) void linear_kernel(const uint16_t* __restrict__ z,
                                                              const uint32_t* __restrict__ trellis,
                                                              const uint16_t* __restrict__ svh,
                                                              void* __restrict__ y, int y_dtype,
                                                              int rows, int in_dim, int out_dim,
                                                              int layout) {
  __shared__ float partial[WAVES * (NR < kRowsPerPass ? NR : kRowsPerPass) * kBlock];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  // This strip's tile row kt = wave, and the words between the wave's tile rows.
  const StreamStrides st = stream_strides<BITS>(layout, in_dim, out_dim);
  const uint32_t* __restrict__ tp = trellis + (size_t)wave * st.row + (size_t)strip * st.strip;
  const size_t step_words = (size_t)WAVES * st.row;
  const int off = lane * BITS;

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

  StreamWalk<BITS, WAVES, NR> walk{tp, step_words, off, iters};
  walk.prime();
  walk.run(zrow, acc);

  // Cross-wave sums in wave order, then the output rotation, scale and svh.
  finish_pass<WAVES, NR>(acc, partial, wave, lane, nr, r0, strip, out_dim, svh, y, y_dtype);
}

// The walk of linear_lds_kernel: the stream ring of StreamWalk with PF = 2 (a step
// of 8 or more rows runs long enough that two tile rows in flight cover the
// stream's latency), plus the wave's z slice for each step staged through a
// wave-private LDS slot.
template <int BITS, int WAVES, int NR>
struct LdsWalk {
  static_assert(2 * NR <= kWave, "a lane stages one (row, k-half) of the step's z");
  static constexpr int PF = 2;
  static constexpr int RING = PF + 1;
  const uint32_t* __restrict__ tp;
  size_t step_words;
  int off, iters;
  const uint4* __restrict__ zsrc;  // this lane's 16 bytes of z for step 0
  uint4* zslot;                    // the wave's LDS slot: row r, k-half h at [2r + h]
  bool stager;                     // lane < 2 * NR
  uint32_t ring[RING][BITS];
  uint4 zn;

  __device__ __forceinline__ const uint32_t* share(int i) const {
    return tp + (size_t)min(i, iters - 1) * step_words;
  }
  __device__ __forceinline__ uint4 zload(int i) const { return zsrc[(size_t)min(i, iters - 1) * (WAVES * 2)]; }

  __device__ __forceinline__ void prime() {
    zn = zload(0);
#pragma unroll
    for (int d = 0; d < PF; ++d) load_share<BITS>(ring[d], share(d), off);
  }

  // Step i, decoding ring slot D = i % RING; the load for step i + PF refills
  // the slot step i - 1 freed.
  template <int D>
  __device__ __forceinline__ void step(int i, float (&acc)[NR][2]) {
    const uint4 zc = zn;
    zn = zload(i + 1);  // issued before the next stream load: loads complete in order
    load_share<BITS>(ring[(D + PF) % RING], share(i + PF), off);
    if (stager) zslot[__lane_id()] = zc;
    half2_t wp[2][8];
    decode_lane<BITS>(ring[D], wp);
    // Row r + 1's z is read while row r's chains run. The empty asm after row
    // r takes its accumulators and orders memory, so the chains cannot sink
    // below later rows' reads and at most two rows of z (16 registers) are live.
    uint4 lo = zslot[0];
    uint4 hi = zslot[1];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const uint32_t zp[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (r + 1 < NR) {
        lo = zslot[2 * r + 2];
        hi = zslot[2 * r + 3];
      }
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        const half2_t zz = __builtin_bit_cast(half2_t, zp[p]);
        acc[r][0] = __builtin_amdgcn_fdot2(zz, wp[0][p], acc[r][0], false);
        acc[r][1] = __builtin_amdgcn_fdot2(zz, wp[1][p], acc[r][1], false);
      }
      asm volatile("" : "+v"(acc[r][0]), "+v"(acc[r][1])::"memory");
    }
  }

  __device__ __forceinline__ void run(float (&acc)[NR][2]) {
    static_assert(RING == 3, "the step lists below name the ring slots");
    int it = 0;
    for (; it + RING <= iters; it += RING) {
      step<0>(it, acc);
      step<1>(it + 1, acc);
      step<2>(it + 2, acc);
    }
    if (it < iters) step<0>(it, acc);
    if (it + 1 < iters) step<1>(it + 1, acc);
  }
};

template <int BITS, int WAVES, int NR>
__global__ __launch_bounds__(kWave* WAVES) __attribute__((amdgpu_waves_per_eu(4))) void linear_lds_kernel(
    const uint16_t* __restrict__ z, const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh,
    void* __restrict__ y, int y_dtype, int rows, int in_dim, int out_dim, int layout) {
  __shared__ float partial[WAVES * kRowsPerPass * kBlock];
  __shared__ uint4 zslot[WAVES][2 * NR];

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;
  const StreamStrides st = stream_strides<BITS>(layout, in_dim, out_dim);

  // Lane l stages row min(l / 2, nr - 1), k-half l % 2 of tile row kt = wave + i * WAVES.
  const int zr = min(lane >> 1, nr - 1);
  LdsWalk<BITS, WAVES, NR> walk{
      trellis + (size_t)wave * st.row + (size_t)strip * st.strip,
      (size_t)WAVES * st.row,
      lane * BITS,
      iters,
      reinterpret_cast<const uint4*>(z + (size_t)(r0 + zr) * in_dim + wave * 16 + (lane & 1) * 8),
      zslot[wave],
      lane < 2 * NR};

  float acc[NR][2];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r][0] = acc[r][1] = 0.0f;
  walk.prime();
  walk.run(acc);

  finish_pass<WAVES, NR>(acc, partial, wave, lane, nr, r0, strip, out_dim, svh, y, y_dtype);
}

// One launch of the variant with row capacity NR: z through scalar loads for
// NR <= kScalarZRows, else through LDS.
template <int BITS, int WAVES, int NR>
static void launch_nr(dim3 grid, const uint16_t* z, const uint32_t* trellis, const uint16_t* svh, void* y,
                      int y_dtype, int rows, int in_dim, int out_dim, int layout, hipStream_t stream) {
  if constexpr (NR <= kScalarZRows) {
    hipLaunchKernelGGL((linear_kernel<BITS, WAVES, NR>), grid, dim3(kWave * WAVES), 0, stream, z, trellis, svh,
                       y, y_dtype, rows, in_dim, out_dim, layout);
  } else {
    hipLaunchKernelGGL((linear_lds_kernel<BITS, WAVES, NR>), grid, dim3(kWave * WAVES), 0, stream, z, trellis,
                       svh, y, y_dtype, rows, in_dim, out_dim, layout);
  }
}

template <int BITS, int WAVES>
static hipError_t launch_bw(int rows, int in_dim, int out_dim, const uint16_t* z,
                            const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int layout,
                            int split, hipStream_t stream) {
  const int full = rows / kRowsPerPass;
  const int rest = rows % kRowsPerPass;
  const int strips = out_dim / kBlock;
  auto use_cs = [&](int passes) { return split < 0 ? column_split(out_dim, passes, WAVES) : split == 1; };
  if (full > 0) {
    const dim3 grid(strips, full);
    if (use_cs(full)) {
      launch_linear_cs(BITS, WAVES, 16, grid, z, trellis, svh, y, y_dtype, full * kRowsPerPass, in_dim, out_dim,
                       layout, stream);
    } else {
      launch_nr<BITS, WAVES, 16>(grid, z, trellis, svh, y, y_dtype, full * kRowsPerPass, in_dim, out_dim, layout,
                                 stream);
    }
  }
  if (rest > 0) {
    const size_t off = (size_t)full * kRowsPerPass;
    const uint16_t* zr = z + off * in_dim;
    void* yr = (y_dtype == TF_DT_F32) ? (void*)(static_cast<float*>(y) + off * out_dim)
                                      : (void*)(static_cast<uint16_t*>(y) + off * out_dim);
    const dim3 grid(strips, 1);
    const int cap = rows_bucket(rest);
    if (use_cs(1)) {
      launch_linear_cs(BITS, WAVES, cap, grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream);
    } else {
      switch (cap) {
        case 1: launch_nr<BITS, WAVES, 1>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
        case 2: launch_nr<BITS, WAVES, 2>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
        case 4: launch_nr<BITS, WAVES, 4>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
        case 8: launch_nr<BITS, WAVES, 8>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
        case 12: launch_nr<BITS, WAVES, 12>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
        default: launch_nr<BITS, WAVES, 16>(grid, zr, trellis, svh, yr, y_dtype, rest, in_dim, out_dim, layout, stream); break;
      }
    }
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_b(int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                           const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int layout,
                           int split, hipStream_t stream) {
  if (waves == 8)
    return launch_bw<BITS, 8>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
  return launch_bw<BITS, 4>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
}

hipError_t launch_linear(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                         const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int layout,
                         hipStream_t stream, int split) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_b<2>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
    case 3: return launch_b<3>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
    case 4: return launch_b<4>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
    case 5: return launch_b<5>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
    case 6: return launch_b<6>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
    default: return launch_b<8>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, layout, split, stream);
  }
}

template <int BITS, int WAVES>
static hipError_t launch_prompt_bw(int rows, int in_dim, int out_dim, const uint16_t* z,
                                   const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                   hipStream_t stream) {
  const int full = rows / kPromptRowsPerPass;
  const int rest = rows % kPromptRowsPerPass;
  if (full > 0) {
    hipLaunchKernelGGL((linear_lds_kernel<BITS, WAVES, kPromptRowsPerPass>), dim3(out_dim / kBlock, full),
                       dim3(kWave * WAVES), 0, stream, z, trellis, svh, y, y_dtype, full * kPromptRowsPerPass,
                       in_dim, out_dim, kLayoutTiles);
  }
  if (rest > 0) {
    const size_t off = (size_t)full * kPromptRowsPerPass;
    void* yr = (y_dtype == TF_DT_F32) ? (void*)(static_cast<float*>(y) + off * out_dim)
                                      : (void*)(static_cast<uint16_t*>(y) + off * out_dim);
    return launch_bw<BITS, WAVES>(rest, in_dim, out_dim, z + off * in_dim, trellis, svh, yr, y_dtype,
                                  kLayoutTiles, -1, stream);
  }
  return hipGetLastError();
}

template <int BITS>
static hipError_t launch_prompt_b(int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                                  const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                  hipStream_t stream) {
  if (waves == 8) return launch_prompt_bw<BITS, 8>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
  return launch_prompt_bw<BITS, 4>(rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
}

hipError_t launch_linear_prompt(int bits, int waves, int rows, int in_dim, int out_dim, const uint16_t* z,
                                const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype,
                                hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: return launch_prompt_b<2>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 3: return launch_prompt_b<3>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 4: return launch_prompt_b<4>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 5: return launch_prompt_b<5>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    case 6: return launch_prompt_b<6>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
    default: return launch_prompt_b<8>(waves, rows, in_dim, out_dim, z, trellis, svh, y, y_dtype, stream);
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
  uint32_t w[BITS];
  load_share<BITS>(w, tp, lane * BITS);
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
