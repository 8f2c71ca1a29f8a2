// The whole decode-row projection in one launch: rot_in, then the v_dot2 linear.
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "What this changes": rot_in's fp16 rows feed the trellis linear.
// Here every workgroup first rotates the rows of its pass into LDS (the same
// rot_in_block the rot_in kernel runs, so the same fp16 bits), while its first
// stream loads are already in flight, then runs the linear's own tile-row walk
// (StreamWalk: same waves, same k order, same finish) reading z from LDS instead
// of global memory. y is therefore bit-identical to tf_exl3_rot_in followed by
// tf_exl3_linear, without the second launch or the round trip of z through HBM.
//
// Every workgroup rotates all of its pass's rows (the waves split the 128-blocks),
// so the rotation is repeated once per strip: for one 5120-wide row about 5% more
// VALU work than the linear alone, plus z read from LDS instead of through the
// scalar cache; on the LM head that costs about what the saved launch does, while
// on a one-strip layer (the indexer), whose step is mostly launch latency, the
// single launch takes about 60% of the two launches' time. The host sizes passes so
// the rows' z and the partial sums fit in LDS.
#include "exl3_launch.hpp"
#include "exl3_strip.hpp"

namespace tf_exl3 {

// Waves per SIMD the single launch is compiled for: at one row a pass, 8, so that a
// grid as wide as the LM head's (1010 workgroups of 8 waves) is resident at once (at
// 6 waves per SIMD three quarters of it were, and the rest ran as a second
// generation behind them); larger passes keep the compiler's choice (at 2 rows and
// 6 bits the 64-register budget of 8 waves would spill).
template <int NR>
constexpr int project_waves_per_eu() {
  return NR == 1 ? 8 : 1;
}

template <int BITS, int WAVES, int NR>
__global__ __launch_bounds__(kWave* WAVES) __attribute__((amdgpu_waves_per_eu(project_waves_per_eu<NR>()))) void
project_kernel(const void* __restrict__ x, int x_dtype, const uint16_t* __restrict__ suh,
               const uint32_t* __restrict__ trellis, const uint16_t* __restrict__ svh, void* __restrict__ y,
               int y_dtype, int rows, int in_dim, int out_dim) {
  extern __shared__ uint32_t lds[];  // z: [NR][in_dim] fp16, then partial: [WAVES][NR][128] fp32
  uint16_t* zl = reinterpret_cast<uint16_t*>(lds);
  float* partial = reinterpret_cast<float*>(lds + (size_t)NR * in_dim / 2);

  const int lane = __lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int strip = blockIdx.x;
  const int r0 = blockIdx.y * NR;
  const int nr = min(NR, rows - r0);
  const int iters = in_dim / 16 / WAVES;

  const size_t row_words = (size_t)(out_dim / 16) * 8 * BITS;
  StreamWalk<BITS, WAVES, NR> walk{trellis + (size_t)wave * row_words + (size_t)strip * 64 * BITS,
                                   (size_t)WAVES * row_words, lane * BITS, iters};

  // rot_in of this pass's rows into LDS: wave w takes 128-blocks w, w + WAVES, ...
  // in chunks of kChunk. A chunk's loads all go out before its first use, and the
  // first chunk's before the stream prime (loads complete in issue order, so the
  // rotation never waits behind the stream). Four blocks a chunk keep the registers
  // of the loads in flight within the 8-waves-per-SIMD budget.
  constexpr int kChunk = 4;
  const int bpr = in_dim / kBlock;
  const int total = nr * bpr;
  bool primed = false;
  for (int c0 = wave; c0 < total; c0 += kChunk * WAVES) {
    uint32_t xr[kChunk][2];
    uint16_t gr[kChunk][2];
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int b = min(c0 + j * WAVES, total - 1);
      const int rr = b / bpr;
      const int kb = b - rr * bpr;
      const size_t base = (size_t)(r0 + rr) * in_dim + (size_t)kb * kBlock + lane;
      xr[j][0] = load_raw(x, x_dtype, base);
      xr[j][1] = load_raw(x, x_dtype, base + 64);
      gr[j][0] = suh[kb * kBlock + lane];
      gr[j][1] = suh[kb * kBlock + lane + 64];
    }
    if (!primed) {
      walk.prime();
      primed = true;
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const int b = c0 + j * WAVES;
      if (b < total) {
        const int rr = b / bpr;
        const int kb = b - rr * bpr;
        uint16_t z0, z1;
        rot_in_math(widen_raw(xr[j][0], x_dtype), widen_raw(xr[j][1], x_dtype), f16_bits_to_f32(gr[j][0]),
                    f16_bits_to_f32(gr[j][1]), z0, z1);
        zl[rr * in_dim + kb * kBlock + lane] = z0;
        zl[rr * in_dim + kb * kBlock + lane + 64] = z1;
      }
    }
  }
  if (!primed) walk.prime();
  __syncthreads();

  // Row r reads its z pairs from LDS; padded rows (r >= nr) repeat the last row.
  const uint32_t* zrow_m[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int rr = r < nr ? r : nr - 1;
    zrow_m[r] = lds + (size_t)rr * in_dim / 2 + wave * 8;
  }
  const uint32_t* const(&zrow)[NR] = zrow_m;

  float acc[NR][2];
#pragma unroll
  for (int r = 0; r < NR; ++r) acc[r][0] = acc[r][1] = 0.0f;
  walk.run(zrow, acc);

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

template <int BITS, int WAVES, int NR>
static void launch_p(const void* x, int x_dtype, const uint16_t* suh, const uint32_t* trellis,
                     const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim, int out_dim,
                     hipStream_t stream) {
  const size_t lds = project_lds_bytes(WAVES, NR, in_dim);
  const dim3 grid(out_dim / kBlock, (rows + NR - 1) / NR);
  hipLaunchKernelGGL((project_kernel<BITS, WAVES, NR>), grid, dim3(kWave * WAVES), lds, stream, x, x_dtype,
                     suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim);
}

template <int BITS, int WAVES>
static void launch_pw(int nr_cap, const void* x, int x_dtype, const uint16_t* suh, const uint32_t* trellis,
                      const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim, int out_dim,
                      hipStream_t stream) {
  switch (nr_cap) {
    case 1: launch_p<BITS, WAVES, 1>(x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 2: launch_p<BITS, WAVES, 2>(x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 4: launch_p<BITS, WAVES, 4>(x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 8: launch_p<BITS, WAVES, 8>(x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    default: launch_p<BITS, WAVES, 16>(x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
  }
}

template <int BITS>
static void launch_pb(int waves, int nr_cap, const void* x, int x_dtype, const uint16_t* suh,
                      const uint32_t* trellis, const uint16_t* svh, void* y, int y_dtype, int rows, int in_dim,
                      int out_dim, hipStream_t stream) {
  if (waves == 8) {
    launch_pw<BITS, 8>(nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream);
  } else {
    launch_pw<BITS, 4>(nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream);
  }
}

hipError_t launch_project(int bits, int waves, int nr_cap, int rows, int in_dim, int out_dim, const void* x,
                          int x_dtype, const uint16_t* suh, const uint32_t* trellis, const uint16_t* svh, void* y,
                          int y_dtype, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  switch (bits) {
    case 2: launch_pb<2>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 3: launch_pb<3>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 4: launch_pb<4>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 5: launch_pb<5>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    case 6: launch_pb<6>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
    default: launch_pb<8>(waves, nr_cap, x, x_dtype, suh, trellis, svh, y, y_dtype, rows, in_dim, out_dim, stream); break;
  }
  return hipGetLastError();
}

}  // namespace tf_exl3
