// Repacker from the tile layout to the strips layout.
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows", "Checks on this head": the linear runs on the checkpoint's tile
// layout and on a strips layout. Both store a strip's tile row (its 8 tiles,
// 64 * bits words) contiguously; the tile layout orders those chunks by tile row
// then strip, the strips layout by strip then tile row, so each 128-column strip
// becomes one contiguous stream. The repack moves chunk (kt, s) from
// (kt * strips + s) to (s * in_dim/16 + kt), unchanged.
//
// One wave per chunk, four chunks (consecutive tile rows of one strip) per
// workgroup; lanes copy consecutive words, so both reads and writes coalesce.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace tf_exl3 {

constexpr int kRepackWaves = 4;

__global__ __launch_bounds__(kWave* kRepackWaves) void repack_strips_kernel(const uint32_t* __restrict__ tiles,
                                                                            uint32_t* __restrict__ strips,
                                                                            int chunk_words, int kt_n, int s_n) {
  const int s = blockIdx.x;
  const int kt = blockIdx.y * kRepackWaves + (threadIdx.x >> 6);
  if (kt >= kt_n) return;
  const uint32_t* __restrict__ src = tiles + ((size_t)kt * s_n + s) * chunk_words;
  uint32_t* __restrict__ dst = strips + ((size_t)s * kt_n + kt) * chunk_words;
  for (int i = __lane_id(); i < chunk_words; i += kWave) dst[i] = src[i];
}

hipError_t launch_repack_strips(int bits, int in_dim, int out_dim, const uint32_t* tiles, uint32_t* strips,
                                hipStream_t stream) {
  const int kt_n = in_dim / 16;
  const int s_n = out_dim / kBlock;
  const dim3 grid(s_n, (kt_n + kRepackWaves - 1) / kRepackWaves);
  hipLaunchKernelGGL(repack_strips_kernel, grid, dim3(kWave * kRepackWaves), 0, stream, tiles, strips, 64 * bits,
                     kt_n, s_n);
  return hipGetLastError();
}

}  // namespace tf_exl3
