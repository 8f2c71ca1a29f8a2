// rot_in: z = RN16(RN32(H128(RN32(x * suh)) * s)) per 128-wide block of each row.
//
// TensorFold pull request "hip exl3: the input rotation and trellis linear for
// decode rows": "What this changes" (x times suh, rotated by 128, rounded to
// fp16 once: the fp32 product, the butterflies, then the scale) and "Checks on
// this head" (multiply by the fp32 scale rather than divide; keep the fp32
// product and the fp16 conversion as two roundings).
//
// One wave per 128-block: lane l holds elements l and l + 64 (fwht128_wave).
// The work is a few hundred KiB per call, so the kernel is latency-bound; four
// waves per workgroup keep the grid small.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"
#include "tf_exl3.h"

namespace tf_exl3 {

constexpr int kRotWaves = 4;

template <int XDT>
__global__ __launch_bounds__(kWave* kRotWaves) void rot_in_kernel(const void* __restrict__ x,
                                                                  const uint16_t* __restrict__ suh,
                                                                  uint16_t* __restrict__ z,
                                                                  int blocks_per_row,
                                                                  long long n_blocks) {
  const int lane = __lane_id();
  const long long blk = (long long)blockIdx.x * kRotWaves + (threadIdx.x >> 6);
  if (blk >= n_blocks) return;
  const int kb = (int)(blk % blocks_per_row);
  const size_t base = (size_t)blk * kBlock;  // row * in_dim + kb * 128
  uint16_t z0, z1;
  rot_in_block<XDT>(x, base, suh, kb * kBlock, lane, z0, z1);
  z[base + lane] = z0;
  z[base + lane + 64] = z1;
}

hipError_t launch_rot_in(const void* x, int x_dtype, const uint16_t* suh, uint16_t* z, int rows,
                         int in_dim, hipStream_t stream) {
  const int bpr = in_dim / kBlock;
  const long long n_blocks = (long long)rows * bpr;
  if (n_blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)((n_blocks + kRotWaves - 1) / kRotWaves));
  const dim3 block(kWave * kRotWaves);
  switch (x_dtype) {
    case TF_DT_F32:
      hipLaunchKernelGGL(rot_in_kernel<TF_DT_F32>, grid, block, 0, stream, x, suh, z, bpr, n_blocks);
      break;
    case TF_DT_F16:
      hipLaunchKernelGGL(rot_in_kernel<TF_DT_F16>, grid, block, 0, stream, x, suh, z, bpr, n_blocks);
      break;
    default:
      hipLaunchKernelGGL(rot_in_kernel<TF_DT_BF16>, grid, block, 0, stream, x, suh, z, bpr, n_blocks);
      break;
  }
  return hipGetLastError();
}

}  // namespace tf_exl3
