// Calibration kernels for measurement: a plain copy and a read-only stream.
// Both move 16 bytes per lane per access in wave-contiguous 1 KiB runs, the
// same access form the linear uses for its weight stream, so hardware byte
// counters read on them scale the linear's counters, and the read stream gives
// the HBM read rate this device actually sustains.
#include "exl3_device.hpp"
#include "exl3_launch.hpp"

namespace tf_exl3 {

constexpr int kCalibThreads = 256;
constexpr int kCalibUnroll = 8;

__global__ __launch_bounds__(kCalibThreads) void copy_kernel(const uint4* __restrict__ src,
                                                              uint4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kCalibThreads;
  size_t i = (size_t)blockIdx.x * kCalibThreads + threadIdx.x;
  for (; i + (kCalibUnroll - 1) * stride < n16; i += kCalibUnroll * stride) {
    uint4 v[kCalibUnroll];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kCalibUnroll; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Reads src in contiguous 64 KiB segments per workgroup (16 loads of 16 bytes in
// flight per lane, nontemporal: the data is read once), the fastest read form
// measured on this device. Writes the XOR of what each thread read to out, which
// keeps every load live; a ragged tail shorter than a segment is read one
// 16-byte unit per thread.
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kCalibThreads) void stream_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                     uint32_t* __restrict__ out) {
  constexpr size_t seg = (size_t)kCalibThreads * kReadUnroll;
  uint32_t acc = 0;
  size_t s = blockIdx.x;
  for (; (s + 1) * seg <= n16; s += gridDim.x) {
    const u32x4* p = src + s * seg + threadIdx.x;
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = __builtin_nontemporal_load(p + u * kCalibThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  const size_t full = n16 / seg * seg;
  for (size_t i = full + (size_t)blockIdx.x * kCalibThreads + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * kCalibThreads) {
    const u32x4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(size_t)blockIdx.x * kCalibThreads + threadIdx.x] = acc;
}

hipError_t launch_copy(const void* src, void* dst, size_t bytes, int blocks, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(kCalibThreads), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), bytes / 16);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kCalibThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, out);
  return hipGetLastError();
}

}  // namespace tf_exl3
