// Small device utilities shared by the entry points.
#include "ssd_common.h"

namespace ssd {
namespace {

// dst[i] = src ? src[i] : 0 over `words` 32-bit words (a kernel rather than
// hipMemcpyAsync/hipMemsetAsync so that it records cleanly into HIP graphs).
__global__ void copy_or_zero_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                    size_t words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < words;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0u;
}

// The same over 16-byte words, for 16-byte aligned buffers.
__global__ void copy_or_zero_x4_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                       size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : make_uint4(0u, 0u, 0u, 0u);
}

__global__ void copy_or_zero_u16_kernel(uint16_t* __restrict__ dst,
                                        const uint16_t* __restrict__ src, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : (uint16_t)0;
}

}  // namespace

hipError_t launch_copy_or_zero(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  const bool x4 = bytes % 16 == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0 &&
                  reinterpret_cast<uintptr_t>(src) % 16 == 0;
  if (x4) {
    // 4 words in flight per thread per pass; at most 8192 workgroups (32 per CU)
    const size_t n = bytes / 16;
    const unsigned blocks = (unsigned)std::min<size_t>(8192, (n + 255) / 256);
    hipLaunchKernelGGL(copy_or_zero_x4_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), n);
    return hipGetLastError();
  }
  const unsigned blocks = (unsigned)std::min<size_t>(1024, (bytes / 4 + 255) / 256 + 1);
  if (bytes % 4 == 0)
    hipLaunchKernelGGL(copy_or_zero_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<uint32_t*>(dst), static_cast<const uint32_t*>(src), bytes / 4);
  else
    hipLaunchKernelGGL(copy_or_zero_u16_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<uint16_t*>(dst), static_cast<const uint16_t*>(src), bytes / 2);
  return hipGetLastError();
}

}  // namespace ssd
