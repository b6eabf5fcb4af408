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

// The same over 16-byte words, for 16-byte aligned buffers: 4 words in flight
// per thread, non-temporal (the data is streamed once).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void copy_or_zero_x4_kernel(u32x4* __restrict__ dst,
                                                              const u32x4* __restrict__ src,
                                                              size_t n) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t base = blockIdx.x * (size_t)256 * U + threadIdx.x; base < n; base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * 256;
      v[u] = u32x4{0u, 0u, 0u, 0u};
      if (src != nullptr && i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * 256;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
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
    // at most 16384 workgroups (64 per CU), 1024 words each per pass
    const size_t n = bytes / 16;
    const unsigned blocks = (unsigned)std::min<size_t>(16384, (n + 1023) / 1024);
    hipLaunchKernelGGL(copy_or_zero_x4_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
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
